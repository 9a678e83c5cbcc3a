// device_common.hpp -- small device helpers shared by the gfx950 kernels of the
// W2A8 BitLinear library (bf16 conversion, byte transposes, wave reductions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// bf16 bit pattern -> fp32: bf16 is the upper half of binary32, so this is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even: the hardware conversion
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 values -> two bf16 (low half first), one conversion instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const f2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// 4x4 byte transpose: d[b] holds bytes (b, 0..3) of a 16-byte group; on return e[i]
// holds byte i of d[0], d[1], d[2], d[3] (in that order).  v_perm_b32 picks bytes
// from the 8-byte pool {hi:lo}, selector values 0-3 address lo, 4-7 address hi.
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t d[4], uint32_t e[4]) {
    uint32_t lo01 = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u);  // d0.0 d1.0 d0.1 d1.1
    uint32_t hi01 = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u);  // d0.2 d1.2 d0.3 d1.3
    uint32_t lo23 = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);  // d2.0 d3.0 d2.1 d3.1
    uint32_t hi23 = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);  // d2.2 d3.2 d2.3 d3.3
    e[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);           // d0.0 d1.0 d2.0 d3.0
    e[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);           // d0.1 d1.1 d2.1 d3.1
    e[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    e[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Sum of the four signed bytes of v (dot product with 0x01010101).
__device__ __forceinline__ int sum_i8x4(uint32_t v, int acc) {
    return __builtin_amdgcn_sdot4((int)v, 0x01010101, acc, false);
}

// Signed weight bytes from 2-bit codes: field i (bits 2i..2i+1) of each byte of d,
// code c -> w = c - 1 as int8 {0xFF, 0x00, 0x01, 0x02} through a v_perm lookup.  The
// code 3, which packing never writes, decodes as +2 like in the mask-based unpack, so
// every int8 kernel reads any byte the same way.
template <int I>
__device__ __forceinline__ uint32_t ternary_field_i8(uint32_t d) {
    uint32_t sel = (d >> (2 * I)) & 0x03030303u;
    return __builtin_amdgcn_perm(0u, 0x020100FFu, sel);
}

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15): xor 1 and xor 2 by
// quad permutes, then the 8-lane and 16-lane mirrors; every lane of the row gets the
// result.  All on the VALU: no LDS round trip per step, unlike lane shuffles.
template <typename Op>
__device__ __forceinline__ uint32_t row16_reduce(uint32_t v, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // mirror
    return v;
}
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    return row16_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int row16_sum(int v) {
    return (int)row16_reduce((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Wave-wide reductions (every lane active) with a uniform result: the row reduction,
// then the four row results read out with v_readlane.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_dpp(uint32_t v, Op op) {
    v = row16_reduce(v, op);
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return op(op(a, b), op(c, d));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce_dpp(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ int wave_sum_i32(int v) {
    return (int)wave_reduce_dpp((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Store one output element in the requested dtype (0 = f32, 1 = bf16, 2 = int32).
__device__ __forceinline__ void store_out(void* out, int64_t idx, int dtype, int acc, float s,
                                          float inv_a) {
    if (dtype == 2) {
        static_cast<int*>(out)[idx] = acc;
    } else {
        float v = ((float)acc * s) * inv_a;
        if (dtype == 0)
            static_cast<float*>(out)[idx] = v;
        else
            static_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
    }
}

// Quantize 16 bf16 values (h: 8 words, 2 values each, low half first) with scale a into
// 16 int8 codes, packed transposed for the operand layout: byte b of e[i] is the code of
// element 4 b + i.  The code is rint(fl(x * a)) with ties to even: adding 1.5 * 2^23 to
// fl(x * a) (|x * a| < 2^22) rounds it to an integer in one fp32 addition, and the low
// byte of the sum's bit pattern is that integer in two's complement.  The clamp to
// +-127 of the definition never binds here: a = fl(127 / amax) and |x| <= amax give
// |fl(x * a)| <= 127 (1 + 2^-23) < 127.5.
__device__ __forceinline__ void quant16_t(const uint32_t h[8], float a, uint32_t e[4]) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    uint32_t v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[2 * j] = __float_as_uint(bf16_bits_to_f32(h[j]) * a + kMagic);
        v[2 * j + 1] = __float_as_uint(__uint_as_float(h[j] & 0xFFFF0000u) * a + kMagic);
    }
    // low bytes of elements i, 4+i (bytes 0, 1) and 8+i, 12+i (bytes 2, 3); selector 0x0c
    // gives a zero byte
#pragma unroll
    for (int i = 0; i < 4; ++i)
        e[i] = __builtin_amdgcn_perm(v[4 + i], v[i], 0x0c0c0400u) |
               __builtin_amdgcn_perm(v[12 + i], v[8 + i], 0x04000c0cu);
}

// max |x| of 16 bf16 values as bf16 bits (a monotone key for non-negative values),
// two lanes at a time with the packed 16-bit integer max.
__device__ __forceinline__ uint32_t absmax_bits16(const uint32_t h[8]) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = __builtin_bit_cast(u16x2, h[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < 8; ++j)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, h[j] & 0x7FFF7FFFu));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// Per-token max |x| of bf16 activations as bf16 bits with the sign cleared.  x is a
// buffer resource over the (M, K) rows (M * K * 2 bytes).  Wave w of W scans rows w,
// w + W, ...; lane 0 writes the maximum of row m to slot[m].  A lane asks for a batch of
// 8 loads (16 bytes each when W16, i.e. K % 8 == 0, else 8 bytes; zeros past the row)
// and for the next batch before it reduces the current one, so the scan waits about
// once per batch pair instead of once per load of every row.
template <bool W16>
__device__ __forceinline__ void scan_absmax_rows(__amdgpu_buffer_rsrc_t x, int M, int K, int w,
                                                 int W, uint32_t* slot) {
    constexpr int PE = W16 ? 8 : 4;   // bf16 values per load
    constexpr int NB = 8;             // loads per lane per batch
    constexpr int NWD = NB * PE / 2;  // words per lane per batch
    const int lane = threadIdx.x & 63;
    const int span = 64 * NB * PE;          // row elements per batch
    const int bpr = (K + span - 1) / span;  // batches per row
    const int items = (w < M ? (M - 1 - w) / W + 1 : 0) * bpr;
    auto load = [&](int t, uint32_t (&v)[NWD]) {
        const int r = t / bpr;
        const int m = w + W * r, kb = (t - r * bpr) * span;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int k = kb + PE * (lane + 64 * i);
            // K % PE == 0: a load is wholly inside its row or wholly past its end
            const uint32_t off =
                (t < items && k < K) ? (uint32_t)(((int64_t)m * K + k) * 2) : 0x80000000u;
            if constexpr (W16) {
                const auto u = __builtin_amdgcn_raw_buffer_load_b128(x, off, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) v[4 * i + j] = u[j];
            } else {
                const auto u = __builtin_amdgcn_raw_buffer_load_b64(x, off, 0, 0);
                v[2 * i] = u[0];
                v[2 * i + 1] = u[1];
            }
        }
    };
    uint32_t mx = 0;
    auto reduce = [&](int t, const uint32_t (&v)[NWD]) {
#pragma unroll
        for (int i = 0; i < NWD; i += 8) mx = max(mx, absmax_bits16(v + i));
        if ((t + 1) % bpr == 0) {  // the last batch of its row (uniform)
            const uint32_t r = wave_max_u32(mx);
            if (lane == 0) slot[w + W * (t / bpr)] = r;
            mx = 0;
        }
    };
    uint32_t a[NWD], b[NWD];
    load(0, a);
    for (int t = 0; t < items; t += 2) {
        load(t + 1, b);  // past the wave's rows: zeros, never reduced
        reduce(t, a);
        load(t + 2, a);
        if (t + 1 < items) reduce(t + 1, b);
    }
}

// Element-order codes of a transposed group (for the optional copy of the codes).
__device__ __forceinline__ void untranspose(const uint32_t e[4], uint32_t d[4]) {
    transpose4x4_bytes(e, d);  // the 4x4 byte transpose is its own inverse
}

template <bool FAST>
__device__ __forceinline__ void store_codes16(int8_t* xq_out, int K, int m, int k0,
                                              const uint32_t d[4]) {
    int8_t* dst = xq_out + (int64_t)m * K + k0;
    if (FAST) {
        if (k0 < K) *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (k0 + j < K) dst[j] = (int8_t)(d[j >> 2] >> (8 * (j & 3)));
    }
}

}  // namespace bitnet
