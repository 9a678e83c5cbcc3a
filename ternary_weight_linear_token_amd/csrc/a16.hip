// a16.hip -- ternary weights times bf16 activations, no activation quantization
// (W1.58A16), on gfx950 bf16 matrix cores with fp32 accumulation, 1 <= M <= 16.
//
// What it computes ("将 BitNet 三元查找表集成到自定义 Triton 内核中": mixed-precision serving
// with 16-bit activations and an fp32 accumulator; "BitNet 深度实战" §2.2: with ternary
// weights the product needs only additions and subtractions):
//   out[m,n] = w_scale[n] * sum_k x[m,k] * w[n,k],   w from the packed 2-bit codes.
//
// Design:
//  * A block (4 wave64s) owns 16 output rows and all of K; the waves take interleaved
//    256-weight chunks, and a lane loads 16 packed bytes (64 weights) of one row per
//    chunk, as in the int8 decode kernel.  Operand B of v_mfma_f32_16x16x32_bf16 is the
//    weights (columns = output rows), operand A the activations (rows = tokens).
//  * Weights become bf16 operands by byte lookups only.  For field i of the four bytes
//    of a packed dword, one mask turns the four codes into v_perm selectors, one v_perm
//    looks up the high byte of bf16(2w) (0xC0, 0x00, 0x40 for w = -1, 0, +1; the low byte
//    of +-2 is zero), and two v_perm interleave those with zero low bytes.  A register
//    pair so holds 2w for k = i, 4+i, 8+i, 12+i of the dword's 16-weight group; the
//    factor 2 is exact and is removed at the end.  About 1.2 VALU ops per weight.
//  * Activations are read straight from memory (at most 16 rows, L2-resident): a lane
//    loads its 16-element group (32 bytes) and v_perm gathers the same k order.
//  * Every product is exact in fp32 (bf16 times -2, 0 or 2); the matrix cores add in
//    fp32, and the four waves' partial sums are added in a fixed order.
//  * K must be a multiple of 64 (16-byte aligned packed rows, whole 16-element groups).
#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kA16Waves = 4;
constexpr uint32_t kA16OOB = 0x80000000u;  // buffer offset past every resource: reads 0
// high bytes of bf16(2w) by code (w = code - 1): 0xC0 (-2), 0x00 (0), 0x40 (+2), 0 (unused)
constexpr uint32_t kHiTable = 0x004000C0u;

struct A16Args {
    const uint16_t* x;
    const uint8_t* packed;
    const float* w_scale;
    void* out;
    int M, N, K;
    int out_dtype;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t a16_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 a16_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Operand B for fields (f, f + 1) of packed dword d: 2w at k = f, f+4, f+8, f+12, f+1,
// f+5, f+9, f+13 of the dword's 16-weight group.
__device__ __forceinline__ bf16x8 weights_b(uint32_t d, int f) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t sel = (d >> (2 * (f + h))) & 0x03030303u;
        const uint32_t hi = __builtin_amdgcn_perm(kHiTable, kHiTable, sel);
        r[2 * h] = __builtin_amdgcn_perm(0u, hi, 0x010C000Cu);      // (2w of byte 0, byte 1)
        r[2 * h + 1] = __builtin_amdgcn_perm(0u, hi, 0x030C020Cu);  // (byte 2, byte 3)
    }
    return __builtin_bit_cast(bf16x8, r);
}

// Operand A for fields (f, f + 1): x at the same k order, from the group's 16 elements
// held as 8 dwords (element pairs).
__device__ __forceinline__ bf16x8 acts_a(const uint32_t (&X)[8], int f) {
    const int j = f >> 1;  // 0 for f = 0, 1 for f = 2
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(X[2 + j], X[0 + j], 0x05040100u);  // (x_f, x_{f+4})
    r[1] = __builtin_amdgcn_perm(X[6 + j], X[4 + j], 0x05040100u);  // (x_{f+8}, x_{f+12})
    r[2] = __builtin_amdgcn_perm(X[2 + j], X[0 + j], 0x07060302u);  // (x_{f+1}, x_{f+5})
    r[3] = __builtin_amdgcn_perm(X[6 + j], X[4 + j], 0x07060302u);  // (x_{f+9}, x_{f+13})
    return __builtin_bit_cast(bf16x8, r);
}

__global__ __launch_bounds__(64 * kA16Waves) void a16_kernel(A16Args p) {
    __shared__ float red[kA16Waves * 4 * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = p.M, N = p.N, K = p.K;
    const int row_bytes = K / 4;
    const int n0 = blockIdx.x * 16;
    const int rows = min(16, N - n0);
    const int l16 = lane & 15, q = lane >> 4;
    const int nch = (K + 255) / 256;

    const __amdgpu_buffer_rsrc_t w_rsrc =
        a16_rsrc(p.packed + (int64_t)n0 * row_bytes, (uint32_t)(rows * row_bytes));
    const __amdgpu_buffer_rsrc_t x_rsrc = a16_rsrc(p.x, (uint32_t)(M * K * 2));
    const uint32_t w_lane = (uint32_t)(l16 * row_bytes + 16 * q);
    const bool x_row = l16 < M;  // this lane's operand-A row holds a token

    // chunk j of this wave: its 16 packed bytes and its four 16-element activation groups
    // (zeros past K or past the wave's chunks)
    auto load = [&](int j, u32x4& w, uint32_t (&X)[4][8]) {
        const int c = wave + kA16Waves * j;
        const bool live = c < nch;
        w = a16_load16(w_rsrc, live ? w_lane + 64 * c : kA16OOB);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k0 = 256 * c + 64 * q + 16 * s;
            const uint32_t off = (live && x_row && k0 < K) ? (uint32_t)((l16 * K + k0) * 2) : kA16OOB;
            const u32x4 v0 = a16_load16(x_rsrc, off);
            const u32x4 v1 = a16_load16(x_rsrc, off + 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                X[s][e] = v0[e];
                X[s][4 + e] = v1[e];
            }
        }
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int nj = (nch - wave + kA16Waves - 1) / kA16Waves;  // chunks of this wave
    u32x4 w_cur;
    uint32_t X_cur[4][8];
    load(0, w_cur, X_cur);
    for (int j = 0; j < nj; ++j) {
        u32x4 w_nxt;
        uint32_t X_nxt[4][8];
        load(j + 1, w_nxt, X_nxt);  // past the wave's chunks: out-of-range offsets, zeros
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int f = 0; f < 4; f += 2)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acts_a(X_cur[s], f),
                                                              weights_b(w_cur[s], f), acc, 0, 0, 0);
        w_cur = w_nxt;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) X_cur[s][e] = X_nxt[s][e];
    }

    // 16x16 fp32 accumulator layout: lane l, register r -> row 4*(l/16)+r, column l%16
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (tid < 16 * M) {
        const int m = tid >> 4, col = tid & 15;
        if (col < rows) {
            const int l = 16 * (m >> 2) + col, r = m & 3;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < kA16Waves; ++w) sum += red[(w * 4 + r) * 64 + l];
            const float v = (0.5f * sum) * p.w_scale[n0 + col];  // 0.5: the weights were 2w
            const int64_t o = (int64_t)m * N + n0 + col;
            if (p.out_dtype == 0)
                static_cast<float*>(p.out)[o] = v;
            else
                static_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
        }
    }
}

}  // namespace

hipError_t launch_a16(const uint16_t* x, const uint8_t* packed, const float* w_scale, int64_t M,
                      int64_t N, int64_t K, void* out, int out_dtype, hipStream_t stream) {
    if (M < 1 || M > 16 || N < 1 || K % 64 != 0 || (out_dtype != 0 && out_dtype != 1) ||
        M * K * 2 > INT32_MAX)
        return hipErrorInvalidValue;
    A16Args a;
    a.x = x;
    a.packed = packed;
    a.w_scale = w_scale;
    a.out = out;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.out_dtype = out_dtype;
    hipLaunchKernelGGL(a16_kernel, dim3((unsigned)((N + 15) / 16)), dim3(64 * kA16Waves), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace bitnet
