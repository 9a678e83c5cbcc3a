// b3.hip -- ternary weights at 1.6 bits per weight (five per byte) on gfx950: conversion
// from the 2-bit interface format, and the decode product with the per-token activation
// quantization fused in (one token).
//
// Format ("将 BitNet 三元查找表集成到自定义 Triton 内核中": four to five ternary values per
// uint8; "BitNet 1-bit LLM推理优化" §2.1 and §3.1: packing below 2 bits per weight): byte j
// of a row holds weights k = 5j .. 5j+4, whose codes c = w + 1 are the base-3 digits of
// v = 81 c0 + 27 c1 + 9 c2 + 3 c3 + c4 (the first weight the most significant), stored as
// q = ceil(256 v / 243).  Multiplying q by 3 repeatedly then yields the digits in order as
// the integer parts (the byte-wide fraction carries the rest).  Rows are padded with
// weights 0 to whole 320-weight chunks (64 bytes).
//
// Product (M = 1, "BitNet 深度实战" §4.4: int8 activations times ternary weights into
// int32): a block of four waves owns 16 output rows; its waves take runs of two
// consecutive chunks in turn.  A lane loads 16 packed bytes (80 weights) of one row per
// chunk and spreads them into eight registers of two 16-bit fields.  Each field is
// multiplied by 3 five times without clearing the integer parts in between (they stay
// below 256 for four rounds, then the fields are masked once): after round i the high
// byte of a field is H_i = 3 H_(i-1) + c_i.  Those registers feed the int8 matrix cores
// as they are: the activation operand holds zeros at the fields' low bytes, so only the
// H bytes count.  With a second accumulator pairing round i's activations with round
// i-1's H, sum x c = sum_i x_i H_i - 3 sum_i x_i H_(i-1), no per-digit extraction at all:
// one 24-bit multiply per two weights and round, 56 VALU operations and 16 matrix
// products per lane and chunk (80 weights), against 20 and 4 per 64 weights for the
// mask-based 2-bit decode: this path trades compute for 20% fewer weight bytes.
//
// The block quantizes the activations once (max |x| per wave, one barrier for the token
// maximum) into LDS, laid out so that the 16-byte operand of (chunk, lane group, digit
// round, half) is one aligned read: [0, x(p), 0, x(p+1), ...] for the eight packed bytes p
// of that half.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

namespace {

constexpr int kB3Chunk = 320;       // weights per chunk and row (64 packed bytes)
constexpr int kB3ChunkLds = 640;    // staged activation bytes per chunk
constexpr int kB3Waves = 4;
constexpr int kB3Threads = 64 * kB3Waves;
constexpr int kB3Run = 2;           // consecutive chunks per wave run (128-byte lines)
constexpr uint32_t kB3OOB = 0x80000000u;

__host__ __device__ constexpr int b3_chunk_of(int w, int j) {
    return kB3Run * (w + kB3Waves * (j / kB3Run)) + j % kB3Run;
}
__host__ __device__ constexpr int b3_chunks_of_wave(int w, int nch) {
    const int span = kB3Run * kB3Waves, r = nch % span - kB3Run * w;
    return (nch / span) * kB3Run + (r < 0 ? 0 : (r > kB3Run ? kB3Run : r));
}

struct B3Args {
    const uint16_t* x;
    const uint8_t* b3;
    const float* w_scale;
    void* out;
    int N, K, nch, out_dtype;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t b3_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 b3_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// wave-wide max with a uniform result (DPP row steps, then v_readlane)
__device__ __forceinline__ uint32_t b3_wave_max(uint32_t v) {
    v = wave_max_u32(v);
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Template parameters: XW activation windows (40 elements) per lane; U chunks per weight
// batch; SINGLE when one batch covers a wave's chunks.
template <int XW, int U, bool SINGLE>
__global__ __launch_bounds__(kB3Threads) void b3_gemv_kernel(B3Args p) {
    extern __shared__ __align__(16) unsigned char x_lds[];
    __shared__ uint32_t s_wmax[kB3Waves];
    __shared__ int s_red[kB3Waves][16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = p.N, K = p.K, nch = p.nch;
    const int RB = nch * 64;
    const int n0 = (int)blockIdx.x * 16;
    const int rows = min(16, N - n0);
    const int mrow = lane & 15, kq = lane >> 4;
    const int cpw = b3_chunks_of_wave(wave, nch);

    // Operand-A reads of the lanes of token rows 1-15 go to a zeroed 160-byte area after
    // the staged chunks, so every lane reads unconditionally.
    const int zero_off = nch * kB3ChunkLds;
    if (tid < 10) *reinterpret_cast<uint4*>(x_lds + zero_off + 16 * tid) = make_uint4(0u, 0u, 0u, 0u);

    // the weight scale of this thread's output column, requested first
    const float ws = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        b3_rsrc(p.w_scale + n0, (uint32_t)(rows * 4)), tid < 16 ? 4u * tid : kB3OOB, 0, 0));

    // Activation windows of this wave: window v = 8 j + 2 g + h covers the 40 elements of
    // chunk chunk_of(wave, j), lane group g, half h: k0 = 320 c + 80 g + 40 h, five 16-byte
    // loads (K % 8 == 0: each load lies wholly inside or wholly past the row).
    const __amdgpu_buffer_rsrc_t x_rsrc = b3_rsrc(p.x, (uint32_t)(K * 2));
    uint32_t held[XW][20];
#pragma unroll
    for (int t = 0; t < XW; ++t) {
        const int v = lane + 64 * t, j = v >> 3, sub = v & 7;
        const int k0 = kB3Chunk * b3_chunk_of(wave, j) + 80 * (sub >> 1) + 40 * (sub & 1);
        const bool ok = j < cpw;
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const uint4 d = b3_load16(x_rsrc, ok ? (uint32_t)(2 * k0 + 16 * u) : kB3OOB);
            held[t][4 * u] = d.x;
            held[t][4 * u + 1] = d.y;
            held[t][4 * u + 2] = d.z;
            held[t][4 * u + 3] = d.w;
        }
    }

    // the first batch of weights: lane (row mrow, lane group kq) reads 16 bytes per chunk
    const __amdgpu_buffer_rsrc_t w_rsrc =
        b3_rsrc(p.b3 + (int64_t)n0 * RB, (uint32_t)(rows * RB));
    const uint32_t w_lane = (uint32_t)(mrow * RB + 16 * kq);
    auto load_batch = [&](uint4 (&w)[U], int j0) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int j = j0 + uu;
            w[uu] = b3_load16(w_rsrc, j < cpw ? w_lane + 64u * b3_chunk_of(wave, j) : kB3OOB);
        }
    };
    uint4 wa[U];
    load_batch(wa, 0);

    // ---- token maximum, scale, quantization into LDS ----
    uint32_t mx = 0;
#pragma unroll
    for (int t = 0; t < XW; ++t)
#pragma unroll
        for (int u = 0; u < 20; ++u) {
            const uint32_t a = held[t][u] & 0x7FFF7FFFu;
            mx = max(mx, max(a & 0xFFFFu, a >> 16));
        }
    mx = b3_wave_max(mx);
    if (lane == 0) s_wmax[wave] = mx;
    __syncthreads();  // also orders the zero area before any read of it
    float amax = bf16_bits_to_f32(max(max(s_wmax[0], s_wmax[1]), max(s_wmax[2], s_wmax[3])));
    amax = amax < 1e-5f ? 1e-5f : amax;
    const float a = 127.0f / amax;

    // codes rint(fl(x a)) (one fp32 add of 1.5 * 2^23 rounds half to even; the clamp to
    // +-127 cannot bind since |fl(x a)| <= 127 (1 + 2^-23)); window codes in 10 words
    constexpr float kMagic = 12582912.0f;
    int csum = 0;
#pragma unroll
    for (int t = 0; t < XW; ++t) {
        const int v = lane + 64 * t, j = v >> 3, sub = v & 7;
        if (j < cpw) {
            uint32_t cw[10];
#pragma unroll
            for (int d = 0; d < 10; ++d) {
                uint32_t b[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t h = held[t][(4 * d + e) >> 1];
                    const float f = (e & 1) ? __uint_as_float(h & 0xFFFF0000u) : bf16_bits_to_f32(h);
                    b[e] = __float_as_uint(f * a + kMagic);
                }
                cw[d] = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) |
                        __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
                csum = sum_i8x4(cw[d], csum);
            }
            // slot (digit i, this window's half): dword d = [0, code(10 d + i), 0,
            // code(10 d + 5 + i)], code(e) = byte e of cw
            unsigned char* base = x_lds + ((b3_chunk_of(wave, j) * 4 + (sub >> 1)) * 5) * 32 + 16 * (sub & 1);
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                uint32_t s4[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    constexpr uint32_t kZ = 0x0Cu;  // selector of a zero byte
                    const int e0 = 10 * d + i, e1 = 10 * d + 5 + i;
                    const int w0 = e0 >> 2, w1 = e1 >> 2;
                    // bytes from {hi = cw[w1], lo = cw[w0]}: lo byte e0 % 4, hi byte 4 + e1 % 4
                    const uint32_t sel = kZ | ((uint32_t)(e0 & 3) << 8) | (kZ << 16) |
                                         ((uint32_t)(4 + (e1 & 3)) << 24);
                    s4[d] = __builtin_amdgcn_perm(cw[w1], cw[w0], sel);
                }
                *reinterpret_cast<uint4*>(base + 32 * i) = make_uint4(s4[0], s4[1], s4[2], s4[3]);
            }
        }
    }
    csum = (int)wave_sum_i32(csum);  // codes of this wave's chunks (all of them 0 past K)
    // the wave reads only the slots it wrote, and a wave's LDS operations complete in
    // order; keep the compiler from hoisting the reads
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // ---- products ----
    v4i acc = {0, 0, 0, 0}, accx = {0, 0, 0, 0};
    auto compute_batch = [&](const uint4 (&w)[U], int j0) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int j = j0 + uu;
            if (j < cpw) {  // uniform over the wave
                const int c = b3_chunk_of(wave, j);
                const uint32_t w4[4] = {w[uu].x, w[uu].y, w[uu].z, w[uu].w};
                // t[4h + d]: packed bytes 8h + 2d (low field) and 8h + 2d + 1 (high field)
                uint32_t t[8];
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    t[r] = __builtin_amdgcn_perm(0u, w4[r >> 1], (r & 1) ? 0x0C030C02u : 0x0C010C00u);
                // the ten activation operands of the chunk, requested together
                const unsigned char* slot = x_lds + (mrow == 0 ? ((c * 4 + kq) * 5) * 32 : zero_off);
                v4i A[5][2];
#pragma unroll
                for (int i = 0; i < 5; ++i)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        A[i][h] = *reinterpret_cast<const v4i*>(slot + 32 * i + 16 * h);
                v4i prev[2];
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    if (i == 4) {
#pragma unroll
                        for (int r = 0; r < 8; ++r) t[r] &= 0x00FF00FFu;
                    }
#pragma unroll
                    for (int r = 0; r < 8; ++r) t[r] += t[r] << 1;  // x3 in both fields
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const v4i B = {(int)t[4 * h], (int)t[4 * h + 1], (int)t[4 * h + 2],
                                       (int)t[4 * h + 3]};
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i][h], B, acc, 0, 0, 0);
                        if (i >= 1 && i <= 3)
                            accx = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i][h], prev[h], accx, 0, 0, 0);
                        prev[h] = B;
                    }
                }
            }
        }
    };
    if constexpr (SINGLE) {
        compute_batch(wa, 0);
    } else {
        uint4 wb[U];
        for (int j0 = 0; j0 < cpw; j0 += 2 * U) {
            load_batch(wb, j0 + U);
            compute_batch(wa, j0);
            if (j0 + U >= cpw) break;
            load_batch(wa, j0 + 2 * U);
            compute_batch(wb, j0 + U);
        }
    }

    // ---- combine the waves and write: token 0 is row 0 of the 16x16 accumulators
    // (register 0 of lanes 0-15) ----
    if (lane < 16) s_red[wave][lane] = acc[0] - 3 * accx[0] - csum;
    __syncthreads();
    if (tid < rows) {
        const int total = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
        store_out(p.out, n0 + tid, p.out_dtype, total, ws, __builtin_amdgcn_rcpf(a));
    }
}

// One thread per output byte: five weights of the 2-bit interface format (code w + 1 in
// bits 2i..2i+1, a field holding the unused code 3 read as weight 0, weights past K as 0)
// into one byte q = ceil(256 v / 243).
__global__ __launch_bounds__(256) void b3_pack_kernel(const uint8_t* __restrict__ packed,
                                                      int64_t N, int64_t K, int64_t RB,
                                                      uint8_t* __restrict__ b3) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= N * RB) return;
    const int64_t n = idx / RB, j = idx - n * RB;
    const uint8_t* row = packed + n * (K / 4);
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int64_t k = 5 * j + i;
        uint32_t c = 1;  // weight 0
        if (k < K) {
            c = (row[k >> 2] >> (2 * (k & 3))) & 3u;
            if (c == 3u) c = 1;
        }
        v = 3 * v + c;
    }
    b3[idx] = (uint8_t)((256 * v + 242) / 243);
}

template <int XW>
hipError_t launch_b3_xw(const B3Args& a, dim3 grid, size_t lds, hipStream_t stream) {
    const int cpw = b3_chunks_of_wave(0, a.nch);
    if (cpw <= 4)
        hipLaunchKernelGGL((b3_gemv_kernel<XW, 4, true>), grid, dim3(kB3Threads), lds, stream, a);
    else if (cpw <= 8)
        hipLaunchKernelGGL((b3_gemv_kernel<XW, 8, true>), grid, dim3(kB3Threads), lds, stream, a);
    else
        hipLaunchKernelGGL((b3_gemv_kernel<XW, 8, false>), grid, dim3(kB3Threads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

int64_t b3_row_bytes(int64_t K) { return (K + kB3Chunk - 1) / kB3Chunk * 64; }

hipError_t launch_pack_b3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* b3,
                          hipStream_t stream) {
    const int64_t RB = b3_row_bytes(K);
    const int64_t total = N * RB;
    hipLaunchKernelGGL(b3_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       packed, N, K, RB, b3);
    return hipGetLastError();
}

hipError_t launch_quant_gemv_b3(const uint16_t* x, const uint8_t* b3, const float* w_scale,
                                int64_t N, int64_t K, void* out, int out_dtype,
                                hipStream_t stream) {
    B3Args a;
    a.x = x;
    a.b3 = b3;
    a.w_scale = w_scale;
    a.out = out;
    a.N = (int)N;
    a.K = (int)K;
    a.nch = (int)((K + kB3Chunk - 1) / kB3Chunk);
    a.out_dtype = out_dtype;
    const size_t lds = (size_t)a.nch * kB3ChunkLds + 160;  // chunks + the zero area
    const dim3 grid((unsigned)((N + 15) / 16));
    // windows per lane: 8 per chunk of the busiest wave, over 64 lanes
    const int xw = (8 * b3_chunks_of_wave(0, a.nch) + 63) / 64;
    if (xw <= 1) return launch_b3_xw<1>(a, grid, lds, stream);
    if (xw <= 2) return launch_b3_xw<2>(a, grid, lds, stream);
    return launch_b3_xw<3>(a, grid, lds, stream);
}

}  // namespace bitnet
