// skinny.hip -- weight-streaming W2A8 product for 1 <= M <= 16 on gfx950, with the
// per-token activation quantization optionally fused into the same launch.
//
// What it computes ("BitNet 深度实战" (chenxutan.com) §4.4; "BitNet-Triton" (zingnex.cn)
// 技术架构 §1-§3): out[m,n] = acc[m,n] * w_scale[n] / a_scale[m] with
// acc[m,n] = sum_k xq[m,k] * w[n,k] exact in int32 and w the 2-bit codes of the packed
// (N, K/4) array, unpacked in registers.  The fused variant first quantizes the bf16
// activations (per-token absmax, 127/max|x|, round half even) inside every block.
//
// Design (decode is a stream over the packed weights; the pages' own kernels were
// written for NVIDIA warps and dp4a, none of that is reused here):
//  * A block (4 wave64s) owns 16 output rows and all of K.  The four waves take
//    interleaved 256-weight chunks of K; a lane loads 16 packed bytes (64 weights) of
//    one row per chunk, a wave 16 rows x 64 bytes, with 128-bit loads.
//  * The activations (M <= 16 rows) sit in LDS; each chunk feeds int8 matrix-core
//    products v_mfma_i32_16x16x64_i8 with the activations as operand A (rows m) and
//    the weight codes as operand B (columns n).
//  * Unpack without a full decode: field i of every byte is isolated by one mask
//    (d & 0x03030303, d & 0x0C0C0C0C, d & 0x30303030, (d >> 2) & 0x30303030), giving the
//    code c = w + 1 times 1, 4, 16, 16.  Three int32 accumulators take the three scales;
//    at the end acc = acc1 + acc4/4 + acc16/16 - sum_k xq[m,k] (the divisions are exact).
//    Five VALU ops per 16 weights.
//  * The activations are stored in LDS in the k-order that makes operand A match: within
//    every 64-element group, position 16 i + 4 r + b holds k = 16 r + 4 b + i.  Any
//    common permutation of k on both operands leaves the dot product unchanged.
//  * Per-wave int32 partials are combined through LDS; one pass writes the outputs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

namespace {

constexpr int kSkThreads = 256;
constexpr int kSkWaves = 4;
constexpr int kSkXBudget = 48 * 1024;  // LDS bytes for the staged activations
constexpr int kSkMisc = 256;           // s_amax, s_rowsum, s_a, s_inva (16 entries each)

struct SkinnyArgs {
    const int8_t* xq;
    const float* a_scale;
    const uint16_t* xb;
    const uint8_t* packed;
    const float* w_scale;
    void* out;
    int8_t* xq_out;
    float* a_out;
    int M, N, K;
    int Kp;  // K rounded up to a multiple of 256
    int KS;  // K-stage length staged in LDS at once (multiple of 256)
    int out_dtype;
};

// 16 packed bytes at byte offset `off` of packed row `n` (zeros past the row end).
template <bool ALIGNED>
__device__ __forceinline__ uint4 load_w16(const uint8_t* __restrict__ packed, int64_t row_bytes,
                                          int n, int64_t off) {
    const uint8_t* src = packed + (int64_t)n * row_bytes + off;
    if (ALIGNED) return *reinterpret_cast<const uint4*>(src);
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (off + j < row_bytes) d[j >> 2] |= (uint32_t)src[j] << (8 * (j & 3));
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// Quantize 16 bf16 values (h: 8 words, 2 values each, low half first) with scale a into
// 16 int8 codes d[0..3] (value j in byte j%4 of d[j/4]).
__device__ __forceinline__ void quant16(const uint32_t h[8], float a, uint32_t d[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t word = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t hw = h[2 * b + (t >> 1)];
            const uint32_t bits = (t & 1) ? (hw >> 16) : (hw & 0xFFFFu);
            float r = rintf(bf16_bits_to_f32(bits) * a);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            word |= ((uint32_t)(int)r & 0xFFu) << (8 * t);
        }
        d[b] = word;
    }
}

// Load 16 bf16 activations x[m][k0 .. k0+15] (zeros past K) as 8 words.
template <bool ALIGNED>
__device__ __forceinline__ void load_x16_bf16(const uint16_t* __restrict__ xb, int K, int m,
                                              int k0, uint32_t h[8]) {
    const uint16_t* src = xb + (int64_t)m * K + k0;
    if (ALIGNED) {
        const uint4 v0 = reinterpret_cast<const uint4*>(src)[0];
        const uint4 v1 = reinterpret_cast<const uint4*>(src)[1];
        h[0] = v0.x; h[1] = v0.y; h[2] = v0.z; h[3] = v0.w;
        h[4] = v1.x; h[5] = v1.y; h[6] = v1.z; h[7] = v1.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t lo = (k0 + 2 * j < K) ? src[2 * j] : 0u;
            const uint32_t hi = (k0 + 2 * j + 1 < K) ? src[2 * j + 1] : 0u;
            h[j] = lo | (hi << 16);
        }
    }
}

__device__ __forceinline__ uint32_t absmax_bits16(const uint32_t h[8]) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t a = h[j] & 0x7FFF7FFFu;
        mx = max(mx, max(a & 0xFFFFu, a >> 16));
    }
    return mx;
}

// One 16-element group of activations, quantized (d), into the permuted LDS layout;
// also adds its code sum to s_rowsum[m] and (block 0, if requested) writes the codes.
template <bool ALIGNED>
__device__ __forceinline__ void put_group(unsigned char* x_lds, int KSP, int* s_rowsum, int m,
                                          int u, const uint32_t d[4]) {
    const int rs = sum_i8x4(d[0], sum_i8x4(d[1], sum_i8x4(d[2], sum_i8x4(d[3], 0))));
    atomicAdd(&s_rowsum[m], rs);
    uint32_t e[4];
    transpose4x4_bytes(d, e);
    unsigned char* dst = x_lds + m * KSP + (u >> 2) * 64 + 4 * (u & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(dst + 16 * i) = e[i];
}

template <bool ALIGNED>
__device__ __forceinline__ void store_codes16(int8_t* xq_out, int K, int m, int k0,
                                              const uint32_t d[4]) {
    int8_t* dst = xq_out + (int64_t)m * K + k0;
    if (ALIGNED) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (k0 + j < K) dst[j] = (int8_t)(d[j >> 2] >> (8 * (j & 3)));
    }
}

constexpr int kU = 4;  // 256-weight chunks per wave per batch (loads in flight per lane)

// XREG > 0: the block's activation groups (at most XREG per thread, single K stage) stay
// in registers between the max pass and the quantization pass.
template <int NG, bool FUSED, bool ALIGNED, int XREG>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkinnyArgs p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int KSP = p.KS + 16;  // padded LDS row stride: spreads rows over the banks
    const int M = p.M, N = p.N, K = p.K;
    unsigned char* x_lds = smem;
    uint32_t* s_amax = reinterpret_cast<uint32_t*>(smem + M * KSP);
    int* s_rowsum = reinterpret_cast<int*>(s_amax + 16);
    float* s_a = reinterpret_cast<float*>(s_rowsum + 16);
    float* s_inva = s_a + 16;
    int* red = reinterpret_cast<int*>(smem + M * KSP + kSkMisc);  // [waves][NG][4][64]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row_bytes = K / 4;
    const int n0 = blockIdx.x * (16 * NG);
    const int mrow = lane & 15;  // operand-A row (token) and operand-B column of this lane
    const int q = lane >> 4;     // k-group of this lane inside a 256-weight chunk
    const bool a_active = mrow < M;

    // weights of chunks c0 + 4*uu (uu < kU) of the stage starting at byte stage_off
    auto load_batch = [&](uint4 (&w)[kU][NG], int c0, int nch, int64_t stage_off) {
#pragma unroll
        for (int uu = 0; uu < kU; ++uu) {
            const int c = c0 + kSkWaves * uu;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int n = n0 + 16 * g + mrow;
                w[uu][g] = (c < nch && n < N)
                               ? load_w16<ALIGNED>(p.packed, row_bytes, n, stage_off + c * 64 + 16 * q)
                               : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    v4i acc1[NG], acc4[NG], acc16[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc1[g] = acc4[g] = acc16[g] = v4i{0, 0, 0, 0};

    auto compute_batch = [&](const uint4 (&w)[kU][NG], int c0, int nch) {
#pragma unroll
        for (int uu = 0; uu < kU; ++uu) {
            const int c = c0 + kSkWaves * uu;
            if (c >= nch) break;
            v4i A[4];
            if (a_active) {
                const unsigned char* src = x_lds + mrow * KSP + (c * 4 + q) * 64;
#pragma unroll
                for (int i = 0; i < 4; ++i) A[i] = *reinterpret_cast<const v4i*>(src + 16 * i);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) A[i] = v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t w4[4] = {w[uu][g].x, w[uu][g].y, w[uu][g].z, w[uu][g].w};
                v4i b0, b1, b2, b3;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    b0[r] = (int)(w4[r] & 0x03030303u);
                    b1[r] = (int)(w4[r] & 0x0C0C0C0Cu);
                    b2[r] = (int)(w4[r] & 0x30303030u);
                    b3[r] = (int)((w4[r] >> 2) & 0x30303030u);
                }
                acc1[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[0], b0, acc1[g], 0, 0, 0);
                acc4[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[1], b1, acc4[g], 0, 0, 0);
                acc16[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2], b2, acc16[g], 0, 0, 0);
                acc16[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[3], b3, acc16[g], 0, 0, 0);
            }
        }
    };

    // The first weight batch is requested before anything else, so its memory latency
    // overlaps the activation phases below.
    uint4 cur[kU][NG], nxt[kU][NG];
    {
        const int len0 = min(p.KS, p.Kp);
        load_batch(cur, wave, len0 >> 8, 0);
    }

    if (tid < 16) {
        s_amax[tid] = 0u;
        s_rowsum[tid] = 0;
    }
    __syncthreads();

    uint32_t held[XREG > 0 ? XREG : 1][8];
    if constexpr (FUSED) {
        if constexpr (XREG > 0) {
            const int gpr = p.Kp >> 4;
#pragma unroll
            for (int t = 0; t < XREG; ++t) {
                const int gi = tid + t * kSkThreads;
                if (gi < M * gpr) {
                    const int m = gi / gpr, u = gi - m * gpr;
                    load_x16_bf16<ALIGNED>(p.xb, K, m, 16 * u, held[t]);
                }
            }
            uint32_t mx = 0;
            int mcur = -1;
#pragma unroll
            for (int t = 0; t < XREG; ++t) {
                const int gi = tid + t * kSkThreads;
                if (gi < M * gpr) {
                    const int m = gi / gpr;
                    if (m != mcur && mcur >= 0) {
                        atomicMax(&s_amax[mcur], mx);
                        mx = 0;
                    }
                    mcur = m;
                    mx = max(mx, absmax_bits16(held[t]));
                }
            }
            if (M == 1) {
                mx = wave_max_u32(mx);
                if (lane == 0) atomicMax(&s_amax[0], mx);
            } else if (mcur >= 0) {
                atomicMax(&s_amax[mcur], mx);
            }
        } else {
            // max |x| per token over the whole row, 4 elements per load
            const int64_t groups = K / 4;
            for (int m = 0; m < M; ++m) {
                const uint2* row = reinterpret_cast<const uint2*>(p.xb + (int64_t)m * K);
                uint32_t mx = 0;
                for (int64_t g = tid; g < groups; g += kSkThreads) {
                    const uint2 v = row[g];
                    const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu;
                    mx = max(mx, max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16)));
                }
                mx = wave_max_u32(mx);
                if (lane == 0) atomicMax(&s_amax[m], mx);
            }
        }
        __syncthreads();
    }
    if (tid < M) {
        float a;
        if constexpr (FUSED) {
            float amax = bf16_bits_to_f32(s_amax[tid]);
            amax = amax < 1e-5f ? 1e-5f : amax;
            a = 127.0f / amax;
            if (blockIdx.x == 0 && p.a_out) p.a_out[tid] = a;
        } else {
            a = p.a_scale[tid];
        }
        s_a[tid] = a;
        s_inva[tid] = 1.0f / a;
    }

    for (int ks = 0; ks < p.Kp; ks += p.KS) {
        const int len = min(p.KS, p.Kp - ks);
        const int nch = len >> 8;
        const int64_t stage_off = ks >> 2;
        if (ks > 0) load_batch(cur, wave, nch, stage_off);
        __syncthreads();  // previous stage consumed; s_a visible

        // ---- stage activations [ks, ks+len) of all M rows into LDS, permuted ----
        const int gpr = len >> 4;  // 16-element groups per row
        if (FUSED && XREG > 0) {
#pragma unroll
            for (int t = 0; t < (XREG > 0 ? XREG : 1); ++t) {
                const int gi = tid + t * kSkThreads;
                if (gi < M * gpr) {
                    const int m = gi / gpr, u = gi - m * gpr;
                    uint32_t d[4];
                    quant16(held[t], s_a[m], d);
                    if (blockIdx.x == 0 && p.xq_out) store_codes16<ALIGNED>(p.xq_out, K, m, 16 * u, d);
                    put_group<ALIGNED>(x_lds, KSP, s_rowsum, m, u, d);
                }
            }
        } else {
            for (int gi = tid; gi < M * gpr; gi += kSkThreads) {
                const int m = gi / gpr, u = gi - m * gpr;
                const int k0 = ks + 16 * u;
                uint32_t d[4];
                if constexpr (FUSED) {
                    uint32_t h[8];
                    load_x16_bf16<ALIGNED>(p.xb, K, m, k0, h);
                    quant16(h, s_a[m], d);
                    if (blockIdx.x == 0 && p.xq_out) store_codes16<ALIGNED>(p.xq_out, K, m, k0, d);
                } else {
                    const int8_t* src = p.xq + (int64_t)m * K + k0;
                    if (ALIGNED) {
                        const uint4 v = *reinterpret_cast<const uint4*>(src);
                        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
                    } else {
                        d[0] = d[1] = d[2] = d[3] = 0u;
#pragma unroll
                        for (int j = 0; j < 16; ++j)
                            if (k0 + j < K) d[j >> 2] |= (uint32_t)(uint8_t)src[j] << (8 * (j & 3));
                    }
                }
                put_group<ALIGNED>(x_lds, KSP, s_rowsum, m, u, d);
            }
        }
        __syncthreads();

        // ---- stream the packed weights of this stage: two register batches in flight ----
        for (int c0 = wave; c0 < nch; c0 += kSkWaves * kU) {
            const int c1 = c0 + kSkWaves * kU;
            if (c1 < nch) load_batch(nxt, c1, nch, stage_off);
            compute_batch(cur, c0, nch);
            if (c1 < nch) {
#pragma unroll
                for (int uu = 0; uu < kU; ++uu)
#pragma unroll
                    for (int g = 0; g < NG; ++g) cur[uu][g] = nxt[uu][g];
            }
        }
    }

    // ---- combine the four waves' partials and write the outputs ----
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const v4i t = acc1[g] + (acc4[g] >> 2) + (acc16[g] >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * NG + g) * 4 + r) * 64 + lane] = t[r];
    }
    __syncthreads();
    for (int idx = tid; idx < NG * 256; idx += kSkThreads) {
        const int g = idx >> 8, r = (idx >> 6) & 3, l = idx & 63;
        // 16x16 int32 accumulator layout: lane l, register r -> row 4*(l/16)+r, column l%16
        const int m = 4 * (l >> 4) + r;
        const int n = n0 + 16 * g + (l & 15);
        if (m < M && n < N) {
            int acc = -s_rowsum[m];
#pragma unroll
            for (int w = 0; w < kSkWaves; ++w) acc += red[((w * NG + g) * 4 + r) * 64 + l];
            store_out(p.out, (int64_t)m * N + n, p.out_dtype, acc, p.w_scale[n], s_inva[m]);
        }
    }
}

template <int NG, bool FUSED, int XREG>
hipError_t dispatch_aligned(const SkinnyArgs& a, bool aligned, dim3 grid, size_t lds,
                            hipStream_t stream) {
    if (aligned)
        hipLaunchKernelGGL((skinny_kernel<NG, FUSED, true, XREG>), grid, dim3(kSkThreads), lds,
                           stream, a);
    else
        hipLaunchKernelGGL((skinny_kernel<NG, FUSED, false, XREG>), grid, dim3(kSkThreads), lds,
                           stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const int8_t* xq, const float* a_scale, const uint16_t* x_bf16,
                         const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                         int64_t K, void* out, int out_dtype, int8_t* xq_out, float* a_out,
                         hipStream_t stream) {
    SkinnyArgs a;
    a.xq = xq;
    a.a_scale = a_scale;
    a.xb = x_bf16;
    a.packed = packed;
    a.w_scale = w_scale;
    a.out = out;
    a.xq_out = xq_out;
    a.a_out = a_out;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.Kp = (int)((K + 255) / 256 * 256);
    int ks = ((kSkXBudget / (int)M) - 16) / 256 * 256;
    if (ks < 256) ks = 256;
    a.KS = ks < a.Kp ? ks : a.Kp;
    a.out_dtype = out_dtype;
    constexpr int NG = 1;
    const size_t lds = (size_t)M * (a.KS + 16) + kSkMisc + (size_t)kSkWaves * NG * 4 * 64 * 4;
    const dim3 grid((unsigned)((N + 16 * NG - 1) / (16 * NG)));
    const bool aligned = (K % 256) == 0;
    if (x_bf16) {
        // activations held in registers between the two passes when one K stage covers
        // the row and the block's groups fit two per thread
        const bool hold = a.KS >= a.Kp && (int64_t)M * (a.Kp / 16) <= 2 * kSkThreads;
        if (hold) return dispatch_aligned<NG, true, 2>(a, aligned, grid, lds, stream);
        return dispatch_aligned<NG, true, 0>(a, aligned, grid, lds, stream);
    }
    return dispatch_aligned<NG, false, 0>(a, aligned, grid, lds, stream);
}

}  // namespace bitnet
