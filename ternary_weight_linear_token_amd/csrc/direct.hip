// direct.hip -- W2A8 product for a few tokens (2 <= M <= 32) with the int8 activations
// read straight from memory into matrix-core operands (no LDS staging).
//
// What it computes ("BitNet 深度实战" §4.4; "BitNet-Triton" 技术架构 §1-§2): out[m,n] =
// acc[m,n] * w_scale[n] / a_scale[m] with acc = sum_k xq[m,k] * w[n,k] exact in int32.
//
// Design (same block shape as the single-token decode kernel; what differs is where the
// activations come from):
//  * A block (4 wave64s) owns 16 output rows and all of K; the waves take interleaved
//    256-weight chunks; a lane loads 16 packed bytes (64 weights) of one row per chunk.
//  * Each packed dword (16 weights) is one v_mfma_i32_16x16x64_i8 operand B: field i of
//    its four bytes, mapped by a v_perm lookup to the signed weight, fills register i,
//    so byte b of register i holds k = 4 b + i.
//  * Operand A (rows = tokens) is the lane's 16 int8 activations of the same 16 k,
//    loaded directly (the activations are at most 32 rows, L2-resident) and put in the
//    same order by a 4x4 byte transpose.  With several tokens this avoids the staging,
//    atomics and barriers the single-token kernel uses to build its LDS copy.  17 to 32
//    tokens take two 16-token tiles: each weight operand feeds two products, one per
//    tile (int8 input only).
//  * Chunks go in batches of U (1, 2 or 4 by K), two batches in flight: the next batch
//    is requested before the current one is multiplied; chunks past the end read zeros
//    through out-of-range buffer offsets.
//  * int32 partials of the four waves are added through LDS, then rescaled.
//  * Fused variant (bf16 activations): the block first finds every token's max |x| (wave
//    w scans rows w, w + 4, ... with batched loads, one barrier; the first batch of
//    weights is already on its way), then each lane quantizes
//    its 16 activations per operand in registers (fp32 multiply, round half to even by
//    the 1.5 * 2^23 addition), already in the transposed order.  The first block also
//    writes the codes and scales when asked.
//  * K must be a multiple of 64 (16-byte aligned rows); other K use the staged kernel.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

namespace {

typedef int v4i_d __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_d __attribute__((ext_vector_type(4)));

constexpr int kDrWaves = 4;
constexpr uint32_t kDrOOB = 0x80000000u;  // buffer offset past every resource: reads 0

struct DirectArgs {
    const int8_t* xq;
    const float* a_scale;
    const uint16_t* xb;  // bf16 activations (fused variant)
    int8_t* xq_out;      // optional copies (fused variant, first block)
    float* a_out;
    const uint8_t* packed;
    const float* w_scale;
    void* out;
    int M, N, K;
    int out_dtype;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dr_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4_d dr_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_d, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int U, bool FUSED, int MT>
__global__ __launch_bounds__(64 * kDrWaves) void gemv_direct_kernel(DirectArgs p) {
    static_assert(MT == 1 || (MT == 2 && !FUSED), "two token tiles on int8 input only");
    __shared__ int red[kDrWaves * MT * 4 * 64];
    __shared__ uint32_t s_max[kDrWaves][16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = p.M, N = p.N, K = p.K;
    const int row_bytes = K / 4;
    const int n0 = blockIdx.x * 16;
    const int rows = min(16, N - n0);
    const int l16 = lane & 15, q = lane >> 4;
    const int nch = (K + 255) / 256;

    const float ws_n = p.w_scale[n0 + min(l16, rows - 1)];  // used by threads tid < 16 M
    const __amdgpu_buffer_rsrc_t w_rsrc =
        dr_rsrc(p.packed + (int64_t)n0 * row_bytes, (uint32_t)(rows * row_bytes));
    const __amdgpu_buffer_rsrc_t x_rsrc =
        FUSED ? dr_rsrc(p.xb, (uint32_t)(M * K * 2)) : dr_rsrc(p.xq, (uint32_t)(M * K));
    const uint32_t w_lane = (uint32_t)(l16 * row_bytes + 16 * q);
    const bool x_row = l16 < M;   // this lane's token of the first tile
    constexpr int XW = FUSED ? 2 : 1;  // 16-byte loads per 16-activation group

    // chunk j of this wave: 16 packed bytes and, per token tile, the four 16-activation
    // groups
    auto load = [&](int j, u32x4_d& w, u32x4_d (&X)[MT][4][XW]) {
        const int c = wave + kDrWaves * j;
        const bool live = c < nch;
        w = dr_load16(w_rsrc, live ? w_lane + 64 * c : kDrOOB);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k0 = 256 * c + 64 * q + 16 * s;
                const int mrow = 16 * t + l16;
                const bool ok = live && mrow < M && k0 < K;
#pragma unroll
                for (int h = 0; h < XW; ++h)
                    X[t][s][h] = dr_load16(x_rsrc, ok ? (uint32_t)((mrow * K + k0) * XW + 16 * h) : kDrOOB);
            }
    };

    // batches of U chunks, two in flight: batch t + 1 is requested before batch t is
    // multiplied; batches past the wave's chunks read zeros.  The first batch is requested
    // before the fused scan, so its trip from memory overlaps the scan.
    const int nj = (nch - wave + kDrWaves - 1) / kDrWaves;  // chunks of this wave
    u32x4_d wA[U], XA[U][MT][4][XW], wB[U], XB[U][MT][4][XW];
#pragma unroll
    for (int u = 0; u < U; ++u) load(u, wA[u], XA[u]);

    // fused: every token's scale 127 / max|x| from a scan of its row by one wave
    float a_row = 0.f;  // scale of this lane's token (fused)
    if constexpr (FUSED) {
        scan_absmax_rows<true>(x_rsrc, M, K, wave, kDrWaves, s_max[wave]);
        __syncthreads();
        const int mr = x_row ? l16 : 0;
        float amax = bf16_bits_to_f32(s_max[mr % kDrWaves][mr]);  // written by wave mr % 4
        amax = amax < 1e-5f ? 1e-5f : amax;
        a_row = 127.0f / amax;
        if (blockIdx.x == 0 && p.a_out && lane < M && tid < 64) p.a_out[lane] = a_row;
    }

    v4i_d acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4i_d{0, 0, 0, 0};
    auto compute = [&](int j, const u32x4_d& w, const u32x4_d (&Xt)[MT][4][XW]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t d = w[s];
            const v4i_d b = {(int)ternary_field_i8<0>(d), (int)ternary_field_i8<1>(d),
                             (int)ternary_field_i8<2>(d), (int)ternary_field_i8<3>(d)};
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const u32x4_d (&X)[4][XW] = Xt[t];
                uint32_t e[4];
                if constexpr (FUSED) {
                    const uint32_t h[8] = {X[s][0][0], X[s][0][1], X[s][0][2], X[s][0][3],
                                           X[s][1][0], X[s][1][1], X[s][1][2], X[s][1][3]};
                    quant16_t(h, a_row, e);
                    const int k0 = 256 * (wave + kDrWaves * j) + 64 * q + 16 * s;
                    if (blockIdx.x == 0 && p.xq_out && x_row && k0 < K) {
                        uint32_t dd[4];
                        untranspose(e, dd);
                        store_codes16<true>(p.xq_out, K, l16, k0, dd);
                    }
                } else {
                    const uint32_t xs[4] = {X[s][0][0], X[s][0][1], X[s][0][2], X[s][0][3]};
                    transpose4x4_bytes(xs, e);
                }
                const v4i_d a = {(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
            }
        }
    };
    for (int j0 = 0; j0 < nj; j0 += 2 * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) load(j0 + U + u, wB[u], XB[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j0 + u < nj) compute(j0 + u, wA[u], XA[u]);
        if (j0 + U >= nj) break;
#pragma unroll
        for (int u = 0; u < U; ++u) load(j0 + 2 * U + u, wA[u], XA[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j0 + U + u < nj) compute(j0 + U + u, wB[u], XB[u]);
    }

    // 16x16 int32 accumulator layout: lane l, register r -> row 4*(l/16)+r, column l%16
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * MT + t) * 4 + r) * 64 + lane] = acc[t][r];
    __syncthreads();
    for (int idx = tid; idx < 16 * M; idx += 64 * kDrWaves) {
        const int m = idx >> 4, col = idx & 15;
        if (col < rows) {
            const int t = m >> 4, mm = m & 15;
            const int l = 16 * (mm >> 2) + col, r = mm & 3;
            int sum = 0;
#pragma unroll
            for (int w = 0; w < kDrWaves; ++w) sum += red[((w * MT + t) * 4 + r) * 64 + l];
            // 1/a: v_rcp_f32 is within 1 ulp, and the rescale stays within 3 ulp
            float a_m;
            if constexpr (FUSED) {
                float amax = bf16_bits_to_f32(s_max[m % kDrWaves][m]);
                amax = amax < 1e-5f ? 1e-5f : amax;
                a_m = 127.0f / amax;
            } else {
                a_m = p.a_scale[m];
            }
            const float inv_a = __builtin_amdgcn_rcpf(a_m);
            store_out(p.out, (int64_t)m * N + n0 + col, p.out_dtype, sum, ws_n, inv_a);
        }
    }
}

}  // namespace

hipError_t launch_gemv_direct(const int8_t* xq, const float* a_scale, const uint16_t* x_bf16,
                              const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                              int64_t K, void* out, int out_dtype, int8_t* xq_out, float* a_out,
                              hipStream_t stream) {
    const bool fused = x_bf16 != nullptr;
    if (M < 1 || M > (fused ? 16 : 32) || N < 1 || K % 64 != 0 || M * K * 2 > INT32_MAX)
        return hipErrorInvalidValue;
    DirectArgs a;
    a.xq = xq;
    a.a_scale = a_scale;
    a.xb = x_bf16;
    a.xq_out = xq_out;
    a.a_out = a_out;
    a.packed = packed;
    a.w_scale = w_scale;
    a.out = out;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.out_dtype = out_dtype;
    const dim3 grid((unsigned)((N + 15) / 16)), blk(64 * kDrWaves);
    const int nj = ((K + 255) / 256 + kDrWaves - 1) / kDrWaves;  // chunks per wave
    if (M > 16) {
        // two token tiles: at most two chunks per batch (their activations double the
        // registers a batch holds)
        if (nj <= 2) hipLaunchKernelGGL((gemv_direct_kernel<1, false, 2>), grid, blk, 0, stream, a);
        else hipLaunchKernelGGL((gemv_direct_kernel<2, false, 2>), grid, blk, 0, stream, a);
    } else if (nj <= 2) {
        if (fused) hipLaunchKernelGGL((gemv_direct_kernel<1, true, 1>), grid, blk, 0, stream, a);
        else hipLaunchKernelGGL((gemv_direct_kernel<1, false, 1>), grid, blk, 0, stream, a);
    } else if (nj <= 8) {
        if (fused) hipLaunchKernelGGL((gemv_direct_kernel<2, true, 1>), grid, blk, 0, stream, a);
        else hipLaunchKernelGGL((gemv_direct_kernel<2, false, 1>), grid, blk, 0, stream, a);
    } else {
        if (fused) hipLaunchKernelGGL((gemv_direct_kernel<4, true, 1>), grid, blk, 0, stream, a);
        else hipLaunchKernelGGL((gemv_direct_kernel<4, false, 1>), grid, blk, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace bitnet
