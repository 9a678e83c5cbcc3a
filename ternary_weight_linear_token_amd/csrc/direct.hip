// direct.hip -- W2A8 product for a few tokens (2 <= M <= 16) with the int8 activations
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
//    loaded directly (the activations are at most 16 rows, L2-resident) and put in the
//    same order by a 4x4 byte transpose.  With several tokens this avoids the staging,
//    atomics and barriers the single-token kernel uses to build its LDS copy.
//  * Chunks go in batches of U (1, 2 or 4 by K), two batches in flight: the next batch
//    is requested before the current one is multiplied; chunks past the end read zeros
//    through out-of-range buffer offsets.
//  * int32 partials of the four waves are added through LDS, then rescaled.
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

template <int U>
__global__ __launch_bounds__(64 * kDrWaves) void gemv_direct_kernel(DirectArgs p) {
    __shared__ int red[kDrWaves * 4 * 64];
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
    const __amdgpu_buffer_rsrc_t x_rsrc = dr_rsrc(p.xq, (uint32_t)(M * K));
    const uint32_t w_lane = (uint32_t)(l16 * row_bytes + 16 * q);
    const bool x_row = l16 < M;

    // chunk j of this wave: 16 packed bytes and the four 16-byte activation groups
    auto load = [&](int j, u32x4_d& w, u32x4_d (&X)[4]) {
        const int c = wave + kDrWaves * j;
        const bool live = c < nch;
        w = dr_load16(w_rsrc, live ? w_lane + 64 * c : kDrOOB);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k0 = 256 * c + 64 * q + 16 * s;
            X[s] = dr_load16(x_rsrc, (live && x_row && k0 < K) ? (uint32_t)(l16 * K + k0) : kDrOOB);
        }
    };

    v4i_d acc = {0, 0, 0, 0};
    auto compute = [&](const u32x4_d& w, const u32x4_d (&X)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t d = w[s];
            const v4i_d b = {(int)ternary_field_i8<0>(d), (int)ternary_field_i8<1>(d),
                             (int)ternary_field_i8<2>(d), (int)ternary_field_i8<3>(d)};
            const uint32_t xs[4] = {X[s][0], X[s][1], X[s][2], X[s][3]};
            uint32_t e[4];
            transpose4x4_bytes(xs, e);
            const v4i_d a = {(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
        }
    };
    // batches of U chunks, two in flight: batch t + 1 is requested before batch t is
    // multiplied; batches past the wave's chunks read zeros
    const int nj = (nch - wave + kDrWaves - 1) / kDrWaves;  // chunks of this wave
    u32x4_d wA[U], XA[U][4], wB[U], XB[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) load(u, wA[u], XA[u]);
    for (int j0 = 0; j0 < nj; j0 += 2 * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) load(j0 + U + u, wB[u], XB[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) compute(wA[u], XA[u]);
        if (j0 + U >= nj) break;
#pragma unroll
        for (int u = 0; u < U; ++u) load(j0 + 2 * U + u, wA[u], XA[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) compute(wB[u], XB[u]);
    }

    // 16x16 int32 accumulator layout: lane l, register r -> row 4*(l/16)+r, column l%16
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
    __syncthreads();
    if (tid < 16 * M) {
        const int m = tid >> 4, col = tid & 15;
        if (col < rows) {
            const int l = 16 * (m >> 2) + col, r = m & 3;
            int sum = 0;
#pragma unroll
            for (int w = 0; w < kDrWaves; ++w) sum += red[(w * 4 + r) * 64 + l];
            // 1/a: v_rcp_f32 is within 1 ulp, and the rescale stays within 3 ulp
            const float inv_a = __builtin_amdgcn_rcpf(p.a_scale[m]);
            store_out(p.out, (int64_t)m * N + n0 + col, p.out_dtype, sum, ws_n, inv_a);
        }
    }
}

}  // namespace

hipError_t launch_gemv_direct(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                              const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                              int out_dtype, hipStream_t stream) {
    if (M < 1 || M > 16 || N < 1 || K % 64 != 0 || M * K > INT32_MAX) return hipErrorInvalidValue;
    DirectArgs a;
    a.xq = xq;
    a.a_scale = a_scale;
    a.packed = packed;
    a.w_scale = w_scale;
    a.out = out;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.out_dtype = out_dtype;
    const dim3 grid((unsigned)((N + 15) / 16)), blk(64 * kDrWaves);
    const int nj = ((K + 255) / 256 + kDrWaves - 1) / kDrWaves;  // chunks per wave
    if (nj <= 2)
        hipLaunchKernelGGL(gemv_direct_kernel<1>, grid, blk, 0, stream, a);
    else if (nj <= 8)
        hipLaunchKernelGGL(gemv_direct_kernel<2>, grid, blk, 0, stream, a);
    else
        hipLaunchKernelGGL(gemv_direct_kernel<4>, grid, blk, 0, stream, a);
    return hipGetLastError();
}

}  // namespace bitnet
