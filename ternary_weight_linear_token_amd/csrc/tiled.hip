// tiled.hip -- tiled W2A8 product for prefill-sized M on gfx950 int8 matrix cores.
//
// What it computes ("BitNet 深度实战" (chenxutan.com) §4.4; "BitNet-Triton" (zingnex.cn)
// 技术架构 §1-§2): out[m,n] = acc[m,n] * w_scale[n] / a_scale[m], acc exact in int32,
// from int8 activations xq (M, K) and the packed 2-bit weights (N, K/4).  Prefill is a
// dense contraction, so it runs on v_mfma_i32_32x32x32_i8.
//
// Design:
//  * Block tile BM x BN x 64 (k), four wave64s in a 2 x 2 grid, each a (BM/2) x (BN/2)
//    tile of 32x32 accumulator blocks.  Double-buffered LDS, one barrier per k-step;
//    the next k-step's global loads are in flight while the current one computes.
//  * Operand A (activations) is staged in LDS with every aligned 16-byte group of k
//    transposed as a 4x4 byte matrix (position 4 r + b holds k = 4 b + r), rows padded
//    to 80 bytes so the 128-bit fragment reads do not collide in the LDS banks.
//  * Operand B stays packed in LDS (4x fewer bytes than int8).  A lane reads 8 packed
//    bytes (32 weights) and unpacks them in registers: field i of each byte is masked
//    out and mapped through a v_perm byte lookup to the signed int8 weight (c - 1), so
//    register i, byte b holds weight k = 4 b + i -- the same k-order as operand A.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

namespace {

constexpr int kTdThreads = 256;
constexpr int kBK = 64;           // k per LDS stage
constexpr int kAStride = kBK + 16;  // padded A row in LDS (bytes)
constexpr int kBStride = kBK / 4;   // packed B row in LDS (bytes)

struct TiledArgs {
    const int8_t* xq;
    const float* a_scale;
    const uint8_t* packed;
    const float* w_scale;
    void* out;
    int M, N, K;
    int tiles_n;
    int out_dtype;
};

template <int BM, int BN, bool ALIGNED>
__global__ __launch_bounds__(kTdThreads) void tiled_kernel(TiledArgs p) {
    constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
    constexpr int MB = WM / 32, NB = WN / 32;  // 32x32 blocks per wave
    constexpr int A_VEC = BM * (kBK / 16) / kTdThreads;  // 16-byte A loads per thread
    static_assert(A_VEC >= 1 && BN <= kTdThreads, "tile/thread mismatch");

    __shared__ __align__(16) unsigned char a_lds[2][BM * kAStride];
    __shared__ __align__(16) unsigned char b_lds[2][BN * kBStride];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tile_m = blockIdx.x / p.tiles_n;
    const int tile_n = blockIdx.x - tile_m * p.tiles_n;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int64_t row_bytes = K / 4;
    const int nk = (K + kBK - 1) / kBK;

    uint4 a_reg[A_VEC];
    uint4 b_reg;

    auto load_stage = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < A_VEC; ++j) {
            const int idx = tid + j * kTdThreads;
            const int row = idx >> 2, col = idx & 3;
            const int m = m0 + row;
            const int kk = k0 + 16 * col;
            if (m < M) {
                const int8_t* src = p.xq + (int64_t)m * K + kk;
                if (ALIGNED) {
                    a_reg[j] = *reinterpret_cast<const uint4*>(src);
                } else {
                    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        if (kk + t < K) d[t >> 2] |= (uint32_t)(uint8_t)src[t] << (8 * (t & 3));
                    a_reg[j] = make_uint4(d[0], d[1], d[2], d[3]);
                }
            } else {
                a_reg[j] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        if (tid < BN) {
            const int n = n0 + tid;
            const int64_t off = (int64_t)(k0 / 4);
            if (n < N) {
                const uint8_t* src = p.packed + (int64_t)n * row_bytes + off;
                if (ALIGNED) {
                    b_reg = *reinterpret_cast<const uint4*>(src);
                } else {
                    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        if (off + t < row_bytes) d[t >> 2] |= (uint32_t)src[t] << (8 * (t & 3));
                    b_reg = make_uint4(d[0], d[1], d[2], d[3]);
                }
            } else {
                b_reg = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    auto store_stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < A_VEC; ++j) {
            const int idx = tid + j * kTdThreads;
            const int row = idx >> 2, col = idx & 3;
            const uint32_t d[4] = {a_reg[j].x, a_reg[j].y, a_reg[j].z, a_reg[j].w};
            uint32_t e[4];
            transpose4x4_bytes(d, e);
            *reinterpret_cast<uint4*>(&a_lds[buf][row * kAStride + 16 * col]) =
                make_uint4(e[0], e[1], e[2], e[3]);
        }
        if (tid < BN) *reinterpret_cast<uint4*>(&b_lds[buf][tid * kBStride]) = b_reg;
    };

    v16i acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    load_stage(0);
    store_stage(0);
    __syncthreads();

    const int l32 = lane & 31, q = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage(kt + 1);

#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // 16-weight group j = 2 q + s of this 64-k stage
            v4i A[MB], B[NB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                A[i] = *reinterpret_cast<const v4i*>(
                    &a_lds[buf][(wm * WM + 32 * i + l32) * kAStride + 16 * (2 * q + s)]);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const uint32_t d = *reinterpret_cast<const uint32_t*>(
                    &b_lds[buf][(wn * WN + 32 * j + l32) * kBStride + 4 * (2 * q + s)]);
                B[j][0] = (int)ternary_field_i8<0>(d);
                B[j][1] = (int)ternary_field_i8<1>(d);
                B[j][2] = (int)ternary_field_i8<2>(d);
                B[j][3] = (int)ternary_field_i8<3>(d);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], acc[i][j], 0, 0, 0);
        }

        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // 32x32 int32 accumulator layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
    // column l%32.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int n = n0 + wn * WN + 32 * j + l32;
            const float s = n < N ? p.w_scale[n] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WM + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
                if (m < M && n < N) {
                    const float inv_a = 1.0f / p.a_scale[m];
                    store_out(p.out, (int64_t)m * N + n, p.out_dtype, acc[i][j][r], s, inv_a);
                }
            }
        }
    }
}

template <int BM, int BN>
hipError_t launch_tile(TiledArgs a, bool aligned, hipStream_t stream) {
    const int tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * a.tiles_n));
    if (aligned)
        hipLaunchKernelGGL((tiled_kernel<BM, BN, true>), grid, dim3(kTdThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((tiled_kernel<BM, BN, false>), grid, dim3(kTdThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tiled(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                        const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                        int out_dtype, hipStream_t stream) {
    TiledArgs a;
    a.xq = xq;
    a.a_scale = a_scale;
    a.packed = packed;
    a.w_scale = w_scale;
    a.out = out;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_n = 0;
    a.out_dtype = out_dtype;
    const bool aligned = (K % kBK) == 0;
    return launch_tile<128, 128>(a, aligned, stream);
}

}  // namespace bitnet
