// tiled.hip -- tiled W2A8 product for prefill-sized M on gfx950 int8 matrix cores.
//
// What it computes ("BitNet 深度实战" (chenxutan.com) §4.4; "BitNet-Triton" (zingnex.cn)
// 技术架构 §1-§2): out[m,n] = acc[m,n] * w_scale[n] / a_scale[m], acc exact in int32,
// from int8 activations xq (M, K) and the packed 2-bit weights (N, K/4).  Prefill is a
// dense contraction, so it runs on v_mfma_i32_32x32x32_i8.
//
// Design:
//  * Block tile BM x BN, k-stage BK = 64 or 128, four wave64s in a (4/WGN) x WGN grid, each a
//    tile of 32x32 int32 accumulator blocks.  Tall wave tiles amortize the weight
//    unpack over more rows: the 256x256 blocks use a 1 x 4 grid (256 x 64 per wave,
//    half the unpack of a 2 x 2 grid for twice the activation fragment reads).
//  * Loads are raw buffer loads through per-block descriptors whose range ends at the
//    last valid row: rows past M or N read as zero without any branch, and per-stage
//    offsets are scalar, so address arithmetic stays off the vector ALU.
//  * Software pipeline: D register sets hold the loads of the next D stages; stages past
//    the end read zeros through out-of-range buffer offsets, so every step issues the
//    same loads and products and only the oldest set is waited for.  Within a step the
//    matrix products are interleaved (scheduling-group hints) with the next step's
//    weight unpack, loads and activation transpose, so the vector ALU work overlaps the
//    matrix cores.
//  * Operand A (activations) goes through LDS (double-buffered, one barrier per stage)
//    with every aligned 16-byte k-group transposed as a 4x4 byte matrix (position
//    4 r + b holds k = 4 b + r); rows padded by 16 bytes (80 or 144) so the 128-bit
//    fragment reads are conflict-free.
//  * Operand B (packed weights, 4x fewer bytes than int8) is loaded straight into the
//    registers of the waves that use it, 8 or 16 bytes (two or four 16-weight groups)
//    per lane per 32 columns and stage, and unpacked there: field i of each byte is masked out and mapped by a
//    v_perm byte lookup to the signed weight (c - 1), so register i, byte b holds weight
//    k = 4 b + i -- the same k-order as operand A.
//  * Small grids split K inside the block: 128x128 blocks of two four-wave k-groups and
//    64x128 blocks of four (alternate k-stages, accumulators combined through LDS), so
//    each SIMD interleaves two or four waves.  Across blocks, K is split only through a
//    second launch: units write int32 partial tiles to the caller's workspace and the
//    reduce kernel adds them (handing partials between blocks inside one launch needs
//    device-scope release/acquire across the XCDs' L2s, which costs more than it saves).
//  * Full-chip grids use 128x128 blocks of one k-group (waves 1 x 4): two blocks per CU,
//    so each SIMD interleaves two waves of different tiles.  The tile shape, k-stage and
//    K slices of a launch are the ones with the least estimated time (plan_tiles).
//  * Blocks are mapped to work units XCD by XCD (dispatch assigns consecutive blocks to
//    the 8 XCDs in turn), and units are ordered in panels of tile rows, so an XCD's L2
//    holds a few activation row panels and a few weight column panels.
//  * Grouped launches: up to BITNET_MAX_GROUPS weight matrices that read the same
//    activations (q, k, v; gate, up) share one grid; a block finds its matrix by scalar
//    compares of its work unit against the groups' first units.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

namespace {

constexpr int kTdThreads = 256;
constexpr int kXcds = 8;

constexpr int kTdGroups = BITNET_MAX_GROUPS;

struct TiledArgs {
    const int8_t* xq;
    const float* a_scale;
    // weight matrices that share the activations: group g owns the work units
    // first[g] .. first[g + 1] - 1 (row panel major, tiles_n[g] tiles per panel)
    int groups;
    int first[kTdGroups];
    int g_N[kTdGroups];
    int g_tiles_n[kTdGroups];
    const uint8_t* g_packed[kTdGroups];
    const float* g_wscale[kTdGroups];
    void* g_out[kTdGroups];
    int M, K;
    int units;       // tiles of all groups, times ksplit
    int units_per_xcd;
    // split of K across blocks (one weight matrix only): unit u takes k-stages
    // [s * split_stages, (s + 1) * split_stages) of tile u - s * (units / ksplit), s =
    // u / (units / ksplit), and writes its int32 partial sums to g_out[0] + s * split_stride
    // (the reduce kernel adds the ksplit partials and rescales)
    int ksplit;
    int split_stages;
    int64_t split_stride;
    int gm;          // tile rows per panel of the unit order (see the kernel)
    int out_dtype;
};

template <int BM, int BN, int D, int G, int WGN, int BK, bool ALIGNED, int DT>
__global__ __launch_bounds__(kTdThreads * G) void tiled_kernel(TiledArgs p) {
    static_assert(BK == 64 || BK == 128, "k per LDS stage");
    constexpr int KS = BK / 32;          // 32-k matrix products per stage and column block
    constexpr int kAStride = BK + 16;    // padded A row in LDS (bytes)
    constexpr int APR = BK / 16;         // 16-byte A pieces per row and stage
    constexpr int WGM = 4 / WGN;                 // waves along M and N
    constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
    constexpr int MB = WM / 32, NB = WN / 32;  // 32x32 blocks per wave
    constexpr int AV = BM * APR / kTdThreads;  // 16-byte A loads per thread per stage
    constexpr int BROWS_PER_THREAD = (BN + kTdThreads - 1) / kTdThreads;
    static_assert(AV >= 1, "tile/thread mismatch");
    (void)BROWS_PER_THREAD;

    static_assert(G == 1 || G == 2 || G == 4, "k-groups per block");
    static_assert(G == 1 || MB % 2 == 0, "k-group combine splits the accumulator rows");
    // LDS: the groups' double-buffered activation stages, reused after the k loop for the
    // combine of the groups' accumulators and the per-wave epilogue scratch
    constexpr int kStageBytes = G * 2 * BM * kAStride;
    constexpr int kGroupAccBytes = 4 * MB * NB * 16 * 64 * 4;  // one group's accumulators
    constexpr int kRedBytes = G == 4 ? 4 * kGroupAccBytes : (G == 2 ? kGroupAccBytes / 2 : 0);
    constexpr int kEpiBytes = (G == 1 ? 1 : 2) * 4 * 32 * 36 * 4;
    constexpr int kLdsBytes = kStageBytes > kRedBytes ? (kStageBytes > kEpiBytes ? kStageBytes : kEpiBytes)
                                                      : (kRedBytes > kEpiBytes ? kRedBytes : kEpiBytes);
    __shared__ __align__(16) unsigned char smem[kLdsBytes];
    __shared__ float s_inva[BM];

    // ---- work unit of this block (XCD-contiguous) ----
    const int xcd = blockIdx.x % kXcds;
    const int unit_all = xcd * p.units_per_xcd + blockIdx.x / kXcds;
    if (unit_all >= p.units) return;
    // split of K: the unit's slice s and its unit within the slice (scalar arithmetic)
    const int per_split = p.units / p.ksplit;
    const int split = unit_all / per_split;
    const int unit = unit_all - split * per_split;
    // the unit's weight matrix: the last group whose first unit is at most `unit`
    // (scalar compares and selects on the kernel arguments)
    int first = p.first[0], N = p.g_N[0], tiles_n = p.g_tiles_n[0];
    const uint8_t* packed = p.g_packed[0];
    const float* w_scale = p.g_wscale[0];
    void* out = p.g_out[0];
#pragma unroll
    for (int i = 1; i < kTdGroups; ++i) {
        if (i < p.groups && unit >= p.first[i]) {
            first = p.first[i];
            N = p.g_N[i];
            tiles_n = p.g_tiles_n[i];
            packed = p.g_packed[i];
            w_scale = p.g_wscale[i];
            out = p.g_out[i];
        }
    }
    if (DT == 2 && p.ksplit > 1) out = static_cast<int*>(out) + split * p.split_stride;
    // A group's tiles are ordered in panels of gm tile rows, column by column inside a
    // panel, so the run of consecutive units one XCD takes is a block of about gm x
    // (run / gm) tiles: its L2 holds gm activation row panels and run / gm weight column
    // panels instead of one row panel and every column panel.
    const int tile = unit - first;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int panel = tile / (p.gm * tiles_n);
    const int rem = tile - panel * p.gm * tiles_n;
    const int pm = min(p.gm, tiles_m - panel * p.gm);  // rows of this (possibly last) panel
    const int tile_m = panel * p.gm + rem % pm;
    const int tile_n = rem / pm;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // G groups of four waves; group g takes the k-stages g, g + G, g + 2G, ... of the
    // block's range with its own LDS buffers and registers; their accumulators are
    // combined through LDS at the end.  With G = 2 (4) every SIMD holds two (four) waves
    // whose memory, LDS and matrix-core phases interleave.
    // group and wave indices are uniform per wave; readfirstlane tells the compiler so,
    // which keeps the per-stage buffer offsets in scalar registers
    const int g = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8);  // 256 threads per group
    const int tid = threadIdx.x & 255, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    unsigned char (*a_lds)[BM * kAStride] =
        reinterpret_cast<unsigned char (*)[BM * kAStride]>(smem + g * 2 * BM * kAStride);
    const int M = p.M, K = p.K;
    const int64_t row_bytes = K / 4;
    // the k-stages of this unit: all of K, or one slice of it when K is split
    const int nk_all = (K + BK - 1) / BK;
    const int k_first = split * p.split_stages;
    const int nk = min(nk_all, k_first + p.split_stages);

    for (int i = (int)threadIdx.x; i < BM; i += kTdThreads * G) {
        const int m = m0 + i;
        s_inva[i] = m < M ? 1.0f / p.a_scale[m] : 0.0f;
    }

    // Buffer descriptors of this block's A row panel and B column panel; their ranges
    // stop at the last valid row, so loads past M or N return zeros.
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(p.xq) + (int64_t)m0 * K, (short)0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed) + (int64_t)n0 * row_bytes, (short)0,
        (int)(rows_b * row_bytes), 0x00020000);

    // A: thread tid loads AV 16-byte pieces per stage (rows idx/4, k-groups idx%4).
    // B: lane (l32, q) of wave (wm, wn) loads, for each of its NB column blocks, the 8
    //    packed bytes k/4 = 8q .. 8q+7 of row n0 + wn*WN + 32 j + l32.
    const int l32 = lane & 31, q = lane >> 5;
    int a_voff[AV];
#pragma unroll
    for (int j = 0; j < AV; ++j) {
        const int idx = tid + j * kTdThreads;
        a_voff[j] = (idx / APR) * K + 16 * (idx % APR);
    }
    int b_voff[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) b_voff[j] = (wn * WN + 32 * j + l32) * (int)row_bytes + (BK / 8) * q;

    static_assert(D == 2 || D == 4, "pipeline depth");
    // B registers of one stage: per column block, KS packed dwords (16 weights each)
    using BVec = std::conditional_t<KS == 2, uint2, uint4>;
    uint4 a_reg[D][AV];
    BVec b_reg[D][NB];

    // Stage kt of K; a stage past the end (kt >= nk) reads as zeros: its scalar offset
    // lies beyond both descriptors' ranges (the 32-bit sum with any in-range voffset
    // cannot wrap), so the products it feeds add nothing.
    auto load_stage = [&](uint4 (&ar)[AV], BVec (&br)[NB], int kt) {
        const bool live = kt < nk;
        const int k0 = live ? kt * BK : 0;
        if (ALIGNED) {
            const uint32_t sa = live ? (uint32_t)k0 : 0x80000000u;
            const uint32_t sb = live ? (uint32_t)(k0 / 4) : 0x80000000u;
#pragma unroll
            for (int j = 0; j < AV; ++j)
                ar[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff[j], sa, 0));
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if constexpr (KS == 2)
                    br[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(b_rsrc, b_voff[j], sb, 0));
                else
                    br[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_voff[j], sb, 0));
            }
        } else if (!live) {
#pragma unroll
            for (int j = 0; j < AV; ++j) ar[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int j = 0; j < NB; ++j) br[j] = BVec{};
        } else {
            // K not a multiple of the stage: byte loads, zero past the end of each row
#pragma unroll
            for (int j = 0; j < AV; ++j) {
                const int idx = tid + j * kTdThreads;
                const int row = idx / APR, kk = k0 + 16 * (idx % APR);
                uint32_t d[4] = {0u, 0u, 0u, 0u};
                if (row < rows_a) {
                    const int8_t* src = p.xq + (int64_t)(m0 + row) * K + kk;
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        if (kk + t < K) d[t >> 2] |= (uint32_t)(uint8_t)src[t] << (8 * (t & 3));
                }
                ar[j] = make_uint4(d[0], d[1], d[2], d[3]);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int row = wn * WN + 32 * j + l32;
                const int64_t off = k0 / 4 + (BK / 8) * q;
                uint32_t d[KS];
#pragma unroll
                for (int t = 0; t < KS; ++t) d[t] = 0u;
                if (row < rows_b) {
                    const uint8_t* src = packed + (int64_t)(n0 + row) * row_bytes + off;
#pragma unroll
                    for (int t = 0; t < BK / 8; ++t)
                        if (off + t < row_bytes) d[t >> 2] |= (uint32_t)src[t] << (8 * (t & 3));
                }
                if constexpr (KS == 2)
                    br[j] = make_uint2(d[0], d[1]);
                else
                    br[j] = make_uint4(d[0], d[1], d[2], d[3]);
            }
        }
    };

    auto store_stage = [&](const uint4 (&ar)[AV], int buf) {
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int idx = tid + j * kTdThreads;
            const int row = idx / APR, col = idx % APR;
            const uint32_t d[4] = {ar[j].x, ar[j].y, ar[j].z, ar[j].w};
            uint32_t e[4];
            transpose4x4_bytes(d, e);
            *reinterpret_cast<uint4*>(&a_lds[buf][row * kAStride + 16 * col]) =
                make_uint4(e[0], e[1], e[2], e[3]);
        }
    };

    v16i acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // Weight operands of one stage, unpacked: B[s][j] feeds k-substep s, column block j.
    // Lane group q owns the 16-weight groups 2q + s of the 64-k stage.
    auto unpack_b = [&](const BVec (&br)[NB], v4i (&Bu)[KS][NB]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                uint32_t d;
                if constexpr (KS == 2)
                    d = s == 0 ? br[j].x : br[j].y;
                else
                    d = s == 0 ? br[j].x : (s == 1 ? br[j].y : (s == 2 ? br[j].z : br[j].w));
                Bu[s][j][0] = (int)ternary_field_i8<0>(d);
                Bu[s][j][1] = (int)ternary_field_i8<1>(d);
                Bu[s][j][2] = (int)ternary_field_i8<2>(d);
                Bu[s][j][3] = (int)ternary_field_i8<3>(d);
            }
    };
    auto read_a = [&](int buf, v4i (&A)[KS][MB]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int i = 0; i < MB; ++i)
                A[s][i] = *reinterpret_cast<const v4i*>(
                    &a_lds[buf][(wm * WM + 32 * i + l32) * kAStride + 16 * (KS * q + s)]);
    };
    auto mfma_stage = [&](const v4i (&A)[KS][MB], const v4i (&Bu)[KS][NB]) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[s][i], Bu[s][j], acc[i][j], 0, 0, 0);
    };

    // D register sets hold the loads of the next D stages.  Step t: read stage t's A
    // fragments from LDS buffer t%2, refill register set t%D with the loads of stage t+D,
    // unpack stage t+1's weights (already in registers), move stage t+1's A into the
    // other LDS buffer (last read before the previous barrier) and issue stage t's
    // matrix products; one barrier per step.  Every full group of D steps issues the same
    // loads, so the compiler waits only for the oldest set; the loop runs whole groups
    // (the accumulators keep one live range) and the remaining < D steps run in a tail
    // without new loads.
    // Group g's stages are g, g + G, g + 2G, ...; every group runs nsteps steps, and a
    // step past the group's last stage multiplies zeros (see load_stage), so the matrix
    // products are unconditional and each step is one scheduling region.
    const int nsteps = (nk - k_first + G - 1) / G;
    auto stage_of = [&](int i) { return k_first + g + G * i; };
    // One step: the A fragments of this step are read first; then this step's matrix
    // products are interleaved with the next step's weight unpack, the loads D steps
    // ahead and the transposed store of the next step's activations, so the vector ALU
    // and LDS work hides under the matrix cores.
    constexpr int kMf = KS * MB * NB;                              // products per step
    constexpr int kVa = (KS * NB * 11 + AV * 8 + kMf - 1) / kMf;   // VALU per product
    auto schedule_step = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, KS * MB, 0);  // A fragment reads
        __builtin_amdgcn_sched_group_barrier(0x020, AV + NB, 0);  // loads D steps ahead
#pragma unroll
        for (int i = 0; i < kMf; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one product
            __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);  // unpack / transpose
        }
        __builtin_amdgcn_sched_group_barrier(0x200, AV, 0);       // next A into LDS
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load_stage(a_reg[d], b_reg[d], stage_of(d));
    store_stage(a_reg[0], 0);
    v4i Bu[2][KS][NB];
    unpack_b(b_reg[0], Bu[0]);
    __syncthreads();
    int it = 0;
    for (; it + D <= nsteps; it += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            v4i A[KS][MB];
            read_a(u & 1, A);
            load_stage(a_reg[u], b_reg[u], stage_of(it + u + D));
            unpack_b(b_reg[(u + 1) % D], Bu[(u + 1) & 1]);
            store_stage(a_reg[(u + 1) % D], (u + 1) & 1);
            mfma_stage(A, Bu[u & 1]);
            schedule_step();
            __syncthreads();
        }
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u) {
        if (it + u >= nsteps) break;
        v4i A[KS][MB];
        read_a(u & 1, A);
        if (it + u + 1 < nsteps) {
            unpack_b(b_reg[u + 1], Bu[(u + 1) & 1]);
            store_stage(a_reg[u + 1], (u + 1) & 1);
        }
        mfma_stage(A, Bu[u & 1]);
        __syncthreads();
    }

    // ---- epilogue: each 32x32 accumulator block goes through a per-wave LDS scratch
    // (32 rows x 36 ints) so that a lane ends up with 16 consecutive columns of one row
    // and stores them with 16-byte writes.  32x32 int32 accumulator layout: lane l,
    // register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32. ----
    constexpr int kEpiStride = 36;
    int* scratch = reinterpret_cast<int*>(smem) + (g * 4 + wave) * (32 * kEpiStride);
    const int erow = lane >> 1, ecol = (lane & 1) * 16;
    // 16-byte stores need 16-byte aligned row starts: N % 8 == 0 for bf16, N % 4 == 0
    // for 4-byte outputs (column offsets are multiples of 16)
    const bool vec_ok = (N % (DT == 1 ? 8 : 4)) == 0;

    auto emit_block = [&](int i, int j, const int (&v)[16]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) scratch[(8 * (r >> 2) + 4 * q + (r & 3)) * kEpiStride + l32] = v[r];
        int row[16];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int4 x = *reinterpret_cast<const int4*>(&scratch[erow * kEpiStride + ecol + 4 * t]);
            row[4 * t] = x.x; row[4 * t + 1] = x.y; row[4 * t + 2] = x.z; row[4 * t + 3] = x.w;
        }
        const int ml = wm * WM + 32 * i + erow;
        const int m = m0 + ml;
        const int nb = n0 + wn * WN + 32 * j + ecol;
        if (m < M) {
            const float inv_a = s_inva[ml];
            const int64_t o = (int64_t)m * N + nb;
            if (vec_ok && nb + 16 <= N) {
                if (DT == 2) {
                    int4* dst = reinterpret_cast<int4*>(static_cast<int*>(out) + o);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        dst[t] = make_int4(row[4 * t], row[4 * t + 1], row[4 * t + 2], row[4 * t + 3]);
                } else {
                    float f[16];
                    const float4* ws = reinterpret_cast<const float4*>(w_scale + nb);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float4 sc = ws[t];
                        f[4 * t] = ((float)row[4 * t] * sc.x) * inv_a;
                        f[4 * t + 1] = ((float)row[4 * t + 1] * sc.y) * inv_a;
                        f[4 * t + 2] = ((float)row[4 * t + 2] * sc.z) * inv_a;
                        f[4 * t + 3] = ((float)row[4 * t + 3] * sc.w) * inv_a;
                    }
                    if (DT == 0) {
                        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + o);
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            dst[t] = make_float4(f[4 * t], f[4 * t + 1], f[4 * t + 2], f[4 * t + 3]);
                    } else {
                        uint32_t h[8];
#pragma unroll
                        for (int t = 0; t < 8; ++t) h[t] = f32x2_to_bf16x2_rne(f[2 * t], f[2 * t + 1]);
                        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o);
                        dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
                        dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    if (nb + t < N) store_out(out, o + t, DT, row[t], w_scale[nb + t], inv_a);
            }
        }
        // keep consecutive blocks from being interleaved (bounds the live registers)
        __builtin_amdgcn_sched_barrier(0);
    };

    // every k-stage ended with a barrier: the A buffers are free for the epilogue scratch
    if constexpr (G == 4) {
        // ---- one pass: every group's partial sums go to LDS, then group g adds up, over
        // the four groups, the quarter of the tile it owns -- accumulator block g / 2,
        // registers 8 (g % 2) .. +7, i.e. rows 16 (g % 2) .. +15 of that block -- and
        // writes it straight from the accumulator layout (lane l: column l % 32) ----
        static_assert(MB == 2 && NB == 1, "one accumulator quarter per k-group");
        int* part = reinterpret_cast<int*>(smem);
        auto slot = [&](int gg, int i, int r) {
            return (((gg * 4 + wave) * MB + i) * 16 + r) * 64 + lane;
        };
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[slot(g, i, r)] = acc[i][0][r];
        __syncthreads();
        const int io = g >> 1, ho = g & 1;
        int v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            int sum = 0;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) sum += part[slot(gg, io, 8 * ho + t)];
            v[t] = sum;
        }
        const int nb = n0 + wn * WN + l32;
        if (nb < N) {
            const float ws = DT == 2 ? 0.0f : w_scale[nb];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int r = 8 * ho + t;
                const int ml = wm * WM + 32 * io + 8 * (r >> 2) + 4 * q + (r & 3);
                if (m0 + ml < M)
                    store_out(out, (int64_t)(m0 + ml) * N + nb, DT, v[t], ws, s_inva[ml]);
            }
        }
        return;
    }
    if constexpr (G == 2) {
        // ---- combine groups 0 and 1: group 0 ends up owning accumulator rows blocks
        // i < MB/2, group 1 the others; each half goes through LDS in its own phase ----
        constexpr int H = MB / 2;
        int* red = reinterpret_cast<int*>(smem);
        auto slot = [&](int ih, int j, int r) { return (((wave * H + ih) * NB + j) * 16 + r) * 64 + lane; };
        if (g == 1) {
#pragma unroll
            for (int ih = 0; ih < H; ++ih)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[slot(ih, j, r)] = acc[ih][j][r];
        }
        __syncthreads();
        if (g == 0) {
#pragma unroll
            for (int ih = 0; ih < H; ++ih)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[ih][j][r] += red[slot(ih, j, r)];
        }
        __syncthreads();
        if (g == 0) {
#pragma unroll
            for (int ih = 0; ih < H; ++ih)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[slot(ih, j, r)] = acc[H + ih][j][r];
        }
        __syncthreads();
        if (g == 1) {
#pragma unroll
            for (int ih = 0; ih < H; ++ih)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[H + ih][j][r] += red[slot(ih, j, r)];
        }
        __syncthreads();  // red is reused as epilogue scratch below
#pragma unroll
        for (int ih = 0; ih < H; ++ih)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                int v[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = g == 0 ? acc[ih][j][r] : acc[H + ih][j][r];
                emit_block(g == 0 ? ih : H + ih, j, v);
            }
        return;
    }

#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            int v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = acc[i][j][r];
            emit_block(i, j, v);
        }
}

struct TilePlan {
    int bm, bn, g;     // block tile and k-groups per block
    int bk;            // k per LDS stage
    int ksplit;        // slices of K across blocks (1: none)
    int split_stages;  // k-stages per slice
};

// Compute units of the current device, queried once per device (atomics: concurrent
// first calls at worst repeat the query).
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Optional override for tuning: BITNET_TILED_CONFIG="bm,bn,g" or "bm,bn,g,ksplit", one of
// the compiled configurations (256,256,1 / 256,128,1 / 128,128,2 / 128,128,1 / 64,128,4), with an
// optional number of K slices (used only where splitting is allowed); read once per
// process.
struct ConfigOverride {
    bool on = false;
    int bm = 0, bn = 0, g = 0, ksplit = 0;
};

const ConfigOverride& config_override() {
    static const ConfigOverride c = [] {
        ConfigOverride r;
        const char* e = std::getenv("BITNET_TILED_CONFIG");
        int a = 0, b = 0, g = 0, ks = 0;
        const int n = e ? std::sscanf(e, "%d,%d,%d,%d", &a, &b, &g, &ks) : 0;
        r.on = n >= 3 &&
               ((a == 256 && b == 256 && g == 1) || (a == 256 && b == 128 && g == 1) ||
                (a == 128 && b == 128 && g == 2) || (a == 128 && b == 128 && g == 1) ||
                (a == 64 && b == 128 && g == 4)) &&
               (n == 3 || (ks >= 1 && ks <= 64));
        r.bm = a;
        r.bn = b;
        r.g = g;
        r.ksplit = n == 4 ? ks : 0;
        return r;
    }();  // thread-safe initialization of a function-local static
    return c;
}

// Tile shape: the compiled configuration with the least estimated time.  Every
// configuration runs one block per CU, so a launch takes ceil(units / CUs) rounds, and
// a round costs about the same whether it is full or not (a lone tile is bound by its
// own latency, not by the matrix cores).  A round's cost is a fixed part plus a part per
// unit of K, fitted to launches of each configuration on the 2B-shaped prefill products
// (M = 512, N = 2560, K = 256 .. 5120, one round): small tiles start and finish soonest
// (64x128 blocks with four k-groups: four waves per SIMD), large tiles amortize the
// weight unpack and the activation transpose over more products per k.  128-k stages
// (half the barriers and twice the bytes per load of 64-k stages) need K % 128 == 0;
// the 256x256 tile keeps 64-k stages (128-k ones spill its registers).
//
// Where the caller provides a workspace, K may also be split into slices taken by
// different blocks (more units per round, fewer k per unit): each unit writes its int32
// partial tile, and a second launch adds the slices' partials (exact in int32, so the
// result is bit-identical to the unsplit product) and rescales.  A split costs a fixed
// part (the second launch) plus a part per byte of int32 partials (written by the first
// launch, read by the second), fitted on M = 32 .. 256 products with K = 4096 .. 28672
// and 1 to 16 slices: about 1 us per MB, far below streaming rate -- more active blocks
// per round also raise every block's cost per K.
struct TileCost {
    int bm, bn, g, bk;
    double fixed_us, per_k_us;
};
constexpr TileCost kTileCosts[] = {
    {64, 128, 4, 128, 5.4, 2.13e-3},
    {128, 128, 2, 128, 6.3, 3.42e-3},
    {256, 128, 1, 128, 8.2, 6.61e-3},
    {64, 128, 4, 64, 4.7, 2.96e-3},
    {128, 128, 2, 64, 6.4, 4.5e-3},
    {256, 128, 1, 64, 7.0, 7.3e-3},
    {256, 256, 1, 64, 10.5, 11.7e-3},
};
constexpr double kSplitFixedUs = 1.5;      // the reduce launch
constexpr double kSplitUsPerByte = 1.0e-6;  // per byte of int32 partials
constexpr int kMaxSplit = 16;
constexpr int64_t kMaxSplitBytes = int64_t(64) << 20;  // int32 partials of all slices

TilePlan plan_tiles(int64_t M, int64_t K, const int64_t* N, int groups, int64_t cus,
                    bool allow_split) {
    TilePlan t;
    int64_t n_all = 0;
    for (int i = 0; i < groups; ++i) n_all += N[i];
    const ConfigOverride& ov = config_override();
    if (ov.on) {
        t.bm = ov.bm;
        t.bn = ov.bn;
        t.g = ov.g;
        t.bk = (K % 128 == 0 && !(t.bm == 256 && t.bn == 256)) ? 128 : 64;
        const int nk = (int)((K + t.bk - 1) / t.bk);
        const int ks = allow_split && ov.ksplit > 1 ? ov.ksplit : 1;
        t.split_stages = (nk + ks - 1) / ks;
        t.ksplit = (nk + t.split_stages - 1) / t.split_stages;  // no empty slice
        if (t.ksplit > 1 && t.ksplit * M * n_all * 4 > kMaxSplitBytes) {
            t.ksplit = 1;
            t.split_stages = nk;
        }
        return t;
    }
    double best = -1.0;
    for (const TileCost& c : kTileCosts) {
        if (K % c.bk != 0 && c.bk != 64) continue;
        int64_t tiles_n = 0;
        for (int i = 0; i < groups; ++i) tiles_n += (N[i] + c.bn - 1) / c.bn;
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * tiles_n;
        const int nk = (int)((K + c.bk - 1) / c.bk);
        for (int ks = 1; ks <= (allow_split ? kMaxSplit : 1); ++ks) {
            const int stages = (nk + ks - 1) / ks;
            const int slices = (nk + stages - 1) / stages;
            if (slices != ks) continue;                     // a slice would be empty
            if (ks > 1 && stages < c.g) break;              // k-groups without a stage
            const int64_t part_bytes = (int64_t)ks * M * n_all * 4;
            if (ks > 1 && part_bytes > kMaxSplitBytes) break;
            const int64_t units = tiles * ks;
            double est = (double)((units + cus - 1) / cus) *
                         (c.fixed_us + c.per_k_us * (double)stages * c.bk);
            if (ks > 1) est += kSplitFixedUs + kSplitUsPerByte * (double)part_bytes;
            if (best < 0.0 || est < best) {
                best = est;
                t.bm = c.bm;
                t.bn = c.bn;
                t.g = c.g;
                t.bk = c.bk;
                t.ksplit = ks;
                t.split_stages = stages;
            }
        }
    }
    // Full-chip grids: where the model picks a 256-row tile unsplit and 128x128 tiles
    // give every CU at least one, the 128x128 tile with one k-group runs instead.  Two of
    // its blocks fit a CU (registers and LDS), so each SIMD interleaves two waves, which
    // the one-round fits above cannot see; measured 2-12% faster on the 8B (M = 2048)
    // and 70B (M = 1024) products, never slower there.
    if (t.bm == 256 && t.ksplit == 1) {
        int64_t tiles_n = 0;
        for (int i = 0; i < groups; ++i) tiles_n += (N[i] + 127) / 128;
        if (((M + 127) / 128) * tiles_n >= cus) {
            t.bm = 128;
            t.bn = 128;
            t.g = 1;
            t.bk = K % 128 == 0 ? 128 : 64;
            t.split_stages = (int)((K + t.bk - 1) / t.bk);
        }
    }
    return t;
}

// Adds the ksplit int32 partial products of every output (slice s at part + s * stride)
// in slice order -- exact, so any order gives the same sum -- and rescales like the tiled
// epilogue: ((float)acc * w_scale[n]) * (1 / a_scale[m]).  VEC: N % 4 == 0, four
// consecutive outputs of one row per thread; else one output per thread.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const int* __restrict__ part, int ksplit,
                                                            int64_t stride, int M, int N,
                                                            const float* __restrict__ a_scale,
                                                            const float* __restrict__ w_scale,
                                                            void* __restrict__ out) {
    constexpr int V = VEC ? 4 : 1;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;  // first output
    if (i >= (int64_t)M * N) return;
    const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
    // every slice's load is issued before the first add (the loop is unrolled over the
    // largest slice count, the slice test is uniform), so the reads overlap
    int acc[V];
    if constexpr (VEC) {
        int4 v[kMaxSplit];
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
            if (s < ksplit) v[s] = *reinterpret_cast<const int4*>(part + s * stride + i);
        int4 sum = v[0];
#pragma unroll
        for (int s = 1; s < kMaxSplit; ++s) {
            if (s < ksplit) {
                sum.x += v[s].x;
                sum.y += v[s].y;
                sum.z += v[s].z;
                sum.w += v[s].w;
            }
        }
        acc[0] = sum.x;
        acc[1] = sum.y;
        acc[2] = sum.z;
        acc[3] = sum.w;
    } else {
        int v[kMaxSplit];
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
            if (s < ksplit) v[s] = part[s * stride + i];
        int sum = v[0];
#pragma unroll
        for (int s = 1; s < kMaxSplit; ++s)
            if (s < ksplit) sum += v[s];
        acc[0] = sum;
    }
    if constexpr (DT == 2) {
        if constexpr (VEC)
            *reinterpret_cast<int4*>(static_cast<int*>(out) + i) = make_int4(acc[0], acc[1], acc[2], acc[3]);
        else
            static_cast<int*>(out)[i] = acc[0];
        return;
    }
    const float inv_a = 1.0f / a_scale[m];
    float f[V];
#pragma unroll
    for (int t = 0; t < V; ++t) f[t] = ((float)acc[t] * w_scale[n + t]) * inv_a;
    if constexpr (DT == 0) {
        if constexpr (VEC)
            *reinterpret_cast<float4*>(static_cast<float*>(out) + i) = make_float4(f[0], f[1], f[2], f[3]);
        else
            static_cast<float*>(out)[i] = f[0];
    } else {
        if constexpr (VEC)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i) =
                make_uint2(f32x2_to_bf16x2_rne(f[0], f[1]), f32x2_to_bf16x2_rne(f[2], f[3]));
        else
            static_cast<uint16_t*>(out)[i] = f32_to_bf16_rne(f[0]);
    }
}

template <int DT>
hipError_t launch_reduce(const int* part, int ksplit, int M, int N, const float* a_scale,
                         const float* w_scale, void* out, hipStream_t stream) {
    const int64_t total = (int64_t)M * N;
    const bool vec = N % 4 == 0;
    const int64_t threads = vec ? total / 4 : total;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (vec)
        hipLaunchKernelGGL((splitk_reduce_kernel<DT, true>), grid, dim3(256), 0, stream, part, ksplit,
                           total, M, N, a_scale, w_scale, out);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<DT, false>), grid, dim3(256), 0, stream, part, ksplit,
                           total, M, N, a_scale, w_scale, out);
    return hipGetLastError();
}

template <int BM, int BN, int D, int G, int WGN, int BK>
hipError_t launch_plan(TiledArgs a, const int64_t* N, const TilePlan& t, int* part,
                       hipStream_t stream) {
    const bool aligned = (a.K % BK) == 0;
    const int tiles_m = (a.M + BM - 1) / BM;
    int units = 0;
    for (int i = 0; i < kTdGroups; ++i) {
        const int tn = i < a.groups ? (int)((N[i] + BN - 1) / BN) : 0;
        a.first[i] = units;
        a.g_tiles_n[i] = tn;
        units += tiles_m * tn;
    }
    if (units == 0) return hipSuccess;
    const bool split = t.ksplit > 1;
    void* const final_out = a.g_out[0];
    const int final_dtype = a.out_dtype;
    a.ksplit = t.ksplit;
    a.split_stages = t.split_stages;
    a.split_stride = split ? (int64_t)a.M * a.g_N[0] : 0;
    if (split) {
        // the units write int32 partial tiles into the workspace; the reduce launch
        // below adds them and writes the requested output
        a.g_out[0] = part;
        a.out_dtype = 2;
    }
    a.units = units * t.ksplit;
    a.units_per_xcd = (a.units + kXcds - 1) / kXcds;
    // panel height: an XCD's run of units_per_xcd tiles as gm rows by units_per_xcd / gm
    // columns reads gm * BM * K activation bytes and (units_per_xcd / gm) * BN * K / 4
    // weight bytes, least at gm = sqrt(units_per_xcd * BN / (4 BM))
    a.gm = (int)(std::sqrt((double)a.units_per_xcd * BN / (4.0 * BM)) + 0.5);
    a.gm = a.gm < 1 ? 1 : (a.gm > tiles_m ? tiles_m : a.gm);
    const dim3 grid((unsigned)(a.units_per_xcd * kXcds));
    const dim3 blk(kTdThreads * G);
    if constexpr (BK == 128) {
        // planned only for K % 128 == 0: the aligned kernels alone are built
        if (!aligned) return hipErrorInvalidValue;
        switch (a.out_dtype) {
            case 0: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, true, 0>), grid, blk, 0, stream, a); break;
            case 1: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, true, 1>), grid, blk, 0, stream, a); break;
            default: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, true, 2>), grid, blk, 0, stream, a); break;
        }
    } else {
        switch (a.out_dtype * 2 + (aligned ? 1 : 0)) {
            case 0: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, false, 0>), grid, blk, 0, stream, a); break;
            case 1: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, true, 0>), grid, blk, 0, stream, a); break;
            case 2: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, false, 1>), grid, blk, 0, stream, a); break;
            case 3: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, true, 1>), grid, blk, 0, stream, a); break;
            case 4: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, false, 2>), grid, blk, 0, stream, a); break;
            default: hipLaunchKernelGGL((tiled_kernel<BM, BN, D, G, WGN, BK, true, 2>), grid, blk, 0, stream, a); break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    switch (final_dtype) {
        case 0: return launch_reduce<0>(part, t.ksplit, a.M, a.g_N[0], a.a_scale, a.g_wscale[0], final_out, stream);
        case 1: return launch_reduce<1>(part, t.ksplit, a.M, a.g_N[0], a.a_scale, a.g_wscale[0], final_out, stream);
        default: return launch_reduce<2>(part, t.ksplit, a.M, a.g_N[0], a.a_scale, a.g_wscale[0], final_out, stream);
    }
}

hipError_t launch_tiled_impl(const int8_t* xq, const float* a_scale, int groups,
                             const uint8_t* const* packed, const float* const* w_scale,
                             const int64_t* N, void* const* out, int64_t M, int64_t K,
                             int out_dtype, int* part, size_t part_bytes, hipStream_t stream) {
    if (groups < 1 || groups > kTdGroups) return hipErrorInvalidValue;
    TiledArgs a;
    a.xq = xq;
    a.a_scale = a_scale;
    a.groups = groups;
    for (int i = 0; i < kTdGroups; ++i) {
        const bool on = i < groups;
        a.g_N[i] = on ? (int)N[i] : 0;
        a.g_packed[i] = on ? packed[i] : nullptr;
        a.g_wscale[i] = on ? w_scale[i] : nullptr;
        a.g_out[i] = on ? out[i] : nullptr;
    }
    a.M = (int)M;
    a.K = (int)K;
    a.out_dtype = out_dtype;
    int64_t n_all[kTdGroups];
    for (int i = 0; i < kTdGroups; ++i) n_all[i] = i < groups ? N[i] : 0;
    // K is split only for one matrix and a workspace that holds the planned partials
    bool allow_split = groups == 1 && part != nullptr;
    if (allow_split) {
        const TilePlan ts = plan_tiles(M, K, n_all, 1, device_cus(), true);
        allow_split = ts.ksplit > 1 && (size_t)ts.ksplit * (size_t)M * (size_t)N[0] * 4 <= part_bytes;
    }
    const TilePlan t = plan_tiles(M, K, n_all, groups, device_cus(), allow_split);
    // register sets in flight: 64-k stages 4 (2 for 256x256); 128-k stages 2, or 4 for
    // the 256x128 tile (its accumulators live in the matrix-core registers)
    if (t.bm == 256 && t.bn == 256) return launch_plan<256, 256, 2, 1, 4, 64>(a, n_all, t, part, stream);
    // 128x128, one k-group: waves in a 1 x 4 grid (128 x 32 each), four register sets
    if (t.bm == 128 && t.g == 1) {
        if (t.bk == 128) return launch_plan<128, 128, 4, 1, 4, 128>(a, n_all, t, part, stream);
        return launch_plan<128, 128, 4, 1, 4, 64>(a, n_all, t, part, stream);
    }
    if (t.bk == 128) {
        if (t.bm == 256) return launch_plan<256, 128, 4, 1, 2, 128>(a, n_all, t, part, stream);
        if (t.bm == 64) return launch_plan<64, 128, 2, 4, 4, 128>(a, n_all, t, part, stream);
        return launch_plan<128, 128, 2, 2, 2, 128>(a, n_all, t, part, stream);
    }
    if (t.bm == 256) return launch_plan<256, 128, 4, 1, 2, 64>(a, n_all, t, part, stream);
    if (t.bm == 64) return launch_plan<64, 128, 4, 4, 4, 64>(a, n_all, t, part, stream);
    return launch_plan<128, 128, 4, 2, 2, 64>(a, n_all, t, part, stream);
}

}  // namespace

size_t tiled_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1) return 0;
    const TilePlan t = plan_tiles(M, K, &N, 1, device_cus(), true);
    return t.ksplit > 1 ? (size_t)t.ksplit * (size_t)M * (size_t)N * 4 : 0;
}

void tiled_plan(int64_t M, int64_t K, int groups, const int64_t* N, int64_t cus, int* plan) {
    const TilePlan t = plan_tiles(M, K, N, groups, cus > 0 ? cus : device_cus(), groups == 1);
    plan[0] = t.bm;
    plan[1] = t.bn;
    plan[2] = t.g;
    plan[3] = t.bk;
    plan[4] = t.ksplit;
}

hipError_t launch_tiled_grouped(const int8_t* xq, const float* a_scale, int groups,
                                const uint8_t* const* packed, const float* const* w_scale,
                                const int64_t* N, void* const* out, int64_t M, int64_t K,
                                int out_dtype, hipStream_t stream) {
    return launch_tiled_impl(xq, a_scale, groups, packed, w_scale, N, out, M, K, out_dtype,
                             nullptr, 0, stream);
}

hipError_t launch_tiled(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                        const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                        int out_dtype, void* workspace, size_t ws_bytes, hipStream_t stream) {
    void* outs[1] = {out};
    return launch_tiled_impl(xq, a_scale, 1, &packed, &w_scale, &N, outs, M, K, out_dtype,
                             static_cast<int*>(workspace), ws_bytes, stream);
}

}  // namespace bitnet
