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
//    one row per chunk, a wave 16 rows x 64 bytes, with 128-bit buffer loads.
//  * Latency first: the scales and activations are requested, then the block's weights
//    (all of them when a wave's share fits in U chunks, else the first of a
//    double-buffered series of U-chunk batches), and only then does the activation
//    quantization run, so it overlaps the weights' trip from memory.  The loads are
//    unconditional: a chunk or row outside the problem gets an offset past the buffer
//    resource's range, which reads as zeros, so the compiler counts the loads in flight
//    exactly and never has to drain them all before the first use.  When the
//    activations are staged in loops instead (more than fit in registers), the first
//    weight batch is requested before them.
//  * Fused max |x| scan of the staged variant: wave w reads rows w, w + 4, ... with
//    batches of independent loads, two batches in flight, before one block barrier.
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
//  * Per-row maxima and code sums are reduced per wave (wave reductions at M = 1, atomics
//    on the wave's own LDS slots otherwise), so no block-wide atomic is contended.
//  * Per-wave int32 partials are combined through LDS; one pass writes the outputs.
//  * One token over a large grid (768+ blocks of 16 rows): a block takes two 16-row
//    tiles, whose weight operands share each activation operand, so half as many
//    blocks read and quantize the activations.
//  * Grouped launches: up to kSkGroups weight matrices that read the same activations
//    (q, k and v of an attention block; gate and up of an MLP) share one launch.  The
//    grid is the concatenation of the groups' row blocks; a block picks its group with
//    scalar compares of its index, so each group costs exactly what it costs alone,
//    minus one launch.
#include <atomic>

#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

namespace {

#ifndef BITNET_SKINNY_WAVES
#define BITNET_SKINNY_WAVES 4
#endif
constexpr int kSkWaves = BITNET_SKINNY_WAVES;
constexpr int kSkThreads = 64 * kSkWaves;
#ifndef BITNET_SKINNY_RUN
#define BITNET_SKINNY_RUN 2
#endif
// A wave takes runs of kSkRun consecutive 256-weight chunks (64 bytes of each row per
// chunk), so its back-to-back loads cover whole 128-byte lines of every row.
constexpr int kSkRun = BITNET_SKINNY_RUN;

// j-th chunk of wave w: runs of kSkRun chunks, dealt to the waves in turn
__host__ __device__ constexpr int chunk_of(int w, int j) {
    return kSkRun * (w + kSkWaves * (j / kSkRun)) + j % kSkRun;
}
// number of chunks of a stage of nch chunks that wave w owns, and the largest over waves
__host__ __device__ constexpr int chunks_of_wave(int w, int nch) {
    const int span = kSkRun * kSkWaves, r = nch % span - kSkRun * w;
    return (nch / span) * kSkRun + (r < 0 ? 0 : (r > kSkRun ? kSkRun : r));
}
// The same with the last, partial round of runs spread one chunk per wave in turn, so
// that no wave owns more than one chunk above another (one token, one K stage of at most
// three chunks per wave: the 2560-wide projections take 3, 3, 2, 2 chunks instead of 4,
// 2, 2, 2).  Only for launches with a single K stage: with several, a wave's LDS slots
// must not depend on the stage, or it would overwrite activations that another wave
// still reads.  Slots j past a wave's share map to chunks >= nch.
__host__ __device__ constexpr int chunk_of_spread(int w, int j, int nch) {
    const int span = kSkRun * kSkWaves, full = nch / span;
    return j < full * kSkRun ? chunk_of(w, j) : full * span + w + kSkWaves * (j - full * kSkRun);
}
__host__ __device__ constexpr int chunks_of_wave_spread(int w, int nch) {
    const int span = kSkRun * kSkWaves, tail = nch % span;
    return (nch / span) * kSkRun + (tail > w ? (tail - w + kSkWaves - 1) / kSkWaves : 0);
}
constexpr int kSkXBudget = 48 * 1024;   // LDS bytes for the staged activations
constexpr int kSkMaxM = 64;                    // rows of activations (tokens) per launch
constexpr int kSkMisc = kSkWaves * kSkMaxM * 8 + kSkMaxM * 4;  // s_wmax, s_wsum [waves][64]; s_inva [64]
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset beyond every resource: reads 0

// a[i] for a wave-uniform i < 4, as scalar selects (no indexed copy of the kernel
// arguments)
template <typename T>
__device__ __forceinline__ T pick(const T (&a)[4], int i) {
    T r = a[0];
    r = i == 1 ? a[1] : r;
    r = i == 2 ? a[2] : r;
    r = i == 3 ? a[3] : r;
    return r;
}

constexpr int kSkGroups = BITNET_MAX_GROUPS;
// Fewest 16-row blocks (three per CU of a 256-CU chip) at which a one-token launch
// switches to 32-row blocks: with fewer, the halved grid leaves CUs idle.
#ifndef BITNET_SKINNY_TWO_TILE_MIN_BLOCKS
#define BITNET_SKINNY_TWO_TILE_MIN_BLOCKS 768
#endif
constexpr int64_t kSkTwoTileMinBlocks = BITNET_SKINNY_TWO_TILE_MIN_BLOCKS;

struct SkinnyArgs {
    const int8_t* xq;
    const float* a_scale;
    const uint16_t* xb;
    int8_t* xq_out;
    float* a_out;
    // group g owns the blocks first[g] .. first[g + 1] - 1 (groups with no rows own none)
    int groups;
    int first[kSkGroups];
    int g_N[kSkGroups];
    const uint8_t* g_packed[kSkGroups];
    const float* g_wscale[kSkGroups];
    void* g_out[kSkGroups];
    int M, K;
    int Kp;  // K rounded up to a multiple of 256
    int KS;  // K-stage length staged in LDS at once (multiple of 256)
    int out_dtype;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// 16 packed bytes at byte offset `off` of packed row `n`, byte by byte, zeros past the
// row end (the path for K not a multiple of 64, whose rows are not 16-byte aligned).
__device__ __forceinline__ uint4 load_w16_bytes(const uint8_t* __restrict__ packed,
                                                int64_t row_bytes, int n, int64_t off) {
    const uint8_t* src = packed + (int64_t)n * row_bytes + off;
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (off + j < row_bytes) d[j >> 2] |= (uint32_t)src[j] << (8 * (j & 3));
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// 16 bf16 activations x[m][k0 .. k0+15] as 8 words, element by element, zeros past K.
__device__ __forceinline__ void load_x16_bf16_elems(const uint16_t* __restrict__ xb, int K, int m,
                                                    int k0, uint32_t h[8]) {
    const uint16_t* src = xb + (int64_t)m * K + k0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (k0 + 2 * j < K) ? src[2 * j] : 0u;
        const uint32_t hi = (k0 + 2 * j + 1 < K) ? src[2 * j + 1] : 0u;
        h[j] = lo | (hi << 16);
    }
}

// One 16-element group, already transposed (byte b of e[i] = element 4 b + i), into the
// permuted LDS layout; returns the sum of its codes.
__device__ __forceinline__ int put_group_t(unsigned char* x_lds, int KSP, int m, int u,
                                           const uint32_t e[4]) {
    const int rs = sum_i8x4(e[0], sum_i8x4(e[1], sum_i8x4(e[2], sum_i8x4(e[3], 0))));
    unsigned char* dst = x_lds + m * KSP + (u >> 2) * 64 + 4 * (u & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(dst + 16 * i) = e[i];
    return rs;
}

// Template parameters:
//  FUSED  - quantize bf16 activations in the kernel (else read int8 codes + a_scale)
//  FAST   - K % 64 == 0: rows are 16-byte aligned, buffer loads for the weights
//  XH     - activation groups held in registers per lane (0: staged in loops instead);
//           only with a single K stage
//  U      - weight chunks per wave per batch
//  SINGLE - one batch covers a wave's whole share of K (single K stage)
//  MC     - M fixed at compile time (1), or 0 for M read from the arguments
//  MT     - 16-row tiles of tokens (M <= 16 MT); the weights of a chunk feed all of them
//  PAIR   - SwiGLU pair: the block multiplies the same 16 rows of two matrices (gate =
//           group 0, up = group 1) and writes silu(gate) * up
//  NR     - 16-row tiles of one matrix per block (1 or 2; 2 with one token only): the
//           tiles share the block's copy of the activations
template <bool FUSED, bool FAST, int XH, int U, bool SINGLE, int MC, int MT = 1, bool PAIR = false,
          int NR = 1>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkinnyArgs p) {
    static_assert(NR == 1 || (NR == 2 && MC == 1 && FAST && !PAIR), "two row tiles: one token");
    constexpr int NW = PAIR ? 2 : NR;  // weight operands per chunk (matrices or row tiles)
    extern __shared__ __align__(16) unsigned char smem[];
    const int KSP = p.KS + 16;  // padded LDS row stride: spreads rows over the banks
    // one token, one batch of three chunks: the spread deal (see chunk_of_spread)
    constexpr bool kSpread = MC == 1 && SINGLE && U == 3;
    auto chunk_at = [](int w, int j, int nch) {
        return kSpread ? chunk_of_spread(w, j, nch) : chunk_of(w, j);
    };
    const int M = MC > 0 ? MC : p.M;
    const int K = p.K;
    // this block's group: uniform, resolved with scalar selects
    int gi = 0;
#pragma unroll
    for (int i = 1; i < kSkGroups; ++i)
        if (i < p.groups && (int)blockIdx.x >= p.first[i]) gi = i;
    const int N = pick(p.g_N, gi);
    const uint8_t* packed_v[NW];
    const float* w_scale_v[NW];
    packed_v[0] = pick(p.g_packed, gi);
    w_scale_v[0] = pick(p.g_wscale, gi);
    if constexpr (PAIR) {
        packed_v[1] = p.g_packed[1];
        w_scale_v[1] = p.g_wscale[1];
    } else if constexpr (NR == 2) {
        packed_v[1] = packed_v[0];
        w_scale_v[1] = w_scale_v[0];
    }
    void* const out = pick(p.g_out, gi);
    unsigned char* x_lds = smem;
    // per-wave partial results: s_wmax[w][m] = max |x| bits seen by wave w in row m,
    // s_wsum[w][m] = sum of the codes of row m staged by wave w
    uint32_t* s_wmax = reinterpret_cast<uint32_t*>(smem + M * KSP);
    int* s_wsum = reinterpret_cast<int*>(s_wmax + kSkMaxM * kSkWaves);
    float* s_inva = reinterpret_cast<float*>(s_wsum + kSkMaxM * kSkWaves);
    int* red = reinterpret_cast<int*>(smem + M * KSP + kSkMisc);  // [waves][MT][4][64]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
    const int row_bytes = K / 4;
    const int n0 = ((int)blockIdx.x - pick(p.first, gi)) * 16 * NR;
    // first row and row count (0 past the end of N) of operand v's 16-row tile
    int nv0[NW], rows_v[NW];
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        nv0[v] = min(n0 + (PAIR ? 0 : 16 * v), N);
        rows_v[v] = min(16, N - nv0[v]);
    }
    const int rows = rows_v[0];
    const int mrow = lane & 15;  // operand-A row (token) and operand-B column of this lane
    const int q = lane >> 4;     // k-group of this lane inside a 256-weight chunk
    const bool row_leader = (lane & 15) == 0;

    // scales needed at the end, requested first (threads tid < 16 M NR write outputs)
    float ws_n[NW];
#pragma unroll
    for (int v = 0; v < NW; ++v)
        ws_n[v] = buf_load_f32(make_rsrc(w_scale_v[v] + nv0[v], (uint32_t)(rows_v[v] * 4)),
                               tid < 16 * M * NR ? (uint32_t)(4 * (tid & 15)) : kOOB);
    float a_in = 0.0f;  // M = 1: every thread holds the token's scale
    if constexpr (!FUSED)
        a_in = buf_load_f32(make_rsrc(p.a_scale, (uint32_t)(M * 4)),
                            MC == 1 ? 0u : (tid < M ? 4u * tid : kOOB));

    // the block's weight rows (fewer than 16 at the end of N); reads past them give 0
    __amdgpu_buffer_rsrc_t w_rsrc[NW];
#pragma unroll
    for (int v = 0; v < NW; ++v)
        w_rsrc[v] = make_rsrc(packed_v[v] + (int64_t)nv0[v] * row_bytes,
                              (uint32_t)(rows_v[v] * row_bytes));
    const uint32_t w_lane = (uint32_t)(mrow * row_bytes + 16 * q);

    // chunks c = wave + 4 * (j0 + uu), uu < U, of the stage starting at byte stage_off;
    // w[uu * NW + v] holds chunk uu of matrix v
    auto load_batch = [&](uint4 (&w)[U * NW], int j0, int stage_off, int nch) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int c = chunk_at(wave, j0 + uu, nch);
            const int cb = stage_off + c * 64;  // the chunk's first byte in the row
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                if (FAST) {
                    const uint32_t off = (c < nch && cb + 16 * q < row_bytes) ? w_lane + cb : kOOB;
                    w[uu * NW + v] = buf_load16(w_rsrc[v], off);
                } else {
                    const int n = n0 + mrow;
                    w[uu * NW + v] = (n < N && c < nch)
                                         ? load_w16_bytes(packed_v[v], row_bytes, n, cb + 16 * q)
                                         : make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
    };

    v4i acc1[NW][MT], acc4[NW][MT], acc16[NW][MT];
#pragma unroll
    for (int v = 0; v < NW; ++v)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc1[v][t] = acc4[v][t] = acc16[v][t] = v4i{0, 0, 0, 0};

    auto compute_batch = [&](const uint4 (&w)[U * NW], int j0, int nch) {
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int c = chunk_at(wave, j0 + uu, nch);
            // With M = 1 and one batch, chunks past the stage are multiplied as well: their
            // weights read as zeros and their operand-A reads stay inside the LDS block.
            if ((MC == 1 && SINGLE) || c < nch) {
                v4i b0[NW], b1[NW], b2[NW], b3[NW];
#pragma unroll
                for (int v = 0; v < NW; ++v) {
                    const uint4 wv = w[uu * NW + v];
                    const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        b0[v][r] = (int)(w4[r] & 0x03030303u);
                        b1[v][r] = (int)(w4[r] & 0x0C0C0C0Cu);
                        b2[v][r] = (int)(w4[r] & 0x30303030u);
                        b3[v][r] = (int)((w4[r] >> 2) & 0x30303030u);
                    }
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {  // the unpacked weights feed every token tile
                    v4i A[4];
                    if constexpr (MC == 1) {
                        // one token: every lane reads row 0's fragment (a broadcast read),
                        // so no branch guards it and the reads can be issued before the
                        // weights arrive; rows 1-15 of the products repeat row 0 and are
                        // never read
                        const unsigned char* src = x_lds + (c * 4 + q) * 64;
#pragma unroll
                        for (int i = 0; i < 4; ++i) A[i] = *reinterpret_cast<const v4i*>(src + 16 * i);
                    } else {
                        // rows past M read row M - 1 (staged, so inside the block's LDS):
                        // no branch guards the read, and the products of those rows are
                        // never combined or stored
                        const int row = min(16 * t + mrow, M - 1);
                        const unsigned char* src = x_lds + row * KSP + (c * 4 + q) * 64;
#pragma unroll
                        for (int i = 0; i < 4; ++i) A[i] = *reinterpret_cast<const v4i*>(src + 16 * i);
                    }
#pragma unroll
                    for (int v = 0; v < NW; ++v) {
                        acc1[v][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[0], b0[v], acc1[v][t], 0, 0, 0);
                        acc4[v][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[1], b1[v], acc4[v][t], 0, 0, 0);
                        acc16[v][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2], b2[v], acc16[v][t], 0, 0, 0);
                        acc16[v][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[3], b3[v], acc16[v][t], 0, 0, 0);
                    }
                }
            }
        }
    };

    // each wave clears its own slots (LDS operations of one wave complete in order)
    s_wmax[wave * kSkMaxM + lane] = 0u;  // one slot per token row (64 = lanes)
    s_wsum[wave * kSkMaxM + lane] = 0;
    // the activation scale 127 / max|x| of token m from the waves' maxima
    auto fused_scale = [&](int m) -> float {
        uint32_t mx = s_wmax[m];
#pragma unroll
        for (int w = 1; w < kSkWaves; ++w) mx = max(mx, s_wmax[kSkMaxM * w + m]);
        float amax = bf16_bits_to_f32(mx);
        amax = amax < 1e-5f ? 1e-5f : amax;
        return 127.0f / amax;
    };

    // Staging is wave-local: wave w stages exactly the chunks c = w + 4 j it multiplies,
    // all M rows, so no block barrier separates staging from use.  The wave's 16-element
    // groups are numbered g = (j * M + m) * 16 + i (activations k = 256 c + 16 i ..
    // + 15 of row m); lane l takes g = l + 64 t, so the 16 lanes of a DPP row share
    // (j, m) and reduce their per-row partials with DPP before one LDS atomic.
    const int nch0 = min(p.KS, p.Kp) >> 8;  // chunks of the first (or only) K stage
    auto group_of = [&](int g, int& m, int& c, int& i) {
        i = g & 15;
        const int jm = g >> 4, j = jm / M;
        m = jm - j * M;
        c = chunk_at(wave, j, nch0);
    };

    uint4 wa[U * NW];
    float a_m1 = 0.0f;  // M = 1, fused: the token's scale, uniform
    int wsum_m1 = 0;    // M = 1: code sum of the activations this wave staged, uniform
    if constexpr (XH > 0) {
        // ---- single K stage, activations held in registers: requested before weights ----
        constexpr int XW = FUSED ? 8 : 4;
        uint32_t held[XH][XW];
#pragma unroll
        for (int t = 0; t < XH; ++t) {
            int m, c, i;
            group_of(lane + 64 * t, m, c, i);
            const int k0 = 256 * c + 16 * i;
            const bool ok = c < nch0 && k0 < K;
            if constexpr (FUSED) {
                const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(p.xb, (uint32_t)(M * K * 2));
                const uint32_t off = ok ? (uint32_t)((m * K + k0) * 2) : kOOB;
                const uint4 v0 = buf_load16(x_rsrc, off), v1 = buf_load16(x_rsrc, off + 16);
                held[t][0] = v0.x; held[t][1] = v0.y; held[t][2] = v0.z; held[t][3] = v0.w;
                held[t][4] = v1.x; held[t][5] = v1.y; held[t][6] = v1.z; held[t][7] = v1.w;
            } else {
                const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(p.xq, (uint32_t)(M * K));
                const uint4 v0 = buf_load16(x_rsrc, ok ? (uint32_t)(m * K + k0) : kOOB);
                held[t][0] = v0.x; held[t][1] = v0.y; held[t][2] = v0.z; held[t][3] = v0.w;
            }
        }
        load_batch(wa, 0, 0, nch0);  // the weights' memory trip overlaps all that follows

        if constexpr (FUSED) {
            if (MC == 1) {
                uint32_t mx = 0;
#pragma unroll
                for (int t = 0; t < XH; ++t) mx = max(mx, absmax_bits16(held[t]));  // 0 if unused
                mx = wave_max_u32(mx);
                if (lane == 0) s_wmax[wave * kSkMaxM] = mx;
            } else {
#pragma unroll
                for (int t = 0; t < XH; ++t) {
                    int m, c, i;
                    group_of(lane + 64 * t, m, c, i);
                    const uint32_t mx = row16_max(absmax_bits16(held[t]));
                    if (row_leader && c < nch0) atomicMax(&s_wmax[wave * kSkMaxM + m], mx);
                }
            }
            __syncthreads();
        }
        if constexpr (FUSED && MC == 1) a_m1 = fused_scale(0);
        int rsum = 0;
#pragma unroll
        for (int t = 0; t < XH; ++t) {
            int m, c, i;
            group_of(lane + 64 * t, m, c, i);
            uint32_t e[4];
            if constexpr (FUSED) {
                quant16_t(held[t], MC == 1 ? a_m1 : fused_scale(m), e);
                if (blockIdx.x == 0 && p.xq_out && c < nch0) {
                    uint32_t d[4];
                    untranspose(e, d);
                    store_codes16<FAST>(p.xq_out, K, m, 256 * c + 16 * i, d);
                }
            } else {
                transpose4x4_bytes(held[t], e);
            }
            int rs = 0;
            if (c < nch0) rs = put_group_t(x_lds, KSP, m, 16 * c + i, e);
            if (MC == 1) {
                rsum += rs;
            } else {
                rs = row16_sum(rs);
                if (row_leader && c < nch0) atomicAdd(&s_wsum[wave * kSkMaxM + m], rs);
            }
        }
        if (MC == 1) wsum_m1 = wave_sum_i32(rsum);
    } else {
        // the first weights of stage 0 are requested before the activations are read
        load_batch(wa, 0, 0, nch0);
        if constexpr (FUSED) {
            // ---- max |x| per token over the whole row: wave w scans rows w, w + 4, ... ----
            const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(p.xb, (uint32_t)(M * K * 2));
            if (K % 8 == 0)
                scan_absmax_rows<true>(x_rsrc, M, K, wave, kSkWaves, s_wmax + wave * kSkMaxM);
            else
                scan_absmax_rows<false>(x_rsrc, M, K, wave, kSkWaves, s_wmax + wave * kSkMaxM);
            __syncthreads();
        }
    }

    auto run_stage = [&](int ks) {
        const int len = min(p.KS, p.Kp - ks);
        const int nch = len >> 8;
        const int stage_off = ks >> 2;
        if constexpr (XH == 0) {
            // ---- stage this wave's chunks of [ks, ks+len), all M rows, into LDS ----
            // SB groups per lane are requested together (unconditional buffer loads, zeros
            // past K or past the wave's groups) before any of them is used.
            const int cnt = M * chunks_of_wave(wave, nch) * 16;
            constexpr int SB = FUSED ? 4 : 8;
            constexpr int XW = FUSED ? 8 : 4;
            const __amdgpu_buffer_rsrc_t x_rsrc =
                FUSED ? make_rsrc(p.xb, (uint32_t)(M * K * 2)) : make_rsrc(p.xq, (uint32_t)(M * K));
            for (int g0 = lane; g0 < cnt; g0 += 64 * SB) {  // the 16 lanes of a row stay together
                uint32_t h[SB][XW];
#pragma unroll
                for (int b = 0; b < SB; ++b) {
                    int m, c, i;
                    group_of(g0 + 64 * b, m, c, i);
                    const int k0 = ks + 256 * c + 16 * i;
                    const bool ok = g0 + 64 * b < cnt && k0 < K;
                    if (FAST) {
                        if constexpr (FUSED) {
                            const uint32_t off = ok ? (uint32_t)((m * K + k0) * 2) : kOOB;
                            const uint4 v0 = buf_load16(x_rsrc, off), v1 = buf_load16(x_rsrc, off + 16);
                            h[b][0] = v0.x; h[b][1] = v0.y; h[b][2] = v0.z; h[b][3] = v0.w;
                            h[b][4] = v1.x; h[b][5] = v1.y; h[b][6] = v1.z; h[b][7] = v1.w;
                        } else {
                            const uint4 v = buf_load16(x_rsrc, ok ? (uint32_t)(m * K + k0) : kOOB);
                            h[b][0] = v.x; h[b][1] = v.y; h[b][2] = v.z; h[b][3] = v.w;
                        }
                    } else if (g0 + 64 * b < cnt) {
                        if constexpr (FUSED) {
                            load_x16_bf16_elems(p.xb, K, m, k0, h[b]);
                        } else {
                            const int8_t* src = p.xq + (int64_t)m * K + k0;
                            uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                            for (int j = 0; j < 16; ++j)
                                if (k0 + j < K) d[j >> 2] |= (uint32_t)(uint8_t)src[j] << (8 * (j & 3));
#pragma unroll
                            for (int j = 0; j < 4; ++j) h[b][j] = d[j];
                        }
                    }
                }
#pragma unroll
                for (int b = 0; b < SB; ++b) {
                    if (g0 + 64 * b < cnt) {  // uniform over the 16 lanes of a row
                        int m, c, i;
                        group_of(g0 + 64 * b, m, c, i);
                        const int k0 = ks + 256 * c + 16 * i;
                        uint32_t e[4];
                        if constexpr (FUSED) {
                            quant16_t(h[b], fused_scale(m), e);
                            if (blockIdx.x == 0 && p.xq_out) {
                                uint32_t d[4];
                                untranspose(e, d);
                                store_codes16<FAST>(p.xq_out, K, m, k0, d);
                            }
                        } else {
                            transpose4x4_bytes(h[b], e);
                        }
                        const int rs = row16_sum(put_group_t(x_lds, KSP, m, 16 * c + i, e));
                        if (row_leader) atomicAdd(&s_wsum[wave * kSkMaxM + m], rs);
                    }
                }
            }
            if (ks > 0) load_batch(wa, 0, stage_off, nch);  // stage 0's: before the scan
        }
        // The activations this wave multiplies are its own LDS writes, and the LDS
        // operations of a wave complete in order; keep the compiler from hoisting reads.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();

        // ---- stream the packed weights of this stage ----
        if constexpr (SINGLE) {
            compute_batch(wa, 0, nch);
        } else {
            const int cpw = chunks_of_wave(0, nch);  // chunks per wave (wave 0 has the most)
            uint4 wb[U * NW];
            for (int j0 = 0; j0 < cpw; j0 += 2 * U) {
                load_batch(wb, j0 + U, stage_off, nch);  // zeros when past the stage
                compute_batch(wa, j0, nch);
                if (j0 + U >= cpw) break;
                load_batch(wa, j0 + 2 * U, stage_off, nch);
                compute_batch(wb, j0 + U, nch);
            }
        }
    };
    if constexpr (XH > 0) {
        run_stage(0);  // a single K stage
    } else {
        for (int ks = 0; ks < p.Kp; ks += p.KS) run_stage(ks);
    }

    // ---- combine the four waves' partials and write the outputs ----
    // 1/a: v_rcp_f32 is within 1 ulp, and the rescale below stays within 3 ulp
    if constexpr (MC == 1) {
        if (FUSED && blockIdx.x == 0 && tid == 0 && p.a_out) p.a_out[0] = a_m1;
    } else if (tid < M) {
        const float a = FUSED ? fused_scale(tid) : a_in;
        if (FUSED && blockIdx.x == 0 && p.a_out) p.a_out[tid] = a;
        s_inva[tid] = __builtin_amdgcn_rcpf(a);
    }
    constexpr int kRedSet = kSkWaves * MT * 4 * 64;  // ints per matrix in `red`
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        if constexpr (MC == 1) {
            // row 0 of the accumulators: register 0 of lanes 0-15
            if (lane < 16)
                red[v * kRedSet + wave * 256 + lane] =
                    acc1[v][0][0] + (acc4[v][0][0] >> 2) + (acc16[v][0][0] >> 4) - wsum_m1;
        } else {
            // this wave's partials minus the code sums of the activations it staged (its
            // own LDS slots, so no barrier is needed to read them)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4i s4 = acc1[v][t] + (acc4[v][t] >> 2) + (acc16[v][t] >> 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * t + 4 * (lane >> 4) + r;
                    if (m < M)
                        red[v * kRedSet + ((wave * MT + t) * 4 + r) * 64 + lane] =
                            s4[r] - s_wsum[wave * kSkMaxM + m];
                }
            }
        }
    }
    __syncthreads();
    if constexpr (NR == 2) {
        // one token, two row tiles: thread tid < 32 writes column tid % 16 of tile tid / 16
        if (tid < 32) {
            const bool hi = tid >= 16;
            const int col = tid & 15;
            if (col < (hi ? rows_v[1] : rows_v[0])) {
                int acc = 0;
#pragma unroll
                for (int w = 0; w < kSkWaves; ++w) acc += red[(hi ? kRedSet : 0) + w * 256 + col];
                const float inv_a = __builtin_amdgcn_rcpf(FUSED ? a_m1 : a_in);
                store_out(out, (int64_t)(hi ? nv0[1] : nv0[0]) + col, p.out_dtype, acc,
                          hi ? ws_n[1] : ws_n[0], inv_a);
            }
        }
        return;
    }
    for (int idx = tid; idx < 16 * M; idx += kSkThreads) {
        // 16x16 int32 accumulator layout: lane l, register r -> row 4*(l/16)+r, column l%16
        const int m = idx >> 4, col = idx & 15;
        const int t = m >> 4, ml = m & 15;
        const int l = 16 * (ml >> 2) + col, r = ml & 3;
        if (col < rows) {
            int acc[NW];
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                acc[v] = 0;
#pragma unroll
                for (int w = 0; w < kSkWaves; ++w) acc[v] += red[v * kRedSet + ((w * MT + t) * 4 + r) * 64 + l];
            }
            const float inv_a = MC == 1 ? __builtin_amdgcn_rcpf(FUSED ? a_m1 : a_in) : s_inva[m];
            // the first pass holds its column's weight scale (loaded early); later passes
            // (M > 16) read it again
            const int64_t o = (int64_t)m * N + n0 + col;
            if constexpr (PAIR) {
                // h = silu(g) * u with g, u the two products rescaled exactly as a plain
                // output (fp32, same roundings); silu(g) = g / (1 + exp(-g))
                const float g = ((float)acc[0] * (idx == tid ? ws_n[0] : w_scale_v[0][n0 + col])) * inv_a;
                const float u = ((float)acc[1] * (idx == tid ? ws_n[1] : w_scale_v[1][n0 + col])) * inv_a;
                const float h = (g / (1.0f + expf(-g))) * u;
                if (p.out_dtype == 0)
                    static_cast<float*>(out)[o] = h;
                else
                    static_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(h);
            } else {
                const float wsc = idx == tid ? ws_n[0] : w_scale_v[0][n0 + col];
                store_out(out, o, p.out_dtype, acc[0], wsc, inv_a);
            }
        }
    }
}

// Dynamic LDS beyond the default 64 KB limit must be granted per kernel and device.
// Each instantiation of launch_one grants its kernel the whole 160 KB a block may use
// (so no later, larger request needs a second grant), once per device; the flags are
// atomics, so concurrent first calls at worst repeat the idempotent grant.
constexpr int kSkMaxDevices = 64;
constexpr int kSkLdsMax = 160 * 1024;

template <bool FUSED, bool FAST, int XH, int U, bool SINGLE, int MC = 0, int MT = 1, bool PAIR = false,
          int NR = 1>
hipError_t launch_one(const SkinnyArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
    static std::atomic<bool> granted[kSkMaxDevices];
    auto* kernel = &skinny_kernel<FUSED, FAST, XH, U, SINGLE, MC, MT, PAIR, NR>;
    if (lds > 65536) {
        if (lds > (size_t)kSkLdsMax) return hipErrorInvalidValue;
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kSkMaxDevices) return hipErrorInvalidDevice;
        if (!granted[dev].load(std::memory_order_acquire)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kSkLdsMax);
            if (e != hipSuccess) return e;
            granted[dev].store(true, std::memory_order_release);
        }
    }
    hipLaunchKernelGGL(kernel, grid, dim3(kSkThreads), lds, stream, a);
    return hipGetLastError();
}

// Batch shape: U = 4 or 8 chunks per wave; SINGLE when one batch holds a wave's share.
template <bool FUSED, int XH, bool PAIR = false>
hipError_t launch_fast(const SkinnyArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
    const int cpw = chunks_of_wave(0, a.KS / 256);
    const bool one_stage = a.KS >= a.Kp;
    if (one_stage && cpw <= 4) return launch_one<FUSED, true, XH, 4, true, 0, 1, PAIR>(a, grid, lds, stream);
    if (one_stage && cpw <= 8) return launch_one<FUSED, true, XH, 8, true, 0, 1, PAIR>(a, grid, lds, stream);
    return launch_one<FUSED, true, XH, 8, false, 0, 1, PAIR>(a, grid, lds, stream);
}

// One token (decode), a single K stage of at most 32 chunks per wave: the M = 1
// specializations, by K.
template <bool FUSED, bool PAIR = false, int NR = 1>
hipError_t launch_m1(const SkinnyArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
    const int cpw = chunks_of_wave(0, a.Kp / 256);
    // more than one round of runs, and three chunks per wave at most under the spread
    // deal (9 to 12 chunks): one batch of exactly three
    if (a.Kp / 256 > kSkRun * kSkWaves && chunks_of_wave_spread(0, a.Kp / 256) <= 3)
        return launch_one<FUSED, true, 1, 3, true, 1, 1, PAIR, NR>(a, grid, lds, stream);
    if (cpw <= 4) return launch_one<FUSED, true, 1, 4, true, 1, 1, PAIR, NR>(a, grid, lds, stream);
    if (cpw <= 8) return launch_one<FUSED, true, 2, 8, true, 1, 1, PAIR, NR>(a, grid, lds, stream);
    if (cpw <= 16) return launch_one<FUSED, true, 4, 8, false, 1, 1, PAIR, NR>(a, grid, lds, stream);
    return launch_one<FUSED, true, 8, 8, false, 1, 1, PAIR, NR>(a, grid, lds, stream);
}
bool m1_fits(const SkinnyArgs& a) {
    return a.M == 1 && a.KS >= a.Kp && chunks_of_wave(0, a.Kp / 256) <= 32;
}

// Held activation groups per lane: M * (chunks per wave) * 16 groups over 64 lanes.
template <bool FUSED, bool PAIR = false>
hipError_t launch_held(const SkinnyArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
    const int cpw = chunks_of_wave(0, a.Kp / 256);
    const int per_lane = (a.M * cpw + 3) / 4;
    if (m1_fits(a)) return launch_m1<FUSED, PAIR>(a, grid, lds, stream);
    if (a.KS >= a.Kp) {
        if (per_lane <= 1) return launch_fast<FUSED, 1, PAIR>(a, grid, lds, stream);
        if (per_lane <= 2) return launch_fast<FUSED, 2, PAIR>(a, grid, lds, stream);
        if (per_lane <= 4) return launch_fast<FUSED, 4, PAIR>(a, grid, lds, stream);
        if (per_lane <= 8) return launch_fast<FUSED, 8, PAIR>(a, grid, lds, stream);
    }
    return launch_fast<FUSED, 0, PAIR>(a, grid, lds, stream);
}

// K stage length: the activations of a stage (M rows) fit the LDS budget.
void set_stage(SkinnyArgs& a, int64_t M, int64_t K) {
    a.M = (int)M;
    a.K = (int)K;
    a.Kp = (int)((K + 255) / 256 * 256);
    int ks = ((kSkXBudget / (int)M) - 16) / 256 * 256;
    if (ks < 256) ks = 256;
    a.KS = ks < a.Kp ? ks : a.Kp;
}

}  // namespace

hipError_t launch_skinny(const int8_t* xq, const float* a_scale, const uint16_t* x_bf16,
                         const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                         int64_t K, void* out, int out_dtype, int8_t* xq_out, float* a_out,
                         hipStream_t stream) {
    return launch_skinny_grouped(xq, a_scale, x_bf16, 1, &packed, &w_scale, &N, &out, M, K,
                                 out_dtype, xq_out, a_out, stream);
}

hipError_t launch_skinny_grouped(const int8_t* xq, const float* a_scale, const uint16_t* x_bf16,
                                 int groups, const uint8_t* const* packed,
                                 const float* const* w_scale, const int64_t* N,
                                 void* const* out, int64_t M, int64_t K, int out_dtype,
                                 int8_t* xq_out, float* a_out, hipStream_t stream) {
    if (groups < 1 || groups > kSkGroups) return hipErrorInvalidValue;
    SkinnyArgs a = {};
    a.xq = xq;
    a.a_scale = a_scale;
    a.xb = x_bf16;
    a.xq_out = xq_out;
    a.a_out = a_out;
    a.groups = groups;
    set_stage(a, M, K);
    a.out_dtype = out_dtype;
    // One token over many rows: blocks of two 16-row tiles, so half as many blocks read
    // (and, fused, quantize) the activations.
    int64_t blocks16 = 0;
    for (int g = 0; g < groups; ++g) blocks16 += (N[g] + 15) / 16;
    const int nr = (K % 64 == 0 && m1_fits(a) && blocks16 >= kSkTwoTileMinBlocks) ? 2 : 1;
    int64_t blocks = 0;
    for (int g = 0; g < kSkGroups; ++g) {
        const bool live = g < groups;
        a.first[g] = (int)blocks;
        a.g_N[g] = live ? (int)N[g] : 0;
        a.g_packed[g] = live ? packed[g] : nullptr;
        a.g_wscale[g] = live ? w_scale[g] : nullptr;
        a.g_out[g] = live ? out[g] : nullptr;
        if (live) blocks += (N[g] + 16 * nr - 1) / (16 * nr);
    }
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const size_t lds = (size_t)M * (a.KS + 16) + kSkMisc + (size_t)nr * kSkWaves * 4 * 64 * 4;
    const dim3 grid((unsigned)blocks);
    const bool fused = x_bf16 != nullptr;
    if (nr == 2)
        return fused ? launch_m1<true, false, 2>(a, grid, lds, stream)
                     : launch_m1<false, false, 2>(a, grid, lds, stream);
    if (M > 16) {
        if (fused) return hipErrorInvalidValue;  // the fused entry point takes M <= 16
        // 17..64 tokens (int8 input only): 2 or 4 token tiles per chunk of weights.  The
        // activations of a K stage sit in LDS (up to 160 KB); a stage holds at least one
        // full round of chunk runs, so that every wave has work.
        const int mt = M <= 32 ? 2 : 4;
        const size_t red_bytes = (size_t)kSkWaves * mt * 4 * 64 * 4;
        const size_t budget = 160 * 1024 - kSkMisc - red_bytes;
        constexpr int round = 256 * kSkRun * kSkWaves;  // weights per round of chunk runs
        int kst = (int)((budget / M - 16) / round) * round;
        if (kst < round) kst = round;
        a.KS = kst < a.Kp ? kst : a.Kp;
        const size_t lds_m = (size_t)M * (a.KS + 16) + kSkMisc + red_bytes;
        if (K % 64 != 0) {
            if (mt == 2) return launch_one<false, false, 0, 4, false, 0, 2>(a, grid, lds_m, stream);
            return launch_one<false, false, 0, 4, false, 0, 4>(a, grid, lds_m, stream);
        }
        if (mt == 2) return launch_one<false, true, 0, 4, false, 0, 2>(a, grid, lds_m, stream);
        return launch_one<false, true, 0, 4, false, 0, 4>(a, grid, lds_m, stream);
    }
    if (K % 64 != 0) {
        if (fused) return launch_one<true, false, 0, 4, false>(a, grid, lds, stream);
        return launch_one<false, false, 0, 4, false>(a, grid, lds, stream);
    }
    return fused ? launch_held<true>(a, grid, lds, stream) : launch_held<false>(a, grid, lds, stream);
}

hipError_t launch_skinny_swiglu(const uint16_t* x_bf16, const uint8_t* packed_gate,
                                const float* w_scale_gate, const uint8_t* packed_up,
                                const float* w_scale_up, int64_t M, int64_t N, int64_t K,
                                void* out, int out_dtype, int8_t* xq_out, float* a_out,
                                hipStream_t stream) {
    if (M < 1 || M > 16 || N < 1 || out_dtype == 2) return hipErrorInvalidValue;
    SkinnyArgs a = {};
    a.xb = x_bf16;
    a.xq_out = xq_out;
    a.a_out = a_out;
    a.groups = 1;  // the blocks cover N rows once; each reads gate (0) and up (1)
    a.g_N[0] = a.g_N[1] = (int)N;
    a.g_packed[0] = packed_gate;
    a.g_packed[1] = packed_up;
    a.g_wscale[0] = w_scale_gate;
    a.g_wscale[1] = w_scale_up;
    a.g_out[0] = out;
    set_stage(a, M, K);
    a.out_dtype = out_dtype;
    const size_t lds = (size_t)M * (a.KS + 16) + kSkMisc + (size_t)2 * kSkWaves * 4 * 64 * 4;
    const dim3 grid((unsigned)((N + 15) / 16));
    if (K % 64 != 0) return launch_one<true, false, 0, 4, false, 0, 1, true>(a, grid, lds, stream);
    return launch_held<true, true>(a, grid, lds, stream);
}

}  // namespace bitnet
