// pack_quant.hip -- offline weight packing and per-token activation quantization for
// gfx950.
//
// Weight packing follows "BitNet 深度实战" (chenxutan.com) §2.4 (per-row absmean scale,
// round, clamp to {-1,0,+1}) and §4.3 (four 2-bit weights per byte, the first in the
// low bits), with code = w + 1, into the (N, K/4) uint8 array of "BitNet-Triton"
// (zingnex.cn) 技术架构 §1.  Activation quantization follows "BitNet-Triton" 技术架构 §3
// (one fused launch) with the per-token absmax scale 127 / max|x|.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bitnet {

// ---------------------------------------------------------------- weight scale ---
// The absmean of each row is an fp64 sum over k in ascending order (a fixed order, so
// the scale is reproducible bit for bit), divided by K, rounded once to fp32 and clamped
// below at 1e-5.  A block owns kScRows rows: its four waves load 64-column tiles of
// them with coalesced 16-byte reads into LDS, and lane r of the first wave adds row r's
// 64 values of the tile in order while the next tile is already in flight.
constexpr int kScRows = 64, kScCols = 64, kScStride = kScCols + 1;

__global__ __launch_bounds__(256) void weight_scale_kernel(const float* __restrict__ w,
                                                           int64_t N, int64_t K,
                                                           float* __restrict__ scale) {
    __shared__ float tile[kScRows * kScStride];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * kScRows;
    const int rows = (int)min((int64_t)kScRows, N - r0);
    const int64_t ntiles = (K + kScCols - 1) / kScCols;
    // thread tid moves the 16-byte pieces p = tid + 256 j (row p / 16, columns 4 (p % 16) ..)
    constexpr int kPieces = kScRows * kScCols / 4 / 256;
    float4 held[kPieces];
    auto load = [&](int64_t t) {
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
            const int piece = tid + 256 * j, row = piece >> 4;
            const int64_t col = t * kScCols + 4 * (piece & 15);
            // K % 4 == 0: a piece is either wholly inside the row or wholly past its end
            held[j] = (row < rows && col < K)
                          ? *reinterpret_cast<const float4*>(w + (r0 + row) * K + col)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    double sum = 0.0;
    load(0);
    for (int64_t t = 0; t < ntiles; ++t) {
        __syncthreads();  // the previous tile has been summed
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
            const int piece = tid + 256 * j;
            float* dst = &tile[(piece >> 4) * kScStride + 4 * (piece & 15)];
            dst[0] = held[j].x;
            dst[1] = held[j].y;
            dst[2] = held[j].z;
            dst[3] = held[j].w;
        }
        __syncthreads();
        if (t + 1 < ntiles) load(t + 1);
        if (tid < kScRows) {
            const int cols = (int)min((int64_t)kScCols, K - t * kScCols);
            const float* src = &tile[tid * kScStride];
            for (int c = 0; c < cols; ++c) sum += fabs((double)src[c]);
        }
    }
    if (tid < rows) {
        const float s = (float)(sum / (double)K);
        scale[r0 + tid] = s < 1e-5f ? 1e-5f : s;
    }
}

// ---------------------------------------------------------------- weight codes ---
// One thread per packed byte (4 weights): q = clamp(rne(w / s), -1, 1) with one IEEE
// fp32 division, code = q + 1 in bits 2i..2i+1.
__global__ __launch_bounds__(256) void weight_codes_kernel(const float* __restrict__ w,
                                                           const float* __restrict__ scale,
                                                           int64_t N, int64_t K,
                                                           uint8_t* __restrict__ packed) {
    const int64_t kb = K / 4;
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * kb) return;
    int64_t n = idx / kb;
    const float s = scale[n];
    const float4 v = *reinterpret_cast<const float4*>(w + idx * 4);
    const float vals[4] = {v.x, v.y, v.z, v.w};
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float r = rintf(vals[i] / s);
        r = fminf(fmaxf(r, -1.0f), 1.0f);
        byte |= (uint32_t)((int)r + 1) << (2 * i);
    }
    packed[idx] = (uint8_t)byte;
}

// One thread per packed byte -> four int8 codes (inspection / tests).
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ packed,
                                                     int64_t total_bytes,
                                                     int8_t* __restrict__ codes) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total_bytes) return;
    uint32_t b = packed[idx];
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) out |= (uint32_t)(uint8_t)((int)((b >> (2 * i)) & 3u) - 1) << (8 * i);
    *reinterpret_cast<uint32_t*>(codes + idx * 4) = out;
}

// ------------------------------------------------------- activation quantization ---
// A token row is taken by WPR waves (1, 2 or 4) of a 256-thread block, 4 / WPR rows per
// block: few rows get more waves each, so that a launch has enough waves in flight.  Lane
// l of the row's waves takes the V-element groups l, l + 64 WPR, ... (V = 8, 16-byte
// loads, when K % 8 == 0, else 4).  Pass 1: max |x| as the integer max of the bf16
// magnitude bits (monotone in |x| for finite values), reduced across the wave and, with
// WPR > 1, across the row's waves through LDS (one barrier).  Pass 2: a = 127 /
// max(amax, 1e-5) (IEEE division), q = clamp(rne(x * a), +-127).  Rows of up to G groups
// per lane keep their loads in registers between the passes (all issued before the first
// use); longer rows (G == 0) read the row twice, the second time from cache.
// MODE 0: per-token scale (both passes).  Per-tensor scale, three launches: MODE 1 runs
// pass 1 only and leaves the row's max magnitude bits in a_scale[m]; tensor_scale_kernel
// reduces them and writes the common scale to every a_scale[m]; MODE 2 runs pass 2 with
// the scale read from a_scale[m].
template <int V>
struct QVec {
    uint32_t w[V / 2];  // V bf16 values, two per word, low half first
};

template <int V>
__device__ __forceinline__ QVec<V> load_qvec(const uint16_t* row, int64_t g) {
    QVec<V> v;
    if constexpr (V == 8) {
        const uint4 t = reinterpret_cast<const uint4*>(row)[g];
        v.w[0] = t.x; v.w[1] = t.y; v.w[2] = t.z; v.w[3] = t.w;
    } else {
        const uint2 t = reinterpret_cast<const uint2*>(row)[g];
        v.w[0] = t.x; v.w[1] = t.y;
    }
    return v;
}

template <int V>
__device__ __forceinline__ uint32_t qvec_max_bits(const QVec<V>& v, uint32_t mx) {
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
        const uint32_t a = v.w[i] & 0x7FFF7FFFu;
        mx = max(mx, max(a & 0xFFFFu, a >> 16));
    }
    return mx;
}

template <int G, int MODE, int V, int WPR>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                        int64_t M, int64_t K,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ a_scale) {
    static_assert(V == 4 || V == 8, "elements per load");
    static_assert(WPR == 1 || WPR == 2 || WPR == 4, "waves per row");
    constexpr int kRows = 4 / WPR, kStride = 64 * WPR;
    __shared__ uint32_t s_max[4];
    const int wave = threadIdx.x >> 6;
    const int lr = (wave % WPR) * 64 + (threadIdx.x & 63);  // lane within the row's waves
    const int64_t m = (int64_t)blockIdx.x * kRows + wave / WPR;
    // with one wave per row a finished wave leaves; with more, every wave reaches the
    // barrier and rows past M only skip their loads and stores
    if (WPR == 1 && m >= M) return;
    const bool live = m < M;
    const int64_t groups = live ? K / V : 0;
    const uint16_t* row = x + (live ? m : 0) * K;

    QVec<V> held[G > 0 ? G : 1];
    uint32_t mx = 0;
    if (G > 0) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int64_t g = lr + (int64_t)i * kStride;
            if (g < groups) {
                held[i] = load_qvec<V>(row, g);
            } else {
#pragma unroll
                for (int t = 0; t < V / 2; ++t) held[i].w[t] = 0u;
            }
        }
        if (MODE != 2) {
#pragma unroll
            for (int i = 0; i < G; ++i) mx = qvec_max_bits<V>(held[i], mx);
        }
    } else if (MODE != 2) {
        for (int64_t g = lr; g < groups; g += kStride) mx = qvec_max_bits<V>(load_qvec<V>(row, g), mx);
    }
    float a = 0.0f;
    if constexpr (MODE == 2) {
        if (live) a = a_scale[m];
    } else {
        mx = wave_max_u32(mx);
        if constexpr (WPR > 1) {
            if ((threadIdx.x & 63) == 0) s_max[wave] = mx;
            __syncthreads();
            const int w0 = wave - wave % WPR;
            mx = s_max[w0];
#pragma unroll
            for (int w = 1; w < WPR; ++w) mx = max(mx, s_max[w0 + w]);
        }
        if constexpr (MODE == 1) {
            if (live && lr == 0) reinterpret_cast<uint32_t*>(a_scale)[m] = mx;  // bits of max |x|
            return;
        }
        float amax = bf16_bits_to_f32(mx);
        amax = amax < 1e-5f ? 1e-5f : amax;
        a = 127.0f / amax;
        if (live && lr == 0) a_scale[m] = a;
    }

    // V codes per group: one word (V = 4) or two (V = 8)
    auto quantv = [&](const QVec<V>& v, uint32_t (&packed)[V / 4]) {
#pragma unroll
        for (int w = 0; w < V / 4; ++w) {
            const uint32_t h[4] = {v.w[2 * w] & 0xFFFFu, v.w[2 * w] >> 16, v.w[2 * w + 1] & 0xFFFFu,
                                   v.w[2 * w + 1] >> 16};
            uint32_t p = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float r = rintf(bf16_bits_to_f32(h[j]) * a);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                p |= ((uint32_t)(int)r & 0xFFu) << (8 * j);
            }
            packed[w] = p;
        }
    };
    auto store = [&](int64_t g, const uint32_t (&packed)[V / 4]) {
        if constexpr (V == 8)
            reinterpret_cast<uint2*>(xq + m * K)[g] = make_uint2(packed[0], packed[1]);
        else
            reinterpret_cast<uint32_t*>(xq + m * K)[g] = packed[0];
    };
    if (G > 0) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int64_t g = lr + (int64_t)i * kStride;
            if (g < groups) {
                uint32_t packed[V / 4];
                quantv(held[i], packed);
                store(g, packed);
            }
        }
    } else {
        for (int64_t g = lr; g < groups; g += kStride) {
            uint32_t packed[V / 4];
            quantv(load_qvec<V>(row, g), packed);
            store(g, packed);
        }
    }
}

// One block: the tensor's max magnitude from the rows' (a_scale[m] holds the bits of the
// bf16 max |x| of row m), then a = 127 / max(amax, 1e-5) into every a_scale[m].
__global__ __launch_bounds__(256) void tensor_scale_kernel(int64_t M, float* __restrict__ a_scale) {
    __shared__ uint32_t s_max[4];
    const int tid = threadIdx.x;
    uint32_t mx = 0;
    const uint32_t* bits = reinterpret_cast<const uint32_t*>(a_scale);
    for (int64_t m = tid; m < M; m += 256) mx = max(mx, bits[m]);
    mx = wave_max_u32(mx);
    if ((tid & 63) == 0) s_max[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    float amax = bf16_bits_to_f32(mx);
    amax = amax < 1e-5f ? 1e-5f : amax;
    const float a = 127.0f / amax;
    for (int64_t m = tid; m < M; m += 256) a_scale[m] = a;
}

// ------------------------------------------------------------- code tables ---
// Field value -> weight for a table, -2 for a code the table leaves unused.
//   table 0 (this library): code = w + 1  (00 -> -1, 01 -> 0, 10 -> +1, 11 unused)
//   table 1 ("BitNet 深度实战" §4.3):      (00 -> 0, 01 -> -1, 11 -> +1, 10 unused)
__device__ __forceinline__ int code_to_weight(int table, uint32_t c) {
    if (table == 0) return c == 3u ? -2 : (int)c - 1;
    return c == 0u ? 0 : (c == 1u ? -1 : (c == 3u ? 1 : -2));
}
__device__ __forceinline__ uint32_t weight_to_code(int table, int w) {
    if (table == 0) return (uint32_t)(w + 1);
    return w == 0 ? 0u : (w < 0 ? 1u : 3u);
}

// One thread per 4 packed bytes (16 weights); fields keep their positions.  A field
// holding its table's unused code becomes weight 0 and is counted in *invalid (if
// given).
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* in,
                                                     int64_t bytes, int from, int to,
                                                     uint8_t* out,  // may alias in
                                                     int* __restrict__ invalid) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= bytes) return;
    const int n = bytes - i < 4 ? (int)(bytes - i) : 4;
    uint32_t d = 0;
    for (int b = 0; b < n; ++b) d |= (uint32_t)in[i + b] << (8 * b);
    uint32_t r = 0;
    int bad = 0;
#pragma unroll
    for (int f = 0; f < 16; ++f) {
        int w = code_to_weight(from, (d >> (2 * f)) & 3u);
        if (w == -2) {
            ++bad;
            w = 0;
        }
        r |= weight_to_code(to, w) << (2 * f);
    }
    for (int b = 0; b < n; ++b) out[i + b] = (uint8_t)(r >> (8 * b));
    if (bad && invalid) atomicAdd(invalid, bad);
}

// ------------------------------------------------------------------ launchers ---

hipError_t launch_pack_weights(const float* w, int64_t N, int64_t K, uint8_t* packed,
                               float* scale, hipStream_t stream) {
    dim3 blk(256);
    hipLaunchKernelGGL(weight_scale_kernel, dim3((unsigned)((N + kScRows - 1) / kScRows)), blk, 0,
                       stream, w, N, K, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t total = N * (K / 4);
    hipLaunchKernelGGL(weight_codes_kernel, dim3((unsigned)((total + 255) / 256)), blk, 0,
                       stream, w, scale, N, K, packed);
    return hipGetLastError();
}

hipError_t launch_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* codes,
                                 hipStream_t stream) {
    int64_t total = N * (K / 4);
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       packed, total, codes);
    return hipGetLastError();
}

template <int MODE, int V, int WPR>
hipError_t launch_quant_rows_w(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                               float* a_scale, hipStream_t stream) {
    const int64_t groups = K / V;
    const int64_t per_lane = (groups + 64 * WPR - 1) / (64 * WPR);
    constexpr int kRows = 4 / WPR;
    dim3 grid((unsigned)((M + kRows - 1) / kRows)), blk(256);
    if (per_lane <= 2)
        hipLaunchKernelGGL((quant_act_kernel<2, MODE, V, WPR>), grid, blk, 0, stream, x, M, K, xq, a_scale);
    else if (per_lane <= 4)
        hipLaunchKernelGGL((quant_act_kernel<4, MODE, V, WPR>), grid, blk, 0, stream, x, M, K, xq, a_scale);
    else if (per_lane <= 8)
        hipLaunchKernelGGL((quant_act_kernel<8, MODE, V, WPR>), grid, blk, 0, stream, x, M, K, xq, a_scale);
    else if (per_lane <= 16)
        hipLaunchKernelGGL((quant_act_kernel<16, MODE, V, WPR>), grid, blk, 0, stream, x, M, K, xq, a_scale);
    else
        hipLaunchKernelGGL((quant_act_kernel<0, MODE, V, WPR>), grid, blk, 0, stream, x, M, K, xq, a_scale);
    return hipGetLastError();
}

// Waves per row: enough waves in the launch (about 2048, eight per CU) to cover the
// memory latency, one per row once M alone provides them -- but, up to four, enough that
// a lane holds at most four groups of its row: a long row is then read once, with all its
// loads issued together, instead of twice in a loop, and by more waves (2048 x 14336:
// 33.3 -> 19.3 us; 2048 x 4096: 7.9 -> 7.2 us).
template <int MODE, int V>
hipError_t launch_quant_rows_v(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                               float* a_scale, hipStream_t stream) {
    int wpr = M <= 512 ? 4 : (M <= 1024 ? 2 : 1);
    while (wpr < 4 && (K / V + 64 * wpr - 1) / (64 * wpr) > 4) wpr *= 2;
    if (wpr == 4) return launch_quant_rows_w<MODE, V, 4>(x, M, K, xq, a_scale, stream);
    if (wpr == 2) return launch_quant_rows_w<MODE, V, 2>(x, M, K, xq, a_scale, stream);
    return launch_quant_rows_w<MODE, V, 1>(x, M, K, xq, a_scale, stream);
}

// 16-byte loads when rows are whole 8-element groups (K % 8 == 0), else 8-byte ones
template <int MODE>
hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* a_scale,
                             hipStream_t stream) {
    if (K % 8 == 0) return launch_quant_rows_v<MODE, 8>(x, M, K, xq, a_scale, stream);
    return launch_quant_rows_v<MODE, 4>(x, M, K, xq, a_scale, stream);
}

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* a_scale,
                            hipStream_t stream) {
    return launch_quant_rows<0>(x, M, K, xq, a_scale, stream);
}

hipError_t launch_quant_act_per_tensor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                                       float* a_scale, hipStream_t stream) {
    hipError_t e = launch_quant_rows<1>(x, M, K, xq, a_scale, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(256), 0, stream, M, a_scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_quant_rows<2>(x, M, K, xq, a_scale, stream);
}

hipError_t launch_repack_codes(const uint8_t* in, int64_t N, int64_t K, int from, int to,
                               uint8_t* out, int* invalid, hipStream_t stream) {
    const int64_t bytes = N * (K / 4);
    const int64_t threads = (bytes + 3) / 4;
    hipLaunchKernelGGL(repack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, in, bytes, from, to, out, invalid);
    return hipGetLastError();
}

}  // namespace bitnet
