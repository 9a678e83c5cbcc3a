// ceilings.hip -- two microbenchmarks that measure what this chip sustains, reported
// beside the roofline fractions so that a fraction of the datasheet peak can be read
// against what is attainable here.  They are not part of the BitLinear path and live in
// their own library (libbitnet_probes.so).
//
//  * bitnet_probe_mfma_i8: every wave runs NACC independent v_mfma_i32_32x32x32_i8
//    accumulator chains on register operands drawn from seeded random words (matrix-core
//    power, and so the sustained clock, depends on the operand values), no memory
//    traffic inside the loop.  ops = 2 * 32 * 32 * 32 * NACC * iters per wave.  When a
//    clock buffer is given, the first lane of every wave also records the core-cycle
//    counter and the constant-rate wall counter around its loop, so the host can read
//    the clock the matrix cores sustained (cycles / wall ticks x the wall rate).
//  * bitnet_probe_read: a streaming read of 16-byte words, each block over its own
//    contiguous share, XOR-folded into one word per thread (so the loads cannot be
//    dropped).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
constexpr int kNacc = 8;
constexpr int kSeedWords = 4096;

__global__ __launch_bounds__(256) void mfma_i8_loop(const int32_t* __restrict__ seed, int iters,
                                                    int32_t* __restrict__ out,
                                                    uint64_t* __restrict__ clk) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int b = (t * 8) & (kSeedWords - 1);
    v4i A = {seed[b], seed[b + 1], seed[b + 2], seed[b + 3]};
    v4i B = {seed[b + 4], seed[b + 5], seed[b + 6], seed[b + 7]};
    v16i acc[kNacc];
#pragma unroll
    for (int j = 0; j < kNacc; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0;
    const uint64_t c0 = (uint64_t)clock64(), w0 = (uint64_t)wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kNacc; ++j)
            acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, acc[j], 0, 0, 0);
    }
    // read once the last products are issued; the few hundred cycles they still take are
    // negligible next to the loop's millions
    const uint64_t c1 = (uint64_t)clock64(), w1 = (uint64_t)wall_clock64();
    if (clk && (threadIdx.x & 63) == 0) {
        const int wv = t >> 6;
        clk[2 * wv] = c1 - c0;
        clk[2 * wv + 1] = w1 - w0;
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < kNacc; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[t] = s;
}

// Each block streams its own contiguous share of the buffer, eight 16-byte loads in
// flight per thread (contiguous per-block regions sustain more than a grid-stride walk).
__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ src, int64_t n,
                                                   uint32_t* __restrict__ out) {
    // every pass issues its U loads (predicated past the share's end) before any is
    // used, so a thread with a short share still waits for one memory trip per pass
    constexpr int U = 8;
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < n ? lo + per : n;
    uint32_t a = 0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += U * 256) {
        uint4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = i + u * 256 < hi ? src[i + u * 256] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int u = 0; u < U; ++u) a ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = a;
}

}  // namespace

extern "C" {

// seed: kSeedWords (4096) int32 words on the device; out: blocks * 256 int32 words;
// clk: NULL, or blocks * 4 * 2 uint64 words (per wave: core cycles, wall ticks of its loop).
// Returns a hipError_t value (0 = launched).
int bitnet_probe_mfma_i8(const int32_t* seed, int32_t* out, uint64_t* clk, int blocks,
                         int iters, void* stream) {
    if (!seed || !out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_i8_loop, dim3((unsigned)blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), seed, iters, out, clk);
    return (int)hipGetLastError();
}

// Frequency (Hz) of the constant-rate wall counter of the current device, 0 on error.
double bitnet_probe_wall_clock_hz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0.0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0.0;
    return 1e3 * (double)khz;
}

// Operations one bitnet_probe_mfma_i8 launch performs.
double bitnet_probe_mfma_i8_ops(int blocks, int iters) {
    return 2.0 * 32 * 32 * 32 * kNacc * (double)iters * blocks * 4;
}

// src: n16 16-byte words on the device (16-byte aligned); out: blocks * 256 uint32 words.
int bitnet_probe_read(const void* src, int64_t n16, uint32_t* out, int blocks, void* stream) {
    if (!src || !out || n16 < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read, dim3((unsigned)blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const uint4*>(src), n16,
                       out);
    return (int)hipGetLastError();
}

}  // extern "C"
