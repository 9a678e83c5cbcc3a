// api.hip -- the extern "C" entry points declared in include/bitnet_w2a8.h.
//
// Every entry point validates its arguments on the host, before any HIP call, and
// returns a bitnet_status code; nothing throws across the ABI.  Work is enqueued on the
// caller's stream; nothing here synchronizes or allocates.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "bitnet_w2a8.h"
#include "kernels.hpp"

// Fewest tokens the fused quant + GEMV entry point sends to the register-quantizing
// kernel (K % 64 == 0); fewer go to the staged kernel.
#ifndef BITNET_FUSED_DIRECT_MIN_M
#define BITNET_FUSED_DIRECT_MIN_M 12
#endif

namespace {

thread_local char g_last_hip_error[256] = "";

int record_hip(hipError_t e) {
    if (e == hipSuccess) return BITNET_OK;
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s (%d)", hipGetErrorString(e),
                  (int)e);
    return BITNET_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record_hip(e);
    if (dev < 0 || dev >= kMaxDevices) return BITNET_ERR_DEVICE;
    int state = g_arch[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return record_hip(e);
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch[dev].store(state, std::memory_order_release);
    }
    return state == 1 ? BITNET_OK : BITNET_ERR_DEVICE;
}

// Shared shape checks: M, N >= 0, 4 <= K <= BITNET_MAX_K, K % 4 == 0, sizes that fit the
// kernels' 32-bit indices and grids.
int check_shape(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 1) return BITNET_ERR_INVALID_ARG;
    if (K > BITNET_MAX_K) return BITNET_ERR_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX) return BITNET_ERR_INVALID_ARG;
    if (K % 4 != 0) return BITNET_ERR_UNALIGNED;
    return BITNET_OK;
}

bool valid_dtype(int dt) {
    return dt == BITNET_OUT_F32 || dt == BITNET_OUT_BF16 || dt == BITNET_OUT_I32;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// int8 product for M <= 16: the kernel that stages the activations in LDS for one to
// three tokens (and for four to seven with large N), the one that reads them straight
// into the matrix-core operands above (K % 64 == 0).  Measured crossover; both give
// identical outputs.
hipError_t launch_small_m(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                          const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                          int out_dtype, hipStream_t stream) {
    const bool direct = K % 64 == 0 && (M >= 8 || (M >= 4 && N <= 4096));
    if (direct)
        return bitnet::launch_gemv_direct(xq, a_scale, nullptr, packed, w_scale, M, N, K, out,
                                          out_dtype, nullptr, nullptr, stream);
    return bitnet::launch_skinny(xq, a_scale, nullptr, packed, w_scale, M, N, K, out, out_dtype,
                                 nullptr, nullptr, stream);
}

// The product of bitnet_w2a8_gemm once its arguments are validated.  Auto: the
// weight-streaming kernels while the product is small enough that one round of their
// blocks beats the tiled kernel (whose single-round grids cost about the same for any M
// up to 64): always up to 4 tokens, up to 16 while the weights are at most 16 MB, the
// direct kernel up to 32 tokens while N * K <= 2^25, and the staged kernel's token tiles
// up to 32 while M * N is small; else the tiled kernel, which may split K through the
// workspace.
int gemm_launch(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                const float* w_scale, int64_t M, int64_t N, int64_t K, void* out, int out_dtype,
                int algo, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (algo == BITNET_ALGO_SKINNY)
        return record_hip(bitnet::launch_skinny(xq, a_scale, nullptr, packed, w_scale, M, N, K,
                                                out, out_dtype, nullptr, nullptr, stream));
    if (algo == BITNET_ALGO_AUTO) {
        if (M <= 4 || (M <= 16 && N * K <= ((int64_t)1 << 26)))
            return record_hip(launch_small_m(xq, a_scale, packed, w_scale, M, N, K, out,
                                             out_dtype, stream));
        // 17 to 32 tokens: the direct kernel's two token tiles while the activations it
        // re-reads per 16-row block (M * K bytes each) stay cheap next to the weights
        if (M <= 32 && K % 64 == 0 && N * K <= ((int64_t)1 << 25))
            return record_hip(bitnet::launch_gemv_direct(xq, a_scale, nullptr, packed, w_scale,
                                                         M, N, K, out, out_dtype, nullptr,
                                                         nullptr, stream));
        if (M <= 32 && M * N <= 131072)
            return record_hip(bitnet::launch_skinny(xq, a_scale, nullptr, packed, w_scale, M, N,
                                                    K, out, out_dtype, nullptr, nullptr, stream));
    }
    return record_hip(bitnet::launch_tiled(xq, a_scale, packed, w_scale, M, N, K, out, out_dtype,
                                           workspace, ws_bytes, stream));
}

// ---- device scratch of the allocation-free product (bitnet_w2a8_gemm_noalloc) ----
// The int32 partial sums of a split-K product live in this file-scope array: one copy on
// every GPU the library runs on, allocated with the code object and held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: its address on a device is taken once per device with hipGetSymbolAddress
// (that device current) and only that address reaches kernels.  Every call on a GPU
// shares its copy, so calls that overlap on one GPU (different streams) race; the
// partials need no clearing, as every call writes each one before reading it.
constexpr size_t kScratchBytes = BITNET_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) int scratch[kScratchBytes / sizeof(int)];

struct ScratchSlot {
    std::mutex lock;
    std::atomic<void*> ptr{nullptr};
};
ScratchSlot g_scratch_slot[kMaxDevices];

// This device's scratch address (dev is the current device), looked up on the first
// call on the device; a failed lookup is retried by the next call.
hipError_t scratch_address(int dev, void** out) {
    ScratchSlot& slot = g_scratch_slot[dev];
    void* p = slot.ptr.load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> guard(slot.lock);
        p = slot.ptr.load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            slot.ptr.store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

int bitnet_abi_version(void) { return BITNET_ABI_VERSION; }

const char* bitnet_status_str(int status) {
    switch (status) {
        case BITNET_OK: return "ok";
        case BITNET_ERR_INVALID_ARG: return "invalid argument";
        case BITNET_ERR_UNALIGNED: return "unaligned size or pointer";
        case BITNET_ERR_WORKSPACE: return "workspace too small";
        case BITNET_ERR_HIP: return "HIP runtime error";
        case BITNET_ERR_DEVICE: return "unsupported device (gfx950 required)";
        default: return "unknown status";
    }
}

const char* bitnet_last_hip_error(void) { return g_last_hip_error; }

int bitnet_pack_weights(const float* w, int64_t N, int64_t K, uint8_t* packed, float* w_scale,
                        void* stream) {
    int st = check_shape(0, N, K);
    if (st) return st;
    if (N == 0) return BITNET_OK;
    if (!w || !packed || !w_scale) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(w_scale)) return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_pack_weights(w, N, K, packed, w_scale, as_stream(stream)));
}

int bitnet_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* codes,
                          void* stream) {
    int st = check_shape(0, N, K);
    if (st) return st;
    if (N == 0) return BITNET_OK;
    if (!packed || !codes) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(codes)) return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_unpack_weights(packed, N, K, codes, as_stream(stream)));
}

int bitnet_quant_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* a_scale,
                     void* stream) {
    int st = check_shape(M, 0, K);
    if (st) return st;
    if (M == 0) return BITNET_OK;
    if (!x || !xq || !a_scale) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(a_scale)) return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_quant_act(x, M, K, xq, a_scale, as_stream(stream)));
}

int bitnet_w2a8_gemv(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                     const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                     int out_dtype, void* stream) {
    if (!valid_dtype(out_dtype)) return BITNET_ERR_INVALID_ARG;
    int st = check_shape(M, N, K);
    if (st) return st;
    if (M > BITNET_GEMV_MAX_M) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!xq || !a_scale || !packed || !w_scale || !out) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(a_scale) || !aligned16(packed) || !aligned16(w_scale) ||
        !aligned16(out))
        return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(launch_small_m(xq, a_scale, packed, w_scale, M, N, K, out, out_dtype,
                                     as_stream(stream)));
}

size_t bitnet_w2a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (check_shape(M, N, K) != BITNET_OK) return 0;
    return bitnet::tiled_workspace_size(M, N, K);
}

int bitnet_w2a8_gemm(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                     const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                     int out_dtype, int algo, void* workspace, size_t ws_bytes, void* stream) {
    if (!valid_dtype(out_dtype)) return BITNET_ERR_INVALID_ARG;
    if (algo != BITNET_ALGO_AUTO && algo != BITNET_ALGO_SKINNY && algo != BITNET_ALGO_TILED)
        return BITNET_ERR_INVALID_ARG;
    int st = check_shape(M, N, K);
    if (st) return st;
    if (algo == BITNET_ALGO_SKINNY && M > BITNET_SKINNY_MAX_M) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!xq || !a_scale || !packed || !w_scale || !out) return BITNET_ERR_INVALID_ARG;
    if (ws_bytes > 0 && !workspace) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(a_scale) || !aligned16(packed) || !aligned16(w_scale) ||
        !aligned16(out) || !aligned16(workspace))
        return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return gemm_launch(xq, a_scale, packed, w_scale, M, N, K, out, out_dtype, algo, workspace,
                       ws_bytes, as_stream(stream));
}

int bitnet_w2a8_gemm_noalloc(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                             const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                             int out_dtype, int algo, void* stream) {
    if (!valid_dtype(out_dtype)) return BITNET_ERR_INVALID_ARG;
    if (algo != BITNET_ALGO_AUTO && algo != BITNET_ALGO_SKINNY && algo != BITNET_ALGO_TILED)
        return BITNET_ERR_INVALID_ARG;
    int st = check_shape(M, N, K);
    if (st) return st;
    if (algo == BITNET_ALGO_SKINNY && M > BITNET_SKINNY_MAX_M) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!xq || !a_scale || !packed || !w_scale || !out) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(a_scale) || !aligned16(packed) || !aligned16(w_scale) ||
        !aligned16(out))
        return BITNET_ERR_UNALIGNED;
    // the planned partials must fit the fixed scratch (never the case below 32 MB: the
    // planner itself keeps partials under 64 MB)
    if (bitnet::tiled_workspace_size(M, N, K) > kScratchBytes) return BITNET_ERR_WORKSPACE;
    if ((st = check_device())) return st;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record_hip(e);
    void* ws = nullptr;
    if ((e = scratch_address(dev, &ws)) != hipSuccess) return record_hip(e);
    return gemm_launch(xq, a_scale, packed, w_scale, M, N, K, out, out_dtype, algo, ws,
                       kScratchBytes, as_stream(stream));
}

int bitnet_pack_b3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* b3, void* stream) {
    int st = check_shape(0, N, K);
    if (st) return st;
    if (N == 0) return BITNET_OK;
    if (!packed || !b3) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(b3)) return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_pack_b3(packed, N, K, b3, as_stream(stream)));
}

int bitnet_quant_gemv_b3(const uint16_t* x, const uint8_t* b3, const float* w_scale, int64_t M,
                         int64_t N, int64_t K, void* out, int out_dtype, void* stream) {
    if (!valid_dtype(out_dtype)) return BITNET_ERR_INVALID_ARG;
    int st = check_shape(M, N, K);
    if (st) return st;
    if (K % 8 != 0) return BITNET_ERR_UNALIGNED;
    if (M > 1 || K > BITNET_B3_MAX_K) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!x || !b3 || !w_scale || !out) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(b3) || !aligned16(w_scale) || !aligned16(out))
        return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_quant_gemv_b3(x, b3, w_scale, N, K, out, out_dtype,
                                                   as_stream(stream)));
}

int bitnet_w2a8_gemm_grouped(const int8_t* xq, const float* a_scale, int64_t M, int64_t K,
                             int64_t groups, const uint8_t* const* packed,
                             const float* const* w_scale, const int64_t* N, void* const* out,
                             int out_dtype, void* stream) {
    if (!valid_dtype(out_dtype)) return BITNET_ERR_INVALID_ARG;
    if (groups < 1 || groups > BITNET_MAX_GROUPS) return BITNET_ERR_INVALID_ARG;
    if (!packed || !w_scale || !N || !out) return BITNET_ERR_INVALID_ARG;
    int64_t total_n = 0;
    for (int64_t g = 0; g < groups; ++g) {
        int st = check_shape(M, N[g], K);
        if (st) return st;
        total_n += N[g];
    }
    if (total_n > INT32_MAX) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || total_n == 0) return BITNET_OK;
    if (!xq || !a_scale) return BITNET_ERR_INVALID_ARG;
    for (int64_t g = 0; g < groups; ++g) {
        if (N[g] == 0) continue;
        if (!packed[g] || !w_scale[g] || !out[g]) return BITNET_ERR_INVALID_ARG;
        if (!aligned16(packed[g]) || !aligned16(w_scale[g]) || !aligned16(out[g]))
            return BITNET_ERR_UNALIGNED;
    }
    if (!aligned16(xq) || !aligned16(a_scale)) return BITNET_ERR_UNALIGNED;
    int st = check_device();
    if (st) return st;
    return record_hip(bitnet::launch_tiled_grouped(xq, a_scale, (int)groups, packed, w_scale, N,
                                                   out, M, K, out_dtype, as_stream(stream)));
}

int bitnet_w2a8_gemm_plan(int64_t M, int64_t K, int64_t groups, const int64_t* N, int64_t cus,
                          int32_t* plan) {
    if (groups < 1 || groups > BITNET_MAX_GROUPS || !N || !plan || M < 1)
        return BITNET_ERR_INVALID_ARG;
    int64_t total_n = 0;
    for (int64_t g = 0; g < groups; ++g) {
        int st = check_shape(M, N[g], K);
        if (st) return st;
        total_n += N[g];
    }
    if (total_n == 0 || total_n > INT32_MAX) return BITNET_ERR_INVALID_ARG;
    int p[5];
    bitnet::tiled_plan(M, K, (int)groups, N, cus, p);
    for (int i = 0; i < 5; ++i) plan[i] = p[i];
    return BITNET_OK;
}

int bitnet_quant_gemv(const uint16_t* x, const uint8_t* packed, const float* w_scale,
                      int64_t M, int64_t N, int64_t K, void* out, int out_dtype,
                      int8_t* xq_out, float* a_scale_out, void* stream) {
    if (!valid_dtype(out_dtype)) return BITNET_ERR_INVALID_ARG;
    int st = check_shape(M, N, K);
    if (st) return st;
    if (M > BITNET_GEMV_MAX_M) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!x || !packed || !w_scale || !out) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(w_scale) || !aligned16(out) ||
        !aligned16(xq_out) || !aligned16(a_scale_out))
        return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    // 12 to 16 tokens: the kernel that quantizes in registers (its whole-row max scan is
    // cheaper there than the staged kernel's LDS copy); fewer: the staged kernel
    if (M >= BITNET_FUSED_DIRECT_MIN_M && K % 64 == 0)
        return record_hip(bitnet::launch_gemv_direct(nullptr, nullptr, x, packed, w_scale, M, N,
                                                     K, out, out_dtype, xq_out, a_scale_out,
                                                     as_stream(stream)));
    return record_hip(bitnet::launch_skinny(nullptr, nullptr, x, packed, w_scale, M, N, K, out,
                                            out_dtype, xq_out, a_scale_out, as_stream(stream)));
}

int bitnet_quant_gemv_grouped(const uint16_t* x, int64_t M, int64_t K, int64_t groups,
                              const uint8_t* const* packed, const float* const* w_scale,
                              const int64_t* N, void* const* out, int out_dtype,
                              int8_t* xq_out, float* a_scale_out, void* stream) {
    if (!valid_dtype(out_dtype)) return BITNET_ERR_INVALID_ARG;
    if (groups < 1 || groups > BITNET_MAX_GROUPS) return BITNET_ERR_INVALID_ARG;
    if (!packed || !w_scale || !N || !out) return BITNET_ERR_INVALID_ARG;
    int64_t total_n = 0;
    for (int64_t g = 0; g < groups; ++g) {
        int st = check_shape(M, N[g], K);
        if (st) return st;
        total_n += N[g];
    }
    if (M > BITNET_GEMV_MAX_M) return BITNET_ERR_INVALID_ARG;
    if (total_n > INT32_MAX) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || total_n == 0) return BITNET_OK;
    if (!x) return BITNET_ERR_INVALID_ARG;
    for (int64_t g = 0; g < groups; ++g) {
        if (N[g] == 0) continue;
        if (!packed[g] || !w_scale[g] || !out[g]) return BITNET_ERR_INVALID_ARG;
        if (!aligned16(packed[g]) || !aligned16(w_scale[g]) || !aligned16(out[g]))
            return BITNET_ERR_UNALIGNED;
    }
    if (!aligned16(x) || !aligned16(xq_out) || !aligned16(a_scale_out)) return BITNET_ERR_UNALIGNED;
    int st = check_device();
    if (st) return st;
    return record_hip(bitnet::launch_skinny_grouped(nullptr, nullptr, x, (int)groups, packed,
                                                    w_scale, N, out, M, K, out_dtype, xq_out,
                                                    a_scale_out, as_stream(stream)));
}

int bitnet_quant_act_per_tensor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                                float* a_scale, void* stream) {
    int st = check_shape(M, 0, K);
    if (st) return st;
    if (M == 0) return BITNET_OK;
    if (!x || !xq || !a_scale) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(a_scale)) return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_quant_act_per_tensor(x, M, K, xq, a_scale, as_stream(stream)));
}

int bitnet_repack_codes(const uint8_t* in, int64_t N, int64_t K, int from_table, int to_table,
                        uint8_t* out, int32_t* invalid_count, void* stream) {
    const auto valid_table = [](int t) { return t == BITNET_CODES_OFFSET || t == BITNET_CODES_SIGN; };
    if (!valid_table(from_table) || !valid_table(to_table)) return BITNET_ERR_INVALID_ARG;
    int st = check_shape(0, N, K);
    if (st) return st;
    if (N == 0) return BITNET_OK;
    if (!in || !out) return BITNET_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(invalid_count) & 3u) != 0) return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_repack_codes(in, N, K, from_table, to_table, out,
                                                  invalid_count, as_stream(stream)));
}

int bitnet_a16_gemv(const uint16_t* x, const uint8_t* packed, const float* w_scale, int64_t M,
                    int64_t N, int64_t K, void* out, int out_dtype, void* stream) {
    if (out_dtype != BITNET_OUT_F32 && out_dtype != BITNET_OUT_BF16) return BITNET_ERR_INVALID_ARG;
    int st = check_shape(M, N, K);
    if (st) return st;
    if (K % 64 != 0) return BITNET_ERR_UNALIGNED;
    if (M > BITNET_GEMV_MAX_M) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!x || !packed || !w_scale || !out) return BITNET_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(w_scale) || !aligned16(out))
        return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_a16(x, packed, w_scale, M, N, K, out, out_dtype,
                                         as_stream(stream)));
}

int bitnet_quant_gemv_swiglu(const uint16_t* x, const uint8_t* packed_gate,
                             const float* w_scale_gate, const uint8_t* packed_up,
                             const float* w_scale_up, int64_t M, int64_t N, int64_t K, void* h,
                             int out_dtype, int8_t* xq_out, float* a_scale_out, void* stream) {
    if (out_dtype != BITNET_OUT_F32 && out_dtype != BITNET_OUT_BF16) return BITNET_ERR_INVALID_ARG;
    int st = check_shape(M, N, K);
    if (st) return st;
    if (M > BITNET_GEMV_MAX_M) return BITNET_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!x || !packed_gate || !w_scale_gate || !packed_up || !w_scale_up || !h)
        return BITNET_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(packed_gate) || !aligned16(w_scale_gate) ||
        !aligned16(packed_up) || !aligned16(w_scale_up) || !aligned16(h) || !aligned16(xq_out) ||
        !aligned16(a_scale_out))
        return BITNET_ERR_UNALIGNED;
    if ((st = check_device())) return st;
    return record_hip(bitnet::launch_skinny_swiglu(x, packed_gate, w_scale_gate, packed_up,
                                                   w_scale_up, M, N, K, h, out_dtype, xq_out,
                                                   a_scale_out, as_stream(stream)));
}

}  // extern "C"
