/*
 * bitnet_w2a8.h -- C ABI of the MI355X (gfx950) BitNet b1.58 W2A8 BitLinear matmul.
 *
 * The operation (one BitLinear layer, no bias):
 *   out[m, n] = acc[m, n] * w_scale[n] / a_scale[m]
 *   acc[m, n] = sum_k xq[m, k] * w[n, k]          (exact, int32)
 * with w in {-1, 0, +1} stored 2 bits per weight, and xq the int8 per-token absmax
 * quantization of bf16 activations x.
 *
 * Pages this follows (cited by title and section):
 *   "BitNet 深度实战：微软 32K Star 的 1-bit LLM 推理框架" (chenxutan.com):
 *       §2.4 absmean weight quantization; §3.2 BitLinear (bias=False);
 *       §4.3 four 2-bit weights per byte, first weight in the low bits;
 *       §4.4 int8 activations x ternary weights accumulated in int32.
 *   "BitNet-Triton：消费级GPU上的1.58-bit大模型推理加速方案" (zingnex.cn), 技术架构:
 *       §1 (N, K/4) uint8 packed weights unpacked inside the matmul kernel;
 *       §2 int8 matrix-core products; §3 activation quantization fused into one launch.
 *   "BitNet 1-bit LLM推理优化：内存布局、量化策略与硬件加速" (blog.hotdry.top):
 *       §3.1 encode offline / decode just before compute; §3.2 the W2A8 path;
 *       §5.3 dimensions that break the alignment unit are rejected.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major and
 *     contiguous, 16-byte aligned, valid until the enqueued work completes.  The
 *     library allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is enqueued
 *     on it and the call returns; nothing synchronizes.
 *   - Arguments are validated on the host before any HIP call.  On a validation error
 *     no work is enqueued and no output is touched.  Kernel faults surface at the
 *     caller's next synchronization as HIP errors.
 *   - M == 0 or N == 0 is a valid empty problem: BITNET_OK, nothing enqueued, and the
 *     tensor pointers are not examined (empty tensors may have NULL data).
 *   - K must be a positive multiple of 4 and at most BITNET_MAX_K.
 *   - Inputs must be finite (NaN / Inf give unspecified results).
 *   - Entry points are reentrant and thread-safe; calls on one stream are ordered.
 *   - Only gfx950 devices are supported (BITNET_ERR_DEVICE otherwise).
 *
 * Packed weight layout (the interface format, produced by bitnet_pack_weights):
 *   packed[n * (K/4) + j] holds weights k = 4j .. 4j+3 of output row n; weight
 *   k = 4j + i sits in bits 2i .. 2i+1 as the code (w + 1): -1 -> 0b00, 0 -> 0b01,
 *   +1 -> 0b10.  0b11 is never produced.  A buffer that holds it anyway (e.g. weights
 *   packed with the other code table of "BitNet 深度实战" §4.3 and not converted by
 *   bitnet_repack_codes) is decoded as w = code - 1 = +2 by every int8 product entry
 *   point, whatever kernel a call takes, and as 0 by bitnet_a16_gemv.
 */
#ifndef BITNET_W2A8_H
#define BITNET_W2A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITNET_ABI_VERSION 2
/* Largest supported K: keeps every int32 partial sum exact with margin. */
#define BITNET_MAX_K (1 << 20)

typedef enum {
    BITNET_OK = 0,
    BITNET_ERR_INVALID_ARG = 1, /* null pointer, negative size, K == 0, bad enum, M range */
    BITNET_ERR_UNALIGNED = 2,   /* K % 4 != 0, or a pointer not 16-byte aligned          */
    BITNET_ERR_WORKSPACE = 3,   /* device scratch too small for the call                  */
    BITNET_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed             */
    BITNET_ERR_DEVICE = 5       /* the current device is not gfx950                       */
} bitnet_status;

typedef enum {
    BITNET_OUT_F32 = 0,  /* float   (M, N) */
    BITNET_OUT_BF16 = 1, /* bf16    (M, N), stored as uint16 bit patterns, RNE of fp32 */
    BITNET_OUT_I32 = 2   /* int32   (M, N), the raw exact accumulator acc[m, n]        */
} bitnet_out_dtype;

typedef enum {
    BITNET_ALGO_AUTO = 0,   /* weight-streaming kernels for small products, else TILED */
    BITNET_ALGO_SKINNY = 1, /* weight-streaming kernel, M <= BITNET_SKINNY_MAX_M      */
    BITNET_ALGO_TILED = 2   /* tiled int8 matrix-core kernel, any M                    */
} bitnet_algo;

#define BITNET_SKINNY_MAX_M 64
#define BITNET_GEMV_MAX_M 16
/* Most weight matrices one grouped launch takes (bitnet_quant_gemv_grouped). */
#define BITNET_MAX_GROUPS 4

/* ABI version of the loaded library (BITNET_ABI_VERSION at build time). */
int bitnet_abi_version(void);

/* Static, never-NULL description of a status code (unknown codes included). */
const char* bitnet_status_str(int status);

/* Text of the last HIP error seen by this thread inside the library ("" if none). */
const char* bitnet_last_hip_error(void);

/*
 * bitnet_pack_weights -- offline weight preparation ("BitNet 深度实战" §2.4, §4.3).
 *   w        : float (N, K) latent weights.
 *   packed   : uint8 (N, K/4) output, layout above.
 *   w_scale  : float (N) output, w_scale[n] = max(mean_k |w[n,k]|, 1e-5), the mean being
 *              an fp64 sum over k in ascending order divided by K, rounded once to fp32.
 *   Codes: clamp(round_half_even(w[n,k] / w_scale[n]), -1, 1), fp32 IEEE division.
 */
int bitnet_pack_weights(const float* w, int64_t N, int64_t K, uint8_t* packed, float* w_scale,
                        void* stream);

/*
 * bitnet_unpack_weights -- inverse of the packing, for inspection and tests.
 *   codes : int8 (N, K) output, w = code - 1: {-1, 0, +1} (+2 for a field holding 0b11).
 */
int bitnet_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* codes,
                          void* stream);

/*
 * bitnet_quant_act -- per-token absmax int8 activation quantization in one launch
 * ("BitNet-Triton" 技术架构 §3; "BitNet 1-bit LLM推理优化" §3.2).
 *   x       : bf16 (M, K) as uint16 bit patterns.
 *   xq      : int8 (M, K) output, clamp(round_half_even(x * a_scale[m]), -127, 127).
 *   a_scale : float (M) output, a_scale[m] = 127 / max(max_k |x[m,k]|, 1e-5)
 *             (one fp32 IEEE division; the product x * a_scale is one fp32 multiply).
 */
int bitnet_quant_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* a_scale,
                     void* stream);

/*
 * bitnet_quant_act_per_tensor -- the same quantization with one scale for the whole
 * tensor ("BitNet 1-bit LLM推理优化" §2.2: the I2_S kernel keeps the per-tensor int8
 * activation quantization used in training; §3.2: per-tensor or per-channel scales):
 *   a = 127 / max(max_{m,k} |x[m,k]|, 1e-5), written to every a_scale[m] (so the product
 *   entry points take it unchanged); xq[m,k] = clamp(round_half_even(x * a), -127, 127).
 * At M = 1 it equals bitnet_quant_act.  Three launches (row maxima, which use a_scale as
 * scratch; the tensor scale; the codes).
 */
int bitnet_quant_act_per_tensor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                                float* a_scale, void* stream);

/* 2-bit code tables for bitnet_repack_codes. */
typedef enum {
    BITNET_CODES_OFFSET = 0, /* this library: code = w + 1 (00 -1, 01 0, 10 +1, 11 unused) */
    BITNET_CODES_SIGN = 1    /* "BitNet 深度实战" §4.3: 00 0, 01 -1, 11 +1, 10 unused         */
} bitnet_code_table;

/*
 * bitnet_repack_codes -- rewrite a packed (N, K/4) array from one code table to the
 * other (same bit positions: weight 4j+i in bits 2i..2i+1 of byte j).  Converts weights
 * packed with the page's table for use here, and back.  in and out may be the same
 * buffer.  A field holding its table's unused code becomes weight 0; when
 * invalid_count (a device int32, caller-zeroed, 4-byte aligned, else
 * BITNET_ERR_UNALIGNED) is given, the number of such fields is added to it.
 */
int bitnet_repack_codes(const uint8_t* in, int64_t N, int64_t K, int from_table, int to_table,
                        uint8_t* out, int32_t* invalid_count, void* stream);

/*
 * bitnet_w2a8_gemv -- decode-sized product, 1 <= M <= BITNET_GEMV_MAX_M
 * ("BitNet 深度实战" §4.4; "BitNet-Triton" 技术架构 §1).
 *   xq, a_scale       : as produced by bitnet_quant_act.
 *   packed, w_scale   : as produced by bitnet_pack_weights.
 *   out               : (M, N) of out_dtype (bitnet_out_dtype).
 * out = acc * w_scale[n] * (1 / a_scale[m]) in fp32 (within 3 fp32 roundings of the exact
 * value); bf16 is the RNE of that fp32 value; int32 is acc itself.
 * M > BITNET_GEMV_MAX_M returns BITNET_ERR_INVALID_ARG.
 */
int bitnet_w2a8_gemv(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                     const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                     int out_dtype, void* stream);

/*
 * bitnet_w2a8_gemm -- the same product for any M >= 0: prefill, where the int8 products
 * run on the matrix cores ("BitNet-Triton" 技术架构 §2: int8 tensor-core GEMM for the
 * prefill phase; "BitNet 深度实战" §4.4: int8 x ternary accumulated in int32).
 *   xq, a_scale, packed, w_scale, out, out_dtype : as in bitnet_w2a8_gemv.
 *   algo : which kernel (bitnet_algo); an addition to the plain product signature that
 *          only selects among kernels with identical results.  BITNET_ALGO_SKINNY with
 *          M > BITNET_SKINNY_MAX_M returns BITNET_ERR_INVALID_ARG.
 * Workspace (optional, caller-owned device memory, 16-byte aligned): when the tiled
 * kernel runs and ws_bytes >= bitnet_w2a8_gemm_workspace_size(M, N, K) > 0, K is split
 * into slices taken by different blocks -- for grids with too few output tiles to fill
 * the chip, e.g. a few dozen tokens times a large K -- each writing its int32 partial
 * sums into the workspace, and a second launch adds the slices (exact in int32) and
 * rescales.  With a smaller workspace (or NULL and 0) the call runs unsplit.  Outputs are
 * bit-identical either way.  The workspace is scratch: its contents on return are
 * unspecified, and calls that share one must be ordered (e.g. on one stream).
 * ws_bytes > 0 with workspace NULL returns BITNET_ERR_INVALID_ARG.
 * bitnet_w2a8_gemm_workspace_size returns 0 for invalid sizes and when the best plan on
 * the current device does not split (then no workspace is ever used).
 */
size_t bitnet_w2a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
int bitnet_w2a8_gemm(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                     const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                     int out_dtype, int algo, void* workspace, size_t ws_bytes, void* stream);

/*
 * bitnet_w2a8_gemm_noalloc -- bitnet_w2a8_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments minus the workspace, the same kernels and bit-identical
 * outputs, with the split-K partial sums in a fixed device scratch array that the
 * library holds on every GPU it runs on until the process ends
 * (BITNET_NOALLOC_SCRATCH_BYTES, 32 MB).  The call allocates nothing.
 *   Returns BITNET_ERR_WORKSPACE, before any HIP call, when the tiled plan for (M, N, K)
 *   needs more partials than the scratch holds (only with K in the tens of thousands
 *   and M, N in the thousands).
 *   All calls on one GPU share its scratch: calls that overlap on a GPU (different
 *   streams, or different host threads without ordering) race and give undefined
 *   outputs; order them, e.g. on one stream.  Nothing in the scratch needs clearing.
 */
#define BITNET_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int bitnet_w2a8_gemm_noalloc(const int8_t* xq, const float* a_scale, const uint8_t* packed,
                             const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                             int out_dtype, int algo, void* stream);

/*
 * bitnet_w2a8_gemm_grouped -- the tiled product (BITNET_ALGO_TILED) for several weight
 * matrices that read the same int8 activations, in one launch: a prefill-sized batch
 * through q, k and v, or through gate and up, of the LLaMA block in "BitNet 深度实战" §3.2
 * (every nn.Linear a BitLinear layer; q, k, v share their input, and so do gate and up).
 *   xq, a_scale      : int8 (M, K) codes and float (M) scales, shared; M >= 0.
 *   groups           : 1 <= groups <= BITNET_MAX_GROUPS.
 *   packed, w_scale, N, out : HOST arrays of `groups` entries, read during the call only;
 *                      entry g is one product exactly as bitnet_w2a8_gemm's packed
 *                      (N[g], K/4), w_scale (N[g]) and out (M, N[g]) arguments (device
 *                      pointers, caller-owned).  N[g] == 0 is allowed and touches nothing
 *                      of that entry.
 *   out_dtype        : one output type for every group.
 * The tile shape is chosen for the launch's total tile count; each out[g] is
 * bit-identical to bitnet_w2a8_gemm(..., BITNET_ALGO_TILED, ...) on entry g alone (every
 * tile shape yields the exact int32 sum and the same rescale).  Output buffers must not
 * overlap one another or any input.
 */
int bitnet_w2a8_gemm_grouped(const int8_t* xq, const float* a_scale, int64_t M, int64_t K,
                             int64_t groups, const uint8_t* const* packed,
                             const float* const* w_scale, const int64_t* N, void* const* out,
                             int out_dtype, void* stream);

/*
 * bitnet_w2a8_gemm_plan -- the tile plan a tiled launch takes for M tokens, K columns and
 * `groups` weight matrices of N[g] rows (HOST array), on a device with `cus` compute
 * units (cus <= 0: the current device's; with no device the count defaults to 256):
 * groups == 1 describes bitnet_w2a8_gemm (BITNET_ALGO_TILED, or the tiled route of
 * BITNET_ALGO_AUTO) given its workspace, groups > 1 bitnet_w2a8_gemm_grouped, which never
 * splits K.  Host-only: launches nothing.
 *   plan : HOST int32[5] output = block rows, block columns, k-groups per block (waves
 *          per block / 4), k per LDS stage, slices of K across blocks (1: unsplit).
 * The plan is the compiled tile configuration and K split with the least estimated time
 * (rounds of one block per CU times a per-configuration cost fitted on this chip, plus
 * the reduce launch of a split); the environment variable BITNET_TILED_CONFIG="bm,bn,g"
 * or "bm,bn,g,slices" (read once per process) overrides the choice.
 * Returns BITNET_ERR_INVALID_ARG for M < 1, groups outside 1..BITNET_MAX_GROUPS, N[g] < 0,
 * no rows at all, or NULL arrays; BITNET_ERR_UNALIGNED for K % 4 != 0.
 */
int bitnet_w2a8_gemm_plan(int64_t M, int64_t K, int64_t groups, const int64_t* N, int64_t cus,
                          int32_t* plan);

/*
 * bitnet_quant_gemv -- activation quantization fused into the decode product, one
 * launch ("BitNet-Triton" 技术架构 §3: the quantization folded into the matmul launch).
 *   x               : bf16 (M, K) as uint16, 1 <= M <= BITNET_GEMV_MAX_M.
 *   packed, w_scale : as produced by bitnet_pack_weights.
 *   out             : (M, N) of out_dtype, same arithmetic as bitnet_w2a8_gemv.
 *   xq_out, a_scale_out : optional (NULL = not written) copies of the quantized
 *                     activations and scales, bit-identical to bitnet_quant_act.
 */
int bitnet_quant_gemv(const uint16_t* x, const uint8_t* packed, const float* w_scale,
                      int64_t M, int64_t N, int64_t K, void* out, int out_dtype,
                      int8_t* xq_out, float* a_scale_out, void* stream);

/*
 * bitnet_quant_gemv_grouped -- bitnet_quant_gemv for several weight matrices that read
 * the same activations, in one launch.  In the model of "BitNet 深度实战" §3.2 (a LLaMA
 * block with every nn.Linear replaced by BitLinear) q, k and v project the same hidden
 * states, and so do the MLP's gate and up projections.
 *   x                : bf16 (M, K) as uint16, 1 <= M <= BITNET_GEMV_MAX_M, shared.
 *   groups           : 1 <= groups <= BITNET_MAX_GROUPS.
 *   packed, w_scale, N, out : HOST arrays of `groups` entries, read during the call only;
 *                      entry g describes one product exactly as bitnet_quant_gemv's
 *                      packed (N[g], K/4), w_scale (N[g]) and out (M, N[g]) arguments
 *                      (device pointers, caller-owned).  N[g] == 0 is allowed and
 *                      touches nothing of that entry.
 *   out_dtype        : one output type for every group.
 *   xq_out, a_scale_out : optional copies of the quantized activations, as in
 *                      bitnet_quant_gemv (written once).
 * Each out[g] is bit-identical to bitnet_quant_gemv on entry g alone.  Output buffers
 * must not overlap one another or any input.
 */
int bitnet_quant_gemv_grouped(const uint16_t* x, int64_t M, int64_t K, int64_t groups,
                              const uint8_t* const* packed, const float* const* w_scale,
                              const int64_t* N, void* const* out, int out_dtype,
                              int8_t* xq_out, float* a_scale_out, void* stream);

/*
 * bitnet_quant_gemv_swiglu -- the decode MLP's first half in one launch ("BitNet 深度实战"
 * §3.2: the MLP computes down(silu(gate(x)) * up(x)) with gate, up and down BitLinear
 * layers).  Both products read the same quantized x; a block multiplies the same rows of
 * the two matrices and writes
 *   h[m,n] = silu(g[m,n]) * u[m,n],  silu(g) = g / (1 + exp(-g)),
 * where g and u are the fp32 outputs bitnet_quant_gemv would write for (packed_gate,
 * w_scale_gate) and (packed_up, w_scale_up); the SiLU and the product are fp32.
 *   x                 : bf16 (M, K) as uint16, 1 <= M <= BITNET_GEMV_MAX_M.
 *   packed_gate/_up   : uint8 (N, K/4) each; w_scale_gate/_up: float (N) each.
 *   h                 : (M, N), BITNET_OUT_F32 or BITNET_OUT_BF16 (RNE of the fp32 value);
 *                       BITNET_OUT_I32 is rejected (BITNET_ERR_INVALID_ARG).
 *   xq_out, a_scale_out : optional copies of the quantized activations, as in
 *                       bitnet_quant_gemv.
 * h is what bitnet_quant_gemv_swiglu's caller feeds (as bf16) to the down projection,
 * e.g. bitnet_quant_gemv with K = N.
 */
int bitnet_quant_gemv_swiglu(const uint16_t* x, const uint8_t* packed_gate,
                             const float* w_scale_gate, const uint8_t* packed_up,
                             const float* w_scale_up, int64_t M, int64_t N, int64_t K, void* h,
                             int out_dtype, int8_t* xq_out, float* a_scale_out, void* stream);

/*
 * bitnet_a16_gemv -- the ternary weights times bf16 activations with no activation
 * quantization (W1.58A16): "将 BitNet 三元查找表集成到自定义 Triton 内核中" serves ternary
 * weights with 16-bit activations and an fp32 accumulator; "BitNet 深度实战" §2.2: the
 * product needs only additions and subtractions.
 *   out[m,n] = w_scale[n] * sum_k x[m,k] * w[n,k]
 *   x               : bf16 (M, K) as uint16, 1 <= M <= BITNET_GEMV_MAX_M.
 *   packed, w_scale : as produced by bitnet_pack_weights; K % 64 == 0 (else
 *                     BITNET_ERR_UNALIGNED).
 *   out             : (M, N), BITNET_OUT_F32 or BITNET_OUT_BF16 (RNE of the fp32 value);
 *                     BITNET_OUT_I32 is rejected.
 * Each product x * w is exact; the sum is accumulated in fp32 (any order), so
 * |out - exact| <= (K + 2) * 2^-24 * w_scale[n] * sum_k |x[m,k] * w[n,k]|.
 */
int bitnet_a16_gemv(const uint16_t* x, const uint8_t* packed, const float* w_scale, int64_t M,
                    int64_t N, int64_t K, void* out, int out_dtype, void* stream);

/*
 * Ternary weights at 1.6 bits per weight, five per byte ("将 BitNet 三元查找表集成到自定义
 * Triton 内核中": a uint8 bitmap of four to five ternary values per byte; "BitNet 1-bit
 * LLM推理优化" §2.1 / §3.1: packing below 2 bits per weight, 3 weights in 5 bits).
 * Layout: (N, BITNET_B3_ROW_BYTES(K)) uint8, rows padded with weights 0 to whole chunks
 * of 320 weights (64 bytes).  Byte j of row n holds weights k = 5j .. 5j+4: with codes
 * c = w + 1, v = 81 c[5j] + 27 c[5j+1] + 9 c[5j+2] + 3 c[5j+3] + c[5j+4] (0 .. 242) is
 * stored as ceil(256 v / 243), so v = floor(byte * 243 / 256).  20% fewer weight bytes
 * than the 2-bit format (a 70B-class layer set: 171 MB instead of 214 MB).
 */
#define BITNET_B3_ROW_BYTES(K) (64 * (((K) + 319) / 320))
#define BITNET_B3_MAX_K 30720

/*
 * bitnet_pack_b3 -- convert a packed (N, K/4) array of the 2-bit format above into the
 * five-per-byte format.
 *   packed : uint8 (N, K/4), as produced by bitnet_pack_weights.  A field holding the
 *            unused code 0b11 becomes weight 0.
 *   b3     : uint8 (N, BITNET_B3_ROW_BYTES(K)) output.
 */
int bitnet_pack_b3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* b3, void* stream);

/*
 * bitnet_quant_gemv_b3 -- bitnet_quant_gemv on weights in the five-per-byte format, for
 * one token (M = 1, the decode step): the per-token int8 quantization of x fused into
 * the product, int32 accumulation, the same rescale and outputs as bitnet_quant_gemv
 * (fp32 within 3 roundings of the exact value, bf16 its RNE, int32 the exact acc).
 *   x       : bf16 (1, K) as uint16; K % 8 == 0 (else BITNET_ERR_UNALIGNED) and
 *             K <= BITNET_B3_MAX_K; M other than 0 or 1 returns BITNET_ERR_INVALID_ARG.
 *   b3      : uint8 (N, BITNET_B3_ROW_BYTES(K)), as produced by bitnet_pack_b3.
 *   w_scale : float (N), as produced by bitnet_pack_weights.
 *   out     : (1, N) of out_dtype.
 */
int bitnet_quant_gemv_b3(const uint16_t* x, const uint8_t* b3, const float* w_scale, int64_t M,
                         int64_t N, int64_t K, void* out, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_W2A8_H */
