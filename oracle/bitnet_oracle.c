/*
 * bitnet_oracle.c -- plain, slow, obviously correct CPU oracle for the BitNet b1.58
 * W2A8 BitLinear matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file: only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Every function follows one passage of the source pages (cited by page title and
 * section).  Scalar loops only; floating point in the precision each step states;
 * built with -O2 -ffp-contract=off and no fast-math, so every float operation below is
 * a single IEEE-754 operation in round-to-nearest-even.
 *
 * Pages:
 *   [Triton]  "BitNet-Triton：消费级GPU上的1.58-bit大模型推理加速方案" (zingnex.cn)
 *   [Deep]    "BitNet 深度实战：微软 32K Star 的 1-bit LLM 推理框架" (chenxutan.com)
 *   [Layout]  "BitNet 1-bit LLM推理优化：内存布局、量化策略与硬件加速" (blog.hotdry.top)
 *
 * Return codes: 0 = ok, -1 = bad argument, 1 = a clamp that the definition says can
 * never fire did fire (reported, not hidden).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- bf16 helpers --- */

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a double to the nearest bf16 (8 significant bits), ties to even, in ONE
 * rounding step: scale to an integer grid by an exact power of two, nearbyint (the
 * default FE_TONEAREST mode is round-half-even), scale back (exact).  Overflow gives
 * +-inf.  Finite inputs only. */
static uint16_t f64_to_bf16_rne(double x) {
    if (x == 0.0) return signbit(x) ? 0x8000u : 0x0000u;
    int e = ilogb(x);                 /* |x| in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;           /* bf16 subnormal grid is fixed at 2^-133 */
    double quantum = ldexp(1.0, e - 7);
    double r = nearbyint(x / quantum) * quantum;
    float f = (float)r;               /* exact: r has <= 8 significant bits (or is inf) */
    if (fabs(r) >= ldexp(1.0, 128)) f = (x > 0) ? INFINITY : -INFINITY;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------- O1: absmean weight ternarization --- */

/*
 * [Deep] §2.4 (量化函数的细节), function quantize_weights: the scale is the mean of
 * |W| along the last (input, K) dimension, i.e. one scale per output row n, clamped
 * below at eps = 1e-5; the codes are round(W / scale) clamped to [-1, 1].
 * [Deep] §3.2 (BitLinear._quantize_weight) repeats the same formula.
 *
 * Readings where the page is silent:
 *   - mean: fp64 sum of |W[n,k]| for k ascending, divided by K in fp64, rounded once
 *     to fp32;
 *   - W / scale: one fp32 IEEE division (the page's tensors are fp32);
 *   - round: half-to-even (torch.round), done by nearbyintf.
 * Works for any K >= 1 (the worked example has K = 6).
 */
int oracle_weight_quant(const float* W, int64_t N, int64_t K, int8_t* q, float* scale) {
    if (!W || !q || !scale || N < 0 || K < 1) return -1;
    for (int64_t n = 0; n < N; ++n) {
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k) sum += fabs((double)W[n * K + k]);
        float s = (float)(sum / (double)K);
        if (s < 1e-5f) s = 1e-5f;
        scale[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            float r = nearbyintf(W[n * K + k] / s);
            if (r > 1.0f) r = 1.0f;
            if (r < -1.0f) r = -1.0f;
            q[n * K + k] = (int8_t)r;
        }
    }
    return 0;
}

/* ------------------------------------------------------ 2-bit packing / unpack --- */

/*
 * [Triton] 技术架构 §1 (2-bit打包存储): weights are stored as an (N, K/4) uint8 array,
 * four ternary weights per byte.
 * [Deep] §4.3 (位打包): the first of the four weights occupies bits 0-1, the second bits
 * 2-3, the third bits 4-5, the fourth bits 6-7.
 * Code values: code = w + 1 (w = -1 -> 0b00, 0 -> 0b01, +1 -> 0b10; 0b11 unused).  The
 * page uses a different code table (11 -> +1, 00 -> 0, 01 -> -1); the library stores
 * w + 1 so that the code is an unsigned digit and w = code - 1 (oracle_repack converts).
 * K must be a multiple of 4.
 */
int oracle_pack(const int8_t* q, int64_t N, int64_t K, uint8_t* packed) {
    if (!q || !packed || N < 0 || K < 4 || K % 4 != 0) return -1;
    int64_t KB = K / 4;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < KB; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                int w = q[n * K + 4 * j + i];
                if (w < -1 || w > 1) return -1;
                unsigned code = (unsigned)(w + 1);
                byte |= code << (2 * i);
            }
            packed[n * KB + j] = (uint8_t)byte;
        }
    }
    return 0;
}

/* Inverse of oracle_pack: weight k of row n is field (k mod 4) of byte k/4, minus 1.
 * Returns 1 if a field holds the unused code 0b11 (it is then decoded as +2 so the
 * caller can see it). */
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q) {
    if (!q || !packed || N < 0 || K < 4 || K % 4 != 0) return -1;
    int64_t KB = K / 4;
    int bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            unsigned code = (packed[n * KB + k / 4] >> (2 * (k % 4))) & 3u;
            if (code == 3u) bad = 1;
            q[n * K + k] = (int8_t)((int)code - 1);
        }
    }
    return bad;
}

/* ------------------------------------- 1.6-bit packing: five weights per byte --- */

/*
 * [LUT] (its three integration steps): ternary weights go into a packed uint8 bitmap,
 * four to five of them per 8-bit byte.  [Layout] §2.1 / §3.1: the TL encoding packs
 * three weights into 5 bits (1.67 bits per weight) to beat the 2 bits of a plain code.
 * Five per byte is possible because 3^5 = 243 <= 256.
 *
 * Readings where the pages are silent:
 *   - byte j of a row holds weights k = 5j .. 5j+4; their codes c = w + 1 in {0, 1, 2}
 *     are the base-3 digits of v = c[5j]*81 + c[5j+1]*27 + c[5j+2]*9 + c[5j+3]*3 +
 *     c[5j+4] (the first weight the most significant digit);
 *   - the stored byte is ceil(256 v / 243), i.e. v/243 rounded up to a multiple of
 *     1/256: then v = floor(byte * 243 / 256), and the digits also come out by repeated
 *     multiplication by 3 (each digit is the integer part, the byte-wide fraction stays);
 *   - a row holds B3_CHUNK-weight chunks (64 bytes): K is padded up to a multiple of 320
 *     with weights 0, so rows start 64-byte aligned.
 */
#define B3_CHUNK 320
static int64_t b3_row_bytes(int64_t K) { return (K + B3_CHUNK - 1) / B3_CHUNK * 64; }

int64_t oracle_b3_row_bytes(int64_t K) { return K < 1 ? -1 : b3_row_bytes(K); }

int oracle_pack_b3(const int8_t* q, int64_t N, int64_t K, uint8_t* out) {
    if (!q || !out || N < 0 || K < 1) return -1;
    const int64_t RB = b3_row_bytes(K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < RB; ++j) {
            int v = 0;
            for (int i = 0; i < 5; ++i) {
                const int64_t k = 5 * j + i;
                const int w = k < K ? q[n * K + k] : 0;
                if (w < -1 || w > 1) return -1;
                v = 3 * v + (w + 1);
            }
            out[n * RB + j] = (uint8_t)((256 * v + 242) / 243); /* ceil(256 v / 243) */
        }
    }
    return 0;
}

/* Inverse of oracle_pack_b3: v = floor(byte * 243 / 256), digits by division.  Returns 1
 * if a padding weight (k >= K) is not 0. */
int oracle_unpack_b3(const uint8_t* b3, int64_t N, int64_t K, int8_t* q) {
    if (!b3 || !q || N < 0 || K < 1) return -1;
    const int64_t RB = b3_row_bytes(K);
    int bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < RB; ++j) {
            const int v = (b3[n * RB + j] * 243) / 256;
            for (int i = 0; i < 5; ++i) {
                int p = 1;
                for (int t = i; t < 4; ++t) p *= 3;
                const int w = (v / p) % 3 - 1; /* digit i, the first the most significant */
                const int64_t k = 5 * j + i;
                if (k < K) q[n * K + k] = (int8_t)w;
                else if (w != 0) bad = 1;
            }
        }
    }
    return bad;
}

/* O3 on the five-per-byte format: acc[m, n] = sum_k xq[m, k] * w[n, k], each w decoded
 * from its byte as above. */
int oracle_accumulate_b3(const int8_t* xq, const uint8_t* b3, int64_t M, int64_t N, int64_t K,
                         int32_t* acc) {
    if (!xq || !b3 || !acc || M < 0 || N < 0 || K < 1) return -1;
    const int64_t RB = b3_row_bytes(K);
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k) {
                const int v = (b3[n * RB + k / 5] * 243) / 256;
                int p = 1;
                for (int t = (int)(k % 5); t < 4; ++t) p *= 3;
                sum += (int64_t)xq[m * K + k] * ((v / p) % 3 - 1);
            }
            if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
            acc[m * N + n] = (int32_t)sum;
        }
    }
    return overflow ? -1 : 0;
}

/* -------------------------------------- O2: per-token absmax int8 activations --- */

/*
 * [Triton] 技术架构 §2 and §3: activations are quantized to int8 (one fused launch per
 * layer).  [Layout] §3.2 (激活量化策略): an int8 activation scale aligned with training.
 * Per-token absmax, scale = 127 / max|x|, round half to even, clamp to [-127, 127].
 *
 * Readings: x is bf16 and widened exactly to fp32; amax is clamped below at 1e-5 (an
 * all-zero row then quantizes to zeros, mirroring the weight eps); the scale is one
 * fp32 IEEE division; x * scale is one fp32 multiply, then round-half-even.
 * a_scale[m] stores 127 / amax (multiply to quantize, divide to dequantize).
 */
int oracle_act_quant(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* a_scale) {
    if (!x || !xq || !a_scale || M < 0 || K < 1) return -1;
    int clamped = 0;
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(bf16_to_f32(x[m * K + k]));
            if (v > amax) amax = v;
        }
        if (amax < 1e-5f) amax = 1e-5f;
        float a = 127.0f / amax;
        a_scale[m] = a;
        for (int64_t k = 0; k < K; ++k) {
            float p = bf16_to_f32(x[m * K + k]) * a;
            float r = nearbyintf(p);
            if (r > 127.0f) { r = 127.0f; clamped = 1; }
            if (r < -127.0f) { r = -127.0f; clamped = 1; }
            xq[m * K + k] = (int8_t)r;
        }
    }
    return clamped;
}

/*
 * Per-tensor variant. [Layout] §2.2 (I2_S): the MAD kernel keeps the per-tensor int8
 * activation quantization of training; [Layout] §3.2: per-tensor or per-channel scales.
 * amax is the max |x| over the whole (M, K) tensor (clamped below at 1e-5), scale =
 * 127 / amax for every row, codes as above.
 */
int oracle_act_quant_per_tensor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                                float* a_scale) {
    if (!x || !xq || !a_scale || M < 0 || K < 1) return -1;
    float amax = 0.0f;
    for (int64_t i = 0; i < M * K; ++i) {
        float v = fabsf(bf16_to_f32(x[i]));
        if (v > amax) amax = v;
    }
    const float amax_t = amax < 1e-5f ? 1e-5f : amax;
    const float a_t = 127.0f / amax_t;
    int clamped = 0;
    for (int64_t m = 0; m < M; ++m) {
        a_scale[m] = a_t;
        for (int64_t k = 0; k < K; ++k) {
            float r = nearbyintf(bf16_to_f32(x[m * K + k]) * a_t);
            if (r > 127.0f) { r = 127.0f; clamped = 1; }
            if (r < -127.0f) { r = -127.0f; clamped = 1; }
            xq[m * K + k] = (int8_t)r;
        }
    }
    return clamped;
}

/* -------------------------------------------------- O3: exact int accumulation --- */

/* Decode weight (n, k) from the packed array: the inverse of the byte layout above. */
static int weight_at(const uint8_t* packed, int64_t KB, int64_t n, int64_t k) {
    unsigned code = (packed[n * KB + k / 4] >> (2 * (k % 4))) & 3u;
    return (int)code - 1;
}

/*
 * [Deep] §4.4 (查找表加速), ternary_matmul_int8: int8 activations [M,K] times ternary
 * weights [N,K] into int32 outputs [M,N]; +1 adds the activation, -1 subtracts it, 0
 * skips it.  Here written as the plain sum acc[m,n] = sum_k xq[m,k] * w[n,k], kept in a
 * 64-bit integer and checked to fit int32 (|acc| <= 127 K).
 * Parallel over rows n only (each output is still one sequential sum).
 */
int oracle_accumulate(const int8_t* xq, const uint8_t* packed, int64_t M, int64_t N,
                      int64_t K, int32_t* acc) {
    if (!xq || !packed || !acc || M < 0 || N < 0 || K < 4 || K % 4 != 0) return -1;
    int64_t KB = K / 4;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)xq[m * K + k] * weight_at(packed, KB, n, k);
            if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
            acc[m * N + n] = (int32_t)sum;
        }
    }
    return overflow ? -1 : 0;
}

/* ------------------------------------------------------------- O4: rescale --- */

/*
 * [Deep] §2.4: the effective weight is w_q * scale; [Deep] §2.3 and §3.2: the layer
 * output is linear(x, w_q * scale) with no bias.  With x ~= xq / a_scale (inverse of
 * O2), out[m,n] = acc[m,n] * scale[n] / a_scale[m].  Evaluated in fp64, then rounded
 * once to fp32 (RNE) and once to bf16 (RNE).  Any output pointer may be NULL.
 */
static void rescale_one(int32_t acc, float s, float a, double* ref, float* f32,
                        uint16_t* bf16) {
    double r = (double)acc * (double)s / (double)a;
    if (ref) *ref = r;
    if (f32) *f32 = (float)r;
    if (bf16) *bf16 = f64_to_bf16_rne(r);
}

int oracle_rescale(const int32_t* acc, const float* a_scale, const float* w_scale, int64_t M,
                   int64_t N, double* ref, float* out_f32, uint16_t* out_bf16) {
    if (!acc || !a_scale || !w_scale || M < 0 || N < 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t i = m * N + n;
            rescale_one(acc[i], w_scale[n], a_scale[m], ref ? ref + i : NULL,
                        out_f32 ? out_f32 + i : NULL, out_bf16 ? out_bf16 + i : NULL);
        }
    return 0;
}

/* ------------------------------------------------------ code table conversion --- */

/*
 * [Deep] §4.3 (位打包) prints a second 2-bit code table: 11 -> +1, 00 -> 0, 01 -> -1, 10
 * never used, with the same bit positions (weight 4j+i in bits 2i..2i+1).  Table 0 is
 * this library's code = w + 1 (11 never used).  Each field is decoded with the source
 * table and encoded with the destination table; a field holding the unused code is
 * counted and written as weight 0.  Returns the count (or -1 on bad arguments).
 */
static int table_weight(int table, unsigned c) {
    static const int offset_table[4] = {-1, 0, 1, 99};
    static const int sign_table[4] = {0, -1, 99, 1};
    return table == 0 ? offset_table[c] : sign_table[c];
}

static unsigned table_code(int table, int w) {
    if (table == 0) return (unsigned)(w + 1);
    return w == 1 ? 3u : (w == -1 ? 1u : 0u);
}

int64_t oracle_repack(const uint8_t* in, int64_t N, int64_t K, int from, int to, uint8_t* out) {
    if (!in || !out || N < 0 || K < 4 || K % 4 || from < 0 || from > 1 || to < 0 || to > 1)
        return -1;
    int64_t bad = 0;
    for (int64_t j = 0; j < N * (K / 4); ++j) {
        unsigned byte = 0;
        for (int i = 0; i < 4; ++i) {
            int w = table_weight(from, (in[j] >> (2 * i)) & 3u);
            if (w == 99) { ++bad; w = 0; }
            byte |= table_code(to, w) << (2 * i);
        }
        out[j] = (uint8_t)byte;
    }
    return bad;
}

/* -------------------------------------- O6: bf16 activations x ternary (W1.58A16) --- */

/*
 * [LUT] (introduction and its precision settings): mixed-precision serving multiplies
 * ternary weights with 16-bit activations and accumulates in fp32; [Deep] §2.2: with
 * W in {-1, 0, +1}, Y = X @ W needs only additions and subtractions.  No activation
 * quantization: out[m,n] = w_scale[n] * sum_k x[m,k] * w[n,k], w from the packed codes.
 * Evaluated in fp64 (every product x * w is exact); sumabs[m,n] = w_scale[n] *
 * sum_k |x[m,k] * w[n,k]| is returned for the error bound of a float32 sum.
 */
int oracle_a16(const uint16_t* x, const uint8_t* packed, const float* w_scale, int64_t M,
               int64_t N, int64_t K, double* ref, double* sumabs) {
    if (!x || !packed || !w_scale || !ref || !sumabs || M < 0 || N < 0 || K < 4 || K % 4)
        return -1;
    const int64_t KB = K / 4;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double t = (double)bf16_to_f32(x[m * K + k]) * weight_at(packed, KB, n, k);
                s += t;
                sa += fabs(t);
            }
            ref[m * N + n] = s * (double)w_scale[n];
            sumabs[m * N + n] = sa * (double)w_scale[n];
        }
    return 0;
}

/* ------------------------------------------------------- O5: SwiGLU of the MLP --- */

/*
 * [Deep] §3.2 (BitLlamaMLP): the MLP's hidden activation is act_fn(gate_proj(x)) *
 * up_proj(x) with act_fn = F.silu, and silu(g) = g * sigmoid(g) = g / (1 + exp(-g)).
 * g and u are the two projections' exact outputs (O4's fp64 values); h is evaluated in
 * fp64.
 */
int oracle_swiglu(const double* g, const double* u, int64_t count, double* h) {
    if (!g || !u || !h || count < 0) return -1;
    for (int64_t t = 0; t < count; ++t) h[t] = g[t] / (1.0 + exp(-g[t])) * u[t];
    return 0;
}

/* fp64 -> bf16 (RNE) exposed for the oracle's own pin tests. */
void oracle_f64_to_bf16(const double* x, int64_t count, uint16_t* out) {
    for (int64_t t = 0; t < count; ++t) out[t] = f64_to_bf16_rne(x[t]);
}

/* Threads the OpenMP loops above use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
