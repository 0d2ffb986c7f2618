/*
 * CPU oracle for the Llama-family forward pass. TEST INFRASTRUCTURE ONLY: it
 * is loaded by the tests, by the smoke check and by the bench's CPU-baseline
 * leg, never by the library it checks, and it shares no code with it.
 *
 * It is the plain definition, in the precision the pages fix: the Java engine
 * of "The Forward Pass in Java" (codeloopback.dev) computes in fp32 `float`,
 * accumulates the RMSNorm sum of squares in double (Example 4), evaluates cos,
 * sin and exp in double and rounds them to float (Examples 6, 8, Project 18),
 * and rounds K and V through binary16 when it stores them (Example 10). Every
 * dot product is one sequential fp32 sum over the input index (Example 5).
 * Build flags: -O2 -fno-fast-math -ffp-contract=off, so no multiply-add is
 * fused (FMA fusion is a named source of divergence in "What a Llama model
 * computes, and why", section 8).
 *
 * OpenMP splits only over independent output rows or heads, so each output is
 * computed by one thread in a fixed order and the result does not depend on
 * the thread count ("The Engine", design notes on threading).
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * against values the pages print, closed forms, invariants and brute force.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_Q8_0 8

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_MISSING (-2)
#define ORC_ERR_SHAPE (-3)
#define ORC_ERR_DTYPE (-4)
#define ORC_ERR_SIZE (-5)
#define ORC_ERR_POS (-6)
#define ORC_ERR_OOM (-7)

/* attn_window / attn_sinks: "The Engine", its built-in attentions sliding:N
 * and sink:s,w (0 = the full causal span); attn_temp_scale / attn_temp_len:
 * "What a Llama model computes, and why", section 6, Mistral 3's attention
 * temperature (beta and the original context; beta 0 = none). */
typedef struct {
    int32_t dim, n_layers, n_heads, n_kv_heads, head_dim, ffn, vocab, n_ctx, rope_dims, rope_neox;
    float eps, rope_base;
    int32_t attn_window, attn_sinks;
    float attn_temp_scale;
    int32_t attn_temp_len;
    /* YaRN ("What a Llama model computes, and why", section 6; Peng et al.,
     * 2023): scale factor (0 = off), original context, ramp ends */
    float yarn_factor;
    int32_t yarn_orig_ctx;
    float yarn_beta_fast, yarn_beta_slow;
    /* 0: float activations (the Java engine); 1: llama.cpp's rounding points
     * ("What a Llama model computes, and why", section 8) */
    int32_t numerics;
} orc_config;

typedef struct {
    const char* name;
    int32_t dtype;
    int32_t n_dims;
    int64_t ne[2];
    const void* data;
    size_t nbytes;
} orc_tensor;

/* ------------------------------------------------------------------------
 * binary16 <-> binary32, written from IEEE 754-2008 (round to nearest even,
 * subnormals kept). "Loading GGUF with the FFM API", Example 7 states the
 * rounding rule; the F16 KV cache of "The Forward Pass in Java", Example 10
 * stores through it.
 * ---------------------------------------------------------------------- */
float orc_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    float f;
    if (e == 0) {
        f = ldexpf((float)m, -24); /* zero or subnormal: m * 2^-24, exact in float */
        uint32_t b;
        memcpy(&b, &f, 4);
        b |= sign;
        memcpy(&f, &b, 4);
        return f;
    }
    uint32_t b;
    if (e == 31)
        b = sign | 0x7f800000u | (m << 13);
    else
        b = sign | ((e - 15 + 127) << 23) | (m << 13);
    memcpy(&f, &b, 4);
    return f;
}

uint16_t orc_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) return sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u); /* NaN stays NaN */
    int e = (int)(ax >> 23) - 127;                                                /* unbiased exponent */
    uint32_t sig = (ax & 0x7fffffu) | 0x800000u;                                  /* 24-bit significand */
    if (ax == 0) return sign;
    /* Number of low significand bits to drop: 13 in the normal range, more below. */
    int drop = (e >= -14) ? 13 : 13 + (-14 - e);
    if (drop > 24) return sign; /* below half of the smallest subnormal */
    uint32_t kept = sig >> drop;
    uint32_t rem = sig & ((1u << drop) - 1u), halfway = 1u << (drop - 1);
    if (rem > halfway || (rem == halfway && (kept & 1u))) kept += 1u;
    uint32_t h;
    if (e >= -14)
        h = ((uint32_t)(e + 15) << 10) + (kept - 0x400u); /* implicit bit removed; a carry bumps the exponent */
    else
        h = kept; /* subnormal (a carry to 0x400 is the smallest normal) */
    if (h >= 0x7c00u) h = 0x7c00u; /* overflow to infinity */
    return sign | (uint16_t)h;
}

/* ------------------------------------------------------------------------
 * Dequantisation to float ("The Forward Pass in Java", Example 2; "Loading
 * GGUF with the FFM API", Examples 7 and 8): F32 is copied, F16 is converted
 * per value, a Q8_0 block {fp16 d, int8 qs[32]} decodes to d * qs[j].
 * ---------------------------------------------------------------------- */
int orc_dequantize(int32_t dtype, const void* data, int64_t n, float* out) {
    const uint8_t* p = (const uint8_t*)data;
    if (dtype == ORC_F32) {
        memcpy(out, data, (size_t)n * 4);
        return ORC_OK;
    }
    if (dtype == ORC_F16) {
        for (int64_t i = 0; i < n; i++) {
            uint16_t h = (uint16_t)(p[2 * i] | (p[2 * i + 1] << 8));
            out[i] = orc_f16_to_f32(h);
        }
        return ORC_OK;
    }
    if (dtype == ORC_Q8_0) {
        if (n % 32) return ORC_ERR_SHAPE;
        for (int64_t b = 0; b < n / 32; b++) {
            const uint8_t* blk = p + 34 * b;
            float d = orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int j = 0; j < 32; j++) out[32 * b + j] = d * (float)(int8_t)blk[2 + j];
        }
        return ORC_OK;
    }
    return ORC_ERR_DTYPE;
}

/*
 * Q8_0 encoding of 32-value blocks ("Loading GGUF with the FFM API", the Q8_0
 * section and Example 8's quantizer; "The Forward Pass in Java", Example 2).
 * The block's scale is its largest magnitude divided by 127, in float. Each
 * code is the value times the scale's float reciprocal, rounded to the nearest
 * integer with halves away from zero (C's roundf is that rule); an all-zero
 * block has scale 0 and codes 0. The stored scale is the binary16 rounding of
 * the float scale. Used for the pages' worked Q8_0 examples and for the
 * rounding mode's product inputs; the workloads draw their Q8_0 blocks
 * directly.
 */
static float q8_block_scale(const float* x) {
    float amax = 0.0f;
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(x[j]));
    return amax / 127.0f;
}

static void q8_encode_block(const float* x, uint8_t* blk) {
    const float d = q8_block_scale(x);
    const float inv = d > 0.0f ? 1.0f / d : 0.0f;
    int8_t* codes = (int8_t*)(blk + 2);
    for (int j = 0; j < 32; j++) codes[j] = (int8_t)roundf(x[j] * inv);
    const uint16_t dh = orc_f32_to_f16(d);
    blk[0] = (uint8_t)dh;
    blk[1] = (uint8_t)(dh >> 8);
}

int orc_quantize_q8_0(const float* x, int64_t n, uint8_t* out) {
    if (n % 32) return ORC_ERR_SHAPE;
    for (int64_t b = 0; b < n / 32; b++) q8_encode_block(x + 32 * b, out + 34 * b);
    return ORC_OK;
}

/* llama.cpp's rounding of a matrix product's input ("What a Llama model
 * computes, and why", section 8): for Q8_0 weights each block of 32 is
 * quantized as orc_quantize_q8_0 does (Example 8's quantizer) and the product
 * sees the block's binary16 scale times its code; for F16 weights the input is
 * rounded to binary16; F32 weights see it unchanged. In place, n values. */
int orc_round_input(float* x, int64_t n, int32_t dtype) {
    if (dtype == ORC_F16) {
        for (int64_t i = 0; i < n; i++) x[i] = orc_f16_to_f32(orc_f32_to_f16(x[i])); /* binary16 RNE */
        return ORC_OK;
    }
    if (dtype != ORC_Q8_0) return ORC_OK;
    if (n % 32) return ORC_ERR_SHAPE;
    uint8_t blk[34];
    for (int64_t b = 0; b < n / 32; b++) {
        orc_quantize_q8_0(x + 32 * b, 32, blk);
        orc_dequantize(ORC_Q8_0, blk, 32, x + 32 * b);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * The operations of the forward pass ("The Forward Pass in Java",
 * Examples 3-10 and Project 18; "What a Llama model computes, and why",
 * section 2).
 * ---------------------------------------------------------------------- */

/* RMSNorm ("The Forward Pass in Java", Example 4; "What a Llama model computes,
 * and why", section 2): out = x * r * w with r = 1 / sqrt(mean(x^2) + eps). The
 * mean square is accumulated in double over i ascending, r is evaluated in
 * double and rounded to float once, and each output is (x_i * r) * w_i in
 * float. */
static double mean_square(const float* x, int32_t n) {
    double acc = 0.0;
    for (int32_t i = 0; i < n; i++) acc += (double)x[i] * (double)x[i];
    return acc / (double)n;
}

void orc_rmsnorm(float* out, const float* x, const float* w, int32_t n, float eps) {
    const float r = (float)(1.0 / sqrt(mean_square(x, n) + (double)eps));
    for (int32_t i = 0; i < n; i++) out[i] = x[i] * r * w[i];
}

/* One sequential fp32 dot product over i ascending (Example 5). Two other
 * builds of this file evaluate the same definition in another valid way, used
 * only to measure how far the rounding of the sums alone moves a workload's
 * logits ("What a Llama model computes, and why", section 8, names summation
 * order as a source of divergence between implementations):
 *  - ORC_DOT_DESCENDING (liboracle_desc.so) sums the same fp32 products over i
 *    descending;
 *  - ORC_SUM_F64 (liboracle_f64.so) accumulates every sum of the layer and the
 *    attention (these dot products, the attention scores, the softmax total
 *    and the weighted sum of V) in double and rounds it to float once: the
 *    definition summed almost exactly. */
#ifdef ORC_SUM_F64
typedef double acc_t;
#else
typedef float acc_t;
#endif
static float dot(const float* w, const float* x, int64_t n) {
    acc_t s = 0;
#ifdef ORC_DOT_DESCENDING
    for (int64_t i = n - 1; i >= 0; i--) s += (acc_t)w[i] * x[i];
#else
    for (int64_t i = 0; i < n; i++) s += (acc_t)w[i] * x[i];
#endif
    return (float)s;
}

/* Matrix-vector product in GGUF order, Example 5: a tensor with dims
 * [cols, rows] stores row r at r * cols; out[r] = sum_i w[r*cols + i] * x[i]. */
void orc_matvec(float* out, const float* w, const float* x, int32_t rows, int32_t cols) {
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < rows; r++) out[r] = dot(w + (int64_t)r * cols, x, cols);
}

/* The same product for n inputs at once, row-outer: each weight row is read
 * once and dotted with every input, each dot exactly as orc_matvec computes it
 * ("What a Llama model computes, and why", section 4: a batch reads each weight
 * once, and each row of the batched product performs the vector product's
 * operations). x is [n][cols], out is [n][rows]. */
void orc_matmul(float* out, const float* w, const float* x, int32_t n, int32_t rows, int32_t cols) {
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < rows; r++)
        for (int32_t t = 0; t < n; t++) out[(int64_t)t * rows + r] = dot(w + (int64_t)r * cols, x + (int64_t)t * cols, cols);
}

/* The rotation angles of one position, Example 6: theta_scale = base^(-2/n_rot)
 * evaluated in double and rounded to float; theta starts at pos and is
 * multiplied by theta_scale in float once per pair; cos and sin are taken in
 * double and rounded to float. With frequency factors ("What a Llama model
 * computes, and why", sections 2.4 and 6: theta_i = p base^(-2i/n) / f_i, one
 * divisor per pair from rope_freqs.weight) pair i's angle is that theta
 * divided by freq[i] in float; freq NULL means every f_i = 1. */
/* YaRN's per-pair angle change and its attention rescaling, as the YaRN paper
 * (Peng et al., 2023) defines them and "What a Llama model computes, and
 * why", section 6, describes them: pair i, of base frequency
 * theta_i = base^(-2i/n) radians per position, completes r = L theta_i / (2 pi)
 * turns over the original context L. The ramp g(r) is 0 below beta_slow, 1
 * above beta_fast and linear in between; the angle a becomes
 * (1 - g) a / s + g a (fast pairs keep theirs, slow pairs are interpolated by
 * the factor s), evaluated in double and rounded to float. Both q and k are
 * scaled by m = 1 + 0.1 ln s (so the logits by m^2), folded into cos and sin. */
typedef struct {
    float factor;
    int32_t orig_ctx;
    float beta_fast, beta_slow;
} orc_yarn;

double orc_yarn_ramp(const orc_yarn* y, int32_t i, int32_t rope_dims, float base) {
    const double theta = pow((double)base, -2.0 * i / rope_dims);
    const double r = (double)y->orig_ctx * theta / 6.283185307179586476925286766559;
    if (r < y->beta_slow) return 0.0;
    if (r > y->beta_fast) return 1.0;
    return (r - y->beta_slow) / ((double)y->beta_fast - y->beta_slow);
}

void orc_rope_cos_sin_y(int32_t pos, int32_t rope_dims, float base, const float* freq, const orc_yarn* y,
                        float* cos_out, float* sin_out) {
    float theta_scale = (float)pow((double)base, -2.0 / rope_dims);
    float theta = (float)pos;
    const double m = y ? 1.0 + 0.1 * log((double)y->factor) : 1.0;
    for (int32_t i = 0; i < rope_dims / 2; i++) {
        float angle = freq ? theta / freq[i] : theta;
        if (y) {
            const double g = orc_yarn_ramp(y, i, rope_dims, base);
            angle = (float)((1.0 - g) * ((double)angle / y->factor) + g * (double)angle);
        }
        cos_out[i] = (float)(m * cos((double)angle));
        sin_out[i] = (float)(m * sin((double)angle));
        theta *= theta_scale;
    }
}

void orc_rope_cos_sin_ff(int32_t pos, int32_t rope_dims, float base, const float* freq, float* cos_out,
                         float* sin_out) {
    orc_rope_cos_sin_y(pos, rope_dims, base, freq, NULL, cos_out, sin_out);
}

void orc_rope_cos_sin(int32_t pos, int32_t rope_dims, float base, float* cos_out, float* sin_out) {
    orc_rope_cos_sin_ff(pos, rope_dims, base, NULL, cos_out, sin_out);
}

/* RoPE, Example 6: rotate pair i of every head by theta_i. Normal layout pairs
 * (2i, 2i+1); NEOX pairs (i, i + n_rot/2). Dimensions past n_rot are left alone. */
void orc_rope_y(float* vec, int32_t n_heads, int32_t head_dim, int32_t rope_dims, int32_t pos, float base,
                int32_t neox, const float* freq, const orc_yarn* y) {
    float* c = (float*)malloc(sizeof(float) * (size_t)(rope_dims / 2 + 1));
    float* s = (float*)malloc(sizeof(float) * (size_t)(rope_dims / 2 + 1));
    orc_rope_cos_sin_y(pos, rope_dims, base, freq, y, c, s);
    for (int32_t h = 0; h < n_heads; h++) {
        for (int32_t i = 0; i < rope_dims / 2; i++) {
            int32_t a = h * head_dim + (neox ? i : 2 * i);
            int32_t b = neox ? a + rope_dims / 2 : a + 1;
            float x0 = vec[a], x1 = vec[b];
            vec[a] = x0 * c[i] - x1 * s[i];
            vec[b] = x0 * s[i] + x1 * c[i];
        }
    }
    free(c);
    free(s);
}

void orc_rope_ff(float* vec, int32_t n_heads, int32_t head_dim, int32_t rope_dims, int32_t pos, float base,
                 int32_t neox, const float* freq) {
    orc_rope_y(vec, n_heads, head_dim, rope_dims, pos, base, neox, freq, NULL);
}

void orc_rope(float* vec, int32_t n_heads, int32_t head_dim, int32_t rope_dims, int32_t pos, float base, int32_t neox) {
    orc_rope_ff(vec, n_heads, head_dim, rope_dims, pos, base, neox, NULL);
}

/* silu(z) = z / (1 + e^-z), Example 8. */
float orc_silu(float z) { return z / (1.0f + (float)exp(-(double)z)); }

/* Greedy choice, Example 9: the first index of the strict maximum (a later
 * equal value never replaces the one found first). */
int32_t orc_argmax(const float* v, int32_t n) {
    int32_t at = 0;
    float top = v[0];
    for (int32_t i = 1; i < n; i++)
        if (v[i] > top) {
            top = v[i];
            at = i;
        }
    return at;
}

/*
 * Cached grouped-query attention for one token at position pos, Example 7 and
 * Project 18. The caches hold binary16 bits in the pages' flat layout: row t of
 * kv head g starts at t * kv_dim + g * head_dim. Query head h reads kv head
 * h / (n_heads / n_kv_heads). Scores are divided by (float)sqrt(head_dim); the
 * softmax subtracts the maximum, takes exp in double rounded to float, sums in
 * float over t ascending; then out_h = sum_t (e_t / sum) * V_t.
 * `weights`, when not NULL, receives the normalised weights [n_heads][pos+1].
 */
/* Mistral 3's attention temperature ("What a Llama model computes, and why",
 * section 6, the family table and the temperature section): the query at
 * position pos is scaled by 1 + beta * ln(floor(pos / len) + 1), exactly 1
 * below len. Evaluated in double, rounded to float. beta 0: no temperature. */
float orc_attn_temp(int32_t pos, float beta, int32_t len) {
    if (beta == 0.0f || len <= 0) return 1.0f;
    return (float)(1.0 + (double)beta * log((double)(pos / len) + 1.0));
}

/* Whether cache row t is attended by the query at position pos: every row up
 * to pos for the full causal span (window 0); with window w > 0 only the last
 * w rows (pos - w < t <= pos, sliding:N of "The Engine"), plus the first
 * `sinks` rows (sink:s,w, the sinks-plus-window eviction). */
int orc_attends(int32_t t, int32_t pos, int32_t window, int32_t sinks) {
    if (t < 0 || t > pos) return 0;
    if (window <= 0) return 1;
    return t > pos - window || t < sinks;
}

/* Scaled dot-product attention of one token over the F16 cache ("The Forward
 * Pass in Java", Example 7; "What a Llama model computes, and why", section 2):
 * for query head h, reading KV head h / (n_heads / n_kv_heads),
 *   s_t = (q_h . K_t) / sqrt(head_dim) over the attended rows t,
 *   p_t = exp(s_t - max s) / sum exp(s_t - max s),
 *   out_h = sum_t p_t V_t.
 * q is first scaled by the temperature of pos (float). Each dot product is a
 * float sum over the dimensions in order; sqrt(head_dim) is taken in double
 * and rounded to float, and the score is divided by it; exp is taken in double
 * and rounded to float; the sum of the exponentials is a float sum over t
 * ascending; p_t is one float division; out_h accumulates p_t V_t over t
 * ascending. weights (optional) gets [n_heads][pos + 1] probabilities, 0 for
 * rows not attended.
 *
 * round16 (llama.cpp's rounding points, "What a Llama model computes, and
 * why", section 8): the temperature-scaled query is rounded to binary16 before
 * the dot products, and each p_t, after the division, before it weights V;
 * weights then receives the rounded probabilities. */
static float f16_round(float x) { return orc_f16_to_f32(orc_f32_to_f16(x)); }

/* s_t for the attended rows of 0..pos (others untouched); returns max s_t. */
static float attn_scores(float* s, const float* q, const uint16_t* kc, int32_t kv_dim, int32_t kv_off, int32_t hd,
                         int32_t pos, int32_t window, int32_t sinks) {
    const float root = (float)sqrt((double)hd);
    float top = -INFINITY;
    for (int32_t t = 0; t <= pos; t++) {
        if (!orc_attends(t, pos, window, sinks)) continue;
        const uint16_t* k = kc + (int64_t)t * kv_dim + kv_off;
        acc_t acc = 0;
        for (int32_t i = 0; i < hd; i++) acc += (acc_t)q[i] * orc_f16_to_f32(k[i]);
        s[t] = (float)acc / root;
        top = fmaxf(top, s[t]);
    }
    return top;
}

/* s_t -> p_t in place over the attended rows; rows not attended get 0. */
static void attn_softmax(float* s, float top, int32_t pos, int32_t window, int32_t sinks, int32_t round16) {
    acc_t sum = 0;
    for (int32_t t = 0; t <= pos; t++)
        if (orc_attends(t, pos, window, sinks)) {
            s[t] = (float)exp((double)(s[t] - top));
            sum += s[t];
        }
    const float total = (float)sum;
    for (int32_t t = 0; t <= pos; t++) {
        float p = orc_attends(t, pos, window, sinks) ? s[t] / total : 0.0f;
        s[t] = round16 ? f16_round(p) : p;
    }
}

/* out = sum of p_t V_t over the attended rows, t ascending. */
static void attn_weighted_sum(float* out, const float* p, const uint16_t* vc, int32_t kv_dim, int32_t kv_off,
                              int32_t hd, int32_t pos, int32_t window, int32_t sinks) {
    acc_t* acc = (acc_t*)calloc((size_t)hd, sizeof(acc_t));
    for (int32_t t = 0; t <= pos; t++) {
        if (!orc_attends(t, pos, window, sinks)) continue;
        const uint16_t* v = vc + (int64_t)t * kv_dim + kv_off;
        for (int32_t i = 0; i < hd; i++) acc[i] += (acc_t)p[t] * orc_f16_to_f32(v[i]);
    }
    for (int32_t i = 0; i < hd; i++) out[i] = (float)acc[i];
    free(acc);
}

void orc_attention_nx(float* out, const float* q, const uint16_t* kcache, const uint16_t* vcache, int32_t n_heads,
                      int32_t n_kv_heads, int32_t head_dim, int32_t pos, int32_t window, int32_t sinks,
                      float temp_scale, int32_t temp_len, int32_t round16, float* weights) {
    const int32_t kv_dim = n_kv_heads * head_dim, group = n_heads / n_kv_heads;
    const float tau = orc_attn_temp(pos, temp_scale, temp_len);
    for (int32_t i = 0; i < n_heads * head_dim; i++) out[i] = 0.0f;
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < n_heads; h++) {
        float* s = (float*)malloc(sizeof(float) * (size_t)(pos + 1));
        float* qh = (float*)malloc(sizeof(float) * (size_t)head_dim);
        const int32_t kv_off = (h / group) * head_dim;
        for (int32_t i = 0; i < head_dim; i++) {
            qh[i] = tau * q[h * head_dim + i];
            if (round16) qh[i] = f16_round(qh[i]);
        }
        const float top = attn_scores(s, qh, kcache, kv_dim, kv_off, head_dim, pos, window, sinks);
        attn_softmax(s, top, pos, window, sinks, round16);
        if (weights) memcpy(weights + (int64_t)h * (pos + 1), s, sizeof(float) * (size_t)(pos + 1));
        attn_weighted_sum(out + h * head_dim, s, vcache, kv_dim, kv_off, head_dim, pos, window, sinks);
        free(qh);
        free(s);
    }
}

void orc_attention_ex(float* out, const float* q, const uint16_t* kcache, const uint16_t* vcache, int32_t n_heads,
                      int32_t n_kv_heads, int32_t head_dim, int32_t pos, int32_t window, int32_t sinks,
                      float temp_scale, int32_t temp_len, float* weights) {
    orc_attention_nx(out, q, kcache, vcache, n_heads, n_kv_heads, head_dim, pos, window, sinks, temp_scale, temp_len, 0,
                     weights);
}

/* The full causal span without temperature. */
void orc_attention(float* out, const float* q, const uint16_t* kcache, const uint16_t* vcache, int32_t n_heads,
                   int32_t n_kv_heads, int32_t head_dim, int32_t pos, float* weights) {
    orc_attention_ex(out, q, kcache, vcache, n_heads, n_kv_heads, head_dim, pos, 0, 0, 0.0f, 0, weights);
}

/* ------------------------------------------------------------------------
 * The model: Project 18's Llama class as plain C ("The Forward Pass in Java",
 * Example 13) with the prefill batch of "What a Llama model computes, and
 * why", section 4.
 * ---------------------------------------------------------------------- */
typedef struct {
    float *attn_norm, *wq, *wk, *wv, *bq, *bk, *bv, *wo, *ffn_norm, *gate, *up, *down;
    int32_t dt_q, dt_k, dt_v, dt_o, dt_gate, dt_up, dt_down; /* stored types of the matrices */
} orc_layer;

typedef struct orc_model {
    orc_config c;
    float *tok_embd, *out_norm, *output;
    float* rope_freqs; /* optional per-pair divisors (rope_freqs.weight) or NULL */
    orc_yarn yarn;
    const orc_yarn* yarn_on; /* &yarn, or NULL without YaRN */
    int tied;
    int32_t dt_out; /* stored type of the output (or tied embedding) matrix */
    orc_layer* layers;
    uint16_t *kcache, *vcache; /* [layer][n_ctx][kv_dim] binary16 bits */
    int32_t len;
} orc_model;

static const orc_tensor* find(const orc_tensor* ts, int32_t n, const char* name) {
    for (int32_t i = 0; i < n; i++)
        if (ts[i].name && strcmp(ts[i].name, name) == 0) return &ts[i];
    return NULL;
}

static int32_t last_dtype; /* stored type of the tensor take() read last (load is single-threaded) */

static int64_t need_bytes(int32_t dtype, int64_t n) {
    if (dtype == ORC_F32) return 4 * n;
    if (dtype == ORC_F16) return 2 * n;
    if (dtype == ORC_Q8_0) return n / 32 * 34;
    return -1;
}

/* Fetch tensor `name` with dims (ne0[, ne1]) and dequantise it into a new array. */
static int take(const orc_tensor* ts, int32_t n, const char* name, int64_t ne0, int64_t ne1, int optional,
                float** out) {
    const orc_tensor* t = find(ts, n, name);
    *out = NULL;
    if (t) last_dtype = t->dtype;
    if (!t) return optional ? ORC_OK : ORC_ERR_MISSING;
    int dims = ne1 > 0 ? 2 : 1;
    if (t->n_dims != dims || t->ne[0] != ne0 || (dims == 2 && t->ne[1] != ne1)) return ORC_ERR_SHAPE;
    if (t->dtype != ORC_F32 && t->dtype != ORC_F16 && t->dtype != ORC_Q8_0) return ORC_ERR_DTYPE;
    if (t->dtype == ORC_Q8_0 && ne0 % 32) return ORC_ERR_SHAPE;
    int64_t cnt = ne0 * (dims == 2 ? ne1 : 1);
    if (!t->data || (int64_t)t->nbytes < need_bytes(t->dtype, cnt)) return ORC_ERR_SIZE;
    *out = (float*)malloc(sizeof(float) * (size_t)cnt);
    if (!*out) return ORC_ERR_OOM;
    return orc_dequantize(t->dtype, t->data, cnt, *out);
}

void orc_free(orc_model* m);

int orc_load(const orc_config* cfg, const orc_tensor* ts, int32_t n, orc_model** out) {
    *out = NULL;
    const orc_config c = *cfg;
    if (c.dim <= 0 || c.n_layers <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 || c.ffn <= 0 ||
        c.vocab <= 0 || c.n_ctx <= 0 || c.n_heads % c.n_kv_heads || c.rope_dims <= 0 || c.rope_dims > c.head_dim ||
        c.rope_dims % 2 || c.attn_window < 0 || c.attn_sinks < 0 || (c.attn_sinks > 0 && c.attn_window == 0) ||
        !(c.attn_temp_scale >= 0.0f && c.attn_temp_scale < INFINITY) || (c.attn_temp_scale > 0.0f && c.attn_temp_len <= 0) ||
        !(c.yarn_factor == 0.0f || (c.yarn_factor >= 1.0f && c.yarn_factor < INFINITY && c.yarn_orig_ctx > 0 &&
                                    c.yarn_beta_slow >= 0.0f && c.yarn_beta_fast > c.yarn_beta_slow &&
                                    c.yarn_beta_fast < INFINITY)) || (c.numerics != 0 && c.numerics != 1))
        return ORC_ERR_ARG;
    orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
    m->c = c;
    if (c.yarn_factor > 0.0f) {
        m->yarn.factor = c.yarn_factor;
        m->yarn.orig_ctx = c.yarn_orig_ctx;
        m->yarn.beta_fast = c.yarn_beta_fast;
        m->yarn.beta_slow = c.yarn_beta_slow;
        m->yarn_on = &m->yarn;
    }
    m->layers = (orc_layer*)calloc((size_t)c.n_layers, sizeof(orc_layer));
    int32_t qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    int rc = take(ts, n, "token_embd.weight", c.dim, c.vocab, 0, &m->tok_embd);
    if (!rc) rc = take(ts, n, "output_norm.weight", c.dim, 0, 0, &m->out_norm);
    m->dt_out = last_dtype; /* the embedding's, unless an output matrix follows */
    if (!rc) rc = take(ts, n, "output.weight", c.dim, c.vocab, 1, &m->output);
    if (!rc && m->output) m->dt_out = last_dtype;
    if (!rc) rc = take(ts, n, "rope_freqs.weight", c.rope_dims / 2, 0, 1, &m->rope_freqs);
    if (!rc && !m->output) { /* tied embeddings (Example 9) */
        m->output = m->tok_embd;
        m->tied = 1;
    }
    char name[128];
    for (int32_t l = 0; l < c.n_layers && !rc; l++) {
        orc_layer* L = &m->layers[l];
#define TAKE(field, suffix, a, b, opt)                                      \
    if (!rc) {                                                              \
        snprintf(name, sizeof name, "blk.%d.%s", (int)l, suffix);           \
        rc = take(ts, n, name, a, b, opt, &L->field);                       \
    }
        TAKE(attn_norm, "attn_norm.weight", c.dim, 0, 0)
        TAKE(wq, "attn_q.weight", c.dim, qd, 0)
        L->dt_q = last_dtype;
        TAKE(wk, "attn_k.weight", c.dim, kvd, 0)
        L->dt_k = last_dtype;
        TAKE(wv, "attn_v.weight", c.dim, kvd, 0)
        L->dt_v = last_dtype;
        TAKE(bq, "attn_q.bias", qd, 0, 1)
        TAKE(bk, "attn_k.bias", kvd, 0, 1)
        TAKE(bv, "attn_v.bias", kvd, 0, 1)
        TAKE(wo, "attn_output.weight", qd, c.dim, 0)
        L->dt_o = last_dtype;
        TAKE(ffn_norm, "ffn_norm.weight", c.dim, 0, 0)
        TAKE(gate, "ffn_gate.weight", c.dim, c.ffn, 0)
        L->dt_gate = last_dtype;
        TAKE(up, "ffn_up.weight", c.dim, c.ffn, 0)
        L->dt_up = last_dtype;
        TAKE(down, "ffn_down.weight", c.ffn, c.dim, 0)
        L->dt_down = last_dtype;
#undef TAKE
        if (!rc && !((L->bq && L->bk && L->bv) || (!L->bq && !L->bk && !L->bv))) rc = ORC_ERR_MISSING;
    }
    if (!rc) {
        size_t cache = (size_t)c.n_layers * (size_t)c.n_ctx * (size_t)kvd;
        m->kcache = (uint16_t*)calloc(cache, 2);
        m->vcache = (uint16_t*)calloc(cache, 2);
        if (!m->kcache || !m->vcache) rc = ORC_ERR_OOM;
    }
    if (rc) {
        orc_free(m);
        return rc;
    }
    *out = m;
    return ORC_OK;
}

void orc_free(orc_model* m) {
    if (!m) return;
    if (m->layers) {
        for (int32_t l = 0; l < m->c.n_layers; l++) {
            orc_layer* L = &m->layers[l];
            float* ps[] = {L->attn_norm, L->wq, L->wk, L->wv, L->bq, L->bk, L->bv, L->wo, L->ffn_norm, L->gate, L->up, L->down};
            for (size_t i = 0; i < sizeof ps / sizeof ps[0]; i++) free(ps[i]);
        }
        free(m->layers);
    }
    if (!m->tied) free(m->output);
    free(m->tok_embd);
    free(m->out_norm);
    free(m->rope_freqs);
    free(m->kcache);
    free(m->vcache);
    free(m);
}

static void add_bias(float* x, const float* b, int32_t n) {
    if (b)
        for (int32_t i = 0; i < n; i++) x[i] += b[i];
}

/* Store one position's K and V, rounding through binary16 (Example 10). */
static void store_kv(orc_model* m, int32_t l, int32_t pos, const float* k, const float* v) {
    int32_t kvd = m->c.n_kv_heads * m->c.head_dim;
    size_t base = ((size_t)l * (size_t)m->c.n_ctx + (size_t)pos) * (size_t)kvd;
    for (int32_t i = 0; i < kvd; i++) {
        m->kcache[base + i] = orc_f32_to_f16(k[i]);
        m->vcache[base + i] = orc_f32_to_f16(v[i]);
    }
}

static const uint16_t* layer_k(const orc_model* m, int32_t l) {
    return m->kcache + (size_t)l * (size_t)m->c.n_ctx * (size_t)(m->c.n_kv_heads * m->c.head_dim);
}
static const uint16_t* layer_v(const orc_model* m, int32_t l) {
    return m->vcache + (size_t)l * (size_t)m->c.n_ctx * (size_t)(m->c.n_kv_heads * m->c.head_dim);
}

/* out[t][rows] = W x_t for the n inputs x (n x cols), with x rounded for W's
 * stored type first when the model uses llama.cpp's rounding points; tmp has
 * room for n x cols floats. */
static void product(const orc_model* m, float* out, const float* w, int32_t dt, const float* x, int32_t n, int32_t rows,
                    int32_t cols, float* tmp) {
    if (m->c.numerics && dt != ORC_F32) {
        memcpy(tmp, x, sizeof(float) * (size_t)n * (size_t)cols);
        for (int32_t t = 0; t < n; t++) orc_round_input(tmp + (int64_t)t * cols, cols, dt);
        x = tmp;
    }
    orc_matmul(out, w, x, n, rows, cols);
}

/*
 * One token at position pos (Project 18, forward): fills the cache at pos in
 * every layer and writes the logits. Requires 0 <= pos <= len and pos < n_ctx;
 * afterwards len = pos + 1.
 */
int orc_forward(orc_model* m, int32_t token, int32_t pos, float* logits) {
    const orc_config c = m->c;
    if (token < 0 || token >= c.vocab) return ORC_ERR_ARG;
    if (pos < 0 || pos > m->len || pos >= c.n_ctx) return ORC_ERR_POS;
    int32_t qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    float* x = (float*)malloc(sizeof(float) * (size_t)c.dim);
    float* xb = (float*)malloc(sizeof(float) * (size_t)(c.dim > qd ? c.dim : qd));
    float* q = (float*)malloc(sizeof(float) * (size_t)qd);
    float* k = (float*)malloc(sizeof(float) * (size_t)kvd);
    float* v = (float*)malloc(sizeof(float) * (size_t)kvd);
    float* heads = (float*)malloc(sizeof(float) * (size_t)qd);
    float* hb = (float*)malloc(sizeof(float) * (size_t)c.ffn);
    float* hb2 = (float*)malloc(sizeof(float) * (size_t)c.ffn);
    int32_t widest = c.ffn > c.dim ? c.ffn : c.dim;
    if (qd > widest) widest = qd;
    float* tmp = (float*)malloc(sizeof(float) * (size_t)widest);

    memcpy(x, m->tok_embd + (int64_t)token * c.dim, sizeof(float) * (size_t)c.dim); /* Example 3 */
    for (int32_t l = 0; l < c.n_layers; l++) {
        const orc_layer* w = &m->layers[l];
        orc_rmsnorm(xb, x, w->attn_norm, c.dim, c.eps);
        product(m, q, w->wq, w->dt_q, xb, 1, qd, c.dim, tmp);
        product(m, k, w->wk, w->dt_k, xb, 1, kvd, c.dim, tmp);
        product(m, v, w->wv, w->dt_v, xb, 1, kvd, c.dim, tmp);
        add_bias(q, w->bq, qd);
        add_bias(k, w->bk, kvd);
        add_bias(v, w->bv, kvd);
        orc_rope_y(q, c.n_heads, c.head_dim, c.rope_dims, pos, c.rope_base, c.rope_neox, m->rope_freqs, m->yarn_on);
        orc_rope_y(k, c.n_kv_heads, c.head_dim, c.rope_dims, pos, c.rope_base, c.rope_neox, m->rope_freqs, m->yarn_on);
        store_kv(m, l, pos, k, v);
        orc_attention_nx(heads, q, layer_k(m, l), layer_v(m, l), c.n_heads, c.n_kv_heads, c.head_dim, pos,
                         c.attn_window, c.attn_sinks, c.attn_temp_scale, c.attn_temp_len, c.numerics, NULL);
        product(m, xb, w->wo, w->dt_o, heads, 1, c.dim, qd, tmp);
        for (int32_t i = 0; i < c.dim; i++) x[i] += xb[i];
        orc_rmsnorm(xb, x, w->ffn_norm, c.dim, c.eps);
        product(m, hb, w->gate, w->dt_gate, xb, 1, c.ffn, c.dim, tmp);
        product(m, hb2, w->up, w->dt_up, xb, 1, c.ffn, c.dim, tmp);
        for (int32_t i = 0; i < c.ffn; i++) hb[i] = orc_silu(hb[i]) * hb2[i];
        product(m, xb, w->down, w->dt_down, hb, 1, c.dim, c.ffn, tmp);
        for (int32_t i = 0; i < c.dim; i++) x[i] += xb[i];
    }
    orc_rmsnorm(xb, x, m->out_norm, c.dim, c.eps);
    product(m, logits, m->output, m->dt_out, xb, 1, c.vocab, c.dim, tmp);
    m->len = pos + 1;
    free(x); free(xb); free(q); free(k); free(v); free(heads); free(hb); free(hb2); free(tmp);
    return ORC_OK;
}

/*
 * Prefill of n tokens at positions len .. len+n-1 ("What a Llama model
 * computes, and why", section 4): the products run row-outer over the batch,
 * RMSNorm, RoPE and attention per token, and token i attends cache rows
 * 0 .. len+i. Each token goes through exactly the operations of orc_forward, so
 * the logits and cache equal token-by-token decoding bit for bit. The logits
 * of the last token are written. Afterwards len += n.
 */
/* Logits of the batch rows rows[0..n_rows) (indices into tokens) into
 * out[r * vocab], after the same row-outer pass ("What a Llama model computes,
 * and why", section 4: every row of a prompt has its own next-token logits). */
int orc_prefill_rows(orc_model* m, const int32_t* tokens, int32_t n, const int32_t* rows, int32_t n_rows, float* out) {
    const orc_config c = m->c;
    if (n <= 0 || n_rows <= 0) return ORC_ERR_ARG;
    for (int32_t r = 0; r < n_rows; r++)
        if (rows[r] < 0 || rows[r] >= n) return ORC_ERR_ARG;
    if ((int64_t)m->len + n > c.n_ctx) return ORC_ERR_POS;
    for (int32_t i = 0; i < n; i++)
        if (tokens[i] < 0 || tokens[i] >= c.vocab) return ORC_ERR_ARG;
    int32_t qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim, len = m->len;
    int32_t wide = c.dim > qd ? c.dim : qd;
    float* X = (float*)malloc(sizeof(float) * (size_t)n * (size_t)c.dim);
    float* XB = (float*)malloc(sizeof(float) * (size_t)n * (size_t)wide);
    float* Q = (float*)malloc(sizeof(float) * (size_t)n * (size_t)qd);
    float* K = (float*)malloc(sizeof(float) * (size_t)n * (size_t)kvd);
    float* V = (float*)malloc(sizeof(float) * (size_t)n * (size_t)kvd);
    float* HEADS = (float*)malloc(sizeof(float) * (size_t)n * (size_t)qd);
    float* HB = (float*)malloc(sizeof(float) * (size_t)n * (size_t)c.ffn);
    float* HB2 = (float*)malloc(sizeof(float) * (size_t)n * (size_t)c.ffn);
    int32_t widest = c.ffn > wide ? c.ffn : wide;
    float* TMP = (float*)malloc(sizeof(float) * (size_t)n * (size_t)widest);
    if (!X || !XB || !Q || !K || !V || !HEADS || !HB || !HB2 || !TMP) {
        free(X); free(XB); free(Q); free(K); free(V); free(HEADS); free(HB); free(HB2); free(TMP);
        return ORC_ERR_OOM;
    }
    for (int32_t t = 0; t < n; t++)
        memcpy(X + (int64_t)t * c.dim, m->tok_embd + (int64_t)tokens[t] * c.dim, sizeof(float) * (size_t)c.dim);
    for (int32_t l = 0; l < c.n_layers; l++) {
        const orc_layer* w = &m->layers[l];
        for (int32_t t = 0; t < n; t++) orc_rmsnorm(XB + (int64_t)t * c.dim, X + (int64_t)t * c.dim, w->attn_norm, c.dim, c.eps);
        product(m, Q, w->wq, w->dt_q, XB, n, qd, c.dim, TMP);
        product(m, K, w->wk, w->dt_k, XB, n, kvd, c.dim, TMP);
        product(m, V, w->wv, w->dt_v, XB, n, kvd, c.dim, TMP);
        for (int32_t t = 0; t < n; t++) {
            float *q = Q + (int64_t)t * qd, *k = K + (int64_t)t * kvd, *v = V + (int64_t)t * kvd;
            add_bias(q, w->bq, qd);
            add_bias(k, w->bk, kvd);
            add_bias(v, w->bv, kvd);
            orc_rope_y(q, c.n_heads, c.head_dim, c.rope_dims, len + t, c.rope_base, c.rope_neox, m->rope_freqs, m->yarn_on);
            orc_rope_y(k, c.n_kv_heads, c.head_dim, c.rope_dims, len + t, c.rope_base, c.rope_neox, m->rope_freqs, m->yarn_on);
            store_kv(m, l, len + t, k, v);
        }
        for (int32_t t = 0; t < n; t++)
            orc_attention_nx(HEADS + (int64_t)t * qd, Q + (int64_t)t * qd, layer_k(m, l), layer_v(m, l), c.n_heads,
                             c.n_kv_heads, c.head_dim, len + t, c.attn_window, c.attn_sinks, c.attn_temp_scale,
                             c.attn_temp_len, c.numerics, NULL);
        product(m, XB, w->wo, w->dt_o, HEADS, n, c.dim, qd, TMP);
        for (int64_t i = 0; i < (int64_t)n * c.dim; i++) X[i] += XB[i];
        for (int32_t t = 0; t < n; t++) orc_rmsnorm(XB + (int64_t)t * c.dim, X + (int64_t)t * c.dim, w->ffn_norm, c.dim, c.eps);
        product(m, HB, w->gate, w->dt_gate, XB, n, c.ffn, c.dim, TMP);
        product(m, HB2, w->up, w->dt_up, XB, n, c.ffn, c.dim, TMP);
        for (int64_t i = 0; i < (int64_t)n * c.ffn; i++) HB[i] = orc_silu(HB[i]) * HB2[i];
        product(m, XB, w->down, w->dt_down, HB, n, c.dim, c.ffn, TMP);
        for (int64_t i = 0; i < (int64_t)n * c.dim; i++) X[i] += XB[i];
    }
    for (int32_t r = 0; r < n_rows; r++) {
        orc_rmsnorm(XB, X + (int64_t)rows[r] * c.dim, m->out_norm, c.dim, c.eps);
        product(m, out + (int64_t)r * c.vocab, m->output, m->dt_out, XB, 1, c.vocab, c.dim, TMP);
    }
    m->len = len + n;
    free(X); free(XB); free(Q); free(K); free(V); free(HEADS); free(HB); free(HB2); free(TMP);
    return ORC_OK;
}

/* The last row's logits only (the next token after the prompt). */
int orc_prefill(orc_model* m, const int32_t* tokens, int32_t n, float* logits) {
    if (n <= 0) return ORC_ERR_ARG;
    const int32_t last = n - 1;
    return orc_prefill_rows(m, tokens, n, &last, 1, logits);
}

/* A new sequence: the cache length returns to 0 ("The Engine", reset). */
void orc_reset(orc_model* m) { m->len = 0; }

int32_t orc_kv_len(const orc_model* m) { return m->len; }

/* Binary16 bits of K and V of one layer at one position, kv_dim values each. */
int orc_kv_read(const orc_model* m, int32_t layer, int32_t pos, uint16_t* k, uint16_t* v) {
    if (layer < 0 || layer >= m->c.n_layers || pos < 0 || pos >= m->c.n_ctx) return ORC_ERR_ARG;
    int32_t kvd = m->c.n_kv_heads * m->c.head_dim;
    size_t base = ((size_t)layer * (size_t)m->c.n_ctx + (size_t)pos) * (size_t)kvd;
    memcpy(k, m->kcache + base, (size_t)kvd * 2);
    memcpy(v, m->vcache + base, (size_t)kvd * 2);
    return ORC_OK;
}

/* Binary16 bits of K and V written to one layer at one position (kv_dim
 * values each): a cache filled from outside, for timing decode steps at a
 * given cache length without running the prompt first. */
int orc_kv_write(orc_model* m, int32_t layer, int32_t pos, const uint16_t* k, const uint16_t* v) {
    if (layer < 0 || layer >= m->c.n_layers || pos < 0 || pos >= m->c.n_ctx) return ORC_ERR_ARG;
    int32_t kvd = m->c.n_kv_heads * m->c.head_dim;
    size_t base = ((size_t)layer * (size_t)m->c.n_ctx + (size_t)pos) * (size_t)kvd;
    memcpy(m->kcache + base, k, (size_t)kvd * 2);
    memcpy(m->vcache + base, v, (size_t)kvd * 2);
    return ORC_OK;
}

/* Declares cache rows 0..len-1 valid (0 <= len <= n_ctx). */
int orc_set_len(orc_model* m, int32_t len) {
    if (len < 0 || len > m->c.n_ctx) return ORC_ERR_ARG;
    m->len = len;
    return ORC_OK;
}

/* Threads of the OpenMP loops (the results do not depend on it). */
void orc_set_threads(int32_t n) {
    if (n > 0) omp_set_num_threads(n);
}
int32_t orc_max_threads(void) { return omp_get_max_threads(); }

/* Size of one layer in weights ("The Forward Pass in Java", Example 1):
 * 2 d^2 + 2 d kv_dim + 3 d ffn + 2 d (biases not counted). */
int64_t orc_weights_per_layer(int64_t dim, int64_t kv_dim, int64_t ffn) {
    return 2 * dim * dim + 2 * dim * kv_dim + 3 * dim * ffn + 2 * dim;
}
