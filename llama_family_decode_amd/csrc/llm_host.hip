// Host runtime of libllm: the C ABI of include/llm.h, tensor-set validation,
// the weight packer, the KV-cache arenas and the per-token launch graph.
#include "llm.h"
#include "llm_ops.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"

using namespace llm;

namespace {

thread_local std::string g_load_error;

// 256-byte aligned sub-allocation of an arena; with a null base it only measures.
struct Arena {
    char* base = nullptr;
    size_t off = 0;
    void* take(size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return base ? base + o : (void*)(uintptr_t)(o + 1);  // non-null placeholder when measuring
    }
};

size_t mat_bytes_w(int dtype, int64_t rows, int64_t cols) {
    return dtype == DT_F32 ? (size_t)(rows * cols * 4) : dtype == DT_F16 ? (size_t)(rows * cols * 2) : (size_t)(rows * cols);
}
size_t mat_bytes_s(int dtype, int64_t rows, int64_t cols) { return dtype == DT_Q8 ? (size_t)(rows * (cols / 32) * 2) : 0; }

int64_t src_bytes(int dtype, int64_t n) { return dtype == DT_F32 ? 4 * n : dtype == DT_F16 ? 2 * n : n / 32 * 34; }

struct TensorRef {
    const llm_tensor* t = nullptr;
};

struct Validated {
    const llm_tensor* embd;
    const llm_tensor* out;  // null when tied
    const llm_tensor* out_norm;
    const llm_tensor* rope_freqs;  // optional per-pair RoPE divisors
    struct L {
        const llm_tensor *attn_norm, *q, *k, *v, *bq, *bk, *bv, *o, *ffn_norm, *gate, *up, *down;
    };
    std::vector<L> layers;
    bool bias;
};

const llm_tensor* find(const llm_tensor* ts, int32_t n, const char* name) {
    for (int32_t i = 0; i < n; i++)
        if (ts[i].name && strcmp(ts[i].name, name) == 0) return &ts[i];
    return nullptr;
}

int check_tensor(const llm_tensor* t, const char* name, int64_t ne0, int64_t ne1, bool matrix, std::string& err) {
    char buf[256];
    if (!t) {
        snprintf(buf, sizeof buf, "missing tensor %s", name);
        err = buf;
        return LLM_ERR_MISSING;
    }
    const int dims = ne1 > 0 ? 2 : 1;
    if (t->n_dims != dims || t->ne[0] != ne0 || (dims == 2 && t->ne[1] != ne1)) {
        snprintf(buf, sizeof buf, "tensor %s has dims [%lld, %lld] (n_dims %d); expected [%lld, %lld]", name,
                 (long long)t->ne[0], (long long)t->ne[1], t->n_dims, (long long)ne0, (long long)(dims == 2 ? ne1 : 1));
        err = buf;
        return LLM_ERR_SHAPE;
    }
    if (matrix) {
        if (t->dtype != DT_F32 && t->dtype != DT_F16 && t->dtype != DT_Q8) {
            snprintf(buf, sizeof buf, "tensor %s has unsupported type %d", name, t->dtype);
            err = buf;
            return LLM_ERR_DTYPE;
        }
    } else if (t->dtype != DT_F32) {
        snprintf(buf, sizeof buf, "tensor %s must be F32 (type %d given)", name, t->dtype);
        err = buf;
        return LLM_ERR_DTYPE;
    }
    const int64_t n = ne0 * (dims == 2 ? ne1 : 1);
    if (!t->data || (int64_t)t->nbytes < src_bytes(t->dtype, n)) {
        snprintf(buf, sizeof buf, "tensor %s: %zu bytes given, %lld needed", name, t->nbytes,
                 (long long)src_bytes(t->dtype, n));
        err = buf;
        return LLM_ERR_SIZE;
    }
    return LLM_OK;
}

SpanCfg span_cfg(const llm_config& c) { return SpanCfg{c.attn_window, c.attn_sinks, c.attn_temp_scale, c.attn_temp_len}; }

int validate(const llm_config* c, const llm_tensor* ts, int32_t n, Validated& V, std::string& err) {
    if (!c || (!ts && n > 0) || n < 0) {
        err = "null config or tensor list";
        return LLM_ERR_ARG;
    }
    if (c->dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->ffn <= 0 ||
        c->vocab <= 0 || c->n_ctx <= 0 || c->rope_dims <= 0 || c->rope_dims > c->head_dim || (c->rope_dims & 1) ||
        c->n_heads % c->n_kv_heads || !(c->eps >= 0.0f) || !(c->rope_base > 0.0f) ||
        (c->rope_neox != 0 && c->rope_neox != 1)) {
        err = "invalid config";
        return LLM_ERR_ARG;
    }
    if (c->attn_window < 0 || c->attn_sinks < 0 || (c->attn_sinks > 0 && c->attn_window == 0) ||
        !(c->attn_temp_scale >= 0.0f && c->attn_temp_scale < INFINITY) ||
        (c->attn_temp_scale > 0.0f && c->attn_temp_len <= 0)) {
        err = "invalid attention span or temperature";
        return LLM_ERR_ARG;
    }
    if (c->numerics != 0 && c->numerics != 1) {
        err = "numerics must be 0 or 1";
        return LLM_ERR_ARG;
    }
    if (!(c->yarn_factor == 0.0f ||
          (c->yarn_factor >= 1.0f && c->yarn_factor < INFINITY && c->yarn_orig_ctx > 0 && c->yarn_beta_slow >= 0.0f &&
           c->yarn_beta_fast > c->yarn_beta_slow && c->yarn_beta_fast < INFINITY))) {
        err = "invalid YaRN parameters";
        return LLM_ERR_ARG;
    }
    const int G = c->n_heads / c->n_kv_heads;
    const int64_t qd = (int64_t)c->n_heads * c->head_dim, kvd = (int64_t)c->n_kv_heads * c->head_dim;
    if (c->head_dim % 8 || c->head_dim > kMaxHeadDim || !(G == 1 || G == 2 || G == 4 || G == 8) || c->dim % 32 ||
        c->dim > kMaxCols || qd % 32 || qd > kMaxCols || c->ffn % 32 || c->ffn > kMaxCols || c->n_ctx > (1 << 20) ||
        (int64_t)c->vocab * c->dim > ((int64_t)1 << 40)) {
        err = "config beyond the supported limits (widths multiple of 32 and <= 16384, head_dim multiple of 8 and <= 256, "
              "group size 1/2/4/8, n_ctx <= 2^20)";
        return LLM_ERR_LIMIT;
    }
    int rc;
    V.embd = find(ts, n, "token_embd.weight");
    if ((rc = check_tensor(V.embd, "token_embd.weight", c->dim, c->vocab, true, err))) return rc;
    V.out_norm = find(ts, n, "output_norm.weight");
    if ((rc = check_tensor(V.out_norm, "output_norm.weight", c->dim, 0, false, err))) return rc;
    V.out = find(ts, n, "output.weight");
    if (V.out && (rc = check_tensor(V.out, "output.weight", c->dim, c->vocab, true, err))) return rc;
    V.rope_freqs = find(ts, n, "rope_freqs.weight");
    if (V.rope_freqs && (rc = check_tensor(V.rope_freqs, "rope_freqs.weight", c->rope_dims / 2, 0, false, err)))
        return rc;
    V.layers.resize(c->n_layers);
    char nm[128];
    int n_bias = 0;
    for (int l = 0; l < c->n_layers; l++) {
        Validated::L& L = V.layers[l];
#define GET(field, suffix, a, b, mat)                                       \
    snprintf(nm, sizeof nm, "blk.%d.%s", l, suffix);                        \
    L.field = find(ts, n, nm);                                              \
    if ((rc = check_tensor(L.field, nm, a, b, mat, err))) return rc;
        GET(attn_norm, "attn_norm.weight", c->dim, 0, false)
        GET(q, "attn_q.weight", c->dim, qd, true)
        GET(k, "attn_k.weight", c->dim, kvd, true)
        GET(v, "attn_v.weight", c->dim, kvd, true)
        GET(o, "attn_output.weight", qd, c->dim, true)
        GET(ffn_norm, "ffn_norm.weight", c->dim, 0, false)
        GET(gate, "ffn_gate.weight", c->dim, c->ffn, true)
        GET(up, "ffn_up.weight", c->dim, c->ffn, true)
        GET(down, "ffn_down.weight", c->ffn, c->dim, true)
#undef GET
        snprintf(nm, sizeof nm, "blk.%d.attn_q.bias", l);
        L.bq = find(ts, n, nm);
        snprintf(nm, sizeof nm, "blk.%d.attn_k.bias", l);
        L.bk = find(ts, n, nm);
        snprintf(nm, sizeof nm, "blk.%d.attn_v.bias", l);
        L.bv = find(ts, n, nm);
        const int nb = (L.bq != nullptr) + (L.bk != nullptr) + (L.bv != nullptr);
        if (nb != 0 && nb != 3) {
            snprintf(nm, sizeof nm, "layer %d has only some of the q/k/v biases", l);
            err = nm;
            return LLM_ERR_MISSING;
        }
        if (nb) {
            if ((rc = check_tensor(L.bq, "attn_q.bias", qd, 0, false, err))) return rc;
            if ((rc = check_tensor(L.bk, "attn_k.bias", kvd, 0, false, err))) return rc;
            if ((rc = check_tensor(L.bv, "attn_v.bias", kvd, 0, false, err))) return rc;
        }
        n_bias += nb ? 1 : 0;
        if (L.q->dtype != L.k->dtype || L.q->dtype != L.v->dtype) {
            snprintf(nm, sizeof nm, "layer %d: attn_q, attn_k and attn_v must share one type", l);
            err = nm;
            return LLM_ERR_DTYPE;
        }
        if (L.gate->dtype != L.up->dtype) {
            snprintf(nm, sizeof nm, "layer %d: ffn_gate and ffn_up must share one type", l);
            err = nm;
            return LLM_ERR_DTYPE;
        }
    }
    if (n_bias != 0 && n_bias != c->n_layers) {
        err = "q/k/v biases must be present in every layer or in none";
        return LLM_ERR_MISSING;
    }
    V.bias = n_bias > 0;
    return LLM_OK;
}

// Everything a context places in its three arenas.
struct Layout {
    // weights
    Mat embd, out;
    const float* out_norm;
    std::vector<LayerW> layers;
    // kv
    __half *kc, *vc;
    size_t kv_layer;  // elements per layer of one cache
    // scratch
    State* st;
    float2* rope;
    const float* rope_freqs;  // device copy of rope_freqs.weight or nullptr
    float *x, *q, *ao, *u, *logits, *attn_part;
    int *gen_out, *ptok;
    LayerW* dlayers;  // device copy of the layer table (persistent step kernel)
    // per-layer activations of the persistent step kernel (strides padded to 256 bytes)
    float *sqkv, *spart, *spst, *spo, *spd, *su;
    long long qkv_stride, part_stride, u_stride, pstride, pst_stride;
    unsigned long long* sbar;
    unsigned long long* strace;
    float *X, *Hf, *QKV, *Q, *Of, *Uf, *ws;
    __half *Hh, *Hl, *Oh, *Ol, *Uh, *Ul;  // binary16 hi/lo planes of Hf, Of, Uf
    int8_t* Ci;                           // rounding mode: Q8_0 codes of a product's input rows (tiled int8)
    float* Cs;                            // and their block scales (fp32), or nullptr
    float* Xc;                            // the wanted rows' residuals (last prefill layer)
    float* attn_stats;                    // span max and sum per (row, head) of the rounded passes
    int* xcd;                             // the XCD of each step-kernel block (load-time check)
    int* sel;                             // prompt rows whose logits are wanted (chunk-relative)
    int* selo;                            // and their output rows
    size_t ws_floats;
    int n_split;
    size_t wbytes, kvbytes, sbytes;
};

Mat place_mat(Arena& A, int dtype, int rows, int cols) {
    Mat m;
    m.dtype = dtype;
    m.rows = rows;
    m.cols = cols;
    m.w = A.take(mat_bytes_w(dtype, rows, cols));
    m.s = dtype == DT_Q8 ? (const uint16_t*)A.take(mat_bytes_s(dtype, rows, cols)) : nullptr;
    m.wt = nullptr;
    m.st = nullptr;
    m.wi = nullptr;
    m.si = nullptr;
    return m;
}

// Layer matrices in F16 also get the tiled copy the prefill products read.
// Q8_0 ones get binary16 codes (exact) plus their block scales per K step, or
// under llama.cpp's rounding points (numerics 1), whose products are integer,
// the tiled int8 codes plus their scales as fp32.
void place_tiled(Arena& A, Mat& m, int numerics) {
    if (m.cols % 32) return;
    if (m.dtype == DT_F16) {
        m.wt = A.take(tiled_w_bytes(m.rows, m.cols));
    } else if (m.dtype == DT_Q8 && !numerics) {
        m.wt = A.take(tiled_w_bytes(m.rows, m.cols));
        m.st = A.take(tiled_s_bytes(m.rows, m.cols));
    } else if (m.dtype == DT_Q8) {
        m.wi = A.take(tiled_i8_bytes(m.rows, m.cols));
        m.si = (const float*)A.take(tiled_sf_bytes(m.rows, m.cols));
    }
}

int decode_splits(const llm_config* c) {
    int s = 512 / c->n_kv_heads;
    if (s < 1) s = 1;
    if (s > 256) s = 256;
    return s;
}

void make_layout(const llm_config* c, const Validated& V, void* wb, void* kb, void* sb, Layout& L) {
    const int qd = c->n_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
    Arena W;
    W.base = (char*)wb;
    L.embd = place_mat(W, V.embd->dtype, c->vocab, c->dim);
    L.out_norm = (const float*)W.take((size_t)c->dim * 4);
    L.out = V.out ? place_mat(W, V.out->dtype, c->vocab, c->dim) : L.embd;
    place_tiled(W, L.out, c->numerics);  // for the batched vocabulary product of chosen prompt rows
    L.rope_freqs = V.rope_freqs ? (const float*)W.take((size_t)(c->rope_dims / 2) * 4) : nullptr;
    L.layers.resize(c->n_layers);
    for (int l = 0; l < c->n_layers; l++) {
        const Validated::L& S = V.layers[l];
        LayerW& D = L.layers[l];
        D.attn_norm = (const float*)W.take((size_t)c->dim * 4);
        D.qkv = place_mat(W, S.q->dtype, qd + 2 * kvd, c->dim);
        D.bqkv = V.bias ? (const float*)W.take((size_t)(qd + 2 * kvd) * 4) : nullptr;
        D.o = place_mat(W, S.o->dtype, c->dim, qd);
        D.ffn_norm = (const float*)W.take((size_t)c->dim * 4);
        D.gu = place_mat(W, S.gate->dtype, 2 * c->ffn, c->dim);
        D.down = place_mat(W, S.down->dtype, c->dim, c->ffn);
        place_tiled(W, D.qkv, c->numerics);
        place_tiled(W, D.o, c->numerics);
        place_tiled(W, D.gu, c->numerics);
        place_tiled(W, D.down, c->numerics);
    }
    L.wbytes = W.off;

    Arena K;
    K.base = (char*)kb;
    L.kv_layer = (size_t)c->n_kv_heads * c->n_ctx * c->head_dim;
    L.kc = (__half*)K.take(L.kv_layer * c->n_layers * 2);
    L.vc = (__half*)K.take(L.kv_layer * c->n_layers * 2);
    L.kvbytes = K.off;

    Arena S;
    S.base = (char*)sb;
    const int G = c->n_heads / c->n_kv_heads;
    // rows of one prefill batch; the matrix-core products keep their binary16
    // activation planes in whole tiles of kTileA rows
    const int C = kPrefillChunk;
    static_assert(kPrefillChunk % kTileA == 0, "prefill batches hold whole activation tiles");
    L.n_split = decode_splits(c);
    L.st = (State*)S.take(sizeof(State));
    L.rope = (float2*)S.take((size_t)c->n_ctx * (c->rope_dims / 2) * sizeof(float2));
    L.x = (float*)S.take((size_t)c->dim * 4);
    L.q = (float*)S.take((size_t)qd * 4);
    L.ao = (float*)S.take((size_t)qd * 4);
    L.u = (float*)S.take((size_t)c->ffn * 4);
    L.logits = (float*)S.take((size_t)c->vocab * 4);
    // split partials: kMaxSplit splits of one decode query, or one split per
    // prefill row (the rounded-probability passes write them for every row)
    L.attn_part = (float*)S.take((size_t)(kMaxSplit > C ? kMaxSplit : C) * c->n_kv_heads * G * (c->head_dim + 2) * 4);
    L.attn_stats = (float*)S.take((size_t)C * c->n_heads * 2 * 4);
    L.dlayers = (LayerW*)S.take((size_t)c->n_layers * sizeof(LayerW));
    auto pad64 = [](long long n) { return (n + 63) / 64 * 64; };
    L.qkv_stride = pad64(qd + 2 * kvd);
    L.part_stride = pad64((long long)kStepMaxSplit * c->n_kv_heads * G * (c->head_dim + 2));
    L.pst_stride = pad64((long long)kStepMaxSplit * c->n_kv_heads * G * 2);
    L.u_stride = pad64(c->ffn);
    L.pstride = pad64(c->dim);
    L.sqkv = (float*)S.take((size_t)c->n_layers * L.qkv_stride * 4);
    L.spart = (float*)S.take((size_t)c->n_layers * L.part_stride * 4);
    L.spst = (float*)S.take((size_t)c->n_layers * L.pst_stride * 4);
    L.spo = (float*)S.take((size_t)c->n_layers * kStepGroups * L.pstride * 4);
    L.spd = (float*)S.take((size_t)c->n_layers * kStepGroups * L.pstride * 4);
    L.su = (float*)S.take((size_t)c->n_layers * L.u_stride * 4);
    L.sbar = (unsigned long long*)S.take((size_t)kBarSlots * kBarStride * 8);
    L.strace = (unsigned long long*)S.take((size_t)(kStepPhases * c->n_layers + 2) * 8);
    L.gen_out = (int*)S.take((size_t)c->n_ctx * 4);
    L.xcd = (int*)S.take((size_t)kMaxStepGrid * 4);
    L.ptok = (int*)S.take((size_t)C * 4);
    L.X = (float*)S.take((size_t)C * c->dim * 4);
    L.Hf = (float*)S.take((size_t)C * c->dim * 4);
    L.QKV = (float*)S.take((size_t)C * (qd + 2 * kvd) * 4);
    L.Q = (float*)S.take((size_t)C * qd * 4);
    L.Of = (float*)S.take((size_t)C * qd * 4);
    L.Uf = (float*)S.take((size_t)C * c->ffn * 4);
    L.Hh = (__half*)S.take((size_t)C * c->dim * 2);
    L.Hl = (__half*)S.take((size_t)C * c->dim * 2);
    L.Oh = (__half*)S.take((size_t)C * qd * 2);
    L.Ol = (__half*)S.take((size_t)C * qd * 2);
    L.Uh = (__half*)S.take((size_t)C * c->ffn * 2);
    L.Xc = (float*)S.take((size_t)C * c->dim * 4);
    L.sel = (int*)S.take((size_t)c->n_ctx * 4);
    L.selo = (int*)S.take((size_t)c->n_ctx * 4);
    L.Ul = (__half*)S.take((size_t)C * c->ffn * 2);
    // the rounding mode's Q8_0 codes and scales of one product's input rows
    // (the widest input: dim, q or ffn columns)
    L.Ci = nullptr;
    L.Cs = nullptr;
    if (c->numerics) {
        int kmax = c->dim > qd ? c->dim : qd;
        if (c->ffn > kmax) kmax = c->ffn;
        L.Ci = (int8_t*)S.take((size_t)C * kmax);
        L.Cs = (float*)S.take((size_t)C * (kmax / 32) * 4);
    }
    // split-K partials (up to 8 splits) of the prefill products with at most
    // max(q|k|v, dim) rows
    L.ws_floats = (size_t)8 * C * (qd + 2 * kvd > c->dim ? qd + 2 * kvd : c->dim);
    L.ws = (float*)S.take(L.ws_floats * 4);
    L.sbytes = S.off;
}

// Host-side packing of one source matrix into (part of) a device-layout matrix:
// source row r becomes packed row row0 + r * rstride.
void pack_rows(const llm_tensor* t, int rows, int cols, int row0, int rstride, std::vector<uint8_t>& w,
               std::vector<uint16_t>& s) {
    const uint8_t* src = (const uint8_t*)t->data;
    if (t->dtype == DT_F32 || t->dtype == DT_F16) {
        const size_t rb = (size_t)cols * (t->dtype == DT_F32 ? 4 : 2);
        for (int r = 0; r < rows; r++) memcpy(w.data() + (size_t)(row0 + r * rstride) * rb, src + (size_t)r * rb, rb);
    } else {
        const int nb = cols / 32;
        for (int r = 0; r < rows; r++) {
            const size_t pr = (size_t)(row0 + r * rstride);
            for (int b = 0; b < nb; b++) {
                const uint8_t* blk = src + ((size_t)r * nb + b) * 34;
                s[pr * nb + b] = (uint16_t)(blk[0] | (blk[1] << 8));
                memcpy(w.data() + pr * cols + (size_t)b * 32, blk + 2, 32);
            }
        }
    }
}

}  // namespace

struct llm_ctx {
    llm_config cfg;
    int qd, kvd, G;
    hipStream_t stream;
    hipStream_t cap = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t gexec = nullptr;
    bool use_graph = true;
    void *wbase = nullptr, *kvbase = nullptr, *sbase = nullptr;
    bool own_w = false, own_kv = false, own_s = false;
    Layout L;
    int32_t len = 0;
    bool poisoned = false;
    int device = -1;  // the device current at load
    std::string err;
    int g_qkv, g_o, g_gu, g_down, g_vocab;
    bool use_step = false;  // persistent step kernel (else the launch graph)
    int step_grid = 0, step_lds = 0;
    const void* step_fn = nullptr;
    bool step_special = false;  // a step kernel compiled for this shape
    StepArgs step;
    std::vector<int32_t> sel_out, sel_row;  // wanted prefill rows (host copies stay alive for the async upload)
};

namespace {

int fail(llm_ctx* c, int rc, const std::string& msg) {
    if (c) c->err = msg;
    return rc;
}

int dev_fail(llm_ctx* c, hipError_t e, const char* what) {
    c->poisoned = true;
    c->err = std::string(what) + ": " + hipGetErrorString(e);
    return LLM_ERR_DEVICE;
}

#define HIPCHK(ctx, expr)                                   \
    do {                                                    \
        hipError_t e_ = (expr);                             \
        if (e_ != hipSuccess) return dev_fail(ctx, e_, #expr); \
    } while (0)

GemvArgs base_args(llm_ctx* c) {
    GemvArgs a;
    memset(&a, 0, sizeof a);
    a.eps = c->cfg.eps;
    a.st = c->L.st;
    a.n_heads = c->cfg.n_heads;
    a.n_kv_heads = c->cfg.n_kv_heads;
    a.head_dim = c->cfg.head_dim;
    a.n_rot = c->cfg.rope_dims;
    a.neox = c->cfg.rope_neox;
    a.n_ctx = c->cfg.n_ctx;
    a.rope = c->L.rope;
    a.rnd = c->cfg.numerics;
    return a;
}

// Vocabulary product + argmax over residual row `xin` (decode: L.x; prefill: last row of X).
hipError_t enqueue_logits(llm_ctx* c, const float* xin, hipStream_t s) {
    GemvArgs a = base_args(c);
    a.W = c->L.out;
    a.xin = xin;
    a.gain = c->L.out_norm;
    a.y = c->L.logits;
    a.gen_out = c->L.gen_out;
    a.gen_cap = c->cfg.n_ctx;
    hipError_t e = launch_gemv(PRO_NORM, EPI_ARGMAX, a, c->g_vocab, s);
    if (e != hipSuccess) return e;
    return launch_argmax_finalize(c->L.st, c->L.gen_out, c->cfg.n_ctx, s);
}

// The five stages of one layer of the decode step.
hipError_t stage_qkv(llm_ctx* c, int l, const float* xin, bool embed, float* q, hipStream_t s) {
    const Layout& L = c->L;
    const LayerW& W = L.layers[l];
    GemvArgs a = base_args(c);
    a.W = W.qkv;
    a.gain = W.attn_norm;
    a.y = q;
    a.bias = W.bqkv;
    a.kc = L.kc + (size_t)l * L.kv_layer;
    a.vc = L.vc + (size_t)l * L.kv_layer;
    if (embed) {
        a.E = L.embd;
        a.xres = L.x;
        return launch_gemv(PRO_EMBED, EPI_QKV, a, c->g_qkv, s);
    }
    a.xin = xin;
    return launch_gemv(PRO_NORM, EPI_QKV, a, c->g_qkv, s);
}

hipError_t stage_attn(llm_ctx* c, int l, const float* q, float* out, hipStream_t s) {
    const Layout& L = c->L;
    const llm_config& cf = c->cfg;
    AttnArgs t;
    memset(&t, 0, sizeof t);
    t.q = q;
    t.kc = L.kc + (size_t)l * L.kv_layer;
    t.vc = L.vc + (size_t)l * L.kv_layer;
    t.out = out;
    t.part = L.attn_part;
    t.st = L.st;
    t.n_heads = cf.n_heads;
    t.n_kv_heads = cf.n_kv_heads;
    t.head_dim = cf.head_dim;
    t.n_ctx = cf.n_ctx;
    t.n_split = L.n_split;
    t.scale_div = (float)sqrt((double)cf.head_dim);
    t.span = span_cfg(cf);
    t.rnd = cf.numerics;
    t.stats = L.attn_stats;
    return launch_attn(t, 1, s);
}

hipError_t stage_o(llm_ctx* c, int l, const float* in, float* x, hipStream_t s) {
    GemvArgs o = base_args(c);
    o.W = c->L.layers[l].o;
    o.xin = in;
    o.y = x;
    return launch_gemv(PRO_PLAIN, EPI_RESID, o, c->g_o, s);
}

hipError_t stage_ffn_up(llm_ctx* c, int l, const float* x, float* u, hipStream_t s) {
    GemvArgs g = base_args(c);
    g.W = c->L.layers[l].gu;
    g.xin = x;
    g.gain = c->L.layers[l].ffn_norm;
    g.y = u;
    return launch_gemv(PRO_NORM, EPI_SWIGLU, g, c->g_gu, s);
}

hipError_t stage_down(llm_ctx* c, int l, const float* u, float* x, hipStream_t s) {
    GemvArgs d = base_args(c);
    d.W = c->L.layers[l].down;
    d.xin = u;
    d.y = x;
    return launch_gemv(PRO_PLAIN, EPI_RESID, d, c->g_down, s);
}

// One decode step: 5 launches per layer + the logits launch. Token and position
// come from the device State.
hipError_t enqueue_step(llm_ctx* c, hipStream_t s) {
    const Layout& L = c->L;
    hipError_t e;
    for (int l = 0; l < c->cfg.n_layers; l++) {
        if ((e = stage_qkv(c, l, L.x, l == 0, L.q, s)) != hipSuccess) return e;
        if ((e = stage_attn(c, l, L.q, L.ao, s)) != hipSuccess) return e;
        if ((e = stage_o(c, l, L.ao, L.x, s)) != hipSuccess) return e;
        if ((e = stage_ffn_up(c, l, L.x, L.u, s)) != hipSuccess) return e;
        if ((e = stage_down(c, l, L.u, L.x, s)) != hipSuccess) return e;
    }
    return enqueue_logits(c, L.x, s);
}

int run_step(llm_ctx* c) {
    if (c->use_step) {
        HIPCHK(c, launch_step(c->step, c->step_fn, c->step_grid, c->step_lds, c->stream));
        return LLM_OK;
    }
    if (c->use_graph) {
        if (!c->gexec) {
            HIPCHK(c, hipStreamBeginCapture(c->cap, hipStreamCaptureModeRelaxed));
            hipError_t e = enqueue_step(c, c->cap);
            hipGraph_t g = nullptr;
            hipError_t e2 = hipStreamEndCapture(c->cap, &g);
            if (e != hipSuccess) return dev_fail(c, e, "enqueue_step (capture)");
            if (e2 != hipSuccess) return dev_fail(c, e2, "hipStreamEndCapture");
            c->graph = g;
            HIPCHK(c, hipGraphInstantiate(&c->gexec, c->graph, nullptr, nullptr, 0));
        }
        HIPCHK(c, hipGraphLaunch(c->gexec, c->stream));
    } else {
        hipError_t e = enqueue_step(c, c->stream);
        if (e != hipSuccess) return dev_fail(c, e, "enqueue_step");
    }
    return LLM_OK;
}

int finish(llm_ctx* c, float* d_logits, int32_t* h_next) {
    if (d_logits)
        HIPCHK(c, hipMemcpyAsync(d_logits, c->L.logits, (size_t)c->cfg.vocab * 4, hipMemcpyDeviceToDevice, c->stream));
    if (h_next) {
        State st;
        HIPCHK(c, hipMemcpyAsync(&st, c->L.st, sizeof st, hipMemcpyDeviceToHost, c->stream));
        HIPCHK(c, hipStreamSynchronize(c->stream));
        *h_next = st.next;
        if (st.abort) {
            c->poisoned = true;
            return fail(c, LLM_ERR_DEVICE, "a grid barrier of the step kernel timed out");
        }
        if (st.nonfinite) return fail(c, LLM_ERR_NONFINITE, "a logit is NaN or infinite");
    }
    return LLM_OK;
}

int check_ctx(const llm_ctx* c) {
    if (!c) return LLM_ERR_ARG;
    if (c->poisoned) return LLM_ERR_DEVICE;
    return LLM_OK;
}

void release(llm_ctx* c) {
    if (!c) return;
    if (c->gexec) (void)hipGraphExecDestroy(c->gexec);
    if (c->graph) (void)hipGraphDestroy(c->graph);
    if (c->cap) (void)hipStreamDestroy(c->cap);
    if (c->own_w && c->wbase) (void)hipFree(c->wbase);
    if (c->own_kv && c->kvbase) (void)hipFree(c->kvbase);
    if (c->own_s && c->sbase) (void)hipFree(c->sbase);
    delete c;
}

}  // namespace

extern "C" {

int llm_plan(const llm_config* cfg, const llm_tensor* tensors, int32_t n, size_t* weight_bytes, size_t* kv_bytes,
             size_t* scratch_bytes) {
    Validated V;
    std::string err;
    int rc = validate(cfg, tensors, n, V, err);
    if (rc) {
        g_load_error = err;
        return rc;
    }
    Layout L;
    make_layout(cfg, V, nullptr, nullptr, nullptr, L);
    if (weight_bytes) *weight_bytes = L.wbytes;
    if (kv_bytes) *kv_bytes = L.kvbytes;
    if (scratch_bytes) *scratch_bytes = L.sbytes;
    return LLM_OK;
}

int llm_load_weights(const llm_config* cfg, const llm_tensor* tensors, int32_t n, void* d_weights, void* d_kv,
                     void* d_scratch, void* hip_stream, llm_ctx** out) {
    if (!out) return LLM_ERR_ARG;
    *out = nullptr;
    Validated V;
    std::string err;
    int rc = validate(cfg, tensors, n, V, err);
    if (rc) {
        g_load_error = err;
        return rc;
    }
    if (V.rope_freqs) {  // values are read only here (llm_plan may see placeholder data)
        const float* f = (const float*)V.rope_freqs->data;
        for (int i = 0; i < cfg->rope_dims / 2; i++)
            if (!(f[i] > 0.f) || !isfinite(f[i])) {
                g_load_error = "rope_freqs.weight must hold finite positive divisors";
                return LLM_ERR_ARG;
            }
    }
    Layout M;
    make_layout(cfg, V, nullptr, nullptr, nullptr, M);
    llm_ctx* c = new llm_ctx();
    c->cfg = *cfg;
    c->qd = cfg->n_heads * cfg->head_dim;
    c->kvd = cfg->n_kv_heads * cfg->head_dim;
    c->G = cfg->n_heads / cfg->n_kv_heads;
    c->stream = (hipStream_t)hip_stream;
    if (hipGetDevice(&c->device) != hipSuccess) {
        release(c);
        g_load_error = "hipGetDevice failed";
        return LLM_ERR_DEVICE;
    }
    const char* ng = getenv("LLM_NO_GRAPH");
    c->use_graph = !(ng && ng[0] == '1');
    auto bail = [&](int code, const std::string& msg) {
        g_load_error = msg;
        release(c);
        return code;
    };
    auto alloc = [&](void* given, size_t bytes, void** dst, bool* own) -> bool {
        if (given) {
            if ((uintptr_t)given & 255) return false;
            *dst = given;
            return true;
        }
        if (hipMalloc(dst, bytes ? bytes : 256) != hipSuccess) {
            *dst = nullptr;
            return false;
        }
        *own = true;
        return true;
    };
    if (!alloc(d_weights, M.wbytes, &c->wbase, &c->own_w) || !alloc(d_kv, M.kvbytes, &c->kvbase, &c->own_kv) ||
        !alloc(d_scratch, M.sbytes, &c->sbase, &c->own_s))
        return bail(LLM_ERR_OOM, "device arena allocation failed (or a given arena is not 256-byte aligned)");
    make_layout(cfg, V, c->wbase, c->kvbase, c->sbase, c->L);
    Layout& L = c->L;
    hipStream_t s = c->stream;
    const int qd = c->qd, kvd = c->kvd;

    // ---- pack and upload the weights
    auto upload = [&](const void* dst, const void* src, size_t bytes) -> bool {
        return hipMemcpyAsync((void*)dst, src, bytes, hipMemcpyHostToDevice, s) == hipSuccess &&
               hipStreamSynchronize(s) == hipSuccess;
    };
    auto upload_mat = [&](const Mat& m, std::initializer_list<const llm_tensor*> parts, int mode) -> bool {
        // mode 0: one tensor; 1: row concatenation; 2: row interleave
        std::vector<uint8_t> w(mat_bytes_w(m.dtype, m.rows, m.cols));
        std::vector<uint16_t> sc(m.dtype == DT_Q8 ? (size_t)m.rows * (m.cols / 32) : 0);
        int row0 = 0, idx = 0;
        const int np = (int)parts.size();
        for (const llm_tensor* t : parts) {
            const int rows = (int)t->ne[1];
            if (mode == 2)
                pack_rows(t, rows, m.cols, idx, np, w, sc);
            else
                pack_rows(t, rows, m.cols, row0, 1, w, sc);
            row0 += rows;
            idx++;
        }
        if (!upload(m.w, w.data(), w.size())) return false;
        if (m.dtype == DT_Q8 && !upload(m.s, sc.data(), sc.size() * 2)) return false;
        return true;
    };
    bool ok = upload_mat(L.embd, {V.embd}, 0) && upload(L.out_norm, V.out_norm->data, (size_t)cfg->dim * 4);
    if (ok && V.rope_freqs) ok = upload(L.rope_freqs, V.rope_freqs->data, (size_t)(cfg->rope_dims / 2) * 4);
    if (ok && V.out) ok = upload_mat(L.out, {V.out}, 0);
    for (int l = 0; ok && l < cfg->n_layers; l++) {
        const Validated::L& S = V.layers[l];
        LayerW& D = L.layers[l];
        ok = upload(D.attn_norm, S.attn_norm->data, (size_t)cfg->dim * 4) && upload_mat(D.qkv, {S.q, S.k, S.v}, 1) &&
             upload(D.ffn_norm, S.ffn_norm->data, (size_t)cfg->dim * 4) && upload_mat(D.o, {S.o}, 0) &&
             upload_mat(D.gu, {S.gate, S.up}, 2) && upload_mat(D.down, {S.down}, 0);
        if (ok && V.bias) {
            std::vector<float> b((size_t)qd + 2 * kvd);
            memcpy(b.data(), S.bq->data, (size_t)qd * 4);
            memcpy(b.data() + qd, S.bk->data, (size_t)kvd * 4);
            memcpy(b.data() + qd + kvd, S.bv->data, (size_t)kvd * 4);
            ok = upload(D.bqkv, b.data(), b.size() * 4);
        }
    }
    for (int l = 0; ok && l < cfg->n_layers; l++) {
        const LayerW& D = L.layers[l];
        for (const Mat* m : {&D.qkv, &D.o, &D.gu, &D.down})
            if (m->wt || m->wi) ok = ok && launch_tile_w(*m, s) == hipSuccess;
    }
    if (ok && (L.out.wt || L.out.wi)) ok = launch_tile_w(L.out, s) == hipSuccess;
    if (!ok) return bail(LLM_ERR_DEVICE, "weight upload failed");

    // ---- RoPE table and zeroed state
    const YarnCfg yarn{cfg->yarn_factor, cfg->yarn_orig_ctx, cfg->yarn_beta_fast, cfg->yarn_beta_slow};
    if (launch_rope_table(L.rope, cfg->n_ctx, cfg->rope_dims, cfg->rope_base, L.rope_freqs, yarn, s) != hipSuccess ||
        hipMemsetAsync(L.st, 0, sizeof(State), s) != hipSuccess ||
        hipMemsetAsync(L.sbar, 0, (size_t)kBarSlots * kBarStride * 8, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return bail(LLM_ERR_DEVICE, "initialisation kernels failed");

    c->g_qkv = gemv_grid(PRO_NORM, EPI_QKV, qd + 2 * kvd);
    c->g_o = gemv_grid(PRO_PLAIN, EPI_RESID, cfg->dim);
    c->g_gu = gemv_grid(PRO_NORM, EPI_SWIGLU, 2 * cfg->ffn);
    c->g_down = gemv_grid(PRO_PLAIN, EPI_RESID, cfg->dim);
    c->g_vocab = gemv_grid(PRO_NORM, EPI_ARGMAX, cfg->vocab);

    // persistent step kernel
    {
        StepArgs& A = c->step;
        memset(&A, 0, sizeof A);
        A.layers = L.dlayers;
        A.n_layers = cfg->n_layers;
        A.embd = L.embd;
        A.out = L.out;
        A.out_norm = L.out_norm;
        A.kc = L.kc;
        A.vc = L.vc;
        A.kv_layer = (long long)L.kv_layer;
        A.rope = L.rope;
        A.st = L.st;
        A.bar = L.sbar;
        A.qkv = L.sqkv;
        A.part = L.spart;
        A.pst = L.spst;
        A.po = L.spo;
        A.pd = L.spd;
        A.u = L.su;
        A.qkv_stride = L.qkv_stride;
        A.part_stride = L.part_stride;
        A.pst_stride = L.pst_stride;
        A.u_stride = L.u_stride;
        A.pstride = L.pstride;
        A.logits = L.logits;
        const char* tr = getenv("LLM_STEP_TRACE");
        A.trace = (tr && tr[0] == '1') ? L.strace : nullptr;
        A.gen_out = L.gen_out;
        A.gen_cap = cfg->n_ctx;
        A.dim = cfg->dim;
        A.n_heads = cfg->n_heads;
        A.n_kv_heads = cfg->n_kv_heads;
        A.head_dim = cfg->head_dim;
        A.n_rot = cfg->rope_dims;
        A.neox = cfg->rope_neox;
        A.n_ctx = cfg->n_ctx;
        A.ffn = cfg->ffn;
        A.vocab = cfg->vocab;
        A.eps = cfg->eps;
        A.scale_div = (float)sqrt((double)cfg->head_dim);
        A.span = span_cfg(*cfg);
        A.rnd = cfg->numerics;
        if (!upload(L.dlayers, L.layers.data(), L.layers.size() * sizeof(LayerW)))
            return bail(LLM_ERR_DEVICE, "layer table upload failed");
        // The persistent kernel needs one weight type for all layer matrices.
        const int dt = L.layers[0].qkv.dtype;
        bool same = true;
        for (const LayerW& w : L.layers)
            same = same && w.qkv.dtype == dt && w.o.dtype == dt && w.gu.dtype == dt && w.down.dtype == dt;
        const char* sk = getenv("LLM_STEP");
        const bool want = !(sk && strcmp(sk, "graph") == 0);
        c->step_grid = want && same ? step_grid(A, dt, &c->step_lds, &c->step_fn, &c->step_special) : 0;
        // its groups exchange values through their XCD's L2
        if (c->step_grid > kMaxStepGrid || (c->step_grid > 0 && !step_groups_share_l2(c->step_grid, L.xcd, s))) {
            (void)hipGetLastError();
            c->step_grid = 0;
        }
        c->use_step = c->step_grid > 0;
    }

    if (c->use_graph && hipStreamCreateWithFlags(&c->cap, hipStreamNonBlocking) != hipSuccess)
        return bail(LLM_ERR_DEVICE, "stream creation failed");
    // One direct step (token 0 at position 0) sets the kernels' launch attributes
    // before any capture; it only writes cache row 0, which is invalid while len = 0.
    if (launch_set_state(L.st, 0, 0, 0, s) != hipSuccess || enqueue_step(c, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return bail(LLM_ERR_DEVICE, std::string("first step failed: ") + hipGetErrorString(hipGetLastError()));
    if (c->use_step) {
        if (launch_set_state(L.st, 0, 0, 0, s) != hipSuccess ||
            launch_step(c->step, c->step_fn, c->step_grid, c->step_lds, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
            (void)hipGetLastError();
            c->use_step = false;  // the step kernel did not launch: the launch graph runs the steps
        } else {
            State st;
            if (hipMemcpy(&st, L.st, sizeof st, hipMemcpyDeviceToHost) != hipSuccess || st.abort)
                return bail(LLM_ERR_DEVICE, "step kernel failed its first run");
        }
    }
    c->len = 0;
    *out = c;
    return LLM_OK;
}

int llm_decode(llm_ctx* c, int32_t token, int32_t pos, float* d_logits, int32_t* h_next) {
    int rc = check_ctx(c);
    if (rc) return rc;
    if (token < 0 || token >= c->cfg.vocab) return fail(c, LLM_ERR_TOKEN, "token out of range");
    if (pos < 0 || pos > c->len || pos >= c->cfg.n_ctx) return fail(c, LLM_ERR_POS, "position out of range");
    HIPCHK(c, launch_set_state(c->L.st, token, pos, 0, c->stream));
    if ((rc = run_step(c))) return rc;
    c->len = pos + 1;
    return finish(c, d_logits, h_next);
}

int llm_generate(llm_ctx* c, int32_t token, int32_t n_steps, int32_t* h_tokens) {
    int rc = check_ctx(c);
    if (rc) return rc;
    if (n_steps <= 0 || !h_tokens) return fail(c, LLM_ERR_ARG, "n_steps must be positive and h_tokens set");
    if (token < 0 || token >= c->cfg.vocab) return fail(c, LLM_ERR_TOKEN, "token out of range");
    if ((int64_t)c->len + n_steps > c->cfg.n_ctx) return fail(c, LLM_ERR_CTX_FULL, "generation would pass n_ctx");
    HIPCHK(c, launch_set_state(c->L.st, token, c->len, 1, c->stream));
    for (int i = 0; i < n_steps; i++)
        if ((rc = run_step(c))) return rc;
    HIPCHK(c, hipMemcpyAsync(h_tokens, c->L.gen_out, (size_t)n_steps * 4, hipMemcpyDeviceToHost, c->stream));
    State st;
    HIPCHK(c, hipMemcpyAsync(&st, c->L.st, sizeof st, hipMemcpyDeviceToHost, c->stream));
    HIPCHK(c, hipStreamSynchronize(c->stream));
    c->len += n_steps;
    if (st.abort) {
        c->poisoned = true;
        return fail(c, LLM_ERR_DEVICE, "a grid barrier of the step kernel timed out");
    }
    if (st.nonfinite) return fail(c, LLM_ERR_NONFINITE, "a logit is NaN or infinite");
    return LLM_OK;
}

// The batched prompt pass ("What a Llama model computes, and why", section 4)
// over chunks of kPrefillChunk rows. The last layer's output product and FFN
// run only on the rows whose logits are wanted (every row still writes its
// K/V): the chunk's wanted rows are gathered into a compact batch first.
// rows_out: for each wanted row, in output order, its index in the prompt;
// with d_rows the logits of output j go to d_rows[j*vocab] (vocabulary
// product over the compact batch), else exactly one row (the last) is wanted
// and goes through the decode vocabulary kernel and argmax.
// With llama.cpp's rounding points (numerics 1) a Q8_0 product takes its
// rounded inputs as Q8_0 codes and runs on the integer matrix cores (int8
// codes times int8 codes per block).
static bool prefill_codes(const llm_ctx* c, const Mat& w) {
    return c->cfg.numerics && w.dtype == DT_Q8 && w.wi && c->L.Ci;
}
// The operand of a prefill product with input rows f and their hi/lo planes h,
// l. With rounded inputs an F16 product's lo plane is zero: one matrix-core
// pass (a rounded Q8_0 input, f16(d) * code, still needs both planes, unless
// the product runs on its codes).
static GemmA prefill_operand(const llm_ctx* c, const Mat& w, const float* f, const __half* h, const __half* l) {
    const __half* lo = c->cfg.numerics && w.dtype == DT_F16 ? nullptr : l;
    return prefill_codes(c, w) ? GemmA{f, h, lo, c->L.Ci, c->L.Cs} : GemmA{f, h, lo, nullptr, nullptr};
}
// Whether product w reads only its input's binary16 hi/lo planes (the tiled
// matrix-core product in float numerics), so that no kernel needs the input's
// fp32 rows: the rounding mode rounds those rows, and the other product
// kernels read them.
static bool prefill_planes_only(const llm_ctx* c, const Mat& w) {
    return !c->cfg.numerics && w.wt && (w.dtype == DT_F16 || (w.dtype == DT_Q8 && w.st)) && w.cols % 32 == 0;
}

static int prefill_pass(llm_ctx* c, const int32_t* h_tokens, int32_t n, const std::vector<int32_t>& rows_out,
                        float* d_rows) {
    const llm_config& cf = c->cfg;
    Layout& L = c->L;
    hipStream_t s = c->stream;
    const int qd = c->qd, kvd = c->kvd, qkvd = qd + 2 * kvd;
    const int nr = (int)rows_out.size();
    int rc = LLM_OK;
    const bool rnd = cf.numerics != 0;  // llama.cpp's rounding of every product input
    auto ga = [&](const Mat& w, const float* f, const __half* h, const __half* l) {
        return prefill_operand(c, w, f, h, l);
    };
    auto round_rows = [&](float* X, int rows, int K, const Mat& w, __half* H, __half* Lp) {
        return prefill_codes(c, w) ? launch_round_rows(X, rows, K, w.dtype, nullptr, nullptr, s, L.Ci, L.Cs)
                                   : launch_round_rows(X, rows, K, w.dtype, H, Lp, s);
    };
    // RMSNorm of the residual rows X (after adding the S split-K partials of
    // the workspace, if S > 0) as the input of product w: its Q8_0 codes when
    // w runs on them, else the fp32 rows and their hi/lo planes
    auto norm_rows = [&](const float* P, int S, float* X, int rows, const float* gain, const Mat& w) {
        float* Yf = prefill_planes_only(c, w) ? nullptr : L.Hf;
        __half *Yh = L.Hh, *Yl = L.Hl;
        int8_t* C = nullptr;
        float* CS = nullptr;
        if (prefill_codes(c, w)) {
            Yf = nullptr;
            Yh = Yl = nullptr;
            C = L.Ci;
            CS = L.Cs;
        }
        return S ? launch_reduce_norm_rows(P, S, rows, X, cf.dim, gain, cf.eps, Yf, Yh, Yl, s, C, CS)
                 : launch_rmsnorm_rows(X, gain, rows, cf.dim, cf.eps, Yf, Yh, Yl, s, C, CS);
    };
    // the wanted rows grouped by chunk, output order kept within a chunk:
    // c->sel_out[p] = output index, c->sel_row[p] = prompt row
    c->sel_out.clear();
    c->sel_row.clear();
    std::vector<int> chunk_begin;
    for (int done = 0; done < n; done += kPrefillChunk) {
        chunk_begin.push_back((int)c->sel_out.size());
        const int end = done + kPrefillChunk < n ? done + kPrefillChunk : n;
        for (int j = 0; j < nr; j++)
            if (rows_out[j] >= done && rows_out[j] < end) {
                c->sel_out.push_back(j);
                c->sel_row.push_back(rows_out[j] - done);
            }
    }
    chunk_begin.push_back((int)c->sel_out.size());
    HIPCHK(c, hipMemcpyAsync(L.sel, c->sel_row.data(), (size_t)nr * 4, hipMemcpyHostToDevice, s));
    if (d_rows) HIPCHK(c, hipMemcpyAsync(L.selo, c->sel_out.data(), (size_t)nr * 4, hipMemcpyHostToDevice, s));
    int ci = 0;
    for (int done = 0; done < n; done += kPrefillChunk, ci++) {
        const int m = (n - done) < kPrefillChunk ? (n - done) : kPrefillChunk;
        const int p0 = c->len;
        const int sb = chunk_begin[ci], k = chunk_begin[ci + 1] - sb;  // wanted rows of this chunk
        HIPCHK(c, hipMemcpyAsync(L.ptok, h_tokens + done, (size_t)m * 4, hipMemcpyHostToDevice, s));
        HIPCHK(c, launch_embed_rows(L.embd, L.ptok, m, L.X, cf.dim, s));
        bool normed = false;  // Hf/Hh/Hl already hold this layer's attention-norm rows
        for (int l = 0; l < cf.n_layers; l++) {
            const LayerW& W = L.layers[l];
            const bool last = l == cf.n_layers - 1;
            __half* kc = L.kc + (size_t)l * L.kv_layer;
            __half* vc = L.vc + (size_t)l * L.kv_layer;
            // (an integer product's codes come from the norm itself)
            if (!normed) HIPCHK(c, norm_rows(nullptr, 0, L.X, m, W.attn_norm, W.qkv));
            normed = false;
            if (rnd && !prefill_codes(c, W.qkv)) HIPCHK(c, round_rows(L.Hf, m, cf.dim, W.qkv, L.Hh, L.Hl));
            // (with head_dim 64 and every pair rotated, the product applies RoPE
            // and writes q and the cache rows itself where it can)
            const RopeArgs ro{L.rope, L.Q, kc, vc, p0, cf.n_heads, cf.n_kv_heads, cf.n_ctx, cf.rope_neox};
            int ro_done = 0;
            HIPCHK(c, launch_gemm(EPI_STORE, W.qkv, ga(W.qkv, L.Hf, L.Hh, L.Hl), m, L.QKV, qkvd, W.bqkv, nullptr,
                                  nullptr, L.ws, L.ws_floats, s, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  cf.head_dim == 64 && cf.rope_dims == 64 ? &ro : nullptr, &ro_done));
            if (!ro_done)
                HIPCHK(c, launch_rope_kv_rows(L.QKV, m, p0, cf.n_heads, cf.n_kv_heads, cf.head_dim, cf.rope_dims,
                                              cf.rope_neox, cf.n_ctx, L.rope, L.Q, kc, vc, s));
            AttnArgs t;
            memset(&t, 0, sizeof t);
            t.q = L.Q;
            t.kc = kc;
            t.vc = vc;
            t.out = L.Of;
            t.out_h = nullptr;
            t.part = L.attn_part;
            t.st = nullptr;
            t.p0 = p0;
            t.n_heads = cf.n_heads;
            t.n_kv_heads = cf.n_kv_heads;
            t.head_dim = cf.head_dim;
            t.n_ctx = cf.n_ctx;
            t.n_split = 1;
            t.scale_div = (float)sqrt((double)cf.head_dim);
            t.span = span_cfg(cf);
            t.rnd = cf.numerics;
            t.stats = L.attn_stats;
            const bool mfma_attn = cf.head_dim == 64 && (64 % (cf.n_heads / cf.n_kv_heads)) == 0;
            // (no hi/lo planes where the output product runs on the codes, no
            // fp32 rows where it reads only the planes, except in the last
            // layer, whose rows are gathered)
            // (in the rounding mode the attention writes the output product's
            // Q8_0 codes itself, except in the last layer, whose rows are
            // gathered first)
            const bool o_codes = prefill_codes(c, W.o), o_fused = rnd && o_codes && mfma_attn && !last;
            const bool o_rows = last || (!prefill_planes_only(c, W.o) && !o_fused);
            if (mfma_attn)
                HIPCHK(c, launch_attn_prefill_mfma(L.Q, kc, vc, o_rows ? L.Of : nullptr, o_codes ? nullptr : L.Oh,
                                                   o_codes ? nullptr : L.Ol, m, p0, cf.n_heads, cf.n_kv_heads,
                                                   cf.head_dim, cf.n_ctx, t.scale_div, t.span, rnd, L.ws, L.ws_floats,
                                                   s, o_fused ? L.Ci : nullptr, o_fused ? L.Cs : nullptr));
            else
                HIPCHK(c, launch_attn(t, m, s));
            // output product + residual, RMSNorm, gate/up + SwiGLU, down +
            // residual over mr rows (attention outputs `of`, residuals X)
            auto post_attention = [&](const float* of, float* X, int mr, bool o_done) -> int {
                if (rnd && !o_done)
                    HIPCHK(c, round_rows((float*)of, mr, qd, W.o, L.Oh, L.Ol));
                else if (W.o.wt && (last || !mfma_attn))  // the planes the tiled product reads
                    HIPCHK(c, launch_split_hl(of, mr, qd, L.Oh, L.Ol, s));
                // a split-K output product's reduction is fused with the FFN norm
                int S = 0;
                HIPCHK(c, launch_gemm(EPI_RESID, W.o, ga(W.o, of, L.Oh, L.Ol), mr, X, cf.dim, nullptr, nullptr,
                                      nullptr, L.ws, L.ws_floats, s, nullptr, &S));
                HIPCHK(c, norm_rows(L.ws, S, X, mr, W.ffn_norm, W.gu));
                if (rnd && !prefill_codes(c, W.gu)) HIPCHK(c, round_rows(L.Hf, mr, cf.dim, W.gu, L.Hh, L.Hl));
                // (no hi/lo planes of the SwiGLU output where down runs on the
                // codes; in the rounding mode the gate/up product may write
                // those codes itself, into the fp32 rows' buffer, which it then
                // leaves unused: kPrefillChunk x ffn bytes of codes, then the
                // block scales)
                const bool d_codes = prefill_codes(c, W.down);
                int8_t* uc = (int8_t*)L.Uf;
                float* ucs = (float*)(uc + (size_t)kPrefillChunk * cf.ffn);
                int u_done = 0;
                HIPCHK(c, launch_gemm(EPI_SWIGLU, W.gu, ga(W.gu, L.Hf, L.Hh, L.Hl), mr,
                                      prefill_planes_only(c, W.down) ? nullptr : L.Uf, cf.ffn, nullptr,
                                      d_codes ? nullptr : L.Uh, d_codes ? nullptr : L.Ul, L.ws, L.ws_floats, s,
                                      nullptr, nullptr, d_codes ? uc : nullptr, ucs, &u_done));
                if (rnd && !u_done) HIPCHK(c, round_rows(L.Uf, mr, cf.ffn, W.down, L.Uh, L.Ul));
                const GemmA da = u_done ? GemmA{nullptr, nullptr, nullptr, uc, ucs} : ga(W.down, L.Uf, L.Uh, L.Ul);
                // before another layer a split-K down product's reduction is
                // fused with that layer's attention norm
                HIPCHK(c, launch_gemm(EPI_RESID, W.down, da, mr, X, cf.dim, nullptr, nullptr, nullptr, L.ws,
                                      L.ws_floats, s, nullptr, last ? nullptr : &S));
                if (!last && S) {
                    HIPCHK(c, norm_rows(L.ws, S, X, mr, L.layers[l + 1].attn_norm, L.layers[l + 1].qkv));
                    normed = true;
                }
                return LLM_OK;
            };
            if (!last) {
                if ((rc = post_attention(L.Of, L.X, m, o_fused))) return rc;
                continue;
            }
            // The last layer: only the wanted rows go on, gathered into compact
            // batches of at most one chunk's rows (repeated rows can make a
            // chunk want more rows than it holds); each batch then gets the
            // final RMSNorm and the vocabulary product.
            for (int b0 = 0; b0 < k; b0 += kPrefillChunk) {
                const int kb = k - b0 < kPrefillChunk ? k - b0 : kPrefillChunk;
                HIPCHK(c, launch_gather_rows(L.Of, qd, L.sel + sb + b0, kb, L.Q, s));
                HIPCHK(c, launch_gather_rows(L.X, cf.dim, L.sel + sb + b0, kb, L.Xc, s));
                if ((rc = post_attention(L.Q, L.Xc, kb, false))) return rc;
                if (d_rows) {
                    // product rows land at their output indices
                    HIPCHK(c, launch_rmsnorm_rows(L.Xc, L.out_norm, kb, cf.dim, cf.eps, L.Hf, L.Hh, L.Hl, s));
                    if (rnd) HIPCHK(c, round_rows(L.Hf, kb, cf.dim, L.out, L.Hh, L.Hl));
                    HIPCHK(c, launch_gemm(EPI_STORE, L.out, ga(L.out, L.Hf, L.Hh, L.Hl), kb, d_rows, cf.vocab, nullptr,
                                          nullptr, nullptr, L.ws, L.ws_floats, s, L.selo + sb + b0));
                } else {
                    // the one wanted row (the prompt's last) through the decode
                    // vocabulary kernel and argmax
                    HIPCHK(c, launch_set_state(L.st, 0, p0 + m - 1, 0, s));
                    HIPCHK(c, enqueue_logits(c, L.Xc, s));
                }
            }
        }
        c->len += m;
    }
    return LLM_OK;
}

static int check_prompt(llm_ctx* c, const int32_t* h_tokens, int32_t n) {
    if (n <= 0 || !h_tokens) return fail(c, LLM_ERR_ARG, "n must be positive and h_tokens set");
    for (int i = 0; i < n; i++)
        if (h_tokens[i] < 0 || h_tokens[i] >= c->cfg.vocab) return fail(c, LLM_ERR_TOKEN, "token out of range");
    if ((int64_t)c->len + n > c->cfg.n_ctx) return fail(c, LLM_ERR_CTX_FULL, "prefill would pass n_ctx");
    return LLM_OK;
}

int llm_prefill(llm_ctx* c, const int32_t* h_tokens, int32_t n, float* d_logits, int32_t* h_next) {
    int rc = check_ctx(c);
    if (rc) return rc;
    if ((rc = check_prompt(c, h_tokens, n))) return rc;
    const std::vector<int32_t> last{n - 1};
    if ((rc = prefill_pass(c, h_tokens, n, last, nullptr))) return rc;
    return finish(c, d_logits, h_next);
}

int llm_prefill_rows(llm_ctx* c, const int32_t* h_tokens, int32_t n, const int32_t* h_rows, int32_t n_rows,
                     float* d_logits) {
    int rc = check_ctx(c);
    if (rc) return rc;
    if ((rc = check_prompt(c, h_tokens, n))) return rc;
    if (!d_logits) return fail(c, LLM_ERR_ARG, "d_logits must be set");
    std::vector<int32_t> rows;
    if (h_rows) {
        if (n_rows <= 0 || n_rows > c->cfg.n_ctx) return fail(c, LLM_ERR_ARG, "n_rows must be in 1..n_ctx");
        rows.assign(h_rows, h_rows + n_rows);
        for (int32_t r : rows)
            if (r < 0 || r >= n) return fail(c, LLM_ERR_ARG, "a row index is outside the prompt");
    } else {
        if (n_rows != n) return fail(c, LLM_ERR_ARG, "with h_rows NULL, n_rows must equal n");
        rows.resize(n);
        for (int32_t i = 0; i < n; i++) rows[i] = i;
    }
    return prefill_pass(c, h_tokens, n, rows, d_logits);
}

int llm_reset(llm_ctx* c) {
    int rc = check_ctx(c);
    if (rc) return rc;
    c->len = 0;
    return LLM_OK;
}

void llm_free(llm_ctx* c) {
    if (!c) return;
    if (c->stream) (void)hipStreamSynchronize(c->stream);
    else (void)hipDeviceSynchronize();
    release(c);
}

const char* llm_last_error(const llm_ctx* c) { return c ? c->err.c_str() : g_load_error.c_str(); }

const float* llm_logits(const llm_ctx* c) { return c ? c->L.logits : nullptr; }

int32_t llm_kv_len(const llm_ctx* c) { return c ? c->len : -1; }

int llm_kv_read(const llm_ctx* cc, int32_t layer, int32_t pos, uint16_t* h_k, uint16_t* h_v) {
    llm_ctx* c = (llm_ctx*)cc;
    int rc = check_ctx(c);
    if (rc) return rc;
    if (layer < 0 || layer >= c->cfg.n_layers || pos < 0 || pos >= c->cfg.n_ctx || !h_k || !h_v)
        return fail(c, LLM_ERR_ARG, "kv_read: layer/pos out of range or null output");
    const Layout& L = c->L;
    const size_t hd = c->cfg.head_dim;
    const size_t pitch = (size_t)c->cfg.n_ctx * hd * 2;
    const char* kb = (const char*)(L.kc + (size_t)layer * L.kv_layer + (size_t)pos * hd);
    const char* vb = (const char*)(L.vc + (size_t)layer * L.kv_layer + (size_t)pos * hd);
    HIPCHK(c, hipMemcpy2DAsync(h_k, hd * 2, kb, pitch, hd * 2, c->cfg.n_kv_heads, hipMemcpyDeviceToHost, c->stream));
    HIPCHK(c, hipMemcpy2DAsync(h_v, hd * 2, vb, pitch, hd * 2, c->cfg.n_kv_heads, hipMemcpyDeviceToHost, c->stream));
    HIPCHK(c, hipStreamSynchronize(c->stream));
    return LLM_OK;
}

// ------------------------------------------------------------------ llm_ops.h
namespace {
int check_layer(llm_ctx* c, int32_t layer) {
    int rc = check_ctx(c);
    if (rc) return rc;
    if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, LLM_ERR_ARG, "layer out of range");
    return LLM_OK;
}
}  // namespace

int llm_op_qkv(llm_ctx* c, int32_t layer, int32_t pos, const float* d_x, float* d_q) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (pos < 0 || pos >= c->cfg.n_ctx || !d_x || !d_q) return fail(c, LLM_ERR_ARG, "bad position or pointer");
    HIPCHK(c, launch_set_state(c->L.st, 0, pos, 0, c->stream));
    HIPCHK(c, stage_qkv(c, layer, d_x, false, d_q, c->stream));
    return LLM_OK;
}

int llm_op_attention(llm_ctx* c, int32_t layer, int32_t pos, const float* d_q, float* d_out) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (pos < 0 || pos >= c->cfg.n_ctx || !d_q || !d_out) return fail(c, LLM_ERR_ARG, "bad position or pointer");
    HIPCHK(c, launch_set_state(c->L.st, 0, pos, 0, c->stream));
    HIPCHK(c, stage_attn(c, layer, d_q, d_out, c->stream));
    return LLM_OK;
}

int llm_op_o(llm_ctx* c, int32_t layer, const float* d_in, float* d_x) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (!d_in || !d_x) return fail(c, LLM_ERR_ARG, "null pointer");
    HIPCHK(c, stage_o(c, layer, d_in, d_x, c->stream));
    return LLM_OK;
}

int llm_op_ffn_up(llm_ctx* c, int32_t layer, const float* d_x, float* d_u) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (!d_x || !d_u) return fail(c, LLM_ERR_ARG, "null pointer");
    HIPCHK(c, stage_ffn_up(c, layer, d_x, d_u, c->stream));
    return LLM_OK;
}

int llm_op_down(llm_ctx* c, int32_t layer, const float* d_u, float* d_x) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (!d_u || !d_x) return fail(c, LLM_ERR_ARG, "null pointer");
    HIPCHK(c, stage_down(c, layer, d_u, d_x, c->stream));
    return LLM_OK;
}

int llm_op_logits(llm_ctx* c, const float* d_x, float* d_logits, int32_t* h_next) {
    int rc = check_ctx(c);
    if (rc) return rc;
    if (!d_x) return fail(c, LLM_ERR_ARG, "null pointer");
    HIPCHK(c, launch_set_state(c->L.st, 0, 0, 0, c->stream));
    HIPCHK(c, enqueue_logits(c, d_x, c->stream));
    return finish(c, d_logits, h_next);
}

int llm_op_kv_write(llm_ctx* c, int32_t layer, int32_t pos0, int32_t n_pos, const uint16_t* h_k, const uint16_t* h_v) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (pos0 < 0 || n_pos < 0 || (int64_t)pos0 + n_pos > c->cfg.n_ctx || !h_k || !h_v)
        return fail(c, LLM_ERR_ARG, "rows out of range or null pointer");
    if (n_pos == 0) return LLM_OK;
    const Layout& L = c->L;
    const size_t hd = c->cfg.head_dim, kvd = (size_t)c->kvd;
    // the pages' [pos][kv_head*head_dim] rows become head-major [kv_head][pos][head_dim]
    for (int g = 0; g < c->cfg.n_kv_heads; g++) {
        char* kd = (char*)(L.kc + (size_t)layer * L.kv_layer + ((size_t)g * c->cfg.n_ctx + pos0) * hd);
        char* vd = (char*)(L.vc + (size_t)layer * L.kv_layer + ((size_t)g * c->cfg.n_ctx + pos0) * hd);
        HIPCHK(c, hipMemcpy2DAsync(kd, hd * 2, h_k + g * hd, kvd * 2, hd * 2, n_pos, hipMemcpyHostToDevice, c->stream));
        HIPCHK(c, hipMemcpy2DAsync(vd, hd * 2, h_v + g * hd, kvd * 2, hd * 2, n_pos, hipMemcpyHostToDevice, c->stream));
    }
    HIPCHK(c, hipStreamSynchronize(c->stream));
    return LLM_OK;
}

int llm_op_time(llm_ctx* c, int32_t stage, int32_t layer, int32_t pos, int32_t n_launch, float* h_ms) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (stage < LLM_STAGE_QKV || stage > LLM_STAGE_STEP || n_launch <= 0 || !h_ms || pos < 0 || pos >= c->cfg.n_ctx)
        return fail(c, LLM_ERR_ARG, "bad stage, position, count or pointer");
    const Layout& L = c->L;
    hipStream_t s = c->stream;
    HIPCHK(c, launch_set_state(L.st, 0, pos, 0, s));
    // the persistent kernel reads token and position from the state: with the
    // feedback off every launch recomputes the same step
    auto one = [&]() -> hipError_t {
        switch (stage) {
            case LLM_STAGE_QKV: return stage_qkv(c, layer, L.x, false, L.q, s);
            case LLM_STAGE_ATTN: return stage_attn(c, layer, L.q, L.ao, s);
            case LLM_STAGE_O: return stage_o(c, layer, L.ao, L.x, s);
            case LLM_STAGE_FFN_UP: return stage_ffn_up(c, layer, L.x, L.u, s);
            case LLM_STAGE_DOWN: return stage_down(c, layer, L.u, L.x, s);
            case LLM_STAGE_STEP:
                if (c->use_step) return launch_step(c->step, c->step_fn, c->step_grid, c->step_lds, s);
                return enqueue_step(c, s);
            default: return enqueue_logits(c, L.x, s);
        }
    };
    HIPCHK(c, one());  // warm
    hipEvent_t e0, e1;
    HIPCHK(c, hipEventCreate(&e0));
    HIPCHK(c, hipEventCreate(&e1));
    hipError_t e = hipEventRecord(e0, s);
    for (int i = 0; e == hipSuccess && i < n_launch; i++) e = one();
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (e != hipSuccess) return dev_fail(c, e, "llm_op_time");
    *h_ms = ms / (float)n_launch;
    return LLM_OK;
}

int llm_op_time_prefill_product(llm_ctx* c, int32_t product, int32_t layer, int32_t n_rows, int32_t n_launch,
                                float* h_ms) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (product < LLM_PRODUCT_QKV || product > LLM_PRODUCT_DOWN || n_rows < 1 || n_rows > kPrefillChunk ||
        n_launch <= 0 || !h_ms)
        return fail(c, LLM_ERR_ARG, "bad product, row count, launch count or pointer");
    Layout& L = c->L;
    const LayerW& W = L.layers[layer];
    hipStream_t s = c->stream;
    const int qkvd = c->qd + 2 * c->kvd;
    // the prompt pass's operands and epilogues; a residual product's split-K
    // partials stay in the workspace (the pass adds them in its next RMSNorm)
    auto one = [&]() -> hipError_t {
        int S = 0;
        switch (product) {
            case LLM_PRODUCT_QKV:
                return launch_gemm(EPI_STORE, W.qkv, prefill_operand(c, W.qkv, L.Hf, L.Hh, L.Hl), n_rows, L.QKV, qkvd,
                                   W.bqkv, nullptr, nullptr, L.ws, L.ws_floats, s);
            case LLM_PRODUCT_O:
                return launch_gemm(EPI_RESID, W.o, prefill_operand(c, W.o, L.Of, L.Oh, L.Ol), n_rows, L.X, c->cfg.dim,
                                   nullptr, nullptr, nullptr, L.ws, L.ws_floats, s, nullptr, &S);
            case LLM_PRODUCT_GATE_UP: {
                const bool d_codes = prefill_codes(c, W.down);
                return launch_gemm(EPI_SWIGLU, W.gu, prefill_operand(c, W.gu, L.Hf, L.Hh, L.Hl), n_rows,
                                   prefill_planes_only(c, W.down) ? nullptr : L.Uf, c->cfg.ffn, nullptr, d_codes ? nullptr : L.Uh, d_codes ? nullptr : L.Ul, L.ws,
                                   L.ws_floats, s);
            }
            default:
                return launch_gemm(EPI_RESID, W.down, prefill_operand(c, W.down, L.Uf, L.Uh, L.Ul), n_rows, L.X,
                                   c->cfg.dim, nullptr, nullptr, nullptr, L.ws, L.ws_floats, s, nullptr, &S);
        }
    };
    HIPCHK(c, one());  // warm
    hipEvent_t e0, e1;
    HIPCHK(c, hipEventCreate(&e0));
    HIPCHK(c, hipEventCreate(&e1));
    hipError_t e = hipEventRecord(e0, s);
    for (int i = 0; e == hipSuccess && i < n_launch; i++) e = one();
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (e != hipSuccess) return dev_fail(c, e, "llm_op_time_prefill_product");
    *h_ms = ms / (float)n_launch;
    return LLM_OK;
}

int llm_op_prefill_chunk(void) { return kPrefillChunk; }

int llm_op_prefill_int8(llm_ctx* c) {
    int rc = check_ctx(c);
    if (rc) return rc;
    return c->cfg.numerics && c->L.Ci && !c->L.layers.empty() && c->L.layers[0].qkv.wi ? 1 : 0;
}

int llm_op_step_kind(llm_ctx* c) {
    int rc = check_ctx(c);
    if (rc) return rc;
    return c->use_step ? (c->step_special ? 2 : 1) : 0;
}

int llm_op_step_trace(llm_ctx* c, uint64_t* h_out, int32_t n) {
    int rc = check_ctx(c);
    if (rc) return rc;
    const int total = kStepPhases * c->cfg.n_layers + 2;
    if (!h_out || n < total) return fail(c, LLM_ERR_ARG, "output too small");
    if (!c->use_step || !c->step.trace) return fail(c, LLM_ERR_ARG, "step trace is off (set LLM_STEP_TRACE=1 before loading)");
    HIPCHK(c, hipMemcpyAsync(h_out, c->L.strace, (size_t)total * 8, hipMemcpyDeviceToHost, c->stream));
    HIPCHK(c, hipStreamSynchronize(c->stream));
    return LLM_OK;
}

int llm_rewind(llm_ctx* c, int32_t len) {
    int rc = check_ctx(c);
    if (rc) return rc;
    if (len < 0 || len > c->len) return fail(c, LLM_ERR_POS, "rewind length beyond kv_len");
    c->len = len;
    return LLM_OK;
}

// ------------------------------------------------- allocation-free attention
// llm_op_attention_noalloc keeps everything its kernels write besides the
// output in this array (each device holds its own copy until the process
// ends): the position state, the split partials (m, l, o) and, with the
// rounding mode, the span maxima and sums.
}  // extern "C"

static __device__ __align__(256) unsigned char scratch[LLM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // the array's device address on each device

// The array's address on `dev` (which must be current): looked up once per
// device with hipGetSymbolAddress. Host code never uses the array's own name
// as an address.
hipError_t noalloc_scratch(int dev, char** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = p;
    }
    *out = (char*)g_scratch_dev[dev];
    return hipSuccess;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }
}  // namespace

extern "C" {

int llm_op_attention_noalloc(llm_ctx* c, int32_t layer, int32_t pos, const float* d_q, float* d_out) {
    int rc = check_layer(c, layer);
    if (rc) return rc;
    if (pos < 0 || pos >= c->cfg.n_ctx || !d_q || !d_out) return fail(c, LLM_ERR_ARG, "bad position or pointer");
    const llm_config& cf = c->cfg;
    const int n_split = c->L.n_split;
    // the state, the split partials of one query, the span statistics of one query
    const size_t st_bytes = round256(sizeof(State));
    const size_t part_bytes = round256((size_t)n_split * cf.n_kv_heads * c->G * (cf.head_dim + 2) * sizeof(float));
    const size_t stats_bytes = round256((size_t)cf.n_heads * 2 * sizeof(float));
    if (st_bytes + part_bytes + stats_bytes > (size_t)LLM_NOALLOC_SCRATCH_BYTES)
        return fail(c, LLM_ERR_LIMIT, "the attention's split partials exceed the allocation-free scratch");
    int dev = -1;
    HIPCHK(c, hipGetDevice(&dev));
    if (dev != c->device) return fail(c, LLM_ERR_ARG, "the context's device must be the current device");
    char* base = nullptr;
    HIPCHK(c, noalloc_scratch(dev, &base));
    State* st = (State*)base;
    HIPCHK(c, launch_set_state(st, 0, pos, 0, c->stream));
    const Layout& L = c->L;
    AttnArgs t;
    memset(&t, 0, sizeof t);
    t.q = d_q;
    t.kc = L.kc + (size_t)layer * L.kv_layer;
    t.vc = L.vc + (size_t)layer * L.kv_layer;
    t.out = d_out;
    t.part = (float*)(base + st_bytes);
    t.st = st;
    t.n_heads = cf.n_heads;
    t.n_kv_heads = cf.n_kv_heads;
    t.head_dim = cf.head_dim;
    t.n_ctx = cf.n_ctx;
    t.n_split = n_split;
    t.scale_div = (float)sqrt((double)cf.head_dim);
    t.span = span_cfg(cf);
    t.rnd = cf.numerics;
    t.stats = (float*)(base + st_bytes + part_bytes);
    HIPCHK(c, launch_attn(t, 1, c->stream));
    return LLM_OK;
}

}  // extern "C"
