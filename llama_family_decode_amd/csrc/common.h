// Internal types shared by the host runtime and the gfx950 kernels of libllm.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace llm {

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_Q8 = 8 };

// A weight matrix in device layout: `rows` output rows of `cols` inputs.
//  F32/F16: row r at w + r * cols elements (cols % 32 == 0, so rows are 64/128-byte aligned).
//  Q8_0:    int8 quants row r at w + r * cols bytes; fp16 scales row r at s + r * cols/32,
//           scale b of row r belonging to quants [32b, 32b+32).
struct Mat {
    int dtype;
    int rows, cols;
    const void* w;
    const uint16_t* s;
    const void* wt;  // the prefill products' tiled binary16 copy (Q8_0: of the codes), or nullptr
    const void* st;  // Q8_0 with wt: the block scales, [256-row tile][K step][256] binary16
    const void* wi;  // Q8_0 under llama.cpp's rounding points: the tiled int8 codes, or nullptr
    const float* si; // with wi: the block scales as fp32, [256-row tile][K step][256]
};

// Tiled binary16 layout of the prefill products' operands: rows in tiles of
// TM (128 for activations, 256 for weights), K in steps of 32; tile t, step
// ks, 16-row group g is one contiguous 1 KB piece at ((t*nk + ks)*(TM/16) + g)
// KB, nk = K/32, whose 16-byte slot 4r + (c ^ swz(r)) holds row r's elements
// 8c .. 8c+7 of the step, swz(r) = ((r >> 1) ^ (r >> 3)) & 3 (the LDS order of
// the product kernel, so one DMA moves one piece).
constexpr int kTileA = 128, kTileW = 256;
__host__ __device__ inline int tile_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__host__ __device__ inline size_t tile_off(int m, int k, int K, int TM) {
    const int nk = K >> 5, t = m / TM, rr = m - t * TM, g = rr >> 4, r = rr & 15;
    const int ks = k >> 5, c = (k >> 3) & 3, e = k & 7;
    return (((size_t)t * nk + ks) * (TM >> 4) + g) * 512 + (size_t)(4 * r + (c ^ tile_swz(r))) * 8 + e;
}
inline size_t tiled_w_bytes(int rows, int cols) { return (size_t)((rows + kTileW - 1) / kTileW) * kTileW * cols * 2; }
inline size_t tiled_s_bytes(int rows, int cols) {
    return (size_t)((rows + kTileW - 1) / kTileW) * kTileW * (cols / 32) * 2;
}
// Tiled int8 layout of Q8_0 codes (the integer products of llama.cpp's
// rounding points): rows in tiles of TM, K in steps of 32; tile t, step ks is
// one contiguous TM x 32-byte piece, row r's 32 codes at 32 r with their two
// 16-byte halves swapped when i8_swz(r) is set. A fragment read takes one half
// of 32 consecutive rows; the swap puts the rows of any 8 (or 16) consecutive
// lanes in distinct 16-byte bank groups.
// The block scales of activation rows: [128-row tile][K step][128] fp32.
__host__ __device__ inline int i8_swz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
__host__ __device__ inline size_t tile_off_i8(int m, int k, int K, int TM) {
    const int nk = K >> 5, t = m / TM, r = m - t * TM;
    return (((size_t)t * nk + (k >> 5)) * TM + r) * 32 + ((((k >> 4) & 1) ^ i8_swz(r)) << 4) + (k & 15);
}
__host__ __device__ inline size_t tile_off_s(int m, int kb, int K, int TM) {
    const int t = m / TM;
    return ((size_t)t * (K >> 5) + kb) * TM + (m - t * TM);
}
inline size_t tiled_i8_bytes(int rows, int cols) { return (size_t)((rows + kTileW - 1) / kTileW) * kTileW * cols; }
inline size_t tiled_sf_bytes(int rows, int cols) {
    return (size_t)((rows + kTileW - 1) / kTileW) * kTileW * (cols / 32) * 4;
}

// Attention span and temperature of the config: the query at position p
// attends rows p-window+1..p plus rows 0..sinks-1 (window 0: rows 0..p), with
// q scaled by 1 + temp_scale * ln(floor(p / temp_len) + 1) (temp_scale 0: 1).
struct SpanCfg {
    int window, sinks;
    float temp_scale;
    int temp_len;
};
// The attended rows of position pos as n indices: index j is row j for
// j < ns (sinks below the window), row lo + (j - ns) after; the last index is
// always row pos.
struct Span {
    int n, ns, lo;
};
__host__ __device__ inline Span attn_span(const SpanCfg& c, int pos) {
    if (c.window <= 0) return Span{pos + 1, 0, 0};
    const int lo = pos - c.window + 1 > 0 ? pos - c.window + 1 : 0;
    const int ns = c.sinks < lo ? c.sinks : lo;
    return Span{ns + pos - lo + 1, ns, lo};
}
__host__ __device__ inline int span_row(const Span& s, int j) { return j < s.ns ? j : s.lo + (j - s.ns); }
__host__ __device__ inline bool span_has(const SpanCfg& c, int t, int pos) {
    return t <= pos && (c.window <= 0 || t > pos - c.window || t < c.sinks);
}
// v rounded to binary16 and back
__device__ __forceinline__ float round16(float v) { return __half2float(__float2half_rn(v)); }

// llama.cpp's rounding of 32 consecutive product inputs for Q8_0 weights
// ("What a Llama model computes, and why", section 8, with the Q8_0 quantizer
// of "The Forward Pass in Java", Example 8): d = amax / 127 and its inverse in
// float, codes roundf(x / d) (halves away from zero), values f16(d) * code.
__device__ __forceinline__ void q8_round32(float (&v)[32]) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
    const float d = amax / 127.f, id = d != 0.f ? 1.f / d : 0.f, dh = round16(d);
#pragma unroll
    for (int j = 0; j < 32; j++) v[j] = dh * roundf(v[j] * id);
}

// The query scale, evaluated in double and rounded to float.
__host__ __device__ inline float attn_temp(const SpanCfg& c, int pos) {
    if (c.temp_scale == 0.0f || c.temp_len <= 0) return 1.0f;
    return (float)(1.0 + (double)c.temp_scale * log((double)(pos / c.temp_len) + 1.0));
}

// Decode-step state, resident in device memory so that a captured graph can run
// any step: the kernels read token and pos from here, the argmax writes next.
struct State {
    int token;
    int pos;
    int next;
    int nonfinite;
    int gen_mode;   // 1: the argmax also advances token/pos and appends to gen_out
    int gen_count;
    int epoch;      // launches of the persistent step kernel so far
    int abort;      // set when a grid barrier wait exceeded its spin limit
    unsigned long long best;  // argmax key of the running step (0 = none yet)
};

// Per-block partial of the vocabulary argmax: (max, first index, non-finite seen).
struct ArgPart {
    float val;
    int idx;
    int nonfinite;
    int pad;
};

// One layer's weights in device layout.
struct LayerW {
    const float* attn_norm;
    Mat qkv;            // rows: q | k | v
    const float* bqkv;  // q | k | v bias or nullptr
    Mat o;
    const float* ffn_norm;
    Mat gu;             // rows interleaved: gate j at 2j, up j at 2j+1
    Mat down;
};

// Arguments of the persistent decode-step kernel. Activations that cross
// blocks live in buffers with one copy per layer, so within a launch each
// address is written once, before any block reads it.
struct StepArgs {
    const LayerW* layers;  // device array of n_layers descriptors
    int n_layers;
    Mat embd, out;
    const float* out_norm;
    __half* kc;
    __half* vc;
    long long kv_layer;  // elements of one layer of one cache
    const float2* rope;
    State* st;
    unsigned long long* bar;  // barrier counters, kBarStride u64 apart
    float* qkv;     // q | k | v after bias and RoPE, per layer [n_layers][qkv_stride]
    float* part;    // attention split partials per layer [n_layers][part_stride]
    float* pst;     // rounding mode: the splits' (max, sum) of the first attention pass [n_layers][pst_stride]
    float* po;      // output-product partial sums per layer and group [n_layers][kStepGroups][pstride]
    float* pd;      // down-product partial sums, same layout
    float* u;       // SwiGLU output per layer [n_layers][u_stride]
    float* logits;  // [vocab]
    int* gen_out;
    int gen_cap;
    long long qkv_stride, part_stride, u_stride, pstride, pst_stride;
    unsigned long long* trace;  // nullptr, or wall-clock stamps of block 0 after each barrier
    int dim, n_heads, n_kv_heads, head_dim, n_rot, neox, n_ctx, ffn, vocab;
    int lds_xr, lds_xs, lds_wsp;  // LDS regions (floats)
    int lds_lw;                   // LDS offset (floats) of the copy of the layer table
    float eps, scale_div;
    SpanCfg span;
    int rnd;  // 1: llama.cpp's rounding points (product inputs, q, probabilities)
};

constexpr int kStepGroups = 8;     // block groups of the persistent step kernel (one per XCD)
constexpr int kMaxStepGrid = 4096;  // blocks of the persistent step kernel at most
constexpr int kStepMaxSplit = 64;  // attention splits per KV head of the persistent step kernel
constexpr int kStepPhases = 5;     // barriers per layer of the persistent step kernel
constexpr int kBarSlots = 2 * kStepGroups;  // barrier counters
constexpr int kBarStride = 32;     // u64 elements between counters (256 bytes)

constexpr int kBlock = 256;  // threads per block for all decode kernels (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kMaxCols = 16384;
constexpr int kMaxHeadDim = 256;
constexpr int kMaxGroup = 8;  // n_heads / n_kv_heads must be 1, 2, 4 or 8
constexpr int kMaxSplit = 256;      // position splits of the decode attention
#ifndef LLM_PREFILL_CHUNK
#define LLM_PREFILL_CHUNK 2048
#endif
constexpr int kPrefillChunk = LLM_PREFILL_CHUNK;  // tokens per prefill batch

// Prologue of a vector product: where the input vector comes from.
enum Pro : int {
    PRO_PLAIN = 0,  // x = xin (fp32 vector)
    PRO_NORM = 1,   // x = rmsnorm(xin) * gain
    PRO_EMBED = 2,  // x = rmsnorm(E[token]) * gain, and E[token] becomes the residual stream
};
// Epilogue of a vector product: what happens to the row results.
enum Epi : int {
    EPI_STORE = 0,   // y[r] = acc
    EPI_RESID = 1,   // y[r] += acc (residual add)
    EPI_SWIGLU = 2,  // rows (2j, 2j+1) = (gate j, up j): y[j] = silu(gate) * up
    EPI_QKV = 3,     // bias, RoPE on q and k, q -> y, k and v -> F16 cache at pos
    EPI_ARGMAX = 4,  // y[r] = acc, plus the greedy argmax over all rows
};

struct GemvArgs {
    Mat W;
    const float* xin;
    const float* gain;
    float eps;
    Mat E;            // embedding table (PRO_EMBED)
    float* xres;      // PRO_EMBED: the residual stream written by block 0
    State* st;
    float* y;
    const float* bias;  // EPI_QKV: concatenated q|k|v bias or nullptr
    // EPI_QKV
    int n_heads, n_kv_heads, head_dim, n_rot, neox, n_ctx;
    const float2* rope;  // [n_ctx][n_rot/2] (cos, sin)
    __half* kc;          // this layer's K cache [n_kv_heads][n_ctx][head_dim]
    __half* vc;
    // EPI_ARGMAX
    int* gen_out;
    int gen_cap;
    int rnd;  // llama.cpp's rounding points: round the staged input for W's type
};

struct AttnArgs {
    const float* q;       // [n_q][n_heads*head_dim]
    const __half* kc;     // this layer's caches [n_kv_heads][n_ctx][head_dim]
    const __half* vc;
    float* out;           // fp32 [n_q][n_heads*head_dim]
    __half* out_h;        // optional f16 copy of the output (prefill MFMA input) or nullptr
    float* part;          // split partials
    const State* st;      // decode: P = st->pos + 1
    int p0;               // prefill: query z is at position p0 + z
    int n_heads, n_kv_heads, head_dim, n_ctx;
    int n_split;          // gridDim.x
    float scale_div;      // scores are divided by this ((float)sqrt(head_dim))
    SpanCfg span;
    // llama.cpp's rounding points (q and the probabilities to binary16) run as
    // passes: 1 = split maxima and sums only, 2 = the weighted sum of V with
    // probabilities f16(e^(s - M) / L) from stats ([n_q][n_heads][2]: M, L)
    int rnd;
    float* stats;
};

// YaRN parameters (factor 0: off).
struct YarnCfg {
    float factor;
    int orig_ctx;
    float beta_fast, beta_slow;
};

// Launchers (kernels_decode.hip / kernels_prefill.hip).
// (cos, sin) of every (position, pair) angle; freq (n_rot/2 divisors, or
// nullptr) divides each pair's angle; YaRN (if on) remaps it and scales both.
hipError_t launch_rope_table(float2* tab, int n_pos, int n_rot, float base, const float* freq, const YarnCfg& yarn,
                             hipStream_t s);
hipError_t launch_gemv(int pro, int epi, const GemvArgs& a, int grid, hipStream_t s);
int gemv_grid(int pro, int epi, int rows);
hipError_t launch_attn(const AttnArgs& a, int n_q, hipStream_t s);
hipError_t launch_set_state(State* st, int token, int pos, int gen_mode, hipStream_t s);
hipError_t launch_argmax_finalize(State* st, int* gen_out, int gen_cap, hipStream_t s);
// Persistent step kernel for layer weights of type dtype: the grid (0 if the
// shape or the device does not allow it; also fills the LDS plan of a), the
// kernel chosen (*special: one compiled for this shape), and the launch of one
// step.
int step_grid(StepArgs& a, int dtype, int* lds_bytes, const void** fn, bool* special);
hipError_t launch_step(const StepArgs& a, const void* fn, int grid, int lds_bytes, hipStream_t s);
// Whether a grid of `grid` blocks puts the blocks with equal
// b mod 8 on one XCD (the step kernel's groups share their L2). d_buf holds
// grid ints.
bool step_groups_share_l2(int grid, int* d_buf, hipStream_t s);

struct PrefillBufs;
hipError_t launch_embed_rows(const Mat& E, const int* tokens, int n, float* X, int dim, hipStream_t s);
// Yf = rmsnorm(X) * gain per row; with Yh set also the binary16 hi/lo pair of
// each output (Yh = f16(y), Yl = f16(y - Yh)) in the tiled layout, the
// matrix-core input form; with C and CS (dim a multiple of 32) the outputs'
// Q8_0 codes and block scales in the tiled int8 layout, as launch_round_rows
// writes them (the integer products' input). Yf and Yh may be nullptr.
hipError_t launch_rmsnorm_rows(const float* X, const float* gain, int n, int dim, float eps, float* Yf, __half* Yh,
                               __half* Yl, hipStream_t s, int8_t* C = nullptr, float* CS = nullptr);
// dst[j][0..K) = src[idx[j]][0..K) for j < k (fp32 rows).
hipError_t launch_gather_rows(const float* src, int K, const int* idx, int k, float* dst, hipStream_t s);
// H, L = the tiled binary16 hi/lo planes of the n x K fp32 rows X.
hipError_t launch_split_hl(const float* X, int n, int K, __half* H, __half* L, hipStream_t s);
// llama.cpp's rounding of the n x K fp32 product inputs X for weights of type
// dtype (Q8_0: each 32-block to its quantized values; F16: to binary16), in
// place; H, L (if set) get the rounded rows' tiled hi/lo planes.
// With C and CS (Q8_0 only) the rounded rows' codes and block scales go to the
// tiled int8 layout instead, and X is left as it was (the integer product
// reads only the codes).
hipError_t launch_round_rows(float* X, int n, int K, int dtype, __half* H, __half* L, hipStream_t s,
                             int8_t* C = nullptr, float* CS = nullptr);
// The tiled copy of an F16 matrix (rows padded with zeros to a multiple of 256).
// Fills W.wt (and for Q8_0 W.st) from W's stored rows.
hipError_t launch_tile_w(const Mat& W, hipStream_t s);
// Causal prefill attention of n_q queries at positions p0 .. p0+n_q-1 on the
// matrix cores (head_dim 64 only; hipErrorInvalidValue otherwise): out (if
// set) as fp32 rows [n_q][n_heads*64] and, when out_h is set, their tiled
// binary16 hi/lo planes. With rnd, oc/ocs (if set) receive the rows' Q8_0
// codes and block scales in the tiled int8 layout, as launch_round_rows
// writes them (rnd only: hipErrorInvalidValue otherwise).
hipError_t launch_attn_prefill_mfma(const float* Q, const __half* kc, const __half* vc, float* out, __half* out_h,
                                    __half* out_l, int n_q, int p0, int n_heads, int n_kv_heads, int head_dim,
                                    int n_ctx, float scale_div, const SpanCfg& span, bool rnd, float* ws,
                                    size_t ws_floats, hipStream_t s, int8_t* oc = nullptr, float* ocs = nullptr);
// Activations of a prefill product: fp32 rows (ld K) and, for F16 weights,
// their binary16 hi/lo planes (tiled layout); l = nullptr when the activations
// are binary16 already (one matrix-core pass).
struct GemmA {
    const float* f;
    const __half* h;
    const __half* l;
    // llama.cpp's rounding points with Q8_0 weights: the rows' Q8_0 codes
    // (tiled int8, kTileA rows) and block scales (the binary16 scale as fp32),
    // or nullptr
    const int8_t* c;
    const float* cs;
};
// Y[n][rows] op= A[n][K] * W^T: F16 weights on the matrix cores with the
// hi/lo activation planes, Q8_0 on the matrix cores splitting the fp32 rows,
// F32 on the vector ALUs. SwiGLU also writes its output's hi/lo planes when
// Yh is set. ws (ws_floats floats) holds split-K partials. A plain store may
// scatter its rows: with ymap (device, n entries) row m goes to Y row ymap[m].
// A residual product with defer set leaves a split-K product's S partials in
// ws for the caller (*defer = S; 0 when it wrote Y itself). A SwiGLU product
// given yc/ycs (and no Yh) may write its output as Q8_0 codes and block scales
// in the tiled int8 layout (K = ldy), as launch_round_rows writes them, instead
// of the fp32 rows Y: it does so when its integer path runs over one K split,
// and then sets *yc_done to 1 (else 0, and Y holds the rows).
// A q|k|v product given ro (head_dim 64, every pair rotated) may instead apply
// RoPE to its rows and write q to ro.Q and k, v to this layer's F16 cache, as
// launch_rope_kv_rows does from Y: it does so in its epilogue over one K split
// on the tiled and integer paths, and in the reduction of split-K partials,
// and then sets *ro_done to 1 (else 0, and Y holds the rows).
struct RopeArgs {
    const float2* rope;  // [pos][32] (cos, sin)
    float* Q;            // [n][n_heads * 64]
    __half* kc;          // [n_kv_heads][n_ctx][64]
    __half* vc;
    int p0, n_heads, n_kv_heads, n_ctx, neox;
};
hipError_t launch_gemm(int epi, const Mat& W, const GemmA& A, int n, float* Y, int ldy, const float* bias,
                       __half* Yh, __half* Yl, float* ws, size_t ws_floats, hipStream_t s,
                       const int* ymap = nullptr, int* defer = nullptr, int8_t* yc = nullptr, float* ycs = nullptr,
                       int* yc_done = nullptr, const RopeArgs* ro = nullptr, int* ro_done = nullptr);
// X[m] += the S split-K partials of ws (z order), then Y = rmsnorm(X[m]) * gain
// as launch_rmsnorm_rows computes it.
hipError_t launch_reduce_norm_rows(const float* P, int S, int n, float* X, int dim, const float* gain, float eps,
                                   float* Yf, __half* Yh, __half* Yl, hipStream_t s, int8_t* C = nullptr,
                                   float* CS = nullptr);
hipError_t launch_rope_kv_rows(const float* QKV, int n, int p0, int n_heads, int n_kv_heads, int head_dim, int n_rot,
                               int neox, int n_ctx, const float2* rope, float* Q, __half* kc, __half* vc,
                               hipStream_t s);

// Value of lane l ^ M, for a compile-time M: DPP quad permutes for 1 and 2,
// swizzles (within 32 lanes) for 4, 8 and 16, the gfx950 half swap for 32.
// None of them goes through an LDS address computation as a bpermute does.
template <int M>
__device__ __forceinline__ uint32_t xshfl_u(uint32_t v) {
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    } else if constexpr (M == 4 || M == 8 || M == 16) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));    // bitmask mode, xor M
    } else {
        static_assert(M == 32, "xor offset");
        // swaps lanes 32..63 of the first operand with lanes 0..31 of the second
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? r[0] : r[1];
    }
}
template <int M>
__device__ __forceinline__ float xshfl(float v) { return __uint_as_float(xshfl_u<M>(__float_as_uint(v))); }
template <int M>
__device__ __forceinline__ int xshfl(int v) { return (int)xshfl_u<M>((uint32_t)v); }
template <int M>
__device__ __forceinline__ double xshfl(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = xshfl_u<M>((uint32_t)b), hi = xshfl_u<M>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

}  // namespace llm
