// Decode-step kernels for gfx950 (CDNA4, wave64).
//
// One token's forward pass ("The Forward Pass in Java", Project 18 forward();
// "What a Llama model computes, and why", section 2) runs as five fused
// launches per layer plus one for the logits:
//   1. RMSNorm prologue + Q/K/V vector product + bias + RoPE + F16 KV store
//      (layer 0 also gathers the embedding row, section 2.1)
//   2. flash-decode grouped-query attention over the cache (split over
//      positions, log-sum-exp combine by the last block of each KV head)
//   3. output product + residual add
//   4. RMSNorm prologue + gate/up product + SwiGLU
//   5. down product + residual add
//   6. final RMSNorm prologue + vocabulary product + greedy argmax
// Every product streams its weight rows once with 16-byte loads per lane; the
// input vector is staged once per block in LDS (swizzled so the per-lane reads
// are bank-conflict free) and Q8_0 quants are dequantised in registers. All
// reductions are in a fixed order (no float atomics), so results are
// deterministic run to run.
#include "device_common.h"

namespace llm {

// Stage the product's input vector in LDS (swizzled for weight type DT).
//   PRO_PLAIN: x = xin.   PRO_NORM: x = rmsnorm(xin) * gain.
//   PRO_EMBED: x = rmsnorm(E[token]) * gain; block 0 also writes E[token] to xres.
// RMSNorm ("The Forward Pass in Java", Example 4): the sum of squares is taken
// in double, the scale 1/sqrt(ss/n + eps) is rounded to float once, and
// y = (x * scale) * g.
template <int DT, int PRO>
__device__ void stage_input(const GemvArgs& a, float* xs, double* red) {
    const int K = a.W.cols;
    const int tid = threadIdx.x;
    double ss = 0.0;
    int64_t tok = 0;
    if constexpr (PRO == PRO_EMBED) tok = a.st->token;
    for (int i = tid; i < K; i += kBlock) {
        float v;
        if constexpr (PRO == PRO_EMBED) {
            v = mat_elem(a.E, tok, i);
            if (blockIdx.x == 0) a.xres[i] = v;
        } else {
            v = a.xin[i];
        }
        if constexpr (PRO != PRO_PLAIN) ss += (double)v * (double)v;
        xs[swz<DT>(i)] = v;
    }
    if constexpr (PRO != PRO_PLAIN) {
        double tot = block_sum_d(ss, red);
        const float scale = (float)(1.0 / sqrt(tot / (double)K + (double)a.eps));
        for (int i = tid; i < K; i += kBlock) {
            const int j = swz<DT>(i);
            xs[j] = xs[j] * scale * a.gain[i];
        }
    }
    if constexpr (DT != DT_F32) {
        if (a.rnd) {  // llama.cpp's rounding of the product's input for this weight type
            __syncthreads();
            for (int b = tid; b < K / 32; b += kBlock) {
                float v[32];
#pragma unroll
                for (int j = 0; j < 32; j++) v[j] = xs[swz<DT>(32 * b + j)];
                if constexpr (DT == DT_Q8) {
                    q8_round32(v);
                } else {
#pragma unroll
                    for (int j = 0; j < 32; j++) v[j] = round16(v[j]);
                }
#pragma unroll
                for (int j = 0; j < 32; j++) xs[swz<DT>(32 * b + j)] = v[j];
            }
        }
    }
    __syncthreads();
}

// Rows per wave for each epilogue.
template <int EPI>
struct RowsPer {
    static constexpr int NR = (EPI == EPI_QKV || EPI == EPI_RESID) ? LLM_GEMV_NR_SMALL : LLM_GEMV_NR_BIG;
};

template <int EPI>
__device__ __forceinline__ int n_groups(const GemvArgs& a) {
    constexpr int NR = RowsPer<EPI>::NR;
    return (a.W.rows + NR - 1) / NR;
}

// Rows of group g. For EPI_QKV a group is NR/2 rotation pairs (a, b): within a
// head, pair j < n_rot/2 is (2j, 2j+1) in the normal layout and (j, j + n_rot/2)
// in the NEOX layout ("The Forward Pass in Java", Example 6); the dimensions past
// n_rot form unrotated neighbour pairs.
template <int EPI>
__device__ __forceinline__ void group_rows(const GemvArgs& a, int g, int* rows) {
    constexpr int NR = RowsPer<EPI>::NR;
    if constexpr (EPI == EPI_QKV) {
        const int hp = a.head_dim / 2, half = a.n_rot / 2;
#pragma unroll
        for (int p = 0; p < NR / 2; p++) {
            const int pi = g * (NR / 2) + p;
            const int head = pi / hp, j = pi % hp;
            int ra, rb;
            if (j < half) {
                ra = head * a.head_dim + (a.neox ? j : 2 * j);
                rb = a.neox ? ra + half : ra + 1;
            } else {
                ra = head * a.head_dim + a.n_rot + 2 * (j - half);
                rb = ra + 1;
            }
            rows[2 * p] = ra;
            rows[2 * p + 1] = rb;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NR; i++) rows[i] = g * NR + i;
    }
}

template <int DT, int PRO, int EPI>
__global__ __launch_bounds__(kBlock) void k_gemv(GemvArgs a) {
    extern __shared__ float xs[];
    __shared__ double red[kWaves];
    __shared__ ArgPart wbest[kWaves];
    constexpr int NR = RowsPer<EPI>::NR;
    constexpr int VE = VecW<DT>::VE;
    // chunks per lane whose loads are in flight together (a Q8_0 row of 8192 is 8)
    constexpr int U = (DT == DT_Q8 && NR == LLM_GEMV_NR_SMALL) ? LLM_GEMV_U_Q8 : LLM_GEMV_U;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = a.W.cols, R = a.W.rows;
    const int nch = K / VE;
    const int ng = n_groups<EPI>(a);
    const int g0 = blockIdx.x * kWaves + wave;
    float best = -INFINITY;
    int best_i = 0x7fffffff, nonfinite = 0;

    u32x4 raw[U][NR];
    float sc[U][NR];
    int rows[NR], lrow[NR];
    // Rows and first batch of weight loads of this wave's first group, issued
    // before the input vector is staged: weights do not depend on it.
    if (g0 < ng) {
        group_rows<EPI>(a, g0, rows);
#pragma unroll
        for (int i = 0; i < NR; i++) lrow[i] = rows[i] < R ? rows[i] : R - 1;
        load_batch<DT, NR, U>(a.W, lrow, lane, nch, raw, sc);
    }

    stage_input<DT, PRO>(a, xs, red);

    for (int g = g0; g < ng; g += gridDim.x * kWaves) {
        if (g != g0) {
            group_rows<EPI>(a, g, rows);
#pragma unroll
            for (int i = 0; i < NR; i++) lrow[i] = rows[i] < R ? rows[i] : R - 1;
        }
        float acc[NR];
#pragma unroll
        for (int i = 0; i < NR; i++) acc[i] = 0.f;
        for (int c0 = lane; c0 < nch; c0 += 64 * U) {
            if (g != g0 || c0 != lane) load_batch<DT, NR, U>(a.W, lrow, c0, nch, raw, sc);
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int c = c0 + 64 * u;
                if (c < nch) {
#pragma unroll
                    for (int i = 0; i < NR; i++) {
                        const float p = chunk_dot<DT>(raw[u][i], xs, c);
                        if constexpr (DT == DT_Q8)
                            acc[i] += sc[u][i] * p;
                        else
                            acc[i] += p;
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NR; i++) acc[i] = wave_sum(acc[i]);

        if (lane == 0) {
            if constexpr (EPI == EPI_STORE) {
#pragma unroll
                for (int i = 0; i < NR; i++)
                    if (rows[i] < R) a.y[rows[i]] = acc[i];
            } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
                for (int i = 0; i < NR; i++)
                    if (rows[i] < R) a.y[rows[i]] += acc[i];
            } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int p = 0; p < NR / 2; p++)
                    if (rows[2 * p] < R) a.y[rows[2 * p] / 2] = silu(acc[2 * p]) * acc[2 * p + 1];
            } else if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    if (rows[i] < R) {
                        const float v = acc[i];
                        a.y[rows[i]] = v;
                        if (!isfinite(v)) nonfinite = 1;
                        if (v > best) {  // rows arrive in increasing order: ties keep the first
                            best = v;
                            best_i = rows[i];
                        }
                    }
                }
            } else if constexpr (EPI == EPI_QKV) {
                const int pos = a.st->pos;
                const int qd = a.n_heads * a.head_dim, kvd = a.n_kv_heads * a.head_dim;
                const int hp = a.head_dim / 2, half = a.n_rot / 2;
#pragma unroll
                for (int p = 0; p < NR / 2; p++) {
                    const int ra = rows[2 * p], rb = rows[2 * p + 1];
                    if (ra >= R) continue;
                    float va = acc[2 * p], vb = acc[2 * p + 1];
                    if (a.bias) {
                        va += a.bias[ra];
                        vb += a.bias[rb];
                    }
                    const int pi = g * (NR / 2) + p;
                    const int head = pi / hp, j = pi % hp;
                    if (head < a.n_heads + a.n_kv_heads && j < half) {
                        const float2 cs = a.rope[(size_t)pos * half + j];
const float2 rv = rope_rotate(va, vb, cs);
                        va = rv.x;
                        vb = rv.y;
                    }
                    if (ra < qd) {
                        a.y[ra] = va;
                        a.y[rb] = vb;
                    } else if (ra < qd + kvd) {
                        const int gk = (ra - qd) / a.head_dim, ia = (ra - qd) % a.head_dim, ib = (rb - qd) % a.head_dim;
                        __half* row = a.kc + ((size_t)gk * a.n_ctx + pos) * a.head_dim;
                        row[ia] = f2h(va);
                        row[ib] = f2h(vb);
                    } else {
                        const int gv = (ra - qd - kvd) / a.head_dim, ia = (ra - qd - kvd) % a.head_dim,
                                  ib = (rb - qd - kvd) % a.head_dim;
                        __half* row = a.vc + ((size_t)gv * a.n_ctx + pos) * a.head_dim;
                        row[ia] = f2h(va);
                        row[ib] = f2h(vb);
                    }
                }
            }
        }
    }

    if constexpr (EPI == EPI_ARGMAX) {
        // Pass 1 of the argmax: this block's (max, first index), merged into the
        // step's 64-bit key with one atomic; the finalize launch decodes it.
        if (lane == 0) wbest[wave] = ArgPart{best, best_i, nonfinite, 0};
        __syncthreads();
        if (threadIdx.x == 0) {
            ArgPart b = wbest[0];
            for (int w = 1; w < kWaves; w++) {
                const ArgPart o = wbest[w];
                if (o.val > b.val || (o.val == b.val && o.idx < b.idx)) {
                    b.val = o.val;
                    b.idx = o.idx;
                }
                b.nonfinite |= o.nonfinite;
            }
            if (b.idx != 0x7fffffff) atomicMax(&a.st->best, argmax_key(b.val, b.idx));
            if (b.nonfinite) atomicOr(&a.st->nonfinite, 1);
        }
    }
}

template <int DT, int PRO, int EPI>
static hipError_t launch_one(const GemvArgs& a, int grid, hipStream_t s) {
    const size_t lds = (size_t)lds_floats<DT>(a.W.cols) * sizeof(float);
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)k_gemv<DT, PRO, EPI>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024 + 4096);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    hipLaunchKernelGGL((k_gemv<DT, PRO, EPI>), dim3(grid), dim3(kBlock), lds, s, a);
    return hipGetLastError();
}

template <int PRO, int EPI>
static hipError_t launch_dt(const GemvArgs& a, int grid, hipStream_t s) {
    switch (a.W.dtype) {
        case DT_F32: return launch_one<DT_F32, PRO, EPI>(a, grid, s);
        case DT_F16: return launch_one<DT_F16, PRO, EPI>(a, grid, s);
        case DT_Q8: return launch_one<DT_Q8, PRO, EPI>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

int gemv_grid(int pro, int epi, int rows) {
    (void)pro;
    const int nr = (epi == EPI_QKV || epi == EPI_RESID) ? LLM_GEMV_NR_SMALL : LLM_GEMV_NR_BIG;
    const int groups = (rows + nr - 1) / nr;
    int blocks = (groups + kWaves - 1) / kWaves;
    const int cap = LLM_GEMV_GRID_CAP;
    return blocks < cap ? blocks : cap;
}

hipError_t launch_gemv(int pro, int epi, const GemvArgs& a, int grid, hipStream_t s) {
    if (pro == PRO_EMBED && epi == EPI_QKV) return launch_dt<PRO_EMBED, EPI_QKV>(a, grid, s);
    if (pro == PRO_NORM && epi == EPI_QKV) return launch_dt<PRO_NORM, EPI_QKV>(a, grid, s);
    if (pro == PRO_PLAIN && epi == EPI_RESID) return launch_dt<PRO_PLAIN, EPI_RESID>(a, grid, s);
    if (pro == PRO_NORM && epi == EPI_SWIGLU) return launch_dt<PRO_NORM, EPI_SWIGLU>(a, grid, s);
    if (pro == PRO_NORM && epi == EPI_ARGMAX) return launch_dt<PRO_NORM, EPI_ARGMAX>(a, grid, s);
    if (pro == PRO_PLAIN && epi == EPI_STORE) return launch_dt<PRO_PLAIN, EPI_STORE>(a, grid, s);
    if (pro == PRO_NORM && epi == EPI_STORE) return launch_dt<PRO_NORM, EPI_STORE>(a, grid, s);
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ RoPE table
// Row p holds (cos, sin) of theta_i for i < n_rot/2 ("The Forward Pass in Java",
// Example 6): theta starts at (float)p and is multiplied by theta_scale =
// base^(-2/n_rot) (double, rounded to float) in float once per pair; cos and
// sin are evaluated in double and rounded to float.
// Llama 3 frequency factors divide pair i's angle ("What a Llama model
// computes, and why", sections 2.4 and 6). YaRN (the YaRN paper, Peng et al.,
// 2023, named in section 6) mixes the angle a into (1 - g) a / s + g a, g the
// ramp of the pair's turns r = L base^(-2i/n_rot) / (2 pi) over the original
// context L (0 below beta_slow, 1 above beta_fast), in double, and scales cos
// and sin by 1 + 0.1 ln s.
__global__ void k_rope_table(float2* tab, int n_pos, int half, float theta_scale, float base, const float* freq,
                             YarnCfg y) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_pos) return;
    const int n_rot = 2 * half;
    const bool yarn = y.factor > 0.0f;
    const double m = yarn ? 1.0 + 0.1 * log((double)y.factor) : 1.0;
    float theta = (float)p;
    for (int i = 0; i < half; i++) {
        float angle = freq ? theta / freq[i] : theta;
        if (yarn) {
            const double r = (double)y.orig_ctx * pow((double)base, -2.0 * i / n_rot) / 6.283185307179586476925286766559;
            const double g = r < y.beta_slow ? 0.0 : r > y.beta_fast ? 1.0
                                                 : (r - y.beta_slow) / ((double)y.beta_fast - y.beta_slow);
            angle = (float)((1.0 - g) * ((double)angle / y.factor) + g * (double)angle);
        }
        tab[(size_t)p * half + i] = make_float2((float)(m * cos((double)angle)), (float)(m * sin((double)angle)));
        theta = theta * theta_scale;
    }
}

hipError_t launch_rope_table(float2* tab, int n_pos, int n_rot, float base, const float* freq, const YarnCfg& yarn,
                             hipStream_t s) {
    const int half = n_rot / 2;
    const float theta_scale = (float)pow((double)base, -2.0 / n_rot);  // on the host, as the angle recurrence's start
    hipLaunchKernelGGL(k_rope_table, dim3((n_pos + 255) / 256), dim3(256), 0, s, tab, n_pos, half, theta_scale, base,
                       freq, yarn);
    return hipGetLastError();
}

__global__ void k_set_state(State* st, int token, int pos, int gen_mode) {
    if (threadIdx.x == 0) {
        st->token = token;
        st->pos = pos;
        st->gen_mode = gen_mode;
        st->gen_count = 0;
        st->nonfinite = 0;
        st->best = 0ull;
    }
}

// Pass 2 of the argmax: decode the step's key into the next token; in
// generation mode also feed it back (token = next, pos + 1) and record it.
__global__ void k_argmax_finalize(State* st, int* gen_out, int gen_cap) {
    if (threadIdx.x == 0) {
        const unsigned long long k = st->best;
        const int next = k ? (int)(0xffffffffu - (uint32_t)(k & 0xffffffffull)) : 0;
        st->next = next;
        if (st->gen_mode) {
            const int c = st->gen_count;
            if (c < gen_cap) gen_out[c] = next;
            st->gen_count = c + 1;
            st->token = next;
            st->pos = st->pos + 1;
        }
        st->best = 0ull;
    }
}

hipError_t launch_argmax_finalize(State* st, int* gen_out, int gen_cap, hipStream_t s) {
    hipLaunchKernelGGL(k_argmax_finalize, dim3(1), dim3(64), 0, s, st, gen_out, gen_cap);
    return hipGetLastError();
}

hipError_t launch_set_state(State* st, int token, int pos, int gen_mode, hipStream_t s) {
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(64), 0, s, st, token, pos, gen_mode);
    return hipGetLastError();
}

// ------------------------------------------------------------------ attention
// Grouped-query attention of one token over the F16 cache ("The Forward Pass in
// Java", Example 7; "What a Llama model computes, and why", section 2.5). Query
// head h reads KV head h / G, G = n_heads / n_kv_heads; a block serves all G
// query heads of one KV head, so every K and V row is read once. The positions
// 0..P-1 are split across gridDim.x blocks; within a block they are processed
// in chunks with an online softmax (running max m, sum l, unnormalised output
// o). Scores are divided by sqrt(head_dim). k_attn_combine merges the splits:
// M = max m_s, L = sum l_s e^(m_s - M), out = sum o_s e^(m_s - M) / L.
// The attended rows are the span of the query's position (all rows up to it,
// or a window plus sinks, "The Engine"), taken as a dense index range, and
// q is scaled by the attention temperature of that position.
//
// Thread layout: LPP lanes share one position, each lane holding 8 consecutive
// dimensions (one 16-byte load of a K or V row); PPI = 256/LPP positions per
// step, and a chunk is kAttnSteps steps, whose K and V loads are all issued
// before any of them is used.
template <int G>
__global__ __launch_bounds__(kBlock) void k_attn(AttnArgs a) {
    extern __shared__ float sm[];
    __shared__ float m_run[G], l_run[G], alpha[G];

    const int s = blockIdx.x, g = blockIdx.y, z = blockIdx.z;
    const int hd = a.head_dim;
    const int qpos = a.st ? a.st->pos : a.p0 + z;
    const Span span = attn_span(a.span, qpos);
    const int P = span.n;
    const int S = a.n_split;
    int CH = (P + S - 1) / S;
    CH = (CH + 15) & ~15;
    const int n_active = (P + CH - 1) / CH;
    if (s >= n_active) return;
    const int t_begin = s * CH, t_end = min(P, t_begin + CH);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int LPP = attn_lpp(hd);
    const int PPI = kBlock / LPP;
    const int CHUNK = PPI * kAttnSteps;
    const int sub = tid % LPP, pg = tid / LPP;
    const bool dim_ok = sub * 8 < hd;

    float* sc = sm;                     // [G][CHUNK] scores, then weights
    float* wred = sm + G * CHUNK;       // [kWaves][G][hd] output reduction

    const int qd = a.n_heads * hd;
    const float* qz = a.q + (size_t)z * qd;
    const float tau = attn_temp(a.span, qpos);
    float qv[G][8];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float v = dim_ok ? tau * qz[(g * G + h) * hd + sub * 8 + i] : 0.f;
            qv[h][i] = a.rnd ? round16(v) : v;
        }
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) acc[h][i] = 0.f;
    if (tid < G) {
        m_run[tid] = -INFINITY;
        l_run[tid] = 0.f;
    }

    const __half* kbase = a.kc + (size_t)g * a.n_ctx * hd + sub * 8;
    const __half* vbase = a.vc + (size_t)g * a.n_ctx * hd + sub * 8;
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    for (int c0 = t_begin; c0 < t_end; c0 += CHUNK) {
        const int cn = min(CHUNK, t_end - c0);
        u32x4 kr[kAttnSteps], vr[kAttnSteps];
#pragma unroll
        for (int i = 0; i < kAttnSteps; i++) {
            const int t = pg + i * PPI;
            const bool ok = dim_ok && t < cn;
            const size_t row = (size_t)span_row(span, c0 + t);
            kr[i] = ok ? *(const u32x4*)(kbase + row * hd) : z4;
            vr[i] = ok ? *(const u32x4*)(vbase + row * hd) : z4;
        }
        // scores
#pragma unroll
        for (int i = 0; i < kAttnSteps; i++) {
            const int t = pg + i * PPI;
            float kf[8];
            unpack8(kr[i], kf);
#pragma unroll
            for (int h = 0; h < G; h++) {
                float d = 0.f;
#pragma unroll
                for (int j = 0; j < 8; j++) d += qv[h][j] * kf[j];
                for (int o = 1; o < LPP; o <<= 1) d += __shfl_xor(d, o, 64);
                if (sub == 0 && t < cn) sc[h * CHUNK + t] = d / a.scale_div;
            }
        }
        __syncthreads();
        if (a.rnd == 2) {
            // probabilities from the whole span's max M and sum L, rounded
            // to binary16 before they weight V
            for (int h = wave; h < G; h += kWaves) {
                const float* mz = a.stats + ((size_t)z * a.n_heads + g * G + h) * 2;
                const float M = mz[0], L = mz[1];
                for (int t = lane; t < cn; t += 64) sc[h * CHUNK + t] = round16(expf(sc[h * CHUNK + t] - M) / L);
                if (lane == 0) alpha[h] = 1.f;
            }
        } else
        // chunk max, running max, weights and their sum (one wave per head)
        for (int h = wave; h < G; h += kWaves) {
            float mx = -INFINITY;
            for (int t = lane; t < cn; t += 64) mx = fmaxf(mx, sc[h * CHUNK + t]);
            mx = wave_max(mx);
            const float m_old = m_run[h];
            const float m_new = fmaxf(m_old, mx);
            float ls = 0.f;
            for (int t = lane; t < cn; t += 64) {
                const float e = expf(sc[h * CHUNK + t] - m_new);
                sc[h * CHUNK + t] = e;
                ls += e;
            }
            ls = wave_sum(ls);
            if (lane == 0) {
                const float al = (m_old == -INFINITY) ? 0.f : expf(m_old - m_new);
                alpha[h] = al;
                l_run[h] = l_run[h] * al + ls;
                m_run[h] = m_new;
            }
        }
        __syncthreads();
        // weighted values
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float al = alpha[h];
#pragma unroll
            for (int i = 0; i < 8; i++) acc[h][i] *= al;
        }
#pragma unroll
        for (int i = 0; i < kAttnSteps; i++) {
            const int t = pg + i * PPI;
            if (dim_ok && t < cn && a.rnd != 1) {
                float vf[8];
                unpack8(vr[i], vf);
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float w = sc[h * CHUNK + t];
#pragma unroll
                    for (int j = 0; j < 8; j++) acc[h][j] += w * vf[j];
                }
            }
        }
        __syncthreads();
    }
    // reduce the per-thread outputs over the positions each lane group took
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float v = acc[h][i];
            for (int o = LPP; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
            acc[h][i] = v;
        }
    if (lane < LPP && dim_ok)
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int i = 0; i < 8; i++) wred[(wave * G + h) * hd + sub * 8 + i] = acc[h][i];
    __syncthreads();

    const int GH = G * hd;
    float* outz = a.out + (size_t)z * qd + (size_t)g * G * hd;
    __half* outhz = a.out_h ? a.out_h + (size_t)z * qd + (size_t)g * G * hd : nullptr;
    if (n_active == 1 && a.rnd != 1) {
        for (int e = tid; e < GH; e += kBlock) {
            float o = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; w++) o += wred[w * GH + e];
            const float r = a.rnd == 2 ? o : o / l_run[e / hd];
            outz[e] = r;
            if (outhz) outhz[e] = f2h(r);
        }
        return;
    }
    // this split's (m, l, unnormalised o); k_attn_combine merges the splits
    const int stride = hd + 2;
    float* mypart = a.part + (((size_t)z * a.n_kv_heads + g) * S + s) * (size_t)(G * stride);
    for (int e = tid; e < GH; e += kBlock) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) o += wred[w * GH + e];
        mypart[(e / hd) * stride + 2 + (e % hd)] = o;
    }
    if (tid < G) {
        mypart[tid * stride] = m_run[tid];
        mypart[tid * stride + 1] = l_run[tid];
    }
}

// Merge of the position splits of one KV head's G query heads: M = max m_s,
// L = sum l_s e^(m_s - M), out = sum o_s e^(m_s - M) / L, splits in order.
// When a single split was active the attention kernel wrote out itself.
template <int G>
__global__ __launch_bounds__(kBlock) void k_attn_combine(AttnArgs a) {
    __shared__ float wj[kMaxSplit * G];
    __shared__ float Ls[G];
    const int g = blockIdx.x, z = blockIdx.y;
    const int hd = a.head_dim;
    const int P = attn_span(a.span, a.st ? a.st->pos : a.p0 + z).n;
    const int S = a.n_split;
    int CH = (P + S - 1) / S;
    CH = (CH + 15) & ~15;
    const int n_active = (P + CH - 1) / CH;
    if (n_active == 1) return;
    const int stride = hd + 2, GH = G * hd, qd = a.n_heads * hd;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* parts = a.part + (((size_t)z * a.n_kv_heads + g) * S) * (size_t)(G * stride);
    // split maxima and sums, one wave per head
    for (int h = wave; h < G; h += kWaves) {
        float M = -INFINITY;
        for (int j = lane; j < n_active; j += 64) M = fmaxf(M, parts[(size_t)j * G * stride + h * stride]);
        M = wave_max(M);
        float L = 0.f;
        for (int j = lane; j < n_active; j += 64) {
            const float* pj = parts + (size_t)j * G * stride + h * stride;
            const float f = expf(pj[0] - M);
            wj[j * G + h] = f;
            L += pj[1] * f;
        }
        L = wave_sum(L);
        if (lane == 0) Ls[h] = L;
    }
    __syncthreads();
    float* outz = a.out + (size_t)z * qd + (size_t)g * GH;
    for (int e = tid; e < GH; e += kBlock) {
        const int h = e / hd, d = e % hd;
        const float* po = parts + h * stride + 2 + d;
        float O = 0.f;
#pragma unroll 8
        for (int j = 0; j < n_active; j++) O += wj[j * G + h] * po[(size_t)j * G * stride];
        const float r = O / Ls[h];
        outz[e] = r;
        if (a.out_h) a.out_h[(size_t)z * qd + (size_t)g * GH + e] = f2h(r);
    }
}

// The rounded-probability passes (llama.cpp's rounding points): after pass 1,
// each head's span maximum M = max m_s and sum L = sum l_s e^(m_s - M) over its
// splits, in split order, go to stats.
template <int G>
__global__ __launch_bounds__(64 * G) void k_attn_stats(AttnArgs a) {
    const int g = blockIdx.x, z = blockIdx.y, h = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int P = attn_span(a.span, a.st ? a.st->pos : a.p0 + z).n;
    const int S = a.n_split;
    int CH = (P + S - 1) / S;
    CH = (CH + 15) & ~15;
    const int n_active = (P + CH - 1) / CH;
    const int stride = a.head_dim + 2;
    const float* parts = a.part + (((size_t)z * a.n_kv_heads + g) * S) * (size_t)(G * stride) + h * stride;
    float M = -INFINITY;
    for (int j = lane; j < n_active; j += 64) M = fmaxf(M, parts[(size_t)j * G * stride]);
    M = wave_max(M);
    float L = 0.f;
    if (lane == 0)
        for (int j = 0; j < n_active; j++) L += parts[(size_t)j * G * stride + 1] * expf(parts[(size_t)j * G * stride] - M);
    if (lane == 0) {
        float* st = a.stats + ((size_t)z * a.n_heads + g * G + h) * 2;
        st[0] = M;
        st[1] = L;
    }
}

// After pass 2 with several active splits: out = sum of the splits' outputs,
// in split order.
template <int G>
__global__ __launch_bounds__(kBlock) void k_attn_sum(AttnArgs a) {
    const int g = blockIdx.x, z = blockIdx.y;
    const int hd = a.head_dim;
    const int P = attn_span(a.span, a.st ? a.st->pos : a.p0 + z).n;
    const int S = a.n_split;
    int CH = (P + S - 1) / S;
    CH = (CH + 15) & ~15;
    const int n_active = (P + CH - 1) / CH;
    if (n_active == 1) return;
    const int stride = hd + 2, GH = G * hd, qd = a.n_heads * hd;
    const float* parts = a.part + (((size_t)z * a.n_kv_heads + g) * S) * (size_t)(G * stride);
    for (int e = threadIdx.x; e < GH; e += kBlock) {
        const float* po = parts + (e / hd) * stride + 2 + e % hd;
        float O = 0.f;
        for (int j = 0; j < n_active; j++) O += po[(size_t)j * G * stride];
        a.out[(size_t)z * qd + (size_t)g * GH + e] = O;
        if (a.out_h) a.out_h[(size_t)z * qd + (size_t)g * GH + e] = f2h(O);
    }
}

template <int G>
static hipError_t launch_attn_g(const AttnArgs& a, int n_q, hipStream_t s) {
    const size_t lds = ((size_t)G * attn_chunk(a.head_dim) + (size_t)kWaves * G * a.head_dim) * sizeof(float);
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)k_attn<G>, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    if (a.rnd) {
        AttnArgs p = a;
        p.rnd = 1;  // split maxima and sums
        hipLaunchKernelGGL((k_attn<G>), dim3(a.n_split, a.n_kv_heads, n_q), dim3(kBlock), lds, s, p);
        hipLaunchKernelGGL((k_attn_stats<G>), dim3(a.n_kv_heads, n_q), dim3(64 * G), 0, s, p);
        p.rnd = 2;  // the weighted sum with the rounded probabilities
        hipLaunchKernelGGL((k_attn<G>), dim3(a.n_split, a.n_kv_heads, n_q), dim3(kBlock), lds, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.n_split == 1) return e;
        hipLaunchKernelGGL((k_attn_sum<G>), dim3(a.n_kv_heads, n_q), dim3(kBlock), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_attn<G>), dim3(a.n_split, a.n_kv_heads, n_q), dim3(kBlock), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    hipLaunchKernelGGL((k_attn_combine<G>), dim3(a.n_kv_heads, n_q), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, int n_q, hipStream_t s) {
    switch (a.n_heads / a.n_kv_heads) {
        case 1: return launch_attn_g<1>(a, n_q, s);
        case 2: return launch_attn_g<2>(a, n_q, s);
        case 4: return launch_attn_g<4>(a, n_q, s);
        case 8: return launch_attn_g<8>(a, n_q, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace llm
