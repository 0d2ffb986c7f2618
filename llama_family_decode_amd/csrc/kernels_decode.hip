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
#include "common.h"

#include <math.h>

namespace llm {

// (x0, x1) rotated by the angle whose (cos, sin) is cs, each product rounded
// separately as the pages' RoPE computes it (no fused multiply-add).
__device__ __forceinline__ float2 rope_rotate(float x0, float x1, float2 cs) {
#pragma clang fp contract(off)
    return make_float2(x0 * cs.x - x1 * cs.y, x0 * cs.y + x1 * cs.x);
}

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// Elements per 16-byte chunk of a weight row.
template <int DT>
struct VecW {
    static constexpr int VE = DT == DT_F32 ? 4 : (DT == DT_F16 ? 8 : 16);
    static constexpr int SEG = VE * 64;  // elements read by one wave-wide 16-byte load
};

// Position of input element e in the LDS copy. Lane l's chunk c = 64*seg + l
// covers elements VE*c .. VE*c+VE-1; those are stored as VE/4 float4 pieces at
// seg*SEG + k*256 + 4*l, so each of the lane's ds_read_b128 hits consecutive
// 16-byte slots across the wave.
template <int DT>
__device__ __forceinline__ int swz(int e) {
    if constexpr (DT == DT_F32) {
        return e;
    } else {
        constexpr int VE = VecW<DT>::VE, SEG = VecW<DT>::SEG;
        int seg = e / SEG, w = e % SEG;
        int l = w / VE, k = (w % VE) >> 2, m = w & 3;
        return seg * SEG + k * 256 + 4 * l + m;
    }
}

template <int DT>
__host__ __device__ constexpr int lds_floats(int K) {
    return ((K + VecW<DT>::SEG - 1) / VecW<DT>::SEG) * VecW<DT>::SEG;
}

// Element i of row `row` of an F32/F16/Q8_0 matrix, as float (embedding gather).
__device__ __forceinline__ float mat_elem(const Mat& M, int64_t row, int i) {
    if (M.dtype == DT_F32) return ((const float*)M.w)[row * M.cols + i];
    if (M.dtype == DT_F16) return h2f(((const uint16_t*)M.w)[row * M.cols + i]);
    const int8_t* q = (const int8_t*)M.w;
    float d = h2f(M.s[row * (M.cols / 32) + i / 32]);
    return d * (float)q[row * M.cols + i];
}

// Block-wide sum of doubles, fixed order; every thread gets the result.
__device__ __forceinline__ double block_sum_d(double v, double* red) {
    v = wave_sum_d(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) t += red[w];
    return t;
}

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
    __syncthreads();
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw 16-byte chunk c of row r, loaded with the non-temporal hint (weights are
// streamed once per token).
template <int DT>
__device__ __forceinline__ u32x4 load_chunk(const Mat& W, int r, int c) {
    const char* base;
    if constexpr (DT == DT_F32)
        base = (const char*)W.w + ((size_t)r * W.cols) * 4;
    else if constexpr (DT == DT_F16)
        base = (const char*)W.w + ((size_t)r * W.cols) * 2;
    else
        base = (const char*)W.w + (size_t)r * W.cols;
    return __builtin_nontemporal_load((const u32x4*)base + c);
}

// Partial dot of one chunk with the staged input.
template <int DT>
__device__ __forceinline__ float chunk_dot(u32x4 raw, const float* xs, int c) {
    const int lane = c & 63, seg = c >> 6;
    if constexpr (DT == DT_F32) {
        const float4 x = *(const float4*)(xs + 4 * c);
        float s = __uint_as_float(raw.x) * x.x;
        s += __uint_as_float(raw.y) * x.y;
        s += __uint_as_float(raw.z) * x.z;
        s += __uint_as_float(raw.w) * x.w;
        return s;
    } else if constexpr (DT == DT_F16) {
        const float* b = xs + seg * 512 + 4 * lane;
        const float4 x0 = *(const float4*)(b);
        const float4 x1 = *(const float4*)(b + 256);
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
        float w[8];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            w[2 * k] = h2f((uint16_t)(u[k] & 0xffffu));
            w[2 * k + 1] = h2f((uint16_t)(u[k] >> 16));
        }
        float s = w[0] * x0.x;
        s += w[1] * x0.y;
        s += w[2] * x0.z;
        s += w[3] * x0.w;
        s += w[4] * x1.x;
        s += w[5] * x1.y;
        s += w[6] * x1.z;
        s += w[7] * x1.w;
        return s;
    } else {
        const float* b = xs + seg * 1024 + 4 * lane;
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float4 x = *(const float4*)(b + 256 * k);
            const int w = (int)u[k];
            const float q0 = (float)((w << 24) >> 24), q1 = (float)((w << 16) >> 24);
            const float q2 = (float)((w << 8) >> 24), q3 = (float)(w >> 24);
            s0 += q0 * x.x;
            s1 += q1 * x.y;
            s0 += q2 * x.z;
            s1 += q3 * x.w;
        }
        return s0 + s1;
    }
}

// Rows per wave for each epilogue.
template <int EPI>
struct RowsPer {
    static constexpr int NR = (EPI == EPI_QKV || EPI == EPI_RESID) ? 2 : 4;
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

// Order-preserving 64-bit key of (value, index): a larger value wins, and for
// equal values the smaller index wins, so the maximum key is the first index of
// the strict maximum ("The Forward Pass in Java", Example 9). -0 is taken as +0.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)o << 32) | (unsigned long long)(0xffffffffu - (uint32_t)idx);
}

// fp32 -> binary16 with round to nearest even (the hardware conversion).
__device__ __forceinline__ __half f2h(float v) { return __float2half_rn(v); }

template <int DT, int PRO, int EPI>
__global__ __launch_bounds__(kBlock) void k_gemv(GemvArgs a) {
    extern __shared__ float xs[];
    __shared__ double red[kWaves];
    __shared__ ArgPart wbest[kWaves];
    constexpr int NR = RowsPer<EPI>::NR;
    constexpr int VE = VecW<DT>::VE;
    constexpr int U = (DT == DT_F32) ? 4 : 2;  // chunks per lane loaded before use

    stage_input<DT, PRO>(a, xs, red);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = a.W.cols, R = a.W.rows;
    const int nch = K / VE;
    const int ng = n_groups<EPI>(a);
    float best = -INFINITY;
    int best_i = 0x7fffffff, nonfinite = 0;

    for (int g = blockIdx.x * kWaves + wave; g < ng; g += gridDim.x * kWaves) {
        int rows[NR];
        group_rows<EPI>(a, g, rows);
        int lrow[NR];
#pragma unroll
        for (int i = 0; i < NR; i++) lrow[i] = rows[i] < R ? rows[i] : R - 1;
        float acc[NR];
#pragma unroll
        for (int i = 0; i < NR; i++) acc[i] = 0.f;
        for (int c0 = lane; c0 < nch; c0 += 64 * U) {
            u32x4 raw[U][NR];
            float sc[U][NR];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int c = c0 + 64 * u;
                const int cc = c < nch ? c : c0;
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    raw[u][i] = load_chunk<DT>(a.W, lrow[i], cc);
                    if constexpr (DT == DT_Q8) sc[u][i] = h2f(a.W.s[(size_t)lrow[i] * (K / 32) + cc / 2]);
                }
            }
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
    const int nr = (epi == EPI_QKV || epi == EPI_RESID) ? 2 : 4;
    const int groups = (rows + nr - 1) / nr;
    int blocks = (groups + kWaves - 1) / kWaves;
    const int cap = 2048;
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
// Example 6): theta starts at (float)p and is multiplied by theta_scale in float
// once per pair; cos and sin are evaluated in double and rounded to float.
__global__ void k_rope_table(float2* tab, int n_pos, int half, float theta_scale) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_pos) return;
    float theta = (float)p;
    for (int i = 0; i < half; i++) {
        tab[(size_t)p * half + i] = make_float2((float)cos((double)theta), (float)sin((double)theta));
        theta = theta * theta_scale;
    }
}

hipError_t launch_rope_table(float2* tab, int n_pos, int n_rot, float theta_scale, hipStream_t s) {
    const int half = n_rot / 2;
    hipLaunchKernelGGL(k_rope_table, dim3((n_pos + 255) / 256), dim3(256), 0, s, tab, n_pos, half, theta_scale);
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
// o). Scores are divided by sqrt(head_dim). The last block of a KV head to
// finish merges the splits: M = max m_s, L = sum l_s e^(m_s - M),
// out = sum o_s e^(m_s - M) / L.
//
// Thread layout: LPP lanes share one position, each lane holding 8 consecutive
// dimensions (one 16-byte load of a K or V row); PPI = 256/LPP positions per
// step.
template <int G>
__global__ __launch_bounds__(kBlock) void k_attn(AttnArgs a) {
    extern __shared__ float sm[];
    __shared__ float m_run[G], l_run[G], alpha[G];

    const int s = blockIdx.x, g = blockIdx.y, z = blockIdx.z;
    const int hd = a.head_dim;
    const int P = a.st ? a.st->pos + 1 : a.p0 + z + 1;
    const int S = a.n_split;
    int CH = (P + S - 1) / S;
    CH = (CH + 15) & ~15;
    const int n_active = (P + CH - 1) / CH;
    if (s >= n_active) return;
    const int t_begin = s * CH, t_end = min(P, t_begin + CH);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int LPP = 1;
    while (LPP * 8 < hd) LPP <<= 1;
    const int PPI = kBlock / LPP;
    const int sub = tid % LPP, pg = tid / LPP;
    const bool dim_ok = sub * 8 < hd;

    float* sc = sm;                         // [G][kAttnChunk] scores, then weights
    float* wred = sm + G * kAttnChunk;      // [kWaves][G][hd] output reduction

    const int qd = a.n_heads * hd;
    const float* qz = a.q + (size_t)z * qd;
    float qv[G][8];
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) qv[h][i] = dim_ok ? qz[(g * G + h) * hd + sub * 8 + i] : 0.f;
    float acc[G][8];
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) acc[h][i] = 0.f;
    if (tid < G) {
        m_run[tid] = -INFINITY;
        l_run[tid] = 0.f;
    }

    const __half* kbase = a.kc + (size_t)g * a.n_ctx * hd;
    const __half* vbase = a.vc + (size_t)g * a.n_ctx * hd;

    for (int c0 = t_begin; c0 < t_end; c0 += kAttnChunk) {
        const int cn = min(kAttnChunk, t_end - c0);
        __syncthreads();
        // scores
        for (int tt = pg; tt < ((cn + PPI - 1) / PPI) * PPI; tt += PPI) {
            const bool ok = tt < cn;
            float part[G];
            for (int h = 0; h < G; h++) part[h] = 0.f;
            if (ok && dim_ok) {
                const uint4 raw = *(const uint4*)(kbase + (size_t)(c0 + tt) * hd + sub * 8);
                const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
                float kf[8];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    kf[2 * k] = h2f((uint16_t)(u[k] & 0xffffu));
                    kf[2 * k + 1] = h2f((uint16_t)(u[k] >> 16));
                }
                for (int h = 0; h < G; h++) {
                    float d = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; i++) d += qv[h][i] * kf[i];
                    part[h] = d;
                }
            }
            for (int h = 0; h < G; h++) {
                float d = part[h];
                for (int o = 1; o < LPP; o <<= 1) d += __shfl_xor(d, o, 64);
                if (sub == 0 && ok) sc[h * kAttnChunk + tt] = d / a.scale_div;
            }
        }
        __syncthreads();
        // chunk max, running max, weights and their sum (one wave per head)
        for (int h = wave; h < G; h += kWaves) {
            float mx = -INFINITY;
            for (int t = lane; t < cn; t += 64) mx = fmaxf(mx, sc[h * kAttnChunk + t]);
            mx = wave_max(mx);
            const float m_old = m_run[h];
            const float m_new = fmaxf(m_old, mx);
            float ls = 0.f;
            for (int t = lane; t < cn; t += 64) {
                const float e = expf(sc[h * kAttnChunk + t] - m_new);
                sc[h * kAttnChunk + t] = e;
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
        for (int h = 0; h < G; h++) {
            const float al = alpha[h];
#pragma unroll
            for (int i = 0; i < 8; i++) acc[h][i] *= al;
        }
        if (dim_ok) {
            for (int tt = pg; tt < cn; tt += PPI) {
                const uint4 raw = *(const uint4*)(vbase + (size_t)(c0 + tt) * hd + sub * 8);
                const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
                float vf[8];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    vf[2 * k] = h2f((uint16_t)(u[k] & 0xffffu));
                    vf[2 * k + 1] = h2f((uint16_t)(u[k] >> 16));
                }
                for (int h = 0; h < G; h++) {
                    const float w = sc[h * kAttnChunk + tt];
#pragma unroll
                    for (int i = 0; i < 8; i++) acc[h][i] += w * vf[i];
                }
            }
        }
    }
    // reduce the per-thread outputs over the positions each lane group took
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float v = acc[h][i];
            for (int o = LPP; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
            acc[h][i] = v;
        }
    __syncthreads();
    if (lane < LPP && dim_ok)
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int i = 0; i < 8; i++) wred[(wave * G + h) * hd + sub * 8 + i] = acc[h][i];
    __syncthreads();

    const int GH = G * hd;
    float* outz = a.out + (size_t)z * qd + (size_t)g * G * hd;
    __half* outhz = a.out_h ? a.out_h + (size_t)z * qd + (size_t)g * G * hd : nullptr;
    if (n_active == 1) {
        for (int e = tid; e < GH; e += kBlock) {
            float o = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; w++) o += wred[w * GH + e];
            const float r = o / l_run[e / hd];
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
__global__ __launch_bounds__(kBlock) void k_attn_combine(AttnArgs a) {
    const int g = blockIdx.x, z = blockIdx.y;
    const int hd = a.head_dim, G = a.n_heads / a.n_kv_heads;
    const int P = a.st ? a.st->pos + 1 : a.p0 + z + 1;
    const int S = a.n_split;
    int CH = (P + S - 1) / S;
    CH = (CH + 15) & ~15;
    const int n_active = (P + CH - 1) / CH;
    if (n_active == 1) return;
    const int stride = hd + 2, GH = G * hd, qd = a.n_heads * hd;
    const float* parts = a.part + (((size_t)z * a.n_kv_heads + g) * S) * (size_t)(G * stride);
    float* outz = a.out + (size_t)z * qd + (size_t)g * GH;
    for (int e = threadIdx.x; e < GH; e += kBlock) {
        const int h = e / hd, d = e % hd;
        float M = -INFINITY;
        for (int j = 0; j < n_active; j++) M = fmaxf(M, parts[(size_t)j * G * stride + h * stride]);
        float L = 0.f, O = 0.f;
        for (int j = 0; j < n_active; j++) {
            const float* pj = parts + (size_t)j * G * stride + h * stride;
            const float f = expf(pj[0] - M);
            L += pj[1] * f;
            O += pj[2 + d] * f;
        }
        const float r = O / L;
        outz[e] = r;
        if (a.out_h) a.out_h[(size_t)z * qd + (size_t)g * GH + e] = f2h(r);
    }
}

template <int G>
static hipError_t launch_attn_g(const AttnArgs& a, int n_q, hipStream_t s) {
    const size_t lds = ((size_t)G * kAttnChunk + (size_t)kWaves * G * a.head_dim) * sizeof(float);
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)k_attn<G>, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    hipLaunchKernelGGL((k_attn<G>), dim3(a.n_split, a.n_kv_heads, n_q), dim3(kBlock), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3(a.n_kv_heads, n_q), dim3(kBlock), 0, s, a);
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
