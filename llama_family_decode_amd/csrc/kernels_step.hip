// Persistent decode-step kernel for gfx950: one launch runs one token's whole
// forward pass ("The Forward Pass in Java", Project 18 forward(); "What a Llama
// model computes, and why", section 2) as a sequence of phases separated by
// grid-wide barriers, one 512-thread block per compute unit:
//   per layer: QKV (RMSNorm + products + bias + RoPE + F16 KV store) |
//   attention splits | split merge + output product + residual |
//   RMSNorm + gate/up + SwiGLU | down product + residual;
//   then RMSNorm + vocabulary product + argmax, and the token feedback.
// All blocks are co-resident (cooperative launch). Activations that cross
// blocks are written with agent-scope atomic stores, which reach the point of
// coherence of all the chip's L2 caches without writing back or invalidating
// any of them. Every activation buffer is versioned (one copy per layer, or
// per residual update), so within a launch an address is written once and
// read only after the barrier that follows the write: no cache can hold a
// stale copy of it (caches are invalidated at kernel start), and readers use
// ordinary cached, vectorised loads. A barrier counts arrivals in two levels,
// kBarGroup blocks per first-level counter and the last arrival of a group
// bumping the global counter; counters are never reset, so barrier j (counted
// over all launches) waits for the global count j * groups. Every wait is
// bounded: past the spin limit the block raises the abort flag, every later
// wait returns at once, and the host reports a device error.
#include "device_common.h"

namespace llm {

constexpr int kSpinLimit = 4 << 20;
constexpr int kSB = 512;       // threads per block
constexpr int kSW = kSB / 64;  // waves per block

__device__ __forceinline__ void stc(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier number `j` (counted over all launches) of the grid.
__device__ void grid_sync(State* st, unsigned long long* bar, unsigned long long j) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const int grp = blockIdx.x / kBarGroup, ngrp = (gridDim.x + kBarGroup - 1) / kBarGroup;
        const int gsize = min(kBarGroup, (int)gridDim.x - grp * kBarGroup);
        unsigned long long* gc = bar + (size_t)grp * kBarStride;
        unsigned long long* top = bar + (size_t)kBarGroups * kBarStride;
        const unsigned long long prev = __hip_atomic_fetch_add(gc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev + 1 == j * (unsigned long long)gsize)
            __hip_atomic_fetch_add(top, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long target = j * (unsigned long long)ngrp;
        int spins = 0;
        while (__hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(1);
            if ((++spins & 63) == 0) {
                if (__hip_atomic_load(&st->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
                if (spins > kSpinLimit) {
                    __hip_atomic_store(&st->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
    }
    __syncthreads();
}

// Block-wide sum of doubles in a fixed order; every thread gets the result.
__device__ __forceinline__ double block_sum_s(double v, double* red) {
    v = wave_sum_d(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kSW; w++) t += red[w];
    return t;
}

// Stage the input vector of a product in LDS (swizzled for weight type DT).
//   MODE 0: x = src.  MODE 1: x = rmsnorm(src) * gain ("The Forward Pass in
//   Java", Example 4: sum of squares in double, scale rounded to float once).
//   MODE 2: x = rmsnorm(E[tok]) * gain, and block 0 writes E[tok] to xres.
template <int DT, int MODE>
__device__ void stage_c(const float* src, const Mat* E, int tok, float* xres, const float* gain, float eps, int K,
                        float* xs, double* red) {
    const int tid = threadIdx.x;
    double ss = 0.0;
    for (int i = 4 * tid; i < K; i += 4 * kSB) {
        float4 v;
        if constexpr (MODE == 2) {
            v = make_float4(mat_elem(*E, tok, i), mat_elem(*E, tok, i + 1), mat_elem(*E, tok, i + 2),
                            mat_elem(*E, tok, i + 3));
            if (blockIdx.x == 0) {
                stc(xres + i, v.x);
                stc(xres + i + 1, v.y);
                stc(xres + i + 2, v.z);
                stc(xres + i + 3, v.w);
            }
        } else {
            v = *(const float4*)(src + i);
        }
        if constexpr (MODE != 0)
            ss += (double)v.x * (double)v.x + (double)v.y * (double)v.y + (double)v.z * (double)v.z +
                  (double)v.w * (double)v.w;
        *(float4*)(xs + swz<DT>(i)) = v;  // the swizzle keeps runs of 4 together
    }
    if constexpr (MODE != 0) {
        const double tot = block_sum_s(ss, red);
        const float scale = (float)(1.0 / sqrt(tot / (double)K + (double)eps));
        for (int i = tid; i < K; i += kSB) {
            const int j = swz<DT>(i);
            xs[j] = xs[j] * scale * gain[i];
        }
    }
    __syncthreads();
}

// acc[i] = row rows[i] of W dotted with the staged input (wave-wide sum).
template <int DT, int NR, int U>
__device__ __forceinline__ void gemv_group(const Mat& W, const int* rows, const float* xs, float (&acc)[NR]) {
    constexpr int VE = VecW<DT>::VE;
    const int lane = threadIdx.x & 63;
    const int nch = W.cols / VE;
    int lrow[NR];
#pragma unroll
    for (int i = 0; i < NR; i++) {
        lrow[i] = rows[i] < W.rows ? rows[i] : W.rows - 1;
        acc[i] = 0.f;
    }
    for (int c0 = lane; c0 < nch; c0 += 64 * U) {
        u32x4 raw[U][NR];
        float sc[U][NR];
        load_batch<DT, NR, U>(W, lrow, c0, nch, raw, sc);
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
}

// Attention splits of this step: S splits of CH positions (a multiple of 16)
// for P = pos + 1 cached positions.
__device__ __forceinline__ void attn_splits(int P, int& S, int& CH) {
    S = (P + 255) / 256;
    if (S > kStepMaxSplit) S = kStepMaxSplit;
    CH = (P + S - 1) / S;
    CH = (CH + 15) & ~15;
    S = (P + CH - 1) / CH;
}

// ------------------------------------------------------------------ phases
template <int DT>
__device__ void phase_qkv(const StepArgs& a, const LayerW& L, int layer, int pos, int tok, const float* xin,
                          float* x0, float* qkv, float* xs, double* red) {
    if (layer == 0)
        stage_c<DT, 2>(nullptr, &a.embd, tok, x0, L.attn_norm, a.eps, a.dim, xs, red);
    else
        stage_c<DT, 1>(xin, nullptr, 0, nullptr, L.attn_norm, a.eps, a.dim, xs, red);
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kSW + (threadIdx.x >> 6), nw = gridDim.x * kSW;
    const int hd = a.head_dim, hp = hd / 2, half = a.n_rot / 2;
    const int qd = a.n_heads * hd, kvd = a.n_kv_heads * hd;
    const int npairs = (qd + 2 * kvd) / 2;
    __half* kc = a.kc + (size_t)layer * a.kv_layer;
    __half* vc = a.vc + (size_t)layer * a.kv_layer;
    constexpr int U = DT == DT_Q8 ? 8 : 4;
    for (int pi = gw; pi < npairs; pi += nw) {
        const int head = pi / hp, j = pi % hp;
        int rows[2];
        if (j < half) {
            rows[0] = head * hd + (a.neox ? j : 2 * j);
            rows[1] = a.neox ? rows[0] + half : rows[0] + 1;
        } else {
            rows[0] = head * hd + a.n_rot + 2 * (j - half);
            rows[1] = rows[0] + 1;
        }
        float acc[2];
        gemv_group<DT, 2, U>(L.qkv, rows, xs, acc);
        if (lane == 0) {
            const int ra = rows[0], rb = rows[1];
            float va = acc[0], vb = acc[1];
            if (L.bqkv) {
                va += L.bqkv[ra];
                vb += L.bqkv[rb];
            }
            if (head < a.n_heads + a.n_kv_heads && j < half) {
                const float2 rv = rope_rotate(va, vb, a.rope[(size_t)pos * half + j]);
                va = rv.x;
                vb = rv.y;
            }
            stc(qkv + ra, va);
            stc(qkv + rb, vb);
            if (ra >= qd) {
                const bool isk = ra < qd + kvd;
                const int off = ra - qd - (isk ? 0 : kvd), offb = rb - qd - (isk ? 0 : kvd);
                const int g = off / hd;
                __half* row = (isk ? kc : vc) + ((size_t)g * a.n_ctx + pos) * hd;
                row[off % hd] = f2h(va);
                row[offb % hd] = f2h(vb);
            }
        }
    }
}

// Attention splits (see k_attn): item = kv_head * S + split writes that split's
// (m, l, unnormalised o) for the G query heads of its KV head. Row `pos` is
// taken from the q|k|v buffer of this step, rounded to binary16 as stored.
template <int G>
__device__ void phase_attn(const StepArgs& a, int layer, int pos, const float* qkv, float* part, float* sm,
                           float* m_run, float* l_run, float* alpha) {
    const int hd = a.head_dim, P = pos + 1;
    int S, CH;
    attn_splits(P, S, CH);
    const int qd = a.n_heads * hd, kvd = a.n_kv_heads * hd;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int LPP = attn_lpp(hd), PPI = kSB / LPP, CHUNK = PPI * kAttnSteps;
    const int sub = tid % LPP, pg = tid / LPP;
    const bool dim_ok = sub * 8 < hd;
    float* sc = sm;                   // [G][CHUNK]
    float* wred = sm + G * CHUNK;     // [kSW][G][hd]
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    for (int item = blockIdx.x; item < a.n_kv_heads * S; item += gridDim.x) {
        const int g = item / S, s = item % S;
        const int t_begin = s * CH, t_end = min(P, t_begin + CH);
        float qv[G][8], acc[G][8];
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int i = 0; i < 8; i++) {
                qv[h][i] = dim_ok ? qkv[(g * G + h) * hd + sub * 8 + i] : 0.f;
                acc[h][i] = 0.f;
            }
        __syncthreads();
        if (tid < G) {
            m_run[tid] = -INFINITY;
            l_run[tid] = 0.f;
        }
        const __half* kbase = a.kc + (size_t)layer * a.kv_layer + (size_t)g * a.n_ctx * hd + sub * 8;
        const __half* vbase = a.vc + (size_t)layer * a.kv_layer + (size_t)g * a.n_ctx * hd + sub * 8;
        for (int c0 = t_begin; c0 < t_end; c0 += CHUNK) {
            const int cn = min(CHUNK, t_end - c0);
            u32x4 kr[kAttnSteps], vr[kAttnSteps];
#pragma unroll
            for (int i = 0; i < kAttnSteps; i++) {
                const int t = pg + i * PPI;
                const bool ok = dim_ok && t < cn;
                if (ok && c0 + t == pos) {
                    uint32_t kw[4], vw[4];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const float* kp = qkv + qd + g * hd + sub * 8 + 2 * q;
                        const float* vp = qkv + qd + kvd + g * hd + sub * 8 + 2 * q;
                        kw[q] = (uint32_t)__half_as_ushort(f2h(kp[0])) | ((uint32_t)__half_as_ushort(f2h(kp[1])) << 16);
                        vw[q] = (uint32_t)__half_as_ushort(f2h(vp[0])) | ((uint32_t)__half_as_ushort(f2h(vp[1])) << 16);
                    }
                    kr[i] = (u32x4){kw[0], kw[1], kw[2], kw[3]};
                    vr[i] = (u32x4){vw[0], vw[1], vw[2], vw[3]};
                } else {
                    kr[i] = ok ? *(const u32x4*)(kbase + (size_t)(c0 + t) * hd) : z4;
                    vr[i] = ok ? *(const u32x4*)(vbase + (size_t)(c0 + t) * hd) : z4;
                }
            }
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
            for (int h = wave; h < G; h += kSW) {
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
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float al = alpha[h];
#pragma unroll
                for (int i = 0; i < 8; i++) acc[h][i] *= al;
            }
#pragma unroll
            for (int i = 0; i < kAttnSteps; i++) {
                const int t = pg + i * PPI;
                if (dim_ok && t < cn) {
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
        const int GH = G * hd, stride = hd + 2;
        float* mypart = part + ((size_t)g * S + s) * (size_t)(G * stride);
        for (int e = tid; e < GH; e += kSB) {
            float o = 0.f;
#pragma unroll
            for (int w = 0; w < kSW; w++) o += wred[w * GH + e];
            stc(mypart + (e / hd) * stride + 2 + (e % hd), o);
        }
        if (tid < G) {
            stc(mypart + tid * stride, m_run[tid]);
            stc(mypart + tid * stride + 1, l_run[tid]);
        }
        __syncthreads();
    }
}

// Output stage: every block merges the attention splits of all heads into the
// staged input (M = max m_s, L = sum l_s e^(m_s - M), o = sum o_s e^(m_s - M) /
// L, splits in order), then x_mid[r] = x_in[r] + W_o o for its rows.
template <int DT, int G>
__device__ void phase_o(const StepArgs& a, const LayerW& L, int pos, const float* part, const float* xprev,
                        float* xnext, float* xs, float* wsp) {
    const int hd = a.head_dim, H = a.n_heads, qd = H * hd, stride = hd + 2;
    int S, CH;
    attn_splits(pos + 1, S, CH);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // per (head, split) weights e^(m_s - M) / L into wsp[h * S + s]
    for (int h = wave; h < H; h += kSW) {
        const int g = h / G, hl = h % G;
        float m = -INFINITY, l = 0.f;
        if (lane < S) {
            const float* pj = part + ((size_t)g * S + lane) * (size_t)(G * stride) + hl * stride;
            m = pj[0];
            l = pj[1];
        }
        const float M = wave_max(m);
        const float f = lane < S ? expf(m - M) : 0.f;
        const float Lh = wave_sum(l * f);
        if (lane < S) wsp[h * S + lane] = f / Lh;
    }
    __syncthreads();
    for (int e = tid; e < qd; e += kSB) {
        const int h = e / hd, d = e % hd, g = h / G, hl = h % G;
        const float* po = part + (size_t)g * S * (size_t)(G * stride) + hl * stride + 2 + d;
        float o = 0.f;
        for (int s = 0; s < S; s++) o += wsp[h * S + s] * po[(size_t)s * G * stride];
        xs[swz<DT>(e)] = o;
    }
    __syncthreads();
    const int gw = blockIdx.x * kSW + wave, nw = gridDim.x * kSW;
    constexpr int U = DT == DT_Q8 ? 8 : 4;
    for (int r = gw; r < L.o.rows; r += nw) {
        const int rows[1] = {r};
        float acc[1];
        gemv_group<DT, 1, U>(L.o, rows, xs, acc);
        if (lane == 0) stc(xnext + r, xprev[r] + acc[0]);
    }
}

// x_out[r] = x_mid[r] + W_down u for the block's rows.
template <int DT>
__device__ void phase_down(const StepArgs& a, const Mat& W, const float* u, const float* xprev, float* xnext,
                           float* xs, double* red) {
    stage_c<DT, 0>(u, nullptr, 0, nullptr, nullptr, 0.f, W.cols, xs, red);
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kSW + (threadIdx.x >> 6), nw = gridDim.x * kSW;
    constexpr int U = DT == DT_Q8 ? 8 : 4;
    for (int r = gw; r < W.rows; r += nw) {
        const int rows[1] = {r};
        float acc[1];
        gemv_group<DT, 1, U>(W, rows, xs, acc);
        if (lane == 0) stc(xnext + r, xprev[r] + acc[0]);
    }
}

template <int DT>
__device__ void phase_gateup(const StepArgs& a, const LayerW& L, const float* xin, float* u, float* xs, double* red) {
    stage_c<DT, 1>(xin, nullptr, 0, nullptr, L.ffn_norm, a.eps, a.dim, xs, red);
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kSW + (threadIdx.x >> 6), nw = gridDim.x * kSW;
    const int ng = L.gu.rows / 4;
    for (int g = gw; g < ng; g += nw) {
        const int rows[4] = {4 * g, 4 * g + 1, 4 * g + 2, 4 * g + 3};
        float acc[4];
        gemv_group<DT, 4, 4>(L.gu, rows, xs, acc);
        if (lane == 0) {
            stc(u + 2 * g, silu(acc[0]) * acc[1]);
            stc(u + 2 * g + 1, silu(acc[2]) * acc[3]);
        }
    }
}

template <int DT>
__device__ void phase_logits(const StepArgs& a, const float* xin, float* xs, double* red, ArgPart* wbest) {
    stage_c<DT, 1>(xin, nullptr, 0, nullptr, a.out_norm, a.eps, a.dim, xs, red);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gw = blockIdx.x * kSW + wave, nw = gridDim.x * kSW;
    const int R = a.out.rows, ng = (R + 3) / 4;
    float best = -INFINITY;
    int best_i = 0x7fffffff, nonfinite = 0;
    for (int g = gw; g < ng; g += nw) {
        const int rows[4] = {4 * g, 4 * g + 1, 4 * g + 2, 4 * g + 3};
        float acc[4];
        gemv_group<DT, 4, 4>(a.out, rows, xs, acc);
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (rows[i] < R) {
                    const float v = acc[i];
                    a.logits[rows[i]] = v;
                    if (!isfinite(v)) nonfinite = 1;
                    if (v > best) {  // rows arrive in increasing order: ties keep the first
                        best = v;
                        best_i = rows[i];
                    }
                }
            }
        }
    }
    if (lane == 0) wbest[wave] = ArgPart{best, best_i, nonfinite, 0};
    __syncthreads();
    if (threadIdx.x == 0) {
        ArgPart b = wbest[0];
        for (int w = 1; w < kSW; w++) {
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

template <int G>
__global__ __launch_bounds__(kSB, 1) void k_step(StepArgs a) {
    extern __shared__ float sm[];
    __shared__ double red[kSW];
    __shared__ ArgPart wbest[kSW];
    __shared__ float m_run[kMaxGroup], l_run[kMaxGroup], alpha[kMaxGroup];

    State* st = a.st;
    const int pos = st->pos, tok = st->token, epoch = st->epoch;
    const unsigned long long nb = (unsigned long long)kStepPhases * a.n_layers + 1;
    unsigned long long bar = (unsigned long long)epoch * nb;
    int phase = 0;
    if (a.trace && blockIdx.x == 0 && threadIdx.x == 0) a.trace[0] = wall_clock64();
#define STEP_SYNC()                                                                          \
    do {                                                                                     \
        grid_sync(st, a.bar, ++bar);                                                         \
        ++phase;                                                                             \
        if (a.trace && blockIdx.x == 0 && threadIdx.x == 0) a.trace[phase] = wall_clock64(); \
    } while (0)
#define BY_DTYPE(M, CALL)                 \
    switch ((M).dtype) {                  \
        case DT_F32: CALL(DT_F32); break; \
        case DT_F16: CALL(DT_F16); break; \
        default: CALL(DT_Q8); break;      \
    }

    // LDS: the staged input vector; the output stage keeps its split weights
    // past the largest attention output it stages.
    float* wsp = sm + lds_floats<DT_Q8>(a.n_heads * a.head_dim);
    for (int l = 0; l < a.n_layers; l++) {
        const LayerW L = a.layers[l];
        const float* x_in = a.xv + (size_t)(2 * l) * a.xstride;  // residual entering the layer
        float* x_mid = a.xv + (size_t)(2 * l + 1) * a.xstride;   // after attention
        float* x_out = a.xv + (size_t)(2 * l + 2) * a.xstride;   // after the FFN
        float* qkv = a.qkv + (size_t)l * a.qkv_stride;
        float* part = a.part + (size_t)l * a.part_stride;
        float* u = a.u + (size_t)l * a.u_stride;
#define QKV(D) phase_qkv<D>(a, L, l, pos, tok, x_in, a.xv, qkv, sm, red)
        BY_DTYPE(L.qkv, QKV)
        STEP_SYNC();
        phase_attn<G>(a, l, pos, qkv, part, sm, m_run, l_run, alpha);
        STEP_SYNC();
#define OPROJ(D) phase_o<D, G>(a, L, pos, part, x_in, x_mid, sm, wsp)
        BY_DTYPE(L.o, OPROJ)
        STEP_SYNC();
#define GATEUP(D) phase_gateup<D>(a, L, x_mid, u, sm, red)
        BY_DTYPE(L.gu, GATEUP)
        STEP_SYNC();
#define DOWN(D) phase_down<D>(a, L.down, u, x_mid, x_out, sm, red)
        BY_DTYPE(L.down, DOWN)
        STEP_SYNC();
    }
    const float* x_last = a.xv + (size_t)(2 * a.n_layers) * a.xstride;
#define LOGITS(D) phase_logits<D>(a, x_last, sm, red, wbest)
    BY_DTYPE(a.out, LOGITS)
    STEP_SYNC();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const unsigned long long k = __hip_atomic_load(&st->best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int next = k ? (int)(0xffffffffu - (uint32_t)(k & 0xffffffffull)) : 0;
        st->next = next;
        if (st->gen_mode) {
            const int c = st->gen_count;
            if (c < a.gen_cap) a.gen_out[c] = next;
            st->gen_count = c + 1;
            st->token = next;
            st->pos = pos + 1;
        }
        __hip_atomic_store(&st->best, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        st->epoch = epoch + 1;
    }
#undef STEP_SYNC
#undef BY_DTYPE
#undef QKV
#undef OPROJ
#undef GATEUP
#undef DOWN
#undef LOGITS
}

static int step_lds_bytes(const StepArgs& a) {
    int maxk = a.dim;
    if (a.n_heads * a.head_dim > maxk) maxk = a.n_heads * a.head_dim;
    if (a.ffn > maxk) maxk = a.ffn;
    const int G = a.n_heads / a.n_kv_heads;
    int f = lds_floats<DT_Q8>(maxk);  // the largest swizzle round-up of the three types
    const int att = G * (kSB / attn_lpp(a.head_dim)) * kAttnSteps + kSW * G * a.head_dim;
    const int ost = lds_floats<DT_Q8>(a.n_heads * a.head_dim) + a.n_heads * kStepMaxSplit;  // staged o + split weights
    if (att > f) f = att;
    if (ost > f) f = ost;
    return f * (int)sizeof(float);
}

template <int G>
static int step_grid_g(const StepArgs& a, int lds) {
    static bool attr_done = false;
    if (!attr_done) {
        if (hipFuncSetAttribute((const void*)k_step<G>, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
            return 0;
        attr_done = true;
    }
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_step<G>, kSB, lds) != hipSuccess)
        return 0;
    return per_cu >= 1 ? cus : 0;
}

int step_grid(const StepArgs& a, int* lds_bytes) {
    const int lds = step_lds_bytes(a);
    *lds_bytes = lds;
    switch (a.n_heads / a.n_kv_heads) {
        case 1: return step_grid_g<1>(a, lds);
        case 2: return step_grid_g<2>(a, lds);
        case 4: return step_grid_g<4>(a, lds);
        case 8: return step_grid_g<8>(a, lds);
    }
    return 0;
}

template <int G>
static hipError_t launch_step_g(const StepArgs& a, int grid, int lds, hipStream_t s) {
    StepArgs arg = a;
    void* params[] = {&arg};
    return hipLaunchCooperativeKernel((const void*)k_step<G>, dim3(grid), dim3(kSB), params, (unsigned)lds, s);
}

hipError_t launch_step(const StepArgs& a, int grid, int lds, hipStream_t s) {
    switch (a.n_heads / a.n_kv_heads) {
        case 1: return launch_step_g<1>(a, grid, lds, s);
        case 2: return launch_step_g<2>(a, grid, lds, s);
        case 4: return launch_step_g<4>(a, grid, lds, s);
        case 8: return launch_step_g<8>(a, grid, lds, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace llm
