// Persistent decode-step kernel for gfx950: one launch runs one
// token's whole forward pass ("The Forward Pass in Java", Project 18
// forward(); "What a Llama model computes, and why", section 2), one 512-thread
// block per compute unit.
//
// The grid is split into 8 groups of blocks (block b in group b % 8, which is
// how the dispatcher deals blocks to the chip's 8 XCDs, so a group shares one
// L2). The groups split every layer the way tensor-parallel devices would:
// group x owns a contiguous share of the KV heads (with their query heads) and
// a contiguous share of the FFN hidden units. Per layer:
//   QKV    every block normalises its own copy of the residual; the group
//          computes the q/k/v rows of its heads (+ bias, RoPE, F16 KV store)
//   | group barrier |
//   ATTN   the group's blocks split the cached positions of its KV heads
//   | group barrier |
//   O      every block of the group merges the splits, then the group computes
//          the output product over its heads' columns: a partial sum of W_o o
//   | all-group barrier |
//   GU     every block adds the 8 partial sums to its residual copy (fixed
//          order), normalises; the group computes gate/up of its hidden units
//          and SwiGLU
//   | group barrier |
//   DOWN   the group computes W_down u over its hidden units: a partial sum
//   | all-group barrier |, after which every block adds the partials.
// Then every block takes a share of the vocabulary rows (final RMSNorm,
// product, argmax), and a last all-group barrier precedes the token feedback.
//
// Memory ordering. Values that cross blocks are written with agent-scope
// atomic stores (they reach the coherence point of all L2 caches without
// flushing any cache) into buffers with one copy per layer, so within a launch
// an address is written once and read only after the barrier that follows the
// write; readers then use ordinary cached loads (caches are invalidated at
// kernel start, and no cache line is shared between two buffers). A barrier
// arrival is an atomic add without return, issued only after the block's
// stores have completed. The weights of the next phase do not depend on any
// activation, so each wave issues their loads right after the arrival: they
// stream from HBM while the barrier completes. Counters are never reset:
// barrier j (counted over all launches) waits for j arrivals per group block.
// Every wait is bounded: past the spin limit a block raises the abort flag,
// later waits return at once, and the host reports a device error.
#include "device_common.h"

namespace llm {

static_assert(sizeof(LayerW) % 8 == 0, "the layer table is copied in 8-byte words");
constexpr int kSpinLimit = 4 << 20;
constexpr int kSB = 512;       // threads per block
constexpr int kSW = kSB / 64;  // waves per block
constexpr int kNG = kStepGroups;
constexpr int kPF = 16;        // 16-byte weight chunks a lane holds per batch
constexpr int kStepAttn = 2;   // position steps of 64 threads-groups per attention chunk

typedef unsigned long long u64;

// Compile-time geometry of one product phase: rows read by 2^L lanes, N column
// batches per row; Geo<0, 0> leaves both to the run-time shape.
template <int L_, int N_>
struct Geo {
    static constexpr int L = L_, N = N_;
};
using GeoRT = Geo<0, 0>;

// Stores of values other blocks read after a barrier. Values read only by
// the writer's own group (q|k|v, the SwiGLU output, the attention splits)
// stay in that group's L2: a group's blocks all run on one XCD (the blocks b
// with equal b mod 8, checked at load by step_groups_share_l2), the store has
// reached L2 once the writer's wait_mem returns, and the readers' L1 holds no
// copy (each per-layer buffer is read once per launch, after its write).
// Values every group reads (the output and down partial sums) are written
// through to the device coherence point.
__device__ __forceinline__ void stc(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stl(float* p, float v) { *(__attribute__((address_space(1))) float*)p = v; }
__device__ __forceinline__ u64 ldc(u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void arrive(u64* p) {
    (void)__hip_atomic_fetch_add(p, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this wave's stores (and loads) have completed; also a compiler
// barrier, so no memory access moves across it.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void pin() { asm volatile("" ::: "memory"); }
// The lane index, opaque to the optimiser: address arithmetic derived from it
// is redone at each use instead of being hoisted out of the layer loop (where
// the same values for every layer would stay live in registers).
__device__ __forceinline__ int lane_id() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}
__device__ __forceinline__ int thread_id() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}
// Loads through global-address-space pointers: weights and activations live in
// device memory, and global (not flat) loads count only against the vector
// memory counter, so LDS waits never wait for weight loads in flight.
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const uint16_t g_u16;
typedef __attribute__((address_space(1))) const float g_f32;
__device__ __forceinline__ u32x4 ld_nt(const void* p) { return __builtin_nontemporal_load((g_u32x4*)p); }
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(g_u32x4*)p; }
__device__ __forceinline__ uint32_t ld_u16(const uint16_t* p) { return *(g_u16*)p; }
__device__ __forceinline__ float ldf(const float* p) { return *(g_f32*)p; }
__device__ __forceinline__ float4 ldf4(const float* p) {
    const u32x4 v = ld16(p);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// A wave-uniform value made opaque the same way (kept in a scalar register).
__device__ __forceinline__ int opaque_s(int v) {
    v = __builtin_amdgcn_readfirstlane(v);
    asm volatile("" : "+s"(v));
    return v;
}

__device__ __forceinline__ bool aborted(State* st) {
    return __hip_atomic_load(&st->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}
__device__ __forceinline__ void raise_abort(State* st) {
    __hip_atomic_store(&st->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counter slots (kBarStride u64 apart): group barrier counters 0..7, all-group
// arrival counters 8..15.
__device__ __forceinline__ u64* lcount(const StepArgs& a, int x) { return a.bar + (size_t)x * kBarStride; }
__device__ __forceinline__ u64* gcount(const StepArgs& a, int x) { return a.bar + (size_t)(kNG + x) * kBarStride; }

// Group barrier, first half: all stores of the block have completed (every
// wave ran wait_mem), then one arrival.
__device__ __forceinline__ void group_arrive(const StepArgs& a, int x) {
    __syncthreads();
    if (threadIdx.x == 0) arrive(lcount(a, x));
}
__device__ __forceinline__ void all_arrive(const StepArgs& a, int x) {
    __syncthreads();
    if (threadIdx.x == 0) arrive(gcount(a, x));
}
// Second half: wait for `target` arrivals on the group's counter.
__device__ __forceinline__ void group_wait(const StepArgs& a, int x, u64 target) {
    if (threadIdx.x == 0) {
        u64* c = lcount(a, x);
        int spins = 0;
        while (ldc(c) < target) {
            __builtin_amdgcn_s_sleep(1);
            if ((++spins & 63) == 0) {
                if (aborted(a.st)) break;
                if (spins > kSpinLimit) {
                    raise_abort(a.st);
                    break;
                }
            }
        }
    }
    __syncthreads();
}
// Wait until every group's counter reached `target`: lane i of wave 0 polls
// group i's counter, all 8 in one load.
__device__ __forceinline__ void all_wait(const StepArgs& a, u64 target) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        u64* c = gcount(a, lane & (kNG - 1));
        int spins = 0;
        while (true) {
            const u64 v = lane < kNG ? ldc(c) : target;
            if (__all(v >= target)) break;
            __builtin_amdgcn_s_sleep(1);
            if ((++spins & 63) == 0) {
                if (aborted(a.st)) break;
                if (spins > kSpinLimit) {
                    if (lane == 0) raise_abort(a.st);
                    break;
                }
            }
        }
    }
    __syncthreads();
}

// Sum / max over all 64 lanes (every lane gets the result), in the same
// butterfly order as a plain xor reduction from offset 32 down to 1.
template <class T>
__device__ __forceinline__ T xsum64(T v) {
    v += xshfl<32>(v);
    v += xshfl<16>(v);
    v += xshfl<8>(v);
    v += xshfl<4>(v);
    v += xshfl<2>(v);
    v += xshfl<1>(v);
    return v;
}
__device__ __forceinline__ float xmax64(float v) {
    v = fmaxf(v, xshfl<32>(v));
    v = fmaxf(v, xshfl<16>(v));
    v = fmaxf(v, xshfl<8>(v));
    v = fmaxf(v, xshfl<4>(v));
    v = fmaxf(v, xshfl<2>(v));
    v = fmaxf(v, xshfl<1>(v));
    return v;
}

// v summed over lanes that differ in the bits of [lo, hi) (powers of two),
// from the low offsets up, with uniform conditions.
__device__ __forceinline__ float lane_sum(float v, int lo, int hi) {
    if (lo <= 1 && 1 < hi) v += xshfl<1>(v);
    if (lo <= 2 && 2 < hi) v += xshfl<2>(v);
    if (lo <= 4 && 4 < hi) v += xshfl<4>(v);
    if (lo <= 8 && 8 < hi) v += xshfl<8>(v);
    if (lo <= 16 && 16 < hi) v += xshfl<16>(v);
    if (lo <= 32 && 32 < hi) v += xshfl<32>(v);
    return v;
}
// Each of the N values summed over lanes that differ in the bits of [lo, hi):
// every step is applied to all N values before the next, so the exchanges of
// independent values overlap.
template <int N>
__device__ __forceinline__ void lanes_sum_all(float* v, int lo, int hi) {
#define LSA_STEP(M)                                          \
    if (lo <= (M) && (M) < hi) {                             \
        _Pragma("unroll") for (int i = 0; i < N; i++) v[i] += xshfl<M>(v[i]); \
    }
    LSA_STEP(1)
    LSA_STEP(2)
    LSA_STEP(4)
    LSA_STEP(8)
    LSA_STEP(16)
    LSA_STEP(32)
#undef LSA_STEP
}

// The same from the high offsets down (the order of a reduction over a row's
// lpr lanes).
__device__ __forceinline__ float lane_sum_down(float v, int lpr) {
    if (lpr > 32) v += xshfl<32>(v);
    if (lpr > 16) v += xshfl<16>(v);
    if (lpr > 8) v += xshfl<8>(v);
    if (lpr > 4) v += xshfl<4>(v);
    if (lpr > 2) v += xshfl<2>(v);
    if (lpr > 1) v += xshfl<1>(v);
    return v;
}

// Block-wide sum of doubles in a fixed order; every thread gets the result.
__device__ __forceinline__ double block_sum_s(double v, double* red) {
    v = xsum64(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kSW; w++) t += red[w];
    return t;
}

// xs (swizzled for weight type DT) = rmsnorm(xr) * gain over K elements
// ("The Forward Pass in Java", Example 4: sum of squares in double, the scale
// rounded to float once, then x * scale * gain). Thread t owns the elements
// 4t .. 4t+3 (+ multiples of 4 * kSB): it sums their squares and writes their
// outputs.
// The gain elements 4t .. 4t+3 of the next RMSNorm, loaded ahead of the
// barrier that precedes it.
struct GainPF {
    float4 g;
};
__device__ __forceinline__ void gain_load(GainPF& gp, const float* gain, int K) {
    const int i = 4 * thread_id();
    gp.g = i < K ? ldf4(gain + i) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// xs[swz(i .. i+3)] = v * scale * g
template <int DT>
__device__ __forceinline__ void norm_store4(float* xs, int i, float4 v, float scale, float4 g) {
    float4 o;
    o.x = v.x * scale * g.x;
    o.y = v.y * scale * g.y;
    o.z = v.z * scale * g.z;
    o.w = v.w * scale * g.w;
    *(float4*)(xs + swz<DT>(i)) = o;
}

__device__ __forceinline__ double sq4(float4 v) {
    return (double)v.x * (double)v.x + (double)v.y * (double)v.y + (double)v.z * (double)v.z +
           (double)v.w * (double)v.w;
}

template <int DT>
__device__ __forceinline__ void stage_norm(const float* xr, const float* gain, const GainPF& gp, float eps, int K,
                                           float* xs, double* red) {
    const int tid = thread_id();
    double ss = 0.0;
    for (int i = 4 * tid; i < K; i += 4 * kSB) ss += sq4(*(const float4*)(xr + i));
    const double tot = block_sum_s(ss, red);
    const float scale = (float)(1.0 / sqrt(tot / (double)K + (double)eps));
    for (int i = 4 * tid; i < K; i += 4 * kSB)
        norm_store4<DT>(xs, i, *(const float4*)(xr + i), scale, i == 4 * tid ? gp.g : ldf4(gain + i));
    __syncthreads();
}

// xs (swizzled) = src[0..K), K a multiple of 4.
template <int DT>
__device__ __forceinline__ void stage_copy(const float* src, int K, float* xs) {
    for (int i = 4 * thread_id(); i < K; i += 4 * kSB) *(float4*)(xs + swz<DT>(i)) = ldf4(src + i);
    __syncthreads();
}

// The rounding mode's product input (llama.cpp's rounding points, "What a
// Llama model computes, and why", section 8, with the Q8_0 quantizer of
// "Loading GGUF with the FFM API", Example 8):
// for Q8_0 weights each 32-element block of the staged input becomes its Q8_0
// encoding decoded again (scale max|x|/127 rounded to binary16 after the
// codes are taken), for F16 weights each element its binary16 value; F32
// weights take the input as it is. K is a multiple of 32 and the staged input
// starts at a block boundary, so the 32 lanes of a half-wave hold one block.
// Maximum over the 32 lanes of a half-wave (one Q8_0 block): DPP quad
// permutes and swizzles, none of which computes an LDS address.
__device__ __forceinline__ float half_wave_max(float v) {
    v = fmaxf(v, xshfl<1>(v));
    v = fmaxf(v, xshfl<2>(v));
    v = fmaxf(v, xshfl<4>(v));
    v = fmaxf(v, xshfl<8>(v));
    return fmaxf(v, xshfl<16>(v));
}

template <int DT>
__device__ __forceinline__ void round_input(float* xs, int K) {
    if constexpr (DT != DT_F32) {
        for (int i = thread_id(); i < K; i += kSB) {
            float v = xs[swz<DT>(i)];
            if constexpr (DT == DT_Q8) {
                const float amax = half_wave_max(fabsf(v));
                const float d = amax / 127.f, id = d != 0.f ? 1.f / d : 0.f;
                v = round16(d) * roundf(v * id);
            } else {
                v = round16(v);
            }
            xs[swz<DT>(i)] = v;
        }
        __syncthreads();
    }
}

// v += the contributing groups' partial sums P[g][i .. i+3], groups in order.
__device__ __forceinline__ float4 add4_partials(float4 v, const float* P, long long pstride, int i, unsigned gmask) {
    float4 p[kNG];
#pragma unroll
    for (int g = 0; g < kNG; g++)
        p[g] = (gmask >> g) & 1 ? ldf4(P + g * pstride + i) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int g = 0; g < kNG; g++)
        if ((gmask >> g) & 1) {
            v.x += p[g].x;
            v.y += p[g].y;
            v.z += p[g].z;
            v.w += p[g].w;
        }
    return v;
}

// The rounding mode's Q8_0 product input for the integer products: each
// 32-element block of the staged input quantized as round_input does (the
// same codes and binary16 scale), kept as codes and scales (XChunkI8's
// layout) instead of their decoded values. Thread t takes elements
// t + j * kSB, j < 4, so K <= 4 * kSB (the kernels compiled for one shape).
__device__ __forceinline__ void round_input_i8(float* xs, int K) {
    const int tid = thread_id();
    int code[4];
    float dsc[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int i = tid + j * kSB;
        code[j] = 0;
        dsc[j] = 0.f;
        if (i < K) {  // whole half-waves: K is a multiple of 32
            const float v = xs[swz<DT_Q8>(i)];
            const float amax = half_wave_max(fabsf(v));
            const float d = amax / 127.f, id = d != 0.f ? 1.f / d : 0.f;
            code[j] = (int)roundf(v * id);
            dsc[j] = round16(d);
        }
    }
    __syncthreads();  // every float of the staged input has been read
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int i = tid + j * kSB;
        if (i < K) {
            ((int8_t*)xs)[i] = (int8_t)code[j];
            if ((i & 31) == 0) (xs + K / 4)[i >> 5] = dsc[j];
        }
    }
    __syncthreads();
}

// xr[i] += sum over the groups that contributed of P[g][i], groups in order.
__device__ __forceinline__ void add_partials(float* xr, const float* P, long long pstride, int dim, unsigned gmask) {
    for (int i = 4 * thread_id(); i < dim; i += 4 * kSB)
        *(float4*)(xr + i) = add4_partials(*(const float4*)(xr + i), P, pstride, i, gmask);
    __syncthreads();
}

// add_partials, then stage_norm with `gain`, in one pass: each thread keeps the
// residual elements it updates and normalises them itself.
template <int DT>
__device__ __forceinline__ void add_partials_norm(float* xr, const float* P, long long pstride, int dim, unsigned gmask,
                                                  const float* gain, const GainPF& gp, float eps, float* xs,
                                                  double* red) {
    const int tid = thread_id();
    double ss = 0.0;
    float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 4 * tid; i < dim; i += 4 * kSB) {
        const float4 v = add4_partials(*(const float4*)(xr + i), P, pstride, i, gmask);
        *(float4*)(xr + i) = v;
        if (i == 4 * tid) v0 = v;
        ss += sq4(v);
    }
    const double tot = block_sum_s(ss, red);
    const float scale = (float)(1.0 / sqrt(tot / (double)dim + (double)eps));
    for (int i = 4 * tid; i < dim; i += 4 * kSB)
        norm_store4<DT>(xs, i, i == 4 * tid ? v0 : *(const float4*)(xr + i), scale,
                        i == 4 * tid ? gp.g : ldf4(gain + i));
    __syncthreads();
}

// ------------------------------------------------------ row-parallel products
// A column window of a weight matrix: row r's window starts at w + r*ld
// elements; Q8_0 scales of the window start at s + r*(ld/32).
struct Win {
    const char* w;
    const uint16_t* s;
    long long ld;
    int nch;  // 16-byte chunks per row in the window
};

template <int DT>
__device__ __forceinline__ Win make_win(const Mat& M, int col0, int ncols) {
    constexpr int ES = DT == DT_F32 ? 4 : (DT == DT_F16 ? 2 : 1);
    Win v;
    v.w = (const char*)M.w + (size_t)col0 * ES;
    v.s = DT == DT_Q8 ? M.s + col0 / 32 : nullptr;
    v.ld = M.cols;
    v.nch = ncols / VecW<DT>::VE;
    return v;
}

// One wave's rows [r0, r1) of a product. A row is read by lpr lanes (a power
// of two, 64 unless the window is short), so rpi = 64 / lpr rows share one
// wave-wide load. The wave walks slots: slot k covers row group k / ncb (rpi
// rows) and column batch k % ncb, in which lane l reads chunk l % lpr + lpr *
// batch of row l / lpr of the group. A lane holds kPF slots at a time.
struct WRows {
    Win W;
    int r0, r1;
    int lpr, lsh, rpi, ncb, nslots;
};

__device__ __forceinline__ WRows wave_rows(int n, int nwaves, int wv, int nch, bool pairs) {
    WRows w;
    w.lpr = 64;
    w.lsh = 6;
    if (nch < 64) {
        w.lpr = 1;
        w.lsh = 0;
        while (w.lpr < nch) {
            w.lpr <<= 1;
            w.lsh++;
        }
    }
    w.rpi = 64 >> w.lsh;
    w.ncb = nch > 0 ? (nch + w.lpr - 1) >> w.lsh : 1;
    const int unit = pairs ? 2 * w.rpi : w.rpi;
    int per = (n + nwaves - 1) / nwaves;
    per = (per + unit - 1) / unit * unit;
    w.r0 = wv * per;
    w.r1 = min(n, w.r0 + per);
    if (nch <= 0 || w.r1 < w.r0) w.r1 = w.r0;
    w.nslots = (w.r1 - w.r0 + w.rpi - 1) / w.rpi * w.ncb;
    return w;
}

struct PF {
    u32x4 q[kPF];
    uint32_t s[kPF];  // raw binary16 scales (Q8_0)
};

// A wave with no rows still redefines its buffer, so that no older contents
// stay live across the phases in between.
__device__ __forceinline__ void pf_clear(PF& pf) {
#pragma unroll
    for (int i = 0; i < kPF; i++) {
        pf.q[i] = (u32x4){0u, 0u, 0u, 0u};
        pf.s[i] = 0u;
    }
}

// Issues the loads of slots k0 .. k0 + kPF - 1 (those below nslots) into pf.
// Rows and chunks past the window are clamped to valid ones; wdot ignores
// their values.
// Nothing here waits for the data. rmap (or nullptr) maps wave rows to matrix
// rows, else matrix row = roff + row.
template <int DT>
__device__ __forceinline__ void wload(const WRows& w, const int* rmap, int roff, int k0, PF& pf) {
    constexpr int ES = DT == DT_F32 ? 4 : (DT == DT_F16 ? 2 : 1);
    if (w.nslots == 0) {
        pf_clear(pf);
        return;
    }
    const int lane = lane_id(), sub = lane >> w.lsh, cl = lane & (w.lpr - 1);
    k0 = opaque_s(k0);
    int g = k0 / w.ncb, cb = k0 - g * w.ncb;
#pragma unroll
    for (int k = 0; k < kPF; k++) {
        if (k0 + k < w.nslots) {  // wave-uniform; slots past the wave's rows load nothing
            int row = w.r0 + g * w.rpi + sub;
            row = row < w.r1 ? row : w.r1 - 1;
            const long long ar = rmap ? rmap[row] : roff + row;
            int c = cl + (cb << w.lsh);
            c = c < w.W.nch ? c : w.W.nch - 1;
            pf.q[k] = ld_nt(w.W.w + (ar * w.W.ld * ES + (long long)c * 16));
            if constexpr (DT == DT_Q8) pf.s[k] = ld_u16(w.W.s + (ar * (w.W.ld / 32) + (c >> 1)));
        } else {
            pf.q[k] = (u32x4){0u, 0u, 0u, 0u};
            pf.s[k] = 0u;
        }
        if (++cb == w.ncb) {
            cb = 0;
            ++g;
        }
    }
}

// Kinds of what a product's rows become.
enum StepEmit : int {
    EM_PART = 0,    // P[row] = value (a partial sum of a K-split product)
    EM_QKV = 1,     // RoPE pairs of q/k/v: bias, rotation, qkv buffer, F16 cache
    EM_SWIGLU = 2,  // gate/up pairs: u[row / 2] = silu(gate) * up
    EM_ARGMAX = 3,  // vocabulary rows: logits and the running first maximum
};

struct EmitArgs {
    float* out;
    const float* bias;
    const float2* cs;  // (cos, sin) of this step's position, pair j at cs[j] (LDS)
    __half* kc;
    __half* vc;
    int pos, n_ctx, hd, qd, kvd, half, n_rot, neox;
};

// q/k/v pair (matrix rows ra < rb): bias, RoPE at pos on q and k ("The Forward
// Pass in Java", Example 6), q|k|v -> qkv buffer, k and v -> binary16 cache
// row pos (Example 10).
__device__ __forceinline__ void emit_qkv(const EmitArgs& e, int ra, int rb, float va, float vb) {
    const int kind = ra < e.qd ? 0 : (ra < e.qd + e.kvd ? 1 : 2);
    const int base = kind == 0 ? 0 : (kind == 1 ? e.qd : e.qd + e.kvd);
    const int head = (ra - base) / e.hd, d = ra - base - head * e.hd;
    if (e.bias) {
        va += ldf(e.bias + ra);
        vb += ldf(e.bias + rb);
    }
    if (kind < 2 && d < e.n_rot) {
        const int j = e.neox ? d : d >> 1;
        const float2 r = rope_rotate(va, vb, e.cs[j]);
        va = r.x;
        vb = r.y;
    }
    stl(e.out + ra, va);
    stl(e.out + rb, vb);
    if (kind > 0) {
        __half* row = (kind == 1 ? e.kc : e.vc) + ((size_t)head * e.n_ctx + e.pos) * e.hd;
        row[d] = f2h(va);
        row[rb - base - head * e.hd] = f2h(vb);
    }
}

// One batch of kPF slots starting at slot k0: dot products with the staged
// input xs, summed over the lane's column batches of a row group (acc carries
// a group into the next batch) and then over the group's lpr lanes, then
// emitted. FULL: every slot, row and chunk of the batch is in range.
template <int DT, int EM, bool FULL>
__device__ __forceinline__ void wbatch(const WRows& w, const int* rmap, int roff, const float* xs, const PF& pf,
                                       int k0, int lane, int sub, int cl, const EmitArgs& ea, float& acc,
                                       float& pend, float& best, int& best_i, int& nonfinite) {
    int g = k0 / w.ncb, cb = k0 - g * w.ncb;
#pragma unroll
    for (int k = 0; k < kPF; k++) {
        const int row = w.r0 + g * w.rpi + sub;
        const int c = cl + (cb << w.lsh);
        if (FULL || (row < w.r1 && c < w.W.nch && k0 + k < w.nslots)) {
            const float p = chunk_dot<DT>(pf.q[k], xs, c);
            if constexpr (DT == DT_Q8)
                acc += h2f((uint16_t)pf.s[k]) * p;
            else
                acc += p;
        }
        if (cb == w.ncb - 1 && (FULL || k0 + k < w.nslots)) {  // the group's rows are complete
            float v = lane_sum_down(acc, w.lpr);
            acc = 0.f;
            if constexpr (EM == EM_QKV || EM == EM_SWIGLU) {
                if (w.rpi == 1) {
                    if (lane == 0) {
                        if ((row & 1) == 0) {
                            pend = v;
                        } else if constexpr (EM == EM_QKV) {
                            emit_qkv(ea, rmap[row - 1], rmap[row], pend, v);
                        } else {
                            stl(ea.out + (row >> 1), silu(pend) * v);
                        }
                    }
                } else {
                    const float other = __shfl_down(v, w.lpr, 64);
                    if (cl == 0 && (sub & 1) == 0 && row < w.r1) {
                        if constexpr (EM == EM_QKV)
                            emit_qkv(ea, rmap[row], rmap[row + 1], v, other);
                        else
                            stl(ea.out + (row >> 1), silu(v) * other);
                    }
                }
            } else if (cl == 0 && (FULL || row < w.r1)) {
                if constexpr (EM == EM_PART) {
                    stc(ea.out + row, v);
                } else {
                    const int r = roff + row;
                    ea.out[r] = v;
                    if (!isfinite(v)) nonfinite = 1;
                    if (v > best) {  // a lane's rows arrive in increasing order
                        best = v;
                        best_i = r;
                    }
                }
            }
        }
        if (++cb == w.ncb) {
            cb = 0;
            ++g;
        }
    }
}

// Lane (within its group of 2^LSH lanes) that holds slot s after
// seg_reduce16<LSH>: slot bit 3-j sits at lane bit LSH-1-j.
template <int LSH>
__device__ __forceinline__ int slot_lane(int s) {
    return ((s >> 3) & 1) << (LSH - 1) | ((s >> 2) & 1) << (LSH - 2) | ((s >> 1) & 1) << (LSH - 3) |
           (s & 1) << (LSH - 4);
}

// One halving step of the transposed butterfly: lanes with bit M set keep the
// upper half of the values, the others the lower half; each sends the half it
// drops to lane ^ M and adds what it receives. The exchange is xshfl's (half
// swap, swizzle or DPP), not an LDS permute.
template <int M, int N>
__device__ __forceinline__ void halve(const float (&in)[2 * N], float (&out)[N], int lane) {
    const bool up = lane & M;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const float send = up ? in[i] : in[i + N], keep = up ? in[i + N] : in[i];
        out[i] = keep + xshfl<M>(send);
    }
}

// Sums each of 16 values over every group of 2^LSH lanes (LSH = 4, 5 or 6)
// in 15 + (LSH - 4) exchanges: four halving steps, then plain butterfly
// steps. Lane l ends with the group total of slot slot(l), replicated over the
// 2^(LSH-4) lanes that differ only in the low bits.
template <int LSH>
__device__ __forceinline__ float seg_reduce16(const float (&v)[16], int lane) {
    constexpr int L = 1 << LSH;
    float t8[8], t4[4], t2[2], t1[1];
    halve<L / 2, 8>(v, t8, lane);
    halve<L / 4, 4>(t8, t4, lane);
    halve<L / 8, 2>(t4, t2, lane);
    halve<L / 16, 1>(t2, t1, lane);
    float t = t1[0];
    if constexpr (L / 32 >= 1) t += xshfl<(L / 32 >= 1 ? L / 32 : 1)>(t);
    if constexpr (L / 64 >= 1) t += xshfl<(L / 64 >= 1 ? L / 64 : 1)>(t);
    return t;
}

// One batch of kPF = 16 slots in the dense case: rows read by 2^LSH lanes
// (LSH = 4, 5, 6), every chunk of the window in range (nch a multiple of the
// row's lanes), whole row groups, and for LSH = 6 ncb in {1, 2, 4, 8} so a
// batch holds whole rows (an even number). Lane partials of each row
// accumulate over its ncb slots, one transposed butterfly sums all rows over
// their lanes, and the lanes emit the rows in parallel.
template <int DT, int EM, int LSH, int NCB, bool I8 = false>
__device__ __forceinline__ void wbatch_fast(const WRows& w, const int* rmap, int roff, const float* xs, const PF& pf,
                                            int k0, int lane, const EmitArgs& ea, float& best, int& best_i,
                                            int& nonfinite) {
    static_assert(kPF == 16, "seg_reduce16 takes 16 slots");
    constexpr int L = 1 << LSH, RPI = 64 / L;
    const int ncb = NCB ? NCB : w.ncb;  // a power of two dividing kPF; k0 is a multiple of kPF
    const int sub = lane >> LSH, cl = lane & (L - 1);
    float rv[16];
    if constexpr (NCB > 0) {
        // column batch outer, rows inner: the input chunk of a batch is read
        // from LDS once for all the batch's rows; each row still sums its
        // batches in order
        constexpr int NR = kPF / NCB;
        float acc[NR];
#pragma unroll
        for (int r = 0; r < NR; r++) acc[r] = 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; cb++) {
            XChunk<DT> xc;
            XChunkI8 xi;
            if constexpr (I8)
                xi = xchunk_load_i8(xs, w.W.nch * VecW<DT>::VE, cl + (cb << LSH));
            else
                xc = xchunk_load<DT>(xs, cl + (cb << LSH));
#pragma unroll
            for (int r = 0; r < NR; r++) {
                const int k = r * NCB + cb;
                if (k0 + k < w.nslots) {
                    const float p = I8 ? chunk_dot_i8(pf.q[k], xi) : chunk_dot_x<DT>(pf.q[k], xc);
                    if constexpr (DT == DT_Q8)
                        acc[r] += h2f((uint16_t)pf.s[k]) * p;
                    else
                        acc[r] += p;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kPF; k++) rv[k] = (k % NCB == NCB - 1 && k0 + k < w.nslots) ? acc[k / NCB] : 0.f;
    } else {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < kPF; k++) {
            const int cb = k & (ncb - 1);
            rv[k] = 0.f;
            if (k0 + k < w.nslots) {
                const int c = cl + (cb << LSH);
                const float p = I8 ? chunk_dot_i8(pf.q[k], xchunk_load_i8(xs, w.W.nch * VecW<DT>::VE, c))
                                   : chunk_dot<DT>(pf.q[k], xs, c);
                if constexpr (DT == DT_Q8)
                    acc += h2f((uint16_t)pf.s[k]) * p;
                else
                    acc += p;
                if (cb == ncb - 1) {
                    rv[k] = acc;
                    acc = 0.f;
                }
            }
        }
    }
    const float t = seg_reduce16<LSH>(rv, cl);
    const int s = ((cl >> (LSH - 1)) & 1) * 8 + ((cl >> (LSH - 2)) & 1) * 4 + ((cl >> (LSH - 3)) & 1) * 2 +
                  ((cl >> (LSH - 4)) & 1);
    const int row = w.r0 + (k0 + s) / ncb * RPI + sub;  // the row that ends at slot s
    const bool end = (cl & (L / 16 - 1)) == 0 && (s & (ncb - 1)) == ncb - 1 && k0 + s < w.nslots;
    if constexpr (EM == EM_QKV || EM == EM_SWIGLU) {
        // rows 2i and 2i+1: the odd row ends ncb slots later (whole-wave rows)
        // or sits in the next group of lanes (shorter rows). For an even row
        // that is slot s ^ ncb (a batch starts at an even row), so lane ^ 4 ncb,
        // or lane ^ L (its group index is even): one xshfl exchange. Only even
        // rows use the value.
        float other;
        if constexpr (RPI == 1 && NCB > 0)
            other = xshfl<(1 << (LSH - 4)) * (NCB > 0 ? NCB : 1)>(t);
        else if constexpr (RPI > 1)
            other = xshfl<(RPI > 1 ? L : 1)>(t);
        else
            other = __shfl(t, slot_lane<LSH>((s + ncb) & 15), 64);
        if (end && ((row - w.r0) & 1) == 0) {
            if constexpr (EM == EM_QKV)
                emit_qkv(ea, rmap[row], rmap[row + 1], t, other);
            else
                stl(ea.out + (row >> 1), silu(t) * other);
        }
    } else if (end) {
        if constexpr (EM == EM_PART) {
            stc(ea.out + row, t);
        } else {
            const int r = roff + row;
            ea.out[r] = t;
            if (!isfinite(t)) nonfinite = 1;
            if (t > best) {  // a lane's rows arrive in increasing order
                best = t;
                best_i = r;
            }
        }
    }
}

// The wave's rows. If `prefetched`, pf already holds the first kPF slots
// (issued by wload before the barrier). For pairs, wave ranges start at even
// rows.
template <int DT, int EM, class GEO = GeoRT, bool I8 = false>
__device__ __forceinline__ void wrun(const WRows& w, const int* rmap, int roff, const float* xs, PF& pf,
                                     bool prefetched, const EmitArgs& ea, float& best, int& best_i, int& nonfinite) {
    if (w.nslots == 0) return;
    if constexpr (GEO::L > 0) {  // the shape is known to be dense with this geometry
        const int lane = lane_id();
        for (int k0 = 0; k0 < w.nslots; k0 += kPF) {
            if (!prefetched || k0 > 0) wload<DT>(w, rmap, roff, k0, pf);
            wbatch_fast<DT, EM, GEO::L, GEO::N, I8>(w, rmap, roff, xs, pf, opaque_s(k0), lane, ea, best, best_i,
                                                    nonfinite);
        }
    } else {
    static_assert(!I8, "integer products run in the kernels compiled for one shape");
    const int lane = lane_id(), sub = lane >> w.lsh, cl = lane & (w.lpr - 1);
    const bool dense = w.lsh >= 4 && (w.W.nch & (w.lpr - 1)) == 0 && (w.r1 - w.r0) % w.rpi == 0 && w.ncb <= 8 &&
                       (w.ncb & (w.ncb - 1)) == 0;
    float acc = 0.f, pend = 0.f;
    for (int k0 = 0; k0 < w.nslots; k0 += kPF) {
        if (!prefetched || k0 > 0) wload<DT>(w, rmap, roff, k0, pf);
        const int k0s = opaque_s(k0);
        if (dense && w.lsh == 6)
            wbatch_fast<DT, EM, 6, 0>(w, rmap, roff, xs, pf, k0s, lane, ea, best, best_i, nonfinite);
        else if (dense && w.lsh == 5)
            wbatch_fast<DT, EM, 5, 0>(w, rmap, roff, xs, pf, k0s, lane, ea, best, best_i, nonfinite);
        else if (dense)
            wbatch_fast<DT, EM, 4, 0>(w, rmap, roff, xs, pf, k0s, lane, ea, best, best_i, nonfinite);
        else
            wbatch<DT, EM, false>(w, rmap, roff, xs, pf, k0s, lane, sub, cl, ea, acc, pend, best, best_i, nonfinite);
    }
    }
}

// ------------------------------------------------------------------ attention
// Splits of the P attended rows (the span of pos) of one KV head: S splits of CH
// positions (the last one shorter), S chosen so that the group's items (its KV
// heads times S) cover its blocks, with at least 16 positions per split.
__device__ __forceinline__ void attn_splits(int P, int bg, int n_kv_heads, int& S, int& CH) {
    const int nh_max = (n_kv_heads + kNG - 1) / kNG;
    S = bg / nh_max;
    const int smax = (P + 15) / 16;
    if (S > smax) S = smax;
    if (S > kStepMaxSplit) S = kStepMaxSplit;
    if (S < 1) S = 1;
    CH = (P + S - 1) / S;
    S = (P + CH - 1) / CH;
}

// Loads of the K and V rows a thread needs for span indices c0 + pg + i*PPI
// of KV head g; indices past the split are clamped to the last (row pos: its
// values are not used, row pos itself is substituted from the q|k|v buffer).
__device__ __forceinline__ void attn_kv_load(const StepArgs& a, int layer, int g, int c0, const Span& span,
                                             u32x4 (&kr)[kStepAttn], u32x4 (&vr)[kStepAttn]) {
    const int hd = a.head_dim, LPP = attn_lpp(hd), PPI = kSB / LPP;
    const int tid = thread_id(), sub = tid % LPP, pg = tid / LPP;
    const int sub8 = sub * 8 < hd ? sub * 8 : 0;
    const __half* kb = a.kc + (size_t)layer * a.kv_layer + (size_t)g * a.n_ctx * hd + sub8;
    const __half* vb = a.vc + (size_t)layer * a.kv_layer + (size_t)g * a.n_ctx * hd + sub8;
#pragma unroll
    for (int i = 0; i < kStepAttn; i++) {
        const int t = span_row(span, min(c0 + pg + i * PPI, span.n - 1));
        kr[i] = ld16(kb + (size_t)t * hd);
        vr[i] = ld16(vb + (size_t)t * hd);
    }
}

// The block's items (KV head g, split s) of the group: scaled scores, softmax
// and the weighted sum of V over the split's positions ("The Forward Pass in
// Java", Example 7), kept as (running max m, sum l, unnormalised o) per query
// head of g and written to part[((g*S + s)*G + h)*(hd + 2)]: m, l, o[hd]. The
// G query heads of g are taken GC at a time. Splits run over the span's
// indices (span_row gives the cache row); q is scaled by the attention
// temperature of pos.
//
// The rounding mode ("What a Llama model computes, and why", section 8: q in
// binary16, and the normalised probabilities rounded to binary16 before they weight V) runs
// two passes. Pass 1 keeps only each split's (m, l), written to
// pst[((g*S + s)*G + h)*2]. After a group barrier, pass 2 takes the span's
// M = max m_s and L = sum l_s e^(m_s - M), weights V with f16(e^(x - M)/L), and
// writes each split's o with m = 0 and l = 1 for split 0 (0 for the others),
// so the merge adds the splits' o with weight one.
template <int GC>
__device__ __forceinline__ void attn_items(const StepArgs& a, int layer, int pos, const Span& span, const float* qkv,
                                           float* part, float* pst, int pass, int hlo, int nh, int S, int CH, int rk,
                                           int bg, u32x4 (&kr)[kStepAttn], u32x4 (&vr)[kStepAttn], float* sm,
                                           float* m_run, float* l_run, float* alpha) {
    const int hd = a.head_dim, P = span.n, G = a.n_heads / a.n_kv_heads;
    const float tau = attn_temp(a.span, pos);
    const int qd = a.n_heads * hd, kvd = a.n_kv_heads * hd;
    const int tid = thread_id(), lane = tid & 63, wave = tid >> 6;
    const int LPP = attn_lpp(hd), PPI = kSB / LPP, CHUNK = PPI * kStepAttn;
    const int sub = tid % LPP, pg = tid / LPP;
    const bool dim_ok = sub * 8 < hd;
    const int sub8 = dim_ok ? sub * 8 : 0;
    float* sc = sm;                     // [GC][CHUNK]
    float* wred = sm + GC * CHUNK;      // [kSW][GC][hd]
    float* raw = wred + kSW * GC * hd;  // [GC][CHUNK]: pass 1's scaled scores
    bool have = pass != 2;              // the first chunk of the first item is prefetched
    // Pass 2 of a block with one item, one chunk and one group of query heads
    // (at most one item per block always holds) still has pass 1's V rows in
    // vr and its scores in raw: it takes f16(e^(s - M)/L) from those instead of
    // reloading K/V and recomputing the dot products (the same values, so the
    // same result as the reloading path).
    const bool single = CH <= CHUNK && G <= GC;
    const bool reuse = pass == 2 && single;
    if (reuse) have = true;

    for (int item = rk; item < nh * S; item += bg) {
        const int g = hlo + item / S, s = item % S;
        const int t_begin = s * CH, t_end = min(P, t_begin + CH);
        // this step's K and V row (the split that holds pos), rounded to
        // binary16 as the cache stores them, loaded once per item
        u32x4 kpos = {0u, 0u, 0u, 0u}, vpos = {0u, 0u, 0u, 0u};
        if (P - 1 >= t_begin && P - 1 < t_end) {
            const float4 k0 = ldf4(qkv + qd + g * hd + sub8), k1 = ldf4(qkv + qd + g * hd + sub8 + 4);
            const float4 v0 = ldf4(qkv + qd + kvd + g * hd + sub8), v1 = ldf4(qkv + qd + kvd + g * hd + sub8 + 4);
            auto pk = [](float lo, float hi) {
                return (uint32_t)__half_as_ushort(f2h(lo)) | ((uint32_t)__half_as_ushort(f2h(hi)) << 16);
            };
            kpos = (u32x4){pk(k0.x, k0.y), pk(k0.z, k0.w), pk(k1.x, k1.y), pk(k1.z, k1.w)};
            vpos = (u32x4){pk(v0.x, v0.y), pk(v0.z, v0.w), pk(v1.x, v1.y), pk(v1.z, v1.w)};
        }
        for (int h0 = 0; h0 < G; h0 += GC) {
            float qv[GC][8], acc[GC][8];
#pragma unroll
            for (int h = 0; h < GC; h++) {
                // (a pass 2 that reuses pass 1's scores needs no q)
                const float4 a0 = reuse ? make_float4(0.f, 0.f, 0.f, 0.f) : ldf4(qkv + ((g * G + h0 + h) * hd + sub8));
                const float4 a1 =
                    reuse ? make_float4(0.f, 0.f, 0.f, 0.f) : ldf4(qkv + ((g * G + h0 + h) * hd + sub8 + 4));
                const float f = dim_ok ? tau : 0.f;
                qv[h][0] = a0.x * f;
                qv[h][1] = a0.y * f;
                qv[h][2] = a0.z * f;
                qv[h][3] = a0.w * f;
                qv[h][4] = a1.x * f;
                qv[h][5] = a1.y * f;
                qv[h][6] = a1.z * f;
                qv[h][7] = a1.w * f;
                if (pass != 0)
#pragma unroll
                    for (int i = 0; i < 8; i++) qv[h][i] = round16(qv[h][i]);
#pragma unroll
                for (int i = 0; i < 8; i++) acc[h][i] = 0.f;
            }
            __syncthreads();
            if (pass == 2) {
                // the span's max and sum from pass 1's splits (lane = split)
                for (int h = wave; h < GC; h += kSW) {
                    float m = -INFINITY, l = 0.f;
                    if (lane < S) {
                        const float* pj = pst + (((size_t)g * S + lane) * G + h0 + h) * 2;
                        m = ldf(pj);
                        l = ldf(pj + 1);
                    }
                    const float M = xmax64(m);
                    const float L = xsum64(lane < S ? l * expf(m - M) : 0.f);
                    if (lane == 0) {
                        m_run[h] = M;
                        l_run[h] = L;
                    }
                }
            } else if (tid < GC) {
                m_run[tid] = -INFINITY;
                l_run[tid] = 0.f;
            }
            for (int c0 = t_begin; c0 < t_end; c0 += CHUNK) {
                const int cn = min(CHUNK, t_end - c0);
                if (!have) attn_kv_load(a, layer, g, c0, span, kr, vr);
                have = false;
#pragma unroll
                for (int i = 0; i < kStepAttn; i++) {
                    const int t = pg + i * PPI;
                    if (t < cn && c0 + t == P - 1) {
                        kr[i] = kpos;
                        vr[i] = vpos;
                    }
                }
                if (!reuse) {
                    // scores: each lane's partial dot over its 8 dimensions, then
                    // the sums over the LPP lanes of a position, every step
                    // applied to all of the block's values at once
                    float d[kStepAttn][GC];
#pragma unroll
                    for (int i = 0; i < kStepAttn; i++) {
                        float kf[8];
                        unpack8(kr[i], kf);
#pragma unroll
                        for (int h = 0; h < GC; h++) {
                            float v = 0.f;
#pragma unroll
                            for (int j = 0; j < 8; j++) v += qv[h][j] * kf[j];
                            d[i][h] = v;
                        }
                    }
                    lanes_sum_all<kStepAttn * GC>(&d[0][0], 1, LPP);
#pragma unroll
                    for (int i = 0; i < kStepAttn; i++) {
                        const int t = pg + i * PPI;
#pragma unroll
                        for (int h = 0; h < GC; h++)
                            if (sub == 0 && t < cn) sc[h * CHUNK + t] = d[i][h] / a.scale_div;
                    }
                }
                __syncthreads();
                if (pass == 2) {
                    const float* sv = reuse ? raw : sc;
                    for (int h = wave; h < GC; h += kSW) {
                        const float M = m_run[h], L = l_run[h];
                        for (int t = lane; t < cn; t += 64) sc[h * CHUNK + t] = round16(expf(sv[h * CHUNK + t] - M) / L);
                        if (lane == 0) alpha[h] = 1.f;
                    }
                } else
                for (int h = wave; h < GC; h += kSW) {
                    float mx = -INFINITY;
                    for (int t = lane; t < cn; t += 64) mx = fmaxf(mx, sc[h * CHUNK + t]);
                    mx = xmax64(mx);
                    const float m_old = m_run[h];
                    const float m_new = fmaxf(m_old, mx);
                    float ls = 0.f;
                    for (int t = lane; t < cn; t += 64) {
                        const float x = sc[h * CHUNK + t];
                        if (pass == 1 && single) raw[h * CHUNK + t] = x;
                        const float e = expf(x - m_new);
                        sc[h * CHUNK + t] = e;
                        ls += e;
                    }
                    ls = xsum64(ls);
                    if (lane == 0) {
                        const float al = (m_old == -INFINITY) ? 0.f : expf(m_old - m_new);
                        alpha[h] = al;
                        l_run[h] = l_run[h] * al + ls;
                        m_run[h] = m_new;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int h = 0; h < GC; h++) {
                    const float al = alpha[h];
#pragma unroll
                    for (int i = 0; i < 8; i++) acc[h][i] *= al;
                }
#pragma unroll
                for (int i = 0; i < kStepAttn; i++) {
                    const int t = pg + i * PPI;
                    if (dim_ok && t < cn && pass != 1) {
                        float vf[8];
                        unpack8(vr[i], vf);
#pragma unroll
                        for (int h = 0; h < GC; h++) {
                            const float wgt = sc[h * CHUNK + t];
#pragma unroll
                            for (int j = 0; j < 8; j++) acc[h][j] += wgt * vf[j];
                        }
                    }
                }
                __syncthreads();
            }
            if (h0 + GC < G) have = false;  // the next pass reloads K and V
            if (pass == 1) {
                if (tid < GC) {
                    float* myst = pst + (((size_t)g * S + s) * G + h0 + tid) * 2;
                    stl(myst, m_run[tid]);
                    stl(myst + 1, l_run[tid]);
                }
                __syncthreads();
                continue;
            }
            lanes_sum_all<GC * 8>(&acc[0][0], LPP, 64);
            if (lane < LPP && dim_ok)
#pragma unroll
                for (int h = 0; h < GC; h++)
#pragma unroll
                    for (int i = 0; i < 8; i++) wred[(wave * GC + h) * hd + sub8 + i] = acc[h][i];
            __syncthreads();
            const int GH = GC * hd, stride = hd + 2;
            float* mypart = part + (((size_t)g * S + s) * G + h0) * (size_t)stride;
            for (int e = tid; e < GH; e += kSB) {
                float o = 0.f;
#pragma unroll
                for (int w = 0; w < kSW; w++) o += wred[w * GH + e];
                stl(mypart + (e / hd) * stride + 2 + (e % hd), o);
            }
            if (tid < GC) {
                stl(mypart + tid * stride, pass == 2 ? 0.f : m_run[tid]);
                stl(mypart + tid * stride + 1, pass == 2 ? (s == 0 ? 1.f : 0.f) : l_run[tid]);
            }
            __syncthreads();
        }
    }
}

// Merge of the splits of the group's query heads into xs (swizzled for DT,
// element hl*hd + d for local head hl): with M = max_s m_s and L = sum_s l_s
// e^(m_s - M), o = sum_s o_s e^(m_s - M) / L.
template <int DT>
__device__ __forceinline__ void merge_splits(const StepArgs& a, const float* part, int hlo, int nh, int S, float* xs, float* wsp,
                             float* ored) {
    const int hd = a.head_dim, G = a.n_heads / a.n_kv_heads, stride = hd + 2;
    const int NHL = nh * G, E = NHL * hd;
    const int tid = thread_id(), lane = tid & 63, wave = tid >> 6;
    // o loads first (they do not depend on the weights), then the weights
    const int nsl = E <= kSB ? kSB / E : 1;
    const int e = E <= kSB ? tid % E : tid, sl = E <= kSB ? tid / E : 0;
    constexpr int kU = 16;
    float ov[kU];
    int hl = 0, d = 0;
    const float* po = part;
    const bool act = E <= kSB && sl < nsl;
    if (act) {
        hl = e / hd;
        d = e - hl * hd;
        const int g = hlo + hl / G, h = hl % G;
        po = part + ((size_t)g * S * G + h) * stride + 2 + d;
#pragma unroll
        for (int i = 0; i < kU; i++) {
            const int s = sl + i * nsl;
            ov[i] = s < S ? ldf(po + (size_t)s * G * stride) : 0.f;
        }
    }
    for (int h2 = wave; h2 < NHL; h2 += kSW) {
        const int g = hlo + h2 / G, h = h2 % G;
        float m = -INFINITY, l = 0.f;
        if (lane < S) {
            const float* pj = part + (((size_t)g * S + lane) * G + h) * stride;
            m = ldf(pj);
            l = ldf(pj + 1);
        }
        const float M = xmax64(m);
        const float f = lane < S ? expf(m - M) : 0.f;
        const float Lh = xsum64(l * f);
        if (lane < S) wsp[h2 * S + lane] = f / Lh;
    }
    __syncthreads();
    if (E <= kSB) {
        if (act) {
            float o = 0.f;
#pragma unroll
            for (int i = 0; i < kU; i++) {
                const int s = sl + i * nsl;
                if (s < S) o += wsp[hl * S + s] * ov[i];
            }
            for (int s = sl + kU * nsl; s < S; s += nsl) o += wsp[hl * S + s] * ldf(po + (size_t)s * G * stride);
            ored[sl * E + e] = o;
        }
        __syncthreads();
        if (tid < E) {
            float o = 0.f;
            for (int k = 0; k < nsl; k++) o += ored[k * E + tid];
            xs[swz<DT>(tid)] = o;
        }
    } else {
        for (int e2 = tid; e2 < E; e2 += kSB) {
            const int hl2 = e2 / hd, d2 = e2 - hl2 * hd;
            const int g = hlo + hl2 / G, h = hl2 % G;
            const float* p2 = part + ((size_t)g * S * G + h) * stride + 2 + d2;
            float o = 0.f;
            for (int s = 0; s < S; s++) o += wsp[hl2 * S + s] * ldf(p2 + (size_t)s * G * stride);
            xs[swz<DT>(e2)] = o;
        }
    }
    __syncthreads();
}

// --------------------------------------------------------------------- logits
// xs holds rmsnorm(xr) * output_norm already when `normed` (for DT's swizzle).
template <int DT, class GEO = GeoRT, bool RND = false>
__device__ __forceinline__ void logits_phase(const StepArgs& a, const float* xr, const GainPF& gp, float* xs,
                                             double* red, ArgPart* wbest, bool normed) {
    if (!normed) stage_norm<DT>(xr, a.out_norm, gp, a.eps, a.dim, xs, red);
    if constexpr (RND) round_input<DT>(xs, a.dim);
    const int lane = thread_id() & 63, wave = thread_id() >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(blockIdx.x * kSW + wave);
    WRows w = wave_rows(a.out.rows, gridDim.x * kSW, wv, a.dim / VecW<DT>::VE, false);
    w.W = make_win<DT>(a.out, 0, a.dim);
    EmitArgs ea{};
    ea.out = a.logits;
    float best = -INFINITY;
    int bi = 0x7fffffff, nf = 0;
    PF pf;
    wrun<DT, EM_ARGMAX, GEO>(w, nullptr, 0, xs, pf, false, ea, best, bi, nf);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ob > best || (ob == best && oi < bi)) {
            best = ob;
            bi = oi;
        }
    }
    const int anynf = __any(nf);
    if (lane == 0) wbest[wave] = ArgPart{best, bi, anynf, 0};
    __syncthreads();
    if (threadIdx.x == 0) {
        ArgPart b = wbest[0];
        for (int k = 1; k < kSW; k++) {
            const ArgPart o = wbest[k];
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

// --------------------------------------------------------------------- kernel
// DT: layer weight type. The remaining parameters specialise the kernel for
// one shape (ODT: output matrix type, GA: query heads per attention pass, then
// the geometry of the QKV, output, gate/up, down and vocabulary products);
// ODT = -1, GA = 0 and GeoRT take everything from the run-time shape. RND:
// llama.cpp's rounding points (rounded product inputs, two attention passes).
template <int DT, int ODT, int GA, class GQ, class GO, class GG, class GD, class GL, bool RND>
__global__ __launch_bounds__(kSB, 1) void k_step(StepArgs a) {
    extern __shared__ float sm[];
    __shared__ double red[kSW];
    __shared__ ArgPart wbest[kSW];
    __shared__ float m_run[kMaxGroup], l_run[kMaxGroup], alpha[kMaxGroup];

    State* st = a.st;
    const int pos = st->pos, tok = st->token, epoch = st->epoch;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int x = blockIdx.x % kNG, rk = blockIdx.x / kNG, bg = gridDim.x / kNG;
    const int gwv = __builtin_amdgcn_readfirstlane(rk * kSW + wave), GW = bg * kSW;
    const int hd = a.head_dim, G = a.n_heads / a.n_kv_heads;
    const int qd = a.n_heads * hd, kvd = a.n_kv_heads * hd;
    const int hlo = x * a.n_kv_heads / kNG, nh = (x + 1) * a.n_kv_heads / kNG - hlo;
    const int nbk = a.ffn / 32, flo = x * nbk / kNG * 32, nf = (x + 1) * nbk / kNG * 32 - flo;
    unsigned hmask = 0, fmask = 0;  // groups that own heads / hidden units
    for (int g = 0; g < kNG; g++) {
        if ((g + 1) * a.n_kv_heads / kNG > g * a.n_kv_heads / kNG) hmask |= 1u << g;
        if ((g + 1) * nbk / kNG > g * nbk / kNG) fmask |= 1u << g;
    }
    const Span span = attn_span(a.span, pos);
    int S, CH;
    attn_splits(span.n, bg, a.n_kv_heads, S, CH);
    constexpr int VE = VecW<DT>::VE;

    float* xr = sm;                        // this block's copy of the residual stream
    float* xs = sm + a.lds_xr;             // staged product input, or attention scratch
    float* wsp = xs + a.lds_xs;            // split weights of the merge
    float* ored = wsp + a.lds_wsp;         // merge partial sums [kSB]
    float2* cs = (float2*)(ored + kSB);    // RoPE (cos, sin) of this position, kMaxHeadDim/2 pairs
    // llama.cpp's rounding points on Q8_0 layers in a kernel compiled for the
    // shape: the products' inputs stay Q8_0 codes and the products are integer
    // dot products
    constexpr bool I8 = RND && DT == DT_Q8 && GA > 0;
    auto round_in = [&](int K) {
        if constexpr (I8)
            round_input_i8(xs, K);
        else if constexpr (RND)
            round_input<DT>(xs, K);
    };
    int* qmap = (int*)(cs + kMaxHeadDim / 2);  // the group's q/k/v rows in RoPE-pair order
    // the layer descriptors, copied once, so that the address of a phase's
    // weights is an LDS read rather than a dependent load from device memory
    LayerW* lw = (LayerW*)(sm + a.lds_lw);
    for (int i = tid; i < a.n_layers * (int)(sizeof(LayerW) / 8); i += kSB)
        ((unsigned long long*)lw)[i] = ((const unsigned long long*)a.layers)[i];

    // group barriers per layer: after QKV, (rounding mode: between the two
    // attention passes,) after attention, after gate/up
    const unsigned long long nloc = (RND ? 4ull : 3ull) * a.n_layers, ncro = 2ull * a.n_layers + 1;
    unsigned long long jl = (unsigned long long)epoch * nloc, jc = (unsigned long long)epoch * ncro;
    int phase = 0;
    const bool tr = a.trace && blockIdx.x == 0 && tid == 0;
    if (tr) a.trace[0] = wall_clock64();
#define STAMP()                                  \
    do {                                         \
        ++phase;                                 \
        if (tr) a.trace[phase] = wall_clock64(); \
    } while (0)

    // Rows 2p, 2p+1 of the group's q/k/v share are the two rows RoPE pair p
    // rotates together ("The Forward Pass in Java", Example 6: (2j, 2j+1) in
    // the normal layout, (j, j + n_rot/2) in the NEOX one; dimensions past
    // n_rot pair up unrotated). Pairs run over the group's KV heads, each as
    // its G query heads, then its key and its value head.
    const int n_qkv = nh * (G + 2) * hd, half = a.n_rot / 2;
    for (int p = tid; p < n_qkv / 2; p += kSB) {
        const int hp = hd / 2, hh = p / hp, j = p - hh * hp;
        const int i = hh / (G + 2), sub = hh - i * (G + 2), kvh = hlo + i;
        const int base = sub < G ? (kvh * G + sub) * hd : (sub == G ? qd + kvh * hd : qd + kvd + kvh * hd);
        int ra, rb;
        if (j < half) {
            ra = base + (a.neox ? j : 2 * j);
            rb = a.neox ? ra + half : ra + 1;
        } else {
            ra = base + a.n_rot + 2 * (j - half);
            rb = ra + 1;
        }
        qmap[2 * p] = ra;
        qmap[2 * p + 1] = rb;
    }
    for (int i = tid; i < a.dim; i += kSB) xr[i] = mat_elem(a.embd, tok, i);
    for (int j = tid; j < half; j += kSB) {
        const float* c = (const float*)(a.rope + ((size_t)pos * half + j));
        cs[j] = make_float2(ldf(c), ldf(c + 1));
    }
    __syncthreads();

    WRows wq = wave_rows(n_qkv, GW, gwv, a.dim / VE, true);
    WRows wo = wave_rows(nh > 0 ? a.dim : 0, GW, gwv, nh * G * hd / VE, false);
    WRows wg = wave_rows(2 * nf, GW, gwv, a.dim / VE, true);
    WRows wd = wave_rows(nf > 0 ? a.dim : 0, GW, gwv, nf / VE, false);
    EmitArgs ea{};
    ea.cs = cs;
    ea.pos = pos;
    ea.n_ctx = a.n_ctx;
    ea.hd = hd;
    ea.qd = qd;
    ea.kvd = kvd;
    ea.half = half;
    ea.n_rot = a.n_rot;
    ea.neox = a.neox;
    float best = 0.f;
    int bi = 0, nfin = 0;

    PF pf;
    GainPF gp;
    u32x4 kr[kStepAttn], vr[kStepAttn];
#define KV_PREFETCH(layer)                                                                  \
    do {                                                                                    \
        if (rk < nh * S) {                                                                  \
            attn_kv_load(a, (layer), hlo + rk / S, (rk % S) * CH, span, kr, vr);             \
        } else {                                                                            \
            for (int i_ = 0; i_ < kStepAttn; i_++) kr[i_] = vr[i_] = (u32x4){0u, 0u, 0u, 0u}; \
        }                                                                                   \
    } while (0)
    gain_load(gp, lw[0].attn_norm, a.dim);
    wq.W = make_win<DT>(lw[0].qkv, 0, a.dim);
    wload<DT>(wq, qmap, 0, 0, pf);
    KV_PREFETCH(0);
    pin();

    for (int l = 0; l < a.n_layers; l++) {
        float* qkv = a.qkv + (size_t)l * a.qkv_stride;
        float* part = a.part + (size_t)l * a.part_stride;
        float* pst = a.pst + (size_t)l * a.pst_stride;
        float* u = a.u + (size_t)l * a.u_stride;
        float* po = a.po + (size_t)l * kNG * a.pstride;
        float* pd = a.pd + (size_t)l * kNG * a.pstride;

        // ---- QKV (the previous layer's end left rmsnorm(x) * attn_norm in xs)
        if (l == 0) stage_norm<DT>(xr, lw[0].attn_norm, gp, a.eps, a.dim, xs, red);
        round_in(a.dim);
        ea.out = qkv;
        ea.bias = lw[l].bqkv;
        ea.kc = a.kc + (size_t)l * a.kv_layer;
        ea.vc = a.vc + (size_t)l * a.kv_layer;
        wrun<DT, EM_QKV, GQ, I8>(wq, qmap, 0, xs, pf, true, ea, best, bi, nfin);
        wait_mem();
        group_arrive(a, x);
        group_wait(a, x, ++jl * bg);
        STAMP();

        // ---- attention (the rounding mode: pass 1, group barrier, pass 2)
        for (int pass = RND ? 1 : 0;; pass = 2) {
            if constexpr (GA > 0) {
                attn_items<GA>(a, l, pos, span, qkv, part, pst, pass, hlo, nh, S, CH, rk, bg, kr, vr, xs, m_run, l_run,
                               alpha);
            } else {
                switch (G) {
                    case 1:
                        attn_items<1>(a, l, pos, span, qkv, part, pst, pass, hlo, nh, S, CH, rk, bg, kr, vr, xs, m_run,
                                      l_run, alpha);
                        break;
                    case 2:
                        attn_items<2>(a, l, pos, span, qkv, part, pst, pass, hlo, nh, S, CH, rk, bg, kr, vr, xs, m_run,
                                      l_run, alpha);
                        break;
                    default:
                        attn_items<4>(a, l, pos, span, qkv, part, pst, pass, hlo, nh, S, CH, rk, bg, kr, vr, xs, m_run,
                                      l_run, alpha);
                        break;
                }
            }
            if (pass != 1) break;
            wait_mem();
            group_arrive(a, x);
            group_wait(a, x, ++jl * bg);
        }
        wait_mem();
        group_arrive(a, x);
        wo.W = make_win<DT>(lw[l].o, hlo * G * hd, nh * G * hd);
        wload<DT>(wo, nullptr, 0, 0, pf);
        pin();
        group_wait(a, x, ++jl * bg);
        STAMP();

        // ---- split merge + output product (partial over the group's heads)
        if (nh > 0) {
            merge_splits<DT>(a, part, hlo, nh, S, xs, wsp, ored);
            round_in(nh * G * hd);
            ea.out = po + (size_t)x * a.pstride;
            wrun<DT, EM_PART, GO, I8>(wo, nullptr, 0, xs, pf, true, ea, best, bi, nfin);
        }
        wait_mem();
        all_arrive(a, x);
        gain_load(gp, lw[l].ffn_norm, a.dim);
        wg.W = make_win<DT>(lw[l].gu, 0, a.dim);
        wload<DT>(wg, nullptr, 2 * flo, 0, pf);
        pin();
        all_wait(a, ++jc * bg);
        STAMP();

        // ---- residual, RMSNorm, gate/up + SwiGLU
        add_partials_norm<DT>(xr, po, a.pstride, a.dim, hmask, lw[l].ffn_norm, gp, a.eps, xs, red);
        round_in(a.dim);
        ea.out = u + flo;
        wrun<DT, EM_SWIGLU, GG, I8>(wg, nullptr, 2 * flo, xs, pf, true, ea, best, bi, nfin);
        wait_mem();
        group_arrive(a, x);
        wd.W = make_win<DT>(lw[l].down, flo, nf);
        wload<DT>(wd, nullptr, 0, 0, pf);
        pin();
        group_wait(a, x, ++jl * bg);
        STAMP();

        // ---- down product (partial over the group's hidden units)
        if (nf > 0) {
            stage_copy<DT>(u + flo, nf, xs);
            round_in(nf);
            ea.out = pd + (size_t)x * a.pstride;
            wrun<DT, EM_PART, GD, I8>(wd, nullptr, 0, xs, pf, true, ea, best, bi, nfin);
        }
        wait_mem();
        all_arrive(a, x);
        if (l + 1 < a.n_layers) {
            gain_load(gp, lw[l + 1].attn_norm, a.dim);
            wq.W = make_win<DT>(lw[l + 1].qkv, 0, a.dim);
            wload<DT>(wq, qmap, 0, 0, pf);
            KV_PREFETCH(l + 1);
        } else {
            gain_load(gp, a.out_norm, a.dim);
        }
        pin();
        all_wait(a, ++jc * bg);
        STAMP();
        // the residual, and the next RMSNorm: the next layer's attention norm,
        // or after the last layer the output norm (for the output matrix's
        // swizzle, known here in a kernel compiled for the shape)
        if (l + 1 < a.n_layers)
            add_partials_norm<DT>(xr, pd, a.pstride, a.dim, fmask, lw[l + 1].attn_norm, gp, a.eps, xs, red);
        else if constexpr (ODT >= 0)
            add_partials_norm<ODT>(xr, pd, a.pstride, a.dim, fmask, a.out_norm, gp, a.eps, xs, red);
        else
            add_partials(xr, pd, a.pstride, a.dim, fmask);
    }

    if constexpr (ODT >= 0) {
        logits_phase<ODT, GL, RND>(a, xr, gp, xs, red, wbest, true);
    } else {
        switch (a.out.dtype) {
            case DT_F32: logits_phase<DT_F32, GeoRT, RND>(a, xr, gp, xs, red, wbest, false); break;
            case DT_F16: logits_phase<DT_F16, GeoRT, RND>(a, xr, gp, xs, red, wbest, false); break;
            default: logits_phase<DT_Q8, GeoRT, RND>(a, xr, gp, xs, red, wbest, false); break;
        }
    }
    wait_mem();
    all_arrive(a, x);
    all_wait(a, ++jc * bg);
    STAMP();
    if (blockIdx.x == 0 && tid == 0) {
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
#undef STAMP
}


// ------------------------------------------------------------------- host side
// LDS sizes (floats) of the step kernel's regions for this shape, or false if
// the shape is outside what the kernel handles.
bool step_lds_plan(StepArgs& a, int dtype, int* lds_bytes) {
    const int G = a.n_heads / a.n_kv_heads, hd = a.head_dim;
    if (a.ffn % 32 || a.dim % 32 || (G * hd) % 32 || hd % 8 || hd > kMaxHeadDim) return false;
    const int nh_max = (a.n_kv_heads + kNG - 1) / kNG;
    const int nbk = a.ffn / 32, nf_max = ((nbk + kNG - 1) / kNG) * 32;
    auto lds_any = [](int K) {
        int m = lds_floats<DT_F32>(K);
        if (lds_floats<DT_F16>(K) > m) m = lds_floats<DT_F16>(K);
        if (lds_floats<DT_Q8>(K) > m) m = lds_floats<DT_Q8>(K);
        return m;
    };
    (void)dtype;
    int xs = lds_any(a.dim);
    if (lds_any(nh_max * G * hd) > xs) xs = lds_any(nh_max * G * hd);
    if (lds_any(nf_max) > xs) xs = lds_any(nf_max);
    const int GC = G < 4 ? G : 4;
    // scores, per-wave sums, and the rounding mode's copy of pass 1's scores
    const int att = 2 * GC * (kSB / attn_lpp(hd)) * kStepAttn + kSW * GC * hd;
    if (att > xs) xs = att;
    a.lds_xr = (a.dim + 63) / 64 * 64;
    a.lds_xs = (xs + 63) / 64 * 64;
    a.lds_wsp = (nh_max * G * kStepMaxSplit + 63) / 64 * 64;
    const int qmap = nh_max * (G + 2) * hd;  // ints
    int total = a.lds_xr + a.lds_xs + a.lds_wsp + kSB + kMaxHeadDim + qmap;
    total = (total + 1) & ~1;  // 8-byte alignment for the layer table
    a.lds_lw = total;
    total += a.n_layers * (int)(sizeof(LayerW) / 4);
    *lds_bytes = total * (int)sizeof(float);
    return *lds_bytes <= 150 * 1024;
}

// A specialisation: weight types, query heads per attention pass and the
// (lanes-per-row shift, column batches) of the five products.
struct StepSpec {
    int dt, odt, ga, geo[5][2];
    const void* fn;      // float numerics
    const void* fn_rnd;  // llama.cpp's rounding points
};

static const StepSpec kSpecs[] = {
    // 2048-wide Q8_0 layers, 4 query heads per KV head of 64, 8192 FFN units, F32 vocabulary rows
    {DT_Q8, DT_F32, 4, {{6, 2}, {4, 1}, {6, 2}, {6, 1}, {6, 8}},
     (const void*)k_step<DT_Q8, DT_F32, 4, Geo<6, 2>, Geo<4, 1>, Geo<6, 2>, Geo<6, 1>, Geo<6, 8>, false>,
     (const void*)k_step<DT_Q8, DT_F32, 4, Geo<6, 2>, Geo<4, 1>, Geo<6, 2>, Geo<6, 1>, Geo<6, 8>, true>},
    // the same shape with F16 layers and F16 vocabulary rows
    {DT_F16, DT_F16, 4, {{6, 4}, {5, 1}, {6, 4}, {6, 2}, {6, 4}},
     (const void*)k_step<DT_F16, DT_F16, 4, Geo<6, 4>, Geo<5, 1>, Geo<6, 4>, Geo<6, 2>, Geo<6, 4>, false>,
     (const void*)k_step<DT_F16, DT_F16, 4, Geo<6, 4>, Geo<5, 1>, Geo<6, 4>, Geo<6, 2>, Geo<6, 4>, true>},
};

// The geometry wave_rows gives a product of n rows over a window of nch
// chunks, and whether it is dense (every wave range a whole number of row
// groups, every chunk in range, a power-of-two number of column batches <= 8).
static bool host_geo(int n, int nch, int* lsh, int* ncb) {
    int lpr = 64, sh = 6;
    if (nch < 64) {
        lpr = 1;
        sh = 0;
        while (lpr < nch) {
            lpr <<= 1;
            sh++;
        }
    }
    *lsh = sh;
    *ncb = (nch + lpr - 1) / lpr;
    const int rpi = 64 / lpr;
    return sh >= 4 && nch % lpr == 0 && n % rpi == 0 && *ncb <= 8 && (*ncb & (*ncb - 1)) == 0;
}

static const void* pick_kernel(const StepArgs& a, int dtype, bool* special) {
    *special = false;
    const int G = a.n_heads / a.n_kv_heads, hd = a.head_dim;
    auto ve = [](int dt) { return dt == DT_F32 ? 4 : (dt == DT_F16 ? 8 : 16); };
    const int nh_max = (a.n_kv_heads + kNG - 1) / kNG, nh_min = a.n_kv_heads / kNG;
    const int nbk = a.ffn / 32;
    const bool even = nh_max == nh_min && nbk % kNG == 0;  // every group owns the same share
    int g[5][2];
    bool dense = even;
    if (even) {
        const int nf = nbk / kNG * 32;
        dense = host_geo(nh_max * (G + 2) * hd, a.dim / ve(dtype), &g[0][0], &g[0][1]) &&
                host_geo(a.dim, nh_max * G * hd / ve(dtype), &g[1][0], &g[1][1]) &&
                host_geo(2 * nf, a.dim / ve(dtype), &g[2][0], &g[2][1]) &&
                host_geo(a.dim, nf / ve(dtype), &g[3][0], &g[3][1]) &&
                host_geo(a.out.rows, a.dim / ve(a.out.dtype), &g[4][0], &g[4][1]) && g[0][0] == 6 && g[2][0] == 6;
    }
    if (dense)
        for (const StepSpec& sp : kSpecs) {
            if (sp.dt != dtype || sp.odt != a.out.dtype || (sp.ga != (G < 4 ? G : 4))) continue;
            bool same = true;
            for (int i = 0; i < 5; i++) same = same && sp.geo[i][0] == g[i][0] && sp.geo[i][1] == g[i][1];
            if (same) {
                *special = true;
                return a.rnd ? sp.fn_rnd : sp.fn;
            }
        }
    if (a.rnd) switch (dtype) {
            case DT_F32: return (const void*)k_step<DT_F32, -1, 0, GeoRT, GeoRT, GeoRT, GeoRT, GeoRT, true>;
            case DT_F16: return (const void*)k_step<DT_F16, -1, 0, GeoRT, GeoRT, GeoRT, GeoRT, GeoRT, true>;
            default: return (const void*)k_step<DT_Q8, -1, 0, GeoRT, GeoRT, GeoRT, GeoRT, GeoRT, true>;
        }
    switch (dtype) {
        case DT_F32: return (const void*)k_step<DT_F32, -1, 0, GeoRT, GeoRT, GeoRT, GeoRT, GeoRT, false>;
        case DT_F16: return (const void*)k_step<DT_F16, -1, 0, GeoRT, GeoRT, GeoRT, GeoRT, GeoRT, false>;
        default: return (const void*)k_step<DT_Q8, -1, 0, GeoRT, GeoRT, GeoRT, GeoRT, GeoRT, false>;
    }
}

int step_grid(StepArgs& a, int dtype, int* lds_bytes, const void** fn, bool* special) {
    if (!step_lds_plan(a, dtype, lds_bytes)) return 0;
    *fn = pick_kernel(a, dtype, special);
    if (hipFuncSetAttribute(*fn, hipFuncAttributeMaxDynamicSharedMemorySize, *lds_bytes) != hipSuccess) return 0;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, *fn, kSB, *lds_bytes) != hipSuccess) return 0;
    const int grid = cus / kNG * kNG;
    return per_cu >= 1 && grid >= kNG ? grid : 0;
}

// The XCD (hardware register XCC_ID) each block of a grid runs on.
__global__ void k_xcd_probe(int* out) {
    if (threadIdx.x == 0) out[blockIdx.x] = (int)__builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
}

bool step_groups_share_l2(int grid, int* d_buf, hipStream_t s) {
    void* params[] = {&d_buf};
    if (hipLaunchKernel((const void*)k_xcd_probe, dim3(grid), dim3(kSB), params, 0, s) != hipSuccess)
        return false;
    std::vector<int> x(grid);
    if (hipMemcpyAsync(x.data(), d_buf, (size_t)grid * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return false;
    for (int b = 0; b < grid; b++)
        if (x[b] != x[b % kNG]) return false;
    return true;
}

// An ordinary dispatch: the grid has one block per compute unit and a block
// fits on any of them (step_grid checked both), so on a device running nothing
// else every block is resident at once, which is all the grid barriers need.
// (A cooperative launch gives the same guarantee at ~18 us more per token.)
// Should other work hold compute units, the blocks that started wait at their
// first barrier until the rest are dispatched; the waits are bounded, so a
// grid that cannot become resident ends in the abort flag, not a hang.
hipError_t launch_step(const StepArgs& a, const void* fn, int grid, int lds, hipStream_t s) {
    StepArgs arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(fn, dim3(grid), dim3(kSB), params, (unsigned)lds, s);
}

}  // namespace llm
