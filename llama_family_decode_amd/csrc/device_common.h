// Device helpers shared by the decode kernels (included by each kernel file).
#pragma once

#include "common.h"

#include <math.h>

// Tunables of the vector products (defaults are the measured best).
#ifndef LLM_GEMV_NR_SMALL
#define LLM_GEMV_NR_SMALL 2  // rows per wave for the QKV and residual epilogues
#endif
#ifndef LLM_GEMV_NR_BIG
#define LLM_GEMV_NR_BIG 4    // rows per wave for the SwiGLU, store and argmax epilogues
#endif
#ifndef LLM_GEMV_U_Q8
#define LLM_GEMV_U_Q8 8      // Q8_0 chunks per lane in flight when NR is small
#endif
#ifndef LLM_GEMV_U
#define LLM_GEMV_U 4         // chunks per lane in flight otherwise
#endif
#ifndef LLM_GEMV_GRID_CAP
#define LLM_GEMV_GRID_CAP 2048
#endif
#ifndef LLM_GEMV_NT
#define LLM_GEMV_NT 1        // non-temporal weight loads
#endif

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
#if LLM_GEMV_NT
    return __builtin_nontemporal_load((const u32x4*)base + c);
#else
    return *((const u32x4*)base + c);
#endif
}

// The staged-input values that multiply one 16-byte weight chunk c (VE
// floats, as VE/4 float4 pieces of the swizzled LDS copy).
template <int DT>
struct XChunk {
    float4 v[VecW<DT>::VE / 4];
};

template <int DT>
__device__ __forceinline__ XChunk<DT> xchunk_load(const float* xs, int c) {
    XChunk<DT> x;
    if constexpr (DT == DT_F32) {
        x.v[0] = *(const float4*)(xs + 4 * c);
    } else {
        const float* b = xs + (c >> 6) * VecW<DT>::SEG + 4 * (c & 63);
#pragma unroll
        for (int k = 0; k < VecW<DT>::VE / 4; k++) x.v[k] = *(const float4*)(b + 256 * k);
    }
    return x;
}

// Partial dot of one chunk with its input values.
template <int DT>
__device__ __forceinline__ float chunk_dot_x(u32x4 raw, const XChunk<DT>& x) {
    if constexpr (DT == DT_F32) {
        float s = __uint_as_float(raw.x) * x.v[0].x;
        s += __uint_as_float(raw.y) * x.v[0].y;
        s += __uint_as_float(raw.z) * x.v[0].z;
        s += __uint_as_float(raw.w) * x.v[0].w;
        return s;
    } else if constexpr (DT == DT_F16) {
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
        float w[8];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            w[2 * k] = h2f((uint16_t)(u[k] & 0xffffu));
            w[2 * k + 1] = h2f((uint16_t)(u[k] >> 16));
        }
        float s = w[0] * x.v[0].x;
        s += w[1] * x.v[0].y;
        s += w[2] * x.v[0].z;
        s += w[3] * x.v[0].w;
        s += w[4] * x.v[1].x;
        s += w[5] * x.v[1].y;
        s += w[6] * x.v[1].z;
        s += w[7] * x.v[1].w;
        return s;
    } else {
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int w = (int)u[k];
            const float q0 = (float)((w << 24) >> 24), q1 = (float)((w << 16) >> 24);
            const float q2 = (float)((w << 8) >> 24), q3 = (float)(w >> 24);
            s0 += q0 * x.v[k].x;
            s1 += q1 * x.v[k].y;
            s0 += q2 * x.v[k].z;
            s1 += q3 * x.v[k].w;
        }
        return s0 + s1;
    }
}

// Partial dot of one chunk with the staged input.
template <int DT>
__device__ __forceinline__ float chunk_dot(u32x4 raw, const float* xs, int c) {
    return chunk_dot_x<DT>(raw, xchunk_load<DT>(xs, c));
}

// llama.cpp's rounding points on Q8_0 weights ("What a Llama model computes,
// and why", section 8: the activations are rounded to 8 bits and the product
// is an integer dot per block): the staged input as K int8 codes in element
// order followed by one float scale (binary16-rounded) per 32-block. One
// 16-byte weight chunk c meets the 16 codes at byte 16c and the scale of block
// c / 2.
struct XChunkI8 {
    u32x4 q;
    float d;
};

__device__ __forceinline__ XChunkI8 xchunk_load_i8(const float* xs, int K, int c) {
    XChunkI8 x;
    x.q = *(const u32x4*)((const char*)xs + 16 * c);
    x.d = (xs + K / 4)[c >> 1];
    return x;
}

// Weight codes . input codes as one exact int32 (four 4-way int8 dot
// products), times the input block's scale; the caller applies the weight
// row's block scale.
__device__ __forceinline__ float chunk_dot_i8(u32x4 raw, const XChunkI8& x) {
    int s = __builtin_amdgcn_sdot4((int)raw.x, (int)x.q.x, 0, false);
    s = __builtin_amdgcn_sdot4((int)raw.y, (int)x.q.y, s, false);
    s = __builtin_amdgcn_sdot4((int)raw.z, (int)x.q.z, s, false);
    s = __builtin_amdgcn_sdot4((int)raw.w, (int)x.q.w, s, false);
    return (float)s * x.d;
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

__device__ __forceinline__ void unpack8(u32x4 raw, float* f) {
    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        f[2 * k] = h2f((uint16_t)(u[k] & 0xffffu));
        f[2 * k + 1] = h2f((uint16_t)(u[k] >> 16));
    }
}

// Loads of chunks c0, c0+64, ..., c0+64(U-1) (those below nch) of NR rows.
template <int DT, int NR, int U>
__device__ __forceinline__ void load_batch(const Mat& W, const int* lrow, int c0, int nch, u32x4 (&raw)[U][NR],
                                           float (&sc)[U][NR]) {
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int c = c0 + 64 * u;
        if (c < nch) {
#pragma unroll
            for (int i = 0; i < NR; i++) {
                raw[u][i] = load_chunk<DT>(W, lrow[i], c);
                if constexpr (DT == DT_Q8) sc[u][i] = h2f(W.s[(size_t)lrow[i] * (W.cols / 32) + c / 2]);
            }
        }
    }
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

constexpr int kAttnSteps = 4;

__host__ __device__ inline int attn_lpp(int hd) {
    int l = 1;
    while (l * 8 < hd) l <<= 1;
    return l;
}
__host__ __device__ inline int attn_chunk(int hd) { return (kBlock / attn_lpp(hd)) * kAttnSteps; }

}  // namespace llm
