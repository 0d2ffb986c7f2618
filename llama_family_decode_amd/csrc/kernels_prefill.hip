// Prefill kernels for gfx950: a batch of n tokens at positions p0 .. p0+n-1
// ("What a Llama model computes, and why", section 4). The vector products
// become matrix products over the batch, which run on the matrix cores:
// v_mfma_f32_16x16x32_f16 with fp32 accumulation. F16 weights and Q8_0 quants
// are exact in binary16; each fp32 activation enters as the sum of two
// binary16 numbers (hi = f16(x), lo = f16(x - hi)), two products per tile, so
// the result matches fp32 activations to about 2^-22 relative: rounding the
// activations themselves to binary16 grows through the layers past the
// decode tolerance. Each 32-deep product is one Q8_0 block, so its fp32
// partial is scaled by that block's fp16 scale before it joins the
// accumulator. F32 weights use an fp32 VALU product.
// RMSNorm, RoPE and attention run per token.
#include "common.h"

#include <math.h>

namespace llm {

// (x0, x1) rotated by the angle whose (cos, sin) is cs, each product rounded
// separately as the pages' RoPE computes it (no fused multiply-add).
__device__ __forceinline__ float2 pf_rope_rotate(float x0, float x1, float2 cs) {
#pragma clang fp contract(off)
    return make_float2(x0 * cs.x - x1 * cs.y, x0 * cs.y + x1 * cs.x);
}

__device__ __forceinline__ float pf_h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }
__device__ __forceinline__ float pf_silu(float z) { return z / (1.0f + expf(-z)); }

// One wave's 64 q|k|v columns hc .. hc + 63 (one head: hc % 64 == 0) of row
// m, v0 / v1 the columns hc + r32 and hc + 32 + r32 with the bias added: RoPE
// as k_rope_kv_rows applies it (head_dim 64, every pair rotated; NEOX pairs
// (d, d + 32) in one lane, normal pairs (2p, 2p + 1) in lanes r32 and r32 ^ 1),
// then the Q row or the F16 cache row. Every lane of the wave calls it (the
// pair exchange); rows m >= M write nothing.
__device__ __forceinline__ void rope_store2(const RopeArgs& ro, int m, int M, int hc, int r32, float v0, float v1) {
    const int qd = ro.n_heads * 64, kvd = ro.n_kv_heads * 64, pos = ro.p0 + m;
    float o0 = v0, o1 = v1;
    if (hc < qd + kvd) {
        if (ro.neox) {
            if (m < M) {
                const float2 rv = pf_rope_rotate(v0, v1, ro.rope[(size_t)pos * 32 + r32]);
                o0 = rv.x;
                o1 = rv.y;
            }
        } else {
            const float w0 = xshfl<1>(v0), w1 = xshfl<1>(v1);
            const bool odd = r32 & 1;
            if (m < M) {
                const float2 r0 = pf_rope_rotate(odd ? w0 : v0, odd ? v0 : w0, ro.rope[(size_t)pos * 32 + (r32 >> 1)]);
                const float2 r1 =
                    pf_rope_rotate(odd ? w1 : v1, odd ? v1 : w1, ro.rope[(size_t)pos * 32 + 16 + (r32 >> 1)]);
                o0 = odd ? r0.y : r0.x;
                o1 = odd ? r1.y : r1.x;
            }
        }
    }
    if (m >= M) return;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int n = hc + 32 * j + r32;
        const float o = j ? o1 : o0;
        if (n < qd)
            ro.Q[(size_t)m * qd + n] = o;
        else if (n < qd + kvd)
            ro.kc[((size_t)((n - qd) >> 6) * ro.n_ctx + pos) * 64 + (n & 63)] = __float2half_rn(o);
        else
            ro.vc[((size_t)((n - qd - kvd) >> 6) * ro.n_ctx + pos) * 64 + (n & 63)] = __float2half_rn(o);
    }
}

// ------------------------------------------------------------ embedding rows
__global__ void k_embed_rows(Mat E, const int* tokens, int n, float* X, int dim) {
    const int row = blockIdx.x;
    const int64_t t = tokens[row];
    for (int i = threadIdx.x; i < dim; i += blockDim.x) {
        float v;
        if (E.dtype == DT_F32)
            v = ((const float*)E.w)[t * dim + i];
        else if (E.dtype == DT_F16)
            v = pf_h2f(((const uint16_t*)E.w)[t * dim + i]);
        else
            v = pf_h2f(E.s[t * (dim / 32) + i / 32]) * (float)((const int8_t*)E.w)[t * dim + i];
        X[(size_t)row * dim + i] = v;
    }
}

hipError_t launch_embed_rows(const Mat& E, const int* tokens, int n, float* X, int dim, hipStream_t s) {
    hipLaunchKernelGGL(k_embed_rows, dim3(n), dim3(256), 0, s, E, tokens, n, X, dim);
    return hipGetLastError();
}

// ------------------------------------------------------------ RMSNorm rows
// y = (x * scale) * g with scale = (float)(1 / sqrt(sum(x^2)/n + eps)), the sum in
// double ("The Forward Pass in Java", Example 4).
// Block-wide sum of one double per thread (256 threads).
__device__ __forceinline__ double rows_sum256(double v, double* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// The Q8_0 codes of 8 consecutive values of a row (a quarter of a block, the
// block's four quarters in one DPP quad of lanes), as k_round_rows takes them:
// d = max|y| / 127, codes roundf(y / d) through the float reciprocal, the
// scale d rounded to binary16, to the tiled int8 layout (and the scale, as
// fp32, from the block's first quarter).
__device__ __forceinline__ void q8_codes8(const float (&y)[8], int row, int i0, int K, int8_t* C, float* CS) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(y[e]));
    amax = fmaxf(amax, xshfl<1>(amax));
    amax = fmaxf(amax, xshfl<2>(amax));
    const float d = amax / 127.f, id = d != 0.f ? 1.f / d : 0.f;
    uint32_t q[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e++) q[e >> 2] |= (uint32_t)(uint8_t)(int8_t)roundf(y[e] * id) << (8 * (e & 3));
    *(uint2*)(C + tile_off_i8(row, i0, K, kTileA)) = make_uint2(q[0], q[1]);
    if ((i0 & 31) == 0) CS[tile_off_s(row, i0 >> 5, K, kTileA)] = round16(d);
}

// y = x * scale * g for the 8 values of x at column i0 of `row` (i0 % 8 == 0):
// the fp32 row when Yf is set, the tiled hi/lo planes when Yh is set, one
// 16-byte slot each (the tiled layout keeps 8 consecutive columns of a row
// together), and y's Q8_0 codes and block scales when C is set.
__device__ __forceinline__ void norm_store8(const float (&x)[8], float scale, const float* gain, int row, int i0,
                                           int dim, float* Yf, __half* Yh, __half* Yl, int8_t* C, float* CS) {
    const float4 g0 = *(const float4*)(gain + i0), g1 = *(const float4*)(gain + i0 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = x[e] * scale * g[e];
    if (C) q8_codes8(y, row, i0, dim, C, CS);
    if (Yf) {
        float* yf = Yf + (size_t)row * dim + i0;
        *(float4*)yf = make_float4(y[0], y[1], y[2], y[3]);
        *(float4*)(yf + 4) = make_float4(y[4], y[5], y[6], y[7]);
    }
    if (Yh) {
        __half h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            h[e] = __float2half_rn(y[e]);
            l[e] = __float2half_rn(y[e] - __half2float(h[e]));
        }
        const size_t t = tile_off(row, i0, dim, kTileA);
        *(uint4*)(Yh + t) = *(const uint4*)h;
        *(uint4*)(Yl + t) = *(const uint4*)l;
    }
}

// Y = rmsnorm(X) * gain per row ("The Forward Pass in Java", Example 4): the
// sum of squares in double, the scale 1/sqrt(ss/dim + eps) rounded to float
// once, y = (x * scale) * g. One block of 256 threads per row, 8 columns per
// thread and step.
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const float* X, const float* gain, int dim, float eps, float* Yf,
                                                      __half* Yh, __half* Yl, int8_t* C, float* CS) {
    __shared__ double red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const float* x = X + (size_t)row * dim;
    double ss = 0.0;
    for (int i0 = 8 * tid; i0 < dim; i0 += 8 * 256) {
        const float4 a = *(const float4*)(x + i0), b = *(const float4*)(x + i0 + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; e++) ss += (double)v[e] * (double)v[e];
    }
    const double tot = rows_sum256(ss, red);
    const float scale = (float)(1.0 / sqrt(tot / (double)dim + (double)eps));
    for (int i0 = 8 * tid; i0 < dim; i0 += 8 * 256) {
        const float4 a = *(const float4*)(x + i0), b = *(const float4*)(x + i0 + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        norm_store8(v, scale, gain, row, i0, dim, Yf, Yh, Yl, C, CS);
    }
}

hipError_t launch_rmsnorm_rows(const float* X, const float* gain, int n, int dim, float eps, float* Yf, __half* Yh,
                               __half* Yl, hipStream_t s, int8_t* C, float* CS) {
    // with codes a block's four quarters must be one quad of lanes: whole blocks
    if (dim % 8 || (C && (dim % 32 || !CS))) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_rmsnorm_rows, dim3(n), dim3(256), 0, s, X, gain, dim, eps, Yf, Yh, Yl, C, CS);
    return hipGetLastError();
}

// The split-K reduction of a residual product fused with the next RMSNorm:
// X[m] += sum of the S partials P[z][m] in z order (as k_splitk_reduce adds
// them), then Y = rmsnorm(X[m]) * gain as k_rmsnorm_rows computes it.
__global__ __launch_bounds__(256) void k_reduce_norm_rows(const float* P, int S, int M, float* X, int dim,
                                                          const float* gain, float eps, float* Yf, __half* Yh,
                                                          __half* Yl, int8_t* C, float* CS) {
    __shared__ double red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    float* x = X + (size_t)row * dim;
    const size_t MN = (size_t)M * dim;
    double ss = 0.0;
    for (int i0 = 8 * tid; i0 < dim; i0 += 8 * 256) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int z = 0; z < S; z++) {
            const float* pz = P + z * MN + (size_t)row * dim + i0;
            const float4 a = *(const float4*)pz, b = *(const float4*)(pz + 4);
            acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
            acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
        }
        const float4 a = *(const float4*)(x + i0), b = *(const float4*)(x + i0 + 4);
        const float v[8] = {a.x + acc[0], a.y + acc[1], a.z + acc[2], a.w + acc[3],
                            b.x + acc[4], b.y + acc[5], b.z + acc[6], b.w + acc[7]};
        *(float4*)(x + i0) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)(x + i0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
#pragma unroll
        for (int e = 0; e < 8; e++) ss += (double)v[e] * (double)v[e];
    }
    const double tot = rows_sum256(ss, red);
    const float scale = (float)(1.0 / sqrt(tot / (double)dim + (double)eps));
    for (int i0 = 8 * tid; i0 < dim; i0 += 8 * 256) {  // this thread's own columns, written above
        const float4 a = *(const float4*)(x + i0), b = *(const float4*)(x + i0 + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        norm_store8(v, scale, gain, row, i0, dim, Yf, Yh, Yl, C, CS);
    }
}

hipError_t launch_reduce_norm_rows(const float* P, int S, int n, float* X, int dim, const float* gain, float eps,
                                   float* Yf, __half* Yh, __half* Yl, hipStream_t s, int8_t* C, float* CS) {
    if (dim % 8 || (C && (dim % 32 || !CS))) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_reduce_norm_rows, dim3(n), dim3(256), 0, s, P, S, n, X, dim, gain, eps, Yf, Yh, Yl, C, CS);
    return hipGetLastError();
}

// Eight consecutive elements of one row per thread (two 16-byte loads); a
// Q8_0 block of 32 is one DPP quad of lanes, whose maximum magnitude comes from
// two quad permutes. The rounded values go back to X when keep_x is set; with
// C (Q8_0) the codes go to the tiled int8 layout (8 bytes per thread) and each
// block's scale (its binary16 rounding, as fp32) to CS; H, L get the rounded
// rows' tiled hi/lo planes (one 16-byte slot each per thread).
__global__ __launch_bounds__(256) void k_round_rows(float* X, int K, int dtype, int keep_x, __half* H, __half* L,
                                                    int8_t* C, float* CS) {
    const int row = blockIdx.y, i = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= K) return;  // K is a multiple of 32: a block's quad leaves together
    float* x = X + (size_t)row * K + i;
    const float4 a = *(const float4*)x, b = *(const float4*)(x + 4);
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    if (dtype == DT_Q8) {
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(v[e]));
        amax = fmaxf(amax, xshfl<1>(amax));
        amax = fmaxf(amax, xshfl<2>(amax));
        const float d = amax / 127.f, id = d != 0.f ? 1.f / d : 0.f, dh = round16(d);
        uint32_t q[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float code = roundf(v[e] * id);
            q[e >> 2] |= (uint32_t)(uint8_t)(int8_t)code << (8 * (e & 3));
            v[e] = dh * code;
        }
        if (C) {
            *(uint2*)(C + tile_off_i8(row, i, K, kTileA)) = make_uint2(q[0], q[1]);
            if ((i & 31) == 0) CS[tile_off_s(row, i >> 5, K, kTileA)] = dh;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] = round16(v[e]);
    }
    if (keep_x) {
        *(float4*)x = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)(x + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    if (H) {
        __half h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            h[e] = __float2half_rn(v[e]);
            l[e] = __float2half_rn(v[e] - __half2float(h[e]));
        }
        const size_t t = tile_off(row, i, K, kTileA);
        *(uint4*)(H + t) = *(const uint4*)h;
        *(uint4*)(L + t) = *(const uint4*)l;
    }
}

hipError_t launch_round_rows(float* X, int n, int K, int dtype, __half* H, __half* L, hipStream_t s, int8_t* C,
                             float* CS) {
    if (dtype == DT_F32 || n <= 0) return hipSuccess;
    if (K % 32 || (C && (dtype != DT_Q8 || !CS))) return hipErrorInvalidValue;
    // with codes the product reads only them (its K steps are the 32-blocks)
    const int keep_x = C ? 0 : 1;
    hipLaunchKernelGGL(k_round_rows, dim3((K + 2047) / 2048, n), dim3(256), 0, s, X, K, dtype, keep_x, H, L, C, CS);
    return hipGetLastError();
}

__global__ void k_gather_rows(const float* src, int K, const int* idx, float* dst) {
    const int j = blockIdx.x;
    const float* a = src + (size_t)idx[j] * K;
    for (int i = threadIdx.x; i < K; i += blockDim.x) dst[(size_t)j * K + i] = a[i];
}

hipError_t launch_gather_rows(const float* src, int K, const int* idx, int k, float* dst, hipStream_t s) {
    if (k <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_rows, dim3(k), dim3(256), 0, s, src, K, idx, dst);
    return hipGetLastError();
}

__global__ void k_split_hl(const float* X, int n, int K, __half* H, __half* L) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)n * K) return;
    const int m = (int)(i / K), k = (int)(i % K);
    const float v = X[i];
    const __half h = __float2half_rn(v);
    const size_t t = tile_off(m, k, K, kTileA);
    H[t] = h;
    L[t] = __float2half_rn(v - __half2float(h));
}

hipError_t launch_split_hl(const float* X, int n, int K, __half* H, __half* L, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const size_t total = (size_t)n * K;
    hipLaunchKernelGGL(k_split_hl, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, X, n, K, H, L);
    return hipGetLastError();
}

// One 16-byte piece (8 elements) of the tiled copy per thread; rows past the
// matrix become zeros.
__global__ void k_tile_w(const __half* W, int rows, int cols, int rows_pad, __half* T) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cpr = cols >> 3;
    if (i >= (size_t)rows_pad * cpr) return;
    const int n = (int)(i / cpr), k = (int)(i % cpr) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < rows) v = *(const uint4*)(W + (size_t)n * cols + k);
    *(uint4*)(T + tile_off(n, k, cols, kTileW)) = v;
}

// The same for Q8_0 codes (int8 rows; |code| <= 127 is exact in binary16).
__global__ void k_tile_q8(const int8_t* W, int rows, int cols, int rows_pad, __half* T) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cpr = cols >> 3;
    if (i >= (size_t)rows_pad * cpr) return;
    const int n = (int)(i / cpr), k = (int)(i % cpr) * 8;
    __half h[8];
#pragma unroll
    for (int e = 0; e < 8; e++) h[e] = __float2half_rn(n < rows ? (float)W[(size_t)n * cols + k + e] : 0.f);
    *(uint4*)(T + tile_off(n, k, cols, kTileW)) = *(const uint4*)h;
}

// The same codes as int8 in the tiled int8 layout: one 16-byte piece (half a
// row's 32-code step) per thread; rows past the matrix become zeros.
__global__ void k_tile_i8(const int8_t* W, int rows, int cols, int rows_pad, int8_t* T) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cpr = cols >> 4;
    if (i >= (size_t)rows_pad * cpr) return;
    const int n = (int)(i / cpr), k = (int)(i % cpr) * 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < rows) v = *(const uint4*)(W + (size_t)n * cols + k);
    *(uint4*)(T + tile_off_i8(n, k, cols, kTileW)) = v;
}

// Q8_0 block scales ([rows][cols/32] binary16 bits) as [tile][K step][256]:
// the 256 scales a product tile needs for one 32-deep step are contiguous.
__global__ void k_tile_scales(const uint16_t* S, int rows, int nkb, int rows_pad, uint16_t* T) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)rows_pad * nkb) return;
    const int n = (int)(i % rows_pad), kb = (int)(i / rows_pad);
    const int t = n / kTileW, r = n % kTileW;
    T[((size_t)t * nkb + kb) * kTileW + r] = n < rows ? S[(size_t)n * nkb + kb] : (uint16_t)0;
}

// The same scales as fp32 (the integer products' copy).
__global__ void k_tile_scales_f32(const uint16_t* S, int rows, int nkb, int rows_pad, float* T) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)rows_pad * nkb) return;
    const int n = (int)(i % rows_pad), kb = (int)(i / rows_pad);
    const int t = n / kTileW, r = n % kTileW;
    T[((size_t)t * nkb + kb) * kTileW + r] = n < rows ? __half2float(__ushort_as_half(S[(size_t)n * nkb + kb])) : 0.f;
}

hipError_t launch_tile_w(const Mat& W, hipStream_t s) {
    if ((W.dtype != DT_F16 && W.dtype != DT_Q8) || W.cols % 32 || (!W.wt && !W.wi)) return hipErrorInvalidValue;
    const int rows_pad = (W.rows + kTileW - 1) / kTileW * kTileW;
    const size_t total = (size_t)rows_pad * (W.cols / 8);
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (W.dtype == DT_F16) {
        if (!W.wt) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_tile_w, dim3(grid), dim3(256), 0, s, (const __half*)W.w, W.rows, W.cols, rows_pad,
                           (__half*)W.wt);
        return hipGetLastError();
    }
    const size_t ns = (size_t)rows_pad * (W.cols / 32);
    if (W.wt) {  // binary16 codes and scales (the float numerics' products)
        if (!W.st) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_tile_q8, dim3(grid), dim3(256), 0, s, (const int8_t*)W.w, W.rows, W.cols, rows_pad,
                           (__half*)W.wt);
        hipLaunchKernelGGL(k_tile_scales, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s, W.s, W.rows,
                           W.cols / 32, rows_pad, (uint16_t*)W.st);
    }
    if (W.wi) {  // int8 codes and fp32 scales (the integer products)
        if (!W.si) return hipErrorInvalidValue;
        const size_t n16 = (size_t)rows_pad * (W.cols / 16);
        hipLaunchKernelGGL(k_tile_i8, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, (const int8_t*)W.w, W.rows,
                           W.cols, rows_pad, (int8_t*)W.wi);
        hipLaunchKernelGGL(k_tile_scales_f32, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s, W.s, W.rows,
                           W.cols / 32, rows_pad, (float*)W.si);
    }
    return hipGetLastError();
}

// Output row of product row m: ymap[m] when a row map is given (stores only).
__device__ __forceinline__ int out_row(const int* ymap, int m) { return ymap ? ymap[m] : m; }

// u = silu(gate) * up at Y[m*ldy + j] when Y is set, and its hi/lo pair
// (tiled, K = ldy) when Yh is set.
__device__ __forceinline__ void store_swiglu(float* Y, __half* Yh, __half* Yl, int m, int j, int ldy, float gate,
                                             float up) {
    const float u = pf_silu(gate) * up;
    if (Y) Y[(size_t)m * ldy + j] = u;
    if (Yh) {
        const __half h = __float2half_rn(u);
        const size_t t = tile_off(m, j, ldy, kTileA);
        Yh[t] = h;
        Yl[t] = __float2half_rn(u - __half2float(h));
    }
}

// ------------------------------------------------------------ MFMA GEMM
// Y[m][n] (op)= sum_k A[m][k] * W[n][k] for m < M tokens, n < N weight rows.
// Block tile 128 (m) x 128 (n), K step 32, four waves in a 2 x 2 arrangement,
// each wave 64 x 64 = 4 x 4 tiles of the 16x16x32 instruction. For that
// instruction lane l supplies A[l%16][8*(l/16) + j] and B[8*(l/16) + j][l%16]
// (j < 8) and receives D[4*(l/16) + i][l%16] (i < 4).
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4p __attribute__((ext_vector_type(4)));

constexpr int GB_M = 128, GB_N = 128, GB_K = 32, GB_LD = GB_K + 8;  // LDS row pitch in halfs

// Split K: block z of gridDim.z takes K columns [z*kz, (z+1)*kz); with P set
// it stores its raw partial sums to P[z][m][n] (ld N) instead of applying EPI.
template <int DT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_mfma(Mat W, const float* A, int M, float* Y, int ldy, const float* bias,
                                                   __half* Yh, __half* Yl, int kz, float* P, const int* ymap) {
    // activations as hi + lo binary16 pairs (hi = f16(x), lo = f16(x - hi)),
    // so the products see x to about 2^-22 relative instead of 2^-11
    __shared__ __attribute__((aligned(16))) _Float16 Ah[GB_M * GB_LD];
    __shared__ __attribute__((aligned(16))) _Float16 Al[GB_M * GB_LD];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[GB_N * GB_LD];
    __shared__ float Ss[GB_N];

    const int N = W.rows, K = W.cols, kb = blockIdx.z * kz;
    const int n0 = blockIdx.x * GB_N, m0 = blockIdx.y * GB_M;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // global -> register staging: thread t owns row t/2, k offset 16*(t%2)
    const int lr = tid >> 1, lk = (tid & 1) * 16;
    const int am = m0 + lr, bn = n0 + lr;
    const bool a_ok = am < M, b_ok = bn < N;
    const float* arow = A + (size_t)(a_ok ? am : 0) * K + kb;

    float4 ra0, ra1, ra2, ra3;
    u32x4p rb0, rb1;
    float rs = 0.f;
    const u32x4p z4 = {0u, 0u, 0u, 0u};
    const float4 zf = make_float4(0.f, 0.f, 0.f, 0.f);
    const char* bbase = (const char*)W.w + ((size_t)(b_ok ? bn : 0) * K + kb) * (DT == DT_F16 ? 2 : 1);
    const uint16_t* sbase = (DT == DT_Q8) ? W.s + (size_t)(b_ok ? bn : 0) * (K / 32) + kb / 32 : nullptr;

#define GEMM_GLOAD(k0)                                                                         \
    do {                                                                                       \
        ra0 = a_ok ? *(const float4*)(arow + (k0) + lk) : zf;                                  \
        ra1 = a_ok ? *(const float4*)(arow + (k0) + lk + 4) : zf;                              \
        ra2 = a_ok ? *(const float4*)(arow + (k0) + lk + 8) : zf;                              \
        ra3 = a_ok ? *(const float4*)(arow + (k0) + lk + 12) : zf;                             \
        if constexpr (DT == DT_F16) {                                                          \
            const _Float16* brow = (const _Float16*)bbase;                                     \
            rb0 = b_ok ? __builtin_nontemporal_load((const u32x4p*)(brow + (k0) + lk)) : z4;   \
            rb1 = b_ok ? __builtin_nontemporal_load((const u32x4p*)(brow + (k0) + lk + 8)) : z4; \
        } else {                                                                               \
            rb0 = b_ok ? __builtin_nontemporal_load((const u32x4p*)(bbase + (k0) + lk)) : z4;  \
            rs = b_ok ? pf_h2f(sbase[(k0) / 32]) : 0.f;                                        \
        }                                                                                      \
    } while (0)

    float4v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = (float4v){0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15, fk = (lane >> 4) * 8;
    GEMM_GLOAD(0);
    for (int k0 = 0; k0 < kz; k0 += GB_K) {
        __syncthreads();
        {
            half8 h0, h1, l0, l1;
#define SPLIT(H, L, I, V)                             \
    do {                                              \
        const float v_ = (V);                         \
        const _Float16 t_ = (_Float16)v_;             \
        H[I] = t_;                                    \
        L[I] = (_Float16)(v_ - (float)t_);            \
    } while (0)
            SPLIT(h0, l0, 0, ra0.x); SPLIT(h0, l0, 1, ra0.y); SPLIT(h0, l0, 2, ra0.z); SPLIT(h0, l0, 3, ra0.w);
            SPLIT(h0, l0, 4, ra1.x); SPLIT(h0, l0, 5, ra1.y); SPLIT(h0, l0, 6, ra1.z); SPLIT(h0, l0, 7, ra1.w);
            SPLIT(h1, l1, 0, ra2.x); SPLIT(h1, l1, 1, ra2.y); SPLIT(h1, l1, 2, ra2.z); SPLIT(h1, l1, 3, ra2.w);
            SPLIT(h1, l1, 4, ra3.x); SPLIT(h1, l1, 5, ra3.y); SPLIT(h1, l1, 6, ra3.z); SPLIT(h1, l1, 7, ra3.w);
#undef SPLIT
            *(half8*)(Ah + lr * GB_LD + lk) = h0;
            *(half8*)(Ah + lr * GB_LD + lk + 8) = h1;
            *(half8*)(Al + lr * GB_LD + lk) = l0;
            *(half8*)(Al + lr * GB_LD + lk + 8) = l1;
        }
        if constexpr (DT == DT_F16) {
            *(u32x4p*)(Bs + lr * GB_LD + lk) = rb0;
            *(u32x4p*)(Bs + lr * GB_LD + lk + 8) = rb1;
        } else {
            half8 h0, h1;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int w = (int)rb0[j];
                const _Float16 q0 = (_Float16)((w << 24) >> 24), q1 = (_Float16)((w << 16) >> 24);
                const _Float16 q2 = (_Float16)((w << 8) >> 24), q3 = (_Float16)(w >> 24);
                if (j < 2) {
                    h0[4 * j] = q0; h0[4 * j + 1] = q1; h0[4 * j + 2] = q2; h0[4 * j + 3] = q3;
                } else {
                    h1[4 * j - 8] = q0; h1[4 * j - 7] = q1; h1[4 * j - 6] = q2; h1[4 * j - 5] = q3;
                }
            }
            *(half8*)(Bs + lr * GB_LD + lk) = h0;
            *(half8*)(Bs + lr * GB_LD + lk + 8) = h1;
            if ((tid & 1) == 0) Ss[lr] = rs;
        }
        __syncthreads();
        if (k0 + GB_K < kz) GEMM_GLOAD(k0 + GB_K);
        half8 ah[4], al[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            ah[i] = *(const half8*)(Ah + (64 * wm + 16 * i + fr) * GB_LD + fk);
            al[i] = *(const half8*)(Al + (64 * wm + 16 * i + fr) * GB_LD + fk);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) bf[j] = *(const half8*)(Bs + (64 * wn + 16 * j + fr) * GB_LD + fk);
        if constexpr (DT == DT_F16) {
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bf[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], bf[j], acc[i][j], 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float sc = Ss[64 * wn + 16 * j + fr];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float4v p = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bf[j], (float4v){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], bf[j], p, 0, 0, 0);
                    acc[i][j] += sc * p;
                }
            }
        }
    }
#undef GEMM_GLOAD

    // epilogue
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int n = n0 + 64 * wn + 16 * j + fr;
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int m = m0 + 64 * wm + 16 * i + (lane >> 4) * 4 + e;
                const float v = acc[i][j][e];
                if (P) {
                    if (m < M && n < N) P[((size_t)blockIdx.z * M + m) * N + n] = v;
                } else if constexpr (EPI == EPI_SWIGLU) {
                    const float up = __shfl_xor(v, 1, 64);
                    if ((fr & 1) == 0 && m < M && n < N) store_swiglu(Y, Yh, Yl, m, n / 2, ldy, v, up);
                } else if (m < M && n < N) {
                    if constexpr (EPI == EPI_RESID)
                        Y[(size_t)m * ldy + n] += v;
                    else
                        Y[(size_t)out_row(ymap, m) * ldy + n] = bias ? v + bias[n] : v;
                }
            }
        }
    }
}

// ------------------------------------------------------------ fp32 GEMM (F32 weights)
constexpr int GF_T = 64, GF_K = 16;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(Mat W, const float* A, int M, float* Y, int ldy, const float* bias,
                                                  __half* Yh, __half* Yl, const int* ymap) {
    __shared__ float As[GF_K][GF_T + 4];
    __shared__ float Bs[GF_K][GF_T + 4];
    const int N = W.rows, K = W.cols;
    const int n0 = blockIdx.x * GF_T, m0 = blockIdx.y * GF_T;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const float* Wf = (const float*)W.w;
    float acc[4][4] = {};
    // loader: each thread loads 4 consecutive k of one row for A and for B
    const int lrow = tid >> 2, lk = (tid & 3) * 4;
    for (int k0 = 0; k0 < K; k0 += GF_K) {
        const int am = m0 + lrow, bn = n0 + lrow;
        float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (am < M) av = *(const float4*)(A + (size_t)am * K + k0 + lk);
        if (bn < N) bv = *(const float4*)(Wf + (size_t)bn * K + k0 + lk);
        __syncthreads();
        As[lk + 0][lrow] = av.x; As[lk + 1][lrow] = av.y; As[lk + 2][lrow] = av.z; As[lk + 3][lrow] = av.w;
        Bs[lk + 0][lrow] = bv.x; Bs[lk + 1][lrow] = bv.y; Bs[lk + 2][lrow] = bv.z; Bs[lk + 3][lrow] = bv.w;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < GF_K; k++) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) a[i] = As[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; j++) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] += a[i] * b[j];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            if constexpr (EPI == EPI_SWIGLU) {
                if ((j & 1) == 0) store_swiglu(Y, Yh, Yl, m, n / 2, ldy, acc[i][j], acc[i][j + 1]);
            } else if constexpr (EPI == EPI_RESID) {
                Y[(size_t)m * ldy + n] += acc[i][j];
            } else {
                Y[(size_t)out_row(ymap, m) * ldy + n] = bias ? acc[i][j] + bias[n] : acc[i][j];
            }
        }
    }
}

// Sum of the S split-K partials P[z][m][n] in z order, then the epilogue.
template <int EPI>
__global__ void k_splitk_reduce(const float* P, int S, int M, int N, float* Y, int ldy, const float* bias, __half* Yh,
                                __half* Yl, const int* ymap) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t MN = (size_t)M * N;
    if constexpr (EPI == EPI_SWIGLU) {
        if (2 * i >= MN) return;
        const size_t m = 2 * i / N, n = 2 * i % N;
        float g = 0.f, u = 0.f;
        for (int z = 0; z < S; z++) {
            g += P[z * MN + 2 * i];
            u += P[z * MN + 2 * i + 1];
        }
        store_swiglu(Y, Yh, Yl, (int)m, (int)(n / 2), ldy, g, u);
    } else {
        if (i >= MN) return;
        const size_t m = i / N, n = i % N;
        float v = 0.f;
        for (int z = 0; z < S; z++) v += P[z * MN + i];
        if constexpr (EPI == EPI_RESID)
            Y[m * ldy + n] += v;
        else
            Y[(size_t)out_row(ymap, (int)m) * ldy + n] = bias ? v + bias[n] : v;
    }
}

// The q|k|v rows of the S split-K partials with RoPE and the K/V rows: one
// thread per rotation pair, each value the sum of its partials in z order plus
// the bias (as k_splitk_reduce forms it), then rotated and stored as
// k_rope_kv_rows does (head_dim 64, every pair rotated).
__global__ void k_splitk_rope(const float* P, int S, int n, const float* bias, RopeArgs ro) {
    constexpr int hd = 64, half = 32;
    const int qd = ro.n_heads * hd, kvd = ro.n_kv_heads * hd, W = qd + 2 * kvd;
    const int pairs = W / 2;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * pairs) return;
    const int row = idx / pairs, pi = idx % pairs;
    const int head = pi / half, j = pi % half;
    const int ra = head * hd + (ro.neox ? j : 2 * j), rb = ro.neox ? ra + half : ra + 1;
    const size_t MN = (size_t)n * W, o = (size_t)row * W;
    float va = 0.f, vb = 0.f;
    for (int z = 0; z < S; z++) {
        va += P[z * MN + o + ra];
        vb += P[z * MN + o + rb];
    }
    if (bias) {
        va = va + bias[ra];
        vb = vb + bias[rb];
    }
    const int pos = ro.p0 + row;
    if (head < ro.n_heads + ro.n_kv_heads) {
        const float2 rv = pf_rope_rotate(va, vb, ro.rope[(size_t)pos * half + j]);
        va = rv.x;
        vb = rv.y;
    }
    if (ra < qd) {
        ro.Q[(size_t)row * qd + ra] = va;
        ro.Q[(size_t)row * qd + rb] = vb;
    } else {
        const bool k = ra < qd + kvd;
        const int c0 = ra - qd - (k ? 0 : kvd);
        __half* r = (k ? ro.kc : ro.vc) + ((size_t)(c0 / hd) * ro.n_ctx + pos) * hd;
        r[c0 % hd] = __float2half_rn(va);
        r[(rb - qd - (k ? 0 : kvd)) % hd] = __float2half_rn(vb);
    }
}

// ------------------------------------------------------------ MFMA GEMM, F16 weights
// The same product with the activations' hi/lo planes read from memory (made
// once by the kernel that produces the activations) and every operand tile
// moved global -> LDS by the DMA path (global_load_lds_dwordx4) through a
// four-stage ring, so three K steps are in flight while one is multiplied.
// Block tile 128 (m) x 256 (n), K step 32, eight waves in a 2 x 4
// arrangement, each 64 x 64 = 2 x 2 tiles of the 32x32x16 instruction. A stage
// holds 32 groups of 16 rows x 64 bytes (A hi, A lo: 8 groups each; W: 16
// groups), one 1 KB DMA each; within a group, row r's 16-byte chunk c sits in slot
// 4r + (c ^ (((r >> 1) ^ (r >> 3)) & 3)), so the fragment reads of any 8
// consecutive lanes hit 8 different 16-byte bank groups of a 128-byte bank
// row, and those of any 16 lanes 16 different groups of a 256-byte row.
constexpr int HL_M = 128, HL_N = 256, HL_K = 32, HL_ST = 4, HL_STAGE = 32768;

__device__ __forceinline__ int hl_slot(int r, int c) { return 4 * r + (c ^ tile_swz(r)); }

#ifndef LLM_HL_WAVES
#define LLM_HL_WAVES 8
#endif
// LO = false: the activations are binary16 already (Al holds zeros and its
// products are skipped). Q8: W's tiled copy holds Q8_0 codes; each 32-deep
// step (one Q8_0 block) is multiplied into a fresh accumulator that joins the
// sum scaled by its weight row's block scale, staged with the step.
template <int EPI, int NW, bool LO, bool Q8>
__global__ __launch_bounds__(64 * NW) void k_gemm_hl(Mat W, const __half* Ah, const __half* Al, int M, int kz, int nm,
                                                     int nn, float* Y, int ldy, const float* bias, __half* Yh,
                                                     __half* Yl, float* P, const int* ymap, RopeArgs ro) {
    // NW waves in a 2 x NW/2 arrangement; wave tile 64 x (256 / (NW/2)) as
    // 2 x NJ tiles of the 32x32x16 instruction (on gfx950 it moves twice the
    // operands per cycle of the 16x16x32 one)
    constexpr int WN = NW / 2, NJ = HL_N / WN / 32, ND = 32 / NW;
    // a Q8_0 stage also holds the tile's 256 block scales (wave w moves rows
    // 32w .. 32w+31 with a fifth, four-lane DMA)
    constexpr int STAGE = Q8 ? HL_STAGE + 1024 : HL_STAGE;
    static_assert(!Q8 || NW == 8, "each of 8 waves stages 32 scales");
    __shared__ __attribute__((aligned(1024))) char lds[HL_ST * STAGE];
    const int N = W.rows, K = W.cols;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // tiles that share a weight tile are dealt to one XCD (block b runs on
    // XCD b % 8) and start together, so that tile is fetched into one L2
    int q = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0) q = (q & 7) * (nb >> 3) + (q >> 3);
    const int mt = q % nm, nt = (q / nm) % nn;
    const int z = blockIdx.y;
    const int m0 = mt * HL_M, n0 = nt * HL_N, kb = z * kz;

    // this wave's ND DMA sources: the stage's 32 groups of 16 rows are A hi
    // (groups 0-7), A lo (8-15) and W (16-31), ND consecutive groups a wave;
    // in the tiled layout each is one contiguous 1 KB piece, lane l's 16 bytes
    // at 16 l, already in LDS slot order
    const __half* src[ND];
    const uint16_t* ssrc = nullptr;
    // a K step advances 8 (A) or 16 (W) pieces; a wave's groups are all of one kind
    const size_t kstep = wave * ND < 16 ? 8 * 512 : 16 * 512;
    {
        const int nkK = K / HL_K, kbs = kb / HL_K;
        if constexpr (Q8) ssrc = (const uint16_t*)W.st + ((size_t)nt * nkK + kbs) * HL_N + wave * 32 + (lane & 3) * 8;
#pragma unroll
        for (int i = 0; i < ND; i++) {
            const int grp = wave * ND + i;
            if (grp < 16)
                src[i] = (grp < 8 ? Ah : Al) + (((size_t)mt * nkK + kbs) * 8 + (grp & 7)) * 512 + lane * 8;
            else
                src[i] = (const __half*)W.wt + (((size_t)nt * nkK + kbs) * 16 + (grp - 16)) * 512 + lane * 8;
        }
    }
    const int nk = kz / HL_K;
    auto issue = [&](int ks) {
        char* dst = lds + (ks % HL_ST) * STAGE + wave * ND * 1024;
#pragma unroll
        for (int i = 0; i < ND; i++)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[i] + kstep * ks),
                                             (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
        if constexpr (Q8) {
            if (lane < 4)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(ssrc + (size_t)HL_N * ks),
                    (__attribute__((address_space(3))) void*)(lds + (ks % HL_ST) * STAGE + HL_STAGE + wave * 64), 16, 0,
                    0);
        }
    };

    // For 32x32x16 lane l supplies A[l%32][8*(l/32) + j] and B[8*(l/32) + j][l%32]
    // (j < 8) and receives D[8*(r/4) + 4*(l/32) + r%4][l%32] (r < 16). A
    // 32-row tile spans two 16-row LDS groups; K half kh of a 32-deep step is
    // chunks 2kh and 2kh+1 of each row.
    const int wm = wave / WN, wn = wave % WN;
    const int fgrp = ((lane >> 4) & 1) * 1024;
    const int fslot0 = hl_slot(lane & 15, lane >> 5) * 16 + fgrp;
    const int fslot1 = hl_slot(lane & 15, 2 + (lane >> 5)) * 16 + fgrp;
    float16v acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < NJ; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

    // Waits until at most PEND later stages of this wave's DMAs are in flight
    // and its LDS reads have returned, then for every wave. The s_waitcnt
    // immediate (vmcnt n, lgkmcnt 0, expcnt unconstrained) is a compile-time
    // constant, so a loop built from these waits has no branch in it and the
    // compiler's own wait bookkeeping sees each one on every path.
    auto wait_c = [&](auto pend_c) {
        constexpr int n = decltype(pend_c)::value * (Q8 ? ND + 1 : ND);
        static_assert(n >= 0 && n < 64, "vmcnt holds 6 bits");
        constexpr int imm = (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14);
        // the previous step's products stay before the wait: moved past the
        // barrier they would leave that step with reads and no products
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(imm);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    struct Frag {
        half8 ah[2][2], al[2][2], bf[NJ][2];  // [tile][K half]
        float sc[NJ];                         // Q8: the block scales of this lane's columns
    };
    auto fread = [&](int ks, Frag& F) {
        const char* st = lds + (ks % HL_ST) * STAGE;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const char* a = st + (4 * wm + 2 * i) * 1024;
            F.ah[i][0] = *(const half8*)(a + fslot0);
            F.ah[i][1] = *(const half8*)(a + fslot1);
            if constexpr (LO) {
                F.al[i][0] = *(const half8*)(a + 8192 + fslot0);
                F.al[i][1] = *(const half8*)(a + 8192 + fslot1);
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const char* b = st + 16384 + (2 * NJ * wn + 2 * j) * 1024;
            F.bf[j][0] = *(const half8*)(b + fslot0);
            F.bf[j][1] = *(const half8*)(b + fslot1);
            if constexpr (Q8)
                F.sc[j] = __half2float(*(const __half*)(st + HL_STAGE + 2 * (32 * NJ * wn + 32 * j + (lane & 31))));
        }
    };
    auto fmma = [&](const Frag& F) {
        if constexpr (Q8) {
            float16v t[2][NJ];
#pragma unroll
            for (int kh = 0; kh < 2; kh++)
#pragma unroll
                for (int pl = 0; pl < (LO ? 2 : 1); pl++)
#pragma unroll
                    for (int i = 0; i < 2; i++)
#pragma unroll
                        for (int j = 0; j < NJ; j++)
                            t[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                pl ? F.al[i][kh] : F.ah[i][kh], F.bf[j][kh], kh || pl ? t[i][j] : (float16v){}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < NJ; j++)
#pragma unroll
                    for (int e = 0; e < 16; e++) acc[i][j][e] += F.sc[j] * t[i][j][e];
            return;
        }
#pragma unroll
        for (int kh = 0; kh < 2; kh++)
#pragma unroll
            for (int pl = 0; pl < (LO ? 2 : 1); pl++)
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < NJ; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pl ? F.al[i][kh] : F.ah[i][kh], F.bf[j][kh],
                                                                           acc[i][j], 0, 0, 0);
    };
    // Stage s lives in ring slot s % HL_ST. The fragments of step ks are read
    // during step ks - 1, so while step ks multiplies, the slots hold steps
    // ks+1 (landed) .. ks+HL_ST (in flight).
    using std::integral_constant;
    static_assert(HL_ST == 4, "the prologue and the last steps below are written for a four-stage ring");
    for (int p = 0; p < HL_ST && p < nk; p++) issue(p);
    // stage 0 has landed once at most min(HL_ST, nk) - 1 later stages remain
    if (nk >= 4)
        wait_c(integral_constant<int, 3>{});
    else if (nk == 3)
        wait_c(integral_constant<int, 2>{});
    else if (nk == 2)
        wait_c(integral_constant<int, 1>{});
    else
        wait_c(integral_constant<int, 0>{});
    Frag F0, F1;
    fread(0, F0);
    // One K step: wait for the next step's stage (the last step re-reads its
    // own), refill the slot this step was read from, read the next fragments,
    // multiply the current ones. No branch guards the reads or the products,
    // so the compiler keeps one register assignment and a partial LDS wait.
    // With HL_ST - 1 stages issued ahead, step ks needs stage ks + 1 with at
    // most min(HL_ST - 2, nk - 2 - ks) later stages still in flight: the
    // steady steps (a refill each) wait with HL_ST - 2 in flight, the last
    // min(nk, HL_ST) steps (no refills) with none. (Exact counts there, 2, 1,
    // 0, 0, made the compiler spill the fragments in every instance.)
    auto step = [&](int ks, Frag& cur, Frag& nxt, auto pend_c, auto refill_c) {
        wait_c(pend_c);
        if constexpr (decltype(refill_c)::value) issue(ks + HL_ST);
        fread(min(ks + 1, nk - 1), nxt);
        if constexpr (Q8) {
            // reads first, then the products and their scale folds (the
            // interleaved order below needs more registers than a Q8_0 step
            // has left)
            __builtin_amdgcn_sched_barrier(0);
            fmma(cur);
        } else {
            fmma(cur);
            // the next step's fragment reads interleaved with this step's
            // products, a few at a time: a wave that issued all its reads
            // first would stall on the full LDS queue before its first
            // product (mask 0x100: LDS reads, 0x008: MFMA)
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
    };
    using P0 = integral_constant<int, 0>;
    using P2 = integral_constant<int, 2>;
    using Refill = std::true_type;
    using NoRefill = std::false_type;
    const int nsteady = nk > HL_ST ? nk - HL_ST : 0;
    int ks = 0;
    for (; ks + 1 < nsteady; ks += 2) {
        step(ks, F0, F1, P2{}, Refill{});
        step(ks + 1, F1, F0, P2{}, Refill{});
    }
    if (ks < nsteady) {
        step(ks, F0, F1, P2{}, Refill{});
        ks++;
        F0 = F1;
    }
    for (; ks + 1 < nk; ks += 2) {
        step(ks, F0, F1, P0{}, NoRefill{});
        step(ks + 1, F1, F0, P0{}, NoRefill{});
    }
    if (ks < nk) step(ks, F0, F1, P0{}, NoRefill{});

    if constexpr (EPI == EPI_STORE && NJ == 2) {
        if (ro.Q && !P) {  // q|k|v with RoPE and the K/V rows (one head per wave)
            const int hc = n0 + 64 * wn, r32 = lane & 31;
            if (hc < N) {
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        float v0 = acc[i][0][e], v1 = acc[i][1][e];
                        if (bias) {
                            v0 = v0 + bias[hc + r32];
                            v1 = v1 + bias[hc + 32 + r32];
                        }
                        rope_store2(ro, m, M, hc, r32, v0, v1);
                    }
            }
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        const int n = n0 + 32 * NJ * wn + 32 * j + (lane & 31);
#pragma unroll
        for (int i = 0; i < 2; i++) {
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const float v = acc[i][j][e];
                if (P) {
                    if (m < M && n < N) P[((size_t)z * M + m) * N + n] = v;
                } else if constexpr (EPI == EPI_SWIGLU) {
                    // lanes 2c and 2c + 1 hold the gate and up columns of one
                    // hidden unit for rows m (element e) and m + 1 (e + 1):
                    // one exchange gives the even lane row m's pair and the
                    // odd lane row m + 1's, so every lane computes a unit
                    if ((e & 1) == 0) {
                        const bool odd = lane & 1;
                        const float w = acc[i][j][e + 1];
                        const float r = xshfl<1>(odd ? v : w);
                        const int mr = m + (odd ? 1 : 0);
                        if (mr < M && n < N) store_swiglu(Y, Yh, Yl, mr, n / 2, ldy, odd ? r : v, odd ? w : r);
                    }
                } else if (m < M && n < N) {
                    if constexpr (EPI == EPI_RESID)
                        Y[(size_t)m * ldy + n] += v;
                    else
                        Y[(size_t)out_row(ymap, m) * ldy + n] = bias ? v + bias[n] : v;
                }
            }
        }
    }
}

// ------------------------------------------------------------ MFMA GEMM, int8
// The Q8_0 products under llama.cpp's rounding points ("What a Llama model
// computes, and why", sections 5 and 8: the activations rounded to 8-bit
// blocks and dotted with the 8-bit weights as integers): both operands are
// Q8_0 codes in the tiled int8 layout, one 32-deep K step is one Q8_0 block on
// both sides, and each step's int32 sums (exact, below 2^24 in magnitude)
// join the fp32 accumulator times d_w * d_x (two binary16 scales: their
// product is exact in fp32). Block tile 128 (m) x 256 (n), eight waves in a
// 2 x 4 arrangement, each 64 x 64 = 2 x 2 tiles of v_mfma_i32_32x32x32_i8
// (lane l supplies row l%32's codes 16(l/32) .. +15 of the step; the result
// has the f32 32x32 layout). A stage holds the step's activation codes (4 KB),
// weight codes (8 KB), then the 128 activation and 256 weight scales as fp32
// (1.5 KB), then a zero word that no DMA touches (read by the lanes that supply
// a zero weight scale); an eight-stage DMA ring moves it, two DMAs per wave (a
// step is consumed faster than one of the binary16 kernel, so the ring holds
// more).
constexpr int I8_SW = 4096, I8_SS = 12288, I8_ZERO = 13824, I8_STAGE = 13840, I8_ST = 8;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

template <int EPI>
__global__ __launch_bounds__(512) void k_gemm_i8(Mat W, const int8_t* Ac, const float* As, int M, int kz, int nm,
                                                 int nn, float* Y, int ldy, const float* bias, __half* Yh, __half* Yl,
                                                 float* P, const int* ymap, int8_t* yc, float* ycs, RopeArgs ro) {
    __shared__ __attribute__((aligned(1024))) char lds[I8_ST * I8_STAGE];
    const int N = W.rows, K = W.cols;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // tiles that share a weight tile are dealt to one XCD and start together
    int q = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0) q = (q & 7) * (nb >> 3) + (q >> 3);
    const int mt = q % nm, nt = (q / nm) % nn;
    const int z = blockIdx.y;
    const int m0 = mt * HL_M, n0 = nt * HL_N, kb = z * kz;
    const int nkK = K / HL_K, kbs = kb / HL_K;

    // this wave's two DMAs per stage: waves 0-3 activation rows 32w .. 32w+31
    // and weight rows 32w .. +31; waves 4-7 weight rows 32w .. +31 and 384
    // bytes of the scales (lanes 0-23)
    const char* src0;
    const char* src1 = nullptr;
    size_t adv0, adv1 = 0;
    int dst0, dst1;
    const size_t wtile = ((size_t)nt * nkK + kbs) * HL_N * 32;  // weight codes of step kbs, tile nt
    if (wave < 4) {
        src0 = (const char*)Ac + (((size_t)mt * nkK + kbs) * HL_M + 32 * wave) * 32 + lane * 16;
        adv0 = (size_t)HL_M * 32;
        dst0 = 1024 * wave;
        src1 = (const char*)W.wi + wtile + (size_t)(32 * wave) * 32 + lane * 16;
        adv1 = (size_t)HL_N * 32;
        dst1 = I8_SW + 1024 * wave;
    } else {
        src0 = (const char*)W.wi + wtile + (size_t)(32 * wave) * 32 + lane * 16;
        adv0 = (size_t)HL_N * 32;
        dst0 = I8_SW + 1024 * wave;
        const int b = 384 * (wave - 4) + 16 * lane;  // byte of the stage's scales this lane moves
        dst1 = I8_SS + 384 * (wave - 4);
        if (lane < 24) {
            if (b < 4 * HL_M) {
                src1 = (const char*)(As + ((size_t)mt * nkK + kbs) * HL_M) + b;
                adv1 = (size_t)HL_M * 4;
            } else {
                src1 = (const char*)(W.si + ((size_t)nt * nkK + kbs) * HL_N) + (b - 4 * HL_M);
                adv1 = (size_t)HL_N * 4;
            }
        }
    }
    const int nk = kz / HL_K;
    auto issue = [&](int ks) {
        char* st = lds + (ks % I8_ST) * I8_STAGE;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src0 + adv0 * ks),
                                         (__attribute__((address_space(3))) void*)(st + dst0), 16, 0, 0);
        if (src1)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src1 + adv1 * ks),
                                             (__attribute__((address_space(3))) void*)(st + dst1), 16, 0, 0);
    };
    // waits until at most PEND later stages of this wave's DMAs are in
    // flight and its LDS reads have returned, then for every wave
    auto wait_c = [&](auto pend_c) {
        constexpr int n = decltype(pend_c)::value * 2;
        constexpr int imm = (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(imm);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;
    struct Frag {
        i32x4 a[2], b[2];  // [tile]
        float sx[2];       // the activation scale of row r32 of each tile
        float sw[2];       // the weight scale of column r32 of each tile
    };
    // this lane's half of its row (rows are 32-aligned but for r32, whose
    // bits 2 and 3 pick the half swap of the layout)
    const int hs = 16 * (h ^ i8_swz(r32));
    auto fread = [&](int ks, Frag& F) {
        const char* st = lds + (ks % I8_ST) * I8_STAGE;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int r = 64 * wm + 32 * i;
            F.a[i] = *(const i32x4*)(st + (r + r32) * 32 + hs);
            F.sx[i] = *(const float*)(st + I8_SS + 4 * (r + r32));
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int c = 64 * wn + 32 * j + r32;
            F.b[j] = *(const i32x4*)(st + I8_SW + c * 32 + hs);
            // lanes 32-63 read the stage's zero word: their B[8][j] is 0
            F.sw[j] = *(const float*)(st + (h ? I8_ZERO : I8_SS + 4 * HL_M + 4 * c));
        }
    };
    float16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;
    // The tile's 32 x 32 scale products d_x * d_w come from the f16 matrix
    // cores as a rank-1 product: lane l supplies element 0 of its 8-deep K
    // slice, so A[i][0] = A[i][8] = d_x of row i, B[0][j] = d_w of column j,
    // B[8][j] = 0 and every other element is 0. Both scales are binary16
    // values (the weight's stored scale, the input's rounded one), so their
    // conversion (toward zero) is exact, the matrix cores keep binary16
    // subnormals, and each product is exact in fp32, in the int8 result's
    // layout. That takes 64 multiplies per lane and step off the VALU, which
    // the fold saturates (the fp32 matrix form of the product costs as much
    // VALU time as the multiplies: its peak is the vector fp32 peak).
    //
    // The four tiles of a step are software-pipelined one tile deep: the
    // matrix cores take tile n's products while the VALU folds tile n - 1's
    // (a step's last tile is folded behind the next step's first products,
    // and once more after the last step). pt/pd hold the products of two
    // tiles; slot 1 starts as an empty tile, whose fold adds +0. The empty asm
    // after each fold keeps it ahead of the next step's barrier, past which
    // instruction selection would otherwise sink it.
    i32x16 pt[2];
    float16v pd[2];
#pragma unroll
    for (int e = 0; e < 16; e++) pt[1][e] = 0, pd[1][e] = 0.f;
    auto fold = [&](int n) {
#pragma unroll
        for (int e = 0; e < 16; e++) acc[n >> 1][n & 1][e] += (float)pt[n & 1][e] * pd[n & 1][e];
    };
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 xq[2], wq[2];
#pragma unroll
    for (int t = 0; t < 2; t++) xq[t] = wq[t] = (u32x4){0u, 0u, 0u, 0u};
    auto fmma = [&](const Frag& F) {
#pragma unroll
        for (int n = 0; n < 4; n++) {
            const int i = n >> 1, j = n & 1;
            pt[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F.a[i], F.b[j], (i32x16){}, 0, 0, 0);
            if (n < 2) {
                xq[n].x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(F.sx[n], 0.f));
                wq[n].x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(F.sw[n], 0.f));
            }
            pd[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, xq[i]),
                                                           __builtin_bit_cast(half8, wq[j]), (float16v){}, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            fold((n + 3) & 3);
            asm volatile("" : "+v"(acc[((n + 3) & 3) >> 1][(n + 3) & 1]));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using std::integral_constant;
    // the stages' zero words (the first wait below, an LDS count of 0 and a
    // barrier, orders these stores before every fragment read)
    if (threadIdx.x < I8_ST) *(float*)(lds + threadIdx.x * I8_STAGE + I8_ZERO) = 0.f;
    for (int p = 0; p < I8_ST && p < nk; p++) issue(p);
    // stage 0 has landed once at most I8_ST - 1 later stages remain (a K
    // shorter than the ring waits for all of them)
    if (nk >= I8_ST)
        wait_c(integral_constant<int, I8_ST - 1>{});
    else
        wait_c(integral_constant<int, 0>{});
    Frag F0, F1;
    fread(0, F0);
    // one K step: wait for the next step's stage, refill the slot this step
    // was read from, read the next fragments, multiply the current ones (the
    // steady steps with I8_ST - 2 later stages in flight, the last ones with
    // none)
    auto step = [&](int ks, Frag& cur, Frag& nxt, auto pend_c, auto refill_c) {
        wait_c(pend_c);
        if constexpr (decltype(refill_c)::value) issue(ks + I8_ST);
        fread(min(ks + 1, nk - 1), nxt);
        __builtin_amdgcn_sched_barrier(0);
        fmma(cur);
    };
    using P0 = integral_constant<int, 0>;
    using PS = integral_constant<int, I8_ST - 2>;
    const int nsteady = nk > I8_ST ? nk - I8_ST : 0;
    int ks = 0;
    for (; ks + 1 < nsteady; ks += 2) {
        step(ks, F0, F1, PS{}, std::true_type{});
        step(ks + 1, F1, F0, PS{}, std::true_type{});
    }
    if (ks < nsteady) {
        step(ks, F0, F1, PS{}, std::true_type{});
        ks++;
        F0 = F1;
    }
    for (; ks + 1 < nk; ks += 2) {
        step(ks, F0, F1, P0{}, std::false_type{});
        step(ks + 1, F1, F0, P0{}, std::false_type{});
    }
    if (ks < nk) step(ks, F0, F1, P0{}, std::false_type{});
    fold(3);

    if constexpr (EPI == EPI_STORE) {
        if (ro.Q && !P) {  // q|k|v with RoPE and the K/V rows (one head per wave)
            const int hc = n0 + 64 * wn;
            if (hc < N) {
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
                        float v0 = acc[i][0][e], v1 = acc[i][1][e];
                        if (bias) {
                            v0 = v0 + bias[hc + r32];
                            v1 = v1 + bias[hc + 32 + r32];
                        }
                        rope_store2(ro, m, M, hc, r32, v0, v1);
                    }
            }
            return;
        }
    }
    if constexpr (EPI == EPI_SWIGLU) {
        if (yc && !P) {
            // The down product's input as Q8_0 codes, computed as the row
            // rounding computes them. One block of 32 hidden units of a row is
            // this wave's 64 interleaved columns: units ub + 16 j + k from
            // tile j, unit ub + 16 j + k of row m in lane 2k and of row m + 1
            // in lane 2k + 1 after the pair exchange, so the block's maximum
            // is a reduction over the 16 lanes of one parity.
            const int ub = (n0 + 64 * wn) / 2, k = r32 >> 1;
            const bool odd = lane & 1;
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const int mr = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3) + (odd ? 1 : 0);
                    float u[2];
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const float v = acc[i][j][e], w = acc[i][j][e + 1];
                        const float r = xshfl<1>(odd ? v : w);
                        u[j] = pf_silu(odd ? r : v) * (odd ? w : r);
                    }
                    float amax = fmaxf(fabsf(u[0]), fabsf(u[1]));
                    amax = fmaxf(amax, xshfl<2>(amax));
                    amax = fmaxf(amax, xshfl<4>(amax));
                    amax = fmaxf(amax, xshfl<8>(amax));
                    amax = fmaxf(amax, xshfl<16>(amax));
                    const float d = amax / 127.f, id = d != 0.f ? 1.f / d : 0.f;
                    if (mr < M && 2 * ub < N) {
#pragma unroll
                        for (int j = 0; j < 2; j++)
                            yc[tile_off_i8(mr, ub + 16 * j + k, ldy, kTileA)] = (int8_t)roundf(u[j] * id);
                        if (k == 0) ycs[tile_off_s(mr, ub >> 5, ldy, kTileA)] = round16(d);
                    }
                }
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int n = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
        for (int i = 0; i < 2; i++) {
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
                const float v = acc[i][j][e];
                if (P) {
                    if (m < M && n < N) P[((size_t)z * M + m) * N + n] = v;
                } else if constexpr (EPI == EPI_SWIGLU) {
                    // lanes 2c and 2c + 1 hold the gate and up columns of one
                    // hidden unit for rows m (element e) and m + 1 (e + 1):
                    // one exchange gives the even lane row m's pair and the
                    // odd lane row m + 1's, so every lane computes a unit
                    if ((e & 1) == 0) {
                        const bool odd = lane & 1;
                        const float w = acc[i][j][e + 1];
                        const float r = xshfl<1>(odd ? v : w);
                        const int mr = m + (odd ? 1 : 0);
                        if (mr < M && n < N) store_swiglu(Y, Yh, Yl, mr, n / 2, ldy, odd ? r : v, odd ? w : r);
                    }
                } else if (m < M && n < N) {
                    if constexpr (EPI == EPI_RESID)
                        Y[(size_t)m * ldy + n] += v;
                    else
                        Y[(size_t)out_row(ymap, m) * ldy + n] = bias ? v + bias[n] : v;
                }
            }
        }
    }
}

// Splits of K for an M x N product on tiles of tm x tn: K is halved until the
// blocks fill three quarters of the 256 compute units (one block each; past
// that a split adds a round of blocks plus the reduction and gains nothing),
// each split at least 256 deep and a multiple of 32, the partials within
// ws_floats.
#ifndef LLM_SPLIT_FILL
#define LLM_SPLIT_FILL 192
#endif
static int gemm_splits(int M, int N, int K, int tm, int tn, int smax, size_t ws_floats) {
    const int tiles = ((N + tn - 1) / tn) * ((M + tm - 1) / tm);
    int S = 1;
    while (tiles * S < LLM_SPLIT_FILL && 2 * S <= smax && (K / (2 * S)) % 32 == 0 && K / (2 * S) >= 256 &&
           (size_t)2 * S * M * N <= ws_floats)
        S *= 2;
    return S;
}

template <int EPI>
static hipError_t gemm_epi(const Mat& W, const GemmA& A, int n, float* Y, int ldy, const float* bias, __half* Yh,
                           __half* Yl, float* ws, size_t ws_floats, hipStream_t s, const int* ymap, int* defer,
                           int8_t* yc, float* ycs, int* yc_done, const RopeArgs* ro, int* ro_done) {
    if (defer) *defer = 0;
    if (yc_done) *yc_done = 0;
    if (ro_done) *ro_done = 0;
    const RopeArgs ro_off{};
    const int N = W.rows, K = W.cols;
    int S = 1;
    if (W.dtype == DT_Q8 && W.wi && W.si && A.c && A.cs && K % HL_K == 0) {
        S = gemm_splits(n, N, K, HL_M, HL_N, 8, ws_floats);
        const int nm = (n + HL_M - 1) / HL_M, nn = (N + HL_N - 1) / HL_N;
        // a SwiGLU product over one K split may write its output as codes
        const bool fuse = EPI == EPI_SWIGLU && yc && S == 1 && ldy % 32 == 0;
        // a q|k|v product over one K split may apply RoPE and write Q and the cache rows
        const bool rfuse = EPI == EPI_STORE && ro && S == 1 && !ymap;
        hipLaunchKernelGGL((k_gemm_i8<EPI>), dim3(nm * nn, S), dim3(512), 0, s, W, A.c, A.cs, n, K / S, nm, nn,
                           fuse ? nullptr : Y, ldy, bias, Yh, Yl, S > 1 ? ws : nullptr, ymap, fuse ? yc : nullptr,
                           fuse ? ycs : nullptr, rfuse ? *ro : ro_off);
        if (yc_done) *yc_done = fuse;
        if (ro_done) *ro_done = rfuse;
    } else if (W.dtype == DT_F32) {
        dim3 grid((N + GF_T - 1) / GF_T, (n + GF_T - 1) / GF_T);
        hipLaunchKernelGGL((k_gemm_f32<EPI>), grid, dim3(256), 0, s, W, A.f, n, Y, ldy, bias, Yh, Yl, ymap);
    } else if ((W.dtype == DT_F16 || (W.dtype == DT_Q8 && W.st)) && W.wt && A.h && K % HL_K == 0) {
        S = gemm_splits(n, N, K, HL_M, HL_N, 8, ws_floats);
        const int nm = (n + HL_M - 1) / HL_M, nn = (N + HL_N - 1) / HL_N;
        float* Pw = S > 1 ? ws : nullptr;
        // (the fused q|k|v epilogue needs 64-column wave tiles: eight waves)
        const bool rfuse = EPI == EPI_STORE && ro && S == 1 && !ymap && (W.dtype == DT_Q8 || LLM_HL_WAVES == 8);
        const RopeArgs& rk = rfuse ? *ro : ro_off;
        // without a lo plane the activations are binary16: one product per tile
        if (W.dtype == DT_Q8) {
            if (A.l)
                hipLaunchKernelGGL((k_gemm_hl<EPI, 8, true, true>), dim3(nm * nn, S), dim3(512), 0, s, W, A.h, A.l, n,
                                   K / S, nm, nn, Y, ldy, bias, Yh, Yl, Pw, ymap, rk);
            else
                hipLaunchKernelGGL((k_gemm_hl<EPI, 8, false, true>), dim3(nm * nn, S), dim3(512), 0, s, W, A.h, A.h, n,
                                   K / S, nm, nn, Y, ldy, bias, Yh, Yl, Pw, ymap, rk);
        } else if (A.l) {
            hipLaunchKernelGGL((k_gemm_hl<EPI, LLM_HL_WAVES, true, false>), dim3(nm * nn, S), dim3(64 * LLM_HL_WAVES), 0,
                               s, W, A.h, A.l, n, K / S, nm, nn, Y, ldy, bias, Yh, Yl, Pw, ymap, rk);
        } else {
            hipLaunchKernelGGL((k_gemm_hl<EPI, LLM_HL_WAVES, false, false>), dim3(nm * nn, S), dim3(64 * LLM_HL_WAVES),
                               0, s, W, A.h, A.h, n, K / S, nm, nn, Y, ldy, bias, Yh, Yl, Pw, ymap, rk);
        }
        if (ro_done) *ro_done = rfuse;
    } else {
        S = gemm_splits(n, N, K, GB_M, GB_N, 4, ws_floats);
        dim3 grid((N + GB_N - 1) / GB_N, (n + GB_M - 1) / GB_M, S);
        float* P = S > 1 ? ws : nullptr;
        if (W.dtype == DT_F16)
            hipLaunchKernelGGL((k_gemm_mfma<DT_F16, EPI>), grid, dim3(256), 0, s, W, A.f, n, Y, ldy, bias, Yh, Yl,
                               K / S, P, ymap);
        else
            hipLaunchKernelGGL((k_gemm_mfma<DT_Q8, EPI>), grid, dim3(256), 0, s, W, A.f, n, Y, ldy, bias, Yh, Yl,
                               K / S, P, ymap);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    if (defer) {  // the caller reduces the S partials in ws itself
        *defer = S;
        return hipSuccess;
    }
    if constexpr (EPI == EPI_STORE) {
        if (ro && !ymap) {  // the q|k|v partials go straight to RoPE and the K/V rows
            const int pairs = n * (N / 2);
            hipLaunchKernelGGL(k_splitk_rope, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, s, ws, S, n, bias,
                               *ro);
            if (ro_done) *ro_done = 1;
            return hipGetLastError();
        }
    }
    const size_t items = EPI == EPI_SWIGLU ? (size_t)n * N / 2 : (size_t)n * N;
    hipLaunchKernelGGL((k_splitk_reduce<EPI>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, ws, S, n, N, Y,
                       ldy, bias, Yh, Yl, ymap);
    return hipGetLastError();
}

hipError_t launch_gemm(int epi, const Mat& W, const GemmA& A, int n, float* Y, int ldy, const float* bias,
                       __half* Yh, __half* Yl, float* ws, size_t ws_floats, hipStream_t s, const int* ymap,
                       int* defer, int8_t* yc, float* ycs, int* yc_done, const RopeArgs* ro, int* ro_done) {
    if ((ymap && epi != EPI_STORE) || (defer && epi != EPI_RESID) || (yc && (epi != EPI_SWIGLU || !ycs || Yh)) ||
        (ro && (epi != EPI_STORE || ymap || !ro->Q || !ro->kc || !ro->vc || !ro->rope || Yh || ldy % 64)))
        return hipErrorInvalidValue;
    switch (epi) {
        case EPI_STORE:
            return gemm_epi<EPI_STORE>(W, A, n, Y, ldy, bias, Yh, Yl, ws, ws_floats, s, ymap, defer, yc, ycs, yc_done,
                                       ro, ro_done);
        case EPI_RESID:
            return gemm_epi<EPI_RESID>(W, A, n, Y, ldy, bias, Yh, Yl, ws, ws_floats, s, ymap, defer, yc, ycs, yc_done,
                                       ro, ro_done);
        case EPI_SWIGLU:
            return gemm_epi<EPI_SWIGLU>(W, A, n, Y, ldy, bias, Yh, Yl, ws, ws_floats, s, ymap, defer, yc, ycs,
                                        yc_done, ro, ro_done);
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------ causal attention on the matrix cores
// Prefill attention for head_dim 64 ("The Forward Pass in Java", Example 7,
// over the batch as in "What a Llama model computes, and why", section 4):
// query z at position p0 + z attends cache rows 0 .. p0 + z of its KV head.
// A block takes 64 (token, head) rows that share KV head g: row r is token
// z0 + r / G, query head g*G + r % G; wave w owns rows 16w .. 16w+15. Cache
// rows stream through LDS 64 positions at a time (K as stored, V transposed);
// per chunk each wave forms its 16 x 64 scores with the 16x16x32 instruction
// (q as a hi/lo binary16 pair, K exact), divides them by sqrt(head_dim),
// masks positions past each row's own, updates the running max m and sum l
// of the online softmax, and adds P V (P as a hi/lo pair, V exact) to its
// 16 x 64 output, rescaled by e^(m_old - m_new). Both products run
// transposed (S^T = K Q^T, O^T = V^T P^T): a lane then holds 16 scores and
// 16 outputs of one row, its softmax state is its own (two exchanges per
// reduction), and P^T is the lane's own registers, with no LDS round trip. The result o / l goes out
// as fp32 rows and as their hi/lo planes (the output product's input).
// With an attention span (a window plus sinks) each row masks the positions
// outside its own span, and chunks outside every row's span are skipped; q
// is scaled by its position's attention temperature before the split.
// The rounding mode (llama.cpp's rounding points, "What a Llama model computes, and why",
// section 8): q is rounded to binary16 (one product per score tile), a first
// pass over the chunks finds each row's span maximum M and sum L, and the
// second weights V with the probabilities f16(e^(s - M) / L), which are the
// binary16 operand of the P V product themselves.
// Long contexts split a block's chunks over gridDim.z blocks (cps chunks
// each) that write their rows' (m, l, unnormalised o) to part, [row][head]
// [split][2 + 64]; k_attn_prefill_merge then combines the splits.
constexpr int PA_ROWS = 64, PA_CH = 64, PA_LD = 72;
constexpr float kPaInvDiv = 0.125f;  // 1 / (float)sqrt(64), exact
#ifndef LLM_PA_CHUNKS
#define LLM_PA_CHUNKS 32
#endif
constexpr int kPaChunks = LLM_PA_CHUNKS;

// e^x through the hardware base-2 exponential: x * log2(e) rounded once, then
// v_exp_f32 (within a few ulps of expf over the softmax's range; e^-inf = 0).
__device__ __forceinline__ float pa_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
// e^(x/8) for an unscaled score difference x: the same as pa_exp(x/8), since
// scaling by 1/8 is exact and moves into the constant (log2(e)/8 is exact too)
__device__ __forceinline__ float pa_exp8(float x) {
    return __builtin_amdgcn_exp2f(x * (1.44269504088896341f * 0.125f));
}

template <bool RND>
__global__ __launch_bounds__(256) void k_attn_prefill_mfma(const float* Q, const __half* kc, const __half* vc,
                                                           float* out, __half* out_h, __half* out_l, int n_q, int p0,
                                                           int n_heads, int n_kv_heads, int n_ctx, float scale_div,
                                                           SpanCfg span, int cps, float* part, int8_t* oc,
                                                           float* ocs) {
    constexpr int hd = 64;
    (void)scale_div;  // always 8 here (checked at launch): the scores are scaled by kPaInvDiv = 1/8
    __shared__ __attribute__((aligned(16))) __half Ks[PA_CH * PA_LD];   // [position][dim]
    __shared__ __attribute__((aligned(16))) __half Vt[hd * PA_LD];      // [dim][position]
    const int G = n_heads / n_kv_heads, TB = PA_ROWS / G;
    // blocks are dealt out in index order, so the latest query rows (the most
    // causal work) come first, for every KV head, and short blocks fill the tail
    const int g = blockIdx.x, z0 = (gridDim.y - 1 - blockIdx.y) * TB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qd = n_heads * hd;
    const int lr = lane & 15, lq = lane >> 4;

    // q fragments of this lane's row (row lr of the wave) as hi/lo pairs
    const int ra = 16 * wave + lr;
    const int za = min(z0 + ra / G, n_q - 1), ha = g * G + ra % G;
    half8 qh[2], ql[2];
    const float tau = attn_temp(span, p0 + za);
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
        const float* qp = Q + (size_t)za * qd + ha * hd + 32 * ks + 8 * lq;
        const float4 a0 = *(const float4*)qp, a1 = *(const float4*)(qp + 4);
        const float v[8] = {tau * a0.x, tau * a0.y, tau * a0.z, tau * a0.w,
                            tau * a1.x, tau * a1.y, tau * a1.z, tau * a1.w};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const _Float16 h = (_Float16)v[j];
            qh[ks][j] = h;
            ql[ks][j] = RND ? (_Float16)0.f : (_Float16)(v[j] - (float)h);
        }
    }
    // the lane's row is ra (the row of its q fragments): the products run
    // transposed, S^T = K Q^T and O^T = V^T P^T, so the lane holds 16 of its
    // row's scores and 16 of its row's outputs, and the row's softmax state
    // is the lane's own
    const int rp = p0 + z0 + ra / G;
    float m_run = -INFINITY, l_run = 0.f;
    float4v o[4];
#pragma unroll
    for (int i = 0; i < 4; i++) o[i] = (float4v){0.f, 0.f, 0.f, 0.f};

    const int last = p0 + min(z0 + TB, n_q) - 1;  // the block's last position
    const int rfirst = p0 + z0;                     // and its first
    const int nch = last / PA_CH + 1;
    // chunks in use: with a window, the sink chunks (below the first row's
    // window) and then the chunks from the first row's window start on;
    // virtual chunk v is chunk v for v < nA, cB + (v - nA) after
    int nA = 0, cB = 0;
    if (span.window > 0) {
        const int lo = max(0, p0 + z0 - span.window + 1);
        cB = lo / PA_CH;
        nA = min((span.sinks + PA_CH - 1) / PA_CH, cB);
    }
    const int nv = nA + nch - cB;
    auto chunk_of = [&](int v) { return v < nA ? v : cB + (v - nA); };
    const __half* kbase = kc + (size_t)g * n_ctx * hd;
    const __half* vbase = vc + (size_t)g * n_ctx * hd;
    // loader: thread t moves position t/8 (+32) dims 8*(t%8) .. +8 of K and V
    const int lp = tid >> 3, ld8 = (tid & 7) * 8;
    const u32x4p z4 = {0u, 0u, 0u, 0u};
    u32x4p kr[2], vr[2];
    // (V only where the pass weights it: the rounding mode's first pass reads K alone)
    auto load = [&](int c0, bool with_v) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int t = c0 + lp + 32 * u;
            const bool ok = t <= last;  // rows past the block's last position are never written yet
            kr[u] = ok ? *(const u32x4p*)(kbase + (size_t)t * hd + ld8) : z4;
            if (with_v) vr[u] = ok ? *(const u32x4p*)(vbase + (size_t)t * hd + ld8) : z4;
        }
    };
    float Mrow = 0.f, Lrow = 1.f, Rrow = 1.f;  // rounding mode: the row's span maximum and sum, and 1 / sum
    for (int pass = RND ? 0 : 1; pass < 2; pass++) {
    if (RND && pass == 1) {
        Mrow = m_run;
        Lrow = l_run;
        Rrow = 1.f / Lrow;
    }
    // this block's share of the chunks
    const int v_begin = RND ? 0 : min(nv, (int)blockIdx.z * cps), v_end = RND ? nv : min(nv, v_begin + cps);
    const bool with_v = !RND || pass == 1;
    if (v_begin < v_end) load(chunk_of(v_begin) * PA_CH, with_v);
    for (int v = v_begin; v < v_end; v++) {
        const int c0 = chunk_of(v) * PA_CH;
        __syncthreads();  // the previous chunk's K, V and P reads are done
#pragma unroll
        for (int u = 0; u < 2; u++) {
            *(u32x4p*)(Ks + (lp + 32 * u) * PA_LD + ld8) = kr[u];
            if (with_v) {
                // V transposed: half j of this thread goes to row ld8 + j. Store
                // step s writes half (s + a) & 7, a = ld8 / 8, so that the lanes
                // of one store reach rows of eight different residues mod 8
                // (the same residue for all would put every lane in one group of
                // banks): the eight halves are first rotated left by a.
                const int a = ld8 >> 3;
                uint32_t w[4] = {vr[u][0], vr[u][1], vr[u][2], vr[u][3]};
                uint32_t t[4];
#pragma unroll
                for (int k = 0; k < 4; k++) t[k] = __builtin_amdgcn_alignbit(w[(k + 1) & 3], w[k], 16);
#pragma unroll
                for (int k = 0; k < 4; k++) w[k] = (a & 1) ? t[k] : w[k];
#pragma unroll
                for (int k = 0; k < 4; k++) t[k] = w[(k + 1) & 3];
#pragma unroll
                for (int k = 0; k < 4; k++) w[k] = (a & 2) ? t[k] : w[k];
#pragma unroll
                for (int k = 0; k < 4; k++) t[k] = w[(k + 2) & 3];
#pragma unroll
                for (int k = 0; k < 4; k++) w[k] = (a & 4) ? t[k] : w[k];
                uint16_t* vt16 = (uint16_t*)Vt + lp + 32 * u;
#pragma unroll
                for (int st = 0; st < 8; st++)
                    vt16[(ld8 + ((st + a) & 7)) * PA_LD] = (uint16_t)(w[st >> 1] >> (16 * (st & 1)));
            }
        }
        __syncthreads();
        if (v + 1 < v_end) load(chunk_of(v + 1) * PA_CH, with_v);

        // scores over the chunk, transposed: tile pt covers positions
        // c0 + 16 pt .. +15, and the lane gets its row's scores at positions
        // c0 + 16 pt + 4 lq + i in sc[pt][i]
        float4v sc[4];
#pragma unroll
        for (int pt = 0; pt < 4; pt++) {
            sc[pt] = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const half8 kf = *(const half8*)(Ks + (16 * pt + lr) * PA_LD + 32 * ks + 8 * lq);
                sc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qh[ks], sc[pt], 0, 0, 0);
                if constexpr (!RND) sc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, ql[ks], sc[pt], 0, 0, 0);
            }
        }
        // A chunk every row of the block attends in full needs no mask: all of
        // it at or before the block's first position (causal) and, with a
        // window, after the window start of its last position (rows past the
        // last position are padding, never stored).
        const bool full = c0 + PA_CH - 1 <= rfirst && (span.window <= 0 || c0 > last - span.window);
        // o^T += V^T P^T over the chunk's 64 positions, two 32-deep steps. The
        // K index of a step may map to positions in any order that P^T and
        // V^T share: k = 8 lq + j is position 32 ps + 16 (j / 4) + 4 lq + j % 4,
        // which is the lane's own score sc[2 ps + j / 4][j % 4], and V^T's
        // row d supplies it as two runs of four positions from Vt.
        auto pv = [&](int ps, const half8& ph, bool lo_too, const half8& pl) {
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                const __half* vrow = Vt + (16 * dt + lr) * PA_LD + 32 * ps + 4 * lq;
                const uint2 v0 = *(const uint2*)vrow, v1 = *(const uint2*)(vrow + 16);
                const half8 vf = __builtin_bit_cast(half8, (u32x4p){v0.x, v0.y, v1.x, v1.y});
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph, o[dt], 0, 0, 0);
                if (lo_too) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl, o[dt], 0, 0, 0);
            }
        };
        if (RND && pass == 1) {
            // the rounded probabilities of the whole span, the P V operand as is
#pragma unroll
            for (int ps = 0; ps < 2; ps++) {
                half8 ph;
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const int pt = 2 * ps + (j >> 2), i = j & 3;
                    const int t = c0 + 16 * pt + 4 * lq + i;
                    // e / L, correctly rounded, from the correctly rounded 1 / L:
                    // q = e r is within an ulp of e / L, its residual e - q L is
                    // exact (an FMA), and q + (e - q L) r rounds to e / L
                    // (Markstein's division step) unless the residual
                    // underflows, for quotients below about 2^-120, which are
                    // 0 in binary16 either way
                    const float ex = full || span_has(span, t, rp) ? pa_exp8(sc[pt][i] - Mrow) : 0.f;
                    const float q0 = ex * Rrow;
                    float e = fmaf(fmaf(-q0, Lrow, ex), Rrow, q0);
                    // (rounded to fp32 first, as the quotient is, before binary16)
                    asm volatile("" : "+v"(e));
                    ph[j] = (_Float16)e;
                }
                pv(ps, ph, false, ph);
            }
            continue;
        }
        // online softmax of the lane's row: its 64 scores sit in the four
        // lanes with the same lr, 16 each. The scores and the running maximum
        // stay unscaled (the 1/8 goes into the exponentials, pa_exp8); a chunk
        // the row attends in full has only finite scores, so its maximum is
        // finite and its exponentials need no test for masked positions.
        float mx = -INFINITY;
#pragma unroll
        for (int pt = 0; pt < 4; pt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int t = c0 + 16 * pt + 4 * lq + i;
                const float sv = full || span_has(span, t, rp) ? sc[pt][i] : -INFINITY;
                sc[pt][i] = sv;
                mx = fmaxf(mx, sv);
            }
        mx = fmaxf(mx, xshfl<16>(mx));
        mx = fmaxf(mx, xshfl<32>(mx));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.f : pa_exp8(m_run - m_new);
        float ls = 0.f;
        if (full) {
#pragma unroll
            for (int pt = 0; pt < 4; pt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float e = pa_exp8(sc[pt][i] - m_new);
                    sc[pt][i] = e;
                    ls += e;
                }
        } else {
#pragma unroll
            for (int pt = 0; pt < 4; pt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float e = sc[pt][i] == -INFINITY ? 0.f : pa_exp8(sc[pt][i] - m_new);
                    sc[pt][i] = e;
                    ls += e;
                }
        }
        ls += xshfl<16>(ls);
        ls += xshfl<32>(ls);
        l_run = l_run * alpha + ls;
        m_run = m_new;
        if (RND) continue;  // the first pass only finds M and L
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
            for (int i = 0; i < 4; i++) o[dt][i] *= alpha;
#pragma unroll
        for (int ps = 0; ps < 2; ps++) {
            half8 ph, pl;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float pj = sc[2 * ps + (j >> 2)][j & 3];
                const _Float16 h = (_Float16)pj;
                ph[j] = h;
                pl[j] = (_Float16)(pj - (float)h);
            }
            pv(ps, ph, true, pl);
        }
    }
    }
    const int z = z0 + ra / G, h = g * G + ra % G;
    if (gridDim.z > 1) {  // this split's (m, l, o) of the lane's row for the merge
        const int S = gridDim.z, sp = blockIdx.z;
        if (z < n_q) {
            float* pr = part + (((size_t)z * n_heads + h) * S + sp) * (hd + 2);
            if (lq == 0) {
                pr[0] = m_run * kPaInvDiv;  // the maximum in scaled units (exact)
                pr[1] = l_run;
            }
#pragma unroll
            for (int dt = 0; dt < 4; dt++)
#pragma unroll
                for (int i = 0; i < 4; i++) pr[2 + 16 * dt + 4 * lq + i] = o[dt][i];
        }
        return;
    }
    // out[z][h*64 + d] = o / l for the lane's row, dims 16 dt + 4 lq + i
    if (z >= n_q) return;
    if constexpr (RND) {
        if (oc) {
            // the output product's input as Q8_0 codes, as the row rounding
            // computes them: block bh of the head (dims 32 bh .. +31) is dt
            // 2 bh and 2 bh + 1 of the row's four lanes (same lr)
#pragma unroll
            for (int bh = 0; bh < 2; bh++) {
                float amax = 0.f;
#pragma unroll
                for (int u = 0; u < 2; u++)
#pragma unroll
                    for (int i = 0; i < 4; i++) amax = fmaxf(amax, fabsf(o[2 * bh + u][i]));
                amax = fmaxf(amax, xshfl<16>(amax));
                amax = fmaxf(amax, xshfl<32>(amax));
                const float d = amax / 127.f, id = d != 0.f ? 1.f / d : 0.f;
#pragma unroll
                for (int u = 0; u < 2; u++) {
                    uint32_t q = 0u;
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        q |= (uint32_t)(uint8_t)(int8_t)roundf(o[2 * bh + u][i] * id) << (8 * i);
                    *(uint32_t*)(oc + tile_off_i8(z, h * hd + 32 * bh + 16 * u + 4 * lq, qd, kTileA)) = q;
                }
                if (lq == 0) ocs[tile_off_s(z, (h * hd + 32 * bh) >> 5, qd, kTileA)] = round16(d);
            }
        }
    }
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float v = RND ? o[dt][i] : o[dt][i] / l_run;
            const int col = h * hd + 16 * dt + 4 * lq + i;
            if (out) out[(size_t)z * qd + col] = v;
            if (out_h) {
                const __half hh = __float2half_rn(v);
                const size_t t = tile_off(z, col, qd, kTileA);
                out_h[t] = hh;
                out_l[t] = __float2half_rn(v - __half2float(hh));
            }
        }
}

// The splits of each (row, head): M = max m_s, L = sum l_s e^(m_s - M),
// out = sum o_s e^(m_s - M) / L in split order, with the hi/lo planes. One
// 64-lane wave per (row, head), a lane per dimension.
__global__ __launch_bounds__(256) void k_attn_prefill_merge(const float* part, int S, int n_q, int n_heads, float* out,
                                                            __half* out_h, __half* out_l) {
    constexpr int hd = 64;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6), d = threadIdx.x & 63;
    if (item >= n_q * n_heads) return;
    const int z = item / n_heads, h = item % n_heads;
    const float* pr = part + (size_t)item * S * (hd + 2);
    float M = -INFINITY;
    for (int j = 0; j < S; j++) M = fmaxf(M, pr[(size_t)j * (hd + 2)]);
    float L = 0.f, O = 0.f;
    for (int j = 0; j < S; j++) {
        const float* pj = pr + (size_t)j * (hd + 2);
        const float f = pj[0] == -INFINITY ? 0.f : expf(pj[0] - M);
        L += pj[1] * f;
        O += pj[2 + d] * f;
    }
    const float v = O / L;
    const int qd = n_heads * hd, col = h * hd + d;
    if (out) out[(size_t)z * qd + col] = v;
    if (out_h) {
        const __half hh = __float2half_rn(v);
        const size_t t = tile_off(z, col, qd, kTileA);
        out_h[t] = hh;
        out_l[t] = __float2half_rn(v - __half2float(hh));
    }
}

hipError_t launch_attn_prefill_mfma(const float* Q, const __half* kc, const __half* vc, float* out, __half* out_h,
                                    __half* out_l, int n_q, int p0, int n_heads, int n_kv_heads, int head_dim,
                                    int n_ctx, float scale_div, const SpanCfg& span, bool rnd, float* ws,
                                    size_t ws_floats, hipStream_t s, int8_t* oc, float* ocs) {
    const int G = n_kv_heads > 0 ? n_heads / n_kv_heads : 0;
    // the kernel multiplies the scores by 1/8: exactly the division by
    // (float)sqrt(64) = 8, a power of two
    if (head_dim != 64 || scale_div != 8.0f || G < 1 || G > PA_ROWS || PA_ROWS % G || n_heads % n_kv_heads ||
        n_q <= 0 || (oc && (!rnd || !ocs)))
        return hipErrorInvalidValue;
    const int TB = PA_ROWS / G;
    const dim3 grid(n_kv_heads, (n_q + TB - 1) / TB);  // KV head, query-row block from the last
    if (rnd) {
        hipLaunchKernelGGL(k_attn_prefill_mfma<true>, grid, dim3(256), 0, s, Q, kc, vc, out, out_h, out_l, n_q, p0,
                           n_heads, n_kv_heads, n_ctx, scale_div, span, 0, nullptr, oc, ocs);
        return hipGetLastError();
    }
    // at most kPaChunks chunks of 64 positions per block: longer contexts split
    const int nch = (p0 + n_q - 1) / PA_CH + 1;
    int S = (nch + kPaChunks - 1) / kPaChunks;
    if (S > 8) S = 8;
    while (S > 1 && (size_t)n_q * n_heads * S * (head_dim + 2) > ws_floats) S--;
    const int cps = (nch + S - 1) / S;
    hipLaunchKernelGGL(k_attn_prefill_mfma<false>, dim3(grid.x, grid.y, S), dim3(256), 0, s, Q, kc, vc, out, out_h,
                       out_l, n_q, p0, n_heads, n_kv_heads, n_ctx, scale_div, span, cps, S > 1 ? ws : nullptr, nullptr,
                       nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    hipLaunchKernelGGL(k_attn_prefill_merge, dim3((unsigned)((n_q * n_heads + 3) / 4)), dim3(256), 0, s, ws, S, n_q,
                       n_heads, out, out_h, out_l);
    return hipGetLastError();
}

// ------------------------------------------------------------ RoPE + KV rows
// Row i of the batch is at position p0 + i. Each thread takes one rotation pair
// of one row (pairs as in the decode epilogue: (2j, 2j+1) normal, (j, j+n_rot/2)
// NEOX, "The Forward Pass in Java", Example 6), rotates q and k pairs with the
// table, writes q to Q and k, v to the F16 cache.
__global__ void k_rope_kv_rows(const float* QKV, int n, int p0, int n_heads, int n_kv_heads, int hd, int n_rot,
                               int neox, int n_ctx, const float2* rope, float* Q, __half* kc, __half* vc) {
    const int qd = n_heads * hd, kvd = n_kv_heads * hd, W = qd + 2 * kvd;
    const int hp = hd / 2, half = n_rot / 2;
    const int pairs = W / 2;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * pairs) return;
    const int row = idx / pairs, pi = idx % pairs;
    const int head = pi / hp, j = pi % hp;
    int ra, rb;
    if (j < half) {
        ra = head * hd + (neox ? j : 2 * j);
        rb = neox ? ra + half : ra + 1;
    } else {
        ra = head * hd + n_rot + 2 * (j - half);
        rb = ra + 1;
    }
    const int pos = p0 + row;
    const float* src = QKV + (size_t)row * W;
    float va = src[ra], vb = src[rb];
    if (head < n_heads + n_kv_heads && j < half) {
        const float2 cs = rope[(size_t)pos * half + j];
        const float2 rv = pf_rope_rotate(va, vb, cs);
        va = rv.x;
        vb = rv.y;
    }
    if (ra < qd) {
        Q[(size_t)row * qd + ra] = va;
        Q[(size_t)row * qd + rb] = vb;
    } else if (ra < qd + kvd) {
        const int g = (ra - qd) / hd;
        __half* r = kc + ((size_t)g * n_ctx + pos) * hd;
        r[(ra - qd) % hd] = __float2half_rn(va);
        r[(rb - qd) % hd] = __float2half_rn(vb);
    } else {
        const int g = (ra - qd - kvd) / hd;
        __half* r = vc + ((size_t)g * n_ctx + pos) * hd;
        r[(ra - qd - kvd) % hd] = __float2half_rn(va);
        r[(rb - qd - kvd) % hd] = __float2half_rn(vb);
    }
}

hipError_t launch_rope_kv_rows(const float* QKV, int n, int p0, int n_heads, int n_kv_heads, int head_dim, int n_rot,
                               int neox, int n_ctx, const float2* rope, float* Q, __half* kc, __half* vc,
                               hipStream_t s) {
    const int pairs = (n_heads + 2 * n_kv_heads) * head_dim / 2;
    const int total = n * pairs;
    hipLaunchKernelGGL(k_rope_kv_rows, dim3((total + 255) / 256), dim3(256), 0, s, QKV, n, p0, n_heads, n_kv_heads,
                       head_dim, n_rot, neox, n_ctx, rope, Q, kc, vc);
    return hipGetLastError();
}

}  // namespace llm
