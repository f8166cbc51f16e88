// layernorm.hip -- LayerNorm forward and backward over the rows of an
// (N, C) matrix for gfx950: fp32, bfloat16 or IEEE-half rows, fp32 weight, bias, mean,
// rstd and arithmetic.
//
// Method: "llm.c 的中文注解-20240423", section 1.8 (layernorm_forward_kernel3):
// per row the mean and rstd = 1/sqrt(var + 1e-5) of the row, kept for the
// backward, and out = (x - mean) * rstd * weight + bias.  "LLM Systems 10 &
// 11: Accelerating Transformer Training and Inference" (section 1.2.1,
// LayerNorm) rewrites both directions so that each needs a single
// reduction per row: the forward sums x and x^2 in one pass (variance =
// mean of squares minus squared mean), the backward sums the two terms it
// needs in one pass, storage in 16 bits with fp32 accumulation.
//
// Here:
//  * one wave per row; lanes stride the row 4 elements at a time (16-byte
//    fp32 or 8-byte bf16 loads) when C % 4 == 0, one element otherwise;
//    rows of C <= 2048 (C % 4 == 0) stay in registers between the two
//    sweeps, longer ones are read again (from cache);
//  * forward: one pass of sums of d = x - x[0] and d^2 (shifted data, so
//    that the difference of the two means does not cancel when |mean| is
//    large against the spread; the shift changes neither mean nor
//    variance), one wave reduction, then the row again (from cache) for
//    the output;
//  * backward, input gradient: with g = weight * dout and
//    xhat = (x - mean) * rstd from the forward's mean and rstd, one pass
//    sums g and g * xhat, one wave reduction, then
//    dinp = rstd * (g - mean(g) - xhat * mean(g * xhat));
//  * backward, weight and bias: partial sums of dout * xhat and dout over
//    chunks of 16 rows go to a workspace, and a last kernel adds the chunks
//    in a fixed order, so the result is bitwise deterministic (no atomics).
//    For rows held in registers the input-gradient kernel forms the
//    partials itself (each wave takes 4 rows of the chunk; the 4 waves'
//    sums meet in LDS in wave order); otherwise a separate kernel, in which
//    a thread owns four columns (one when C % 4 != 0) of a chunk, reads the
//    rows again.  dweight and dbias are written (=).
#include "common.hpp"

namespace attn {
namespace {

constexpr int kLnThreads = 256;   // 4 waves, one row each
constexpr int kLnRows = kLnThreads / 64;
constexpr float kLnEps = 1e-5f;
constexpr int kLnColThreads = 256;
constexpr int kLnFusedRpw = 4;   // rows per wave in ln_bwd_fused_kernel (16-row chunks)

struct LnF32 {
    typedef float T;
    static __device__ __forceinline__ float get(float v) { return v; }
    static __device__ __forceinline__ float put(float v) { return v; }
    static __device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[0] = x.x;
        v[1] = x.y;
        v[2] = x.z;
        v[3] = x.w;
    }
    static __device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

struct LnBF16 {
    typedef uint16_t T;
    static __device__ __forceinline__ float get(uint16_t v) {
        return __uint_as_float((uint32_t)v << 16);
    }
    static __device__ __forceinline__ uint16_t put(float v) {   // round to nearest even
        const __bf16 h = (__bf16)v;
        uint16_t u;
        __builtin_memcpy(&u, &h, 2);
        return u;
    }
    static __device__ __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        v[0] = __uint_as_float(x.x << 16);
        v[1] = __uint_as_float(x.x & 0xFFFF0000u);
        v[2] = __uint_as_float(x.y << 16);
        v[3] = __uint_as_float(x.y & 0xFFFF0000u);
    }
    static __device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
        const uint2 x = make_uint2((uint32_t)put(v[0]) | ((uint32_t)put(v[1]) << 16),
                                   (uint32_t)put(v[2]) | ((uint32_t)put(v[3]) << 16));
        *reinterpret_cast<uint2*>(p) = x;
    }
};

struct LnF16 {
    typedef uint16_t T;
    static __device__ __forceinline__ float get(uint16_t v) {
        _Float16 h;
        __builtin_memcpy(&h, &v, 2);
        return (float)h;
    }
    static __device__ __forceinline__ uint16_t put(float v) {   // round to nearest even
        const _Float16 h = (_Float16)v;
        uint16_t u;
        __builtin_memcpy(&u, &h, 2);
        return u;
    }
    static __device__ __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        v[0] = get((uint16_t)(x.x & 0xFFFFu));
        v[1] = get((uint16_t)(x.x >> 16));
        v[2] = get((uint16_t)(x.y & 0xFFFFu));
        v[3] = get((uint16_t)(x.y >> 16));
    }
    static __device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
        const uint2 x = make_uint2((uint32_t)put(v[0]) | ((uint32_t)put(v[1]) << 16),
                                   (uint32_t)put(v[2]) | ((uint32_t)put(v[3]) << 16));
        *reinterpret_cast<uint2*>(p) = x;
    }
};

// VEC consecutive elements starting at p (VEC = 4 needs p 4-element aligned)
template <typename E, int VEC>
__device__ __forceinline__ void load_row(const typename E::T* p, float (&v)[VEC]) {
    if constexpr (VEC == 4) {
        E::load4(p, v);
    } else {
        v[0] = E::get(*p);
    }
}
template <typename E, int VEC>
__device__ __forceinline__ void store_row(typename E::T* p, const float (&v)[VEC]) {
    if constexpr (VEC == 4) {
        E::store4(p, v);
    } else {
        *p = E::put(v[0]);
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// NV > 0: the row (C <= 256 * NV, C % 4 == 0) stays in registers between
// the two sweeps, NV float4 chunks per lane (lane l holds columns
// 4l + 256k .. +3); NV = 0: the second sweep reads the row again.
template <typename E, int VEC, int NV>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_kernel(typename E::T* __restrict__ out,
                                                            float* __restrict__ mean,
                                                            float* __restrict__ rstd,
                                                            const typename E::T* __restrict__ inp,
                                                            const float* __restrict__ weight,
                                                            const float* __restrict__ bias, int N,
                                                            int C) {
    static_assert(NV == 0 || VEC == 4, "a cached row is read in 4-element chunks");
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kLnRows + (threadIdx.x >> 6);
    if (row >= N) return;   // a whole wave; the kernel has no barrier
    const typename E::T* x = inp + (size_t)row * C;
    typename E::T* o = out + (size_t)row * C;
    const float shift = E::get(x[0]);
    float s1 = 0.f, s2 = 0.f;
    if constexpr (NV > 0) {
        float v[NV][4];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = 4 * lane + 256 * k;
            if (i < C) {
                load_row<E, 4>(x + i, v[k]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[k][j] = shift;   // adds 0 to both sums
            }
        }
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float d = v[k][j] - shift;
                s1 += d;
                s2 = fmaf(d, d, s2);
            }
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        const float md = s1 / (float)C;
        const float var = fmaxf(s2 / (float)C - md * md, 0.f);
        const float r = 1.0f / sqrtf(var + kLnEps);
        if (lane == 0) {
            mean[row] = shift + md;
            rstd[row] = r;
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = 4 * lane + 256 * k;
            if (i < C) {
                float w[4], b[4], y[4];
                load_row<LnF32, 4>(weight + i, w);
                load_row<LnF32, 4>(bias + i, b);
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = fmaf(((v[k][j] - shift) - md) * r, w[j], b[j]);
                store_row<E, 4>(o + i, y);
            }
        }
    } else {
        for (int i = lane * VEC; i < C; i += 64 * VEC) {
            float v[VEC];
            load_row<E, VEC>(x + i, v);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float d = v[k] - shift;
                s1 += d;
                s2 = fmaf(d, d, s2);
            }
        }
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        const float md = s1 / (float)C;                       // mean - shift
        const float var = fmaxf(s2 / (float)C - md * md, 0.f);
        const float r = 1.0f / sqrtf(var + kLnEps);
        if (lane == 0) {
            mean[row] = shift + md;
            rstd[row] = r;
        }
        for (int i = lane * VEC; i < C; i += 64 * VEC) {
            float v[VEC], w[VEC], b[VEC], y[VEC];
            load_row<E, VEC>(x + i, v);
            load_row<LnF32, VEC>(weight + i, w);
            load_row<LnF32, VEC>(bias + i, b);
#pragma unroll
            for (int k = 0; k < VEC; ++k) y[k] = fmaf(((v[k] - shift) - md) * r, w[k], b[k]);
            store_row<E, VEC>(o + i, y);
        }
    }
}

// Input gradient; NV as in ln_fwd_kernel (dout and inp rows both cached).
template <typename E, int VEC, int NV>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_dx_kernel(
    typename E::T* __restrict__ dinp, const typename E::T* __restrict__ dout,
    const typename E::T* __restrict__ inp, const float* __restrict__ weight,
    const float* __restrict__ mean, const float* __restrict__ rstd, int N, int C) {
    static_assert(NV == 0 || VEC == 4, "a cached row is read in 4-element chunks");
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kLnRows + (threadIdx.x >> 6);
    if (row >= N) return;
    const typename E::T* x = inp + (size_t)row * C;
    const typename E::T* dy = dout + (size_t)row * C;
    typename E::T* dx = dinp + (size_t)row * C;
    const float m = mean[row], r = rstd[row];
    float sg = 0.f, sgx = 0.f;
    if constexpr (NV > 0) {
        float v[NV][4], g[NV][4];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = 4 * lane + 256 * k;
            if (i < C) {
                float d[4], w[4];
                load_row<E, 4>(x + i, v[k]);
                load_row<E, 4>(dy + i, d);
                load_row<LnF32, 4>(weight + i, w);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g[k][j] = w[j] * d[j];
                    v[k][j] = (v[k][j] - m) * r;   // xhat
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) g[k][j] = v[k][j] = 0.f;
            }
        }
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sg += g[k][j];
                sgx = fmaf(g[k][j], v[k][j], sgx);
            }
        const float a = wave_sum(sg) / (float)C;
        const float c = wave_sum(sgx) / (float)C;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = 4 * lane + 256 * k;
            if (i < C) {
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = r * (g[k][j] - a - v[k][j] * c);
                store_row<E, 4>(dx + i, o);
            }
        }
    } else {
        for (int i = lane * VEC; i < C; i += 64 * VEC) {
            float v[VEC], d[VEC], w[VEC];
            load_row<E, VEC>(x + i, v);
            load_row<E, VEC>(dy + i, d);
            load_row<LnF32, VEC>(weight + i, w);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float g = w[k] * d[k];
                sg += g;
                sgx = fmaf(g, (v[k] - m) * r, sgx);
            }
        }
        const float a = wave_sum(sg) / (float)C;
        const float c = wave_sum(sgx) / (float)C;
        for (int i = lane * VEC; i < C; i += 64 * VEC) {
            float v[VEC], d[VEC], w[VEC], o[VEC];
            load_row<E, VEC>(x + i, v);
            load_row<E, VEC>(dy + i, d);
            load_row<LnF32, VEC>(weight + i, w);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float xhat = (v[k] - m) * r;
                o[k] = r * (w[k] * d[k] - a - xhat * c);
            }
            store_row<E, VEC>(dx + i, o);
        }
    }
}

// Input gradient and the weight/bias partial sums in one kernel, for rows
// held in registers (NV > 0).  A workgroup takes a chunk of kLnRows * RPW
// consecutive rows; wave w handles RPW of them in turn, adding dout * xhat
// and dout into per-lane column sums; the four waves' sums are then added
// through LDS in wave order into part[chunk] (the layout the final kernel
// reads).  Every thread reaches the one barrier: rows past N are skipped,
// not returned from.
template <typename E, int NV, int RPW>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_fused_kernel(
    typename E::T* __restrict__ dinp, float* __restrict__ part,
    const typename E::T* __restrict__ dout, const typename E::T* __restrict__ inp,
    const float* __restrict__ weight, const float* __restrict__ mean,
    const float* __restrict__ rstd, int N, int C) {
    __shared__ float red[kLnRows][2][NV * 256];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int chunk = blockIdx.x;
    const int rbase = chunk * kLnRows * RPW + w * RPW;
    float wv[NV][4], dwa[NV][4], dba[NV][4];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = 4 * lane + 256 * k;
        if (i < C) {
            load_row<LnF32, 4>(weight + i, wv[k]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[k][j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dwa[k][j] = dba[k][j] = 0.f;
    }
    for (int q = 0; q < RPW; ++q) {
        const int row = rbase + q;
        if (row >= N) break;   // wave-uniform
        const typename E::T* x = inp + (size_t)row * C;
        const typename E::T* dy = dout + (size_t)row * C;
        const float m = mean[row], r = rstd[row];
        float xh[NV][4], d[NV][4];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = 4 * lane + 256 * k;
            if (i < C) {
                load_row<E, 4>(x + i, xh[k]);
                load_row<E, 4>(dy + i, d[k]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) xh[k][j] = d[k][j] = 0.f;
            }
        }
        float sg = 0.f, sgx = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * lane + 256 * k;
                xh[k][j] = (i < C) ? (xh[k][j] - m) * r : 0.f;
                const float g = wv[k][j] * d[k][j];
                sg += g;
                sgx = fmaf(g, xh[k][j], sgx);
                dwa[k][j] = fmaf(d[k][j], xh[k][j], dwa[k][j]);
                dba[k][j] += d[k][j];
            }
        const float a = wave_sum(sg) / (float)C;
        const float c = wave_sum(sgx) / (float)C;
        typename E::T* dx = dinp + (size_t)row * C;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = 4 * lane + 256 * k;
            if (i < C) {
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = r * (wv[k][j] * d[k][j] - a - xh[k][j] * c);
                store_row<E, 4>(dx + i, o);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            red[w][0][256 * k + 4 * lane + j] = dwa[k][j];
            red[w][1][256 * k + 4 * lane + j] = dba[k][j];
        }
    __syncthreads();
    float* p = part + (size_t)chunk * 2 * C;
    for (int col = threadIdx.x; col < C; col += kLnThreads) {
        float sw = 0.f, sb = 0.f;
#pragma unroll
        for (int v = 0; v < kLnRows; ++v) {
            sw += red[v][0][col];
            sb += red[v][1][col];
        }
        p[col] = sw;
        p[C + col] = sb;
    }
}

// Partial column sums over rows [chunk * rows, min(N, (chunk + 1) * rows)):
// part[chunk][c] = sum of dout * xhat, part[chunk][C + c] = sum of dout.
// A thread owns VEC consecutive columns; the rows of a chunk are unrolled so
// that their loads are in flight together.
template <typename E, int VEC>
__global__ __launch_bounds__(kLnColThreads) void ln_bwd_cols_kernel(
    float* __restrict__ part, const typename E::T* __restrict__ dout,
    const typename E::T* __restrict__ inp, const float* __restrict__ mean,
    const float* __restrict__ rstd, int N, int C, int rows) {
    const int c = (blockIdx.x * kLnColThreads + threadIdx.x) * VEC;
    if (c >= C) return;
    const int r0 = blockIdx.y * rows;
    const int r1 = min(N, r0 + rows);
    float sw[VEC], sb[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) sw[k] = sb[k] = 0.f;
    int r = r0;
    for (; r + 8 <= r1; r += 8) {
        float d[8][VEC], x[8][VEC];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            load_row<E, VEC>(dout + (size_t)(r + u) * C + c, d[u]);
            load_row<E, VEC>(inp + (size_t)(r + u) * C + c, x[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float m = mean[r + u], q = rstd[r + u];
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                sw[k] = fmaf(d[u][k], (x[u][k] - m) * q, sw[k]);
                sb[k] += d[u][k];
            }
        }
    }
    for (; r < r1; ++r) {
        float d[VEC], x[VEC];
        load_row<E, VEC>(dout + (size_t)r * C + c, d);
        load_row<E, VEC>(inp + (size_t)r * C + c, x);
        const float m = mean[r], q = rstd[r];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            sw[k] = fmaf(d[k], (x[k] - m) * q, sw[k]);
            sb[k] += d[k];
        }
    }
    float* p = part + (size_t)blockIdx.y * 2 * C;
    store_row<LnF32, VEC>(p + c, sw);
    store_row<LnF32, VEC>(p + C + c, sb);
}

// dweight and dbias from the chunk partials: a workgroup takes 64 of the 2C
// partial columns; wave w adds chunks w, w + 16, w + 32, ... in order, and
// wave 0 adds the 16 wave sums in order (a fixed order: deterministic).
constexpr int kLnFinalWaves = 16;

__global__ __launch_bounds__(64 * kLnFinalWaves) void ln_bwd_cols_final_kernel(
    float* __restrict__ dweight, float* __restrict__ dbias, const float* __restrict__ part,
    int nchunks, int C) {
    __shared__ float acc[kLnFinalWaves][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lane;   // of the 2C partial columns
    float s = 0.f;
    if (col < 2 * C) {
        int k = w;
        for (; k + 3 * kLnFinalWaves < nchunks; k += 4 * kLnFinalWaves) {
            const float a = part[(size_t)k * 2 * C + col];
            const float b = part[(size_t)(k + kLnFinalWaves) * 2 * C + col];
            const float c = part[(size_t)(k + 2 * kLnFinalWaves) * 2 * C + col];
            const float d = part[(size_t)(k + 3 * kLnFinalWaves) * 2 * C + col];
            s = (((s + a) + b) + c) + d;
        }
        for (; k < nchunks; k += kLnFinalWaves) s += part[(size_t)k * 2 * C + col];
    }
    acc[w][lane] = s;
    __syncthreads();
    if (w == 0 && col < 2 * C) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kLnFinalWaves; ++i) t += acc[i][lane];
        if (col < C)
            dweight[col] = t;
        else
            dbias[col - C] = t;
    }
}

// Rows of C % 4 == 0 and C <= 2048 stay in registers between the sweeps
// (NV = ceil(C / 256) float4 chunks per lane); others are read twice.
#define LN_ROW_DISPATCH(KERNEL, E, GRID, ...)                                                     \
    do {                                                                                           \
        const int nv = (C % 4 == 0 && C <= 2048) ? (C + 255) / 256 : 0;                           \
        switch (nv) {                                                                              \
            case 1: hipLaunchKernelGGL((KERNEL<E, 4, 1>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            case 2: hipLaunchKernelGGL((KERNEL<E, 4, 2>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            case 3: hipLaunchKernelGGL((KERNEL<E, 4, 3>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            case 4: hipLaunchKernelGGL((KERNEL<E, 4, 4>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            case 5: hipLaunchKernelGGL((KERNEL<E, 4, 5>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            case 6: hipLaunchKernelGGL((KERNEL<E, 4, 6>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            case 7: hipLaunchKernelGGL((KERNEL<E, 4, 7>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            case 8: hipLaunchKernelGGL((KERNEL<E, 4, 8>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); break; \
            default:                                                                               \
                if (C % 4 == 0)                                                                    \
                    hipLaunchKernelGGL((KERNEL<E, 4, 0>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); \
                else                                                                               \
                    hipLaunchKernelGGL((KERNEL<E, 1, 0>), GRID, dim3(kLnThreads), 0, st, __VA_ARGS__); \
        }                                                                                          \
    } while (0)

template <typename E>
hipError_t ln_fwd(typename E::T* out, float* mean, float* rstd, const typename E::T* inp,
                  const float* weight, const float* bias, int N, int C, hipStream_t st) {
    const dim3 grid((unsigned)((N + kLnRows - 1) / kLnRows));
    LN_ROW_DISPATCH(ln_fwd_kernel, E, grid, out, mean, rstd, inp, weight, bias, N, C);
    return hipGetLastError();
}

template <typename E>
hipError_t ln_bwd(typename E::T* dinp, float* dweight, float* dbias, float* ws,
                  const typename E::T* dout, const typename E::T* inp, const float* weight,
                  const float* mean, const float* rstd, int N, int C, hipStream_t st) {
    int rows = 0;
    const int nchunks = layernorm_col_chunks(N, C, &rows);
    const unsigned gf = (unsigned)((2 * (long long)C + 63) / 64);
    const int nv = (C % 4 == 0 && C <= 2048) ? (C + 255) / 256 : 0;
    // rows in registers: the input gradient and the column partials in one
    // kernel (fp32 GPT-2 activations: backward 24.5 -> 17.7 us); otherwise
    // the input gradient, then the column partials reading the rows again
    if (nv > 0 && rows == kLnRows * kLnFusedRpw) {
        const dim3 g((unsigned)nchunks), b(kLnThreads);
        switch (nv) {
#define LN_FUSED_CASE(V)                                                                            \
    case V:                                                                                        \
        hipLaunchKernelGGL((ln_bwd_fused_kernel<E, V, kLnFusedRpw>), g, b, 0, st, dinp, ws, dout,  \
                           inp, weight, mean, rstd, N, C);                                         \
        break;
            LN_FUSED_CASE(1) LN_FUSED_CASE(2) LN_FUSED_CASE(3) LN_FUSED_CASE(4)
            LN_FUSED_CASE(5) LN_FUSED_CASE(6) LN_FUSED_CASE(7) LN_FUSED_CASE(8)
#undef LN_FUSED_CASE
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(ln_bwd_cols_final_kernel, dim3(gf), dim3(64 * kLnFinalWaves), 0, st,
                           dweight, dbias, ws, nchunks, C);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + kLnRows - 1) / kLnRows));
    LN_ROW_DISPATCH(ln_bwd_dx_kernel, E, grid, dinp, dout, inp, weight, mean, rstd, N, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (C % 4 == 0) {
        const unsigned gx = (unsigned)((C / 4 + kLnColThreads - 1) / kLnColThreads);
        hipLaunchKernelGGL((ln_bwd_cols_kernel<E, 4>), dim3(gx, (unsigned)nchunks),
                           dim3(kLnColThreads), 0, st, ws, dout, inp, mean, rstd, N, C, rows);
    } else {
        const unsigned gx = (unsigned)((C + kLnColThreads - 1) / kLnColThreads);
        hipLaunchKernelGGL((ln_bwd_cols_kernel<E, 1>), dim3(gx, (unsigned)nchunks),
                           dim3(kLnColThreads), 0, st, ws, dout, inp, mean, rstd, N, C, rows);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ln_bwd_cols_final_kernel, dim3(gf), dim3(64 * kLnFinalWaves), 0, st,
                       dweight, dbias, ws, nchunks, C);
    return hipGetLastError();
}

}  // namespace

// Row chunks of the weight/bias gradient: 16 rows each (a thread keeps 16
// rows' loads of its columns in flight), more when the chunk count would
// pass 65535 (the grid's y limit).
int layernorm_col_chunks(int N, int C, int* rows_per_chunk) {
    (void)C;
    long long rows = 16;
    if ((N + rows - 1) / rows > 65535) rows = (N + 65534) / 65535;
    *rows_per_chunk = (int)rows;
    return (int)((N + rows - 1) / rows);
}

size_t layernorm_workspace_floats(int N, int C) {
    int rows = 0;
    return (size_t)layernorm_col_chunks(N, C, &rows) * 2 * (size_t)C;
}

hipError_t launch_layernorm_fwd_f32(float* out, float* mean, float* rstd, const float* inp,
                                    const float* weight, const float* bias, int N, int C,
                                    hipStream_t st) {
    return ln_fwd<LnF32>(out, mean, rstd, inp, weight, bias, N, C, st);
}
hipError_t launch_layernorm_fwd_bf16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                                     const float* weight, const float* bias, int N, int C,
                                     hipStream_t st) {
    return ln_fwd<LnBF16>(out, mean, rstd, inp, weight, bias, N, C, st);
}
hipError_t launch_layernorm_bwd_f32(float* dinp, float* dweight, float* dbias, float* ws,
                                    const float* dout, const float* inp, const float* weight,
                                    const float* mean, const float* rstd, int N, int C,
                                    hipStream_t st) {
    return ln_bwd<LnF32>(dinp, dweight, dbias, ws, dout, inp, weight, mean, rstd, N, C, st);
}
hipError_t launch_layernorm_bwd_bf16(uint16_t* dinp, float* dweight, float* dbias, float* ws,
                                     const uint16_t* dout, const uint16_t* inp,
                                     const float* weight, const float* mean, const float* rstd,
                                     int N, int C, hipStream_t st) {
    return ln_bwd<LnBF16>(dinp, dweight, dbias, ws, dout, inp, weight, mean, rstd, N, C, st);
}

}  // namespace attn

namespace attn {
hipError_t launch_layernorm_fwd_f16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                                    const float* weight, const float* bias, int N, int C,
                                    hipStream_t st) {
    return ln_fwd<LnF16>(out, mean, rstd, inp, weight, bias, N, C, st);
}
hipError_t launch_layernorm_bwd_f16(uint16_t* dinp, float* dweight, float* dbias, float* ws,
                                    const uint16_t* dout, const uint16_t* inp, const float* weight,
                                    const float* mean, const float* rstd, int N, int C,
                                    hipStream_t st) {
    return ln_bwd<LnF16>(dinp, dweight, dbias, ws, dout, inp, weight, mean, rstd, N, C, st);
}
}  // namespace attn
