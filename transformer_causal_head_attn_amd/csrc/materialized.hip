// materialized.hip -- attention with the full (B,NH,T,T) matrices written to
// device memory, fp32, as the CPU reference of llm.c
// dev/cuda/attention_backward.cu does it (attention_forward_cpu,
// attention_backward_cpu) and as its GPU sequence permute / sgemm / softmax /
// sgemm / unpermute does, but without the permute passes and with every
// contraction on gfx950 fp32 matrix cores (v_mfma_f32_16x16x4_f32).
//
// Forward:  preatt = Q K^T          (unscaled, every (t, j), masked ones too)
//           att    = softmax_row(scale * preatt) over U(t), exact 0 elsewhere
//           out    = att V
// Backward: datt    = dO V^T        (every (t, j))
//           dpreatt = scale * att * (datt - sum_{j in U(t)} att datt)
//                     (the closed form of softmax_autoregressive_backward_kernel7;
//                      exact 0 above the diagonal)
//           dv = att^T dO,  dq = dpreatt K,  dk = dpreatt^T Q
//
// The two row kernels are bound by memory traffic (each reads one or two
// T x T matrices and writes one); the four products are matrix-core work.
// In causal mode the products skip 64 x 64 blocks of att / dpreatt that lie
// wholly above the diagonal and treat entries above the diagonal as 0, so
// only the lower triangle of an att argument is ever read.
#include "common.hpp"

namespace attn {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr int kLDA = kTile + 4;   // LDS row stride of a 64 x 64 fp32 block

struct Lane {
    int tid, w, l, r16, g;
    __device__ Lane() {
        tid = threadIdx.x;
        w = tid >> 6;
        l = tid & 63;
        r16 = l & 15;
        g = l >> 4;
    }
};

// ------------------------------------------- dense scores M = X Y^T per head
// X rows t and Y rows j are hs-vectors inside packed tensors (row strides
// ldx, ldy elements); M is the head's T x T row-major matrix.  One workgroup
// per 64 x 64 block; each wave owns 16 rows of X in registers.
template <int HS>
__global__ __launch_bounds__(kThreads) void scores_kernel(float* __restrict__ M,
                                                          const float* __restrict__ X,
                                                          const float* __restrict__ Y, int T,
                                                          int NH, size_t ldx, size_t ldy,
                                                          size_t batch_x, size_t batch_y) {
    constexpr int LDK = HS + 4;
    constexpr int KS = HS / 4;
    __shared__ float Ys[kTile * LDK];
    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    const int ct = blockIdx.x % nt;
    const int rt = (blockIdx.x / nt) % nt;
    const int bh = blockIdx.x / (nt * nt);
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const float* xb = X + (size_t)b * batch_x + (size_t)h * HS;
    const float* yb = Y + (size_t)b * batch_y + (size_t)h * HS;

    const int t = rt * kTile + 16 * L.w + L.r16;
    float xr[KS];
#pragma unroll
    for (int c = 0; c < KS / 4; ++c) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < T) v = *reinterpret_cast<const float4*>(xb + (size_t)t * ldx + KS * L.g + 4 * c);
        xr[4 * c + 0] = v.x;
        xr[4 * c + 1] = v.y;
        xr[4 * c + 2] = v.z;
        xr[4 * c + 3] = v.w;
    }
    constexpr int C4 = HS / 4;
    for (int e = L.tid; e < kTile * C4; e += kThreads) {
        const int row = e / C4, c4 = e % C4;
        const int j = ct * kTile + row;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < T) v = *reinterpret_cast<const float4*>(yb + (size_t)j * ldy + 4 * c4);
        *reinterpret_cast<float4*>(Ys + row * LDK + 4 * c4) = v;
    }
    __syncthreads();

    float* mrow = M + ((size_t)bh * T + t) * T;
    const bool vec = (T % 4) == 0;
#pragma unroll
    for (int n = 0; n < kTile / 16; ++n) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const float* yr = Ys + (16 * n + L.r16) * LDK + KS * L.g;
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            const float4 yy = *reinterpret_cast<const float4*>(yr + 4 * c);
            acc = mfma_f32(yy.x, xr[4 * c + 0], acc);
            acc = mfma_f32(yy.y, xr[4 * c + 1], acc);
            acc = mfma_f32(yy.z, xr[4 * c + 2], acc);
            acc = mfma_f32(yy.w, xr[4 * c + 3], acc);
        }
        // acc[i] = M[t][ct*64 + 16n + 4g + i]
        const int j0 = ct * kTile + 16 * n + 4 * L.g;
        if (t < T) {
            if (vec && j0 + 3 < T) {
                *reinterpret_cast<float4*>(mrow + j0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (j0 + i < T) mrow[j0 + i] = acc[i];
            }
        }
    }
}

// ------------------------------------------ C = op(A) Bm per head (T x hs)
// A is the head's T x T matrix (att or dpreatt); op(A) = A, or A^T when
// TRANS.  Bm and C are hs-column slices of packed tensors (row strides ldb,
// ldc).  Causal: A is lower triangular, so output row block rt needs the
// contraction blocks kt <= rt (A) or kt >= rt (A^T); entries above the
// diagonal are read as 0.
template <int HS, bool TRANS>
__global__ __launch_bounds__(kThreads) void apply_kernel(float* __restrict__ Cm,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ Bm, int T,
                                                         int NH, int causal, size_t ldb,
                                                         size_t ldc, size_t batch_b,
                                                         size_t batch_c) {
    constexpr int LDB = HS + 4;
    constexpr int MB = HS / 16;
    __shared__ float As[kTile * kLDA];
    __shared__ float Bs[kTile * LDB];
    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    const int rt = blockIdx.x % nt;
    const int bh = blockIdx.x / nt;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const float* Ah = A + (size_t)bh * T * T;
    const float* bb = Bm + (size_t)b * batch_b + (size_t)h * HS;
    const int row = rt * kTile + 16 * L.w + L.r16;   // this lane's output row

    f32x4 o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    int k0 = 0, k1 = nt;
    if (causal) {
        if (TRANS) k0 = rt;
        else k1 = rt + 1;
    }
    for (int kt = k0; kt < k1; ++kt) {
        __syncthreads();
        // A block: rows R0.., cols C0.. of the T x T matrix
        const int R0 = TRANS ? kt * kTile : rt * kTile;
        const int C0 = TRANS ? rt * kTile : kt * kTile;
        for (int e = L.tid; e < kTile * kTile; e += kThreads) {
            const int r = e / kTile, c = e % kTile;
            const int gr = R0 + r, gc = C0 + c;
            float v = 0.f;
            if (gr < T && gc < T && (!causal || gc <= gr)) v = Ah[(size_t)gr * T + gc];
            As[r * kLDA + c] = v;
        }
        constexpr int C4 = HS / 4;
        for (int e = L.tid; e < kTile * C4; e += kThreads) {
            const int r = e / C4, c4 = e % C4;
            const int k = kt * kTile + r;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < T) v = *reinterpret_cast<const float4*>(bb + (size_t)k * ldb + 4 * c4);
            *reinterpret_cast<float4*>(Bs + r * LDB + 4 * c4) = v;
        }
        __syncthreads();
        // C^T[d][row] += sum_kk Bm[kk][d] * op(A)[row][kk],  kk = 16g + s
        const int lr = 16 * L.w + L.r16;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int kk = 16 * L.g + s;
            const float a = TRANS ? As[kk * kLDA + lr] : As[lr * kLDA + kk];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb] = mfma_f32(Bs[kk * LDB + 16 * mb + L.r16], a, o[mb]);
        }
    }
    if (row < T) {
        float* crow = Cm + (size_t)b * batch_c + (size_t)row * ldc + (size_t)h * HS;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            *reinterpret_cast<float4*>(crow + 16 * mb + 4 * L.g) =
                make_float4(o[mb][0], o[mb][1], o[mb][2], o[mb][3]);
    }
}

// ------------------------------------------------------ row kernels (HBM)
// One wave per row (b, h, t) of the T x T matrices.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// att[t, j] = exp(scale*(preatt[t,j] - max)) / sum over j in U(t); 0 elsewhere.
__global__ __launch_bounds__(kThreads) void softmax_rows_kernel(float* __restrict__ att,
                                                                const float* __restrict__ pre,
                                                                int T, long long rows, int causal,
                                                                float scale_log2) {
    const long long r = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const int t = (int)(r % T);
    const int nj = causal ? t + 1 : T;
    const float* p = pre + (size_t)r * T;
    float* a = att + (size_t)r * T;
    // pass 1: running max and normaliser (log2 domain)
    float m = -INFINITY, l = 0.f;
    for (int j = lane; j < nj; j += 64) {
        const float x = p[j] * scale_log2;
        const float mn = fmaxf(m, x);
        l = l * fast_exp2(m - mn) + fast_exp2(x - mn);
        m = mn;
    }
    const float M = wave_max(m);
    l = (m == -INFINITY) ? 0.f : l * fast_exp2(m - M);
    const float inv = 1.0f / wave_sum(l);
    // pass 2: write every entry of the row
    for (int j = lane; j < T; j += 64) a[j] = (j < nj) ? fast_exp2(p[j] * scale_log2 - M) * inv : 0.f;
}

// dpreatt[t, j] = scale * att * (datt - sum_{j' in U(t)} att datt) on U(t); 0 elsewhere.
__global__ __launch_bounds__(kThreads) void softmax_bwd_rows_kernel(
    float* __restrict__ dpre, const float* __restrict__ att, const float* __restrict__ datt,
    int T, long long rows, int causal, float scale) {
    const long long r = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const int t = (int)(r % T);
    const int nj = causal ? t + 1 : T;
    const float* a = att + (size_t)r * T;
    const float* d = datt + (size_t)r * T;
    float* o = dpre + (size_t)r * T;
    float acc = 0.f;
    for (int j = lane; j < nj; j += 64) acc += a[j] * d[j];
    const float D = wave_sum(acc);
    for (int j = lane; j < T; j += 64) o[j] = (j < nj) ? scale * a[j] * (d[j] - D) : 0.f;
}

template <int HS>
hipError_t fwd_hs(float* out, float* preatt, float* att, const float* qkv, const Shape& s,
                  hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    const size_t C3 = 3 * (size_t)s.C;
    const size_t bstride = (size_t)s.T * C3;
    const long long BH = (long long)s.B * s.NH;
    hipLaunchKernelGGL(scores_kernel<HS>, dim3((unsigned)(BH * nt * nt)), dim3(kThreads), 0, st,
                       preatt, qkv, qkv + s.C, s.T, s.NH, C3, C3, bstride, bstride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = BH * s.T;
    const float scale = (float)(1.0 / sqrt((double)HS));
    hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, st,
                       att, preatt, s.T, rows, s.causal, scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((apply_kernel<HS, false>), dim3((unsigned)(BH * nt)), dim3(kThreads), 0, st,
                       out, att, qkv + 2 * s.C, s.T, s.NH, s.causal, C3, (size_t)s.C, bstride,
                       (size_t)s.T * s.C);
    return hipGetLastError();
}

template <int HS>
hipError_t bwd_hs(float* dqkv, float* dpreatt, float* datt, const float* dout, const float* qkv,
                  const float* att, const Shape& s, hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    const size_t C = (size_t)s.C;
    const size_t C3 = 3 * C;
    const size_t bq = (size_t)s.T * C3, bo = (size_t)s.T * C;
    const long long BH = (long long)s.B * s.NH;
    // datt = dO V^T
    hipLaunchKernelGGL(scores_kernel<HS>, dim3((unsigned)(BH * nt * nt)), dim3(kThreads), 0, st,
                       datt, dout, qkv + 2 * C, s.T, s.NH, C, C3, bo, bq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = BH * s.T;
    const float scale = (float)(1.0 / sqrt((double)HS));
    hipLaunchKernelGGL(softmax_bwd_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0,
                       st, dpreatt, att, datt, s.T, rows, s.causal, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g = (unsigned)(BH * nt);
    // dv = att^T dO
    hipLaunchKernelGGL((apply_kernel<HS, true>), dim3(g), dim3(kThreads), 0, st, dqkv + 2 * C, att,
                       dout, s.T, s.NH, s.causal, C, C3, bo, bq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dq = dpreatt K
    hipLaunchKernelGGL((apply_kernel<HS, false>), dim3(g), dim3(kThreads), 0, st, dqkv, dpreatt,
                       qkv + C, s.T, s.NH, s.causal, C3, C3, bq, bq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dk = dpreatt^T Q
    hipLaunchKernelGGL((apply_kernel<HS, true>), dim3(g), dim3(kThreads), 0, st, dqkv + C, dpreatt,
                       qkv, s.T, s.NH, s.causal, C3, C3, bq, bq);
    return hipGetLastError();
}

}  // namespace

#define ATTN_DISPATCH_HS(fn, ...)                         \
    switch (s.hs) {                                       \
        case 16: return fn<16>(__VA_ARGS__);              \
        case 32: return fn<32>(__VA_ARGS__);              \
        case 64: return fn<64>(__VA_ARGS__);              \
        case 128: return fn<128>(__VA_ARGS__);            \
        default: return hipErrorInvalidValue;             \
    }

hipError_t launch_fwd_materialized(float* out, float* preatt, float* att, const float* qkv,
                                   const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(fwd_hs, out, preatt, att, qkv, s, st)
}

hipError_t launch_bwd_materialized(float* dqkv, float* dpreatt, float* datt, const float* dout,
                                   const float* qkv, const float* att, const Shape& s,
                                   hipStream_t st) {
    ATTN_DISPATCH_HS(bwd_hs, dqkv, dpreatt, datt, dout, qkv, att, s, st)
}

#undef ATTN_DISPATCH_HS

}  // namespace attn
