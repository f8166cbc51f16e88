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
// T x T matrices and writes one; in causal mode the masked upper triangle is
// only written, never read); the dense score products are bound by the fp32
// matrix cores, the four products with an hs-wide operand by both.
// In causal mode the products skip 64 x 64 blocks of att / dpreatt that lie
// wholly above the diagonal and treat entries above the diagonal as 0, so
// only the lower triangle of an att argument is ever read.
#include "common.hpp"
#include "tiles.hpp"

namespace attn {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

// A pointer the whole wave shares, read from lane 0 so that a buffer
// descriptor built from it stays in scalar registers.
template <typename P>
__device__ __forceinline__ P* wave_uniform(P* p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (P*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// apply_kernel: 16-row output blocks per wave, and output rows per workgroup
// (tiles.hpp: the launchers size the grid and the kernel decodes its tile
// with the same functions)
using tiles::kApplyRB;
using tiles::kApplyRows;

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
// per 64-row strip of M: each wave keeps 16 rows of X in registers and the
// workgroup walks the column tiles, staging Y through LDS with the next
// tile's registers loaded while the current one is used.
// VEC (T % 4 == 0): Y loads and M stores are raw buffer operations whose
// descriptors end at row T (loads past it return zeros, stores past it are
// dropped), and a store whose columns lie past T gets an offset past the
// descriptor's end, so no load or store is predicated.  That lets the wait
// for the next tile's loads leave this step's M stores in flight: with
// predicated stores the compiler waited for all of them every step.
// NT: the M stores carry the non-temporal cache hint (the backward's datt:
// backward 581 -> 565 us on the GPT-2 layer; on the forward's preatt, which
// the row softmax reads right after, it cost 3%).
template <int HS, bool VEC, bool NT>
__global__ __launch_bounds__(kThreads) void scores_kernel(float* __restrict__ M,
                                                          const float* __restrict__ X,
                                                          const float* __restrict__ Y, int T,
                                                          int NH, size_t ldx, size_t ldy,
                                                          size_t batch_x, size_t batch_y) {
    constexpr int LDK = HS + 4;
    constexpr int KS = HS / 4;
    constexpr int C4 = HS / 4;
    constexpr int NY = kTile * C4 / kThreads;   // Y float4 per thread per tile
    __shared__ float Ys[kTile * LDK];
    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    // heads run fastest: workgroups go to the 8 XCDs round robin by id, so
    // when the head count B*NH is a multiple of 8 every strip of a head
    // lands on one XCD and its Y rows are fetched into one L2 only (GPT-2
    // layer: 269 MB fetched per call with the strips fastest; materialised
    // forward + backward 956 -> 929-942 us, same bits)
    const int BH = gridDim.x / nt;
    const int bh = blockIdx.x % BH;
    const int rt = blockIdx.x / BH;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const float* xb = X + (size_t)b * batch_x + (size_t)h * HS;
    const float* yb = Y + (size_t)b * batch_y + (size_t)h * HS;

    const int t0 = rt * kTile + 16 * L.w;   // this wave's first row
    const int t = t0 + L.r16;
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
    float4 ry[NY];
    const uint32_t ldyb = (uint32_t)(ldy * 4);
    auto fetch = [&](int ct) {
        if constexpr (VEC) {
            const int valid = min(T - ct * kTile, kTile);
            const uint32_t num = __builtin_amdgcn_readfirstlane((uint32_t)(valid - 1) * ldyb + HS * 4u);
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                wave_uniform(const_cast<float*>(yb + (size_t)ct * kTile * ldy)), (short)0, (int)num,
                0x00020000);
#pragma unroll
            for (int k = 0; k < NY; ++k) {
                const int e = L.tid + k * kThreads;
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)((uint32_t)(e / C4) * ldyb + 16u * (uint32_t)(e % C4)), 0, 0);
                __builtin_memcpy(&ry[k], &x, 16);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NY; ++k) {
                const int e = L.tid + k * kThreads;
                const int j = ct * kTile + e / C4;
                ry[k] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (j < T) ry[k] = *reinterpret_cast<const float4*>(yb + (size_t)j * ldy + 4 * (e % C4));
            }
        }
    };
    float* mrow = M + ((size_t)bh * T + t) * T;
    // VEC: this wave's 16 rows of M (fewer below T; none past it)
    const int wrows = __builtin_amdgcn_readfirstlane(max(0, min(16, T - t0)));
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        wave_uniform(M + ((size_t)bh * T + (size_t)min(t0, T)) * T), (short)0,
        (int)__builtin_amdgcn_readfirstlane((uint32_t)wrows * (uint32_t)T * 4u), 0x00020000);
    // acc[n][i] = M[t][ct*64 + 16n + 4g + i]
    auto store_m = [&](int ct, const f32x4 (&acc)[kTile / 16]) {
#pragma unroll
        for (int n = 0; n < kTile / 16; ++n) {
            const int j0 = ct * kTile + 16 * n + 4 * L.g;
            if constexpr (VEC) {
                // columns j0..j0+3 lie wholly below T or wholly past it (T % 4 == 0)
                const uint32_t off = j0 < T ? ((uint32_t)L.r16 * (uint32_t)T + (uint32_t)j0) * 4u : 0xFFFFFFF0u;
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, acc[n]), rm, (int)off, 0,
                    NT ? 2 : 0);
            } else if (t < T) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (j0 + i < T) mrow[j0 + i] = acc[n][i];
            }
        }
    };
    // A tile's M columns are stored during the next step, right after that
    // step's loads are issued: the wait for a tile's loads also waits for
    // every store issued before it, so the stores get a whole step to land.
    f32x4 prev[kTile / 16];
    fetch(0);
    wait_global_loads();
    for (int ct = 0; ct < nt; ++ct) {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NY; ++k) {
            const int e = L.tid + k * kThreads;
            *reinterpret_cast<float4*>(Ys + (e / C4) * LDK + 4 * (e % C4)) = ry[k];
        }
        __syncthreads();
        if (ct + 1 < nt) fetch(ct + 1);
        if (ct > 0) store_m(ct - 1, prev);
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
            prev[n] = acc;
        }
    }
    store_m(nt - 1, prev);
}

// ------------------------------------------ C = op(A) Bm per head (T x hs)
// A is the head's T x T matrix (att or dpreatt); op(A) = A, or A^T when
// TRANS.  Bm and C are hs-column slices of packed tensors (row strides ldb,
// ldc).  A workgroup owns 64 output rows (16 per wave; two blocks per wave
// measured slower: half the workgroups, fewer resident waves) and walks the
// contraction in 64-wide blocks.  Causal: A is lower triangular, so the
// output rows of block rt need contraction blocks up to the diagonal (A) or
// from it (A^T); entries above the diagonal are read as 0.  op(A) = A reads
// 16 contiguous values of a block row per lane (16-byte loads, row stride 68
// floats); op(A) = A^T reads a block column (row stride 65 floats, so the
// lanes hit distinct banks); Bm rows have stride hs+1 for the same reason.
// The next A and Bm blocks are loaded into registers while the current ones
// are used.
template <int HS, bool TRANS>
__global__ __launch_bounds__(kThreads) void apply_kernel(float* __restrict__ Cm,
                                                         const float* __restrict__ A,
                                                         const float* __restrict__ Bm, int T,
                                                         int NH, int BH, int causal, size_t ldb,
                                                         size_t ldc, size_t batch_b,
                                                         size_t batch_c) {
    constexpr int RB = kApplyRB;                 // 16-row output blocks per wave
    constexpr int BR = kApplyRows;               // output rows per workgroup (64)
    // LDS A block: op(A) = A: BR rows x 64 contraction columns (stride 68);
    // op(A) = A^T: 64 contraction rows x BR output columns (stride BR + 1).
    constexpr int AROWS = TRANS ? kTile : BR;
    constexpr int ACOLS = TRANS ? BR : kTile;
    constexpr int LDA = TRANS ? BR + 1 : kTile + 4;
    constexpr int LDB = HS + 1;
    constexpr int MB = HS / 16;
    constexpr int NA4 = AROWS * ACOLS / 4 / kThreads;   // A float4 per thread per block
    constexpr int C4 = HS / 4;
    constexpr int NB4 = kTile * C4 / kThreads;          // Bm float4 per thread per block
    __shared__ float As[AROWS * LDA];
    __shared__ float Bs[kTile * LDB];
    const Lane L;
    const int nkt = (T + kTile - 1) / kTile;
    // causal: heaviest row tiles first (op(A) = A: row tile rt sees rt + 1
    // blocks; A^T: nkt - rt), heads fastest, so that the last workgroups to
    // start are the lightest (forward 410 -> 380 us, backward 693 -> 595 us on
    // the GPT-2 layer against row tiles in order)
    const tiles::TileId tid = tiles::apply_tile(blockIdx.x, BH, T, causal && !TRANS);
    if (!tid.valid) return;   // whole workgroup: no barrier is reached
    const int bh = tid.bh;
    const int rt = tid.rt;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const float* Ah = A + (size_t)bh * T * T;
    const float* bb = Bm + (size_t)b * batch_b + (size_t)h * HS;
    const int row0 = rt * BR;

    f32x4 o[RB][MB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) o[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    int k0 = 0, k1 = nkt;
    if (causal) {
        if (TRANS) k0 = row0 / kTile;
        else k1 = min(nkt, (row0 + BR - 1) / kTile + 1);
    }
    float4 ra[NA4];
    float4 rbv[NB4];
    const bool vecA = (T % 4) == 0;
    // Loads are raw buffer loads over the rows of the block that lie below T
    // (a load at or past num_records returns zeros), so none is predicated;
    // the causal and column masks are selects, applied only to blocks that
    // hold the diagonal or columns past T.  Word 3 is the gfx9 raw-buffer
    // format word.
    auto fetch = [&](int kt) {
        const int R0 = TRANS ? kt * kTile : row0;   // A rows of the block
        const int C0 = TRANS ? row0 : kt * kTile;   // A columns of the block
        constexpr int CQ = ACOLS / 4;               // float4 per block row
        if (vecA) {
            const uint32_t rowb = (uint32_t)T * 4u;
            const int valid = min(T - R0, AROWS);
            // uniform values: readfirstlane keeps the descriptor in scalar registers
            const uint32_t num = __builtin_amdgcn_readfirstlane(valid > 0 ? (uint32_t)valid * rowb : 0u);
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(Ah + (size_t)R0 * T), (short)0, (int)num, 0x00020000);
#pragma unroll
            for (int k = 0; k < NA4; ++k) {
                const int e = L.tid + k * kThreads;
                const int rr = e / CQ, cc = 4 * (e % CQ);
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)((uint32_t)rr * rowb + (uint32_t)(C0 + cc) * 4u), 0, 0);
                __builtin_memcpy(&ra[k], &x, 16);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NA4; ++k) {
                const int e = L.tid + k * kThreads;
                const int gr = R0 + e / CQ, gc = C0 + 4 * (e % CQ);
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    v[u] = (gr < T && gc + u < T && (!causal || gc + u <= gr)) ? Ah[(size_t)gr * T + gc + u]
                                                                              : 0.f;
                ra[k] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
        const uint32_t ldbb = (uint32_t)(ldb * 4);
        const int bvalid = min(T - kt * kTile, kTile);
        const uint32_t bnum =
            __builtin_amdgcn_readfirstlane(bvalid > 0 ? (uint32_t)(bvalid - 1) * ldbb + HS * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(bb + (size_t)kt * kTile * ldb), (short)0, (int)bnum, 0x00020000);
#pragma unroll
        for (int k = 0; k < NB4; ++k) {
            const int e = L.tid + k * kThreads;
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(
                rb, (int)((uint32_t)(e / C4) * ldbb + 16u * (uint32_t)(e % C4)), 0, 0);
            __builtin_memcpy(&rbv[k], &x, 16);
        }
    };
    auto store = [&](int kt) {
        // LDS holds the A block as it lies in memory: As[r][c] = A[R0 + r][C0 + c].
        // The masks are applied here, when the loads have landed anyway.
        constexpr int CQ = ACOLS / 4;
        const int R0 = TRANS ? kt * kTile : row0;
        const int C0 = TRANS ? row0 : kt * kTile;
        if (vecA && ((C0 + ACOLS > T) || (causal && C0 + ACOLS - 1 > R0))) {
#pragma unroll
            for (int k = 0; k < NA4; ++k) {
                const int e = L.tid + k * kThreads;
                const int gr = R0 + e / CQ, gc = C0 + 4 * (e % CQ);
                ra[k].x = (gc + 0 < T && (!causal || gc + 0 <= gr)) ? ra[k].x : 0.f;
                ra[k].y = (gc + 1 < T && (!causal || gc + 1 <= gr)) ? ra[k].y : 0.f;
                ra[k].z = (gc + 2 < T && (!causal || gc + 2 <= gr)) ? ra[k].z : 0.f;
                ra[k].w = (gc + 3 < T && (!causal || gc + 3 <= gr)) ? ra[k].w : 0.f;
            }
        }
#pragma unroll
        for (int k = 0; k < NA4; ++k) {
            const int e = L.tid + k * kThreads;
            float* d = As + (e / CQ) * LDA + 4 * (e % CQ);
            d[0] = ra[k].x;
            d[1] = ra[k].y;
            d[2] = ra[k].z;
            d[3] = ra[k].w;
        }
#pragma unroll
        for (int k = 0; k < NB4; ++k) {
            const int e = L.tid + k * kThreads;
            float* d = Bs + (e / C4) * LDB + 4 * (e % C4);
            d[0] = rbv[k].x;
            d[1] = rbv[k].y;
            d[2] = rbv[k].z;
            d[3] = rbv[k].w;
        }
    };
    if (k0 < k1) fetch(k0);
    wait_global_loads();
    for (int kt = k0; kt < k1; ++kt) {
        __syncthreads();
        store(kt);
        __syncthreads();
        if (kt + 1 < k1) fetch(kt + 1);
        // C^T[d][row] += sum_kk Bm[kk][d] * op(A)[row][kk],  kk = 16g + s
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int lr = 16 * (L.w * RB + rb) + L.r16;   // output row within the block
            float av[16];
            if (TRANS) {   // op(A)[lr][kk] = A[kk][lr]: a block column
#pragma unroll
                for (int s2 = 0; s2 < 16; ++s2) av[s2] = As[(16 * L.g + s2) * LDA + lr];
            } else {       // a block row, 16 contiguous values
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 q = *reinterpret_cast<const float4*>(As + lr * LDA + 16 * L.g + 4 * c);
                    av[4 * c + 0] = q.x;
                    av[4 * c + 1] = q.y;
                    av[4 * c + 2] = q.z;
                    av[4 * c + 3] = q.w;
                }
            }
#pragma unroll
            for (int s4 = 0; s4 < 16; s4 += 4) {
                float bv[4][MB];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) bv[u][mb] = Bs[(16 * L.g + s4 + u) * LDB + 16 * mb + L.r16];
                // the 4 x MB reads (paired into ds_read2) ahead of their MFMAs,
                // so one wait covers a group instead of one wait per pair
                __builtin_amdgcn_sched_group_barrier(0x100, 4 * MB / 2, 0);   // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 4 * MB, 0);       // MFMAs
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) o[rb][mb] = mfma_f32(bv[u][mb], av[s4 + u], o[rb][mb]);
            }
        }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = row0 + 16 * (L.w * RB + rb) + L.r16;
        if (row < T) {
            float* crow = Cm + (size_t)b * batch_c + (size_t)row * ldc + (size_t)h * HS;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                *reinterpret_cast<float4*>(crow + 16 * mb + 4 * L.g) =
                    make_float4(o[rb][mb][0], o[rb][mb][1], o[rb][mb][2], o[rb][mb][3]);
        }
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
// Row held in registers as NV float4 per lane (T <= 256*NV, T % 4 == 0);
// entries j > t of a causal row are never read (only written as 0).
template <int NV>
__global__ __launch_bounds__(kThreads) void softmax_rows_vec_kernel(
    float* __restrict__ att, const float* __restrict__ pre, int T, long long rows, int causal,
    float scale_log2) {
    const long long r = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const int t = (int)(r % T);
    const int nj = causal ? t + 1 : T;
    const float* p = pre + (size_t)r * T;
    float* a = att + (size_t)r * T;
    float x[NV][4];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int j0 = 4 * (lane + 64 * v);
        float4 q = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (j0 < nj) q = *reinterpret_cast<const float4*>(p + j0);
        x[v][0] = (j0 + 0 < nj) ? q.x : -INFINITY;
        x[v][1] = (j0 + 1 < nj) ? q.y : -INFINITY;
        x[v][2] = (j0 + 2 < nj) ? q.z : -INFINITY;
        x[v][3] = (j0 + 3 < nj) ? q.w : -INFINITY;
        mx = fmaxf(mx, fmaxf(fmaxf(x[v][0], x[v][1]), fmaxf(x[v][2], x[v][3])));
    }
    const float M = wave_max(mx) * scale_log2;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[v][e] = fast_exp2(fmaf(x[v][e], scale_log2, -M));   // masked: exp2(-inf) = 0
            sum += x[v][e];
        }
    const float inv = 1.0f / wave_sum(sum);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int j0 = 4 * (lane + 64 * v);
        if (j0 < T)
            *reinterpret_cast<float4*>(a + j0) =
                make_float4(x[v][0] * inv, x[v][1] * inv, x[v][2] * inv, x[v][3] * inv);
    }
}

// Same for any T: two passes over the row (running max and normaliser, then
// the writes); scalar accesses.
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
    for (int j = lane; j < T; j += 64) a[j] = (j < nj) ? fast_exp2(p[j] * scale_log2 - M) * inv : 0.f;
}

// dpreatt[t, j] = scale * att * (datt - sum_{j' in U(t)} att datt) on U(t); 0
// elsewhere.  Rows held in registers as NV float4 per lane (T <= 256*NV,
// T % 4 == 0): att and datt are read once; entries j > t of a causal row are
// not read.
template <int NV>
__global__ __launch_bounds__(kThreads) void softmax_bwd_rows_vec_kernel(
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
    float av[NV][4], dv[NV][4];
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int j0 = 4 * (lane + 64 * v);
        float4 qa = make_float4(0.f, 0.f, 0.f, 0.f), qd = qa;
        if (j0 < nj) {
            qa = *reinterpret_cast<const float4*>(a + j0);
            qd = *reinterpret_cast<const float4*>(d + j0);
        }
        av[v][0] = (j0 + 0 < nj) ? qa.x : 0.f;
        av[v][1] = (j0 + 1 < nj) ? qa.y : 0.f;
        av[v][2] = (j0 + 2 < nj) ? qa.z : 0.f;
        av[v][3] = (j0 + 3 < nj) ? qa.w : 0.f;
        dv[v][0] = qd.x;
        dv[v][1] = qd.y;
        dv[v][2] = qd.z;
        dv[v][3] = qd.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(av[v][e], dv[v][e], acc);
    }
    const float D = wave_sum(acc);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int j0 = 4 * (lane + 64 * v);
        if (j0 < T)   // masked entries have av = 0 -> exact 0; non-temporal stores (-3%)
            __builtin_nontemporal_store(f32x4{scale * av[v][0] * (dv[v][0] - D),
                                              scale * av[v][1] * (dv[v][1] - D),
                                              scale * av[v][2] * (dv[v][2] - D),
                                              scale * av[v][3] * (dv[v][3] - D)},
                                        reinterpret_cast<f32x4*>(o + j0));
    }
}

// Same for any T: two passes over the row; scalar accesses.
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

hipError_t launch_softmax_bwd_rows(float* dpre, const float* att, const float* datt, int T,
                                   long long rows, int causal, float scale, hipStream_t st) {
    const dim3 grid((unsigned)((rows + 3) / 4)), blk(kThreads);
    if (T % 4 == 0 && T <= 4096) {
        if (T <= 256) hipLaunchKernelGGL(softmax_bwd_rows_vec_kernel<1>, grid, blk, 0, st, dpre, att, datt, T, rows, causal, scale);
        else if (T <= 512) hipLaunchKernelGGL(softmax_bwd_rows_vec_kernel<2>, grid, blk, 0, st, dpre, att, datt, T, rows, causal, scale);
        else if (T <= 1024) hipLaunchKernelGGL(softmax_bwd_rows_vec_kernel<4>, grid, blk, 0, st, dpre, att, datt, T, rows, causal, scale);
        else if (T <= 2048) hipLaunchKernelGGL(softmax_bwd_rows_vec_kernel<8>, grid, blk, 0, st, dpre, att, datt, T, rows, causal, scale);
        else hipLaunchKernelGGL(softmax_bwd_rows_vec_kernel<16>, grid, blk, 0, st, dpre, att, datt, T, rows, causal, scale);
    } else {
        hipLaunchKernelGGL(softmax_bwd_rows_kernel, grid, blk, 0, st, dpre, att, datt, T, rows, causal, scale);
    }
    return hipGetLastError();
}

// Launch the forward row softmax: register-resident rows when they fit.
hipError_t launch_softmax_rows(float* att, const float* pre, int T, long long rows, int causal,
                               float scale_log2, hipStream_t st) {
    const dim3 grid((unsigned)((rows + 3) / 4)), blk(kThreads);
    if (T % 4 == 0 && T <= 4096) {
        if (T <= 256) hipLaunchKernelGGL(softmax_rows_vec_kernel<1>, grid, blk, 0, st, att, pre, T, rows, causal, scale_log2);
        else if (T <= 512) hipLaunchKernelGGL(softmax_rows_vec_kernel<2>, grid, blk, 0, st, att, pre, T, rows, causal, scale_log2);
        else if (T <= 1024) hipLaunchKernelGGL(softmax_rows_vec_kernel<4>, grid, blk, 0, st, att, pre, T, rows, causal, scale_log2);
        else if (T <= 2048) hipLaunchKernelGGL(softmax_rows_vec_kernel<8>, grid, blk, 0, st, att, pre, T, rows, causal, scale_log2);
        else hipLaunchKernelGGL(softmax_rows_vec_kernel<16>, grid, blk, 0, st, att, pre, T, rows, causal, scale_log2);
    } else {
        hipLaunchKernelGGL(softmax_rows_kernel, grid, blk, 0, st, att, pre, T, rows, causal, scale_log2);
    }
    return hipGetLastError();
}

template <int HS>
hipError_t fwd_hs(float* out, float* preatt, float* att, const float* qkv, const Shape& s,
                  hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    const size_t C3 = 3 * (size_t)s.C;
    const size_t bstride = (size_t)s.T * C3;
    const long long BH = (long long)s.B * s.NH;
    if (s.T % 4 == 0)
        hipLaunchKernelGGL((scores_kernel<HS, true, false>), dim3((unsigned)(BH * nt)), dim3(kThreads), 0, st,
                           preatt, qkv, qkv + s.C, s.T, s.NH, C3, C3, bstride, bstride);
    else
        hipLaunchKernelGGL((scores_kernel<HS, false, false>), dim3((unsigned)(BH * nt)), dim3(kThreads), 0,
                           st, preatt, qkv, qkv + s.C, s.T, s.NH, C3, C3, bstride, bstride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = BH * s.T;
    const float scale = (float)(1.0 / sqrt((double)HS));
    e = launch_softmax_rows(att, preatt, s.T, rows, s.causal, scale * kLog2e, st);
    if (e != hipSuccess) return e;
    const long long ga = tiles::apply_grid(BH, s.T);
    if (ga < 1 || ga > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((apply_kernel<HS, false>), dim3((unsigned)ga), dim3(kThreads), 0, st, out, att,
                       qkv + 2 * s.C, s.T, s.NH, (int)BH, s.causal, C3, (size_t)s.C, bstride,
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
    if (s.T % 4 == 0)
        hipLaunchKernelGGL((scores_kernel<HS, true, true>), dim3((unsigned)(BH * nt)), dim3(kThreads), 0, st,
                           datt, dout, qkv + 2 * C, s.T, s.NH, C, C3, bo, bq);
    else
        hipLaunchKernelGGL((scores_kernel<HS, false, true>), dim3((unsigned)(BH * nt)), dim3(kThreads), 0,
                           st, datt, dout, qkv + 2 * C, s.T, s.NH, C, C3, bo, bq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = BH * s.T;
    const float scale = (float)(1.0 / sqrt((double)HS));
    e = launch_softmax_bwd_rows(dpreatt, att, datt, s.T, rows, s.causal, scale, st);
    if (e != hipSuccess) return e;
    const long long gl = tiles::apply_grid(BH, s.T);
    if (gl < 1 || gl > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const unsigned g = (unsigned)gl;
    // dv = att^T dO
    hipLaunchKernelGGL((apply_kernel<HS, true>), dim3(g), dim3(kThreads), 0, st, dqkv + 2 * C, att,
                       dout, s.T, s.NH, (int)BH, s.causal, C, C3, bo, bq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dq = dpreatt K
    hipLaunchKernelGGL((apply_kernel<HS, false>), dim3(g), dim3(kThreads), 0, st, dqkv, dpreatt,
                       qkv + C, s.T, s.NH, (int)BH, s.causal, C3, C3, bq, bq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dk = dpreatt^T Q
    hipLaunchKernelGGL((apply_kernel<HS, true>), dim3(g), dim3(kThreads), 0, st, dqkv + C, dpreatt,
                       qkv, s.T, s.NH, (int)BH, s.causal, C3, C3, bq, bq);
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
