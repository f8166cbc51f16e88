// flash_f32.hip -- fused fp32 attention forward and backward for gfx950.
//
// Method: multi-head self-attention softmax(Q K^T / sqrt(hs)) V per head
// ("Umakini wa kujitegemea, kerneli za CUDA na FlashAttention", section 1),
// computed tile by tile with a running row maximum and normaliser so the
// T x T score matrix never leaves the chip, keeping only the per-row
// log-sum-exp for the backward, which recomputes the probabilities (the
// FlashAttention part of that page).  The backward is the analytic gradient
// of attention_backward_cpu in llm.c dev/cuda/attention_backward.cu with
// the closed-form softmax step of its softmax_autoregressive_backward_kernel7
// (dS = P * (dP - D), D = rowsum(P * dP) = rowsum(dO * O)).
//
// gfx950 mapping (wave64, v_mfma_f32_16x16x4_f32):
//  * a workgroup is 4 waves; each wave owns 16 rows of the 64-row tile it
//    keeps in registers (Q rows in the forward and dQ kernels, K/V rows in
//    the dK/dV kernel) and streams the other operand through LDS in 64-row
//    tiles read straight from the packed (B,T,3C) tensor (no permute pass);
//  * products are arranged so that the score block lands with one query per
//    lane column (S^T = K Q^T in the forward / dQ kernel): a lane then holds
//    16 scores of its own row, row statistics need only an in-lane reduction
//    plus two cross-lane exchanges (xor 16, xor 32), and the probabilities
//    feed the next product (O^T = V^T P^T) straight from the accumulator
//    registers;
//  * the contraction index k of every Q.K product is numbered
//    k = (hs/4)*g + s for lane group g and step s, so each lane's operand
//    values are contiguous and move with 16-byte loads;
//  * causal work skips every key tile beyond the diagonal; in the dQ kernel
//    a workgroup runs a light and a heavy causal tile back to back so all
//    workgroups carry equal work (no tail), while the forward and dK/dV
//    kernels run their tiles heaviest first (measured faster: their
//    occupancy does not divide the paired grid into whole rounds);
//    consecutive workgroup ids walk the heads so that all tiles of a head
//    land on one XCD (one L2) whenever B*NH is a multiple of 8;
//  * the forward raises a row's running maximum only when a tile's maximum
//    exceeds it by more than 2^kLazyMax (log2 domain), as the 16-bit forward
//    does, and folds the scale into the exponent's FMA;
//  * the fused backward (attn_backward) runs a pre-pass that forms
//    D = dO . O and clears dQ, then one dK/dV kernel that also forms dQ and
//    adds it with float atomics (bwd_dkdv_f32_tile with DQ): five
//    contractions per score, memory O(B*NH*T).  Two atomic-free orders stay
//    available as stage calls: the dQ kernel that recomputes S and dP and
//    forms D (bwd_dq_f32_tile), then dK/dV; and, for callers that own an
//    O(T^2) buffer, dK/dV storing dS (bwd_dkdv_f32_tile<HS, true>) so that
//    the dQ kernel (bwd_dq_ds_f32_tile) performs one contraction instead
//    of three.
#include "common.hpp"


namespace attn {
namespace {

constexpr int kTile = 64;      // rows per Q tile and per K/V tile
constexpr float kLazyMax = 8.0f;   // forward: lazy rescale threshold (log2 domain)
constexpr int kThreads = 256;  // 4 waves
// The forward and dQ kernels ask for >= 3 resident waves per SIMD (2 for
// hs = 128; a register cap); the dK/dV kernel does better with more
// registers.

struct Lane {
    int tid, w, l, r16, g;
    __device__ Lane() {
        tid = threadIdx.x;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: per-wave tests branch on scalars
        l = tid & 63;
        r16 = l & 15;
        g = l >> 4;
    }
};

// A kTile x HS fp32 tile held in registers between its global load and its
// LDS store, so the load of the next tile overlaps the current tile's math.
template <int HS>
struct TileRegs {
    static constexpr int C4 = HS / 4;
    static constexpr int N = kTile * C4 / kThreads;   // float4 per thread
    float4 v[N];
    // Raw buffer loads over rows row0 .. min(row0 + kTile, T) - 1: a load at
    // or past num_records returns zeros instead of reading memory, so rows
    // >= T need no predicate (each 16-byte chunk lies wholly inside or wholly
    // past that bound, as ld >= HS).  Word 3 is the gfx9 raw-buffer format word.
    __device__ __forceinline__ void fetch(const float* base, size_t ld, int row0, int T, int tid) {
        const uint32_t ldb = (uint32_t)(ld * 4);
        const int valid = min(T - row0, kTile);
        const uint32_t num = valid > 0 ? (uint32_t)(valid - 1) * ldb + HS * 4u : 0u;
        const float* p = base + (size_t)row0 * ld;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, (int)num, 0x00020000);
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = tid + k * kThreads;
            const int row = e / C4, c4 = e % C4;
            const uint32_t off = (uint32_t)row * ldb + 16u * (uint32_t)c4;
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
            __builtin_memcpy(&v[k], &x, 16);
        }
    }
    template <int LDK>
    __device__ __forceinline__ void store(float* lds, int tid) const {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = tid + k * kThreads;
            const int row = e / C4, c4 = e % C4;
            *reinterpret_cast<float4*>(lds + row * LDK + 4 * c4) = v[k];
        }
    }
};

// Load this lane's HS/4 contiguous values of one row (k = (HS/4)*g + s).
template <int HS>
__device__ __forceinline__ void load_row_part(float (&r)[HS / 4], const float* rowp, bool valid,
                                              int g) {
    constexpr int KS = HS / 4;
#pragma unroll
    for (int c = 0; c < KS / 4; ++c) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) v = *reinterpret_cast<const float4*>(rowp + KS * g + 4 * c);
        r[4 * c + 0] = v.x;
        r[4 * c + 1] = v.y;
        r[4 * c + 2] = v.z;
        r[4 * c + 3] = v.w;
    }
}

// Causal tiles carry unequal work (tile i of a Q-tile kernel sees i+1 key
// tiles, tile j of a K/V-tile kernel nt-j query tiles), so when the grid is
// large enough one workgroup runs tiles i and nt-1-i back to back: every
// workgroup then does nt+1 units and the grid has no tail.  Pairing halves
// the grid, so it is used only while at least two paired workgroups per CU
// remain (pair_tiles on the host).  Otherwise tiles run one per workgroup,
// heaviest first (the longest-first order of kernel 8 in llm.c's
// attention_backward.cu), dealt to the CUs like a snake draft (snake_block;
// the dQ kernel that reads dS -4%, the forward -0.5% on the GPT-2 layer).
// Consecutive workgroup ids walk the heads, so all tiles of a head land on
// one XCD (one L2) whenever B*NH is a multiple of 8.
__device__ __forceinline__ void pair_of_block(int BH, int nt, bool paired, bool heavy_high,
                                              Deal deal, int& bh, int& ta, int& tb) {
    const int bid = paired ? (int)blockIdx.x : snake_block(deal);
    const int rank = bid / BH;
    bh = bid - rank * BH;
    if (paired) {
        ta = rank;
        tb = nt - 1 - rank;
        if (tb == ta) tb = -1;
    } else {   // heaviest tile first, so the last workgroups to start are short
        ta = heavy_high ? nt - 1 - rank : rank;
        tb = -1;
    }
}

__host__ __device__ inline int grid_tiles(int nt, bool paired) { return paired ? (nt + 1) / 2 : nt; }

// dS block store.  The dK/dV kernel can write dS = P * (dP - D) (unscaled)
// for every (64-query tile qt, 64-key tile kt) block it computes, and the dQ
// kernel bwd_dq_ds_f32_tile then forms dQ = scale * dS K from it, instead of
// recomputing S and dP (two of the three contractions of bwd_dq_f32_tile).
// Blocks of one head: kt <= qt in causal mode (row-major lower triangle,
// index qt(qt+1)/2 + kt), all nt^2 otherwise (qt*nt + kt); heads follow each
// other.  Inside a block the 4096 values are in the dQ kernel's operand
// order: [query/16][key/16][lane][4] with lane = query%16 + 16*((key%16)/4)
// and the 4 consecutive keys 4*(key%16/4) .. +3 last, so each wave of the
// dQ kernel loads its matrix-core operands with contiguous 16-byte loads.
constexpr int kDsBlock = kTile * kTile;
__host__ __device__ inline size_t ds_blocks_per_head(int nt, int causal) {
    return causal ? (size_t)nt * (nt + 1) / 2 : (size_t)nt * nt;
}
__host__ __device__ inline size_t ds_block_floats(int qt, int kt, int nt, int causal) {
    return (causal ? (size_t)qt * (qt + 1) / 2 + kt : (size_t)qt * nt + kt) * kDsBlock;
}

// ------------------------------------------------------------------ forward
template <int HS>
__device__ __forceinline__ void fwd_f32_tile(int tile_, int bh_, float* __restrict__ out,
                                             float* __restrict__ lse,
                                             const float* __restrict__ qkv, int T, int C, int NH,
                                             int causal, float scale_log2) {
    constexpr int LDK = HS + 4;
    constexpr int KS = HS / 4;
    constexpr int NB = kTile / 16;   // 16-key blocks per tile
    constexpr int MB = HS / 16;      // 16-column blocks of O
    __shared__ float Ks[kTile * LDK];
    __shared__ float Vs[kTile * LDK];

    const Lane L;
    const int nqt = (T + kTile - 1) / kTile;
    const int qt = tile_, bh = bh_;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const float* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const float* kbase = qbase + C;
    const float* vbase = qbase + 2 * (size_t)C;

    const int qrow = qt * kTile + 16 * L.w + L.r16;
    float qreg[KS];
    load_row_part<HS>(qreg, qbase + (size_t)qrow * C3, qrow < T, L.g);

    float m = -INFINITY;   // running max of scale*log2(e)*s (log2 domain)
    float lsum = 0.f;      // this lane's share of the running normaliser
    f32x4 o[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = causal ? (qt + 1) : nqt;
    TileRegs<HS> rk, rv;
    rk.fetch(kbase, C3, 0, T, L.tid);
    rv.fetch(vbase, C3, 0, T, L.tid);
    wait_global_loads();
    for (int kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        rk.template store<LDK>(Ks, L.tid);
        rv.template store<LDK>(Vs, L.tid);
        __syncthreads();
        if (kt + 1 < nkt) {   // next tile's loads fly while this one is used
            rk.fetch(kbase, C3, (kt + 1) * kTile, T, L.tid);
            rv.fetch(vbase, C3, (kt + 1) * kTile, T, L.tid);
        }

        // S^T blocks: s[n][i] = S[qrow][kt*64 + 16n + 4g + i]; two blocks'
        // chains at a time are interleaved so that consecutive matrix-core
        // ops update different accumulators (a dependent op waits ~54
        // cycles, a chain of one alone runs at ~60% of the issue rate)
        f32x4 s[NB];
#pragma unroll
        for (int np = 0; np < NB; np += 2) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
            const float* k0r = Ks + (16 * np + L.r16) * LDK + KS * L.g;
            const float* k1r = k0r + 16 * LDK;
#pragma unroll
            for (int c = 0; c < KS / 4; ++c) {
                const float4 x = *reinterpret_cast<const float4*>(k0r + 4 * c);
                const float4 y = *reinterpret_cast<const float4*>(k1r + 4 * c);
                a0 = mfma_f32(x.x, qreg[4 * c + 0], a0);
                a1 = mfma_f32(y.x, qreg[4 * c + 0], a1);
                a0 = mfma_f32(x.y, qreg[4 * c + 1], a0);
                a1 = mfma_f32(y.y, qreg[4 * c + 1], a1);
                a0 = mfma_f32(x.z, qreg[4 * c + 2], a0);
                a1 = mfma_f32(y.z, qreg[4 * c + 2], a1);
                a0 = mfma_f32(x.w, qreg[4 * c + 3], a0);
                a1 = mfma_f32(y.w, qreg[4 * c + 3], a1);
            }
            s[np] = a0;
            s[np + 1] = a1;
        }

        // keys >= lim are masked; only the last tile holds the diagonal and
        // the tail (a workgroup-uniform branch)
        if (kt == nkt - 1) {
            const int d = (causal ? min(T, qrow + 1) : T) - (kt * kTile + 4 * L.g);
#pragma unroll
            for (int n = 0; n < NB; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[n][i] = (16 * n + i < d) ? s[n][i] : -INFINITY;
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, s[n][i]);
        mloc = group4_max(mloc) * scale_log2;   // the scale is positive: max commutes with it
        // The running maximum is raised (and O, l rescaled) only when the
        // tile's maximum exceeds it by more than kLazyMax in the log2 domain;
        // a stale maximum changes no result (numerator and denominator share
        // it) and keeps the probabilities below 2^kLazyMax.  The decision is
        // per row; the wave skips the rescale when no row needs one.
        const bool need = mloc > m + kLazyMax;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float alpha = need ? fast_exp2(m - mloc) : 1.0f;   // m = -inf -> 0
            m = need ? mloc : m;
            lsum *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
        }
        const float nm = -m;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(fmaf(s[n][i], scale_log2, nm));
                s[n][i] = p;
                lsum += p;
            }
        }

        // O^T += V^T P^T: o[mb][i'] = O[qrow][16mb + 4g + i']
#pragma unroll
        for (int n = 0; n < NB; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float* vr = Vs + (16 * n + 4 * L.g + i) * LDK + L.r16;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) o[mb] = mfma_f32(vr[16 * mb], s[n][i], o[mb]);
            }
        }
    }

    const float ltot = group4_sum(lsum);
    if (qrow < T) {
        const float inv = 1.0f / ltot;
        float* orow = out + ((size_t)b * T + qrow) * C + (size_t)h * HS;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const f32x4 v = o[mb] * inv;
            *reinterpret_cast<float4*>(orow + 16 * mb + 4 * L.g) = make_float4(v[0], v[1], v[2], v[3]);
        }
        if (L.g == 0) lse[(size_t)bh * T + qrow] = (m + __log2f(ltot)) * kLn2;
    }
}

// ------------------------------------------------------ backward pre-pass
// D[b,h,t] = sum_i dout[b,t,h*hs+i] * out[b,t,h*hs+i], one group of HS/4
// lanes per (b,t,h) row, rows in memory order.
// With dq non-null it also clears the dQ slot of the same row of dqkv (row
// stride 3C), where the fused backward then adds its dQ contributions.
template <int HS>
__global__ __launch_bounds__(kThreads) void prepass_f32_kernel(float* __restrict__ D,
                                                               const float* __restrict__ dout,
                                                               const float* __restrict__ out,
                                                               int T, int NH, long long rows,
                                                               float* __restrict__ dq) {
    constexpr int G = HS / 4;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = gid / G;
    const int part = (int)(gid - row * G);
    float acc = 0.f;
    if (row < rows) {
        const float4 a = *reinterpret_cast<const float4*>(dout + row * HS + 4 * part);
        const float4 c = *reinterpret_cast<const float4*>(out + row * HS + 4 * part);
        acc = a.x * c.x + a.y * c.y + a.z * c.z + a.w * c.w;
        if (dq) {
            const long long bt = row / NH;
            const int h = (int)(row - bt * NH);
            *reinterpret_cast<float4*>(dq + bt * 3 * NH * HS + h * HS + 4 * part) =
                make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && part == 0) {
        const long long bt = row / NH;
        const int h = (int)(row - bt * NH);
        const long long b = bt / T;
        const int t = (int)(bt - b * T);
        D[((size_t)b * NH + h) * T + t] = acc;
    }
}

// ----------------------------------------------------- backward dK / dV
// One workgroup per (64-row K/V tile, head); loops over the Q tiles that see
// it.  Per Q tile: S = Q K^T, P = exp(scale*S - lse), dV^T += dO^T P,
// dP = dO V^T, dS = P * (dP - D), dK^T += Q^T dS (scale applied at the end).
// With STORE_DS it also writes each 64x64 block of dS (unscaled) to the dS
// block store, for the dQ kernel that consumes it (bwd_dq_ds_f32_tile).
// With DQ it also forms dQ: each Q tile's dS block goes through LDS (dSt,
// query rows), and at the start of the next Q tile's step every wave
// multiplies its 16 query rows of it by the key tile (Kt, held transposed
// and scaled for the whole loop); it adds the 16 x HS result into dqkv's dQ
// slot with global float atomics spread over that step's 16-query blocks
// (~1% faster than issuing them together).  The slot must be cleared first
// (the pre-pass does it), and the order of the additions, hence dQ's last
// bits, varies from run to run.  The compiler makes the wait for the next
// tile's prefetched loads also cover every store issued before it; the last
// atomics of a step leave a 16-query block of work before that wait.
template <int HS, bool STORE_DS, bool DQ = false>
__device__ __forceinline__ void bwd_dkdv_f32_tile(
    int tile_, int bh_, float* __restrict__ dqkv, float* __restrict__ dsw,
    const float* __restrict__ dout, const float* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Dws, int T, int C, int NH, int causal, float scale,
    float scale_log2) {
    constexpr int LDK = HS + 4;
    constexpr int KS = HS / 4;
    constexpr int NB = kTile / 16;
    constexpr int MB = HS / 16;
    __shared__ float Qs[kTile * LDK];
    __shared__ float dOs[kTile * LDK];
    // per query row of the streamed tile: -lse*log2e and -D, the starting
    // values of the S and dP products (so P = exp2(S) and dS = P * dP)
    __shared__ __attribute__((aligned(16))) float Ls[kTile];
    __shared__ __attribute__((aligned(16))) float Dl[kTile];
    // per-wave 16 x 16 transpose scratch for the dS store (kTrLd floats a row)
    constexpr int kTrLd = 20, kTrWave = 16 * kTrLd;
    __shared__ __attribute__((aligned(16))) float Tr[STORE_DS ? 4 * kTrWave : 4];
    // DQ: dS of the last Q tile by query row, and the key tile transposed
    // (row = head dimension) and multiplied by scale; rows of 64 keys padded
    // to 68 floats, so the 16 rows of one 16-byte read pass fall on
    // distinct bank groups
    constexpr int LDT = kTile + 4;
    __shared__ __attribute__((aligned(16))) float dSt[DQ ? kTile * LDT : 4];
    __shared__ __attribute__((aligned(16))) float Kt[DQ ? HS * LDT : 4];
    static_assert(!(DQ && STORE_DS), "one dQ route at a time");

    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    const int kt = tile_, bh = bh_;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const float* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const float* kbase = qbase + C;
    const float* vbase = qbase + 2 * (size_t)C;
    const float* dobase = dout + (size_t)b * T * C + (size_t)h * HS;
    const float* lrow = lse + (size_t)bh * T;
    const float* drow = Dws + (size_t)bh * T;

    const int kvrow = kt * kTile + 16 * L.w + L.r16;
    float kreg[KS], vreg[KS];
    load_row_part<HS>(kreg, kbase + (size_t)kvrow * C3, kvrow < T, L.g);
    load_row_part<HS>(vreg, vbase + (size_t)kvrow * C3, kvrow < T, L.g);
    if constexpr (DQ) {   // read by the first dQ product, after the loop's barriers
#pragma unroll
        for (int k = 0; k < KS; ++k) Kt[(KS * L.g + k) * LDT + 16 * L.w + L.r16] = kreg[k] * scale;
    }
    // K enters only S: scaled once by scale*log2e, S comes out in the log2
    // domain of the exponent
#pragma unroll
    for (int k = 0; k < KS; ++k) kreg[k] *= scale_log2;

    f32x4 dk[MB], dv[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        dk[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int qt0 = causal ? kt : 0;
    TileRegs<HS> rq, rd;
    float rl = 0.f, rD = 0.f;
    auto fetch = [&](int qt) {
        rq.fetch(qbase, C3, qt * kTile, T, L.tid);
        rd.fetch(dobase, (size_t)C, qt * kTile, T, L.tid);
        // lse and D are loaded raw and transformed when stored, so nothing
        // waits for them before the next step
        if (L.tid < kTile) {
            const int q = min(qt * kTile + L.tid, T - 1);
            rl = lrow[q];
            rD = drow[q];
        }
    };
    fetch(qt0);
    wait_global_loads();
    // dS store: after the transpose this lane's 4 entries of block (qt, kt)
    // sit at ds_block_floats(qt, kt) + (n * 4 + w) * 256 + ds_lane + 16g
    [[maybe_unused]] const size_t ds_head = (size_t)bh * ds_blocks_per_head(nt, causal) * kDsBlock;
    [[maybe_unused]] const int ds_lane = 64 * (L.r16 >> 2) + 4 * (L.r16 & 3);
    [[maybe_unused]] const bool kv_in = kvrow < T;
    [[maybe_unused]] const bool kv_full = (kt + 1) * kTile <= T;   // no key of the tile past T
    // DQ: dQ rows qtp*64 + 16w + 4g + i, columns 16mb + r16 from dSt and Kt
    // (the contraction runs over the tile's keys 16g + 4c + j in lane group
    // g) into dacc; dq_add then adds row group i of it to dqkv
    [[maybe_unused]] float* dqbase = dqkv + (size_t)b * T * C3 + (size_t)h * HS;
    [[maybe_unused]] f32x4 dacc[MB];
    [[maybe_unused]] auto dq_product = [&]() {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) dacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const float* ar = dSt + (16 * L.w + L.r16) * LDT + 16 * L.g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 a4 = *reinterpret_cast<const float4*>(ar + 4 * c);
            float4 b4[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                b4[mb] = *reinterpret_cast<const float4*>(Kt + (16 * mb + L.r16) * LDT + 16 * L.g +
                                                          4 * c);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) dacc[mb] = mfma_f32(a4.x, b4[mb].x, dacc[mb]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) dacc[mb] = mfma_f32(a4.y, b4[mb].y, dacc[mb]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) dacc[mb] = mfma_f32(a4.z, b4[mb].z, dacc[mb]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) dacc[mb] = mfma_f32(a4.w, b4[mb].w, dacc[mb]);
        }
    };
    [[maybe_unused]] auto dq_add = [&](int qtp, int i) {
        const int q = qtp * kTile + 16 * L.w + 4 * L.g + i;
        if (q < T) {
            float* row = dqbase + (size_t)q * C3 + L.r16;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) unsafeAtomicAdd(row + 16 * mb, dacc[mb][i]);
        }
    };
    for (int qt = qt0; qt < nt; ++qt) {
        __syncthreads();
        rq.template store<LDK>(Qs, L.tid);
        rd.template store<LDK>(dOs, L.tid);
        if (L.tid < kTile) {
            const bool in = qt * kTile + L.tid < T;
            Ls[L.tid] = in ? -rl * kLog2e : -INFINITY;   // -inf -> P = 0
            Dl[L.tid] = in ? -rD : 0.f;
        }
        if constexpr (DQ) {
            // the previous Q tile's dS is complete (first barrier); this
            // step's dS writes come after the second barrier
            if (qt > qt0) dq_product();
            if (qt + 1 < nt) fetch(qt + 1);
            __syncthreads();
        } else {
            __syncthreads();
            if (qt + 1 < nt) fetch(qt + 1);
        }
        const bool diag = causal && (qt == kt);

#pragma unroll
        for (int n = 0; n < NB; ++n) {
            // query qt*64 + 16n + 4g + i, key kvrow: s[i] = (scale*S - lse)*log2e
            // and dp[i] = dP - D (the products start from -lse*log2e and -D)
            f32x4 s = *reinterpret_cast<const f32x4*>(Ls + 16 * n + 4 * L.g);
            f32x4 dp = *reinterpret_cast<const f32x4*>(Dl + 16 * n + 4 * L.g);
            const float* qr = Qs + (16 * n + L.r16) * LDK + KS * L.g;
            const float* dr = dOs + (16 * n + L.r16) * LDK + KS * L.g;
#pragma unroll
            for (int c = 0; c < KS / 4; ++c) {
                const float4 qa = *reinterpret_cast<const float4*>(qr + 4 * c);
                const float4 da = *reinterpret_cast<const float4*>(dr + 4 * c);
                s = mfma_f32(qa.x, kreg[4 * c + 0], s);
                dp = mfma_f32(da.x, vreg[4 * c + 0], dp);
                s = mfma_f32(qa.y, kreg[4 * c + 1], s);
                dp = mfma_f32(da.y, vreg[4 * c + 1], dp);
                s = mfma_f32(qa.z, kreg[4 * c + 2], s);
                dp = mfma_f32(da.z, vreg[4 * c + 2], dp);
                s = mfma_f32(qa.w, kreg[4 * c + 3], s);
                dp = mfma_f32(da.w, vreg[4 * c + 3], dp);
            }
            if (diag) {   // causal: query qt*64 + 16n + 4g + i sees kvrow iff i >= d
                const int d = kvrow - (qt * kTile + 16 * n + 4 * L.g);
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = (i >= d) ? s[i] : -INFINITY;
            }
            float p[4], ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = fast_exp2(s[i]);
                p[i] = pv;
                ds[i] = pv * dp[i];
            }
            if constexpr (STORE_DS) {
                // ds[i] is entry (query 16n + 4g + i, key 16w + 4a + b) of the
                // block, a = r16 / 4, b = r16 % 4; keys past T are stored as
                // 0 (their scores are not masked in a non-causal ragged
                // tile).  The wave's 16 x 16 entries pass through its LDS
                // scratch (row = query, stride 20: conflict-free writes), so
                // that lane (a, b, g) reads back (query 4g + b, keys 4a ..
                // 4a + 3), one 16-byte store of the operand layout.  A wave
                // executes its LDS operations in order; the wave barriers
                // keep the compiler from moving them across each other.
                float x[4];
                if (kv_full) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = ds[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = kv_in ? ds[i] : 0.f;
                }
                float* trw = Tr + L.w * kTrWave;
#pragma unroll
                for (int i = 0; i < 4; ++i) trw[(4 * L.g + i) * kTrLd + L.r16] = x[i];
                __builtin_amdgcn_wave_barrier();
                const float4 y = *reinterpret_cast<const float4*>(
                    trw + (4 * L.g + (L.r16 & 3)) * kTrLd + 4 * (L.r16 >> 2));
                __builtin_amdgcn_wave_barrier();
                float* blk = dsw + ds_head + ds_block_floats(qt, kt, nt, causal) +
                             (size_t)((n * 4 + L.w) * 256 + ds_lane + 4 * (4 * L.g));
                // non-temporal: the store streams past L2 (the dQ kernel reads
                // it back; with the hint on both sides the step is ~1% faster)
                __builtin_nontemporal_store(f32x4{y.x, y.y, y.z, y.w}, reinterpret_cast<f32x4*>(blk));
            }
            if constexpr (DQ) {   // entry (query 16n + 4g + i, key 16w + r16)
#pragma unroll
                for (int i = 0; i < 4; ++i) dSt[(16 * n + 4 * L.g + i) * LDT + 16 * L.w + L.r16] = ds[i];
                // the previous Q tile's dQ atomics, spread over this step
                // (the last two groups after its third 16-query block)
                if (qt > qt0) {
                    if (n < 2) dq_add(qt - 1, n);
                    if (n == 2) {
                        dq_add(qt - 1, 2);
                        dq_add(qt - 1, 3);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ql = 16 * n + 4 * L.g + i;
                const float* dor = dOs + ql * LDK + L.r16;
                const float* qrr = Qs + ql * LDK + L.r16;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    dv[mb] = mfma_f32(dor[16 * mb], p[i], dv[mb]);
                    dk[mb] = mfma_f32(qrr[16 * mb], ds[i], dk[mb]);
                }
            }
        }
    }

    if constexpr (DQ) {
        __syncthreads();
        dq_product();
#pragma unroll
        for (int i = 0; i < 4; ++i) dq_add(nt - 1, i);
    }
    if (kvrow < T) {
        float* dkrow = dqkv + ((size_t)b * T + kvrow) * C3 + C + (size_t)h * HS;
        float* dvrow = dkrow + C;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const f32x4 a = dk[mb] * scale;
            const f32x4 v = dv[mb];
            *reinterpret_cast<float4*>(dkrow + 16 * mb + 4 * L.g) = make_float4(a[0], a[1], a[2], a[3]);
            *reinterpret_cast<float4*>(dvrow + 16 * mb + 4 * L.g) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

// ----------------------------------------------------------- backward dQ
// One workgroup per (64-row Q tile, head); loops over the key tiles it sees.
// It first forms D = dO . O for its rows (written out for the dK/dV kernel,
// which runs after it).  Per K/V tile: S^T = K Q^T, P, dP^T = V dO^T,
// dS = P * (dP - D), dQ^T += K^T dS^T (scale applied at the end).
template <int HS>
__device__ __forceinline__ void bwd_dq_f32_tile(
    int tile_, int bh_, float* __restrict__ dqkv, float* __restrict__ Dws,
    const float* __restrict__ dout, const float* __restrict__ qkv, const float* __restrict__ out,
    const float* __restrict__ lse, int T, int C, int NH, int causal, float scale,
    float scale_log2) {
    constexpr int LDK = HS + 4;
    constexpr int KS = HS / 4;
    constexpr int NB = kTile / 16;
    constexpr int MB = HS / 16;
    __shared__ float Ks[kTile * LDK];
    __shared__ float Vs[kTile * LDK];

    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    const int qt = tile_, bh = bh_;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const float* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const float* kbase = qbase + C;
    const float* vbase = qbase + 2 * (size_t)C;
    const float* dobase = dout + (size_t)b * T * C + (size_t)h * HS;

    const int qrow = qt * kTile + 16 * L.w + L.r16;
    const bool qvalid = qrow < T;
    float qreg[KS], doreg[KS];
    load_row_part<HS>(qreg, qbase + (size_t)qrow * C3, qvalid, L.g);
    load_row_part<HS>(doreg, dobase + (size_t)qrow * C, qvalid, L.g);
    const float l2 = qvalid ? lse[(size_t)bh * T + qrow] * kLog2e : INFINITY;
    // D = dO . O for this row (the pre-pass, fused): the lane's HS/4 columns,
    // then the four lanes of the row; written for the dK/dV kernel.
    float Dq;
    {
        float oreg[KS];
        load_row_part<HS>(oreg, out + (size_t)b * T * C + (size_t)h * HS + (size_t)qrow * C, qvalid, L.g);
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) acc = fmaf(doreg[k], oreg[k], acc);
        Dq = group4_sum(acc);
        if (qvalid && L.g == 0) Dws[(size_t)bh * T + qrow] = Dq;
    }

    f32x4 dq[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) dq[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Q enters only S: scaled by scale*log2e, and the S and dP products start
    // from -lse*log2e and -D, so P = exp2(S) and dS = P * dP
#pragma unroll
    for (int k = 0; k < KS; ++k) qreg[k] *= scale_log2;
    const f32x4 s0 = {-l2, -l2, -l2, -l2}, dp0 = {-Dq, -Dq, -Dq, -Dq};

    const int nkt = causal ? (qt + 1) : nt;
    TileRegs<HS> rk, rv;
    rk.fetch(kbase, C3, 0, T, L.tid);
    rv.fetch(vbase, C3, 0, T, L.tid);
    wait_global_loads();
    for (int kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        rk.template store<LDK>(Ks, L.tid);
        rv.template store<LDK>(Vs, L.tid);
        __syncthreads();
        if (kt + 1 < nkt) {
            rk.fetch(kbase, C3, (kt + 1) * kTile, T, L.tid);
            rv.fetch(vbase, C3, (kt + 1) * kTile, T, L.tid);
        }
        const bool edge = kt == nkt - 1;   // the tile that holds the diagonal and the T tail
        const int lim = causal ? min(T, qrow + 1) : T;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            // s[i] = (scale*S - lse)*log2e, dp[i] = dP - D for qrow and key kt*64 + 16n + 4g + i
            f32x4 s = s0, dp = dp0;
            const float* kr = Ks + (16 * n + L.r16) * LDK + KS * L.g;
            const float* vr = Vs + (16 * n + L.r16) * LDK + KS * L.g;
#pragma unroll
            for (int c = 0; c < KS / 4; ++c) {
                const float4 ka = *reinterpret_cast<const float4*>(kr + 4 * c);
                const float4 va = *reinterpret_cast<const float4*>(vr + 4 * c);
                s = mfma_f32(ka.x, qreg[4 * c + 0], s);
                dp = mfma_f32(va.x, doreg[4 * c + 0], dp);
                s = mfma_f32(ka.y, qreg[4 * c + 1], s);
                dp = mfma_f32(va.y, doreg[4 * c + 1], dp);
                s = mfma_f32(ka.z, qreg[4 * c + 2], s);
                dp = mfma_f32(va.z, doreg[4 * c + 2], dp);
                s = mfma_f32(ka.w, qreg[4 * c + 3], s);
                dp = mfma_f32(va.w, doreg[4 * c + 3], dp);
            }
            if (edge) {   // key kt*64 + 16n + 4g + i stays iff i < d (else P = 0)
                const int d = lim - (kt * kTile + 16 * n + 4 * L.g);
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = (i < d) ? s[i] : -INFINITY;
            }
            float ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ds[i] = fast_exp2(s[i]) * dp[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float* kr2 = Ks + (16 * n + 4 * L.g + i) * LDK + L.r16;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) dq[mb] = mfma_f32(kr2[16 * mb], ds[i], dq[mb]);
            }
        }
    }

    if (qvalid) {
        float* dqrow = dqkv + ((size_t)b * T + qrow) * C3 + (size_t)h * HS;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const f32x4 a = dq[mb] * scale;
            *reinterpret_cast<float4*>(dqrow + 16 * mb + 4 * L.g) = make_float4(a[0], a[1], a[2], a[3]);
        }
    }
}

// ------------------------------------------------- backward dQ from dS
// One workgroup per (64-row Q tile, head); loops over the key tiles it sees
// and forms dQ^T += K^T dS^T from the stored dS blocks (the third
// contraction of bwd_dq_f32_tile, with S and dP not recomputed).  K tiles
// stream through LDS; each lane loads its dS operands (4 consecutive keys of
// its query row per 16-key block) straight from the block store, one tile
// ahead.  Rows >= T are not stored; keys >= T carry dS = 0 and zero K rows.
template <int HS>
__device__ __forceinline__ void bwd_dq_ds_f32_tile(int tile_, int bh_, float* __restrict__ dqkv,
                                                   const float* __restrict__ dsw,
                                                   const float* __restrict__ qkv, int T, int C,
                                                   int NH, int causal, float scale) {
    constexpr int LDK = HS + 4;
    constexpr int MB = HS / 16;
    __shared__ float Ks[kTile * LDK];

    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    const int qt = tile_, bh = bh_;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const float* kbase = qkv + (size_t)b * T * C3 + C + (size_t)h * HS;
    const int qrow = qt * kTile + 16 * L.w + L.r16;

    // this lane's operands of block (qt, kt): row + kt * kDsBlock + n * 256
    const float* dsrow = dsw + (size_t)bh * ds_blocks_per_head(nt, causal) * kDsBlock +
                         ds_block_floats(qt, 0, nt, causal) + (size_t)(L.w * 1024 + 4 * L.l);

    f32x4 dq[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) dq[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = causal ? (qt + 1) : nt;
    TileRegs<HS> rk;
    // two register sets for the dS operands, used in turn: copying a
    // prefetch set into a working set costs 16 moves per tile, which do not
    // overlap the fp32 matrix-core ops
    float4 dA[4], dB[4];
    auto fetch_ds = [&](float4 (&d)[4], int kt) {
        const float* p = dsrow + (size_t)kt * kDsBlock;
#pragma unroll
        for (int n = 0; n < 4; ++n) {   // read once: non-temporal, K tiles keep L2
            const f32x4 t4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + n * 256));
            d[n] = make_float4(t4[0], t4[1], t4[2], t4[3]);
        }
    };
    // one key tile: K to LDS, then the prefetch of key tile kn (K and dS,
    // into nx; kn = kt itself on the last tile, so that no branch separates
    // the two steps of the loop below and the compiler cannot sink the loads
    // past the products), then the products with the dS operands in cur
    auto step = [&](int kt, int kn, const float4 (&cur)[4], float4 (&nx)[4]) {
        __syncthreads();
        rk.template store<LDK>(Ks, L.tid);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        rk.fetch(kbase, C3, kn * kTile, T, L.tid);
        fetch_ds(nx, kn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const float dsv[4] = {cur[n].x, cur[n].y, cur[n].z, cur[n].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // dS[qrow][key 16n + 4g + i] against K row 16n + 4g + i
                const float* kr2 = Ks + (16 * n + 4 * L.g + i) * LDK + L.r16;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) dq[mb] = mfma_f32(kr2[16 * mb], dsv[i], dq[mb]);
            }
        }
    };
    rk.fetch(kbase, C3, 0, T, L.tid);
    fetch_ds(dA, 0);
    wait_global_loads();
    int kt = 0;
    for (; kt + 1 < nkt; kt += 2) {
        step(kt, kt + 1, dA, dB);
        step(kt + 1, min(kt + 2, nkt - 1), dB, dA);
    }
    if (kt < nkt) step(kt, kt, dA, dB);

    if (qrow < T) {
        float* dqrow = dqkv + ((size_t)b * T + qrow) * C3 + (size_t)h * HS;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const f32x4 a = dq[mb] * scale;
            *reinterpret_cast<float4*>(dqrow + 16 * mb + 4 * L.g) = make_float4(a[0], a[1], a[2], a[3]);
        }
    }
}

// ------------------------------------------------------------- kernels
// Each runs its tile function on one tile, or on a balanced pair of causal
// tiles (see pair_of_block).
template <int HS>
__global__ __launch_bounds__(kThreads, HS >= 128 ? 2 : 3) void fwd_f32_kernel(float* __restrict__ out,
                                                              float* __restrict__ lse,
                                                              const float* __restrict__ qkv,
                                                              int T, int C, int NH, int causal,
                                                              float scale_log2, int paired, Deal deal) {
    const int nt = (T + kTile - 1) / kTile;
    int bh, ta, tb;
    pair_of_block(gridDim.x / grid_tiles(nt, paired), nt, paired, causal != 0, deal, bh, ta, tb);
    fwd_f32_tile<HS>(ta, bh, out, lse, qkv, T, C, NH, causal, scale_log2);
    if (tb >= 0) {
        __syncthreads();
        fwd_f32_tile<HS>(tb, bh, out, lse, qkv, T, C, NH, causal, scale_log2);
    }
}

// hs <= 64 without the dS store: three workgroups per CU (162 VGPRs; the
// compiler's own choice was 174, two per CU): GPT-2 layer dK/dV 220 -> 214
// us, same bits.  With the store the same cap spills.  With DQ the LDS
// (68.5 KB at hs = 64) allows two per CU, and 216 VGPRs fit that.
template <int HS, bool STORE_DS, bool DQ = false>
__global__ __launch_bounds__(kThreads, HS >= 128 || STORE_DS ? 1 : (DQ ? 2 : 3)) void bwd_dkdv_f32_kernel(
    float* __restrict__ dqkv, float* __restrict__ dsw, const float* __restrict__ dout,
    const float* __restrict__ qkv, const float* __restrict__ lse, const float* __restrict__ Dws,
    int T, int C, int NH, int causal, float scale, float scale_log2, int paired, Deal deal) {
    const int nt = (T + kTile - 1) / kTile;
    int bh, ta, tb;
    pair_of_block(gridDim.x / grid_tiles(nt, paired), nt, paired, false, deal, bh, ta, tb);
    bwd_dkdv_f32_tile<HS, STORE_DS, DQ>(ta, bh, dqkv, dsw, dout, qkv, lse, Dws, T, C, NH, causal,
                                    scale, scale_log2);
    if (tb >= 0) {
        __syncthreads();
        bwd_dkdv_f32_tile<HS, STORE_DS, DQ>(tb, bh, dqkv, dsw, dout, qkv, lse, Dws, T, C, NH, causal,
                                        scale, scale_log2);
    }
}

template <int HS>
__global__ __launch_bounds__(kThreads) void bwd_dq_ds_f32_kernel(float* __restrict__ dqkv,
                                                                 const float* __restrict__ dsw,
                                                                 const float* __restrict__ qkv,
                                                                 int T, int C, int NH, int causal,
                                                                 float scale, Deal deal) {
    const int nt = (T + kTile - 1) / kTile;
    int bh, ta, tb;
    pair_of_block(gridDim.x / nt, nt, false, causal != 0, deal, bh, ta, tb);
    bwd_dq_ds_f32_tile<HS>(ta, bh, dqkv, dsw, qkv, T, C, NH, causal, scale);
}

template <int HS>
__global__ __launch_bounds__(kThreads, HS >= 128 ? 2 : 3) void bwd_dq_f32_kernel(
    float* __restrict__ dqkv, float* __restrict__ Dws, const float* __restrict__ dout,
    const float* __restrict__ qkv, const float* __restrict__ out, const float* __restrict__ lse,
    int T, int C, int NH, int causal, float scale, float scale_log2, int paired, Deal deal) {
    const int nt = (T + kTile - 1) / kTile;
    int bh, ta, tb;
    pair_of_block(gridDim.x / grid_tiles(nt, paired), nt, paired, causal != 0, deal, bh, ta, tb);
    bwd_dq_f32_tile<HS>(ta, bh, dqkv, Dws, dout, qkv, out, lse, T, C, NH, causal, scale, scale_log2);
    if (tb >= 0) {
        __syncthreads();
        bwd_dq_f32_tile<HS>(tb, bh, dqkv, Dws, dout, qkv, out, lse, T, C, NH, causal, scale, scale_log2);
    }
}

template <int HS>
hipError_t fwd_f32_hs(float* out, float* lse, const float* qkv, const Shape& s, hipStream_t st) {
    const int nqt = (s.T + kTile - 1) / kTile;
    // The forward holds four workgroups per CU (128 VGPRs at hs <= 64) and
    // runs its causal tiles unpaired, heaviest first: the hardware hands the
    // lighter tiles to CUs as slots free, which measured faster than equal
    // pairs (GPT-2 layer -2.5%, long context -2.3%).
    const bool paired = false;
    const unsigned grid = (unsigned)(grid_tiles(nqt, paired) * s.B * s.NH);
    const float scale_log2 = (float)(1.0 / sqrt((double)HS)) * kLog2e;
    hipLaunchKernelGGL(fwd_f32_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, out, lse, qkv, s.T,
                       s.C, s.NH, s.causal, scale_log2, (int)paired,
                       deal_for<fwd_f32_kernel<HS>>(kThreads));
    return hipGetLastError();
}

template <int HS>
hipError_t prepass_f32_hs(float* D, const float* dout, const float* out, const Shape& s,
                          hipStream_t st, float* dq = nullptr) {
    const long long rows = (long long)s.B * s.T * s.NH;
    const long long threads = rows * (HS / 4);
    const unsigned grid = (unsigned)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(prepass_f32_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, D, dout, out,
                       s.T, s.NH, rows, dq);
    return hipGetLastError();
}

template <int HS>
hipError_t dkdv_f32_hs(float* dqkv, float* dsw, const float* dout, const float* qkv,
                       const float* lse, const float* D, const Shape& s, hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    // Two workgroups fit per CU, so equal pairs left the last half round of
    // the GPT-2 layer's grid (768 pairs on 512 slots) running one per CU;
    // unpaired tiles, heaviest first, let the hardware fill freed slots with
    // lighter ones (GPT-2 layer dK/dV -3.4%, long context unchanged).
    const bool paired = false;
    const unsigned grid = (unsigned)(grid_tiles(nt, paired) * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    if (dsw)
        hipLaunchKernelGGL((bwd_dkdv_f32_kernel<HS, true>), dim3(grid), dim3(kThreads), 0, st, dqkv,
                           dsw, dout, qkv, lse, D, s.T, s.C, s.NH, s.causal, scale,
                           scale * kLog2e, (int)paired,
                           deal_for<bwd_dkdv_f32_kernel<HS, true>>(kThreads));
    else
        hipLaunchKernelGGL((bwd_dkdv_f32_kernel<HS, false>), dim3(grid), dim3(kThreads), 0, st,
                           dqkv, dsw, dout, qkv, lse, D, s.T, s.C, s.NH, s.causal, scale,
                           scale * kLog2e, (int)paired,
                           deal_for<bwd_dkdv_f32_kernel<HS, false>>(kThreads));
    return hipGetLastError();
}

// One kernel for dK, dV and dQ (bwd_dkdv_f32_tile with DQ): 5 contractions
// per score instead of the recompute order's 7.  D and a cleared dQ slot
// come from the pre-pass (prepass_f32_hs with dq).
template <int HS>
hipError_t dkdvdq_f32_hs(float* dqkv, const float* dout, const float* qkv, const float* lse,
                         const float* D, const Shape& s, hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    const bool paired = false;   // heaviest first, as the dK/dV kernel
    const unsigned grid = (unsigned)(grid_tiles(nt, paired) * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<HS, false, true>), dim3(grid), dim3(kThreads), 0, st,
                       dqkv, nullptr, dout, qkv, lse, D, s.T, s.C, s.NH, s.causal, scale,
                       scale * kLog2e, (int)paired,
                       deal_for<bwd_dkdv_f32_kernel<HS, false, true>>(kThreads));
    return hipGetLastError();
}

template <int HS>
hipError_t dq_ds_f32_hs(float* dqkv, const float* dsw, const float* qkv, const Shape& s,
                        hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    // one Q tile per workgroup, heaviest first in causal mode
    const unsigned grid = (unsigned)((long long)nt * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    hipLaunchKernelGGL(bwd_dq_ds_f32_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, dqkv, dsw, qkv,
                       s.T, s.C, s.NH, s.causal, scale, deal_for<bwd_dq_ds_f32_kernel<HS>>(kThreads));
    return hipGetLastError();
}

template <int HS>
hipError_t dq_f32_hs(float* dqkv, float* D, const float* dout, const float* qkv, const float* out,
                     const float* lse, const Shape& s, hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    const bool paired = pair_tiles(nt, s.causal, (long long)s.B * s.NH);
    const unsigned grid = (unsigned)(grid_tiles(nt, paired) * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    hipLaunchKernelGGL(bwd_dq_f32_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, dqkv, D, dout, qkv,
                       out, lse, s.T, s.C, s.NH, s.causal, scale, scale * kLog2e, (int)paired,
                       deal_for<bwd_dq_f32_kernel<HS>>(kThreads));
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

hipError_t launch_fwd_f32(float* out, float* lse, const float* qkv, const Shape& s,
                          hipStream_t st) {
    ATTN_DISPATCH_HS(fwd_f32_hs, out, lse, qkv, s, st)
}

hipError_t launch_prepass_f32(float* D, const float* dout, const float* out, const Shape& s,
                              hipStream_t st) {
    ATTN_DISPATCH_HS(prepass_f32_hs, D, dout, out, s, st)
}

hipError_t launch_dkdv_f32(float* dqkv, const float* dout, const float* qkv, const float* lse,
                           const float* D, const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(dkdv_f32_hs, dqkv, nullptr, dout, qkv, lse, D, s, st)
}

hipError_t launch_dkdv_ds_f32(float* dqkv, float* dS, const float* dout, const float* qkv,
                              const float* lse, const float* D, const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(dkdv_f32_hs, dqkv, dS, dout, qkv, lse, D, s, st)
}

hipError_t launch_prepare_f32(float* dqkv, float* D, const float* dout, const float* out,
                             const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(prepass_f32_hs, D, dout, out, s, st, dqkv)
}

hipError_t launch_dkdvdq_f32(float* dqkv, const float* dout, const float* qkv, const float* lse,
                             const float* D, const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(dkdvdq_f32_hs, dqkv, dout, qkv, lse, D, s, st)
}

hipError_t launch_dq_ds_f32(float* dqkv, const float* dS, const float* qkv, const Shape& s,
                            hipStream_t st) {
    ATTN_DISPATCH_HS(dq_ds_f32_hs, dqkv, dS, qkv, s, st)
}

size_t ds_store_floats(const Shape& s) {
    const int nt = (s.T + kTile - 1) / kTile;
    return (size_t)s.B * s.NH * ds_blocks_per_head(nt, s.causal) * kDsBlock;
}

hipError_t launch_dq_f32(float* dqkv, float* D, const float* dout, const float* qkv,
                         const float* out, const float* lse, const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(dq_f32_hs, dqkv, D, dout, qkv, out, lse, s, st)
}

#undef ATTN_DISPATCH_HS

}  // namespace attn
