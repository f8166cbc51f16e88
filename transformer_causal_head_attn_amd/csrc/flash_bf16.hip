// flash_bf16.hip -- fused attention forward and backward with bfloat16
// tensors and fp32 accumulation for gfx950 (v_mfma_f32_16x16x32_bf16).
//
// Same method and tiling as the fp32 kernels (flash_f32.hip): the
// self-attention of "Umakini wa kujitegemea, kerneli za CUDA na
// FlashAttention" (section 1) computed tile by tile with a running softmax,
// keeping only the per-row log-sum-exp, and the analytic backward of
// attention_backward_cpu in llm.c dev/cuda/attention_backward.cu with the
// closed-form softmax gradient of its kernel 7.  Low-precision operands with
// higher-precision accumulation follow the mixed-precision part of "LLM
// Systems 10 & 11: Accelerating Transformer Training and Inference"
// (section 1): Q, K, V, dO are bf16, every product accumulates in fp32, the
// softmax runs in fp32, and P and dS are rounded to bf16 only to enter the
// matrix cores.  lse and D stay fp32.
//
// gfx950 mapping.  One bf16 MFMA contracts 32 k-values: lane group g = l/16
// supplies eight of them.  For Q.K and dO.V the contraction is over hs and a
// lane takes k = 32s + 8g .. +7 (16 contiguous bytes).  For the products
// that contract over keys or queries (P V, dO^T P, Q^T dS, K^T dS^T) the
// operand coming out of the score accumulators holds, in lane group g, the
// rows 16n + 4g + i; a 32-wide step t then pairs score blocks n = 2t, 2t+1
// and lane group g supplies rows {32t + 4g + i, 32t + 16 + 4g + i : i < 4}.
// The matching operand is read from a transposed LDS copy of its tile
// (feature-major), two 8-byte reads per step.  Tiles are staged once from
// global memory into whichever of the row-major and transposed LDS copies
// the kernel needs.
#include "common.hpp"

namespace attn {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr int kLDT = kTile + 8;   // row stride (elements) of transposed tiles

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

template <int HS>
struct BfGeom {
    static constexpr int LDR = HS + 8;                 // row-major tile stride (elements)
    static constexpr int KSTEPS = HS >= 32 ? HS / 32 : 1;
    static constexpr int MB = HS / 16;
    static constexpr int NB = kTile / 16;
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    return as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
}

// Eight bf16 of one row for contraction step s: k = 32s + 8g .. +7.
// Lanes whose k-range lies beyond HS (only when HS = 16) supply zeros.
template <int HS>
__device__ __forceinline__ bf16x8 load_kchunk_global(const uint16_t* rowp, bool valid, int s,
                                                     int g) {
    const int k0 = 32 * s + 8 * g;
    if (!valid || k0 >= HS) return zero_bf16x8();
    return as_bf16x8(*reinterpret_cast<const uint4*>(rowp + k0));
}

template <int HS>
__device__ __forceinline__ bf16x8 load_kchunk_lds(const uint16_t* rowp, int s, int g) {
    const int k0 = 32 * s + 8 * g;
    if (k0 >= HS) return zero_bf16x8();
    return as_bf16x8(*reinterpret_cast<const uint4*>(rowp + k0));
}

// Stage a kTile x HS bf16 tile (global rows row0.., stride ld elements) into
// LDS: row-major copy `rm` (stride LDR) and/or transposed copy `tr`
// (tr[d*kLDT + row], stride kLDT).  Rows >= T are zero.  Each work item
// moves two rows x 8 columns so the transposed copy is written as packed
// pairs of rows (one dword per column).
template <int HS, bool ROW, bool TRANS>
__device__ __forceinline__ void stage_tile_bf16(uint16_t* rm, uint16_t* tr, const uint16_t* base,
                                                size_t ld, int row0, int T, int tid) {
    constexpr int CH = HS / 8;                 // 16-byte chunks per row
    constexpr int ITEMS = (kTile / 2) * CH;
    constexpr int LDR = BfGeom<HS>::LDR;
#pragma unroll
    for (int e = tid; e < ITEMS; e += kThreads) {
        const int rp = e / CH, c = e - (e / CH) * CH;
        const int r0 = 2 * rp;
        const int j0 = row0 + r0;
        uint4 a = make_uint4(0u, 0u, 0u, 0u), b = make_uint4(0u, 0u, 0u, 0u);
        if (j0 < T) a = *reinterpret_cast<const uint4*>(base + (size_t)j0 * ld + 8 * c);
        if (j0 + 1 < T) b = *reinterpret_cast<const uint4*>(base + (size_t)(j0 + 1) * ld + 8 * c);
        if (ROW) {
            *reinterpret_cast<uint4*>(rm + r0 * LDR + 8 * c) = a;
            *reinterpret_cast<uint4*>(rm + (r0 + 1) * LDR + 8 * c) = b;
        }
        if (TRANS) {
            const uint32_t av[4] = {a.x, a.y, a.z, a.w};
            const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // columns 8c + 2q (low halves) and 8c + 2q + 1 (high halves)
                const uint32_t lo = (av[q] & 0xffffu) | (bv[q] << 16);
                const uint32_t hi = (av[q] >> 16) | (bv[q] & 0xffff0000u);
                *reinterpret_cast<uint32_t*>(tr + (8 * c + 2 * q) * kLDT + r0) = lo;
                *reinterpret_cast<uint32_t*>(tr + (8 * c + 2 * q + 1) * kLDT + r0) = hi;
            }
        }
    }
}

// Operand for a key/query-contracting product read from a transposed tile:
// row `d` of tr, entries {32t + 4g + i, 32t + 16 + 4g + i : i < 4}.
__device__ __forceinline__ bf16x8 load_trans_operand(const uint16_t* tr, int d, int t, int g) {
    const uint16_t* p = tr + d * kLDT + 32 * t + 4 * g;
    const uint2 lo = *reinterpret_cast<const uint2*>(p);
    const uint2 hi = *reinterpret_cast<const uint2*>(p + 16);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Pack score-layout values of blocks n = 2t (x) and 2t+1 (y) into the
// matching 8-entry bf16 operand.
__device__ __forceinline__ bf16x8 pack_pair(const f32x4& x, const f32x4& y) {
    bf16x8 r;
    r[0] = (__bf16)x[0];
    r[1] = (__bf16)x[1];
    r[2] = (__bf16)x[2];
    r[3] = (__bf16)x[3];
    r[4] = (__bf16)y[0];
    r[5] = (__bf16)y[1];
    r[6] = (__bf16)y[2];
    r[7] = (__bf16)y[3];
    return r;
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, const f32x4& v) {
    bf16x4 r;
    r[0] = (__bf16)v[0];
    r[1] = (__bf16)v[1];
    r[2] = (__bf16)v[2];
    r[3] = (__bf16)v[3];
    __builtin_memcpy(p, &r, 8);
}

__device__ __forceinline__ void tile_of_block(int BH, int ntiles, bool heavy_first_high,
                                              int& tile, int& bh) {
    const int bid = blockIdx.x;
    const int rank = bid / BH;
    bh = bid - rank * BH;
    tile = heavy_first_high ? (ntiles - 1 - rank) : rank;
}

// ------------------------------------------------------------------ forward
template <int HS>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(uint16_t* __restrict__ out,
                                                            float* __restrict__ lse,
                                                            const uint16_t* __restrict__ qkv,
                                                            int T, int C, int NH, int causal,
                                                            float scale_log2) {
    using G = BfGeom<HS>;
    __shared__ uint16_t Ks[kTile * G::LDR];
    __shared__ uint16_t Vt[HS * kLDT];

    const Lane L;
    const int nqt = (T + kTile - 1) / kTile;
    const int BH = gridDim.x / nqt;
    int qt, bh;
    tile_of_block(BH, nqt, causal != 0, qt, bh);
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const uint16_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint16_t* kbase = qbase + C;
    const uint16_t* vbase = qbase + 2 * (size_t)C;

    const int qrow = qt * kTile + 16 * L.w + L.r16;
    bf16x8 qreg[G::KSTEPS];
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s)
        qreg[s] = load_kchunk_global<HS>(qbase + (size_t)qrow * C3, qrow < T, s, L.g);

    float m = -INFINITY, lsum = 0.f;
    f32x4 o[G::MB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = causal ? (qt + 1) : nqt;
    for (int kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        stage_tile_bf16<HS, true, false>(Ks, nullptr, kbase, C3, kt * kTile, T, L.tid);
        stage_tile_bf16<HS, false, true>(nullptr, Vt, vbase, C3, kt * kTile, T, L.tid);
        __syncthreads();

        f32x4 s[G::NB];
#pragma unroll
        for (int n = 0; n < G::NB; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* kr = Ks + (16 * n + L.r16) * G::LDR;
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st)
                acc = mfma_bf16(load_kchunk_lds<HS>(kr, st, L.g), qreg[st], acc);
            s[n] = acc;
        }

        const bool edge = (kt == nkt - 1);
        float mloc = -INFINITY;
#pragma unroll
        for (int n = 0; n < G::NB; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[n][i] * scale_log2;
                if (edge) {
                    const int kv = kt * kTile + 16 * n + 4 * L.g + i;
                    if (kv >= T || (causal && kv > qrow)) x = -INFINITY;
                }
                s[n][i] = x;
                mloc = fmaxf(mloc, x);
            }
        }
        mloc = group4_max(mloc);
        const float mnew = fmaxf(m, mloc);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        float psum = 0.f;
#pragma unroll
        for (int n = 0; n < G::NB; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[n][i] - mnew);
                s[n][i] = p;
                psum += p;
            }
        }
        lsum = lsum * alpha + psum;
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) o[mb] *= alpha;

        // O^T += V^T P^T, 32 keys per step
#pragma unroll
        for (int t = 0; t < G::NB / 2; ++t) {
            const bf16x8 pb = pack_pair(s[2 * t], s[2 * t + 1]);
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb)
                o[mb] = mfma_bf16(load_trans_operand(Vt, 16 * mb + L.r16, t, L.g), pb, o[mb]);
        }
    }

    const float ltot = group4_sum(lsum);
    if (qrow < T) {
        const float inv = 1.0f / ltot;
        uint16_t* orow = out + ((size_t)b * T + qrow) * C + (size_t)h * HS;
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) store_bf16x4(orow + 16 * mb + 4 * L.g, o[mb] * inv);
        if (L.g == 0) lse[(size_t)bh * T + qrow] = (m + __log2f(ltot)) * kLn2;
    }
}

// ------------------------------------------------------ backward pre-pass
template <int HS>
__global__ __launch_bounds__(kThreads) void prepass_bf16_kernel(float* __restrict__ D,
                                                                const uint16_t* __restrict__ dout,
                                                                const uint16_t* __restrict__ out,
                                                                int T, int NH, long long rows) {
    constexpr int G = HS / 8;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = gid / G;
    const int part = (int)(gid - row * G);
    float acc = 0.f;
    if (row < rows) {
        const uint4 a = *reinterpret_cast<const uint4*>(dout + row * HS + 8 * part);
        const uint4 c = *reinterpret_cast<const uint4*>(out + row * HS + 8 * part);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w};
        const uint32_t cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc += __uint_as_float(av[q] << 16) * __uint_as_float(cv[q] << 16);
            acc += __uint_as_float(av[q] & 0xffff0000u) * __uint_as_float(cv[q] & 0xffff0000u);
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
template <int HS>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_bf16_kernel(
    uint16_t* __restrict__ dqkv, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Dws, int T, int C, int NH, int causal, float scale,
    float scale_log2) {
    using G = BfGeom<HS>;
    __shared__ uint16_t Qs[kTile * G::LDR];
    __shared__ uint16_t dOs[kTile * G::LDR];
    __shared__ uint16_t Qt[HS * kLDT];
    __shared__ uint16_t dOt[HS * kLDT];
    __shared__ float Ls[kTile];
    __shared__ float Dl[kTile];

    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    const int BH = gridDim.x / nt;
    int kt, bh;
    tile_of_block(BH, nt, false, kt, bh);
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const uint16_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint16_t* kbase = qbase + C;
    const uint16_t* vbase = qbase + 2 * (size_t)C;
    const uint16_t* dobase = dout + (size_t)b * T * C + (size_t)h * HS;
    const float* lrow = lse + (size_t)bh * T;
    const float* drow = Dws + (size_t)bh * T;

    const int kvrow = kt * kTile + 16 * L.w + L.r16;
    bf16x8 kreg[G::KSTEPS], vreg[G::KSTEPS];
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s) {
        kreg[s] = load_kchunk_global<HS>(kbase + (size_t)kvrow * C3, kvrow < T, s, L.g);
        vreg[s] = load_kchunk_global<HS>(vbase + (size_t)kvrow * C3, kvrow < T, s, L.g);
    }

    f32x4 dk[G::MB], dv[G::MB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
        dk[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int qt0 = causal ? kt : 0;
    for (int qt = qt0; qt < nt; ++qt) {
        __syncthreads();
        stage_tile_bf16<HS, true, true>(Qs, Qt, qbase, C3, qt * kTile, T, L.tid);
        stage_tile_bf16<HS, true, true>(dOs, dOt, dobase, (size_t)C, qt * kTile, T, L.tid);
        if (L.tid < kTile) {
            const int q = qt * kTile + L.tid;
            Ls[L.tid] = (q < T) ? lrow[q] * kLog2e : INFINITY;
            Dl[L.tid] = (q < T) ? drow[q] : 0.f;
        }
        __syncthreads();
        const bool diag = causal && (qt == kt);

        // p[n][i], ds[n][i] for q = qt*64 + 16n + 4g + i, kv = kvrow
        f32x4 p[G::NB], ds[G::NB];
#pragma unroll
        for (int n = 0; n < G::NB; ++n) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* qr = Qs + (16 * n + L.r16) * G::LDR;
            const uint16_t* dr = dOs + (16 * n + L.r16) * G::LDR;
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st) {
                s = mfma_bf16(load_kchunk_lds<HS>(qr, st, L.g), kreg[st], s);
                dp = mfma_bf16(load_kchunk_lds<HS>(dr, st, L.g), vreg[st], dp);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ql = 16 * n + 4 * L.g + i;
                float pv = fast_exp2(s[i] * scale_log2 - Ls[ql]);
                if (diag && (qt * kTile + ql < kvrow)) pv = 0.f;
                p[n][i] = pv;
                ds[n][i] = pv * (dp[i] - Dl[ql]);
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS, 32 queries per step
#pragma unroll
        for (int t = 0; t < G::NB / 2; ++t) {
            const bf16x8 pb = pack_pair(p[2 * t], p[2 * t + 1]);
            const bf16x8 sb = pack_pair(ds[2 * t], ds[2 * t + 1]);
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb) {
                dv[mb] = mfma_bf16(load_trans_operand(dOt, 16 * mb + L.r16, t, L.g), pb, dv[mb]);
                dk[mb] = mfma_bf16(load_trans_operand(Qt, 16 * mb + L.r16, t, L.g), sb, dk[mb]);
            }
        }
    }

    if (kvrow < T) {
        uint16_t* dkrow = dqkv + ((size_t)b * T + kvrow) * C3 + C + (size_t)h * HS;
        uint16_t* dvrow = dkrow + C;
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) {
            store_bf16x4(dkrow + 16 * mb + 4 * L.g, dk[mb] * scale);
            store_bf16x4(dvrow + 16 * mb + 4 * L.g, dv[mb]);
        }
    }
}

// ----------------------------------------------------------- backward dQ
template <int HS>
__global__ __launch_bounds__(kThreads) void bwd_dq_bf16_kernel(
    uint16_t* __restrict__ dqkv, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Dws, int T, int C, int NH, int causal, float scale,
    float scale_log2) {
    using G = BfGeom<HS>;
    __shared__ uint16_t Ks[kTile * G::LDR];
    __shared__ uint16_t Kt[HS * kLDT];
    __shared__ uint16_t Vs[kTile * G::LDR];

    const Lane L;
    const int nt = (T + kTile - 1) / kTile;
    const int BH = gridDim.x / nt;
    int qt, bh;
    tile_of_block(BH, nt, causal != 0, qt, bh);
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const uint16_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint16_t* kbase = qbase + C;
    const uint16_t* vbase = qbase + 2 * (size_t)C;
    const uint16_t* dobase = dout + (size_t)b * T * C + (size_t)h * HS;

    const int qrow = qt * kTile + 16 * L.w + L.r16;
    const bool qvalid = qrow < T;
    bf16x8 qreg[G::KSTEPS], doreg[G::KSTEPS];
#pragma unroll
    for (int s = 0; s < G::KSTEPS; ++s) {
        qreg[s] = load_kchunk_global<HS>(qbase + (size_t)qrow * C3, qvalid, s, L.g);
        doreg[s] = load_kchunk_global<HS>(dobase + (size_t)qrow * C, qvalid, s, L.g);
    }
    const float l2 = qvalid ? lse[(size_t)bh * T + qrow] * kLog2e : INFINITY;
    const float Dq = qvalid ? Dws[(size_t)bh * T + qrow] : 0.f;

    f32x4 dq[G::MB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) dq[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = causal ? (qt + 1) : nt;
    for (int kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        stage_tile_bf16<HS, true, true>(Ks, Kt, kbase, C3, kt * kTile, T, L.tid);
        stage_tile_bf16<HS, true, false>(Vs, nullptr, vbase, C3, kt * kTile, T, L.tid);
        __syncthreads();
        const bool edge = (kt == nkt - 1);

        f32x4 ds[G::NB];
#pragma unroll
        for (int n = 0; n < G::NB; ++n) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* kr = Ks + (16 * n + L.r16) * G::LDR;
            const uint16_t* vr = Vs + (16 * n + L.r16) * G::LDR;
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st) {
                s = mfma_bf16(load_kchunk_lds<HS>(kr, st, L.g), qreg[st], s);
                dp = mfma_bf16(load_kchunk_lds<HS>(vr, st, L.g), doreg[st], dp);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float pv = fast_exp2(s[i] * scale_log2 - l2);
                if (edge) {
                    const int kv = kt * kTile + 16 * n + 4 * L.g + i;
                    if (kv >= T || (causal && kv > qrow)) pv = 0.f;
                }
                ds[n][i] = pv * (dp[i] - Dq);
            }
        }
        // dQ^T += K^T dS^T, 32 keys per step
#pragma unroll
        for (int t = 0; t < G::NB / 2; ++t) {
            const bf16x8 sb = pack_pair(ds[2 * t], ds[2 * t + 1]);
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb)
                dq[mb] = mfma_bf16(load_trans_operand(Kt, 16 * mb + L.r16, t, L.g), sb, dq[mb]);
        }
    }

    if (qvalid) {
        uint16_t* dqrow = dqkv + ((size_t)b * T + qrow) * C3 + (size_t)h * HS;
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) store_bf16x4(dqrow + 16 * mb + 4 * L.g, dq[mb] * scale);
    }
}

template <int HS>
hipError_t fwd_bf16_hs(uint16_t* out, float* lse, const uint16_t* qkv, const Shape& s,
                       hipStream_t st) {
    const int nqt = (s.T + kTile - 1) / kTile;
    const unsigned grid = (unsigned)(nqt * s.B * s.NH);
    const float scale_log2 = (float)(1.0 / sqrt((double)HS)) * kLog2e;
    hipLaunchKernelGGL(fwd_bf16_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, out, lse, qkv, s.T,
                       s.C, s.NH, s.causal, scale_log2);
    return hipGetLastError();
}

template <int HS>
hipError_t prepass_bf16_hs(float* D, const uint16_t* dout, const uint16_t* out, const Shape& s,
                           hipStream_t st) {
    const long long rows = (long long)s.B * s.T * s.NH;
    const long long threads = rows * (HS / 8);
    const unsigned grid = (unsigned)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(prepass_bf16_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, D, dout, out,
                       s.T, s.NH, rows);
    return hipGetLastError();
}

template <int HS>
hipError_t dkdv_bf16_hs(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                        const float* lse, const float* D, const Shape& s, hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    const unsigned grid = (unsigned)(nt * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    hipLaunchKernelGGL(bwd_dkdv_bf16_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, dqkv, dout,
                       qkv, lse, D, s.T, s.C, s.NH, s.causal, scale, scale * kLog2e);
    return hipGetLastError();
}

template <int HS>
hipError_t dq_bf16_hs(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv, const float* lse,
                      const float* D, const Shape& s, hipStream_t st) {
    const int nt = (s.T + kTile - 1) / kTile;
    const unsigned grid = (unsigned)(nt * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    hipLaunchKernelGGL(bwd_dq_bf16_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, dqkv, dout, qkv,
                       lse, D, s.T, s.C, s.NH, s.causal, scale, scale * kLog2e);
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

hipError_t launch_fwd_bf16(uint16_t* out, float* lse, const uint16_t* qkv, const Shape& s,
                           hipStream_t st) {
    ATTN_DISPATCH_HS(fwd_bf16_hs, out, lse, qkv, s, st)
}

hipError_t launch_prepass_bf16(float* D, const uint16_t* dout, const uint16_t* out,
                               const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(prepass_bf16_hs, D, dout, out, s, st)
}

hipError_t launch_dkdv_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                            const float* lse, const float* D, const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(dkdv_bf16_hs, dqkv, dout, qkv, lse, D, s, st)
}

hipError_t launch_dq_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                          const float* lse, const float* D, const Shape& s, hipStream_t st) {
    ATTN_DISPATCH_HS(dq_bf16_hs, dqkv, dout, qkv, lse, D, s, st)
}

#undef ATTN_DISPATCH_HS

}  // namespace attn
