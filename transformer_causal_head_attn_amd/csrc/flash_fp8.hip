// flash_fp8.hip -- fused attention forward with 8-bit floating-point q, k, v
// (OCP FP8 E4M3: 4 exponent bits, 3 mantissa bits, largest finite value 448)
// and fp32 accumulation, for gfx950 (v_mfma_f32_16x16x32_fp8_fp8).
//
// Same method as the 16-bit forward (flash_half.hip): the self-attention of
// "Umakini wa kujitegemea, kerneli za CUDA na FlashAttention" (section 1)
// computed tile by tile with a running softmax, keeping the per-row
// log-sum-exp.  The operand precision follows the mixed-precision part of
// "LLM Systems 10 & 11: Accelerating Transformer Training and Inference"
// (section 1), which names FP8 for the forward: Q, K and V enter the matrix
// cores as E4M3, every product accumulates in fp32, the softmax runs in
// fp32, and P is rounded to E4M3 (round to nearest even) only to enter the
// P V product.  With the lazy rescale P stays at most 2^8 (E4M3 holds 448);
// probabilities below 2^-10 of the running maximum round to zero.  The row
// sums are formed on the matrix cores from the same rounded P, so the
// normalisation and the weighted sum see the same weights.  out is bfloat16
// (round to nearest even), lse fp32.
//
// gfx950 mapping (the operand layout of the fp8 matrix-core op was probed on
// the GPU: as for the 16-bit op, lane l supplies row l % 16 of A and column
// l % 16 of B at k = 8 (l / 16) .. + 7, one byte each, and holds D[4 (l / 16)
// + r][l % 16] in its result register r):
//  * S^T = K Q^T: a K operand is 8 consecutive bytes of one key row, read
//    from a row-major LDS tile (ds_read_b64); Q stays in registers.
//  * O^T = V^T P^T: P comes straight from the score accumulators (lane
//    group g holds keys 16n + 4g + i, blocks n = 2t, 2t + 1 per 32-key step)
//    and the matching V operand is one ds_read_b64_tr_b8 transposed read of
//    a row-major V tile whose 16-byte groups are swizzled per row.
//  * Every wave owns 32 query rows (two 16-row blocks), four waves a
//    128-row Q tile; keys stream through LDS 64 at a time, the next tile
//    loaded into registers while the current one is used.
#include "common.hpp"



namespace attn {
namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kStream = 64;     // keys per step
constexpr int kQB = 2;          // 16-row blocks per wave
constexpr int kRows = 64 * kQB; // rows per Q tile
constexpr float kLazyMax = 8.0f;

typedef long fp8x8;   // eight E4M3 values, one matrix-core operand

__device__ __forceinline__ f32x4 mfma8(fp8x8 a, fp8x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

template <int HS>
struct Geom8 {
    static constexpr int LDK = HS + 8;         // K tile row stride (bytes): 16 rows -> 16 bank pairs
    static constexpr int LDV = HS;             // V tile row stride (bytes): dense, swizzled
    // V rows: 16-byte group q of row r is stored at group q ^ fv(r); the
    // eight rows one transposed read touches (4g + 0..3 and 16 + 4g + 0..3
    // of a 32-key step) then fall on eight different bank groups (hs = 16
    // has one group per row and keeps a two-way conflict)
    static __device__ __forceinline__ int fv(int r) {
        if constexpr (HS >= 128) return (r & 3) | (((r >> 4) & 1) << 2);
        else if constexpr (HS == 64) return ((r >> 1) & 1) | (((r >> 4) & 1) << 1);
        else if constexpr (HS == 32) return (r >> 4) & 1;
        else return 0;
    }
    static constexpr int KSTEPS = HS >= 32 ? HS / 32 : 1;
    static constexpr int MB = HS / 16;
    static constexpr int CH = HS / 16;         // 16-byte chunks per global row
};

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Buffer descriptor over rows row0 .. min(row0 + kStream, T) - 1 of one head's
// slice (rows ld_bytes apart, row_bytes used per row): loads at or past the
// record limit return zeros, so rows >= T need no predicate.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc8(const uint8_t* base, uint32_t ld_bytes,
                                                             int row0, int T, uint32_t row_bytes) {
    const int valid = min(T - row0, kStream);
    const uint32_t num = valid > 0 ? (uint32_t)(valid - 1) * ld_bytes + row_bytes : 0u;
    const uint8_t* p = base + (size_t)row0 * ld_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)num, 0x00020000);
}

// A kStream x HS byte tile in registers between its global load and its LDS
// store: 16-byte chunks, chunk e = tid + k * kThreads is row e / CH, bytes
// 16 (e % CH) .. + 15.
template <int HS>
struct Tile8 {
    using G = Geom8<HS>;
    static constexpr int TOTAL = kStream * G::CH;
    static constexpr int N = (TOTAL + kThreads - 1) / kThreads;
    static constexpr bool FULL = TOTAL % kThreads == 0;
    uint4 v[N];
    __device__ __forceinline__ void fetch(const uint8_t* base, uint32_t ld_bytes, int row0, int T,
                                          int tid) {
        const __amdgpu_buffer_rsrc_t r = rows_rsrc8(base, ld_bytes, row0, T, HS);
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = tid + k * kThreads;
            const int row = e / G::CH, c = e - row * G::CH;
            v[k] = make_uint4(0u, 0u, 0u, 0u);
            if (FULL || e < TOTAL) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)((uint32_t)row * ld_bytes + 16u * (uint32_t)c), 0, 0);
                __builtin_memcpy(&v[k], &x, 16);
            }
        }
    }
    // row-major K tile (stride LDK; two 8-byte stores per chunk, LDK being
    // a multiple of 8 but not of 16)
    __device__ __forceinline__ void store_rows(uint8_t* lds, int tid) const {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = tid + k * kThreads;
            const int row = e / G::CH, c = e - row * G::CH;
            if (FULL || e < TOTAL) {
                uint64_t* p = reinterpret_cast<uint64_t*>(lds + row * G::LDK + 16 * c);
                p[0] = (uint64_t)v[k].x | ((uint64_t)v[k].y << 32);
                p[1] = (uint64_t)v[k].z | ((uint64_t)v[k].w << 32);
            }
        }
    }
    // swizzled row-major V tile (one 16-byte store per chunk)
    __device__ __forceinline__ void store_swizzled(uint8_t* lds, int tid) const {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = tid + k * kThreads;
            const int row = e / G::CH, c = e - row * G::CH;
            if (FULL || e < TOTAL)
                *reinterpret_cast<uint4*>(lds + row * G::LDV + 16 * (c ^ G::fv(row))) = v[k];
        }
    }
};

// E4M3 bytes of (x0..x3, y0..y3), rounded to nearest even: one matrix-core
// operand in the score accumulators' key order.
__device__ __forceinline__ fp8x8 pack8(const f32x4& x, const f32x4& y) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], hi, true);
    return (fp8x8)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));

// The V^T operand of step t (keys 32t .. 32t + 31), head dimensions 16mb ..
// 16mb + 15, from the swizzled row-major V tile with one transposed read.
// ds_read_b64_tr_b8 (lane layout probed on the GPU): within each 16-lane
// group, lane j receives byte j % 8 of the 8-byte blocks addressed by lanes
// 2e + j / 8 (e = 0..3) and 8 + 2(e - 4) + j / 8 (e = 4..7).  So lane L of
// the group addresses key row key(L / 2) at bytes 16mb + 8(L % 2) .. + 7,
// and lane j ends with V[key(e)][16mb + j] in byte e, where key(e) is the
// score accumulators' key order: 32t + 4g + e for e < 4, 32t + 16 + 4g +
// e - 4 for e >= 4 (g = lane / 16).
template <int HS>
__device__ __forceinline__ fp8x8 v_operand(const uint8_t* Vs, int t, int mb) {
    using G = Geom8<HS>;
    const int lane = threadIdx.x & 63;
    const int L = lane & 15, g = lane >> 4;
    const int e = L >> 1;
    const int row = 32 * t + 4 * g + (e & 3) + 16 * (e >> 2);
    const uint8_t* p = Vs + row * G::LDV + 16 * (mb ^ G::fv(row)) + 8 * (L & 1);
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
    uint64_t u;
    __builtin_memcpy(&u, &r, 8);
    return (fp8x8)u;
}

// fp32 -> bfloat16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Workgroup: a 128-row Q tile of one head (32 rows per wave); keys stream
// through LDS 64 at a time (one K and one V^T buffer; the next tile's
// registers are loaded while the current tile is used).
template <int HS>
__device__ __forceinline__ void fwd_fp8_tile(int qt, int bh, uint16_t* __restrict__ out,
                                             float* __restrict__ lse,
                                             const uint8_t* __restrict__ qkv, int T, int C, int NH,
                                             int causal, float scale_log2, int w, int l) {
    using G = Geom8<HS>;
    constexpr int R = 16 * kQB;
    __shared__ __attribute__((aligned(16))) uint8_t Ks[kStream * G::LDK];
    __shared__ __attribute__((aligned(16))) uint8_t Vs[kStream * G::LDV];

    const int tid = threadIdx.x;
    const int r16 = l & 15, g = l >> 4;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const uint32_t C3 = 3u * (uint32_t)C;   // row stride in bytes
    const uint8_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint8_t* kbase = qbase + C;
    const uint8_t* vbase = qbase + 2 * (size_t)C;

    const int r0 = qt * kRows + w * R;   // this wave's first query row
    fp8x8 qreg[kQB][G::KSTEPS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int q = r0 + 16 * qb + r16;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            const int k0 = 32 * s + 8 * g;
            qreg[qb][s] = (q < T && k0 < HS)
                              ? *reinterpret_cast<const fp8x8*>(qbase + (size_t)q * C3 + k0)
                              : (fp8x8)0;
        }
    }

    float m[kQB];
    f32x4 o[kQB][G::MB], lsum[kQB];
    const fp8x8 ones = (fp8x8)0x3838383838383838ull;   // eight E4M3 1.0
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        m[qb] = -INFINITY;
        lsum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) o[qb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nkt_all = (T + kStream - 1) / kStream;
    const int nkt = causal ? min(nkt_all, (qt * kRows + kRows - 1) / kStream + 1) : nkt_all;
    int last = causal ? min(nkt - 1, (r0 + R - 1) / kStream) : nkt - 1;
    if (r0 >= T) last = -1;

    Tile8<HS> rk, rv;
    rk.fetch(kbase, C3, 0, T, tid);
    rv.fetch(vbase, C3, 0, T, tid);
    wait_global_loads();
    for (int j = 0; j < nkt; ++j) {
        __syncthreads();
        rk.store_rows(Ks, tid);
        rv.store_swizzled(Vs, tid);
        __syncthreads();
        if (j + 1 < nkt) {
            rk.fetch(kbase, C3, (j + 1) * kStream, T, tid);
            rv.fetch(vbase, C3, (j + 1) * kStream, T, tid);
        }
        if (j > last) continue;

        // S^T = K Q^T: sc[qb][n][i] is the score of key 16n + 4g + i with
        // query r0 + 16qb + r16
        f32x4 sc[kQB][4];
        // hs = 128: the score products run at raised issue priority, as in
        // the 16-bit forward (long-context forward 222 -> 208 us; at hs = 64
        // 3% slower, so only there)
        if constexpr (HS >= 128) __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int np = 0; np < 4; np += 2) {
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st) {
#pragma unroll
                for (int n = np; n < np + 2; ++n) {
                    const int k0 = 32 * st + 8 * g;
                    const fp8x8 kc = k0 < HS ? *reinterpret_cast<const fp8x8*>(
                                                   Ks + (16 * n + r16) * G::LDK + k0)
                                             : (fp8x8)0;
#pragma unroll
                    for (int qb = 0; qb < kQB; ++qb)
                        sc[qb][n] = mfma8(kc, qreg[qb][st],
                                          st == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[qb][n]);
                }
            }
        }

        if constexpr (HS >= 128) __builtin_amdgcn_s_setprio(0);
        const int k0 = j * kStream;
        const bool edge = (k0 + kStream > T) || (causal && k0 + kStream - 1 > r0);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int row = r0 + 16 * qb + r16;
            if (edge) {   // key k0 + 16n + 4g + i stays iff 16n + i < d
                const int lim = causal ? min(T, row + 1) : T;
                const int d = lim - (k0 + 4 * g);
#pragma unroll
                for (int n = 0; n < 4; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[qb][n][i] = (16 * n + i < d) ? sc[qb][n][i] : -INFINITY;
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sc[qb][n][i]);
            mloc = group4_max(mloc) * scale_log2;
            // raise the running maximum only by more than kLazyMax (log2
            // domain), so P <= 2^8 stays inside E4M3's range; each row
            // decides for itself
            const bool need = mloc > m[qb] + kLazyMax;
            if (wave_any(need)) {
                const float alpha = need ? fast_exp2(m[qb] - mloc) : 1.0f;
                m[qb] = need ? mloc : m[qb];
                lsum[qb] *= alpha;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) o[qb][mb] *= alpha;
            }
            const float nm = -m[qb];
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[qb][n][i] = fast_exp2(fmaf(sc[qb][n][i], scale_log2, nm));
        }

        // O^T += V^T P^T and the row sums onesT P^T, 32 keys per step
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            fp8x8 pb[kQB];
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                pb[qb] = pack8(sc[qb][2 * t], sc[qb][2 * t + 1]);
                lsum[qb] = mfma8(ones, pb[qb], lsum[qb]);
            }
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb) {
                const fp8x8 vop = v_operand<HS>(Vs, t, mb);
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) o[qb][mb] = mfma8(vop, pb[qb], o[qb][mb]);
            }
        }
    }

#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int row = r0 + 16 * qb + r16;
        if (row < T) {
            const float ltot = lsum[qb][0];
            const float inv = 1.0f / ltot;
            uint16_t* orow = out + ((size_t)b * T + row) * C + (size_t)h * HS;
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb) {
                const f32x4 v = o[qb][mb] * inv;
                const uint2 pk = make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                            bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
                *reinterpret_cast<uint2*>(orow + 16 * mb + 4 * g) = pk;
            }
            if (g == 0) lse[(size_t)bh * T + row] = (m[qb] + __log2f(ltot)) * kLn2;
        }
    }
}

// A head's row slice is hs bytes, less than a 128-byte memory line for
// hs < 128, so 128 / hs neighbouring heads share every line of q, k and v.
// Workgroups are dispatched to the 8 XCDs (8 L2 caches) round robin by id,
// and consecutive ids walk the heads; this remaps the head of id slot c so
// that the G = 128 / hs heads of a line run on one XCD: within each block of
// 8G slots, slot 8s + x (XCD x) takes head G x + s.  Without it every XCD
// fetches whole lines for its part of them (measured: the GPT-2 layer
// forward read 2.0x its compulsory bytes, ViT 3.3x; grouped 1.0x and 1.7x,
// and the ViT forward 43.5 -> 34.8 us).  Identity when BH is not a multiple
// of 8G.
template <int HS>
__device__ __forceinline__ int xcd_group_heads(int bh, int BH) {
    constexpr int G = HS < 128 ? 128 / HS : 1;
    if (G == 1 || BH % (8 * G) != 0) return bh;
    const int blk = bh / (8 * G), c = bh - blk * 8 * G;
    return blk * 8 * G + (c & 7) * G + (c >> 3);
}

template <int HS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(HS >= 128 ? 2 : 3))) void fwd_fp8_kernel(
    uint16_t* __restrict__ out, float* __restrict__ lse, const uint8_t* __restrict__ qkv, int T,
    int C, int NH, int causal, float scale_log2, Deal deal) {
    const int nt = (T + kRows - 1) / kRows;
    int bh, t;
    deal_tile(gridDim.x / nt, nt, causal != 0, deal, bh, t);
    bh = xcd_group_heads<HS>(bh, gridDim.x / nt);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    fwd_fp8_tile<HS>(t, bh, out, lse, qkv, T, C, NH, causal, scale_log2, w, threadIdx.x & 63);
}

template <int HS>
hipError_t fwd_fp8_hs(uint16_t* out, float* lse, const uint8_t* qkv, const Shape& s, hipStream_t st) {
    const int nqt = (s.T + kRows - 1) / kRows;
    const unsigned grid = (unsigned)((long long)nqt * s.B * s.NH);
    const float scale_log2 = (float)(1.0 / sqrt((double)HS)) * kLog2e;
    hipLaunchKernelGGL(fwd_fp8_kernel<HS>, dim3(grid), dim3(kThreads), 0, st, out, lse, qkv, s.T,
                       s.C, s.NH, s.causal, scale_log2, deal_for<fwd_fp8_kernel<HS>>(kThreads));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(uint16_t* out, float* lse, const uint8_t* qkv, const Shape& s,
                          hipStream_t st) {
    switch (s.hs) {
        case 16: return fwd_fp8_hs<16>(out, lse, qkv, s, st);
        case 32: return fwd_fp8_hs<32>(out, lse, qkv, s, st);
        case 64: return fwd_fp8_hs<64>(out, lse, qkv, s, st);
        case 128: return fwd_fp8_hs<128>(out, lse, qkv, s, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
