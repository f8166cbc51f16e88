// flash_half.hip -- fused attention forward and backward with 16-bit
// tensors (bfloat16 or IEEE half) and fp32 accumulation for gfx950
// (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x32_f16).
//
// Same method as the fp32 kernels (flash_f32.hip): the self-attention of
// "Umakini wa kujitegemea, kerneli za CUDA na FlashAttention" (section 1)
// computed tile by tile with a running softmax, keeping only the per-row
// log-sum-exp, and the analytic backward of attention_backward_cpu in llm.c
// dev/cuda/attention_backward.cu with the closed-form softmax gradient of
// its kernel 7.  Low-precision operands with higher-precision accumulation
// follow the mixed-precision part of "LLM Systems 10 & 11: Accelerating
// Transformer Training and Inference" (section 1), which names both bf16 and
// fp16: Q, K, V, dO are 16-bit, every product accumulates in fp32, the
// softmax runs in fp32, and P and dS are rounded to the 16-bit type only to
// enter the matrix cores.  lse and D stay fp32.  The two element types share
// every kernel (the element traits BF16 and F16 below); only the matrix-core
// instruction and the conversions differ.  In fp16 the forward's P stays
// below 2^8 (lazy rescale) and the backward's P below 1, far inside its
// range; dS, out and the gradients must stay below 65504 in magnitude.
//
// gfx950 mapping.
//  * One 16-bit MFMA contracts 32 k-values; lane group g = l/16 supplies eight.
//    For Q.K and dO.V (contraction over hs) a lane takes k = 32s + 8g .. +7,
//    one 16-byte LDS read of a row-major tile.
//  * For the products that contract over keys or queries (P V, dO^T P,
//    Q^T dS, K^T dS^T) the operand that comes out of the score accumulators
//    holds, in lane group g, the rows 16n + 4g + i; a 32-wide step t pairs
//    score blocks n = 2t, 2t+1.  The matching operand (eight rows of one
//    column of a row-major tile) comes from two ds_read_b64_tr_b16
//    transpose reads, so no transposed copy of any tile is kept.
//  * Every wave owns 32 rows (two 16-row blocks) of the tile it keeps in
//    registers, so each operand read from LDS feeds two matrix-core ops;
//    with 16 rows per wave the kernels would need more LDS bandwidth than
//    a CU has.
//  * The next streamed tile is loaded into registers while the current one
//    is used (one LDS buffer, two barriers per step).
//  * Forward: a row's running maximum is only raised (and its O, l
//    rescaled) when the row's tile maximum exceeds it by more than 8 in the
//    log2 domain (probabilities stay below 2^8); otherwise the stale maximum
//    is kept, which changes no result (numerator and denominator share it),
//    and the wave skips the rescale when none of its rows needs one.
#include "common.hpp"

namespace attn {
namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kStream = 64;     // rows of the streamed tile per step
constexpr float kLazyMax = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

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

// Element types of the 16-bit path.  Both fill the same 8-entry matrix-core
// operand layout, accumulate in fp32 and round to nearest even when fp32
// values are converted back (P, dS and the outputs).
struct BF16 {   // bfloat16: v_mfma_f32_16x16x32_bf16
    typedef __bf16 S;
    typedef __bf16 V8 __attribute__((ext_vector_type(8)));
    typedef __bf16 V4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ f32x4 mfma(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float bits_to_f32(uint32_t u) {   // low 16 bits
        return __uint_as_float(u << 16);
    }
    static __device__ __forceinline__ V8 ones() {   // eight 1.0 (0x3F80)
        const uint4 u = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
        V8 r;
        __builtin_memcpy(&r, &u, 16);
        return r;
    }
};
struct F16 {   // IEEE half: v_mfma_f32_16x16x32_f16
    typedef _Float16 S;
    typedef _Float16 V8 __attribute__((ext_vector_type(8)));
    typedef _Float16 V4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ f32x4 mfma(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float bits_to_f32(uint32_t u) {
        const uint16_t h = (uint16_t)u;
        _Float16 x;
        __builtin_memcpy(&x, &h, 2);
        return (float)x;
    }
    static __device__ __forceinline__ V8 ones() {   // eight 1.0 (0x3C00)
        const uint4 u = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
        V8 r;
        __builtin_memcpy(&r, &u, 16);
        return r;
    }
};
template <typename E>
using V8 = typename E::V8;

template <int HS>
struct Geom {
    // LDS row stride (elements; a multiple of 8 keeps 16-byte rows aligned).
    // +16 for hs >= 64 measured faster than +8 (dK/dV at hs = 128: -9%).
    static constexpr int LDR = HS >= 64 ? HS + 16 : HS + 8;
    static constexpr int KSTEPS = HS >= 32 ? HS / 32 : 1;
    static constexpr int MB = HS / 16;
};

template <typename E>
__device__ __forceinline__ V8<E> as_v8(uint4 v) {
    V8<E> r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

template <typename E>
__device__ __forceinline__ V8<E> zero_v8() { return as_v8<E>(make_uint4(0u, 0u, 0u, 0u)); }

// Eight bf16 of one row for contraction step s: k = 32s + 8g .. +7; zeros
// where that range lies beyond HS (only when HS = 16).
template <typename E, int HS>
__device__ __forceinline__ V8<E> row_chunk_global(const uint16_t* rowp, bool valid, int s, int g) {
    const int k0 = 32 * s + 8 * g;
    if (!valid || k0 >= HS) return zero_v8<E>();
    return as_v8<E>(*reinterpret_cast<const uint4*>(rowp + k0));
}

template <typename E, int HS>
__device__ __forceinline__ V8<E> row_chunk_lds(const uint16_t* tile, int row, int s, int g) {
    const int k0 = 32 * s + 8 * g;
    if (k0 >= HS) return zero_v8<E>();
    return as_v8<E>(*reinterpret_cast<const uint4*>(tile + row * Geom<HS>::LDR + k0));
}

__device__ __forceinline__ s16x4 tr_read(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
}

// Column operand from a row-major LDS tile: lane (j = l%16, g) receives
// tile[base + 4g + e][col0 + j] for e < 4 and tile[base + 16 + 4g + e - 4]
// [col0 + j] for e >= 4.  Within a 16-lane group, ds_read_b64_tr_b16 hands
// lane j element (j % 4) of the 8-byte blocks addressed by lanes 4e + j/4, so
// lane i addresses row (.. + i/4), columns col0 + 4(i%4) .. +3.
template <typename E, int HS>
__device__ __forceinline__ V8<E> col_operand(const uint16_t* tile, int base, int col0, int lane) {
    const int j = lane & 15, g = lane >> 4;
    const uint16_t* p = tile + (base + 4 * g + (j >> 2)) * Geom<HS>::LDR + col0 + 4 * (j & 3);
    const s16x4 a = tr_read(p);
    const s16x4 b = tr_read(p + 16 * Geom<HS>::LDR);
    V8<E> r;
    __builtin_memcpy(&r, &a, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
    return r;
}

// Pack score-layout values of blocks n = 2t (x) and 2t+1 (y) into the
// matching 8-entry bf16 operand.
template <typename E>
__device__ __forceinline__ V8<E> pack_pair(const f32x4& x, const f32x4& y) {
    V8<E> r;
    r[0] = (typename E::S)x[0];
    r[1] = (typename E::S)x[1];
    r[2] = (typename E::S)x[2];
    r[3] = (typename E::S)x[3];
    r[4] = (typename E::S)y[0];
    r[5] = (typename E::S)y[1];
    r[6] = (typename E::S)y[2];
    r[7] = (typename E::S)y[3];
    return r;
}

template <typename E>
__device__ __forceinline__ void store4(uint16_t* p, const f32x4& v) {
    typename E::V4 r;
    r[0] = (typename E::S)v[0];
    r[1] = (typename E::S)v[1];
    r[2] = (typename E::S)v[2];
    r[3] = (typename E::S)v[3];
    __builtin_memcpy(p, &r, 8);
}

// Buffer descriptor over rows row0 .. min(row0 + kStream, T) - 1 of one head's
// slice (rows ld_bytes apart, row_bytes used per row).  A raw buffer load
// whose offset lies at or past num_records returns zeros instead of reading
// memory, so the 16-byte loads of rows >= T need no predicate and read
// nothing past the tensor; every chunk is either wholly inside (rows < T) or
// wholly outside (rows >= T, offsets >= (T - row0) * ld_bytes), because
// ld_bytes >= row_bytes.  Word 3 is the gfx9 raw-buffer format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, uint32_t ld_bytes,
                                                            int row0, int T, uint32_t row_bytes) {
    const int valid = min(T - row0, kStream);
    const uint32_t num = valid > 0 ? (uint32_t)(valid - 1) * ld_bytes + row_bytes : 0u;
    const char* p = reinterpret_cast<const char*>(base) + (size_t)row0 * ld_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, (int)num, 0x00020000);
}

// A kStream x HS 16-bit tile held in registers between its global load and
// its LDS store (row-major, stride LDR); rows >= T are zero.
template <int HS, int NT = kThreads>
struct TileRegs {
    static constexpr int CH = HS / 8;                        // 16-byte chunks per row
    static constexpr int TOTAL = kStream * CH;
    static constexpr int N = (TOTAL + NT - 1) / NT;
    static constexpr bool FULL = TOTAL % NT == 0;            // every thread holds N chunks
    uint4 v[N];
    __device__ __forceinline__ void fetch(const uint16_t* base, size_t ld, int row0, int T, int tid) {
        const uint32_t ldb = (uint32_t)(ld * 2);
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(base, ldb, row0, T, HS * 2);
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = tid + k * NT;
            const int row = e / CH, c = e - (e / CH) * CH;
            const uint32_t off = (uint32_t)row * ldb + 16u * (uint32_t)c;
            v[k] = make_uint4(0u, 0u, 0u, 0u);
            if (FULL || e < TOTAL) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
                __builtin_memcpy(&v[k], &x, 16);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = tid + k * NT;
            const int row = e / CH, c = e - (e / CH) * CH;
            if (FULL || e < TOTAL) *reinterpret_cast<uint4*>(lds + row * Geom<HS>::LDR + 8 * c) = v[k];
        }
    }
};

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// ------------------------------------------------------------------ forward
// Key range of one forward workgroup and, for a split of the keys over
// workgroups, where its partial result goes.
struct KeyPart {
    int kt_lo, kt_hi;      // 64-key tiles [kt_lo, kt_hi) (kt_hi clipped to what the tile sees)
    float* o;              // PART: output normalised over the range, fp32 (B, T, C) slab
    float* l;              // PART: log-sum-exp over the range, (B, NH, T) slab
};

// Workgroup: a 4*R-row Q tile of one head (R = 16*QB rows per wave); keys
// stream through LDS 64 at a time (one buffer; the next tile's registers
// are loaded while the current tile is used).
template <typename E, int HS, int QB, bool PART, int NW = 4>
__device__ __forceinline__ void fwd_half_tile(int tile_, int bh_, uint16_t* __restrict__ out,
                                              float* __restrict__ lse,
                                              const uint16_t* __restrict__ qkv, int T, int C,
                                              int NH, int causal, float scale_log2,
                                              KeyPart part) {
    using G = Geom<HS>;
    constexpr int R = 16 * QB;
    constexpr int BM = NW * R;
    __shared__ uint16_t Ks[kStream * G::LDR];
    __shared__ uint16_t Vs[kStream * G::LDR];

    const Lane L;
    const int qt = tile_, bh = bh_;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const uint16_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint16_t* kbase = qbase + C;
    const uint16_t* vbase = qbase + 2 * (size_t)C;

    const int r0 = qt * BM + L.w * R;   // this wave's first query row
    V8<E> qreg[QB][G::KSTEPS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = r0 + 16 * qb + L.r16;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s)
            qreg[qb][s] = row_chunk_global<E, HS>(qbase + (size_t)q * C3, q < T, s, L.g);
    }

    // lsum[qb]: the row sums of the 16-bit P that enter P V, formed on the
    // matrix cores as ones^T P^T (every entry of the block holds the sum of
    // the lane's query row), so the softmax spends no VALU add on them
    float m[QB];
    f32x4 o[QB][G::MB], lsum[QB];
    const V8<E> ones = E::ones();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        lsum[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) o[qb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nkt_all = (T + kStream - 1) / kStream;
    const int nkt_tile = causal ? min(nkt_all, (qt * BM + BM - 1) / kStream + 1) : nkt_all;
    const int kt_lo = PART ? part.kt_lo : 0;
    const int nkt = PART ? min(part.kt_hi, nkt_tile) : nkt_tile;
    // last key tile with a key <= some row of this wave; none when the
    // wave has no row below T (its stores are skipped anyway)
    int last = causal ? min(nkt - 1, (r0 + R - 1) / kStream) : nkt - 1;
    if (r0 >= T) last = -1;

    auto scores = [&](const uint16_t* kt_lds, f32x4 (&sc)[QB][4]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int n = 0; n < 4; ++n) sc[qb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        // two 16-key blocks at a time, contraction step outside them:
        // consecutive matrix-core ops update different accumulators (a
        // dependent op waits ~50 cycles, 3x the issue interval)
#pragma unroll
        for (int np = 0; np < 4; np += 2) {
#pragma unroll
            for (int st = 0; st < G::KSTEPS; ++st) {
#pragma unroll
                for (int n = np; n < np + 2; ++n) {
                    const V8<E> kc = row_chunk_lds<E, HS>(kt_lds, 16 * n + L.r16, st, L.g);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) sc[qb][n] = E::mfma(kc, qreg[qb][st], sc[qb][n]);
                }
            }
        }
    };

    // softmax of tile j in place (scores -> probabilities), then O += P V
    auto consume = [&](int j, f32x4 (&sc)[QB][4], const uint16_t* vt_lds) {
        const int k0 = j * kStream;
        const bool edge = (k0 + kStream > T) || (causal && k0 + kStream - 1 > r0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = r0 + 16 * qb + L.r16;
            if (edge) {   // keys >= lim are masked: key k0 + 4g + 16n + i stays iff 16n + i < d
                const int lim = causal ? min(T, row + 1) : T;
                const int d = lim - (k0 + 4 * L.g);
#pragma unroll
                for (int n = 0; n < 4; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sc[qb][n][i] = (16 * n + i < d) ? sc[qb][n][i] : -INFINITY;
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sc[qb][n][i]);
            mloc = group4_max(mloc) * scale_log2;
            // Each row decides for itself (so a row's result depends on its
            // own scores only); the wave skips the rescale when no row needs it.
            const bool need = mloc > m[qb] + kLazyMax;
            if (wave_any(need)) {
                const float alpha = need ? fast_exp2(m[qb] - mloc) : 1.0f;   // m = -inf -> 0
                m[qb] = need ? mloc : m[qb];
                lsum[qb] *= alpha;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) o[qb][mb] *= alpha;
            }
            const float nm = -m[qb];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sc[qb][n][i] = fast_exp2(fmaf(sc[qb][n][i], scale_log2, nm));
                }
            }
        }
        // O^T += V^T P^T, 32 keys per step
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            V8<E> pb[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                pb[qb] = pack_pair<E>(sc[qb][2 * t], sc[qb][2 * t + 1]);
                lsum[qb] = E::mfma(ones, pb[qb], lsum[qb]);
            }
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb) {
                const V8<E> vop = col_operand<E, HS>(vt_lds, 32 * t, 16 * mb, L.l);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[qb][mb] = E::mfma(vop, pb[qb], o[qb][mb]);
            }
        }
    };

    TileRegs<HS, 64 * NW> rk, rv;
    {
        f32x4 sc[QB][4];
        rk.fetch(kbase, C3, kt_lo * kStream, T, L.tid);
        rv.fetch(vbase, C3, kt_lo * kStream, T, L.tid);
        wait_global_loads();
        for (int j = kt_lo; j < nkt; ++j) {
            __syncthreads();
            rk.store(Ks, L.tid);
            rv.store(Vs, L.tid);
            __syncthreads();
            if (j + 1 < nkt) {
                rk.fetch(kbase, C3, (j + 1) * kStream, T, L.tid);
                rv.fetch(vbase, C3, (j + 1) * kStream, T, L.tid);
            }
            if (j > last) continue;
            // hs = 128: the score products run at raised issue priority, so a
            // wave entering them is not held behind the softmax of the other
            // waves on its SIMD (long-context forward -7%; at hs = 64 +4%, so
            // only there)
            if constexpr (HS >= 128) __builtin_amdgcn_s_setprio(2);
            scores(Ks, sc);
            if constexpr (HS >= 128) __builtin_amdgcn_s_setprio(0);
            consume(j, sc, Vs);
        }
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = r0 + 16 * qb + L.r16;
        const float ltot = lsum[qb][0];
        if (row < T) {
            if constexpr (PART) {
                // a row with no key in the range (its keys all lie past it):
                // out 0, lse -inf, which the merge weighs by exp(-inf) = 0
                const bool any = ltot > 0.f;
                const float inv = any ? 1.0f / ltot : 0.f;
                float* orow = part.o + ((size_t)b * T + row) * C + (size_t)h * HS;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) {
                    const f32x4 v = o[qb][mb] * inv;
                    *reinterpret_cast<float4*>(orow + 16 * mb + 4 * L.g) = make_float4(v[0], v[1], v[2], v[3]);
                }
                if (L.g == 0)
                    part.l[(size_t)bh * T + row] = any ? (m[qb] + __log2f(ltot)) * kLn2 : -INFINITY;
            } else {
                const float inv = 1.0f / ltot;
                uint16_t* orow = out + ((size_t)b * T + row) * C + (size_t)h * HS;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) store4<E>(orow + 16 * mb + 4 * L.g, o[qb][mb] * inv);
                if (L.g == 0) lse[(size_t)bh * T + row] = (m[qb] + __log2f(ltot)) * kLn2;
            }
        }
    }
}

// ------------------------------------------------------ backward pre-pass
template <typename E, int HS>
__global__ __launch_bounds__(kThreads) void prepass_half_kernel(float* __restrict__ D,
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
            acc += E::bits_to_f32(av[q]) * E::bits_to_f32(cv[q]);
            acc += E::bits_to_f32(av[q] >> 16) * E::bits_to_f32(cv[q] >> 16);
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
// Workgroup: a 4*R-row K/V tile of one head (R = 16*KB rows per wave, kept
// in registers); Q and dO stream through LDS 64 rows at a time.
// PART: the workgroup takes the query tiles [part.kt_lo, part.kt_hi) only
// (64-row tiles) and writes its fp32 dk (scaled) and dv sums to the partial
// slab part.o, rows of 2C: [dk | dv] (a later kernel adds the slabs).
template <typename E, int HS, int KB, bool PART, int NW = 4>
__device__ __forceinline__ void bwd_dkdv_half_tile(
    int tile_, int bh_, uint16_t* __restrict__ dqkv, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Dws, int T, int C, int NH, int causal, float scale,
    float scale_log2, KeyPart part) {
    using G = Geom<HS>;
    constexpr int R = 16 * KB;
    constexpr int BN = NW * R;
    __shared__ uint16_t Qs[kStream * G::LDR];
    __shared__ uint16_t dOs[kStream * G::LDR];
    __shared__ float Ls[kStream];
    __shared__ __attribute__((aligned(16))) float Dl[kStream];   // -D per query row

    const Lane L;
    const int kvt = tile_, bh = bh_;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const uint16_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint16_t* kbase = qbase + C;
    const uint16_t* vbase = qbase + 2 * (size_t)C;
    const uint16_t* dobase = dout + (size_t)b * T * C + (size_t)h * HS;
    const float* lrow = lse + (size_t)bh * T;
    const float* drow = Dws + (size_t)bh * T;

    const int c0 = kvt * BN + L.w * R;   // this wave's first key row
    V8<E> kreg[KB][G::KSTEPS], vreg[KB][G::KSTEPS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kv = c0 + 16 * kb + L.r16;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            kreg[kb][s] = row_chunk_global<E, HS>(kbase + (size_t)kv * C3, kv < T, s, L.g);
            vreg[kb][s] = row_chunk_global<E, HS>(vbase + (size_t)kv * C3, kv < T, s, L.g);
        }
    }
    f32x4 dk[KB][G::MB], dv[KB][G::MB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) {
            dk[kb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
            dv[kb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int nqt_all = (T + kStream - 1) / kStream;
    const int nqt = PART ? min(nqt_all, part.kt_hi) : nqt_all;
    const int qt0 = max(causal ? (kvt * BN) / kStream : 0, PART ? part.kt_lo : 0);
    TileRegs<HS, 64 * NW> rq, rd;
    float rl = 0.f, rD = 0.f;
    // lse and D of the tile's rows are loaded raw and only transformed when
    // stored, so nothing waits for them before the next step
    auto fetch = [&](int qt) {
        rq.fetch(qbase, C3, qt * kStream, T, L.tid);
        rd.fetch(dobase, (size_t)C, qt * kStream, T, L.tid);
        if (L.tid < kStream) {
            const int q = min(qt * kStream + L.tid, T - 1);
            rl = lrow[q];
            rD = drow[q];
        }
    };
    fetch(qt0);
    wait_global_loads();
    for (int qt = qt0; qt < nqt; ++qt) {
        __syncthreads();
        rq.store(Qs, L.tid);
        rd.store(dOs, L.tid);
        if (L.tid < kStream) {
            const bool in = qt * kStream + L.tid < T;
            Ls[L.tid] = in ? rl * kLog2e : INFINITY;   // +inf -> P = 0
            Dl[L.tid] = in ? -rD : 0.f;
        }
        __syncthreads();
        if (qt + 1 < nqt) fetch(qt + 1);
        const int q0 = qt * kStream;
        // every query before every key here, or no key row of this wave below T
        if (c0 >= T || (causal && q0 + kStream - 1 < c0)) continue;
        const bool diag = causal && (q0 < c0 + R - 1);

        // Two 16-query blocks n = 2t, 2t+1 at a time: scores and dP, then P and
        // dS packed to bf16 and used at once for dV^T += dO^T P and
        // dK^T += Q^T dS (32 queries per matrix-core step).
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 p[KB][2], ds[KB][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int n = 2 * t + u;
                // s[kb][i], dp[kb][i] for q = q0 + 16n + 4g + i, kv = c0 + 16kb + r16;
                // the dP products start from -D of their query rows, so they
                // end at dP - D and dS = P * (dP - D) needs no subtraction
                const f32x4 dneg = *reinterpret_cast<const f32x4*>(Dl + 16 * n + 4 * L.g);
                f32x4 s[KB], dp[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    dp[kb] = dneg;
                }
#pragma unroll
                for (int st = 0; st < G::KSTEPS; ++st) {
                    const V8<E> qc = row_chunk_lds<E, HS>(Qs, 16 * n + L.r16, st, L.g);
                    const V8<E> dc = row_chunk_lds<E, HS>(dOs, 16 * n + L.r16, st, L.g);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        s[kb] = E::mfma(qc, kreg[kb][st], s[kb]);
                        dp[kb] = E::mfma(dc, vreg[kb][st], dp[kb]);
                    }
                }
                if (diag) {   // query q0 + 16n + 4g + i sees key c0 + 16kb + r16 iff i >= d
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const int d = c0 + 16 * kb + L.r16 - (q0 + 16 * n + 4 * L.g);
#pragma unroll
                        for (int i = 0; i < 4; ++i) s[kb][i] = (i >= d) ? s[kb][i] : -INFINITY;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ql = 16 * n + 4 * L.g + i;
                    const float l2 = Ls[ql];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const float pv = fast_exp2(fmaf(s[kb][i], scale_log2, -l2));
                        p[kb][u][i] = pv;
                        ds[kb][u][i] = pv * dp[kb][i];
                    }
                }
            }
            V8<E> pb[KB], sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                pb[kb] = pack_pair<E>(p[kb][0], p[kb][1]);
                sb[kb] = pack_pair<E>(ds[kb][0], ds[kb][1]);
            }
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb) {
                const V8<E> dop = col_operand<E, HS>(dOs, 32 * t, 16 * mb, L.l);
                const V8<E> qop = col_operand<E, HS>(Qs, 32 * t, 16 * mb, L.l);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    dv[kb][mb] = E::mfma(dop, pb[kb], dv[kb][mb]);
                    dk[kb][mb] = E::mfma(qop, sb[kb], dk[kb][mb]);
                }
            }
        }
    }

#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kv = c0 + 16 * kb + L.r16;
        if (kv < T) {
            if constexpr (PART) {
                float* prow = part.o + ((size_t)b * T + kv) * 2 * C + (size_t)h * HS;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) {
                    const f32x4 a = dk[kb][mb] * scale;
                    const f32x4 v = dv[kb][mb];
                    *reinterpret_cast<float4*>(prow + 16 * mb + 4 * L.g) = make_float4(a[0], a[1], a[2], a[3]);
                    *reinterpret_cast<float4*>(prow + C + 16 * mb + 4 * L.g) = make_float4(v[0], v[1], v[2], v[3]);
                }
            } else {
                uint16_t* dkrow = dqkv + ((size_t)b * T + kv) * C3 + C + (size_t)h * HS;
                uint16_t* dvrow = dkrow + C;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) {
                    store4<E>(dkrow + 16 * mb + 4 * L.g, dk[kb][mb] * scale);
                    store4<E>(dvrow + 16 * mb + 4 * L.g, dv[kb][mb]);
                }
            }
        }
    }
}

// ----------------------------------------------------------- backward dQ
// Workgroup: a 4*R-row Q tile (R = 16*QB rows per wave, Q and dO in
// registers); K and V stream through LDS 64 rows at a time.  It first forms
// D = dO . O for its rows and writes it out for the dK/dV kernel, which runs
// after it.
// PART: the workgroup takes the key tiles [part.kt_lo, part.kt_hi) only and
// writes its fp32 dq sum (scaled) to the partial slab part.o (B, T, C); the
// workgroup of the first key range also writes D.
template <typename E, int HS, int QB, bool PART, int NW = 4>
__device__ __forceinline__ void bwd_dq_half_tile(
    int tile_, int bh_, uint16_t* __restrict__ dqkv, float* __restrict__ Dws,
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ qkv,
    const uint16_t* __restrict__ out, const float* __restrict__ lse, int T, int C, int NH,
    int causal, float scale, float scale_log2, KeyPart part) {
    using G = Geom<HS>;
    constexpr int R = 16 * QB;
    constexpr int BM = NW * R;
    __shared__ uint16_t Ks[kStream * G::LDR];
    __shared__ uint16_t Vs[kStream * G::LDR];

    const Lane L;
    const int qt = tile_, bh = bh_;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const uint16_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint16_t* kbase = qbase + C;
    const uint16_t* vbase = qbase + 2 * (size_t)C;
    const uint16_t* dobase = dout + (size_t)b * T * C + (size_t)h * HS;

    const int r0 = qt * BM + L.w * R;
    V8<E> qreg[QB][G::KSTEPS], doreg[QB][G::KSTEPS];
    float l2[QB], Dq[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = r0 + 16 * qb + L.r16;
        const bool v = q < T;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            qreg[qb][s] = row_chunk_global<E, HS>(qbase + (size_t)q * C3, v, s, L.g);
            doreg[qb][s] = row_chunk_global<E, HS>(dobase + (size_t)q * C, v, s, L.g);
        }
        l2[qb] = v ? lse[(size_t)bh * T + q] * kLog2e : INFINITY;
        // D = dO . O for this row (the pre-pass, fused): the lane's columns,
        // then the four lanes of the row; written for the dK/dV kernel.
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            const V8<E> oc = row_chunk_global<E, HS>(out + ((size_t)b * T + q) * C + (size_t)h * HS, v, s, L.g);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)doreg[qb][s][e], (float)oc[e], acc);
        }
        Dq[qb] = group4_sum(acc);
        if (v && L.g == 0 && (!PART || part.kt_lo == 0)) Dws[(size_t)bh * T + q] = Dq[qb];
    }
    f32x4 dq[QB][G::MB], dneg[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        dneg[qb] = f32x4{-Dq[qb], -Dq[qb], -Dq[qb], -Dq[qb]};
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) dq[qb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nkt_all = (T + kStream - 1) / kStream;
    const int nkt_tile = causal ? min(nkt_all, (qt * BM + BM - 1) / kStream + 1) : nkt_all;
    const int kt_lo = PART ? part.kt_lo : 0;
    const int nkt = PART ? min(nkt_tile, part.kt_hi) : nkt_tile;
    TileRegs<HS, 64 * NW> rk, rv;
    rk.fetch(kbase, C3, kt_lo * kStream, T, L.tid);
    rv.fetch(vbase, C3, kt_lo * kStream, T, L.tid);
    wait_global_loads();
    for (int kt = kt_lo; kt < nkt; ++kt) {
        __syncthreads();
        rk.store(Ks, L.tid);
        rv.store(Vs, L.tid);
        __syncthreads();
        if (kt + 1 < nkt) {
            rk.fetch(kbase, C3, (kt + 1) * kStream, T, L.tid);
            rv.fetch(vbase, C3, (kt + 1) * kStream, T, L.tid);
        }
        const int k0 = kt * kStream;
        if (r0 >= T || (causal && k0 > r0 + R - 1)) continue;   // no row of this wave sees a key here
        const bool edge = (k0 + kStream > T) || (causal && k0 + kStream - 1 > r0);

        // Two 16-key blocks n = 2t, 2t+1 at a time: S^T and dP^T, then dS packed
        // to bf16 and used at once for dQ^T += K^T dS^T (32 keys per step).
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 ds[QB][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int n = 2 * t + u;
                // s[qb][i], dp[qb][i] for q = r0 + 16qb + r16, kv = k0 + 16n + 4g + i;
                // dP starts from -D of the lane's row (dS = P * (dP - D) then
                // needs no subtraction)
                f32x4 s[QB], dp[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    s[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    dp[qb] = dneg[qb];
                }
#pragma unroll
                for (int st = 0; st < G::KSTEPS; ++st) {
                    const V8<E> kc = row_chunk_lds<E, HS>(Ks, 16 * n + L.r16, st, L.g);
                    const V8<E> vc = row_chunk_lds<E, HS>(Vs, 16 * n + L.r16, st, L.g);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        s[qb] = E::mfma(kc, qreg[qb][st], s[qb]);
                        dp[qb] = E::mfma(vc, doreg[qb][st], dp[qb]);
                    }
                }
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    if (edge) {   // key k0 + 16n + 4g + i stays iff i < d (else P = 0)
                        const int row = r0 + 16 * qb + L.r16;
                        const int d = (causal ? min(T, row + 1) : T) - (k0 + 16 * n + 4 * L.g);
#pragma unroll
                        for (int i = 0; i < 4; ++i) s[qb][i] = (i < d) ? s[qb][i] : -INFINITY;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float pv = fast_exp2(fmaf(s[qb][i], scale_log2, -l2[qb]));
                        ds[qb][u][i] = pv * dp[qb][i];
                    }
                }
            }
            V8<E> sb[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sb[qb] = pack_pair<E>(ds[qb][0], ds[qb][1]);
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb) {
                const V8<E> kop = col_operand<E, HS>(Ks, 32 * t, 16 * mb, L.l);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) dq[qb][mb] = E::mfma(kop, sb[qb], dq[qb][mb]);
            }
        }
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q = r0 + 16 * qb + L.r16;
        if (q < T) {
            if constexpr (PART) {
                float* prow = part.o + ((size_t)b * T + q) * C + (size_t)h * HS;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) {
                    const f32x4 v = dq[qb][mb] * scale;
                    *reinterpret_cast<float4*>(prow + 16 * mb + 4 * L.g) = make_float4(v[0], v[1], v[2], v[3]);
                }
            } else {
                uint16_t* dqrow = dqkv + ((size_t)b * T + q) * C3 + (size_t)h * HS;
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) store4<E>(dqrow + 16 * mb + 4 * L.g, dq[qb][mb] * scale);
            }
        }
    }
}

// ------------------------------------------- backward, short sequences
// One workgroup per head for T <= 256 (hs <= 64), so a head's dQ sums over
// keys stay inside one workgroup.  Eight waves each own 32 key rows (K and V
// in registers, dK and dV accumulated), as in the dK/dV kernel, and the
// head's queries stream through LDS 64 at a time.  Per query tile each wave
// also leaves its block of dS^T in LDS; after a barrier the workgroup forms
// the tile's dQ = scale * dS K from it over all the head's keys, with K^T
// (kept in LDS from the start) as the other operand.  So S and dP are formed
// once per score (five products instead of the two kernels' seven), the dS
// never reaches memory, D = dO . O comes from the streamed tiles, and q, k,
// v, out, dout and lse are each read once.
constexpr int kShortT = 256;     // keys per workgroup: 8 waves of 32
constexpr int kShortWaves = 8;

// Column operand with the k order of a row read: lane (j, g) receives
// tile[base + 8g + e][col0 + j], e = 0..7 (the two transpose reads address
// rows base + 8g + i/4 and base + 8g + 4 + i/4; see col_operand for the
// lane mapping of ds_read_b64_tr_b16).
template <typename E>
__device__ __forceinline__ V8<E> col_operand_seq(const uint16_t* tile, int ld, int base, int col0,
                                                 int lane) {
    const int j = lane & 15, g = lane >> 4;
    const uint16_t* p = tile + (base + 8 * g + (j >> 2)) * ld + col0 + 4 * (j & 3);
    const s16x4 a = tr_read(p);
    const s16x4 b = tr_read(p + 4 * ld);
    V8<E> r;
    __builtin_memcpy(&r, &a, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
    return r;
}

template <typename E, int HS>
__device__ __forceinline__ void bwd_short_half_head(
    int bh, uint16_t* __restrict__ dqkv, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, int T, int C, int NH, int causal, float scale,
    float scale_log2) {
    using G = Geom<HS>;
    constexpr int NW = kShortWaves, NT = 64 * NW;
    constexpr int KB = 2, R = 16 * KB;
    static_assert(NW * R == kShortT, "one key row per workgroup slot");
    // K^T row stride: 672 bytes, the same bank offset from row to row (160
    // mod 256) as the hs + 16 stride of the row-major tiles (a 528-byte
    // stride measured 2% slower); dS^T rows: 144 bytes
    constexpr int KTR = kShortT + 80;
    constexpr int DSR = kStream + 8;
    constexpr int PB = G::MB >= 2 ? G::MB / 2 : 1;   // dQ output blocks per wave
    constexpr int CH = HS / 8;                       // 16-byte chunks per row
    static_assert(TileRegs<HS, NT>::N == 1, "one chunk per thread");
    __shared__ __attribute__((aligned(16))) uint16_t Qs[kStream * G::LDR];
    __shared__ __attribute__((aligned(16))) uint16_t dOs[kStream * G::LDR];
    __shared__ __attribute__((aligned(16))) uint16_t KT[HS * KTR];
    __shared__ __attribute__((aligned(16))) uint16_t dST[kShortT * DSR];
    __shared__ float Ls[kStream];
    __shared__ __attribute__((aligned(16))) float Dl[kStream];   // -D per query row

    const Lane L;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const size_t C3 = 3 * (size_t)C;
    const uint16_t* qbase = qkv + (size_t)b * T * C3 + (size_t)h * HS;
    const uint16_t* kbase = qbase + C;
    const uint16_t* vbase = qbase + 2 * (size_t)C;
    const uint16_t* dobase = dout + (size_t)b * T * C + (size_t)h * HS;
    const uint16_t* obase = out + (size_t)b * T * C + (size_t)h * HS;
    const float* lrow = lse + (size_t)bh * T;

    const int c0 = L.w * R;   // this wave's first key row
    V8<E> kreg[KB][G::KSTEPS], vreg[KB][G::KSTEPS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kv = c0 + 16 * kb + L.r16;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            kreg[kb][s] = row_chunk_global<E, HS>(kbase + (size_t)kv * C3, kv < T, s, L.g);
            vreg[kb][s] = row_chunk_global<E, HS>(vbase + (size_t)kv * C3, kv < T, s, L.g);
        }
    }
    f32x4 dk[KB][G::MB], dv[KB][G::MB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) {
            dk[kb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
            dv[kb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int nqt = (T + kStream - 1) / kStream;
    TileRegs<HS, NT> rq, rd, ro;
    float rl = 0.f;
    auto fetch = [&](int qt) {
        rq.fetch(qbase, C3, qt * kStream, T, L.tid);
        rd.fetch(dobase, (size_t)C, qt * kStream, T, L.tid);
        ro.fetch(obase, (size_t)C, qt * kStream, T, L.tid);
        if (L.tid < kStream) rl = lrow[min(qt * kStream + L.tid, T - 1)];
    };
    fetch(0);
    // K^T: lane (key c0 + 16kb + r16, g) holds dims 32s + 8g .. +7 (zeros
    // for keys >= T)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
            const int d0 = 32 * s + 8 * L.g;
            if (d0 < HS) {
                uint16_t u[8];
                __builtin_memcpy(u, &kreg[kb][s], 16);
#pragma unroll
                for (int e = 0; e < 8; ++e) KT[(d0 + e) * KTR + c0 + 16 * kb + L.r16] = u[e];
            }
        }
    wait_global_loads();

    for (int qt = 0; qt < nqt; ++qt) {
        const int q0 = qt * kStream;
        __syncthreads();   // the previous tile's reads of Qs, dOs and dST are done
        rq.store(Qs, L.tid);
        rd.store(dOs, L.tid);
        {   // D = dO . O per query row: the thread's chunk, then the CH threads of the row
            float acc = 0.f;
            if (L.tid < kStream * CH) {
                const uint32_t av[4] = {rd.v[0].x, rd.v[0].y, rd.v[0].z, rd.v[0].w};
                const uint32_t ov[4] = {ro.v[0].x, ro.v[0].y, ro.v[0].z, ro.v[0].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc = fmaf(E::bits_to_f32(av[q]), E::bits_to_f32(ov[q]), acc);
                    acc = fmaf(E::bits_to_f32(av[q] >> 16), E::bits_to_f32(ov[q] >> 16), acc);
                }
            }
#pragma unroll
            for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
            const int row = L.tid / CH;
            if (L.tid < kStream * CH && L.tid % CH == 0) Dl[row] = q0 + row < T ? -acc : 0.f;
        }
        if (L.tid < kStream) Ls[L.tid] = q0 + L.tid < T ? rl * kLog2e : INFINITY;   // +inf -> P = 0
        __syncthreads();
        if (qt + 1 < nqt) fetch(qt + 1);

        // This wave's keys against the tile's queries (skipped when every
        // query precedes every key, or no key row of the wave is below T):
        // dV^T += dO^T P, dK^T += Q^T dS, and dS^T into LDS.
        if (c0 < T && !(causal && q0 + kStream - 1 < c0)) {
            const bool mask = (causal && q0 < c0 + R - 1) || c0 + R > T;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (t == 1 && q0 + 32 >= T) break;   // the tile's last 32 queries all lie past T
                f32x4 p[KB][2], ds[KB][2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int n = 2 * t + u;
                    // s[kb][i], dp[kb][i] for q = q0 + 16n + 4g + i, kv = c0 + 16kb + r16
                    const f32x4 dneg = *reinterpret_cast<const f32x4*>(Dl + 16 * n + 4 * L.g);
                    f32x4 s[KB], dp[KB];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                        dp[kb] = dneg;
                    }
#pragma unroll
                    for (int st = 0; st < G::KSTEPS; ++st) {
                        const V8<E> qc = row_chunk_lds<E, HS>(Qs, 16 * n + L.r16, st, L.g);
                        const V8<E> dc = row_chunk_lds<E, HS>(dOs, 16 * n + L.r16, st, L.g);
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            s[kb] = E::mfma(qc, kreg[kb][st], s[kb]);
                            dp[kb] = E::mfma(dc, vreg[kb][st], dp[kb]);
                        }
                    }
                    if (mask) {   // key kv stays iff kv < T and (causal) kv <= q
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            const int kv = c0 + 16 * kb + L.r16;
                            const int d = causal ? kv - (q0 + 16 * n + 4 * L.g) : -4;
                            const bool in = kv < T;
#pragma unroll
                            for (int i = 0; i < 4; ++i) s[kb][i] = (in && i >= d) ? s[kb][i] : -INFINITY;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float l2 = Ls[16 * n + 4 * L.g + i];
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            const float pv = fast_exp2(fmaf(s[kb][i], scale_log2, -l2));
                            p[kb][u][i] = pv;
                            ds[kb][u][i] = pv * dp[kb][i];
                        }
                    }
                }
                V8<E> pb[KB], sb[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    pb[kb] = pack_pair<E>(p[kb][0], p[kb][1]);
                    sb[kb] = pack_pair<E>(ds[kb][0], ds[kb][1]);
                    // dS^T rows: the packed halves are queries 32t + 4g .. +3 and 32t + 16 + 4g .. +3
                    uint4 raw;
                    __builtin_memcpy(&raw, &sb[kb], 16);
                    uint16_t* drow = dST + (c0 + 16 * kb + L.r16) * DSR + 32 * t + 4 * L.g;
                    *reinterpret_cast<uint2*>(drow) = make_uint2(raw.x, raw.y);
                    *reinterpret_cast<uint2*>(drow + 16) = make_uint2(raw.z, raw.w);
                }
#pragma unroll
                for (int mb = 0; mb < G::MB; ++mb) {
                    const V8<E> dop = col_operand<E, HS>(dOs, 32 * t, 16 * mb, L.l);
                    const V8<E> qop = col_operand<E, HS>(Qs, 32 * t, 16 * mb, L.l);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        dv[kb][mb] = E::mfma(dop, pb[kb], dv[kb][mb]);
                        dk[kb][mb] = E::mfma(qop, sb[kb], dk[kb][mb]);
                    }
                }
            }
        }
        __syncthreads();   // the tile's dS^T is complete

        // dQ^T = K^T dS^T for the tile: wave w takes query block w/2 and PB
        // of the MB column blocks (hs = 16: waves 0..3, one block each);
        // keys up to the tile's last query (causal) or T, 32 at a time.
        {
            const int qb = G::MB >= 2 ? (L.w >> 1) : L.w;
            const int mb0 = G::MB >= 2 ? (L.w & 1) * PB : 0;
            if (qb < 4 && q0 + 16 * qb < T) {
                const int klim = causal ? min(T, q0 + kStream) : T;
                const int nks = (klim + 31) / 32;
                f32x4 acc[PB];
#pragma unroll
                for (int pp = 0; pp < PB; ++pp) acc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int ks = 0; ks < nks; ++ks) {
                    const V8<E> sop = col_operand_seq<E>(dST, DSR, 32 * ks, 16 * qb, L.l);
#pragma unroll
                    for (int pp = 0; pp < PB; ++pp) {
                        const V8<E> kop = as_v8<E>(*reinterpret_cast<const uint4*>(
                            KT + (16 * (mb0 + pp) + L.r16) * KTR + 32 * ks + 8 * L.g));
                        acc[pp] = E::mfma(kop, sop, acc[pp]);
                    }
                }
                const int q = q0 + 16 * qb + L.r16;
                if (q < T) {
                    uint16_t* dqrow = dqkv + ((size_t)b * T + q) * C3 + (size_t)h * HS;
#pragma unroll
                    for (int pp = 0; pp < PB; ++pp)
                        store4<E>(dqrow + 16 * (mb0 + pp) + 4 * L.g, acc[pp] * scale);
                }
            }
        }
    }

#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kv = c0 + 16 * kb + L.r16;
        if (kv < T) {
            uint16_t* dkrow = dqkv + ((size_t)b * T + kv) * C3 + C + (size_t)h * HS;
            uint16_t* dvrow = dkrow + C;
#pragma unroll
            for (int mb = 0; mb < G::MB; ++mb) {
                store4<E>(dkrow + 16 * mb + 4 * L.g, dk[kb][mb] * scale);
                store4<E>(dvrow + 16 * mb + 4 * L.g, dv[kb][mb]);
            }
        }
    }
}

// 16-row blocks per wave in the forward and dQ kernels (measured on the
// GPT-2, ViT and long-context shapes: 2 beats 1 and 4)
// ------------------------------------------------------------- kernels
// Each runs its tile function on the tile deal_tile gives it.
// NW waves per workgroup: 4 (128-row tiles), or 8 (256-row tiles: one tile
// per head for T <= 256, so the streamed K and V are read once per head)
template <typename E, int HS, int QB, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(HS >= 128 ? 2 : NW == 8 ? 4 : 3))) void fwd_half_kernel(uint16_t* __restrict__ out,
                                                            float* __restrict__ lse,
                                                            const uint16_t* __restrict__ qkv,
                                                            int T, int C, int NH, int causal,
                                                            float scale_log2, Deal deal) {
    const int nt = (T + 16 * QB * NW - 1) / (16 * QB * NW);
    int bh, t;
    deal_tile(gridDim.x / nt, nt, causal != 0, deal, bh, t);
    fwd_half_tile<E, HS, QB, false, NW>(t, bh, out, lse, qkv, T, C, NH, causal, scale_log2,
                                        KeyPart{0, 0, nullptr, nullptr});
}

// Split-KV forward: workgroup (rank, bh) of a grid of nqt * nchunk * BH
// takes Q tile nqt - 1 - rank / nchunk (heaviest first) and key chunk
// rank % nchunk (chunk_tiles 64-key tiles); chunks wholly past the tile's
// last key do nothing.  Each writes its partial output and log-sum-exp into
// the chunk's slabs of o_parts (nchunk, B, T, C) and lse_parts
// (nchunk, B, NH, T); merge_kernel combines them per row.
template <typename E, int HS, int QB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(HS >= 128 ? 2 : 3))) void fwd_part_half_kernel(float* __restrict__ o_parts,
                                                            float* __restrict__ lse_parts,
                                                            const uint16_t* __restrict__ qkv,
                                                            int T, int C, int NH, int causal,
                                                            float scale_log2, int BH, int nchunk,
                                                            int chunk_tiles) {
    const int nt = (T + 64 * QB - 1) / (64 * QB);
    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x - rank * BH;
    const int tile = nt - 1 - rank / nchunk;
    const int c = rank - (rank / nchunk) * nchunk;
    if (tile < 0) return;
    const int nkt_all = (T + kStream - 1) / kStream;
    const int nkt_tile = causal ? min(nkt_all, (tile * 64 * QB + 64 * QB - 1) / kStream + 1) : nkt_all;
    const int lo = c * chunk_tiles;
    if (lo >= nkt_tile) return;   // whole workgroup: no barrier is reached
    const size_t B = (size_t)BH / NH;
    KeyPart part{lo, lo + chunk_tiles, o_parts + (size_t)c * B * T * C,
                 lse_parts + (size_t)c * BH * T};
    fwd_half_tile<E, HS, QB, true>(tile, bh, nullptr, nullptr, qkv, T, C, NH, causal, scale_log2,
                                   part);
}

template <typename E, int HS, int KB, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_half_kernel(
    uint16_t* __restrict__ dqkv, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Dws, int T, int C, int NH, int causal, float scale,
    float scale_log2, Deal deal) {
    const int nt = (T + 16 * KB * NW - 1) / (16 * KB * NW);
    int bh, t;
    deal_tile(gridDim.x / nt, nt, false, deal, bh, t);
    bwd_dkdv_half_tile<E, HS, KB, false, NW>(t, bh, dqkv, dout, qkv, lse, Dws, T, C, NH, causal,
                                             scale, scale_log2, KeyPart{0, 0, nullptr, nullptr});
}

template <typename E, int HS, int QB, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(HS >= 128 ? 2 : 3))) void bwd_dq_half_kernel(
    uint16_t* __restrict__ dqkv, float* __restrict__ Dws, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, int T, int C, int NH, int causal, float scale,
    float scale_log2, Deal deal) {
    const int nt = (T + 16 * QB * NW - 1) / (16 * QB * NW);
    int bh, t;
    deal_tile(gridDim.x / nt, nt, causal != 0, deal, bh, t);
    bwd_dq_half_tile<E, HS, QB, false, NW>(t, bh, dqkv, Dws, dout, qkv, out, lse, T, C, NH, causal,
                                           scale, scale_log2, KeyPart{0, 0, nullptr, nullptr});
}

// Short-sequence backward: workgroup bh takes head bh.
template <typename E, int HS>
__global__ __launch_bounds__(64 * kShortWaves) __attribute__((amdgpu_waves_per_eu(2))) void bwd_short_half_kernel(
    uint16_t* __restrict__ dqkv, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, int T, int C, int NH, int causal, float scale,
    float scale_log2) {
    bwd_short_half_head<E, HS>(blockIdx.x, dqkv, dout, qkv, out, lse, T, C, NH, causal, scale,
                               scale_log2);
}

// Split backward.  dQ: workgroup (rank, bh) of nqt * nchunk * BH takes Q
// tile nqt - 1 - rank / nchunk and key chunk rank % nchunk (chunk_tiles
// 64-key tiles; chunks past the tile's last key do nothing), writing its
// dq sum to slab c of dq_parts (nchunk, B, T, C).  dK/dV: workgroup (rank,
// bh) of nkvt * nchunk * BH takes K/V tile rank / nchunk and query chunk
// rank % nchunk (chunk_tiles 64-row query tiles; chunks wholly before the
// tile's first query do nothing), writing dk, dv sums to slab c of
// dkv_parts (nchunk, B, T, 2C).  sum_parts_kernel adds the slabs.
template <typename E, int HS, int QB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(HS >= 128 ? 2 : 3))) void bwd_dq_part_half_kernel(
    float* __restrict__ dq_parts, float* __restrict__ Dws, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, int T, int C, int NH, int causal, float scale,
    float scale_log2, int BH, int nchunk, int chunk_tiles) {
    const int nt = (T + 64 * QB - 1) / (64 * QB);
    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x - rank * BH;
    const int tile = nt - 1 - rank / nchunk;
    const int c = rank - (rank / nchunk) * nchunk;
    if (tile < 0) return;
    const int nkt_all = (T + kStream - 1) / kStream;
    const int nkt_tile = causal ? min(nkt_all, (tile * 64 * QB + 64 * QB - 1) / kStream + 1) : nkt_all;
    const int lo = c * chunk_tiles;
    if (lo >= nkt_tile) return;   // whole workgroup: no barrier is reached
    const size_t B = (size_t)BH / NH;
    KeyPart part{lo, lo + chunk_tiles, dq_parts + (size_t)c * B * T * C, nullptr};
    bwd_dq_half_tile<E, HS, QB, true>(tile, bh, nullptr, Dws, dout, qkv, out, lse, T, C, NH, causal,
                                      scale, scale_log2, part);
}

template <typename E, int HS, int KB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_part_half_kernel(
    float* __restrict__ dkv_parts, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Dws, int T, int C, int NH, int causal, float scale,
    float scale_log2, int BH, int nchunk, int chunk_tiles) {
    constexpr int BN = 64 * KB;
    const int nt = (T + BN - 1) / BN;
    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x - rank * BH;
    const int tile = rank / nchunk;
    const int c = rank - (rank / nchunk) * nchunk;
    if (tile >= nt) return;
    const int nqt_all = (T + kStream - 1) / kStream;
    const int qt0 = causal ? (tile * BN) / kStream : 0;
    const int hi = min(nqt_all, (c + 1) * chunk_tiles);
    if (hi <= qt0) return;        // whole workgroup: no barrier is reached
    const size_t B = (size_t)BH / NH;
    KeyPart part{c * chunk_tiles, hi, dkv_parts + (size_t)c * B * T * 2 * C, nullptr};
    bwd_dkdv_half_tile<E, HS, KB, true>(tile, bh, nullptr, dout, qkv, lse, Dws, T, C, NH, causal,
                                        scale, scale_log2, part);
}

// Sum of the partial slabs into one third (part 0: dq, width C) or two
// thirds (dk, dv, width 2C) of the packed dqkv, rounded once to the 16-bit
// type.  Row t of the dq slabs has parts c < ceil(kend / chunk) (causal:
// kend = the end of its Q tile's keys); key row j of the dk/dv slabs has
// parts c >= first query row of its K/V tile / chunk (causal).  The parts
// are added in increasing c.
template <typename E>
__global__ __launch_bounds__(kThreads) void sum_parts_kernel(uint16_t* __restrict__ dqkv,
                                                             const float* __restrict__ parts,
                                                             int P, int B, int T, int C, int width,
                                                             int col0, int causal, int q_rows,
                                                             int kv_rows, int chunk, long long n4) {
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= n4) return;
    const int W4 = width / 4;
    const long long row = gid / W4;   // b*T + t
    const int c = (int)(gid - row * W4) * 4;
    const int t = (int)(row % T);
    int p0 = 0, p1 = P;
    if (causal && q_rows > 0) p1 = min(P, (min(T, (t / q_rows + 1) * q_rows) + chunk - 1) / chunk);
    if (causal && kv_rows > 0) p0 = ((t / kv_rows) * kv_rows) / chunk;
    const size_t slab = (size_t)B * T * width;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p = p0; p < p1; ++p) {
        const float4 v = *reinterpret_cast<const float4*>(parts + p * slab + (size_t)row * width + c);
        acc[0] += v.x;
        acc[1] += v.y;
        acc[2] += v.z;
        acc[3] += v.w;
    }
    store4<E>(dqkv + (size_t)row * 3 * C + col0 + c, f32x4{acc[0], acc[1], acc[2], acc[3]});
}

constexpr int kQB = 2;
static_assert(64 * kQB == kFwdHalfRows, "forward Q tile rows");
// dK/dV: 32 K/V rows per wave for hs <= 64, 16 for hs = 128 (fewer
// registers, more resident waves; measured faster on the long-context shape)
constexpr int kb_for(int hs) { return hs >= 128 ? 1 : 2; }

// Short sequences (128 < T <= 256, hs <= 64): the forward runs 8-wave
// workgroups of 256 rows, one per head, so every K and V row is read once
// per head instead of once per 128-row tile (ViT-B/16, T = 196: 45.5 ->
// 39.2 us).  The dQ and dK/dV kernels keep 4 waves: at 8 their register
// needs leave one workgroup per CU (dQ 63 -> 72 us, dK/dV 74 -> 84 us; dQ
// held to 4 waves per SIMD spills, 83 us).  The fused backward of such
// shapes runs bwd_short_half_kernel instead (ViT-B/16: dQ + dK/dV 136 us,
// fused 123 us).
template <int HS>
bool short_seq(const Shape& s) { return HS <= 64 && s.T <= 256 && s.T > 128; }

template <typename E, int HS, int NW>
hipError_t fwd_half_nw(uint16_t* out, float* lse, const uint16_t* qkv, const Shape& s,
                       hipStream_t st) {
    constexpr int BM = 16 * kQB * NW;
    const int nqt = (s.T + BM - 1) / BM;
    const unsigned grid = (unsigned)(nqt * s.B * s.NH);
    const float scale_log2 = (float)(1.0 / sqrt((double)HS)) * kLog2e;
    const Deal deal = deal_for<fwd_half_kernel<E, HS, kQB, NW>>(64 * NW);
    hipLaunchKernelGGL((fwd_half_kernel<E, HS, kQB, NW>), dim3(grid), dim3(64 * NW), 0, st, out,
                       lse, qkv, s.T, s.C, s.NH, s.causal, scale_log2, deal);
    return hipGetLastError();
}

template <typename E, int HS>
hipError_t fwd_half_hs(uint16_t* out, float* lse, const uint16_t* qkv, const Shape& s,
                       hipStream_t st) {
    if (short_seq<HS>(s)) return fwd_half_nw<E, HS, 8>(out, lse, qkv, s, st);
    return fwd_half_nw<E, HS, 4>(out, lse, qkv, s, st);
}

template <typename E, int HS>
hipError_t fwd_part_half_hs(float* o_parts, float* lse_parts, const uint16_t* qkv, int chunk_tiles,
                            const Shape& s, hipStream_t st) {
    constexpr int BM = 64 * kQB;
    const int nqt = (s.T + BM - 1) / BM;
    const int nkt = (s.T + kStream - 1) / kStream;
    const int nchunk = (nkt + chunk_tiles - 1) / chunk_tiles;
    const long long BH = (long long)s.B * s.NH;
    const long long grid = (long long)nqt * nchunk * BH;
    if (grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float scale_log2 = (float)(1.0 / sqrt((double)HS)) * kLog2e;
    hipLaunchKernelGGL((fwd_part_half_kernel<E, HS, kQB>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                       o_parts, lse_parts, qkv, s.T, s.C, s.NH, s.causal, scale_log2, (int)BH,
                       nchunk, chunk_tiles);
    return hipGetLastError();
}

template <typename E, int HS>
hipError_t bwd_split_half_hs(uint16_t* dqkv, float* work, const uint16_t* dout,
                             const uint16_t* qkv, const uint16_t* out, const float* lse,
                             int chunk_tiles, const Shape& s, hipStream_t st) {
    constexpr int KB = kb_for(HS);
    const long long BH = (long long)s.B * s.NH;
    const int nt64 = (s.T + kStream - 1) / kStream;
    const int nchunk = (nt64 + chunk_tiles - 1) / chunk_tiles;
    const size_t BTC = (size_t)s.B * s.T * s.C;
    float* D = work;
    float* dq_parts = work + (((size_t)BH * s.T + 63) & ~(size_t)63);
    float* dkv_parts = dq_parts + (size_t)nchunk * BTC;
    const float scale = (float)(1.0 / sqrt((double)HS));
    const int nqt = (s.T + 64 * kQB - 1) / (64 * kQB);
    const int nkvt = (s.T + 64 * KB - 1) / (64 * KB);
    const long long g1 = (long long)nqt * nchunk * BH, g2 = (long long)nkvt * nchunk * BH;
    if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_part_half_kernel<E, HS, kQB>), dim3((unsigned)g1), dim3(kThreads), 0, st,
                       dq_parts, D, dout, qkv, out, lse, s.T, s.C, s.NH, s.causal, scale,
                       scale * kLog2e, (int)BH, nchunk, chunk_tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    long long n4 = (long long)s.B * s.T * (s.C / 4);
    hipLaunchKernelGGL(sum_parts_kernel<E>, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, st, dqkv, dq_parts, nchunk, s.B, s.T, s.C, s.C, 0, s.causal, 64 * kQB, 0,
                       64 * chunk_tiles, n4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_part_half_kernel<E, HS, KB>), dim3((unsigned)g2), dim3(kThreads), 0, st,
                       dkv_parts, dout, qkv, lse, D, s.T, s.C, s.NH, s.causal, scale, scale * kLog2e,
                       (int)BH, nchunk, chunk_tiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    n4 = (long long)s.B * s.T * (2 * s.C / 4);
    hipLaunchKernelGGL(sum_parts_kernel<E>, dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, st, dqkv, dkv_parts, nchunk, s.B, s.T, s.C, 2 * s.C, s.C, s.causal, 0,
                       64 * KB, 64 * chunk_tiles, n4);
    return hipGetLastError();
}

template <typename E, int HS>
hipError_t prepass_half_hs(float* D, const uint16_t* dout, const uint16_t* out, const Shape& s,
                           hipStream_t st) {
    const long long rows = (long long)s.B * s.T * s.NH;
    const long long threads = rows * (HS / 8);
    const unsigned grid = (unsigned)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((prepass_half_kernel<E, HS>), dim3(grid), dim3(kThreads), 0, st, D, dout,
                       out, s.T, s.NH, rows);
    return hipGetLastError();
}

template <typename E, int HS, int NW>
hipError_t dkdv_half_nw(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                        const float* lse, const float* D, const Shape& s, hipStream_t st) {
    constexpr int KB = kb_for(HS);
    constexpr int BN = 16 * KB * NW;
    const int nt = (s.T + BN - 1) / BN;
    const unsigned grid = (unsigned)(nt * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    const Deal deal = deal_for<bwd_dkdv_half_kernel<E, HS, KB, NW>>(64 * NW);
    hipLaunchKernelGGL((bwd_dkdv_half_kernel<E, HS, KB, NW>), dim3(grid), dim3(64 * NW), 0, st,
                       dqkv, dout, qkv, lse, D, s.T, s.C, s.NH, s.causal, scale, scale * kLog2e,
                       deal);
    return hipGetLastError();
}

template <typename E, int HS>
hipError_t dkdv_half_hs(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                        const float* lse, const float* D, const Shape& s, hipStream_t st) {
    return dkdv_half_nw<E, HS, 4>(dqkv, dout, qkv, lse, D, s, st);
}

template <typename E, int HS, int NW>
hipError_t dq_half_nw(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                      const uint16_t* out, const float* lse, const Shape& s, hipStream_t st) {
    constexpr int BM = 16 * kQB * NW;
    const int nt = (s.T + BM - 1) / BM;
    const unsigned grid = (unsigned)(nt * s.B * s.NH);
    const float scale = (float)(1.0 / sqrt((double)HS));
    const Deal deal = deal_for<bwd_dq_half_kernel<E, HS, kQB, NW>>(64 * NW);
    hipLaunchKernelGGL((bwd_dq_half_kernel<E, HS, kQB, NW>), dim3(grid), dim3(64 * NW), 0, st,
                       dqkv, D, dout, qkv, out, lse, s.T, s.C, s.NH, s.causal, scale,
                       scale * kLog2e, deal);
    return hipGetLastError();
}

template <typename E, int HS>
hipError_t dq_half_hs(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                      const uint16_t* out, const float* lse, const Shape& s, hipStream_t st) {
    return dq_half_nw<E, HS, 4>(dqkv, D, dout, qkv, out, lse, s, st);
}

template <typename E, int HS>
hipError_t bwd_short_half_hs(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                             const uint16_t* out, const float* lse, const Shape& s,
                             hipStream_t st) {
    if constexpr (HS > 64) {
        return hipErrorInvalidValue;
    } else {
        if (!bwd_short_applies(s)) return hipErrorInvalidValue;
        const float scale = (float)(1.0 / sqrt((double)HS));
        hipLaunchKernelGGL((bwd_short_half_kernel<E, HS>), dim3((unsigned)(s.B * s.NH)),
                           dim3(64 * kShortWaves), 0, st, dqkv, dout, qkv, out, lse, s.T, s.C, s.NH,
                           s.causal, scale, scale * kLog2e);
        return hipGetLastError();
    }
}

}  // namespace

#define ATTN_DISPATCH_HS(fn, E, ...)                      \
    switch (s.hs) {                                       \
        case 16: return fn<E, 16>(__VA_ARGS__);           \
        case 32: return fn<E, 32>(__VA_ARGS__);           \
        case 64: return fn<E, 64>(__VA_ARGS__);           \
        case 128: return fn<E, 128>(__VA_ARGS__);         \
        default: return hipErrorInvalidValue;             \
    }

#define ATTN_HALF_LAUNCHERS(SFX, E)                                                                \
    hipError_t launch_fwd_##SFX(uint16_t* out, float* lse, const uint16_t* qkv, const Shape& s,  \
                                hipStream_t st) {                                                 \
        ATTN_DISPATCH_HS(fwd_half_hs, E, out, lse, qkv, s, st)                                     \
    }                                                                                              \
    hipError_t launch_fwd_part_##SFX(float* o_parts, float* lse_parts, const uint16_t* qkv,      \
                                     int chunk_tiles, const Shape& s, hipStream_t st) {          \
        ATTN_DISPATCH_HS(fwd_part_half_hs, E, o_parts, lse_parts, qkv, chunk_tiles, s, st)         \
    }                                                                                              \
    hipError_t launch_bwd_split_##SFX(uint16_t* dqkv, float* work, const uint16_t* dout,         \
                                      const uint16_t* qkv, const uint16_t* out, const float* lse, \
                                      int chunk_tiles, const Shape& s, hipStream_t st) {          \
        ATTN_DISPATCH_HS(bwd_split_half_hs, E, dqkv, work, dout, qkv, out, lse, chunk_tiles, s, st)\
    }                                                                                              \
    hipError_t launch_prepass_##SFX(float* D, const uint16_t* dout, const uint16_t* out,          \
                                    const Shape& s, hipStream_t st) {                             \
        ATTN_DISPATCH_HS(prepass_half_hs, E, D, dout, out, s, st)                                  \
    }                                                                                              \
    hipError_t launch_dkdv_##SFX(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,       \
                                 const float* lse, const float* D, const Shape& s,                \
                                 hipStream_t st) {                                                 \
        ATTN_DISPATCH_HS(dkdv_half_hs, E, dqkv, dout, qkv, lse, D, s, st)                          \
    }                                                                                              \
    hipError_t launch_dq_##SFX(uint16_t* dqkv, float* D, const uint16_t* dout,                    \
                               const uint16_t* qkv, const uint16_t* out, const float* lse,        \
                               const Shape& s, hipStream_t st) {                                  \
        ATTN_DISPATCH_HS(dq_half_hs, E, dqkv, D, dout, qkv, out, lse, s, st)                       \
    }                                                                                              \
    hipError_t launch_bwd_short_##SFX(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,  \
                                      const uint16_t* out, const float* lse, const Shape& s,      \
                                      hipStream_t st) {                                            \
        ATTN_DISPATCH_HS(bwd_short_half_hs, E, dqkv, dout, qkv, out, lse, s, st)                   \
    }

ATTN_HALF_LAUNCHERS(bf16, BF16)
ATTN_HALF_LAUNCHERS(f16, F16)

#undef ATTN_HALF_LAUNCHERS
#undef ATTN_DISPATCH_HS

}  // namespace attn
