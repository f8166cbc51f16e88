// decode.hip -- attention of the last query row of each sequence against all
// of its keys, with the key range split over workgroups, and the merge of
// partial (O, lse) results that such a split produces.
//
// Method: the self-attention of "Umakini wa kujitegemea, kerneli za CUDA na
// FlashAttention" (section 1) for one query row, with T_q = 1 as in the
// inference part of "LLM Systems 10 & 11: Accelerating Transformer Training
// and Inference" (section 2).  A split of the keys into disjoint ranges gives
// per range a normalised output o_p and a log-sum-exp lse_p; the full result
// is the same rescale that the online softmax uses ([SW], FlashAttention
// part): L = log sum_p exp(lse_p), out = sum_p exp(lse_p - L) o_p.
//
// gfx950 mapping.  One query row does ~1 flop per byte of K and V, so the
// kernels are HBM-bound and use no matrix cores.  A workgroup of 256 threads
// takes one (sequence, head, key range): G = hs/VEC threads cover one key row
// with 16-byte loads (VEC = 4 fp32 or 8 bf16 values), so a wave reads whole
// 64..256-byte row segments; the key-row dot products finish with lane-xor
// shuffles inside each G-lane group, the softmax over the range runs in LDS,
// and P.V is reduced across the key groups through LDS.  The range length
// (128 or 256 keys) is picked so that the grid keeps >= 2 workgroups per CU.
#include "common.hpp"

namespace attn {
namespace {

constexpr int kThreads = 256;

// Element types: storage type T, VEC values per 16-byte chunk, a chunk as
// fp32 values, and the rounding store of 4 fp32 values (nearest even).
struct EF32 {
    typedef float T;
    static constexpr int VEC = 4;
    static __device__ __forceinline__ void load(float (&x)[4], const float* p) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        x[0] = v.x;
        x[1] = v.y;
        x[2] = v.z;
        x[3] = v.w;
    }
    static __device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <typename H>   // 16-bit types: H::to_f32 / H::from_f32 on bit patterns
struct E16 {
    typedef uint16_t T;
    static constexpr int VEC = 8;
    static __device__ __forceinline__ void load(float (&x)[8], const uint16_t* p) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = H::to_f32((uint16_t)(w[i] & 0xffffu));
            x[2 * i + 1] = H::to_f32((uint16_t)(w[i] >> 16));
        }
    }
    static __device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
        const uint32_t lo = (uint32_t)H::from_f32(v[0]) | ((uint32_t)H::from_f32(v[1]) << 16);
        const uint32_t hi = (uint32_t)H::from_f32(v[2]) | ((uint32_t)H::from_f32(v[3]) << 16);
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    }
};
struct HBF16 {
    static __device__ __forceinline__ float to_f32(uint16_t u) { return bf16_to_f32(u); }
    static __device__ __forceinline__ uint16_t from_f32(float f) { return f32_to_bf16(f); }
};
struct HF16 {
    static __device__ __forceinline__ float to_f32(uint16_t u) {
        _Float16 h;
        __builtin_memcpy(&h, &u, 2);
        return (float)h;
    }
    static __device__ __forceinline__ uint16_t from_f32(float f) {
        const _Float16 h = (_Float16)f;
        uint16_t u;
        __builtin_memcpy(&u, &h, 2);
        return u;
    }
};
typedef E16<HBF16> EBF16;
typedef E16<HF16> EF16;

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

// Partial attention of query row T-1 of head (b, h) against keys
// [r*L, min(T, (r+1)*L)) for r = the workgroup's range.  Writes
// o_part[(r*B + b)*C + h*HS + i] (normalised within the range) and
// lse_part[(r*B + b)*NH + h], i.e. the (nranges, B, 1, C) and
// (nranges, B, NH, 1) layouts that merge_kernel reads.
template <int HS, typename E, int L>
__global__ __launch_bounds__(kThreads) void decode_part_kernel(float* __restrict__ o_part,
                                                               float* __restrict__ lse_part,
                                                               const typename E::T* __restrict__ qkv, int B,
                                                               int T, int C, int NH, int nranges,
                                                               float scale_log2) {
    constexpr int VEC = E::VEC;
    constexpr int G = HS / VEC;          // threads per key row
    constexpr int KPP = kThreads / G;    // key rows per pass
    constexpr int NP = L / KPP;          // passes over the range
    static_assert(L % KPP == 0 && NP >= 1, "range must hold whole passes");
    __shared__ float sc[L];
    __shared__ float red[kThreads / 64];
    __shared__ float buf[KPP * HS];
    __shared__ float col[kThreads];

    const int tid = threadIdx.x;
    const int r = blockIdx.x % nranges;
    const int bh = blockIdx.x / nranges;
    const int b = bh / NH, h = bh - (bh / NH) * NH;
    const int kg = tid / G, sub = tid - (tid / G) * G;
    const size_t C3 = 3 * (size_t)C;
    const typename E::T* base = qkv + (size_t)b * T * C3 + (size_t)h * HS + sub * VEC;
    const int k0 = r * L;

    float q[VEC];
    E::load(q, base + (size_t)(T - 1) * C3);

    // K rows of the range, and its V rows too when they fit in registers
    // (then both loads are in flight together instead of one after the
    // other, around the softmax)
    constexpr bool kEarlyV = NP * VEC <= 64;
    float kx[NP][VEC];
    float vx[kEarlyV ? NP : 1][VEC];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int j = k0 + p * KPP + kg;
#pragma unroll
        for (int i = 0; i < VEC; ++i) kx[p][i] = 0.f;
        if (j < T) E::load(kx[p], base + C + (size_t)j * C3);
    }
    if constexpr (kEarlyV) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int j = k0 + p * KPP + kg;
#pragma unroll
            for (int i = 0; i < VEC; ++i) vx[p][i] = 0.f;
            if (j < T) E::load(vx[p], base + 2 * (size_t)C + (size_t)j * C3);
        }
    }

    // scores (log2 domain) of the range's keys; -inf past T
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int j = k0 + p * KPP + kg;
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) d = fmaf(q[i], kx[p][i], d);
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) d += __shfl_xor(d, off, 64);
        if (sub == 0) sc[p * KPP + kg] = (j < T) ? d * scale_log2 : -INFINITY;
    }
    __syncthreads();

    // softmax over the range (every range holds at least one key)
    float m = -INFINITY;
    for (int i = tid; i < L; i += kThreads) m = fmaxf(m, sc[i]);
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float lsum = 0.f;
    for (int i = tid; i < L; i += kThreads) {
        const float e = fast_exp2(sc[i] - m);   // -inf -> 0
        sc[i] = e;
        lsum += e;
    }
    lsum = wave_sum(lsum);
    __syncthreads();   // everyone has read red[] and written sc[]
    if ((tid & 63) == 0) red[tid >> 6] = lsum;
    __syncthreads();
    lsum = (red[0] + red[1]) + (red[2] + red[3]);

    // sum_j p_j v_j: each thread over its keys and VEC columns, then across
    // the KPP key groups through LDS
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int j = k0 + p * KPP + kg;
        if (j < T) {
            float v[VEC];
            if constexpr (kEarlyV) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) v[i] = vx[p][i];
            } else {
                E::load(v, base + 2 * (size_t)C + (size_t)j * C3);
            }
            const float w = sc[p * KPP + kg];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = fmaf(w, v[i], acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) buf[kg * HS + sub * VEC + i] = acc[i];
    __syncthreads();
    {
        constexpr int R = kThreads / HS;   // partial sums per column
        const int c = tid % HS, part = tid / HS;
        float s = 0.f;
        for (int g = part; g < KPP; g += R) s += buf[g * HS + c];
        col[part * HS + c] = s;
    }
    __syncthreads();
    if (tid < HS) {
        float o = 0.f;
#pragma unroll
        for (int part = 0; part < kThreads / HS; ++part) o += col[part * HS + tid];
        o_part[((size_t)r * B + b) * C + (size_t)h * HS + tid] = o / lsum;
    }
    if (tid == 0) lse_part[((size_t)r * B + b) * NH + h] = (m + __log2f(lsum)) * kLn2;
}

// out[b,t,c..c+3] and lse[b,h,t] from P partial results over disjoint key
// sets: o_parts (P, B, T, C) fp32 normalised per part, lse_parts (P, B, NH, T).
// A row whose parts all have lse = -inf (no key at all) gets out 0, lse -inf.
template <typename OUT>
__global__ __launch_bounds__(kThreads) void merge_kernel(typename OUT::T* __restrict__ out,
                                                         float* __restrict__ lse,
                                                         const float* __restrict__ o_parts,
                                                         const float* __restrict__ lse_parts,
                                                         int P, int B, int T, int C, int NH,
                                                         long long n4, int part_rows,
                                                         int part_keys) {
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= n4) return;
    const int C4 = C / 4;
    const long long row = gid / C4;               // b*T + t
    const int c = (int)(gid - row * C4) * 4;
    const int b = (int)(row / T), t = (int)(row - (long long)b * T);
    // causal split of the keys of part_rows-row query tiles into part_keys
    // chunks: only the chunks up to the tile's last key were written
    if (part_rows > 0) {
        const int kend = min(T, (t / part_rows + 1) * part_rows);
        P = min(P, (kend + part_keys - 1) / part_keys);
    }
    const int hs = C / NH;
    const int h = c / hs;
    const size_t BT = (size_t)B * T;
    // one pass with a running maximum (the online-softmax rescale), eight
    // parts per round so that their loads are in flight together
    constexpr int U = 8;
    float m = -INFINITY, wsum = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < P; p0 += U) {
        float lp[U];
        float4 v[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int p = p0 + i;
            lp[i] = -INFINITY;
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p < P) {
                lp[i] = lse_parts[(((size_t)p * B + b) * NH + h) * T + t];
                v[i] = *reinterpret_cast<const float4*>(o_parts + ((size_t)p * BT + row) * C + c);
            }
        }
        float mb = m;
#pragma unroll
        for (int i = 0; i < U; ++i) mb = fmaxf(mb, lp[i]);
        if (mb == -INFINITY) continue;   // no key in any part so far
        if (mb > m) {   // rescale what was summed against the old maximum
            const float a = fast_exp2((m - mb) * kLog2e);   // m = -inf -> 0
            wsum *= a;
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] *= a;
            m = mb;
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const float w = fast_exp2((lp[i] - m) * kLog2e);   // -inf -> 0
            wsum += w;
            acc[0] = fmaf(w, v[i].x, acc[0]);
            acc[1] = fmaf(w, v[i].y, acc[1]);
            acc[2] = fmaf(w, v[i].z, acc[2]);
            acc[3] = fmaf(w, v[i].w, acc[3]);
        }
    }
    if (m != -INFINITY) {
        const float inv = 1.0f / wsum;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] *= inv;
    }
    OUT::store4(out + (size_t)row * C + c, acc);
    if (c % hs == 0)
        lse[((size_t)b * NH + h) * T + t] = (m == -INFINITY) ? -INFINITY : m + __logf(wsum);
}

template <typename OUT>
hipError_t merge_launch(typename OUT::T* out, float* lse, const float* o_parts, const float* lse_parts, int P,
                        const Shape& s, hipStream_t st, int part_rows = 0, int part_keys = 1) {
    const long long n4 = (long long)s.B * s.T * (s.C / 4);
    const unsigned grid = (unsigned)((n4 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(merge_kernel<OUT>, dim3(grid), dim3(kThreads), 0, st, out, lse, o_parts,
                       lse_parts, P, s.B, s.T, s.C, s.NH, n4, part_rows, part_keys);
    return hipGetLastError();
}

template <int HS, typename E, int L>
hipError_t decode_part_launch(float* o_part, float* lse_part, const typename E::T* qkv, int nranges,
                              const Shape& s, hipStream_t st) {
    const unsigned grid = (unsigned)((long long)nranges * s.B * s.NH);
    const float scale_log2 = (float)(1.0 / sqrt((double)HS)) * kLog2e;
    hipLaunchKernelGGL((decode_part_kernel<HS, E, L>), dim3(grid), dim3(kThreads), 0, st, o_part,
                       lse_part, qkv, s.B, s.T, s.C, s.NH, nranges, scale_log2);
    return hipGetLastError();
}

template <typename E, int L>
hipError_t decode_part_hs(float* o_part, float* lse_part, const typename E::T* qkv, int nranges,
                          const Shape& s, hipStream_t st) {
    switch (s.hs) {
        case 16: return decode_part_launch<16, E, L>(o_part, lse_part, qkv, nranges, s, st);
        case 32: return decode_part_launch<32, E, L>(o_part, lse_part, qkv, nranges, s, st);
        case 64: return decode_part_launch<64, E, L>(o_part, lse_part, qkv, nranges, s, st);
        case 128: return decode_part_launch<128, E, L>(o_part, lse_part, qkv, nranges, s, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename E>
hipError_t decode_launch(typename E::T* out, float* lse, const typename E::T* qkv, float* ws,
                         const Shape& s,
                         hipStream_t st) {
    const int L = decode_range_len(s);
    const int nr = (s.T + L - 1) / L;
    float* o_part = ws;
    float* lse_part = ws + (size_t)nr * s.B * s.C;
    hipError_t e = (L == 256) ? decode_part_hs<E, 256>(o_part, lse_part, qkv, nr, s, st)
                              : decode_part_hs<E, 128>(o_part, lse_part, qkv, nr, s, st);
    if (e != hipSuccess) return e;
    Shape one = s;
    one.T = 1;
    return merge_launch<E>(out, lse, o_part, lse_part, nr, one, st);
}

}  // namespace

int decode_range_len(const Shape& s) {
    const long long bh = (long long)s.B * s.NH;
    return bh * ((s.T + 255) / 256) >= 2LL * device_cu_count() ? 256 : 128;
}

size_t decode_workspace_floats(const Shape& s) {
    const long long nr = (s.T + decode_range_len(s) - 1) / decode_range_len(s);
    return (size_t)(nr * s.B * s.C + nr * s.B * s.NH);
}

hipError_t launch_decode_f32(float* out, float* lse, const float* qkv, float* ws, const Shape& s,
                             hipStream_t st) {
    return decode_launch<EF32>(out, lse, qkv, ws, s, st);
}

hipError_t launch_decode_bf16(uint16_t* out, float* lse, const uint16_t* qkv, float* ws,
                              const Shape& s, hipStream_t st) {
    return decode_launch<EBF16>(out, lse, qkv, ws, s, st);
}

hipError_t launch_merge_f32(float* out, float* lse, const float* o_parts, const float* lse_parts,
                            int P, const Shape& s, hipStream_t st) {
    return merge_launch<EF32>(out, lse, o_parts, lse_parts, P, s, st);
}

hipError_t launch_merge_bf16(uint16_t* out, float* lse, const float* o_parts,
                             const float* lse_parts, int P, const Shape& s, hipStream_t st) {
    return merge_launch<EBF16>(out, lse, o_parts, lse_parts, P, s, st);
}

hipError_t launch_decode_f16(uint16_t* out, float* lse, const uint16_t* qkv, float* ws,
                             const Shape& s, hipStream_t st) {
    return decode_launch<EF16>(out, lse, qkv, ws, s, st);
}

hipError_t launch_merge_f16(uint16_t* out, float* lse, const float* o_parts,
                            const float* lse_parts, int P, const Shape& s, hipStream_t st) {
    return merge_launch<EF16>(out, lse, o_parts, lse_parts, P, s, st);
}

// merge of a causal split-KV forward: rows of part_rows-row query tiles, key
// chunks of part_keys keys (non-causal: every row has all P parts)
hipError_t launch_merge_split_bf16(uint16_t* out, float* lse, const float* o_parts,
                                   const float* lse_parts, int P, int part_rows, int part_keys,
                                   const Shape& s, hipStream_t st) {
    return merge_launch<EBF16>(out, lse, o_parts, lse_parts, P, s, st, s.causal ? part_rows : 0,
                               part_keys);
}
hipError_t launch_merge_split_f16(uint16_t* out, float* lse, const float* o_parts,
                                  const float* lse_parts, int P, int part_rows, int part_keys,
                                  const Shape& s, hipStream_t st) {
    return merge_launch<EF16>(out, lse, o_parts, lse_parts, P, s, st, s.causal ? part_rows : 0,
                              part_keys);
}

}  // namespace attn
