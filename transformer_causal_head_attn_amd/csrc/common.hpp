// common.hpp -- shared device helpers and internal launcher declarations
// for libattn (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include "tiles.hpp"

namespace attn {

// Problem description handed from the C ABI to the launchers.
struct Shape {
    int B, T, C, NH, hs;
    int causal;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reductions over the four lanes l, l^16, l^32, l^48 that share l % 16,
// with gfx950's lane-swap instructions (VALU, no LDS round trip):
// v_permlane32_swap(x, x) returns (lower half, upper half) of the wave in
// every lane position, v_permlane16_swap(x, x) (even row, odd row) of each
// pair of 16-lane rows.  Every lane of a group ends with the same bits.
__device__ __forceinline__ float group4_max(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0): wait until every global load the wave has issued has
// returned (immediate: vmcnt field 0, expcnt 7 and lgkmcnt 15, i.e. no wait on
// those).  Placed after a kernel's prologue loads, it also tells the
// compiler's wait-count tracking that no load is outstanding when the main
// loop starts, so the loop's first uses of the prologue's registers need no
// wait that would also cover the next tile's loads issued in the loop.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// D += A * B on the fp32 matrix cores, one 16x16 output block per wave.
// Lane l supplies A[l%16][l/16] and B[l/16][l%16] (K = 4); the result
// register i of lane l is D[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D += A * B with bf16 operands (K = 32), fp32 accumulate.  Lane l supplies
// eight k-entries of row l%16 of A and eight of column l%16 of B; entry e of
// lane group g = l/16 stands for k = 8g + e.  Only the pairing of A's and B's
// k-slots matters for the sum, so any k numbering shared by both operands
// gives the same product.  The result layout is that of mfma_f32.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 <-> fp32 (round to nearest even; NaN kept quiet).
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
    return __uint_as_float(((uint32_t)u) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Compute units of the current device (cached per device id; host threads
// may race to fill an entry, all with the same value).  A failed query is
// cleared and reads as 256.
inline int device_cu_count() {
    static std::atomic<int> cached[64];   // 0: not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Dealing causal tiles to CUs like a snake draft.  Workgroups that are
// resident together (ids c, c + ncu, c + 2 ncu, ... share a CU when a whole
// round fits on the chip) take a heaviest-first list in alternating
// directions, so a CU that got one of the heaviest tiles in one round gets
// one of the lightest of the next.  The reversal keeps id % 8, the XCD a
// workgroup is dispatched to, and a wrong guess about placement only costs
// balance.  Ids past the resident rounds keep their order.
struct Deal {
    int ncu;      // compute units (a multiple of 8 for the snake)
    int rounds;   // workgroups per CU resident at once (0: no snake)
};
__device__ __forceinline__ int snake_block(Deal deal) {
    int idx = blockIdx.x;
    if ((deal.ncu & 7) == 0 && deal.ncu > 0) {
        const int r = idx / deal.ncu;
        if ((r & 1) && r < deal.rounds && (r + 1) * deal.ncu <= (int)gridDim.x) {
            const int c = idx - r * deal.ncu;
            idx = r * deal.ncu + (deal.ncu - 8 - (c & ~7) + (c & 7));
        }
    }
    return idx;
}

// Causal tiles carry unequal work (tile i of a Q-tile kernel sees i+1 key
// tiles, tile j of a K/V-tile kernel nt-j query tiles).  Tiles run one per
// workgroup, heaviest first (the longest-first order of kernel 8 in llm.c's
// attention_backward.cu), dealt to the CUs like a snake draft: workgroups
// that are resident together (ids c, c + ncu, c + 2 ncu, ... share a CU when
// the whole round fits) take the sorted list in alternating directions, so
// a CU that got one of the heaviest tiles in the first round gets one of the
// lightest of the second.  The reversal keeps id % 8, the XCD a workgroup
// is dispatched to, and a wrong guess about placement only costs balance.
// Workgroups beyond the resident rounds take the lighter tiles as slots
// free.  (Running tiles i and nt-1-i back to back in one workgroup, which
// equalises the work, measured no better on the GPT-2 layer and 2% slower
// at long context.)  Consecutive workgroup ids walk the heads, so all tiles
// of a head land on one XCD (one L2) whenever B*NH is a multiple of 8.
__device__ __forceinline__ void deal_tile(int BH, int nt, bool heavy_high, Deal deal, int& bh,
                                          int& tile) {
    const int idx = snake_block(deal);
    const int rank = idx / BH;
    bh = idx - rank * BH;
    tile = heavy_high ? nt - 1 - rank : rank;
}

// CUs and resident workgroups per CU of `threads`-thread workgroups for a
// kernel (one occupancy query per kernel and device, cached; host threads may
// race to fill an entry, all with the same value).  A failed query is
// cleared and treated as one round.
template <auto Kernel>
Deal deal_for(int threads) {
    static std::atomic<int> cached[64];   // 0: not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return Deal{device_cu_count(), 1};
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Kernel, threads, 0) != hipSuccess ||
            n < 1) {
            (void)hipGetLastError();
            n = 1;
        }
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return Deal{device_cu_count(), n};
}

// Whether the fp32 dQ kernel's causal tiles should run in balanced pairs (one
// light, one heavy per workgroup): only while the paired grid keeps >= 2
// workgroups per CU.  The other kernels run one tile per workgroup.
inline bool pair_tiles(int ntiles, int causal, long long BH) {
    return causal && ntiles > 1 && BH * ((ntiles + 1) / 2) >= 2LL * device_cu_count();
}

// ---- launchers (return hipSuccess or the launch error) ----
// fp32 fused path
hipError_t launch_fwd_f32(float* out, float* lse, const float* qkv, const Shape& s, hipStream_t st);
hipError_t launch_prepass_f32(float* D, const float* dout, const float* out, const Shape& s,
                              hipStream_t st);
hipError_t launch_dkdv_f32(float* dqkv, const float* dout, const float* qkv, const float* lse,
                           const float* D, const Shape& s, hipStream_t st);
hipError_t launch_dq_f32(float* dqkv, float* D, const float* dout, const float* qkv,
                         const float* out, const float* lse, const Shape& s, hipStream_t st);
// the pre-pass that also clears dqkv's dQ slot, and one dK/dV kernel that
// also adds dQ into that slot with atomics
hipError_t launch_prepare_f32(float* dqkv, float* D, const float* dout, const float* out,
                             const Shape& s, hipStream_t st);
hipError_t launch_dkdvdq_f32(float* dqkv, const float* dout, const float* qkv, const float* lse,
                             const float* D, const Shape& s, hipStream_t st);
// dS block store variant of the fp32 backward: dK/dV also writes dS, dQ reads it
size_t ds_store_floats(const Shape& s);
hipError_t launch_dkdv_ds_f32(float* dqkv, float* dS, const float* dout, const float* qkv,
                              const float* lse, const float* D, const Shape& s, hipStream_t st);
hipError_t launch_dq_ds_f32(float* dqkv, const float* dS, const float* qkv, const Shape& s,
                            hipStream_t st);
// bf16 fused path (bf16 tensors as raw 16-bit patterns)
hipError_t launch_fwd_bf16(uint16_t* out, float* lse, const uint16_t* qkv, const Shape& s,
                           hipStream_t st);
hipError_t launch_prepass_bf16(float* D, const uint16_t* dout, const uint16_t* out,
                               const Shape& s, hipStream_t st);
hipError_t launch_dkdv_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                            const float* lse, const float* D, const Shape& s, hipStream_t st);
hipError_t launch_dq_bf16(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                          const uint16_t* out, const float* lse, const Shape& s, hipStream_t st);
// split-KV forward of the 16-bit path: partial (O, lse) per (Q tile, key
// chunk of chunk_tiles 64-key tiles), then the merge per row
constexpr int kFwdHalfRows = 128;   // rows per Q tile of the 16-bit forward
hipError_t launch_fwd_part_bf16(float* o_parts, float* lse_parts, const uint16_t* qkv,
                                int chunk_tiles, const Shape& s, hipStream_t st);
hipError_t launch_fwd_part_f16(float* o_parts, float* lse_parts, const uint16_t* qkv,
                               int chunk_tiles, const Shape& s, hipStream_t st);
hipError_t launch_merge_split_bf16(uint16_t* out, float* lse, const float* o_parts,
                                   const float* lse_parts, int P, int part_rows, int part_keys,
                                   const Shape& s, hipStream_t st);
hipError_t launch_merge_split_f16(uint16_t* out, float* lse, const float* o_parts,
                                  const float* lse_parts, int P, int part_rows, int part_keys,
                                  const Shape& s, hipStream_t st);
// split backward of the 16-bit path (work: D, dq slabs, dk/dv slabs)
hipError_t launch_bwd_split_bf16(uint16_t* dqkv, float* work, const uint16_t* dout,
                                 const uint16_t* qkv, const uint16_t* out, const float* lse,
                                 int chunk_tiles, const Shape& s, hipStream_t st);
hipError_t launch_bwd_split_f16(uint16_t* dqkv, float* work, const uint16_t* dout,
                                const uint16_t* qkv, const uint16_t* out, const float* lse,
                                int chunk_tiles, const Shape& s, hipStream_t st);
// fp16 fused path (IEEE half tensors as raw 16-bit patterns)
hipError_t launch_fwd_f16(uint16_t* out, float* lse, const uint16_t* qkv, const Shape& s,
                          hipStream_t st);
hipError_t launch_prepass_f16(float* D, const uint16_t* dout, const uint16_t* out, const Shape& s,
                              hipStream_t st);
hipError_t launch_dkdv_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                           const float* lse, const float* D, const Shape& s, hipStream_t st);
hipError_t launch_dq_f16(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                         const uint16_t* out, const float* lse, const Shape& s, hipStream_t st);
// Fused 16-bit backward of short sequences (one workgroup per head), used by
// the fused backward entry points where tiles::bwd_short_applies says so.
inline bool bwd_short_applies(const Shape& s) { return tiles::bwd_short_applies(s.T, s.hs); }
hipError_t launch_bwd_short_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                                 const uint16_t* out, const float* lse, const Shape& s,
                                 hipStream_t st);
hipError_t launch_bwd_short_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                                const uint16_t* out, const float* lse, const Shape& s,
                                hipStream_t st);
// fp8 forward (OCP E4M3 q, k, v as raw bytes; bfloat16 out, fp32 lse)
hipError_t launch_fwd_fp8(uint16_t* out, float* lse, const uint8_t* qkv, const Shape& s,
                          hipStream_t st);
// materialised fp32 path
hipError_t launch_fwd_materialized(float* out, float* preatt, float* att, const float* qkv,
                                   const Shape& s, hipStream_t st);
hipError_t launch_bwd_materialized(float* dqkv, float* dpreatt, float* datt, const float* dout,
                                   const float* qkv, const float* att, const Shape& s,
                                   hipStream_t st);

// decode (one query row per sequence, key ranges merged) and the merge of
// partial (O, lse) results
int decode_range_len(const Shape& s);
size_t decode_workspace_floats(const Shape& s);
hipError_t launch_decode_f32(float* out, float* lse, const float* qkv, float* ws, const Shape& s,
                             hipStream_t st);
hipError_t launch_decode_bf16(uint16_t* out, float* lse, const uint16_t* qkv, float* ws,
                              const Shape& s, hipStream_t st);
hipError_t launch_merge_f32(float* out, float* lse, const float* o_parts, const float* lse_parts,
                            int P, const Shape& s, hipStream_t st);
hipError_t launch_merge_bf16(uint16_t* out, float* lse, const float* o_parts,
                             const float* lse_parts, int P, const Shape& s, hipStream_t st);
hipError_t launch_decode_f16(uint16_t* out, float* lse, const uint16_t* qkv, float* ws,
                             const Shape& s, hipStream_t st);
hipError_t launch_merge_f16(uint16_t* out, float* lse, const float* o_parts,
                            const float* lse_parts, int P, const Shape& s, hipStream_t st);

// projections with fused epilogues (gemm.hip): y = x w^T + bias (+ res),
// x (M, K), w (N, K), bias (N), res and y (M, N), row-major
hipError_t launch_gemm_f32(float* y, const float* x, const float* w, const float* bias,
                           const float* res, int M, int N, int K, hipStream_t st);
hipError_t launch_gemm_bf16(uint16_t* y, const uint16_t* x, const uint16_t* w, const float* bias,
                            const uint16_t* res, int M, int N, int K, hipStream_t st);

// LayerNorm over the rows of an (N, C) matrix (layernorm.hip); the backward
// uses layernorm_workspace_floats(N, C) floats of workspace
int layernorm_col_chunks(int N, int C, int* rows_per_chunk);
size_t layernorm_workspace_floats(int N, int C);
hipError_t launch_layernorm_fwd_f32(float* out, float* mean, float* rstd, const float* inp,
                                    const float* weight, const float* bias, int N, int C,
                                    hipStream_t st);
hipError_t launch_layernorm_fwd_bf16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                                     const float* weight, const float* bias, int N, int C,
                                     hipStream_t st);
hipError_t launch_layernorm_bwd_f32(float* dinp, float* dweight, float* dbias, float* ws,
                                    const float* dout, const float* inp, const float* weight,
                                    const float* mean, const float* rstd, int N, int C,
                                    hipStream_t st);
hipError_t launch_layernorm_fwd_f16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                                    const float* weight, const float* bias, int N, int C,
                                    hipStream_t st);
hipError_t launch_layernorm_bwd_f16(uint16_t* dinp, float* dweight, float* dbias, float* ws,
                                    const uint16_t* dout, const uint16_t* inp, const float* weight,
                                    const float* mean, const float* rstd, int N, int C,
                                    hipStream_t st);
hipError_t launch_layernorm_bwd_bf16(uint16_t* dinp, float* dweight, float* dbias, float* ws,
                                     const uint16_t* dout, const uint16_t* inp,
                                     const float* weight, const float* mean, const float* rstd,
                                     int N, int C, hipStream_t st);

}  // namespace attn
