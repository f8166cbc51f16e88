// gemm.hip -- the two projections on either side of the attention block,
// as matrix-core GEMMs with fused epilogues, for gfx950.
//
//   QKV projection:     qkv[m][n] = sum_k x[m][k] w[n][k] + bias[n]
//   output projection:  y[m][n]   = sum_k a[m][k] w[n][k] + bias[n] + res[m][n]
//
// The first forms Q = X W_Q, K = X W_K, V = X W_V of "Umakini wa kujitegemea,
// kerneli za CUDA na FlashAttention" (section 1) for all heads at once, with
// w the (3C, C) matrix whose rows are the columns of [W_Q | W_K | W_V]: its
// output rows are the packed (B, T, 3C) layout the attention kernels read,
// so no permute follows.  The second is the projection after attention
// with the residual connection of "llm.c 的中文注解-20240423" (section
// 1.15, residual_forward_kernel: out = inp1 + inp2) added in the same
// pass.  Folding the bias add and the residual add into the matrix
// product's store is the kernel fusion of "LLM Systems 10 & 11:
// Accelerating Transformer Training and Inference" (section 1): the
// elementwise passes never read or write the (M, N) matrix again.
//
// gfx950 mapping.  The products are arranged as y^T = w x^T: w rows (k
// contiguous) are the first matrix-core operand and x rows (k contiguous)
// the second, both read from LDS tiles with 16-byte loads, and a lane ends
// with 4 consecutive n of one row m, so bias, residual and the output move
// 4 columns per lane.  fp32 (v_mfma_f32_16x16x4_f32): a workgroup of 4
// waves computes a 128 x 128 tile of y, each wave a 64 x 64 quarter as 4 x 4
// blocks of 16 x 16 accumulators; tiles of w and x stream through LDS in
// steps of 32 k-values, the next step's loaded into registers while the
// current one is used.  bf16 (v_mfma_f32_16x16x32_bf16): 128 x 64 tiles
// with two LDS stages filled by direct loads (below).  Rows past M or N come
// back as zeros from buffer loads bounded by the tile's rows; k-chunks past
// K are predicated or read as zeros (K is a multiple of the 16-byte chunk).
#include "common.hpp"

namespace attn {
namespace {

constexpr int kGThreads = 256;
constexpr int kGM = 128;   // output rows (m) per workgroup
constexpr int kGN = 128;   // output columns (n) per workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, size_t ld_bytes,
                                                            int row0, int rows, int nrows) {
    const int valid = min(nrows - row0, rows);
    const uint32_t num = valid > 0 ? (uint32_t)((size_t)valid * ld_bytes) : 0u;
    const char* p = reinterpret_cast<const char*>(base) + (size_t)row0 * ld_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, (int)num, 0x00020000);
}

// A 128-row x (BK * elem = 128 bytes) tile of 16-byte chunks held in
// registers between its global load and its LDS store: 1024 chunks, 4 per
// thread; chunk e = tid + 256 j is row e / 8, chunk e % 8 of the row.
struct Stage {
    uint4 v[4];
    __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t r, size_t ld_bytes, int kbyte0,
                                          int kbytes, int tid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + kGThreads * j;
            const int row = e >> 3, c = e & 7;
            const int kb = kbyte0 + 16 * c;
            v[j] = make_uint4(0u, 0u, 0u, 0u);
            if (kb < kbytes) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(
                    r, (int)((size_t)row * ld_bytes + kb), 0, 0);
                __builtin_memcpy(&v[j], &x, 16);
            }
        }
    }
    // dense 128-byte LDS rows, chunk c of row r at chunk position c ^ swz(r)
    __device__ __forceinline__ void store_swz(char* lds, int tid) const;
};

struct GLane {
    int tid, w, l, r16, g, wn, wm;
    __device__ GLane() {
        tid = threadIdx.x;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        l = tid & 63;
        r16 = l & 15;
        g = l >> 4;
        wn = w & 1;
        wm = w >> 1;
    }
};

typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));

// bf16 operands, fp32 accumulation, bf16 output (round to nearest even);
// bias fp32, residual bf16.  A workgroup computes a 128 (m) x 64 (n) tile
// of y; wave w takes rows 64 (w >> 1) .. +63 and columns 32 (w & 1) .. +31.
// k steps by 64 through two LDS stages that are filled straight from global
// memory (buffer_load_dwordx4 ... lds: one wave instruction moves 64 lanes x
// 16 bytes into 1 KB of consecutive LDS, lane l into bytes 16l .. 16l + 15),
// so the next step's tiles load while the current one is used, with no
// staging registers and one barrier per step.
constexpr int kBM = 128, kBN = 64, kBK = 64;
constexpr int kBWaves = kBM / 32;              // waves: kBM / 64 along m, 2 along n
constexpr int kBThreads = 64 * kBWaves;
constexpr int kWNB = kBN / 32;   // 16-column blocks per wave

// LDS rows are 128 bytes (64 bf16 of k); chunk c of row r sits at chunk
// position c ^ swz(r).  The LDS has 64 four-byte banks (256 bytes), so two
// rows share a bank period: sixteen lanes reading chunk c of rows r .. r + 15
// (one ds_read_b128 pass) land on sixteen distinct 16-byte bank groups when
// the even rows, and the odd rows, take eight distinct positions each.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ void Stage::store_swz(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid + kGThreads * j;
        const int row = e >> 3, c = e & 7;
        *reinterpret_cast<uint4*>(lds + row * 128 + 16 * (c ^ swz(row))) = v[j];
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Tile of workgroup blockIdx.x.  Workgroups go to the 8 XCDs round robin by
// id; when the row-block count is a multiple of 8, XCD x takes row blocks x,
// x + 8, x + 16, ... with every column block, so each row block of x is
// fetched into one XCD's L2 only (otherwise consecutive tiles of one row
// block land on 8 different XCDs and each pulls it from memory).  Within an
// XCD the row blocks run fastest: the resident workgroups share a few column
// blocks of w while the XCD's rows of x stay in its L2 (with the columns
// fastest, all of w and the current rows outgrew the 4 MB L2 at the QKV
// projection: 6x the compulsory bytes fetched, 46 -> 42-44 us).
__device__ __forceinline__ void xcd_tile(int ntn, int ntm, int& tn, int& tm) {
    const int id = blockIdx.x;
    if (ntm % 8 == 0) {
        const int loc = id >> 3;
        const int nmx = ntm >> 3;   // row blocks per XCD
        tm = (id & 7) + 8 * (loc % nmx);
        tn = loc / nmx;
    } else {
        tn = id % ntn;
        tm = id / ntn;
    }
}

// k bytes kb0 .. kb0 + 127 of rows 0 .. ROWS - 1 of the descriptor's rows
// (rows past its record limit read as zeros) into a ROWS x 128-byte tile;
// chunks at or past kbytes get an offset past every record limit, so they
// are zeros too.  The 4 waves share the ROWS / 8 wave loads.
template <int ROWS>
__device__ __forceinline__ void dma_stage(char* tile, __amdgpu_buffer_rsrc_t r, uint32_t ld, int kb0,
                                          int kbytes, int w, int l) {
    constexpr int NI = ROWS / 8;
    static_assert(NI % kBWaves == 0, "whole wave loads per wave");
#pragma unroll
    for (int k = 0; k < NI / kBWaves; ++k) {
        const int q = w + kBWaves * k;
        const int row = 8 * q + (l >> 3);
        const int kb = kb0 + 16 * ((l & 7) ^ swz(row));
        const uint32_t off = kb < kbytes ? (uint32_t)row * ld + (uint32_t)kb : 0x7FFFFFF0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(tile + 1024 * q), 16, (int)off, 0, 0, 0);
    }
}

template <bool RES>
__global__ __launch_bounds__(kBThreads) void gemm_bf16_kernel(uint16_t* __restrict__ y,
                                                              const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              const float* __restrict__ bias,
                                                              const uint16_t* __restrict__ res,
                                                              int M, int N, int K) {
    // two stages in separate arrays, each indexed only by constants: with one
    // array indexed by the step's parity the compiler would wait for the
    // loads in flight before every LDS read
    // a stage: the x tile, then the w tile
    __shared__ __attribute__((aligned(16))) char S0[(kBM + kBN) * 128];
    __shared__ __attribute__((aligned(16))) char S1[(kBM + kBN) * 128];
    const GLane L;
    const int ntn = (N + kBN - 1) / kBN;
    int tn, tm;
    xcd_tile(ntn, (M + kBM - 1) / kBM, tn, tm);
    const int n0 = tn * kBN, m0 = tm * kBM;
    const uint32_t ldb = (uint32_t)K * 2;
    const __amdgpu_buffer_rsrc_t rw = rows_rsrc(w, ldb, n0, kBN, N);
    const __amdgpu_buffer_rsrc_t rx = rows_rsrc(x, ldb, m0, kBM, M);
    const int kbytes = K * 2;
    const int nsteps = (K + kBK - 1) / kBK;

    f32x4 acc[kWNB][4];
#pragma unroll
    for (int i = 0; i < kWNB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](int s, char* Sn) {
        dma_stage<kBM>(Sn, rx, ldb, s * 2 * kBK, kbytes, L.w, L.l);
        dma_stage<kBN>(Sn + kBM * 128, rw, ldb, s * 2 * kBK, kbytes, L.w, L.l);
    };
    auto compute = [&](const char* Sc) {
        const char* Xc = Sc;
        const char* Wc = Sc + kBM * 128;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int c = 4 * ks + L.g;
            gbf16x8 a[kWNB], b[4];
#pragma unroll
            for (int i = 0; i < kWNB; ++i) {
                const int row = (kBN / 2) * L.wn + 16 * i + L.r16;
                const uint4 v = *reinterpret_cast<const uint4*>(Wc + row * 128 + 16 * (c ^ swz(row)));
                __builtin_memcpy(&a[i], &v, 16);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 64 * L.wm + 16 * j + L.r16;
                const uint4 v = *reinterpret_cast<const uint4*>(Xc + row * 128 + 16 * (c ^ swz(row)));
                __builtin_memcpy(&b[j], &v, 16);
            }
#pragma unroll
            for (int i = 0; i < kWNB; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    auto step = [&](int s, const char* Sc, char* Sn) {
        wait_global_loads();   // this wave's loads of step s (the only ones in flight)
        __syncthreads();       // every wave's loads of step s have landed; step s - 1 is read
        if (s + 1 < nsteps) load(s + 1, Sn);
        compute(Sc);
    };
    load(0, S0);
    for (int s = 0; s < nsteps; s += 2) {
        step(s, S0, S1);
        if (s + 1 < nsteps) step(s + 1, S1, S0);
    }

    // acc[i][j] register q: y[m][n], m = m0 + 64 wm + 16 j + r16,
    // n = n0 + (kBN / 2) wn + 16 i + 4 g + q
#pragma unroll
    for (int i = 0; i < kWNB; ++i) {
        const int n = n0 + (kBN / 2) * L.wn + 16 * i + 4 * L.g;
        if (n >= N) continue;   // N % 4 == 0: the four columns are all in or all out
        const float4 bb = *reinterpret_cast<const float4*>(bias + n);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + 64 * L.wm + 16 * j + L.r16;
            if (m >= M) continue;
            float v[4] = {acc[i][j][0] + bb.x, acc[i][j][1] + bb.y, acc[i][j][2] + bb.z,
                          acc[i][j][3] + bb.w};
            if constexpr (RES) {
                const uint2 rr = *reinterpret_cast<const uint2*>(res + (size_t)m * N + n);
                v[0] += bf16_to_f32((uint16_t)(rr.x & 0xffffu));
                v[1] += bf16_to_f32((uint16_t)(rr.x >> 16));
                v[2] += bf16_to_f32((uint16_t)(rr.y & 0xffffu));
                v[3] += bf16_to_f32((uint16_t)(rr.y >> 16));
            }
            const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            *reinterpret_cast<uint2*>(y + (size_t)m * N + n) = make_uint2(lo, hi);
        }
    }
}

// fp32 operands and output on the fp32 matrix cores.  Within a step of
// BK = 32 k-values, contraction step s pairs k = 8 g + s of both operands
// (lane group g), so each lane's values of a row are 8 contiguous floats.
template <bool RES>
__global__ __launch_bounds__(kGThreads) void gemm_f32_kernel(float* __restrict__ y,
                                                             const float* __restrict__ x,
                                                             const float* __restrict__ w,
                                                             const float* __restrict__ bias,
                                                             const float* __restrict__ res, int M,
                                                             int N, int K) {
    constexpr int BK = 32;               // k per step (128 bytes of a row)
    constexpr int LDF = BK;              // dense 128-byte rows, chunks swizzled
    __shared__ __attribute__((aligned(16))) float Ws[kGN * LDF];
    __shared__ __attribute__((aligned(16))) float Xs[kGM * LDF];
    const GLane L;
    const int ntn = (N + kGN - 1) / kGN;
    int tn, tm;
    xcd_tile(ntn, (M + kGM - 1) / kGM, tn, tm);
    const int n0 = tn * kGN, m0 = tm * kGM;
    const size_t ldb = (size_t)K * 4;
    const __amdgpu_buffer_rsrc_t rw = rows_rsrc(w, ldb, n0, kGN, N);
    const __amdgpu_buffer_rsrc_t rx = rows_rsrc(x, ldb, m0, kGM, M);

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Stage sw, sx;
    const int kbytes = K * 4;
    sw.fetch(rw, ldb, 0, kbytes, L.tid);
    sx.fetch(rx, ldb, 0, kbytes, L.tid);
    wait_global_loads();
    for (int k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();
        sw.store_swz(reinterpret_cast<char*>(Ws), L.tid);
        sx.store_swz(reinterpret_cast<char*>(Xs), L.tid);
        __syncthreads();
        if (k0 + BK < K) {
            sw.fetch(rw, ldb, (k0 + BK) * 4, kbytes, L.tid);
            sx.fetch(rx, ldb, (k0 + BK) * 4, kbytes, L.tid);
        }
        float a[4][8], b[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra = 64 * L.wn + 16 * i + L.r16, rb = 64 * L.wm + 16 * i + L.r16;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float4 va = *reinterpret_cast<const float4*>(
                    Ws + ra * LDF + 4 * ((2 * L.g + h) ^ swz(ra)));
                const float4 vb = *reinterpret_cast<const float4*>(
                    Xs + rb * LDF + 4 * ((2 * L.g + h) ^ swz(rb)));
                a[i][4 * h + 0] = va.x;
                a[i][4 * h + 1] = va.y;
                a[i][4 * h + 2] = va.z;
                a[i][4 * h + 3] = va.w;
                b[i][4 * h + 0] = vb.x;
                b[i][4 * h + 1] = vb.y;
                b[i][4 * h + 2] = vb.z;
                b[i][4 * h + 3] = vb.w;
            }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f32(a[i][s], b[j][s], acc[i][j]);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = n0 + 64 * L.wn + 16 * i + 4 * L.g;
        if (n >= N) continue;
        const float4 bb = *reinterpret_cast<const float4*>(bias + n);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + 64 * L.wm + 16 * j + L.r16;
            if (m >= M) continue;
            float4 v = make_float4(acc[i][j][0] + bb.x, acc[i][j][1] + bb.y, acc[i][j][2] + bb.z,
                                   acc[i][j][3] + bb.w);
            if constexpr (RES) {
                const float4 rr = *reinterpret_cast<const float4*>(res + (size_t)m * N + n);
                v.x += rr.x;
                v.y += rr.y;
                v.z += rr.z;
                v.w += rr.w;
            }
            *reinterpret_cast<float4*>(y + (size_t)m * N + n) = v;
        }
    }
}

long long gemm_grid(int M, int N) {
    return (long long)((N + kGN - 1) / kGN) * ((M + kGM - 1) / kGM);
}

}  // namespace

hipError_t launch_gemm_f32(float* y, const float* x, const float* w, const float* bias,
                           const float* res, int M, int N, int K, hipStream_t st) {
    const long long grid = gemm_grid(M, N);
    if (grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (res)
        hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)grid), dim3(kGThreads), 0, st, y, x,
                           w, bias, res, M, N, K);
    else
        hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)grid), dim3(kGThreads), 0, st, y, x,
                           w, bias, res, M, N, K);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(uint16_t* y, const uint16_t* x, const uint16_t* w, const float* bias,
                            const uint16_t* res, int M, int N, int K, hipStream_t st) {
    const long long grid = (long long)((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
    if (grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (res)
        hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3((unsigned)grid), dim3(kBThreads), 0, st, y, x,
                           w, bias, res, M, N, K);
    else
        hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3((unsigned)grid), dim3(kBThreads), 0, st, y, x,
                           w, bias, res, M, N, K);
    return hipGetLastError();
}

}  // namespace attn
