// api.hip -- the C ABI of libattn: argument checks, per-thread stream and
// error state, the per-device backward workspace, and dispatch to the
// kernel launchers.  Declarations and semantics: include/libattn.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/libattn.h"
#include "common.hpp"

namespace {

thread_local hipStream_t g_stream = nullptr;
thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return ATTN_OK;
}

// A byte range [p, p + n) of one tensor argument.
struct Span {
    const void* p;
    size_t n;
    const char* name;
};

bool overlaps(const Span& a, const Span& b) {
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Checks shared by every entry point.  `outs` must not overlap each other or
// any of `ins`.  `mat` adds the T*T limit of the materialised calls.
int check_args(int B, int T, int C, int NH, int causal, const Span* outs, int nout,
               const Span* ins, int nin, bool mat) {
    for (int i = 0; i < nout; ++i)
        if (!outs[i].p) return fail(ATTN_EINVAL, "%s is NULL", outs[i].name);
    for (int i = 0; i < nin; ++i)
        if (!ins[i].p) return fail(ATTN_EINVAL, "%s is NULL", ins[i].name);
    if (B < 1 || T < 1 || NH < 1)
        return fail(ATTN_EINVAL, "B, T and NH must be >= 1 (got B=%d T=%d NH=%d)", B, T, NH);
    if (C < NH || C % NH != 0)
        return fail(ATTN_EINVAL, "C=%d must be a positive multiple of NH=%d", C, NH);
    if (causal != 0 && causal != 1) return fail(ATTN_EINVAL, "causal must be 0 or 1 (got %d)", causal);
    if ((long long)T * 3 * C >= (1LL << 31))
        return fail(ATTN_EINVAL, "T*3C = %lld exceeds the 32-bit in-batch offset range",
                    (long long)T * 3 * C);
    // the kernels' buffer loads address one 64-row tile of fp32 rows (3C
    // floats apart) with 32-bit byte offsets
    if ((long long)64 * 3 * C * 4 >= (1LL << 32))
        return fail(ATTN_EINVAL, "C=%d too large: a 64-row tile of (B,T,3C) rows exceeds the 32-bit buffer offset range", C);
    if (mat && (long long)T * T >= (1LL << 31))
        return fail(ATTN_EINVAL, "T*T = %lld exceeds the 32-bit offset range", (long long)T * T);
    if ((long long)B * NH * (long long)((T + 63) / 64) >= (1LL << 31))
        return fail(ATTN_EINVAL, "too many tiles for one launch");
    for (int i = 0; i < nout; ++i)
        if ((uintptr_t)outs[i].p % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", outs[i].name);
    for (int i = 0; i < nin; ++i)
        if ((uintptr_t)ins[i].p % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", ins[i].name);
    for (int i = 0; i < nout; ++i) {
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(ATTN_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(ATTN_EINVAL, "output %s overlaps input %s", outs[i].name, ins[j].name);
    }
    const int hs = C / NH;
    if (hs != 16 && hs != 32 && hs != 64 && hs != 128)
        return fail(ATTN_EUNSUPPORTED, "head size C/NH = %d is not one of 16, 32, 64, 128", hs);
    return ATTN_OK;
}

attn::Shape shape_of(int B, int T, int C, int NH, int causal) {
    attn::Shape s;
    s.B = B;
    s.T = T;
    s.C = C;
    s.NH = NH;
    s.hs = C / NH;
    s.causal = causal;
    return s;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// ---- per-device grow-only workspace (D for the backward, decode partials,
// LayerNorm column partials) ----
// A call that needs more than the current buffer allocates a larger one and
// keeps the old one on a retired list instead of freeing it: work queued
// earlier on any stream, or a HIP graph captured earlier, may still read or
// write the old buffer.  Only attn_release frees buffers.  Growing therefore
// never synchronises the device.
constexpr int kMaxDevices = 64;
std::mutex g_ws_mutex;
void* g_ws_ptr[kMaxDevices] = {};
size_t g_ws_bytes[kMaxDevices] = {};
std::vector<void*> g_ws_retired[kMaxDevices];

int workspace(size_t bytes, float** out) {
    // ATTN_TEST_FAIL_ALLOC=1 makes the allocation fail before any HIP call,
    // so the error path can be exercised on a host without a GPU.
    const char* forced = getenv("ATTN_TEST_FAIL_ALLOC");
    if (forced && forced[0] == '1') return fail(ATTN_EHIP, "workspace allocation failed (forced)");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_EHIP, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (g_ws_bytes[dev] < bytes) {
        // grow by at least half, so a slowly rising shape retires few buffers
        const size_t want = bytes > g_ws_bytes[dev] + g_ws_bytes[dev] / 2
                                ? bytes : g_ws_bytes[dev] + g_ws_bytes[dev] / 2;
        void* p = nullptr;
        e = hipMalloc(&p, want);
        if (e != hipSuccess) {
            (void)hipGetLastError();   // a failed allocation must not surface at the next launch
            return fail(ATTN_EHIP, "hipMalloc(%zu): %s", want, hipGetErrorString(e));
        }
        if (g_ws_ptr[dev]) g_ws_retired[dev].push_back(g_ws_ptr[dev]);
        g_ws_ptr[dev] = p;
        g_ws_bytes[dev] = want;
    }
    *out = (float*)g_ws_ptr[dev];
    return ATTN_OK;
}

size_t nbytes(long long elems, size_t elem) { return (size_t)elems * elem; }

// ---- fixed scratch for attn_backward_noalloc ----
// A file-scope device array of kNoAllocScratchFloats floats: every GPU the
// library runs on holds its own copy from module load until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory, so kernels are only ever handed the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchFloats = (size_t)4 << 20;   // 16 MiB: B*NH*T <= 4194304
__device__ __align__(256) float scratch[kNoAllocScratchFloats];
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_device(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_EHIP, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(ATTN_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = (float*)p;
    }
    *out = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_set_stream(void* hip_stream) {
    g_stream = (hipStream_t)hip_stream;
    return ok();
}

const char* attn_last_error(void) { return g_err; }

void attn_release(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) cur = -1;
    for (int d = 0; d < kMaxDevices; ++d) {
        if (!g_ws_ptr[d] && g_ws_retired[d].empty()) continue;
        if (hipSetDevice(d) == hipSuccess) {
            if (g_ws_ptr[d]) (void)hipFree(g_ws_ptr[d]);
            for (void* p : g_ws_retired[d]) (void)hipFree(p);
        }
        g_ws_ptr[d] = nullptr;
        g_ws_bytes[d] = 0;
        g_ws_retired[d].clear();
    }
    if (cur >= 0) (void)hipSetDevice(cur);
}

int attn_forward(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                 int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes(BT * C, 4), "out"}, {lse, nbytes(BT * NH, 4), "lse"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 4), "qkv"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 1, false);
    if (rc) return rc;
    return launched(attn::launch_fwd_f32(out, lse, qkv, shape_of(B, T, C, NH, causal), g_stream),
                    "attn_forward launch");
}

int attn_backward(float* dqkv, const float* dout, const float* qkv, const float* out,
                  const float* lse, int B, int T, int C, int NH, int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"},
                        {qkv, nbytes(BT * 3 * C, 4), "qkv"},
                        {out, nbytes(BT * C, 4), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    // the pre-pass (D = dO . O per row, dQ slot cleared), then one kernel
    // for dK, dV and dQ (dQ added with atomics); the only workspace is D,
    // B*NH*T floats
    float* D = nullptr;
    rc = workspace(nbytes(BT * NH, 4), &D);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    hipError_t e = attn::launch_prepare_f32(dqkv, D, dout, out, s, g_stream);
    if (e == hipSuccess) e = attn::launch_dkdvdq_f32(dqkv, dout, qkv, lse, D, s, g_stream);
    return launched(e, "attn_backward launch");
}

int attn_backward_noalloc(float* dqkv, const float* dout, const float* qkv, const float* out,
                          const float* lse, int B, int T, int C, int NH, int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"},
                        {qkv, nbytes(BT * 3 * C, 4), "qkv"},
                        {out, nbytes(BT * C, 4), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    if ((unsigned long long)BT * NH > kNoAllocScratchFloats)
        return fail(ATTN_EINVAL,
                    "attn_backward_noalloc: B*NH*T = %lld exceeds the fixed scratch of %zu floats",
                    BT * NH, kNoAllocScratchFloats);
    // D lives in the fixed scratch: written in full by the pre-pass before
    // the dK/dV/dQ kernel reads it, so nothing needs clearing
    float* D = nullptr;
    rc = scratch_for_device(&D);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    hipError_t e = attn::launch_prepare_f32(dqkv, D, dout, out, s, g_stream);
    if (e == hipSuccess) e = attn::launch_dkdvdq_f32(dqkv, dout, qkv, lse, D, s, g_stream);
    return launched(e, "attn_backward_noalloc launch");
}

uint64_t attn_backward_ds_bytes(int B, int T, int C, int NH, int causal) {
    // the same checks as the calls that use the store, on placeholder pointers
    static const float dummy[4] __attribute__((aligned(16))) = {};
    const Span none[] = {{dummy, 0, "none"}};
    if (check_args(B, T, C, NH, causal, none, 0, none, 0, false) != ATTN_OK) return 0;
    ok();
    return (uint64_t)attn::ds_store_floats(shape_of(B, T, C, NH, causal)) * 4;
}

int attn_backward_dkdv_ds(float* dqkv, float* dS, const float* dout, const float* qkv,
                          const float* lse, const float* D, int B, int T, int C, int NH,
                          int causal) {
    const long long BT = (long long)B * T;
    // dS enters the shared checks with size 0 (null and alignment); its
    // extent is known, and checked for overlaps, once the dimensions pass
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}, {dS, 0, "dS"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"},
                        {qkv, nbytes(BT * 3 * C, 4), "qkv"},
                        {lse, nbytes(BT * NH, 4), "lse"},
                        {D, nbytes(BT * NH, 4), "D"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 4, false);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    const Span ds = {dS, attn::ds_store_floats(s) * 4, "dS"};
    if (overlaps(ds, outs[0])) return fail(ATTN_EINVAL, "dS overlaps dqkv");
    for (const Span& in : ins)
        if (overlaps(ds, in)) return fail(ATTN_EINVAL, "output dS overlaps input %s", in.name);
    return launched(attn::launch_dkdv_ds_f32(dqkv, dS, dout, qkv, lse, D, s, g_stream),
                    "attn_backward_dkdv_ds launch");
}

int attn_backward_dq_ds(float* dqkv, const float* dS, const float* qkv, int B, int T, int C,
                        int NH, int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}};
    const Span ins[] = {{dS, 0, "dS"}, {qkv, nbytes(BT * 3 * C, 4), "qkv"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 2, false);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    const Span ds = {dS, attn::ds_store_floats(s) * 4, "dS"};
    if (overlaps(outs[0], ds)) return fail(ATTN_EINVAL, "output dqkv overlaps input dS");
    return launched(attn::launch_dq_ds_f32(dqkv, dS, qkv, s, g_stream),
                    "attn_backward_dq_ds launch");
}

int attn_backward_preprocess(float* D, const float* dout, const float* out, int B, int T, int C,
                             int NH) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{D, nbytes(BT * NH, 4), "D"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"}, {out, nbytes(BT * C, 4), "out"}};
    int rc = check_args(B, T, C, NH, 0, outs, 1, ins, 2, false);
    if (rc) return rc;
    return launched(attn::launch_prepass_f32(D, dout, out, shape_of(B, T, C, NH, 0), g_stream),
                    "attn_backward_preprocess launch");
}

int attn_backward_prepare(float* dqkv, float* D, const float* dout, const float* out, int B,
                          int T, int C, int NH) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}, {D, nbytes(BT * NH, 4), "D"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"}, {out, nbytes(BT * C, 4), "out"}};
    int rc = check_args(B, T, C, NH, 0, outs, 2, ins, 2, false);
    if (rc) return rc;
    return launched(attn::launch_prepare_f32(dqkv, D, dout, out, shape_of(B, T, C, NH, 0),
                                             g_stream),
                    "attn_backward_prepare launch");
}

int attn_backward_dkdvdq(float* dqkv, const float* dout, const float* qkv, const float* lse,
                         const float* D, int B, int T, int C, int NH, int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"},
                        {qkv, nbytes(BT * 3 * C, 4), "qkv"},
                        {lse, nbytes(BT * NH, 4), "lse"},
                        {D, nbytes(BT * NH, 4), "D"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    return launched(attn::launch_dkdvdq_f32(dqkv, dout, qkv, lse, D,
                                            shape_of(B, T, C, NH, causal), g_stream),
                    "attn_backward_dkdvdq launch");
}

int attn_backward_dkdv(float* dqkv, const float* dout, const float* qkv, const float* lse,
                       const float* D, int B, int T, int C, int NH, int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"},
                        {qkv, nbytes(BT * 3 * C, 4), "qkv"},
                        {lse, nbytes(BT * NH, 4), "lse"},
                        {D, nbytes(BT * NH, 4), "D"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    return launched(attn::launch_dkdv_f32(dqkv, dout, qkv, lse, D, shape_of(B, T, C, NH, causal),
                                          g_stream),
                    "attn_backward_dkdv launch");
}

int attn_backward_dq(float* dqkv, float* D, const float* dout, const float* qkv, const float* out,
                     const float* lse, int B, int T, int C, int NH, int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"}, {D, nbytes(BT * NH, 4), "D"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"},
                        {qkv, nbytes(BT * 3 * C, 4), "qkv"},
                        {out, nbytes(BT * C, 4), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 4, false);
    if (rc) return rc;
    return launched(attn::launch_dq_f32(dqkv, D, dout, qkv, out, lse,
                                        shape_of(B, T, C, NH, causal), g_stream),
                    "attn_backward_dq launch");
}

int attn_forward_bf16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T, int C, int NH,
                      int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes(BT * C, 2), "out"}, {lse, nbytes(BT * NH, 4), "lse"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 2), "qkv"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 1, false);
    if (rc) return rc;
    return launched(attn::launch_fwd_bf16(out, lse, qkv, shape_of(B, T, C, NH, causal), g_stream),
                    "attn_forward_bf16 launch");
}

int attn_forward_fp8(uint16_t* out, float* lse, const uint8_t* qkv, int B, int T, int C, int NH,
                     int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes(BT * C, 2), "out"}, {lse, nbytes(BT * NH, 4), "lse"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 1), "qkv"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 1, false);
    if (rc) return rc;
    return launched(attn::launch_fwd_fp8(out, lse, qkv, shape_of(B, T, C, NH, causal), g_stream),
                    "attn_forward_fp8 launch");
}

int attn_backward_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                       const uint16_t* out, const float* lse, int B, int T, int C, int NH,
                       int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 2), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"},
                        {qkv, nbytes(BT * 3 * C, 2), "qkv"},
                        {out, nbytes(BT * C, 2), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    if (attn::bwd_short_applies(s))   // one fused kernel, no workspace
        return launched(attn::launch_bwd_short_bf16(dqkv, dout, qkv, out, lse, s, g_stream),
                        "attn_backward_bf16 launch");
    float* D = nullptr;
    rc = workspace(nbytes(BT * NH, 4), &D);
    if (rc) return rc;
    hipError_t e = attn::launch_dq_bf16(dqkv, D, dout, qkv, out, lse, s, g_stream);
    if (e == hipSuccess) e = attn::launch_dkdv_bf16(dqkv, dout, qkv, lse, D, s, g_stream);
    return launched(e, "attn_backward_bf16 launch");
}

}  // extern "C"

namespace {
// Split-KV forward geometry: key chunks of `chunk` keys (a multiple of 64)
// over Q tiles of attn::kFwdHalfRows rows.
long long splitkv_items(const attn::Shape& s, int chunk_tiles) {
    const int BM = attn::kFwdHalfRows;
    const int nqt = (s.T + BM - 1) / BM, nkt = (s.T + 63) / 64;
    long long per_head = 0;
    for (int i = 0; i < nqt; ++i) {
        const int kt = s.causal ? std::min(nkt, ((i + 1) * BM + 63) / 64) : nkt;
        per_head += (kt + chunk_tiles - 1) / chunk_tiles;
    }
    return per_head * s.B * s.NH;
}

// The chunk the library picks: the longest power-of-two number of 64-key
// tiles (at least 2) that still gives a workgroup per CU; the whole key
// range (no split) when the unsplit grid already does.  (Two long-context
// heads, T = 8192: 2048-key chunks, 320 workgroups, measured faster than
// 1024-key ones, 576 workgroups, whose partial results cost the merge more.)
int splitkv_auto_chunk(const attn::Shape& s) {
    const long long want = (long long)attn::device_cu_count();
    const int nkt = (s.T + 63) / 64;
    int best = 2;
    for (int ct = 2; ct < 2 * nkt; ct *= 2)
        if (splitkv_items(s, ct) >= want) best = ct;
    if (splitkv_items(s, nkt) >= want) best = nkt;
    return std::min(best, nkt) * 64;
}

size_t splitkv_parts(const attn::Shape& s, int chunk) {
    return (size_t)(((s.T + 63) / 64 + chunk / 64 - 1) / (chunk / 64));
}

size_t splitkv_floats(const attn::Shape& s, int chunk) {
    const size_t P = splitkv_parts(s, chunk);
    return P * ((size_t)s.B * s.T * s.C + (size_t)s.B * s.NH * s.T);
}

// Split backward work: D (B*NH*T floats, rounded up to 64), then the dq
// slabs (P of B*T*C floats) and the dk/dv slabs (P of B*T*2C floats).
size_t bwd_split_floats(const attn::Shape& s, int chunk) {
    const size_t P = splitkv_parts(s, chunk);
    const size_t d = ((size_t)s.B * s.NH * s.T + 63) & ~(size_t)63;
    return P <= 1 ? d : d + 3 * P * (size_t)s.B * s.T * s.C;
}

int check_chunk(int kv_chunk) {
    if (kv_chunk < 0 || kv_chunk % 64 != 0)
        return fail(ATTN_EINVAL, "kv_chunk must be 0 or a positive multiple of 64 (got %d)",
                    kv_chunk);
    return ATTN_OK;
}

int forward_splitkv_any(uint16_t* out, float* lse, const uint16_t* qkv, float* work, int B,
                        int T, int C, int NH, int causal, int kv_chunk, bool f16) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes(BT * C, 2), "out"}, {lse, nbytes(BT * NH, 4), "lse"},
                         {work, 0, "work"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 2), "qkv"}};
    int rc = check_args(B, T, C, NH, causal, outs, 3, ins, 1, false);
    if (rc) return rc;
    if ((rc = check_chunk(kv_chunk))) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    const int chunk = kv_chunk ? std::min(kv_chunk, (T + 63) / 64 * 64) : splitkv_auto_chunk(s);
    const size_t P = splitkv_parts(s, chunk);
    if (P <= 1)   // no split: the plain forward, the work buffer untouched
        return launched(f16 ? attn::launch_fwd_f16(out, lse, qkv, s, g_stream)
                            : attn::launch_fwd_bf16(out, lse, qkv, s, g_stream),
                        "attn_forward_splitkv launch");
    const Span ws = {work, splitkv_floats(s, chunk) * 4, "work"};
    if (overlaps(ws, outs[0]) || overlaps(ws, outs[1]) || overlaps(ws, ins[0]))
        return fail(ATTN_EINVAL, "work overlaps another tensor argument");
    if ((unsigned long long)P * BT * C >= (1ULL << 62)) return fail(ATTN_EINVAL, "work too large");
    float* o_parts = work;
    float* l_parts = work + P * (size_t)BT * C;
    hipError_t e = f16 ? attn::launch_fwd_part_f16(o_parts, l_parts, qkv, chunk / 64, s, g_stream)
                       : attn::launch_fwd_part_bf16(o_parts, l_parts, qkv, chunk / 64, s, g_stream);
    if (e == hipSuccess)
        e = f16 ? attn::launch_merge_split_f16(out, lse, o_parts, l_parts, (int)P,
                                               attn::kFwdHalfRows, chunk, s, g_stream)
                : attn::launch_merge_split_bf16(out, lse, o_parts, l_parts, (int)P,
                                                attn::kFwdHalfRows, chunk, s, g_stream);
    return launched(e, "attn_forward_splitkv launch");
}

int backward_splitkv_any(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                         const uint16_t* out, const float* lse, float* work, int B, int T, int C,
                         int NH, int causal, int kv_chunk, bool f16) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 2), "dqkv"}, {work, 0, "work"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"},
                        {qkv, nbytes(BT * 3 * C, 2), "qkv"},
                        {out, nbytes(BT * C, 2), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 4, false);
    if (rc) return rc;
    if ((rc = check_chunk(kv_chunk))) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    const int chunk = kv_chunk ? std::min(kv_chunk, (T + 63) / 64 * 64) : splitkv_auto_chunk(s);
    const Span ws = {work, bwd_split_floats(s, chunk) * 4, "work"};
    if (overlaps(ws, outs[0])) return fail(ATTN_EINVAL, "work overlaps dqkv");
    for (const Span& in : ins)
        if (overlaps(ws, in)) return fail(ATTN_EINVAL, "work overlaps input %s", in.name);
    hipError_t e;
    if (splitkv_parts(s, chunk) <= 1) {   // no split: the two stages, D in work
        e = f16 ? attn::launch_dq_f16(dqkv, work, dout, qkv, out, lse, s, g_stream)
                : attn::launch_dq_bf16(dqkv, work, dout, qkv, out, lse, s, g_stream);
        if (e == hipSuccess)
            e = f16 ? attn::launch_dkdv_f16(dqkv, dout, qkv, lse, work, s, g_stream)
                    : attn::launch_dkdv_bf16(dqkv, dout, qkv, lse, work, s, g_stream);
    } else {
        e = f16 ? attn::launch_bwd_split_f16(dqkv, work, dout, qkv, out, lse, chunk / 64, s, g_stream)
                : attn::launch_bwd_split_bf16(dqkv, work, dout, qkv, out, lse, chunk / 64, s, g_stream);
    }
    return launched(e, "attn_backward_splitkv launch");
}
}  // namespace

extern "C" {

uint64_t attn_backward_splitkv_bytes(int B, int T, int C, int NH, int causal, int kv_chunk) {
    static const float dummy[4] __attribute__((aligned(16))) = {};
    const Span none[] = {{dummy, 0, "none"}};
    if (check_args(B, T, C, NH, causal, none, 0, none, 0, false) != ATTN_OK) return 0;
    if (check_chunk(kv_chunk) != ATTN_OK) return 0;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    const int chunk = kv_chunk ? std::min(kv_chunk, (T + 63) / 64 * 64) : splitkv_auto_chunk(s);
    ok();
    return (uint64_t)bwd_split_floats(s, chunk) * 4;
}

int attn_backward_splitkv_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                               const uint16_t* out, const float* lse, float* work, int B, int T,
                               int C, int NH, int causal, int kv_chunk) {
    return backward_splitkv_any(dqkv, dout, qkv, out, lse, work, B, T, C, NH, causal, kv_chunk,
                                false);
}

int attn_backward_splitkv_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                              const uint16_t* out, const float* lse, float* work, int B, int T,
                              int C, int NH, int causal, int kv_chunk) {
    return backward_splitkv_any(dqkv, dout, qkv, out, lse, work, B, T, C, NH, causal, kv_chunk,
                                true);
}

int attn_forward_splitkv_chunk(int B, int T, int C, int NH, int causal) {
    static const float dummy[4] __attribute__((aligned(16))) = {};
    const Span none[] = {{dummy, 0, "none"}};
    int rc = check_args(B, T, C, NH, causal, none, 0, none, 0, false);
    if (rc) return rc;
    ok();
    return splitkv_auto_chunk(shape_of(B, T, C, NH, causal));
}

uint64_t attn_forward_splitkv_bytes(int B, int T, int C, int NH, int causal, int kv_chunk) {
    static const float dummy[4] __attribute__((aligned(16))) = {};
    const Span none[] = {{dummy, 0, "none"}};
    if (check_args(B, T, C, NH, causal, none, 0, none, 0, false) != ATTN_OK) return 0;
    if (check_chunk(kv_chunk) != ATTN_OK) return 0;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    const int chunk = kv_chunk ? std::min(kv_chunk, (T + 63) / 64 * 64) : splitkv_auto_chunk(s);
    ok();
    if (splitkv_parts(s, chunk) <= 1) return 0;
    return (uint64_t)splitkv_floats(s, chunk) * 4;
}

int attn_forward_splitkv_bf16(uint16_t* out, float* lse, const uint16_t* qkv, float* work, int B,
                              int T, int C, int NH, int causal, int kv_chunk) {
    return forward_splitkv_any(out, lse, qkv, work, B, T, C, NH, causal, kv_chunk, false);
}

int attn_forward_splitkv_f16(uint16_t* out, float* lse, const uint16_t* qkv, float* work, int B,
                             int T, int C, int NH, int causal, int kv_chunk) {
    return forward_splitkv_any(out, lse, qkv, work, B, T, C, NH, causal, kv_chunk, true);
}

int attn_backward_preprocess_bf16(float* D, const uint16_t* dout, const uint16_t* out, int B,
                                  int T, int C, int NH) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{D, nbytes(BT * NH, 4), "D"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"}, {out, nbytes(BT * C, 2), "out"}};
    int rc = check_args(B, T, C, NH, 0, outs, 1, ins, 2, false);
    if (rc) return rc;
    return launched(attn::launch_prepass_bf16(D, dout, out, shape_of(B, T, C, NH, 0), g_stream),
                    "attn_backward_preprocess_bf16 launch");
}

int attn_backward_dkdv_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                            const float* lse, const float* D, int B, int T, int C, int NH,
                            int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 2), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"},
                        {qkv, nbytes(BT * 3 * C, 2), "qkv"},
                        {lse, nbytes(BT * NH, 4), "lse"},
                        {D, nbytes(BT * NH, 4), "D"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    return launched(attn::launch_dkdv_bf16(dqkv, dout, qkv, lse, D, shape_of(B, T, C, NH, causal),
                                           g_stream),
                    "attn_backward_dkdv_bf16 launch");
}

int attn_backward_dq_bf16(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                          const uint16_t* out, const float* lse, int B, int T, int C, int NH,
                          int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 2), "dqkv"}, {D, nbytes(BT * NH, 4), "D"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"},
                        {qkv, nbytes(BT * 3 * C, 2), "qkv"},
                        {out, nbytes(BT * C, 2), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 4, false);
    if (rc) return rc;
    return launched(attn::launch_dq_bf16(dqkv, D, dout, qkv, out, lse,
                                         shape_of(B, T, C, NH, causal), g_stream),
                    "attn_backward_dq_bf16 launch");
}

int attn_forward_f16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T, int C, int NH,
                      int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes(BT * C, 2), "out"}, {lse, nbytes(BT * NH, 4), "lse"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 2), "qkv"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 1, false);
    if (rc) return rc;
    return launched(attn::launch_fwd_f16(out, lse, qkv, shape_of(B, T, C, NH, causal), g_stream),
                    "attn_forward_f16 launch");
}

int attn_backward_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                       const uint16_t* out, const float* lse, int B, int T, int C, int NH,
                       int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 2), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"},
                        {qkv, nbytes(BT * 3 * C, 2), "qkv"},
                        {out, nbytes(BT * C, 2), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, causal);
    if (attn::bwd_short_applies(s))   // one fused kernel, no workspace
        return launched(attn::launch_bwd_short_f16(dqkv, dout, qkv, out, lse, s, g_stream),
                        "attn_backward_f16 launch");
    float* D = nullptr;
    rc = workspace(nbytes(BT * NH, 4), &D);
    if (rc) return rc;
    hipError_t e = attn::launch_dq_f16(dqkv, D, dout, qkv, out, lse, s, g_stream);
    if (e == hipSuccess) e = attn::launch_dkdv_f16(dqkv, dout, qkv, lse, D, s, g_stream);
    return launched(e, "attn_backward_f16 launch");
}

int attn_backward_preprocess_f16(float* D, const uint16_t* dout, const uint16_t* out, int B,
                                  int T, int C, int NH) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{D, nbytes(BT * NH, 4), "D"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"}, {out, nbytes(BT * C, 2), "out"}};
    int rc = check_args(B, T, C, NH, 0, outs, 1, ins, 2, false);
    if (rc) return rc;
    return launched(attn::launch_prepass_f16(D, dout, out, shape_of(B, T, C, NH, 0), g_stream),
                    "attn_backward_preprocess_f16 launch");
}

int attn_backward_dkdv_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                            const float* lse, const float* D, int B, int T, int C, int NH,
                            int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 2), "dqkv"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"},
                        {qkv, nbytes(BT * 3 * C, 2), "qkv"},
                        {lse, nbytes(BT * NH, 4), "lse"},
                        {D, nbytes(BT * NH, 4), "D"}};
    int rc = check_args(B, T, C, NH, causal, outs, 1, ins, 4, false);
    if (rc) return rc;
    return launched(attn::launch_dkdv_f16(dqkv, dout, qkv, lse, D, shape_of(B, T, C, NH, causal),
                                           g_stream),
                    "attn_backward_dkdv_f16 launch");
}

int attn_backward_dq_f16(uint16_t* dqkv, float* D, const uint16_t* dout, const uint16_t* qkv,
                          const uint16_t* out, const float* lse, int B, int T, int C, int NH,
                          int causal) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 2), "dqkv"}, {D, nbytes(BT * NH, 4), "D"}};
    const Span ins[] = {{dout, nbytes(BT * C, 2), "dout"},
                        {qkv, nbytes(BT * 3 * C, 2), "qkv"},
                        {out, nbytes(BT * C, 2), "out"},
                        {lse, nbytes(BT * NH, 4), "lse"}};
    int rc = check_args(B, T, C, NH, causal, outs, 2, ins, 4, false);
    if (rc) return rc;
    return launched(attn::launch_dq_f16(dqkv, D, dout, qkv, out, lse,
                                         shape_of(B, T, C, NH, causal), g_stream),
                    "attn_backward_dq_f16 launch");
}

int attn_forward_materialized(float* out, float* preatt, float* att, const float* qkv, int B,
                              int T, int C, int NH, int causal) {
    const long long BT = (long long)B * T;
    const long long M = (long long)B * NH * T * T;
    const Span outs[] = {{out, nbytes(BT * C, 4), "out"},
                         {preatt, nbytes(M, 4), "preatt"},
                         {att, nbytes(M, 4), "att"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 4), "qkv"}};
    int rc = check_args(B, T, C, NH, causal, outs, 3, ins, 1, true);
    if (rc) return rc;
    return launched(attn::launch_fwd_materialized(out, preatt, att, qkv,
                                                  shape_of(B, T, C, NH, causal), g_stream),
                    "attn_forward_materialized launch");
}

int attn_backward_materialized(float* dqkv, float* dpreatt, float* datt, const float* dout,
                               const float* qkv, const float* att, int B, int T, int C, int NH,
                               int causal) {
    const long long BT = (long long)B * T;
    const long long M = (long long)B * NH * T * T;
    const Span outs[] = {{dqkv, nbytes(BT * 3 * C, 4), "dqkv"},
                         {dpreatt, nbytes(M, 4), "dpreatt"},
                         {datt, nbytes(M, 4), "datt"}};
    const Span ins[] = {{dout, nbytes(BT * C, 4), "dout"},
                        {qkv, nbytes(BT * 3 * C, 4), "qkv"},
                        {att, nbytes(M, 4), "att"}};
    int rc = check_args(B, T, C, NH, causal, outs, 3, ins, 3, true);
    if (rc) return rc;
    return launched(attn::launch_bwd_materialized(dqkv, dpreatt, datt, dout, qkv, att,
                                                  shape_of(B, T, C, NH, causal), g_stream),
                    "attn_backward_materialized launch");
}

int attn_decode(float* out, float* lse, const float* qkv, int B, int T, int C, int NH) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes((long long)B * C, 4), "out"},
                         {lse, nbytes((long long)B * NH, 4), "lse"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 4), "qkv"}};
    int rc = check_args(B, T, C, NH, 0, outs, 2, ins, 1, false);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, 0);
    float* ws = nullptr;
    rc = workspace(attn::decode_workspace_floats(s) * 4, &ws);
    if (rc) return rc;
    return launched(attn::launch_decode_f32(out, lse, qkv, ws, s, g_stream), "attn_decode launch");
}

int attn_decode_bf16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T, int C, int NH) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes((long long)B * C, 2), "out"},
                         {lse, nbytes((long long)B * NH, 4), "lse"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 2), "qkv"}};
    int rc = check_args(B, T, C, NH, 0, outs, 2, ins, 1, false);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, 0);
    float* ws = nullptr;
    rc = workspace(attn::decode_workspace_floats(s) * 4, &ws);
    if (rc) return rc;
    return launched(attn::launch_decode_bf16(out, lse, qkv, ws, s, g_stream),
                    "attn_decode_bf16 launch");
}

int attn_decode_f16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T, int C, int NH) {
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes((long long)B * C, 2), "out"},
                         {lse, nbytes((long long)B * NH, 4), "lse"}};
    const Span ins[] = {{qkv, nbytes(BT * 3 * C, 2), "qkv"}};
    int rc = check_args(B, T, C, NH, 0, outs, 2, ins, 1, false);
    if (rc) return rc;
    const attn::Shape s = shape_of(B, T, C, NH, 0);
    float* ws = nullptr;
    rc = workspace(attn::decode_workspace_floats(s) * 4, &ws);
    if (rc) return rc;
    return launched(attn::launch_decode_f16(out, lse, qkv, ws, s, g_stream),
                    "attn_decode_f16 launch");
}

namespace {
int check_merge(void* out, size_t out_elem, float* lse, const float* o_parts,
                const float* lse_parts, int nparts, int B, int T, int C, int NH) {
    if (nparts < 1) return fail(ATTN_EINVAL, "nparts must be >= 1 (got %d)", nparts);
    const long long BT = (long long)B * T;
    const Span outs[] = {{out, nbytes(BT * C, out_elem), "out"}, {lse, nbytes(BT * NH, 4), "lse"}};
    const Span ins[] = {{o_parts, nbytes(BT * C * nparts, 4), "o_parts"},
                        {lse_parts, nbytes(BT * NH * nparts, 4), "lse_parts"}};
    return check_args(B, T, C, NH, 0, outs, 2, ins, 2, false);
}
}  // namespace

int attn_merge(float* out, float* lse, const float* o_parts, const float* lse_parts, int nparts,
               int B, int T, int C, int NH) {
    int rc = check_merge(out, 4, lse, o_parts, lse_parts, nparts, B, T, C, NH);
    if (rc) return rc;
    return launched(attn::launch_merge_f32(out, lse, o_parts, lse_parts, nparts,
                                           shape_of(B, T, C, NH, 0), g_stream),
                    "attn_merge launch");
}

int attn_merge_bf16(uint16_t* out, float* lse, const float* o_parts, const float* lse_parts,
                    int nparts, int B, int T, int C, int NH) {
    int rc = check_merge(out, 2, lse, o_parts, lse_parts, nparts, B, T, C, NH);
    if (rc) return rc;
    return launched(attn::launch_merge_bf16(out, lse, o_parts, lse_parts, nparts,
                                            shape_of(B, T, C, NH, 0), g_stream),
                    "attn_merge_bf16 launch");
}

int attn_merge_f16(uint16_t* out, float* lse, const float* o_parts, const float* lse_parts,
                    int nparts, int B, int T, int C, int NH) {
    int rc = check_merge(out, 2, lse, o_parts, lse_parts, nparts, B, T, C, NH);
    if (rc) return rc;
    return launched(attn::launch_merge_f16(out, lse, o_parts, lse_parts, nparts,
                                            shape_of(B, T, C, NH, 0), g_stream),
                    "attn_merge_f16 launch");
}

}  // extern "C"

// ---- LayerNorm ----
namespace {
int check_ln(int N, int C, const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i)
        if (!outs[i].p) return fail(ATTN_EINVAL, "%s is NULL", outs[i].name);
    for (int i = 0; i < nin; ++i)
        if (!ins[i].p) return fail(ATTN_EINVAL, "%s is NULL", ins[i].name);
    if (N < 1 || C < 1) return fail(ATTN_EINVAL, "N and C must be >= 1 (got N=%d C=%d)", N, C);
    for (int i = 0; i < nout; ++i)
        if ((uintptr_t)outs[i].p % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", outs[i].name);
    for (int i = 0; i < nin; ++i)
        if ((uintptr_t)ins[i].p % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", ins[i].name);
    for (int i = 0; i < nout; ++i) {
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(ATTN_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(ATTN_EINVAL, "output %s overlaps input %s", outs[i].name, ins[j].name);
    }
    return ATTN_OK;
}

template <typename T>
int ln_forward_any(T* out, float* mean, float* rstd, const T* inp, const float* weight,
                   const float* bias, int N, int C, const char* name,
                   hipError_t (*launch)(T*, float*, float*, const T*, const float*, const float*,
                                        int, int, hipStream_t)) {
    const long long NC = (long long)N * C;
    const Span outs[] = {{out, nbytes(NC, sizeof(T)), "out"},
                         {mean, nbytes(N, 4), "mean"},
                         {rstd, nbytes(N, 4), "rstd"}};
    const Span ins[] = {{inp, nbytes(NC, sizeof(T)), "inp"},
                        {weight, nbytes(C, 4), "weight"},
                        {bias, nbytes(C, 4), "bias"}};
    int rc = check_ln(N, C, outs, 3, ins, 3);
    if (rc) return rc;
    return launched(launch(out, mean, rstd, inp, weight, bias, N, C, g_stream), name);
}

template <typename T>
int ln_backward_any(T* dinp, float* dweight, float* dbias, const T* dout, const T* inp,
                    const float* weight, const float* mean, const float* rstd, int N, int C,
                    const char* name,
                    hipError_t (*launch)(T*, float*, float*, float*, const T*, const T*,
                                         const float*, const float*, const float*, int, int,
                                         hipStream_t)) {
    const long long NC = (long long)N * C;
    const Span outs[] = {{dinp, nbytes(NC, sizeof(T)), "dinp"},
                         {dweight, nbytes(C, 4), "dweight"},
                         {dbias, nbytes(C, 4), "dbias"}};
    const Span ins[] = {{dout, nbytes(NC, sizeof(T)), "dout"},
                        {inp, nbytes(NC, sizeof(T)), "inp"},
                        {weight, nbytes(C, 4), "weight"},
                        {mean, nbytes(N, 4), "mean"},
                        {rstd, nbytes(N, 4), "rstd"}};
    int rc = check_ln(N, C, outs, 3, ins, 5);
    if (rc) return rc;
    float* ws = nullptr;
    rc = workspace(attn::layernorm_workspace_floats(N, C) * 4, &ws);
    if (rc) return rc;
    return launched(launch(dinp, dweight, dbias, ws, dout, inp, weight, mean, rstd, N, C,
                           g_stream),
                    name);
}
}  // namespace

extern "C" {

int layernorm_forward(float* out, float* mean, float* rstd, const float* inp, const float* weight,
                      const float* bias, int N, int C) {
    return ln_forward_any<float>(out, mean, rstd, inp, weight, bias, N, C,
                                 "layernorm_forward launch", attn::launch_layernorm_fwd_f32);
}

int layernorm_forward_bf16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                           const float* weight, const float* bias, int N, int C) {
    return ln_forward_any<uint16_t>(out, mean, rstd, inp, weight, bias, N, C,
                                    "layernorm_forward_bf16 launch",
                                    attn::launch_layernorm_fwd_bf16);
}

int layernorm_forward_f16(uint16_t* out, float* mean, float* rstd, const uint16_t* inp,
                          const float* weight, const float* bias, int N, int C) {
    return ln_forward_any<uint16_t>(out, mean, rstd, inp, weight, bias, N, C,
                                    "layernorm_forward_f16 launch",
                                    attn::launch_layernorm_fwd_f16);
}

int layernorm_backward_f16(uint16_t* dinp, float* dweight, float* dbias, const uint16_t* dout,
                           const uint16_t* inp, const float* weight, const float* mean,
                           const float* rstd, int N, int C) {
    return ln_backward_any<uint16_t>(dinp, dweight, dbias, dout, inp, weight, mean, rstd, N, C,
                                     "layernorm_backward_f16 launch",
                                     attn::launch_layernorm_bwd_f16);
}

int layernorm_backward(float* dinp, float* dweight, float* dbias, const float* dout,
                       const float* inp, const float* weight, const float* mean, const float* rstd,
                       int N, int C) {
    return ln_backward_any<float>(dinp, dweight, dbias, dout, inp, weight, mean, rstd, N, C,
                                  "layernorm_backward launch", attn::launch_layernorm_bwd_f32);
}

int layernorm_backward_bf16(uint16_t* dinp, float* dweight, float* dbias, const uint16_t* dout,
                            const uint16_t* inp, const float* weight, const float* mean,
                            const float* rstd, int N, int C) {
    return ln_backward_any<uint16_t>(dinp, dweight, dbias, dout, inp, weight, mean, rstd, N, C,
                                     "layernorm_backward_bf16 launch",
                                     attn::launch_layernorm_bwd_bf16);
}

}  // extern "C"

// ---- projections ----
namespace {
int check_proj(int M, int K, int N, int kmul, const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i)
        if (!outs[i].p) return fail(ATTN_EINVAL, "%s is NULL", outs[i].name);
    for (int i = 0; i < nin; ++i)
        if (!ins[i].p) return fail(ATTN_EINVAL, "%s is NULL", ins[i].name);
    if (M < 1 || K < 1 || N < 1)
        return fail(ATTN_EINVAL, "M, K and N must be >= 1 (got M=%d K=%d N=%d)", M, K, N);
    if (K % kmul != 0)
        return fail(ATTN_EINVAL, "K=%d must be a multiple of %d (16-byte rows)", K, kmul);
    if (N % 4 != 0) return fail(ATTN_EINVAL, "N=%d must be a multiple of 4", N);
    // a 128-row tile of rows K elements long is addressed with 32-bit byte offsets
    if ((long long)128 * K * 4 >= (1LL << 31))
        return fail(ATTN_EINVAL, "K=%d too large for the tile offsets", K);
    for (int i = 0; i < nout; ++i)
        if ((uintptr_t)outs[i].p % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", outs[i].name);
    for (int i = 0; i < nin; ++i)
        if ((uintptr_t)ins[i].p % 16) return fail(ATTN_EINVAL, "%s is not 16-byte aligned", ins[i].name);
    for (int i = 0; i < nout; ++i)
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(ATTN_EINVAL, "output %s overlaps input %s", outs[i].name, ins[j].name);
    return ATTN_OK;
}
}  // namespace

extern "C" {

int attn_qkv_projection(float* qkv, const float* x, const float* w, const float* bias, int M, int K,
                        int N) {
    const Span outs[] = {{qkv, nbytes((long long)M * N, 4), "qkv"}};
    const Span ins[] = {{x, nbytes((long long)M * K, 4), "x"},
                        {w, nbytes((long long)N * K, 4), "w"},
                        {bias, nbytes(N, 4), "bias"}};
    int rc = check_proj(M, K, N, 4, outs, 1, ins, 3);
    if (rc) return rc;
    return launched(attn::launch_gemm_f32(qkv, x, w, bias, nullptr, M, N, K, g_stream),
                    "attn_qkv_projection launch");
}

int attn_qkv_projection_bf16(uint16_t* qkv, const uint16_t* x, const uint16_t* w, const float* bias,
                             int M, int K, int N) {
    const Span outs[] = {{qkv, nbytes((long long)M * N, 2), "qkv"}};
    const Span ins[] = {{x, nbytes((long long)M * K, 2), "x"},
                        {w, nbytes((long long)N * K, 2), "w"},
                        {bias, nbytes(N, 4), "bias"}};
    int rc = check_proj(M, K, N, 8, outs, 1, ins, 3);
    if (rc) return rc;
    return launched(attn::launch_gemm_bf16(qkv, x, w, bias, nullptr, M, N, K, g_stream),
                    "attn_qkv_projection_bf16 launch");
}

int attn_out_projection(float* y, const float* a, const float* w, const float* bias,
                        const float* residual, int M, int K, int N) {
    const Span outs[] = {{y, nbytes((long long)M * N, 4), "y"}};
    const Span ins[] = {{a, nbytes((long long)M * K, 4), "a"},
                        {w, nbytes((long long)N * K, 4), "w"},
                        {bias, nbytes(N, 4), "bias"},
                        {residual, nbytes((long long)M * N, 4), "residual"}};
    int rc = check_proj(M, K, N, 4, outs, 1, ins, 4);
    if (rc) return rc;
    return launched(attn::launch_gemm_f32(y, a, w, bias, residual, M, N, K, g_stream),
                    "attn_out_projection launch");
}

int attn_out_projection_bf16(uint16_t* y, const uint16_t* a, const uint16_t* w, const float* bias,
                             const uint16_t* residual, int M, int K, int N) {
    const Span outs[] = {{y, nbytes((long long)M * N, 2), "y"}};
    const Span ins[] = {{a, nbytes((long long)M * K, 2), "a"},
                        {w, nbytes((long long)N * K, 2), "w"},
                        {bias, nbytes(N, 4), "bias"},
                        {residual, nbytes((long long)M * N, 2), "residual"}};
    int rc = check_proj(M, K, N, 8, outs, 1, ins, 4);
    if (rc) return rc;
    return launched(attn::launch_gemm_bf16(y, a, w, bias, residual, M, N, K, g_stream),
                    "attn_out_projection_bf16 launch");
}

}  // extern "C"
