/*
 * A plain C99 caller of libattn through include/libattn.h, with no Python and
 * no torch: device buffers from hipMalloc, the fp32 forward and backward
 * (attn_forward, attn_backward) on small shapes with ragged tails, causal and
 * not, then the results copied back and compared element by element with
 * the fp64 CPU oracle (oracle/oracle.c, linked here as test infrastructure)
 * at the fp32 bounds |gpu - ref| <= 1e-5 + 1e-4 |ref|.  Also the status and
 * message of a rejected call.  Prints one line per case and "c caller ok"
 * at the end; exits 1 on any failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "libattn.h"

/* the oracle's entry points (oracle/oracle.c) */
int oracle_forward(double* out, double* lse, double* preatt, double* att, const double* qkv,
                   int B, int T, int C, int NH, int causal);
int oracle_backward(double* dqkv, double* dpreatt, double* datt, const double* dout,
                    const double* qkv, int B, int T, int C, int NH, int causal);

/* seeded inputs: splitmix64 words, uniforms in (0, 1), Box-Muller normals */
static uint64_t rng_state;
static double uniform01(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return ((double)(z >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
static float normal01(void) {
    const double a = uniform01(), b = uniform01();
    return (float)(sqrt(-2.0 * log(a)) * cos(6.283185307179586 * b));
}

#define HIP_OK(x)                                                                     \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)

/* elementwise bound; returns the number of violations, reports the worst */
static long compare(const char* what, const float* g, const double* r, size_t n) {
    long bad = 0;
    double worst = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const double d = fabs((double)g[i] - r[i]);
        if (!(d <= 1e-5 + 1e-4 * fabs(r[i]))) ++bad;   /* NaN counts as a violation */
        if (d > worst || d != d) worst = d;
    }
    printf("  %-5s max |gpu - oracle| %.3e, %ld of %zu outside the bound\n", what, worst, bad, n);
    return bad;
}

static int run_case(int B, int T, int C, int NH, int causal, uint64_t seed) {
    const size_t nqkv = (size_t)B * T * 3 * C, nio = (size_t)B * T * C, nl = (size_t)B * NH * T;
    float* qkv = malloc(nqkv * sizeof(float));
    float* dout = malloc(nio * sizeof(float));
    float* out = malloc(nio * sizeof(float));
    float* lse = malloc(nl * sizeof(float));
    float* dqkv = malloc(nqkv * sizeof(float));
    double* qkv64 = malloc(nqkv * sizeof(double));
    double* dout64 = malloc(nio * sizeof(double));
    double* out_r = malloc(nio * sizeof(double));
    double* lse_r = malloc(nl * sizeof(double));
    double* dqkv_r = malloc(nqkv * sizeof(double));
    if (!qkv || !dout || !out || !lse || !dqkv || !qkv64 || !dout64 || !out_r || !lse_r || !dqkv_r) {
        fprintf(stderr, "host allocation failed\n");
        exit(1);
    }
    rng_state = seed;
    for (size_t i = 0; i < nqkv; ++i) qkv64[i] = qkv[i] = normal01();
    for (size_t i = 0; i < nio; ++i) dout64[i] = dout[i] = normal01();

    float *d_qkv, *d_dout, *d_out, *d_lse, *d_dqkv;
    HIP_OK(hipMalloc((void**)&d_qkv, nqkv * sizeof(float)));
    HIP_OK(hipMalloc((void**)&d_dout, nio * sizeof(float)));
    HIP_OK(hipMalloc((void**)&d_out, nio * sizeof(float)));
    HIP_OK(hipMalloc((void**)&d_lse, nl * sizeof(float)));
    HIP_OK(hipMalloc((void**)&d_dqkv, nqkv * sizeof(float)));
    HIP_OK(hipMemcpy(d_qkv, qkv, nqkv * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_dout, dout, nio * sizeof(float), hipMemcpyHostToDevice));

    printf("case B%d T%d C%d NH%d causal=%d\n", B, T, C, NH, causal);
    fflush(stdout);
    int rc = attn_forward(d_out, d_lse, d_qkv, B, T, C, NH, causal);
    if (rc == ATTN_OK) rc = attn_backward(d_dqkv, d_dout, d_qkv, d_out, d_lse, B, T, C, NH, causal);
    if (rc != ATTN_OK) {
        printf("  libattn status %d: %s\n", rc, attn_last_error());
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, d_out, nio * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, d_lse, nl * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dqkv, d_dqkv, nqkv * sizeof(float), hipMemcpyDeviceToHost));

    if (oracle_forward(out_r, lse_r, NULL, NULL, qkv64, B, T, C, NH, causal) != 0 ||
        oracle_backward(dqkv_r, NULL, NULL, dout64, qkv64, B, T, C, NH, causal) != 0) {
        printf("  oracle rejected the shape\n");
        return 1;
    }
    long bad = compare("out", out, out_r, nio) + compare("lse", lse, lse_r, nl) +
               compare("dqkv", dqkv, dqkv_r, nqkv);

    HIP_OK(hipFree(d_qkv));
    HIP_OK(hipFree(d_dout));
    HIP_OK(hipFree(d_out));
    HIP_OK(hipFree(d_lse));
    HIP_OK(hipFree(d_dqkv));
    free(qkv); free(dout); free(out); free(lse); free(dqkv);
    free(qkv64); free(dout64); free(out_r); free(lse_r); free(dqkv_r);
    return bad != 0;
}

int main(void) {
    int fail = 0;
    fail |= run_case(2, 97, 128, 2, 1, 11);    /* hs 64, ragged second tile */
    fail |= run_case(1, 130, 256, 4, 0, 12);   /* hs 64, non-causal, three tiles */
    fail |= run_case(2, 70, 64, 4, 1, 13);     /* hs 16 */

    /* a rejected call: C % NH != 0, before any HIP call */
    float* none = NULL;
    HIP_OK(hipMalloc((void**)&none, 256));
    const int rc = attn_forward(none, none + 16, none + 32, 1, 4, 66, 4, 1);
    const char* msg = attn_last_error();
    printf("rejected call: status %d, message \"%s\"\n", rc, msg);
    if (rc != ATTN_EINVAL || msg == NULL || msg[0] == '\0') fail = 1;
    HIP_OK(hipFree(none));

    if (fail) {
        printf("c caller FAILED\n");
        return 1;
    }
    printf("c caller ok\n");
    return 0;
}
