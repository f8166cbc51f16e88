/*
 * oracle.c -- plain fp64 CPU oracle for multi-head scaled-dot-product
 * self-attention, forward and analytic backward, causal or not.
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark call it to check the HIP library.  The
 * library never links, loads or calls it, and the two share no code.
 *
 * Sources (cited by page title and the part of the page followed):
 *   [LLMC]  llm.c dev/cuda/attention_backward.cu (gitea mirror of
 *           karpathy/llm.c): the CPU references attention_forward_cpu
 *           (four passes) and attention_backward_cpu, and the closed-form
 *           softmax backward of softmax_autoregressive_backward_kernel7.
 *   [SW]    "Umakini wa kujitegemea, kerneli za CUDA na FlashAttention",
 *           section 1: Scores = Q K^T / sqrt(d_k), softmax per row, times V;
 *           heads are independent.  Its FlashAttention part says only small
 *           per-row normalisation statistics are kept for the backward pass.
 *
 * Layout (as in [LLMC]): qkv is (B, T, 3C) row-major, and for head h of
 * size hs = C/NH
 *     q[b,t,h,i] = qkv[b,t,      h*hs+i]
 *     k[b,t,h,i] = qkv[b,t,  C + h*hs+i]
 *     v[b,t,h,i] = qkv[b,t, 2C + h*hs+i]
 * out and dout are (B, T, C) with out[b,t,h*hs+i]; lse is (B, NH, T);
 * preatt, att, datt, dpreatt are (B, NH, T, T).  Everything is double.
 *
 * The set of keys a query row t attends to is U(t) = {0..t} when causal
 * and {0..T-1} otherwise ([SW] section 1 for the unmasked form).
 *
 * Readings where the pages leave a choice open:
 *   - the row maximum is taken over U(t) only (softmax is shift invariant,
 *     so this is the same function as a maximum over the whole row);
 *   - preatt holds the unscaled dot products q.k for every j < T (masked
 *     ones included), the 1/sqrt(hs) scale sits inside the exponential;
 *   - masked att and dpreatt entries are exactly 0; datt is dense;
 *   - lse[b,h,t] = scale*max + log(sum), natural log, in the scaled domain;
 *   - gradients are written (=), not accumulated into the caller's buffer.
 *
 * Parallelism only splits independent work (rows in the forward; rows of
 * one head in the backward, with per-thread partial sums for dk and dv
 * that are added in thread order afterwards).  No other blocking, fusion
 * or reordering is done.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

static int check_dims(int B, int T, int C, int NH, int causal) {
    if (B < 1 || T < 1 || NH < 1 || C < NH || C % NH != 0) return ORACLE_EINVAL;
    if (causal != 0 && causal != 1) return ORACLE_EINVAL;
    return ORACLE_OK;
}

void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int oracle_max_threads(void) { return omp_get_max_threads(); }

/*
 * One query row of the forward pass, passes 1 to 3 of attention_forward_cpu
 * in [LLMC].  Fills pre[0..npre) with q.k_j (npre = T when the caller wants
 * the full preatt row, else |U(t)|), a[0..nj) with the softmax probabilities
 * over U(t) = {0..nj-1}, and returns the row's log-sum-exp (scaled domain).
 */
static double softmax_row(double* pre, double* a, const double* q,
                          const double* kbase, size_t row_stride, int hs,
                          int nj, int npre, double scale) {
    /* pass 1: dot products and the maximum over U(t) */
    double mx = -INFINITY;
    for (int j = 0; j < npre; j++) {
        const double* kj = kbase + (size_t)j * row_stride;
        double s = 0.0;
        for (int i = 0; i < hs; i++) s += q[i] * kj[i];
        pre[j] = s;
        if (j < nj && s > mx) mx = s;
    }
    /* pass 2: exponentials of the scaled, shifted scores and their sum */
    double sum = 0.0;
    for (int j = 0; j < nj; j++) {
        a[j] = exp(scale * (pre[j] - mx));
        sum += a[j];
    }
    /* pass 3: normalise (the guard for a zero sum is kept from [LLMC]) */
    double inv = (sum == 0.0) ? 0.0 : 1.0 / sum;
    for (int j = 0; j < nj; j++) a[j] *= inv;
    return scale * mx + log(sum);
}

/*
 * Forward: out (B,T,C), lse (B,NH,T); preatt and att (B,NH,T,T) are written
 * only when non-NULL (the pages' materialised reference).
 */
int oracle_forward(double* out, double* lse, double* preatt, double* att,
                   const double* qkv, int B, int T, int C, int NH, int causal) {
    int rc = check_dims(B, T, C, NH, causal);
    if (rc) return rc;
    if (!out || !lse || !qkv) return ORACLE_EINVAL;
    const int hs = C / NH;
    const size_t C3 = 3 * (size_t)C;
    const double scale = 1.0 / sqrt((double)hs);
    int failed = 0;

#pragma omp parallel
    {
        double* pre = (double*)malloc(sizeof(double) * (size_t)T);
        double* a = (double*)malloc(sizeof(double) * (size_t)T);
        if (!pre || !a) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 8)
        for (int b = 0; b < B; b++)
            for (int t = 0; t < T; t++)
                for (int h = 0; h < NH; h++) {
                    if (!pre || !a) continue;
                    const double* q = qkv + ((size_t)b * T + t) * C3 + (size_t)h * hs;
                    const double* kbase = qkv + (size_t)b * T * C3 + C + (size_t)h * hs;
                    const double* vbase = qkv + (size_t)b * T * C3 + 2 * (size_t)C + (size_t)h * hs;
                    const int nj = causal ? t + 1 : T;
                    const int npre = preatt ? T : nj;
                    double l = softmax_row(pre, a, q, kbase, C3, hs, nj, npre, scale);
                    lse[((size_t)b * NH + h) * T + t] = l;
                    const size_t mrow = (((size_t)b * NH + h) * T + t) * (size_t)T;
                    if (preatt) memcpy(preatt + mrow, pre, sizeof(double) * (size_t)T);
                    if (att) {
                        for (int j = 0; j < T; j++) att[mrow + j] = (j < nj) ? a[j] : 0.0;
                    }
                    /* pass 4: weighted sum of the values over U(t) */
                    double* o = out + ((size_t)b * T + t) * C + (size_t)h * hs;
                    for (int i = 0; i < hs; i++) o[i] = 0.0;
                    for (int j = 0; j < nj; j++) {
                        const double* vj = vbase + (size_t)j * C3;
                        for (int i = 0; i < hs; i++) o[i] += a[j] * vj[i];
                    }
                }
        free(pre);
        free(a);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Forward restricted to query rows [q0, q1) and keys [k0, k1): each row t
 * attends to U(t) intersected with {k0..k1-1}, with the same four passes as
 * oracle_forward.  out is (B, q1-q0, C) and lse is (B, NH, q1-q0).  A row
 * with no key in the range gets out = 0 and lse = -inf (an empty softmax;
 * the pages never form one, so this is the reading used for the partial
 * results that a split of the key range produces).  With q0 = 0, q1 = T,
 * k0 = 0, k1 = T it computes exactly what oracle_forward does, in the same
 * order.
 */
int oracle_forward_block(double* out, double* lse, const double* qkv, int B, int T, int C,
                         int NH, int causal, int q0, int q1, int k0, int k1) {
    int rc = check_dims(B, T, C, NH, causal);
    if (rc) return rc;
    if (!out || !lse || !qkv) return ORACLE_EINVAL;
    if (q0 < 0 || q1 > T || q0 >= q1 || k0 < 0 || k1 > T || k0 > k1) return ORACLE_EINVAL;
    const int hs = C / NH;
    const int nq = q1 - q0;
    const size_t C3 = 3 * (size_t)C;
    const double scale = 1.0 / sqrt((double)hs);
    int failed = 0;

#pragma omp parallel
    {
        double* pre = (double*)malloc(sizeof(double) * (size_t)T);
        double* a = (double*)malloc(sizeof(double) * (size_t)T);
        if (!pre || !a) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for collapse(3) schedule(dynamic, 8)
        for (int b = 0; b < B; b++)
            for (int r = 0; r < nq; r++)
                for (int h = 0; h < NH; h++) {
                    if (!pre || !a) continue;
                    const int t = q0 + r;
                    const double* q = qkv + ((size_t)b * T + t) * C3 + (size_t)h * hs;
                    /* keys k0 .. k0+nj-1: the range cut by the causal limit */
                    const double* kbase = qkv + ((size_t)b * T + k0) * C3 + C + (size_t)h * hs;
                    const double* vbase = qkv + ((size_t)b * T + k0) * C3 + 2 * (size_t)C + (size_t)h * hs;
                    const int hi = causal ? (t + 1 < k1 ? t + 1 : k1) : k1;
                    const int nj = hi > k0 ? hi - k0 : 0;
                    double* o = out + ((size_t)b * nq + r) * C + (size_t)h * hs;
                    for (int i = 0; i < hs; i++) o[i] = 0.0;
                    if (nj == 0) {
                        lse[((size_t)b * NH + h) * nq + r] = -INFINITY;
                        continue;
                    }
                    lse[((size_t)b * NH + h) * nq + r] =
                        softmax_row(pre, a, q, kbase, C3, hs, nj, nj, scale);
                    for (int j = 0; j < nj; j++) {
                        const double* vj = vbase + (size_t)j * C3;
                        for (int i = 0; i < hs; i++) o[i] += a[j] * vj[i];
                    }
                }
        free(pre);
        free(a);
    }
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Backward: dqkv (B,T,3C) is overwritten with [dq | dk | dv].  The forward
 * probabilities are recomputed from qkv row by row, so memory stays O(T)
 * per thread unless datt / dpreatt (B,NH,T,T) are requested (non-NULL).
 *
 * Per query row t of head (b,h), following attention_backward_cpu in [LLMC]:
 *   datt[j]    = v_j . dout_t                         (every j < T)
 *   dv_j      += att[j] * dout_t                      (j in U(t))
 *   dpreatt[j] = scale * att[j] * (datt[j] - sum_{j' in U(t)} att[j'] datt[j'])
 *                                                     (j in U(t), else 0)
 *   dq_t       = sum_j dpreatt[j] * k_j
 *   dk_j      += dpreatt[j] * q_t
 * The dpreatt line is the closed form of the softmax Jacobian product that
 * [LLMC] derives for softmax_autoregressive_backward_kernel7.
 */
int oracle_backward(double* dqkv, double* dpreatt, double* datt,
                    const double* dout, const double* qkv,
                    int B, int T, int C, int NH, int causal) {
    int rc = check_dims(B, T, C, NH, causal);
    if (rc) return rc;
    if (!dqkv || !dout || !qkv) return ORACLE_EINVAL;
    const int hs = C / NH;
    const size_t C3 = 3 * (size_t)C;
    const double scale = 1.0 / sqrt((double)hs);
    const int nth = omp_get_max_threads();
    const size_t part = (size_t)T * hs;
    double* pk = (double*)calloc((size_t)nth * part, sizeof(double));
    double* pv = (double*)calloc((size_t)nth * part, sizeof(double));
    if (!pk || !pv) { free(pk); free(pv); return ORACLE_ENOMEM; }
    int failed = 0;

    memset(dqkv, 0, sizeof(double) * (size_t)B * T * C3);

    for (int b = 0; b < B; b++) {
        for (int h = 0; h < NH; h++) {
            const double* qbase = qkv + (size_t)b * T * C3 + (size_t)h * hs;
            const double* kbase = qbase + C;
            const double* vbase = qbase + 2 * (size_t)C;
            double* dqbase = dqkv + (size_t)b * T * C3 + (size_t)h * hs;
            memset(pk, 0, sizeof(double) * (size_t)nth * part);
            memset(pv, 0, sizeof(double) * (size_t)nth * part);
            int used = 1;
#pragma omp parallel num_threads(nth)
            {
                const int tid = omp_get_thread_num();
#pragma omp single
                used = omp_get_num_threads();
                double* pre = (double*)malloc(sizeof(double) * (size_t)T);
                double* a = (double*)malloc(sizeof(double) * (size_t)T);
                double* da = (double*)malloc(sizeof(double) * (size_t)T);
                double* dp = (double*)malloc(sizeof(double) * (size_t)T);
                if (!pre || !a || !da || !dp) {
#pragma omp atomic write
                    failed = 1;
                }
                double* dk_acc = pk + (size_t)tid * part;
                double* dv_acc = pv + (size_t)tid * part;
#pragma omp for schedule(static, 1)
                for (int t = 0; t < T; t++) {
                    if (!pre || !a || !da || !dp) continue;
                    const double* q = qbase + (size_t)t * C3;
                    const double* go = dout + ((size_t)b * T + t) * C + (size_t)h * hs;
                    const int nj = causal ? t + 1 : T;
                    softmax_row(pre, a, q, kbase, C3, hs, nj, nj, scale);
                    /* through pass 4: datt and dv */
                    const int nda = datt ? T : nj;
                    for (int j = 0; j < nda; j++) {
                        const double* vj = vbase + (size_t)j * C3;
                        double s = 0.0;
                        for (int i = 0; i < hs; i++) s += vj[i] * go[i];
                        da[j] = s;
                    }
                    for (int j = 0; j < nj; j++) {
                        double* dvj = dv_acc + (size_t)j * hs;
                        for (int i = 0; i < hs; i++) dvj[i] += a[j] * go[i];
                    }
                    /* through passes 2 and 3: the softmax */
                    double dot = 0.0;
                    for (int j = 0; j < nj; j++) dot += a[j] * da[j];
                    for (int j = 0; j < nj; j++) dp[j] = scale * a[j] * (da[j] - dot);
                    /* through pass 1: preatt = q . k */
                    double* dq = dqbase + (size_t)t * C3;
                    for (int j = 0; j < nj; j++) {
                        const double* kj = kbase + (size_t)j * C3;
                        double* dkj = dk_acc + (size_t)j * hs;
                        for (int i = 0; i < hs; i++) {
                            dq[i] += dp[j] * kj[i];
                            dkj[i] += dp[j] * q[i];
                        }
                    }
                    const size_t mrow = (((size_t)b * NH + h) * T + t) * (size_t)T;
                    if (datt) memcpy(datt + mrow, da, sizeof(double) * (size_t)T);
                    if (dpreatt) {
                        for (int j = 0; j < T; j++) dpreatt[mrow + j] = (j < nj) ? dp[j] : 0.0;
                    }
                }
                free(pre);
                free(a);
                free(da);
                free(dp);
            }
            /* add the per-thread partial sums of dk and dv in thread order */
            for (int th = 0; th < used; th++) {
                const double* sk = pk + (size_t)th * part;
                const double* sv = pv + (size_t)th * part;
                for (int j = 0; j < T; j++) {
                    double* dk = dqbase + (size_t)j * C3 + C;
                    double* dv = dqbase + (size_t)j * C3 + 2 * (size_t)C;
                    for (int i = 0; i < hs; i++) {
                        dk[i] += sk[(size_t)j * hs + i];
                        dv[i] += sv[(size_t)j * hs + i];
                    }
                }
            }
        }
    }
    free(pk);
    free(pv);
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------ LayerNorm
 * Layer normalisation of each row of an (N, C) matrix, the neighbour of the
 * attention block in a GPT-2 layer.  Sources:
 *   [P1]  "llm.c 的中文注解-20240423", section 1.8 (layernorm_forward_kernel3):
 *         per row the mean, then the mean of squared deviations from it,
 *         rstd = 1/sqrt(var + 1e-5), out = (x - mean) * rstd * weight + bias;
 *         mean and rstd are kept per row.
 *   [P3]  "LLM Systems 10 & 11: Accelerating Transformer Training and
 *         Inference", the LayerNorm part of the reduction section: the
 *         backward in terms of xhat = (x - mean) / sigma and the upstream
 *         gradient, with per-channel weight and bias.
 * The forward is the definition written out, two passes over the row
 * (mean, then variance about it).  The backward is the textbook gradient of
 * that definition: with g = weight * dout and xhat = (x - mean) * rstd,
 *     dinp   = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat)),
 *     dweight[c] = sum over rows of dout * xhat,   dbias[c] = sum of dout.
 * mean and rstd are recomputed here from inp in double precision.  All
 * outputs are written (=).
 */
#define ORACLE_LN_EPS 1e-5

static void ln_row_stats(const double* x, int C, double* mean, double* rstd) {
    double s = 0.0;
    for (int c = 0; c < C; ++c) s += x[c];
    const double m = s / C;
    double v = 0.0;
    for (int c = 0; c < C; ++c) v += (x[c] - m) * (x[c] - m);
    v /= C;
    *mean = m;
    *rstd = 1.0 / sqrt(v + ORACLE_LN_EPS);
}

int oracle_layernorm_forward(double* out, double* mean, double* rstd, const double* inp,
                             const double* weight, const double* bias, int N, int C) {
    if (N < 1 || C < 1) return ORACLE_EINVAL;
#pragma omp parallel for
    for (int r = 0; r < N; ++r) {
        const double* x = inp + (size_t)r * C;
        double m, s;
        ln_row_stats(x, C, &m, &s);
        double* o = out + (size_t)r * C;
        for (int c = 0; c < C; ++c) o[c] = (x[c] - m) * s * weight[c] + bias[c];
        if (mean) mean[r] = m;
        if (rstd) rstd[r] = s;
    }
    return ORACLE_OK;
}

int oracle_layernorm_backward(double* dinp, double* dweight, double* dbias, const double* dout,
                              const double* inp, const double* weight, int N, int C) {
    if (N < 1 || C < 1) return ORACLE_EINVAL;
    double* ms = (double*)malloc(sizeof(double) * 2 * (size_t)N);
    if (!ms) return ORACLE_ENOMEM;
#pragma omp parallel for
    for (int r = 0; r < N; ++r) {
        const double* x = inp + (size_t)r * C;
        const double* dy = dout + (size_t)r * C;
        double m, s;
        ln_row_stats(x, C, &m, &s);
        ms[2 * r] = m;
        ms[2 * r + 1] = s;
        double gmean = 0.0, gxmean = 0.0;
        for (int c = 0; c < C; ++c) {
            const double g = weight[c] * dy[c];
            gmean += g;
            gxmean += g * (x[c] - m) * s;
        }
        gmean /= C;
        gxmean /= C;
        double* dx = dinp + (size_t)r * C;
        for (int c = 0; c < C; ++c) {
            const double xhat = (x[c] - m) * s;
            dx[c] = s * (weight[c] * dy[c] - gmean - xhat * gxmean);
        }
    }
    /* column sums in row order (one thread per column) */
#pragma omp parallel for
    for (int c = 0; c < C; ++c) {
        double dw = 0.0, db = 0.0;
        for (int r = 0; r < N; ++r) {
            const double dy = dout[(size_t)r * C + c];
            dw += dy * (inp[(size_t)r * C + c] - ms[2 * r]) * ms[2 * r + 1];
            db += dy;
        }
        dweight[c] = dw;
        dbias[c] = db;
    }
    free(ms);
    return ORACLE_OK;
}
