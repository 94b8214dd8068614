/*
 * oracle.c -- plain, slow CPU reference for the gated linear-attention
 * forward pass.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the GPU library never does, and
 * this file shares no header, helper or constant with it.
 *
 * What it computes (per batch b and head h, everything in double):
 *
 *   C_0 = 0, or a given initial state              (d_qk x d_hv matrix memory)
 *   C_t = diag(f_t) C_{t-1} + i_t k_t v_t^T         t = 1..T
 *   h_t = C_t^T q_t / sqrt(d_qk)
 *
 * i.e. the step-by-step recurrent form ("FusedRecurrent", O(T) time) listed
 * among the computation forms in the flash-linear-attention README.  The
 * gates follow the three variants:
 *
 *   kind 0, mLSTMsig   : i_t = sigmoid(igate_pre[t]), f_t = sigmoid(fgate_pre[t])
 *                        (sigmoid input gate, no normaliser and no max state:
 *                        "Tiled Flash Linear Attention: More Efficient Linear
 *                        RNN and xLSTM Kernels", research-map summary,
 *                        sections Approach and Surprising findings)
 *   kind 1, scalar decay (RetNet row of the flash-linear-attention README):
 *                        i_t = 1, f_t = gamma_h = sigmoid(fgate_pre[h])
 *   kind 2, per-key-channel gate (data-dependent gates, "Gated Linear
 *                        Attention Transformers with Hardware-Efficient
 *                        Training", Abstract):
 *                        i_t = 1, f_{t,c} = exp(logsigmoid(x_{t,c}) / 16)
 *
 * The same scale 1/sqrt(d_qk) is applied to every variant.  Nothing is
 * rounded on the way: inputs arrive as doubles holding the exact fp32 or
 * bf16 values the GPU sees.
 *
 * Layouts (all row-major, contiguous):
 *   q, k      [B,H,T,d_qk]      v, h [B,H,T,d_hv]
 *   igate_pre [B,H,T]  (kind 0 only; ignored otherwise)
 *   fgate_pre [B,H,T] (kind 0), [H] (kind 1), [B,H,T,d_qk] (kind 2)
 *   states    optional; when non-NULL receives C after every full block of
 *             L steps: [B,H,T/L (floor),d_qk,d_hv]
 *   c0        optional initial state C_0 [B,H,d_qk,d_hv] (NULL: zero)
 *   c_final   optional; receives C_T [B,H,d_qk,d_hv]
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { KIND_MLSTM_SIG = 0, KIND_SCALAR = 1, KIND_GLA = 2 };

/* sigmoid without overflow for either sign of x; exact 0 and 1 at -inf/+inf */
static double sigmoid(double x)
{
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* log(sigmoid(x)) = min(x,0) - log(1 + exp(-|x|)) */
static double log_sigmoid(double x)
{
    double m = x < 0.0 ? x : 0.0;
    return m - log1p(exp(-fabs(x)));
}

/* forget gate of step t for key channel c, and input gate of step t */
static double forget_gate(int kind, const double* fgate_pre, size_t bh, int head,
                          int T, int dqk, int t, int c)
{
    switch (kind) {
    case KIND_MLSTM_SIG: return sigmoid(fgate_pre[bh * (size_t)T + t]);
    case KIND_SCALAR: return sigmoid(fgate_pre[head]);
    default: return exp(log_sigmoid(fgate_pre[(bh * (size_t)T + t) * dqk + c]) / 16.0);
    }
}

static double input_gate(int kind, const double* igate_pre, size_t bh, int T, int t)
{
    return kind == KIND_MLSTM_SIG ? sigmoid(igate_pre[bh * (size_t)T + t]) : 1.0;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Recurrent forward from an initial state.  Returns 0, or -1 on an invalid
 * argument. */
int oracle_fwd_state(const double* q, const double* k, const double* v,
                     const double* igate_pre, const double* fgate_pre,
                     const double* c0, double* h, double* states, double* c_final,
                     int B, int H, int T, int dqk, int dhv, int L, int kind)
{
    if (!q || !k || !v || !fgate_pre || !h) return -1;
    if (B < 0 || H < 0 || T < 0 || dqk < 1 || dhv < 1) return -1;
    if (kind < KIND_MLSTM_SIG || kind > KIND_GLA) return -1;
    if (kind == KIND_MLSTM_SIG && !igate_pre) return -1;
    if (states && L < 1) return -1;
    const long nbh = (long)B * H;
    const int nfull = states ? T / L : 0;
    const double scale = 1.0 / sqrt((double)dqk);
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        const int head = (int)(bh % H);
        double* C = (double*)calloc((size_t)dqk * dhv, sizeof(double));
        double* f = (double*)malloc((size_t)dqk * sizeof(double));
        if (!C || !f) {
            free(C);
            free(f);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        if (c0) memcpy(C, c0 + (size_t)bh * dqk * dhv, (size_t)dqk * dhv * sizeof(double));
        for (int t = 0; t < T; ++t) {
            const double* qt = q + ((size_t)bh * T + t) * dqk;
            const double* kt = k + ((size_t)bh * T + t) * dqk;
            const double* vt = v + ((size_t)bh * T + t) * dhv;
            double* ht = h + ((size_t)bh * T + t) * dhv;
            const double it = input_gate(kind, igate_pre, (size_t)bh, T, t);
            for (int c = 0; c < dqk; ++c)
                f[c] = forget_gate(kind, fgate_pre, (size_t)bh, head, T, dqk, t, c);
            /* C <- diag(f) C + i k v^T */
            for (int c = 0; c < dqk; ++c) {
                double* row = C + (size_t)c * dhv;
                const double ik = it * kt[c];
                for (int j = 0; j < dhv; ++j) row[j] = f[c] * row[j] + ik * vt[j];
            }
            /* h = C^T q / sqrt(d_qk) */
            for (int j = 0; j < dhv; ++j) ht[j] = 0.0;
            for (int c = 0; c < dqk; ++c) {
                const double* row = C + (size_t)c * dhv;
                for (int j = 0; j < dhv; ++j) ht[j] += row[j] * qt[c];
            }
            for (int j = 0; j < dhv; ++j) ht[j] *= scale;
            if (states && (t + 1) % L == 0) {
                int blk = (t + 1) / L - 1;
                memcpy(states + (((size_t)bh * nfull + blk) * dqk) * dhv, C,
                       (size_t)dqk * dhv * sizeof(double));
            }
        }
        if (c_final) memcpy(c_final + (size_t)bh * dqk * dhv, C, (size_t)dqk * dhv * sizeof(double));
        free(C);
        free(f);
    }
    return bad ? -1 : 0;
}

/* Recurrent forward from C_0 = 0. */
int oracle_fwd(const double* q, const double* k, const double* v,
               const double* igate_pre, const double* fgate_pre,
               double* h, double* states,
               int B, int H, int T, int dqk, int dhv, int L, int kind)
{
    return oracle_fwd_state(q, k, v, igate_pre, fgate_pre, NULL, h, states, NULL, B, H, T, dqk, dhv, L,
                            kind);
}

/*
 * Chunk-local log-gate sums, the quantities a chunkwise evaluation works
 * with: for step t in chunk [t0, t0+L),
 *   a[t]  = sum_{r=t0..t} log f_r        (per key channel for kind 2)
 *   li[t] = log i_t
 *   g[k]  = a at the last step of chunk k (a partial last chunk included)
 * Layouts: a [B,H,T] (kind 2: [B,H,T,d_qk]), li [B,H,T],
 *          g [B,H,ceil(T/L)] (kind 2: [B,H,ceil(T/L),d_qk]).
 */
int oracle_log_gates(const double* igate_pre, const double* fgate_pre,
                     double* a, double* li, double* g,
                     int B, int H, int T, int dqk, int L, int kind)
{
    if (!fgate_pre || !a || !li || !g || L < 1 || T < 0 || dqk < 1) return -1;
    if (kind < KIND_MLSTM_SIG || kind > KIND_GLA) return -1;
    if (kind == KIND_MLSTM_SIG && !igate_pre) return -1;
    const long nbh = (long)B * H;
    const int nc = (T + L - 1) / L;
    const int width = kind == KIND_GLA ? dqk : 1;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < nbh; ++bh) {
        const int head = (int)(bh % H);
        for (int kc = 0; kc < nc; ++kc) {
            const int t0 = kc * L, t1 = t0 + L < T ? t0 + L : T;
            for (int c = 0; c < width; ++c) {
                double run = 0.0;
                for (int t = t0; t < t1; ++t) {
                    double lf;
                    if (kind == KIND_MLSTM_SIG) lf = log_sigmoid(fgate_pre[(size_t)bh * T + t]);
                    else if (kind == KIND_SCALAR) lf = log_sigmoid(fgate_pre[head]);
                    else lf = log_sigmoid(fgate_pre[((size_t)bh * T + t) * dqk + c]) / 16.0;
                    run += lf;
                    a[((size_t)bh * T + t) * width + c] = run;
                }
                g[((size_t)bh * nc + kc) * width + c] = run;
            }
            for (int t = t0; t < t1; ++t)
                li[(size_t)bh * T + t] =
                    kind == KIND_MLSTM_SIG ? log_sigmoid(igate_pre[(size_t)bh * T + t]) : 0.0;
        }
    }
    return 0;
}

/* the scalar gate functions, exported so tests can pin them */
double oracle_sigmoid(double x) { return sigmoid(x); }
double oracle_log_sigmoid(double x) { return log_sigmoid(x); }
