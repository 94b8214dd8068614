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

/*
 * Backward pass of the recurrence (reverse-mode derivative, in double).
 * Given dh_t = dL/dh_t, returns dL/dq, dL/dk, dL/dv and the gradients of
 * the gate pre-activations, straight from the recurrence (s = 1/sqrt(d_qk)):
 *
 *   dq_t      = s C_t dh_t
 *   dC_t      = s q_t dh_t^T + diag(f_{t+1}) dC_{t+1}        (dC after the last step: 0)
 *   dk_t      = i_t dC_t v_t          dv_t = i_t dC_t^T k_t      di_t = k_t^T dC_t v_t
 *   df_{t,c}  = sum_j dC_t[c][j] C_{t-1}[c][j]
 *
 * and through the gate functions:
 *   kind 0:  dL/digate_pre_t = di_t i_t (1 - i_t),
 *            dL/dfgate_pre_t = (sum_c df_{t,c}) f_t (1 - f_t)
 *   kind 1:  dL/dfgate_pre[h] = sum over b, t, c of df_{t,c} f_h (1 - f_h)
 *   kind 2:  dL/dx_{t,c} = df_{t,c} f_{t,c} (1 - sigmoid(x_{t,c})) / 16
 * -- the plain derivative everywhere: no floor on the log forget gate (the
 * GPU library's floor at -100 is a convention of that library, not of the
 * function defined here).  C_0 = 0.
 * The forward sweep yields C_t and dq_t; the reverse sweep recomputes the
 * states of each 64-step block from a checkpoint taken in the forward sweep.
 *
 * Layouts as oracle_fwd; dh like h; dq, dk, dv like q, k, v; dig like
 * igate_pre (kind 0; may be NULL otherwise); dfg like fgate_pre.
 */
int oracle_bwd_state(const double* q, const double* k, const double* v,
                     const double* igate_pre, const double* fgate_pre, const double* c0,
                     const double* dh, const double* dcT,
                     double* dq, double* dk, double* dv, double* dig, double* dfg, double* dc0,
                     int B, int H, int T, int dqk, int dhv, int kind)
{
    if (!q || !k || !v || !fgate_pre || !dh || !dq || !dk || !dv || !dfg) return -1;
    if (B < 0 || H < 0 || T < 0 || dqk < 1 || dhv < 1) return -1;
    if (kind < KIND_MLSTM_SIG || kind > KIND_GLA) return -1;
    if (kind == KIND_MLSTM_SIG && (!igate_pre || !dig)) return -1;
    const long nbh = (long)B * H;
    const double scale = 1.0 / sqrt((double)dqk);
    const int BLK = 64;
    const int nck = (T + BLK - 1) / BLK;
    const size_t csz = (size_t)dqk * dhv;
    double* dscal = (double*)calloc((size_t)(nbh > 0 ? nbh : 1), sizeof(double));   /* kind 1: per (b,h) */
    if (!dscal) return -1;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        const int head = (int)(bh % H);
        double* C = (double*)calloc(csz, sizeof(double));
        double* dC = (double*)calloc(csz, sizeof(double));
        double* ck = (double*)malloc((size_t)(nck > 0 ? nck : 1) * csz * sizeof(double));
        double* Cb = (double*)malloc((size_t)BLK * csz * sizeof(double));
        double* f = (double*)malloc((size_t)dqk * sizeof(double));
        double* df = (double*)malloc((size_t)dqk * sizeof(double));
        if (!C || !dC || !ck || !Cb || !f || !df) {
            free(C); free(dC); free(ck); free(Cb); free(f); free(df);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        /* forward sweep from C_0: C_t, dq_t, and the state before every 64-step block */
        if (c0) memcpy(C, c0 + (size_t)bh * csz, csz * sizeof(double));
        if (dcT) memcpy(dC, dcT + (size_t)bh * csz, csz * sizeof(double));
        for (int t = 0; t < T; ++t) {
            if (t % BLK == 0) memcpy(ck + (size_t)(t / BLK) * csz, C, csz * sizeof(double));
            const double* kt = k + ((size_t)bh * T + t) * dqk;
            const double* vt = v + ((size_t)bh * T + t) * dhv;
            const double it = input_gate(kind, igate_pre, (size_t)bh, T, t);
            for (int c = 0; c < dqk; ++c) f[c] = forget_gate(kind, fgate_pre, (size_t)bh, head, T, dqk, t, c);
            for (int c = 0; c < dqk; ++c)
                for (int j = 0; j < dhv; ++j) C[(size_t)c * dhv + j] = f[c] * C[(size_t)c * dhv + j] + it * kt[c] * vt[j];
            const double* dht = dh + ((size_t)bh * T + t) * dhv;
            double* dqt = dq + ((size_t)bh * T + t) * dqk;
            for (int c = 0; c < dqk; ++c) {
                double acc = 0.0;
                for (int j = 0; j < dhv; ++j) acc += C[(size_t)c * dhv + j] * dht[j];
                dqt[c] = scale * acc;
            }
        }
        /* reverse sweep, one block at a time */
        for (int n = nck - 1; n >= 0; --n) {
            const int t0 = n * BLK, t1 = t0 + BLK < T ? t0 + BLK : T;
            /* states after steps t0..t1-1 of this block */
            memcpy(C, ck + (size_t)n * csz, csz * sizeof(double));
            for (int t = t0; t < t1; ++t) {
                const double* kt = k + ((size_t)bh * T + t) * dqk;
                const double* vt = v + ((size_t)bh * T + t) * dhv;
                const double it = input_gate(kind, igate_pre, (size_t)bh, T, t);
                for (int c = 0; c < dqk; ++c) f[c] = forget_gate(kind, fgate_pre, (size_t)bh, head, T, dqk, t, c);
                for (int c = 0; c < dqk; ++c)
                    for (int j = 0; j < dhv; ++j)
                        C[(size_t)c * dhv + j] = f[c] * C[(size_t)c * dhv + j] + it * kt[c] * vt[j];
                memcpy(Cb + (size_t)(t - t0) * csz, C, csz * sizeof(double));
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const double* qt = q + ((size_t)bh * T + t) * dqk;
                const double* kt = k + ((size_t)bh * T + t) * dqk;
                const double* vt = v + ((size_t)bh * T + t) * dhv;
                const double* dht = dh + ((size_t)bh * T + t) * dhv;
                /* dC_t = diag(f_{t+1}) dC_{t+1} + s q_t dh_t^T; for the last step the
                   first term is the gradient dcT of the final state (or 0) */
                if (t + 1 < T)
                    for (int c = 0; c < dqk; ++c) f[c] = forget_gate(kind, fgate_pre, (size_t)bh, head, T, dqk, t + 1, c);
                for (int c = 0; c < dqk; ++c)
                    for (int j = 0; j < dhv; ++j) {
                        double* e = &dC[(size_t)c * dhv + j];
                        *e = (t + 1 < T ? f[c] * *e : *e) + scale * qt[c] * dht[j];
                    }
                const double it = input_gate(kind, igate_pre, (size_t)bh, T, t);
                double* dkt = dk + ((size_t)bh * T + t) * dqk;
                double* dvt = dv + ((size_t)bh * T + t) * dhv;
                double di = 0.0;
                for (int c = 0; c < dqk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dhv; ++j) acc += dC[(size_t)c * dhv + j] * vt[j];
                    dkt[c] = it * acc;
                    di += kt[c] * acc;
                }
                for (int j = 0; j < dhv; ++j) {
                    double acc = 0.0;
                    for (int c = 0; c < dqk; ++c) acc += dC[(size_t)c * dhv + j] * kt[c];
                    dvt[j] = it * acc;
                }
                /* df_{t,c} against the state before step t */
                const double* Cprev = t > t0 ? Cb + (size_t)(t - t0 - 1) * csz : ck + (size_t)n * csz;
                for (int c = 0; c < dqk; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < dhv; ++j) acc += dC[(size_t)c * dhv + j] * Cprev[(size_t)c * dhv + j];
                    df[c] = acc;
                }
                for (int c = 0; c < dqk; ++c) f[c] = forget_gate(kind, fgate_pre, (size_t)bh, head, T, dqk, t, c);
                if (kind == KIND_MLSTM_SIG) {
                    dig[(size_t)bh * T + t] = di * it * (1.0 - it);
                    double sdf = 0.0;
                    for (int c = 0; c < dqk; ++c) sdf += df[c];
                    dfg[(size_t)bh * T + t] = sdf * f[0] * (1.0 - f[0]);
                } else if (kind == KIND_SCALAR) {
                    for (int c = 0; c < dqk; ++c) dscal[bh] += df[c] * f[c] * (1.0 - f[c]);
                } else {
                    for (int c = 0; c < dqk; ++c) {
                        const double x = fgate_pre[((size_t)bh * T + t) * dqk + c];
                        dfg[((size_t)bh * T + t) * dqk + c] = df[c] * f[c] * (1.0 - sigmoid(x)) / 16.0;
                    }
                }
            }
        }
        /* the initial state enters C_1 through the first step's forget gate:
           dL/dC_0 = diag(f_1) dC_1 (dcT itself when T = 0) */
        if (dc0) {
            double* out = dc0 + (size_t)bh * csz;
            if (T > 0)
                for (int c = 0; c < dqk; ++c) f[c] = forget_gate(kind, fgate_pre, (size_t)bh, head, T, dqk, 0, c);
            for (int c = 0; c < dqk; ++c)
                for (int j = 0; j < dhv; ++j) out[(size_t)c * dhv + j] = (T > 0 ? f[c] : 1.0) * dC[(size_t)c * dhv + j];
        }
        free(C); free(dC); free(ck); free(Cb); free(f); free(df);
    }
    if (kind == KIND_SCALAR) {
        for (int hh = 0; hh < H; ++hh) dfg[hh] = 0.0;
        for (long bh = 0; bh < nbh; ++bh) dfg[bh % H] += dscal[bh];
    }
    free(dscal);
    return bad ? -1 : 0;
}

int oracle_bwd(const double* q, const double* k, const double* v,
               const double* igate_pre, const double* fgate_pre, const double* dh,
               double* dq, double* dk, double* dv, double* dig, double* dfg,
               int B, int H, int T, int dqk, int dhv, int kind)
{
    return oracle_bwd_state(q, k, v, igate_pre, fgate_pre, NULL, dh, NULL, dq, dk, dv, dig, dfg, NULL,
                            B, H, T, dqk, dhv, kind);
}

/*
 * mLSTMexp forward (the mLSTM with an exponential input gate, a normaliser
 * state and a max state, which the TFLA research-map summary, Approach,
 * names as what mLSTMsig removes; the pages print no equations, so this is
 * the plainest reading of those words, with the forget gate of mLSTMsig):
 *
 *   i_t = exp(igate_pre_t),  f_t = sigmoid(fgate_pre_t)
 *   C_t = f_t C_{t-1} + i_t k_t v_t^T,   n_t = f_t n_{t-1} + i_t k_t    (C_0 = 0, n_0 = 0)
 *   h_t = (C_t^T q_t / sqrt(d_qk)) / max(|n_t . q_t| / sqrt(d_qk), 1)
 *
 * evaluated step by step with the max state m_t = max(log f_t + m_{t-1},
 * igate_pre_t) (m_0 = -inf) carried beside the stabilised states
 * Cs = C e^{-m}, ns = n e^{-m}:
 *
 *   Cs_t = e^{log f_t + m_{t-1} - m_t} Cs_{t-1} + e^{igate_pre_t - m_t} k_t v_t^T   (ns_t likewise)
 *   h_t  = (Cs_t^T q_t / sqrt(d)) / max(|ns_t . q_t| / sqrt(d), e^{-m_t})
 *
 * which is the same h (numerator and denominator both scaled by e^{-m_t})
 * without the overflow of e^{igate_pre}.  While no input has entered
 * (m_t = -inf: every input gate so far 0, or erased by a forget gate of 0)
 * the states are 0 and h_t = 0.  Layouts as oracle_fwd; igate_pre [B,H,T].
 */
int oracle_fwd_exp(const double* q, const double* k, const double* v,
                   const double* igate_pre, const double* fgate_pre, double* h,
                   int B, int H, int T, int dqk, int dhv)
{
    if (!q || !k || !v || !igate_pre || !fgate_pre || !h) return -1;
    if (B < 0 || H < 0 || T < 0 || dqk < 1 || dhv < 1) return -1;
    const long nbh = (long)B * H;
    const double scale = 1.0 / sqrt((double)dqk);
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        double* C = (double*)calloc((size_t)dqk * dhv, sizeof(double));
        double* n = (double*)calloc((size_t)dqk, sizeof(double));
        if (!C || !n) {
            free(C);
            free(n);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        double m = -INFINITY;
        for (int t = 0; t < T; ++t) {
            const double* qt = q + ((size_t)bh * T + t) * dqk;
            const double* kt = k + ((size_t)bh * T + t) * dqk;
            const double* vt = v + ((size_t)bh * T + t) * dhv;
            double* ht = h + ((size_t)bh * T + t) * dhv;
            const double lf = log_sigmoid(fgate_pre[(size_t)bh * T + t]);
            const double li = igate_pre[(size_t)bh * T + t];
            const double carried = lf + m;                 /* -inf when nothing is carried */
            const double m_new = carried > li ? carried : li;
            if (m_new == -INFINITY) {
                /* no input has entered: C_t = 0, n_t = 0, h_t = 0 */
                memset(C, 0, (size_t)dqk * dhv * sizeof(double));
                memset(n, 0, (size_t)dqk * sizeof(double));
                for (int j = 0; j < dhv; ++j) ht[j] = 0.0;
                m = m_new;
                continue;
            }
            const double fs = carried == -INFINITY ? 0.0 : exp(carried - m_new);
            const double is = li == -INFINITY ? 0.0 : exp(li - m_new);
            for (int c = 0; c < dqk; ++c) {
                double* row = C + (size_t)c * dhv;
                const double ik = is * kt[c];
                for (int j = 0; j < dhv; ++j) row[j] = fs * row[j] + ik * vt[j];
                n[c] = fs * n[c] + ik;
            }
            double den = 0.0;
            for (int c = 0; c < dqk; ++c) den += n[c] * qt[c];
            den = fabs(den) * scale;
            const double lower = exp(-m_new);
            const double div = den > lower ? den : lower;
            for (int j = 0; j < dhv; ++j) ht[j] = 0.0;
            for (int c = 0; c < dqk; ++c) {
                const double* row = C + (size_t)c * dhv;
                for (int j = 0; j < dhv; ++j) ht[j] += row[j] * qt[c];
            }
            for (int j = 0; j < dhv; ++j) ht[j] = ht[j] * scale / div;
            m = m_new;
        }
        free(C);
        free(n);
    }
    return bad ? -1 : 0;
}

/* the scalar gate functions, exported so tests can pin them */
double oracle_sigmoid(double x) { return sigmoid(x); }
double oracle_log_sigmoid(double x) { return log_sigmoid(x); }
