/*
 * Float64 CPU oracle for the Gated DeltaNet recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (page "Inside Qwen3.8-27B: Hybrid DeltaNet Architecture,
 * 256k Context, and 24GB Local Serving", section "Gated DeltaNet Mechanics"):
 * each value head carries a fixed d x d memory matrix S.  At every token the
 * delta rule first removes what S currently associates with the (normalized)
 * key and then writes the new value under that key, with a per-token decay.
 * The page's own formula did not survive text extraction; this follows the
 * gated delta rule that matches every property the page states:
 *
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t                                  (post-update state)
 *
 * S is d_v x d_k, stored row-major [d_v][d_k] (row = value index).  Value head
 * h reads query/key head g = h / (Hv / Hqk) (contiguous groups: the 48 value
 * heads share 16 query/key heads, page "Qwen 3.8 27B Review ...", section 3
 * "Architecture: Gated DeltaNet Hybrid + FP8 Quantization").
 *
 * The token loop is strictly sequential, one token at a time, in float64.
 * Independent (sequence, value-head) chains run in parallel under OpenMP;
 * that changes no arithmetic.  The row-wise form below is the recurrence
 * itself: row i of S_{t-1}(I - beta k k^T) is S_i - beta (S_i . k) k^T, which
 * depends on row i of S only.
 *
 * Layouts (all float64, contiguous, row-major):
 *   q, k   [B, T, Hqk, D]
 *   v, o   [B, T, Hv,  D]
 *   alpha, beta [B, T, Hv]
 *   h0, ht [B, Hv, D, D]   h0 may be NULL (zero state); ht may be NULL (not
 *                          emitted) and may be the same pointer as h0.
 * Returns 0, or -1 for inconsistent sizes.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One (sequence, value head) chain over T tokens.  S (D x D) is in/out. */
static void gdn_chain_f64(const double *q, const double *k, const double *v,
                          const double *alpha, const double *beta,
                          int64_t T, int64_t qk_tstride, int64_t v_tstride,
                          int64_t gate_tstride, int64_t D, double *S, double *o)
{
    for (int64_t t = 0; t < T; ++t) {
        const double *qt = q + t * qk_tstride;
        const double *kt = k + t * qk_tstride;
        const double *vt = v + t * v_tstride;
        double *ot = o + t * v_tstride;
        const double a = alpha[t * gate_tstride];
        const double b = beta[t * gate_tstride];
        for (int64_t i = 0; i < D; ++i) {
            double *Si = S + i * D;
            /* u_i = (S_{t-1} k_t)_i */
            double ui = 0.0;
            for (int64_t j = 0; j < D; ++j)
                ui += Si[j] * kt[j];
            /* row i of  alpha S_{t-1} (I - beta k k^T) + beta v k^T */
            for (int64_t j = 0; j < D; ++j)
                Si[j] = a * (Si[j] - b * ui * kt[j]) + b * vt[i] * kt[j];
            /* o_i = (S_t q_t)_i */
            double oi = 0.0;
            for (int64_t j = 0; j < D; ++j)
                oi += Si[j] * qt[j];
            ot[i] = oi;
        }
    }
}

int oracle_gdn_prefill(const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta,
                       const double *h0, double *o, double *ht,
                       int64_t B, int64_t T, int64_t Hqk, int64_t Hv, int64_t D)
{
    if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || D <= 0 || Hv % Hqk != 0)
        return -1;
    const int64_t G = Hv / Hqk;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * Hv; ++bh) {
        const int64_t b = bh / Hv, h = bh % Hv, g = h / G;
        double *S = (double *)malloc((size_t)(D * D) * sizeof(double));
        if (!S) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        if (h0)
            memcpy(S, h0 + (b * Hv + h) * D * D, (size_t)(D * D) * sizeof(double));
        else
            memset(S, 0, (size_t)(D * D) * sizeof(double));
        gdn_chain_f64(q + (b * T * Hqk + g) * D, k + (b * T * Hqk + g) * D,
                      v + (b * T * Hv + h) * D, alpha + b * T * Hv + h,
                      beta + b * T * Hv + h, T, Hqk * D, Hv * D, Hv, D, S,
                      o + (b * T * Hv + h) * D);
        if (ht)
            memcpy(ht + (b * Hv + h) * D * D, S, (size_t)(D * D) * sizeof(double));
        free(S);
    }
    return bad ? -2 : 0;
}

/*
 * One decode step: the same recurrence applied to a single token per
 * sequence (page "Inside Qwen3.8-27B ...", the note under "The Role of
 * Periodic Gated Attention": at inference the state advances one token at a
 * time).  q, k [B, Hqk, D]; v, o [B, Hv, D]; alpha, beta [B, Hv];
 * state [B, Hv, D, D] updated in place.
 */
int oracle_gdn_decode_step(const double *q, const double *k, const double *v,
                           const double *alpha, const double *beta,
                           double *state, double *o,
                           int64_t B, int64_t Hqk, int64_t Hv, int64_t D)
{
    return oracle_gdn_prefill(q, k, v, alpha, beta, state, o, state, B, 1, Hqk,
                              Hv, D);
}

/*
 * Gradients of the prefill (page "Inside Qwen3.8-27B ...", note under "The
 * Role of Periodic Gated Attention": training runs the same recurrence as
 * prefill, so its backward pass is the derivative of that recurrence).
 *
 * The scalar loss whose gradients are returned is
 *     L = sum_t <dout_t, o_t> + <dht, S_T>
 * i.e. dout is dL/do and dht is dL/dS_T (NULL = zero).  Written per step with
 * u_t = S_{t-1} k_t and d_t = beta_t (v_t - alpha_t u_t), so that
 * S_t = alpha_t S_{t-1} + d_t k_t^T, the chain rule gives, walking t from T
 * down to 1 with G = dL/dS_t (which first takes in dout_t q_t^T):
 *     dq_t     = S_t^T dout_t
 *     e        = G k_t                               (dL/dd_t)
 *     dv_t     = beta_t e
 *     dbeta_t  = e . (v_t - alpha_t u_t)
 *     dalpha_t = <G, S_{t-1}> - beta_t (e . u_t)
 *     f        = -alpha_t beta_t e                   (dL/du_t)
 *     dk_t     = G^T d_t + S_{t-1}^T f
 *     dL/dS_{t-1} = alpha_t G + f k_t^T
 * and dh0 = dL/dS_0.  dq and dk of a query/key head are the sums over the
 * value heads that share it, added in increasing value-head order.
 *
 * Layouts as for oracle_gdn_prefill; dout, dv [B,T,Hv,D]; dq, dk [B,T,Hqk,D];
 * dalpha, dbeta [B,T,Hv]; dht, dh0 [B,Hv,D,D] (dht, h0 and dh0 may be NULL).
 * The forward states S_0..S_T of one value head are kept in memory
 * ((T+1) D^2 doubles per worker).  Returns 0, -1 (sizes) or -2 (memory).
 */
int oracle_gdn_backward(const double *q, const double *k, const double *v,
                        const double *alpha, const double *beta,
                        const double *h0, const double *dout, const double *dht,
                        double *dq, double *dk, double *dv, double *dalpha,
                        double *dbeta, double *dh0,
                        int64_t B, int64_t T, int64_t Hqk, int64_t Hv, int64_t D)
{
    if (B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || D <= 0 || Hv % Hqk != 0)
        return -1;
    const int64_t G = Hv / Hqk, DD = D * D;
    const int64_t qs = Hqk * D, vs = Hv * D;
    int bad = 0;
    memset(dq, 0, (size_t)(B * T * Hqk * D) * sizeof(double));
    memset(dk, 0, (size_t)(B * T * Hqk * D) * sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < B * Hqk; ++bg) {
        const int64_t b = bg / Hqk, g = bg % Hqk;
        double *S = (double *)malloc((size_t)((T + 1) * DD) * sizeof(double));
        double *Gm = (double *)malloc((size_t)DD * sizeof(double));
        double *u = (double *)malloc((size_t)(4 * D) * sizeof(double));
        if (!S || !Gm || !u) {
#pragma omp atomic write
            bad = 1;
            free(S); free(Gm); free(u);
            continue;
        }
        double *d = u + D, *e = u + 2 * D, *f = u + 3 * D;
        const double *qg = q + b * T * qs + g * D, *kg = k + b * T * qs + g * D;
        double *dqg = dq + b * T * qs + g * D, *dkg = dk + b * T * qs + g * D;
        for (int64_t h = g * G; h < (g + 1) * G; ++h) {
            const double *vh = v + b * T * vs + h * D;
            const double *dh = dout + b * T * vs + h * D;
            const double *ah = alpha + b * T * Hv + h, *bh = beta + b * T * Hv + h;
            double *dvh = dv + b * T * vs + h * D;
            /* forward, keeping every state: S + t*DD is S_t */
            if (h0)
                memcpy(S, h0 + (b * Hv + h) * DD, (size_t)DD * sizeof(double));
            else
                memset(S, 0, (size_t)DD * sizeof(double));
            for (int64_t t = 0; t < T; ++t) {
                const double *P = S + t * DD;
                double *N = S + (t + 1) * DD;
                const double *kt = kg + t * qs, *vt = vh + t * vs;
                const double a = ah[t * Hv], be = bh[t * Hv];
                for (int64_t i = 0; i < D; ++i) {
                    double ui = 0.0;
                    for (int64_t j = 0; j < D; ++j)
                        ui += P[i * D + j] * kt[j];
                    const double di = be * (vt[i] - a * ui);
                    for (int64_t j = 0; j < D; ++j)
                        N[i * D + j] = a * P[i * D + j] + di * kt[j];
                }
            }
            /* backward */
            if (dht)
                memcpy(Gm, dht + (b * Hv + h) * DD, (size_t)DD * sizeof(double));
            else
                memset(Gm, 0, (size_t)DD * sizeof(double));
            for (int64_t t = T - 1; t >= 0; --t) {
                const double *P = S + t * DD, *N = S + (t + 1) * DD;
                const double *qt = qg + t * qs, *kt = kg + t * qs;
                const double *vt = vh + t * vs, *dot = dh + t * vs;
                const double a = ah[t * Hv], be = bh[t * Hv];
                double *dqt = dqg + t * qs, *dkt = dkg + t * qs;
                for (int64_t i = 0; i < D; ++i)
                    for (int64_t j = 0; j < D; ++j)
                        Gm[i * D + j] += dot[i] * qt[j];
                for (int64_t j = 0; j < D; ++j) {
                    double s = 0.0;
                    for (int64_t i = 0; i < D; ++i)
                        s += N[i * D + j] * dot[i];
                    dqt[j] += s;
                }
                double db = 0.0, eu = 0.0, gp = 0.0;
                for (int64_t i = 0; i < D; ++i) {
                    double ui = 0.0, ei = 0.0;
                    for (int64_t j = 0; j < D; ++j) {
                        ui += P[i * D + j] * kt[j];
                        ei += Gm[i * D + j] * kt[j];
                        gp += Gm[i * D + j] * P[i * D + j];
                    }
                    u[i] = ui;
                    e[i] = ei;
                    d[i] = be * (vt[i] - a * ui);
                    f[i] = -a * be * ei;
                    dvh[t * vs + i] = be * ei;
                    db += ei * (vt[i] - a * ui);
                    eu += ei * ui;
                }
                dbeta[(b * T + t) * Hv + h] = db;
                dalpha[(b * T + t) * Hv + h] = gp - be * eu;
                for (int64_t j = 0; j < D; ++j) {
                    double s = 0.0;
                    for (int64_t i = 0; i < D; ++i)
                        s += Gm[i * D + j] * d[i] + P[i * D + j] * f[i];
                    dkt[j] += s;
                }
                for (int64_t i = 0; i < D; ++i)
                    for (int64_t j = 0; j < D; ++j)
                        Gm[i * D + j] = a * Gm[i * D + j] + f[i] * kt[j];
            }
            if (dh0)
                memcpy(dh0 + (b * Hv + h) * DD, Gm, (size_t)DD * sizeof(double));
        }
        free(S); free(Gm); free(u);
    }
    return bad ? -2 : 0;
}

/* Team size of an OpenMP parallel region here: the number of threads the
 * chains above really run on (for reporting the CPU baseline). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

/* Sets the team size of the oracle's later parallel regions (the OpenMP
 * runtime this library is linked with, whatever else the process loaded). */
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
