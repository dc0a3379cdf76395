/*
 * kla_oracle.c -- CPU float64 oracle for the Kalman Linear Attention (KLA)
 * scan: the forward pass, its backward pass (gradients, further below) and
 * the fused mixer (gate production, filter, readout; at the end).
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg may call it; the product path never
 * does, and this file shares no code with the HIP library.
 *
 * What it computes.  Every channel (b, h, d) of a [B, H, T, D] tensor runs
 * an independent scalar Kalman filter (Pith review of arXiv 2602.10743,
 * "Load-bearing premise" and the second major comment: diagonal matrices are
 * identified with their diagonal and the scalar recursion is applied per
 * coordinate).  The model is the linear noisy state-space model of the
 * "KLA Part 1" primer, section 2 (eqs. 2.1-2.5) in its scalar, unactuated
 * form:
 *
 *     x_t = a_t x_{t-1} + w_t,    Var(w_t) = p_t            (process noise)
 *     y_t = x_t + v_t,            precision of v_t = phi_t  (observation)
 *
 * The filter is written in the textbook covariance form (mean mu, variance
 * P), one predict step and one update step per token, as the primer's
 * section 5.1 "The Predict-Update Cycle" describes them.  The token evidence
 * enters as the information increment b_t = phi_t * y_t, which is what the
 * information-form update of the Pith review ("Circularity check": the update
 * adds the token-evidence precision) adds to the information mean.  The
 * oracle never divides by phi or p, so phi_t = 0 (a missing observation,
 * primer section 5.1: zero precision leaves the prior unchanged) and
 * p_t = 0 are handled exactly.
 *
 * Outputs, per channel and token t = 1..T (stored at time index t-1):
 *     lam[t]     = 1 / P_t          posterior precision
 *     eta[t]     = mu_t / P_t       posterior information mean
 *     eta_abs[t] = f_t * eta_abs[t-1] + |b_t|,  eta_abs[0] = |eta0|
 * where f_t = a_t P_{t-1} / Ppred_t is the forget gate of the information
 * mean (the precision ratio of the Pith review, "Core claim").  eta_abs is
 * the sum that eta would be if every contribution had the same sign; the
 * parity metric divides eta errors by it because eta itself can cancel.
 *
 * Initial state: lam0 and eta0 are the posterior natural parameters before
 * the first token (precision, information mean), one value per channel.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One channel, T tokens, element stride `stride` (= D in [B,H,T,D]). */
static void kalman_channel(const double *a, const double *p, const double *phi,
                           const double *b, double lam0, double eta0,
                           double *lam, double *eta, double *eta_abs,
                           int64_t T, int64_t stride)
{
    /* posterior at t = 0 in covariance form */
    double P = 1.0 / lam0;
    double mu = eta0 / lam0;
    double mag = fabs(eta0);

    for (int64_t t = 0; t < T; ++t) {
        const int64_t i = t * stride;
        const double at = a[i];
        const double pt = p[i];
        const double phit = phi[i];
        const double bt = b[i];

        /* predict: propagate the previous posterior through the dynamics */
        const double Ppred = at * at * P + pt;
        const double mupred = at * mu;

        /* forget gate of the information mean: a_t * P_{t-1} / Ppred_t */
        const double f = at * P / Ppred;

        /* update: fold in the token evidence (precision phi, information b).
         * S = 1 + phi * Ppred; the gain is K = phi * Ppred / S. */
        const double S = 1.0 + phit * Ppred;
        mu = (mupred + Ppred * bt) / S;
        P = Ppred / S;

        mag = f * mag + fabs(bt);

        lam[i] = 1.0 / P;
        eta[i] = mu / P;
        eta_abs[i] = mag;
    }
}

/*
 * Runs the oracle over a contiguous row-major [B, H, T, D] problem.
 * a, p, phi, b: [B,H,T,D]; lam0, eta0: [B,H,D]; lam, eta, eta_abs: [B,H,T,D].
 * nthreads <= 0 lets OpenMP choose.  Returns 0, or -1 on a bad size.
 */
int kla_oracle_scan(const double *a, const double *p, const double *phi,
                    const double *b, const double *lam0, const double *eta0,
                    double *lam, double *eta, double *eta_abs,
                    int64_t B, int64_t H, int64_t T, int64_t D, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || D < 0)
        return -1;
    const int64_t channels = B * H * D;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t c = 0; c < channels; ++c) {
        const int64_t slab = c / D;
        const int64_t d = c % D;
        const int64_t base = slab * T * D + d;
        kalman_channel(a + base, p + base, phi + base, b + base,
                       lam0[c], eta0[c], lam + base, eta + base,
                       eta_abs + base, T, D);
    }
    return 0;
}

/* Number of threads an OpenMP parallel region uses after the same request. */
int kla_oracle_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Backward pass (vector-Jacobian product) of the scan, per channel.
 *
 * Given upstream gradients g_lam[t], g_eta[t] of a scalar loss with respect
 * to the outputs lam_t, eta_t, returns the gradients with respect to every
 * input: a_t, p_t, phi_t, b_t, lam0, eta0.  This is reverse-mode
 * differentiation of the information-form step of the Pith review
 * ("Circularity check", Theorems 1 and 2):
 *
 *     d_t   = a_t^2 + p_t lam_{t-1}
 *     lam_t = lam_{t-1} / d_t + phi_t
 *     eta_t = (a_t / d_t) eta_{t-1} + b_t
 *
 * whose partial derivatives are
 *     dlam_t/dlam_{t-1} = a^2 / d^2        deta_t/dlam_{t-1} = -a p eta_{t-1} / d^2
 *     deta_t/deta_{t-1} = a / d            dlam_t/dphi_t = 1, deta_t/db_t = 1
 *     dlam_t/da_t = -2 a lam_{t-1} / d^2   deta_t/da_t = eta_{t-1} (p lam_{t-1} - a^2) / d^2
 *     dlam_t/dp_t = -lam_{t-1}^2 / d^2     deta_t/dp_t = -a lam_{t-1} eta_{t-1} / d^2
 * The states lam_t, eta_t come from the same covariance-form filter as the
 * forward oracle.  Walking t from T down to 1, the total adjoints are
 *     Lam_t = g_lam[t] + dlam_{t+1}/dlam_t Lam_{t+1} + deta_{t+1}/dlam_t Eta_{t+1}
 *     Eta_t = g_eta[t] + deta_{t+1}/deta_t Eta_{t+1}
 * and g_phi = Lam, g_b = Eta, g_a = Lam dlam/da + Eta deta/da, etc.;
 * g_lam0, g_eta0 are the adjoints carried past the first token.
 *
 * m_* are cancellation-free magnitudes of the same sums (every term taken
 * with its absolute value, |eta| replaced by eta_abs of the forward pass and
 * p lam - a^2 by p lam + a^2), used by the parity metric.
 */
static void kalman_channel_bwd(const double *a, const double *p, const double *phi,
                               const double *b, double lam0, double eta0,
                               const double *g_lam, const double *g_eta,
                               double *g_a, double *g_p, double *g_phi, double *g_b,
                               double *g_lam0, double *g_eta0,
                               double *m_a, double *m_p, double *m_phi, double *m_b,
                               double *m_lam0, double *m_eta0,
                               int64_t T, int64_t stride, double *work)
{
    /* forward states, index 0 = before the first token */
    double *LAM = work, *ETA = work + (T + 1), *ETA_ABS = work + 2 * (T + 1);
    double P = 1.0 / lam0;
    double mu = eta0 / lam0;
    LAM[0] = lam0;
    ETA[0] = eta0;
    ETA_ABS[0] = fabs(eta0);
    for (int64_t t = 1; t <= T; ++t) {
        const int64_t i = (t - 1) * stride;
        const double at = a[i];
        const double Ppred = at * at * P + p[i];
        const double mupred = at * mu;
        const double f = at * P / Ppred;
        const double S = 1.0 + phi[i] * Ppred;
        mu = (mupred + Ppred * b[i]) / S;
        P = Ppred / S;
        LAM[t] = 1.0 / P;
        ETA[t] = mu / P;
        ETA_ABS[t] = f * ETA_ABS[t - 1] + fabs(b[i]);
    }

    /* reverse sweep; (cl, ce) = adjoint contributions from the tokens after t */
    double cl = 0.0, ce = 0.0, ml = 0.0, me = 0.0;
    for (int64_t t = T; t >= 1; --t) {
        const int64_t i = (t - 1) * stride;
        const double at = a[i];
        const double pt = p[i];
        const double lp = LAM[t - 1];
        const double ep = ETA[t - 1];
        const double eap = ETA_ABS[t - 1];
        const double d = at * at + pt * lp;
        const double d2 = d * d;

        const double Lam = g_lam[i] + cl;
        const double Eta = g_eta[i] + ce;
        const double MLam = fabs(g_lam[i]) + ml;
        const double MEta = fabs(g_eta[i]) + me;

        const double dl_dlp = at * at / d2;
        const double de_dlp = -at * pt * ep / d2;
        const double de_dep = at / d;
        const double dl_da = -2.0 * at * lp / d2;
        const double de_da = ep * (pt * lp - at * at) / d2;
        const double dl_dp = -lp * lp / d2;
        const double de_dp = -at * lp * ep / d2;

        g_phi[i] = Lam;
        g_b[i] = Eta;
        g_a[i] = Lam * dl_da + Eta * de_da;
        g_p[i] = Lam * dl_dp + Eta * de_dp;

        m_phi[i] = MLam;
        m_b[i] = MEta;
        m_a[i] = MLam * fabs(dl_da) + MEta * eap * (pt * lp + at * at) / d2;
        m_p[i] = MLam * lp * lp / d2 + MEta * at * lp * eap / d2;

        cl = dl_dlp * Lam + de_dlp * Eta;
        ce = de_dep * Eta;
        ml = dl_dlp * MLam + at * pt * eap / d2 * MEta;
        me = de_dep * MEta;
    }
    *g_lam0 = cl;
    *g_eta0 = ce;
    *m_lam0 = ml;
    *m_eta0 = me;
}

/*
 * Backward oracle over a contiguous [B, H, T, D] problem.  Inputs as for
 * kla_oracle_scan plus g_lam, g_eta [B,H,T,D].  Outputs g_a, g_p, g_phi, g_b,
 * m_a, m_p, m_phi, m_b [B,H,T,D] and g_lam0, g_eta0, m_lam0, m_eta0 [B,H,D].
 * Returns 0, -1 on a bad size, -2 if scratch memory could not be allocated.
 */
int kla_oracle_scan_bwd(const double *a, const double *p, const double *phi,
                        const double *b, const double *lam0, const double *eta0,
                        const double *g_lam, const double *g_eta,
                        double *g_a, double *g_p, double *g_phi, double *g_b,
                        double *g_lam0, double *g_eta0,
                        double *m_a, double *m_p, double *m_phi, double *m_b,
                        double *m_lam0, double *m_eta0,
                        int64_t B, int64_t H, int64_t T, int64_t D, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || D < 0)
        return -1;
    const int64_t channels = B * H * D;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * 3 * (size_t)(T + 1));
        if (!work) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t c = 0; c < channels; ++c) {
            if (!work)
                continue;
            const int64_t slab = c / D;
            const int64_t d = c % D;
            const int64_t base = slab * T * D + d;
            kalman_channel_bwd(a + base, p + base, phi + base, b + base, lam0[c], eta0[c],
                               g_lam + base, g_eta + base,
                               g_a + base, g_p + base, g_phi + base, g_b + base,
                               g_lam0 + c, g_eta0 + c,
                               m_a + base, m_p + base, m_phi + base, m_b + base,
                               m_lam0 + c, m_eta0 + c, T, D, work);
        }
        free(work);
    }
    return failed ? -2 : 0;
}

/*
 * ---------------------------------------------------------------------------
 * Fused mixer: gate production, filter and readout.
 *
 * A mixer channel observes its token value through an observation operator:
 * the same scalar model as above, with time-invariant dynamics (the OU decay
 * a and the process-noise scale p of the Pith review's free-parameter ledger,
 * one value per (h, d)) and a token observation
 *
 *     v_t = k_t x_t + e_t,    precision of e_t = lam_v_t   (lam_v = 0: none)
 *
 * whose operator k_t and value precision lam_v_t come from the input.  The
 * update is the textbook measurement update with operator k (innovation
 * v - k mupred, gain K = Ppred k / (k^2 Ppred + 1/lam_v), written without
 * dividing by lam_v).  The information-form update of the review
 * ("Circularity check") adds k^2 lam_v to the precision, which this update
 * reproduces.  Readout: q_t times the posterior mean, and the posterior
 * variance itself.
 *
 * Outputs per token: out = q mu, var = P, mu_abs = eta_abs * P (eta_abs the
 * cancellation-free magnitude of the information mean, with increments
 * |k lam_v v| and the forget gate f = a P_{t-1} / Ppred; |mu| <= mu_abs), and
 * per channel the final state lam_T = 1 / P_T, eta_T = mu_T / P_T.
 */
static void mixer_filter(const double *k, const double *v, const double *lv,
                         double a, double p, double lam0, double eta0,
                         double *PV, double *MU, double *MAG, int64_t T, int64_t stride)
{
    /* index 0: the prior; index t: the posterior after token t */
    double P = 1.0 / lam0;
    double mu = eta0 / lam0;
    double mag = fabs(eta0);
    PV[0] = P;
    MU[0] = mu;
    MAG[0] = mag;

    for (int64_t t = 0; t < T; ++t) {
        const int64_t i = t * stride;
        const double kt = k[i];
        const double Ppred = a * a * P + p;
        const double mupred = a * mu;
        const double f = a * P / Ppred;

        /* S = (k^2 Ppred + 1/lam_v) * lam_v, so K = Ppred k lam_v / S */
        const double S = 1.0 + kt * kt * lv[i] * Ppred;
        const double K = Ppred * kt * lv[i] / S;
        mu = mupred + K * (v[i] - kt * mupred);
        P = Ppred / S;

        mag = f * mag + fabs(kt * lv[i] * v[i]);

        PV[t + 1] = P;
        MU[t + 1] = mu;
        MAG[t + 1] = mag;
    }
}

/* The forward outputs of one channel from its filter run. */
static void mixer_channel(const double *q, const double *PV, const double *MU,
                          const double *MAG, double *out, double *var, double *mu_abs,
                          double *lamT, double *etaT, int64_t T, int64_t stride)
{
    for (int64_t t = 0; t < T; ++t) {
        const int64_t i = t * stride;
        out[i] = q[i] * MU[t + 1];
        var[i] = PV[t + 1];
        mu_abs[i] = MAG[t + 1] * PV[t + 1];
    }
    *lamT = 1.0 / PV[T];
    *etaT = MU[T] / PV[T];
}

/*
 * k, v, lv, q: [B,H,T,D]; a, p: [H,D]; lam0, eta0: [B,H,D];
 * out, var, mu_abs: [B,H,T,D]; lamT, etaT: [B,H,D].  Returns 0, -1 on a bad
 * size, -2 if scratch memory could not be allocated.
 */
int kla_oracle_mixer(const double *k, const double *v, const double *lv,
                     const double *q, const double *a, const double *p,
                     const double *lam0, const double *eta0, double *out,
                     double *var, double *mu_abs, double *lamT, double *etaT,
                     int64_t B, int64_t H, int64_t T, int64_t D, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || D < 0)
        return -1;
    const int64_t channels = B * H * D;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int failed = 0;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * 3 * (size_t)(T + 1));
        if (!work) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t c = 0; c < channels; ++c) {
            if (!work)
                continue;
            const int64_t slab = c / D;
            const int64_t d = c % D;
            const int64_t hd = (slab % H) * D + d;
            const int64_t base = slab * T * D + d;
            double *PV = work, *MU = work + (T + 1), *MAG = work + 2 * (T + 1);
            mixer_filter(k + base, v + base, lv + base, a[hd], p[hd], lam0[c], eta0[c],
                         PV, MU, MAG, T, D);
            mixer_channel(q + base, PV, MU, MAG, out + base, var + base, mu_abs + base,
                          lamT + c, etaT + c, T, D);
        }
        free(work);
    }
    return failed ? -2 : 0;
}

/*
 * ---------------------------------------------------------------------------
 * Fused mixer, backward pass (vector-Jacobian product), per channel.
 *
 * Loss = sum_t g_out[t] out_t + g_var[t] var_t with out_t = q_t eta_t / lam_t
 * and var_t = 1 / lam_t.  The readout contributes, per token, the direct
 * adjoints
 *     d/dlam_t = -g_out q eta / lam^2 - g_var / lam^2,   d/deta_t = g_out q / lam,
 *     g_q[t]   = g_out eta / lam
 * which enter the reverse sweep of the filter exactly as g_lam, g_eta do in
 * kalman_channel_bwd (same partial derivatives of Theorems 1 and 2, here
 * with the channel's a, p).  The gate adjoints (Lam_t for phi_t, Eta_t for
 * b_t) reach the token inputs through phi = k^2 lam_v and b = k lam_v v:
 *     g_k = Lam 2 k lam_v + Eta lam_v v,  g_lam_v = Lam k^2 + Eta k v,
 *     g_v = Eta k lam_v,
 * and the channel gates collect their per-token adjoints: g_a = sum_t (Lam
 * dlam/da + Eta deta/da), g_p likewise (summed over the batch by the caller
 * of this routine).  m_* are the cancellation-free magnitudes of the same
 * sums (absolute values of every term, |eta| replaced by its magnitude).
 */
static void mixer_channel_bwd(const double *k, const double *v, const double *lv,
                              const double *q, double a, double p, double lam0,
                              double eta0, const double *g_out, const double *g_var,
                              double *g_k, double *g_v, double *g_lv, double *g_q,
                              double *g_a, double *g_p, double *g_lam0, double *g_eta0,
                              double *m_k, double *m_v, double *m_lv, double *m_q,
                              double *m_a, double *m_p, double *m_lam0, double *m_eta0,
                              int64_t T, int64_t stride, double *work)
{
    /* forward states (index 0 = before the first token): precision, information
     * mean and its magnitude from the same filter run as the forward outputs */
    double *LAM = work, *ETA = work + (T + 1), *EABS = work + 2 * (T + 1);
    mixer_filter(k, v, lv, a, p, lam0, eta0, LAM, ETA, EABS, T, stride);
    for (int64_t t = 0; t <= T; ++t) {
        const double P = LAM[t];
        LAM[t] = 1.0 / P;
        ETA[t] = ETA[t] / P;
    }

    double cl = 0.0, ce = 0.0, ml = 0.0, me = 0.0;
    double ga = 0.0, gp = 0.0, ma = 0.0, mp = 0.0;
    for (int64_t t = T; t >= 1; --t) {
        const int64_t i = (t - 1) * stride;
        const double kt = k[i], vt = v[i], lvt = lv[i], qt = q[i];
        const double lam = LAM[t], eta = ETA[t];

        /* readout adjoints of this token */
        const double gl_dir = -(g_out[i] * qt * eta + g_var[i]) / (lam * lam);
        const double ge_dir = g_out[i] * qt / lam;
        g_q[i] = g_out[i] * eta / lam;
        m_q[i] = fabs(g_out[i]) * EABS[t] / lam;
        const double ml_dir = (fabs(g_out[i] * qt) * EABS[t] + fabs(g_var[i])) / (lam * lam);
        const double me_dir = fabs(g_out[i] * qt) / lam;

        /* the filter step t, as in kalman_channel_bwd */
        const double lp = LAM[t - 1], ep = ETA[t - 1], eap = EABS[t - 1];
        const double d = a * a + p * lp;
        const double d2 = d * d;
        const double Lam = gl_dir + cl;
        const double Eta = ge_dir + ce;
        const double MLam = ml_dir + ml;
        const double MEta = me_dir + me;

        ga += Lam * (-2.0 * a * lp / d2) + Eta * ep * (p * lp - a * a) / d2;
        gp += Lam * (-lp * lp / d2) + Eta * (-a * lp * ep / d2);
        ma += MLam * 2.0 * a * lp / d2 + MEta * eap * (p * lp + a * a) / d2;
        mp += MLam * lp * lp / d2 + MEta * a * lp * eap / d2;

        /* through phi = k^2 lam_v and b = k lam_v v */
        g_k[i] = Lam * 2.0 * kt * lvt + Eta * lvt * vt;
        g_lv[i] = Lam * kt * kt + Eta * kt * vt;
        g_v[i] = Eta * kt * lvt;
        m_k[i] = MLam * fabs(2.0 * kt * lvt) + MEta * fabs(lvt * vt);
        m_lv[i] = MLam * kt * kt + MEta * fabs(kt * vt);
        m_v[i] = MEta * fabs(kt * lvt);

        cl = a * a / d2 * Lam - a * p * ep / d2 * Eta;
        ce = a / d * Eta;
        ml = a * a / d2 * MLam + a * p * eap / d2 * MEta;
        me = a / d * MEta;
    }
    *g_a = ga;
    *g_p = gp;
    *m_a = ma;
    *m_p = mp;
    *g_lam0 = cl;
    *g_eta0 = ce;
    *m_lam0 = ml;
    *m_eta0 = me;
}

/*
 * k, v, lv, q, g_out, g_var: [B,H,T,D]; a, p: [H,D]; lam0, eta0: [B,H,D].
 * Outputs g_k, g_v, g_lv, g_q (+ m_*) [B,H,T,D]; g_a, g_p (+ m_a, m_p)
 * [H,D], summed over the batch in order b = 0..B-1; g_lam0, g_eta0 (+ m_*)
 * [B,H,D].  Returns 0, -1 on a bad size, -2 if scratch memory failed.
 */
int kla_oracle_mixer_bwd(const double *k, const double *v, const double *lv,
                         const double *q, const double *a, const double *p,
                         const double *lam0, const double *eta0,
                         const double *g_out, const double *g_var,
                         double *g_k, double *g_v, double *g_lv, double *g_q,
                         double *g_a, double *g_p, double *g_lam0, double *g_eta0,
                         double *m_k, double *m_v, double *m_lv, double *m_q,
                         double *m_a, double *m_p, double *m_lam0, double *m_eta0,
                         int64_t B, int64_t H, int64_t T, int64_t D, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || D < 0)
        return -1;
    const int64_t channels = B * H * D;
    int failed = 0;
    /* per (b, h, d) channel sums of the gate adjoints, added over b below */
    double *part = (double *)malloc(sizeof(double) * 4 * (size_t)(channels > 0 ? channels : 1));
    if (!part)
        return -2;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * 3 * (size_t)(T + 1));
        if (!work) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t c = 0; c < channels; ++c) {
            if (!work)
                continue;
            const int64_t slab = c / D;
            const int64_t d = c % D;
            const int64_t hd = (slab % H) * D + d;
            const int64_t base = slab * T * D + d;
            mixer_channel_bwd(k + base, v + base, lv + base, q + base, a[hd], p[hd],
                              lam0[c], eta0[c], g_out + base, g_var + base,
                              g_k + base, g_v + base, g_lv + base, g_q + base,
                              part + 4 * c, part + 4 * c + 1, g_lam0 + c, g_eta0 + c,
                              m_k + base, m_v + base, m_lv + base, m_q + base,
                              part + 4 * c + 2, part + 4 * c + 3, m_lam0 + c, m_eta0 + c,
                              T, D, work);
        }
        free(work);
    }
    for (int64_t hd = 0; hd < H * D; ++hd) {
        g_a[hd] = g_p[hd] = m_a[hd] = m_p[hd] = 0.0;
    }
    for (int64_t c = 0; c < channels; ++c) {
        const int64_t hd = ((c / D) % H) * D + c % D;
        g_a[hd] += part[4 * c];
        g_p[hd] += part[4 * c + 1];
        m_a[hd] += part[4 * c + 2];
        m_p[hd] += part[4 * c + 3];
    }
    free(part);
    return failed ? -2 : 0;
}
