/*
 * kla_oracle.c -- CPU float64 oracle for the Kalman Linear Attention (KLA)
 * scan forward pass.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
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
