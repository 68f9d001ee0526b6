/*
 * Plain fp64 CPU oracle of alpha-entmax attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may call
 * this file. It shares no code with the GPU library and is written for a
 * reader who checks it against the pages by eye: no blocking, no fusion, every
 * quantity computed straight from its definition, in double precision.
 *
 * Sources (gist.science summaries of "AdaSplash-2: Faster Differentiable Sparse
 * Attention"; the pages give prose, no formulas beyond the bound of
 * Proposition 1):
 *   - alpha-entmax gives a sparse, differentiable distribution with exact zeros;
 *     its normaliser tau plays the role of log-sum-exp and is a root of a
 *     monotone equation (AdaSplash-2 (zh, ja, es) §1 "problem").
 *   - histogram initialisation: scores mapped into a unit window, B bins,
 *     tau_h solves the B-bin problem, tau* - h < tau_h <= tau* with h the bin
 *     width (AdaSplash-2 (zh) §2.1, AdaSplash-2 (ja) §2.1 "Proposition 1",
 *     AdaSplash-2 (es) §2A).
 *   - block mask: a key block is marked when it holds a non-zero weight,
 *     32 blocks per 32-bit word (AdaSplash-2 (zh) §2.3, AdaSplash-2 (ja) §2.3).
 * Readings where the pages are silent (formula, scale of tau, bin grid, bin
 * representative, backward) are listed at the top of each function.
 *
 * Reading of the transform: with scores s_ij = scale * q_i . k_j,
 *   x_ij = (alpha - 1) s_ij,   p_ij = [x_ij - tau_i]_+^(1/(alpha-1)),
 * and tau_i is the unique root of f(tau) = sum_j [x_ij - tau]_+^kappa - 1,
 * kappa = 1/(alpha-1). This is the standard alpha-entmax (Peters, Niculae,
 * Martins 2019) written on the x-scale, where tau* lies in
 * [x_max - 1, x_max - n^(1-alpha)], a window of width at most 1.
 *
 * Position bias (NAPE heads: half of the heads without position encoding, half
 * with ALiBi; AdaSplash-2 (it) §4, AdaSplash-2 (zh) §4.2): a head with slope m adds
 * -m |i - j| to every score s_ij before the transform, so
 *   x_ij = (alpha - 1) (scale q_i . k_j - m |i - j|),
 * and m = 0 is a head without position encoding. Under the causal mask
 * |i - j| = i - j. Everything downstream (tau, histogram, mask, gradients) sees
 * the biased scores; the bias does not depend on q or k, so the gradient
 * formulas keep their form.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* f(tau) + 1 = sum_j [x_j - tau]_+^kappa. */
static double entmax_mass(const double *x, long n, double tau, double kappa)
{
    double s = 0.0;
    for (long j = 0; j < n; ++j) {
        double t = x[j] - tau;
        if (t > 0.0)
            s += pow(t, kappa);
    }
    return s;
}

/*
 * tau* by bisection on f(tau) = sum_j [x_j - tau]_+^kappa - 1 (AdaSplash-2 (zh, ja, es),
 * §1: tau is found by root-finding; bisection is the plain method).
 * Bracket: f(x_max - 1) >= 0 because the largest term alone is 1;
 * f(x_max - n^(1-alpha)) <= 0 because each term is at most 1/n.
 * Stops at width 1e-12 (or when the midpoint no longer moves) and returns the
 * midpoint.
 */
double oracle_entmax_tau(const double *x, long n, double alpha)
{
    double kappa = 1.0 / (alpha - 1.0);
    double xmax = -INFINITY;
    for (long j = 0; j < n; ++j)
        if (x[j] > xmax)
            xmax = x[j];
    double lo = xmax - 1.0;
    double hi = xmax - pow((double)n, 1.0 - alpha);
    for (int it = 0; it < 400 && hi - lo > 1e-12; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi)
            break;
        if (entmax_mass(x, n, mid, kappa) - 1.0 >= 0.0)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5 * (lo + hi);
}

/*
 * Histogram of one row on the anchored grid (AdaSplash-2 (zh) §2.1, AdaSplash-2 (it)
 * §2A, AdaSplash-2 (ja) §2.1, AdaSplash-2 (es) §2A: scores mapped to a unit
 * window and counted in B bins).
 * Reading: bins are the cells [m/B, (m+1)/B) of the absolute grid of step
 * h = 1/B; the window is the B cells ending with the cell of x_max, i.e.
 * T = floor(x_max * B) and bin k (0 <= k < B) counts the x with
 * floor(x * B) = T - B + 1 + k. Values below the window are not counted.
 * The row's top cell index T is returned in *T_out.
 */
void oracle_histogram(const double *x, long n, int B, int32_t *counts, int64_t *T_out)
{
    double xmax = -INFINITY;
    for (long j = 0; j < n; ++j)
        if (x[j] > xmax)
            xmax = x[j];
    int64_t T = (int64_t)floor(xmax * B);
    for (int k = 0; k < B; ++k)
        counts[k] = 0;
    for (long j = 0; j < n; ++j) {
        int64_t m = (int64_t)floor(x[j] * B);
        int64_t k = m - (T - B + 1);
        if (k >= 0 && k < B)
            counts[k] += 1;
    }
    *T_out = T;
}

/*
 * tau_h: root of the B-bin problem sum_k c_k [l_k - tau]_+^kappa = 1, where
 * each count sits at the lower edge l_k = (T - B + 1 + k)/B of its bin (reading
 * of "the n-root problem becomes a sum over B bins", AdaSplash-2 (zh) §2.1; lower
 * edges make tau_h a lower bound, Proposition 1). Bisection on
 * [l_top - 1, l_top]: at l_top - 1 the top bin alone (count >= 1) gives >= 1.
 * Returns the lower end of the final bracket, so the B-bin mass there is >= 1.
 */
double oracle_tau_from_hist(const int32_t *counts, int64_t T, int B, double alpha)
{
    double kappa = 1.0 / (alpha - 1.0);
    double ltop = (double)T / (double)B;
    double lo = ltop - 1.0, hi = ltop;
    for (int it = 0; it < 400 && hi - lo > 1e-12; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi)
            break;
        double s = 0.0;
        for (int k = 0; k < B; ++k) {
            double lk = (double)(T - B + 1 + k) / (double)B;
            double t = lk - mid;
            if (counts[k] > 0 && t > 0.0)
                s += (double)counts[k] * pow(t, kappa);
        }
        if (s - 1.0 >= 0.0)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

/* biased score of query i and key j: scale q_i . k_j - slope |i - j| */
static double score(long d, const double *qi, const double *kj, double scale, double slope,
                    long i, long j)
{
    double s = 0.0;
    for (long c = 0; c < d; ++c)
        s += qi[c] * kj[c];
    return scale * s - slope * fabs((double)(i - j));
}

/* scores of row i against keys 0..nv-1 on the x-scale */
static void row_x(long d, long i, const double *qi, const double *k, long nv, double alpha,
                  double scale, double slope, double *x)
{
    for (long j = 0; j < nv; ++j)
        x[j] = (alpha - 1.0) * score(d, qi, k + j * d, scale, slope, i, j);
}

/*
 * Dense forward for rows [r0, r1) of one query head (arrays are [n, d] row-major).
 * For each row i, with valid keys j < nv (nv = i+1 if causal, else n):
 *   x_j = (alpha-1) (scale q_i.k_j - slope |i-j|) ; tau_i = root of f (bisection above);
 *   p_j = [x_j - tau_i]_+^kappa (no renormalisation) ; o_i = sum_j p_j v_j;
 *   histogram counts and T of the row, tau_h from the B-bin problem;
 *   rowbits: bit J of the row's W = ceil(n/Bc) words (LSB first, 32 per word)
 *   is set when key block J holds a j with p_j > 0 (AdaSplash-2 (zh) §2.3);
 *   xgap_i = min_j |x_j - tau_i| (distance of the nearest score to the threshold);
 *   psum_i = sum_j p_j (equals 1 up to rounding).
 * Any output pointer may be NULL except o and tau.
 */
void oracle_attn_fwd_rows(long n, long d, const double *q, const double *k, const double *v,
                          double alpha, double scale, double slope, int causal, int B, int Bc,
                          long r0, long r1, double *o, double *tau, double *tau_h,
                          int32_t *counts, int64_t *T, uint32_t *rowbits, double *xgap,
                          double *psum)
{
    double kappa = 1.0 / (alpha - 1.0);
    long W = (n + 32 * (long)Bc - 1) / (32 * (long)Bc);
    double *x = (double *)malloc(sizeof(double) * (size_t)n);
    for (long i = r0; i < r1; ++i) {
        long nv = causal ? i + 1 : n;
        row_x(d, i, q + i * d, k, nv, alpha, scale, slope, x);
        double t = oracle_entmax_tau(x, nv, alpha);
        tau[i - r0] = t;
        double *oi = o + (i - r0) * d;
        for (long c = 0; c < d; ++c)
            oi[c] = 0.0;
        double ps = 0.0, gap = INFINITY;
        if (rowbits)
            memset(rowbits + (i - r0) * W, 0, sizeof(uint32_t) * (size_t)W);
        for (long j = 0; j < nv; ++j) {
            double diff = x[j] - t;
            if (fabs(diff) < gap)
                gap = fabs(diff);
            if (diff > 0.0) {
                double p = pow(diff, kappa);
                ps += p;
                for (long c = 0; c < d; ++c)
                    oi[c] += p * v[j * d + c];
                if (rowbits) {
                    long J = j / Bc;
                    rowbits[(i - r0) * W + J / 32] |= (uint32_t)1u << (J % 32);
                }
            }
        }
        if (xgap)
            xgap[i - r0] = gap;
        if (psum)
            psum[i - r0] = ps;
        if (counts && T) {
            oracle_histogram(x, nv, B, counts + (i - r0) * B, T + (i - r0));
            if (tau_h)
                tau_h[i - r0] = oracle_tau_from_hist(counts + (i - r0) * B, T[i - r0], B, alpha);
        }
    }
    free(x);
}

/*
 * Backward, per query row, for rows [r0, r1) of one query head.
 * Reading (the pages only say the backward also skips zero blocks): the exact
 * gradient of alpha-entmax. On the support, p = [x - tau]^kappa gives
 * dp_i/ds_j = g_i (delta_ij - g_j / sum_k g_k) with g = [x - tau]_+^(kappa-1)
 * = p^(2-alpha) (and g = 0 off the support). With dP_j = dO_i . v_j:
 *   delta_i = sum_j g_j dP_j / sum_j g_j,  dS_j = g_j (dP_j - delta_i),
 *   dq_i = scale * sum_j dS_j k_j.
 * tau must be the forward's tau of the same rows.
 */
void oracle_attn_bwd_rows(long n, long d, const double *q, const double *k, const double *v,
                          const double *dout, const double *tau, double alpha, double scale,
                          double slope, int causal, long r0, long r1, double *dq, double *delta)
{
    double kappa = 1.0 / (alpha - 1.0);
    double *x = (double *)malloc(sizeof(double) * (size_t)n);
    double *dp = (double *)malloc(sizeof(double) * (size_t)n);
    double *g = (double *)malloc(sizeof(double) * (size_t)n);
    for (long i = r0; i < r1; ++i) {
        long nv = causal ? i + 1 : n;
        row_x(d, i, q + i * d, k, nv, alpha, scale, slope, x);
        double t = tau[i - r0];
        double sg = 0.0, sgdp = 0.0;
        for (long j = 0; j < nv; ++j) {
            double diff = x[j] - t;
            g[j] = diff > 0.0 ? pow(diff, kappa - 1.0) : 0.0;
            double s = 0.0;
            for (long c = 0; c < d; ++c)
                s += dout[i * d + c] * v[j * d + c];
            dp[j] = s;
            sg += g[j];
            sgdp += g[j] * dp[j];
        }
        double del = sgdp / sg;
        if (delta)
            delta[i - r0] = del;
        double *dqi = dq + (i - r0) * d;
        for (long c = 0; c < d; ++c)
            dqi[c] = 0.0;
        for (long j = 0; j < nv; ++j) {
            double ds = g[j] * (dp[j] - del);
            if (ds != 0.0)
                for (long c = 0; c < d; ++c)
                    dqi[c] += scale * ds * k[j * d + c];
        }
    }
    free(x);
    free(dp);
    free(g);
}

/*
 * Backward, per key, for keys [j0, j1) of one KV head shared by G query heads
 * (grouped-query attention: the KV head's gradients sum over its query heads).
 * q, dout: [G, n, d]; tau, delta: [G, n] (forward tau and the delta of
 * oracle_attn_bwd_rows); slopes: [G] position-bias slopes of those heads, or NULL
 * for none. For each key j, over heads g and valid rows i:
 *   dk_j = scale * sum dS_ij q_i,   dv_j = sum p_ij dO_i.
 */
void oracle_attn_bwd_keys(long n, long d, long G, const double *q, const double *k,
                          const double *v, const double *dout, const double *tau,
                          const double *delta, double alpha, double scale,
                          const double *slopes, int causal, long j0, long j1, double *dk,
                          double *dv)
{
    double kappa = 1.0 / (alpha - 1.0);
    for (long j = j0; j < j1; ++j) {
        double *dkj = dk + (j - j0) * d, *dvj = dv + (j - j0) * d;
        for (long c = 0; c < d; ++c) {
            dkj[c] = 0.0;
            dvj[c] = 0.0;
        }
        for (long gh = 0; gh < G; ++gh) {
            const double *qg = q + gh * n * d, *dog = dout + gh * n * d;
            double slope = slopes ? slopes[gh] : 0.0;
            for (long i = causal ? j : 0; i < n; ++i) {
                double x = (alpha - 1.0) * score(d, qg + i * d, k + j * d, scale, slope, i, j);
                double diff = x - tau[gh * n + i];
                if (!(diff > 0.0))
                    continue;
                double p = pow(diff, kappa);
                double gg = pow(diff, kappa - 1.0);
                double dpij = 0.0;
                for (long c = 0; c < d; ++c)
                    dpij += dog[i * d + c] * v[j * d + c];
                double ds = gg * (dpij - delta[gh * n + i]);
                for (long c = 0; c < d; ++c) {
                    dkj[c] += scale * ds * qg[i * d + c];
                    dvj[c] += p * dog[i * d + c];
                }
            }
        }
    }
}
