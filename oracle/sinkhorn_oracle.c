/*
 * fp64 CPU oracle for log-domain Sinkhorn.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library.  The product path (the HIP library) never calls it and
 * shares no code with it.  It is plain and slow on purpose: every step is the
 * textbook definition, written out, in double precision, from the fp32 inputs
 * upcast to double.
 *
 * Sources (page titles as printed on gist.science):
 *  - "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
 *    technical summary, "Problemstellung" (EOT between weighted point clouds
 *    solved by Sinkhorn iterations), "Methodik" intro (squared Euclidean cost)
 *    and "Methodik" section 1 (the stabilised log-domain update: a potential
 *    is minus eps times a log-sum-exp over the other side of
 *    (other potential - cost)/eps; the other update is symmetric).
 *    Section 2 of the same page states the log-sum-exp reductions are exact.
 *  - The Birkhoff projection pages ("Aceleración de la Proyección de Birkhoff
 *    para Hiper-conexiones ...", section 2 and its French twin): projecting a
 *    4x4 matrix onto the doubly-stochastic matrices is entropic OT with unit
 *    marginals, iterated by Sinkhorn-Knopp; section 2.1 subtracts the maximum
 *    before exponentiating; section 1 names 20 fixed iterations. Section 2.1
 *    also solves the dual by Newton's method in the 3 free variables left
 *    after removing the shift, with closed-form gradient and Hessian;
 *    section 2.2 differentiates the projection implicitly, with the matrix of
 *    the last Newton step.
 *
 * Convention (the pages put log b inside the log-sum-exp; here eps*log a sits
 * outside it, which gives the same plan with f' = f + eps log a and
 * g' = g + eps log b):
 *
 *   C_ij = sum_k (x_ik - y_jk)^2                          (direct difference)
 *   f_i  <- eps*log a_i - eps*LSE_j((g_j - C_ij)/eps)
 *   g_j  <- eps*log b_j - eps*LSE_i((f_i - C_ij)/eps)    (with the new f)
 *   LSE(v) = M + log(sum exp(v - M)),  M = max v          (two passes)
 *   P_ij = exp((f_i + g_j - C_ij)/eps)                     (never stored)
 *
 * One iteration is one f half-step followed by one g half-step.  f and g are
 * in/out: the first half-step reads g.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static double sq_dist(const double *p, const double *q, int d)
{
    double c = 0.0;
    for (int k = 0; k < d; ++k) {
        double t = p[k] - q[k];
        c += t * t;
    }
    return c;
}

/*
 * Cosine cost ("FlashSinkhorn ...", significance section: the method applies
 * to the squared Euclidean cost and to the cosine distance after
 * normalisation): C = 1 - p.q / (|p| |q|), from its definition. Undefined
 * for a zero vector (NaN here).
 */
static double cos_dist(const double *p, const double *q, int d)
{
    double pq = 0.0, pp = 0.0, qq = 0.0;
    for (int k = 0; k < d; ++k) {
        pq += p[k] * q[k];
        pp += p[k] * p[k];
        qq += q[k] * q[k];
    }
    return 1.0 - pq / (sqrt(pp) * sqrt(qq));
}

/* Cost kinds: 0 squared Euclidean, 1 cosine. */
static double cost_of(const double *p, const double *q, int d, int kind)
{
    return kind == 1 ? cos_dist(p, q, d) : sq_dist(p, q, d);
}

/*
 * One half-step for the side whose points are P (np x d, weights w):
 *   out_i = eps*log w_i - eps*LSE_j((other_j - C(P_i, Q_j))/eps)
 * over all nq points Q_j with potentials other_j.  rows == NULL updates every
 * i in [0, np) and writes out[i]; otherwise it updates rows[r] for
 * r in [0, nrows) and writes out[r].
 */
static void half_update_kind(const double *P, const double *Q, const double *w,
                             const double *other, int64_t np, int64_t nq, int d,
                             double eps, const int64_t *rows, int64_t nrows,
                             double *out, int kind)
{
    int64_t count = rows ? nrows : np;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < count; ++r) {
        int64_t i = rows ? rows[r] : r;
        const double *pi = P + i * (int64_t)d;
        double mx = -INFINITY;
        for (int64_t j = 0; j < nq; ++j) {
            double v = (other[j] - cost_of(pi, Q + j * (int64_t)d, d, kind)) / eps;
            if (v > mx)
                mx = v;
        }
        double s = 0.0;
        for (int64_t j = 0; j < nq; ++j) {
            double v = (other[j] - cost_of(pi, Q + j * (int64_t)d, d, kind)) / eps;
            s += exp(v - mx);
        }
        out[r] = eps * log(w[i]) - eps * (mx + log(s));
    }
}

void oracle_half_update(const double *P, const double *Q, const double *w,
                        const double *other, int64_t np, int64_t nq, int d,
                        double eps, const int64_t *rows, int64_t nrows,
                        double *out)
{
    half_update_kind(P, Q, w, other, np, nq, d, eps, rows, nrows, out, 0);
}

/*
 * iters alternating iterations at one eps, in place on f (n) and g (m).
 */
void oracle_sinkhorn_kind(const double *x, const double *y, const double *a,
                          const double *b, int64_t n, int64_t m, int d, double eps,
                          int iters, double *f, double *g, int kind)
{
    for (int k = 0; k < iters; ++k) {
        half_update_kind(x, y, a, g, n, m, d, eps, NULL, 0, f, kind);
        half_update_kind(y, x, b, f, m, n, d, eps, NULL, 0, g, kind);
    }
}

void oracle_sinkhorn(const double *x, const double *y, const double *a,
                     const double *b, int64_t n, int64_t m, int d, double eps,
                     int iters, double *f, double *g)
{
    oracle_sinkhorn_kind(x, y, a, b, n, m, d, eps, iters, f, g, 0);
}

/*
 * Statistics of the plan P_ij = exp((f_i + g_j - C_ij)/eps), never stored:
 *   cost     = sum_ij P_ij C_ij
 *   rowsum_i = sum_j P_ij,  colsum_j = sum_i P_ij
 *   marg[0]  = sum_i |rowsum_i - a_i|,  marg[1] = sum_j |colsum_j - b_j|
 * rowsum / colsum may be NULL.  Per-row and per-column partials are added in
 * index order.
 */
void oracle_plan_stats_kind(const double *x, const double *y, const double *a,
                            const double *b, const double *f, const double *g,
                            int64_t n, int64_t m, int d, double eps, double *cost,
                            double *marg, double *rowsum, double *colsum, int kind)
{
    double *rs = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *rc = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double *cs = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0, c = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double cij = cost_of(x + i * (int64_t)d, y + j * (int64_t)d, d, kind);
            double p = exp((f[i] + g[j] - cij) / eps);
            s += p;
            c += p * cij;
        }
        rs[i] = s;
        rc[i] = c;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < m; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            double cij = cost_of(x + i * (int64_t)d, y + j * (int64_t)d, d, kind);
            s += exp((f[i] + g[j] - cij) / eps);
        }
        cs[j] = s;
    }
    double tc = 0.0, mr = 0.0, mc = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        tc += rc[i];
        mr += fabs(rs[i] - a[i]);
        if (rowsum)
            rowsum[i] = rs[i];
    }
    for (int64_t j = 0; j < m; ++j) {
        mc += fabs(cs[j] - b[j]);
        if (colsum)
            colsum[j] = cs[j];
    }
    *cost = tc;
    marg[0] = mr;
    marg[1] = mc;
    free(rs);
    free(rc);
    free(cs);
}

void oracle_plan_stats(const double *x, const double *y, const double *a,
                       const double *b, const double *f, const double *g,
                       int64_t n, int64_t m, int d, double eps, double *cost,
                       double *marg, double *rowsum, double *colsum)
{
    oracle_plan_stats_kind(x, y, a, b, f, g, n, m, d, eps, cost, marg, rowsum, colsum, 0);
}

/*
 * Transport application ("FlashSinkhorn ...", Methodik section 3: the
 * barycentric projection and the gradients are weighted averages under the
 * plan, computed without storing it):
 *   out[i*dv + k] = sum_j P_ij v[j*dv + k],  P_ij = exp((f_i + g_j - C_ij)/eps)
 * Terms are added in index order j.
 */
void oracle_transport_apply(const double *x, const double *y, const double *f,
                            const double *g, int64_t n, int64_t m, int d,
                            double eps, const double *v, int dv, double *out)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n; ++i) {
        for (int k = 0; k < dv; ++k)
            out[i * dv + k] = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double p = exp((f[i] + g[j] - sq_dist(x + i * (int64_t)d, y + j * (int64_t)d, d)) / eps);
            for (int k = 0; k < dv; ++k)
                out[i * dv + k] += p * v[j * dv + k];
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Batched 4x4 Birkhoff projection: EOT with a = b = 1 and cost = -L.       */
/* ---------------------------------------------------------------------- */

static double lse4(const double v[4])
{
    double mx = v[0];
    for (int k = 1; k < 4; ++k)
        if (v[k] > mx)
            mx = v[k];
    double s = 0.0;
    for (int k = 0; k < 4; ++k)
        s += exp(v[k] - mx);
    return mx + log(s);
}

/* One iteration on one matrix: f from g, then g from the new f. */
static void birk_iter(const double L[16], double eps, double f[4], double g[4])
{
    double v[4];
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j)
            v[j] = (g[j] + L[4 * i + j]) / eps;
        f[i] = -eps * lse4(v);
    }
    for (int j = 0; j < 4; ++j) {
        for (int i = 0; i < 4; ++i)
            v[i] = (f[i] + L[4 * i + j]) / eps;
        g[j] = -eps * lse4(v);
    }
}

/* P_ij = exp((f_i + g_j + L_ij)/eps) and the larger of the worst row-sum and
 * worst column-sum deviation from 1. */
static double birk_plan(const double L[16], double eps, const double f[4],
                        const double g[4], double P[16])
{
    double err = 0.0;
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j)
            P[4 * i + j] = exp((f[i] + g[j] + L[4 * i + j]) / eps);
    for (int i = 0; i < 4; ++i) {
        double s = P[4 * i] + P[4 * i + 1] + P[4 * i + 2] + P[4 * i + 3];
        if (fabs(s - 1.0) > err)
            err = fabs(s - 1.0);
    }
    for (int j = 0; j < 4; ++j) {
        double s = P[j] + P[4 + j] + P[8 + j] + P[12 + j];
        if (fabs(s - 1.0) > err)
            err = fabs(s - 1.0);
    }
    return err;
}

/*
 * For each of the B matrices (L row-major, 16 doubles each): start from g = 0,
 * iterate; with tol >= 0 stop after the first iteration k >= 1 whose plan has
 * error <= tol, else after max_iters; with tol < 0 run exactly max_iters.
 * Writes the plan to P and the iteration count reached to iters_out (nullable).
 */
void oracle_birkhoff4(const double *L, int64_t B, double eps, int max_iters,
                      double tol, double *P, int32_t *iters_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < B; ++bi) {
        const double *Lb = L + 16 * bi;
        double f[4] = {0, 0, 0, 0}, g[4] = {0, 0, 0, 0};
        int k = 0;
        for (k = 1; k <= max_iters; ++k) {
            birk_iter(Lb, eps, f, g);
            if (tol >= 0.0) {
                double tmp[16];
                if (birk_plan(Lb, eps, f, g, tmp) <= tol)
                    break;
            }
        }
        if (k > max_iters)
            k = max_iters;
        birk_plan(Lb, eps, f, g, P + 16 * bi);
        if (iters_out)
            iters_out[bi] = k;
    }
}

/* Exactly iters[b] iterations for matrix b (replay of a given count); also
 * returns each plan's error in err (nullable). */
void oracle_birkhoff4_replay(const double *L, int64_t B, double eps,
                             const int32_t *iters, double *P, double *err)
{
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < B; ++bi) {
        const double *Lb = L + 16 * bi;
        double f[4] = {0, 0, 0, 0}, g[4] = {0, 0, 0, 0};
        for (int k = 0; k < iters[bi]; ++k)
            birk_iter(Lb, eps, f, g);
        double e = birk_plan(Lb, eps, f, g, P + 16 * bi);
        if (err)
            err[bi] = e;
    }
}

/* ---------------------------------------------------------------------- */
/* 4x4 projection by Newton's method on the dual, and its backward.         */
/* ---------------------------------------------------------------------- */

/*
 * Semi-dual of the 4x4 problem (a = b = 1, cost -L): for column potentials
 * g (g[3] = 0 removes the shift (f + c, g - c)), the row potentials are
 * f_i(g) = -eps LSE_j((g_j + L_ij)/eps), P_ij = exp((f_i + g_j + L_ij)/eps)
 * has unit row sums, and the concave objective
 *     F(g) = sum_i f_i(g) + sum_j g_j
 * has gradient dF/dg_j = 1 - c_j (c_j the column sums of P) and Hessian
 *     d2F/dg_j dg_k = -(c_j delta_jk - sum_i P_ij P_ik) / eps.
 * Row softmax with the row maximum subtracted first.
 */
static double birk_rows(const double L[16], double eps, const double g[4], double P[16],
                        double *mag)
{
    double F = g[0] + g[1] + g[2] + g[3];
    double m = fabs(g[0]) + fabs(g[1]) + fabs(g[2]) + fabs(g[3]);
    for (int i = 0; i < 4; ++i) {
        double v[4];
        for (int j = 0; j < 4; ++j)
            v[j] = (g[j] + L[4 * i + j]) / eps;
        double mx = v[0];
        for (int j = 1; j < 4; ++j)
            if (v[j] > mx)
                mx = v[j];
        double s = 0.0;
        for (int j = 0; j < 4; ++j)
            s += exp(v[j] - mx);
        for (int j = 0; j < 4; ++j)
            P[4 * i + j] = exp(v[j] - mx) / s;
        F -= eps * (mx + log(s));
        m += fabs(eps * (mx + log(s)));
    }
    if (mag)
        *mag = m;
    return F;
}

/* Solve the symmetric positive definite 3x3 system A x = r (Cholesky). */
static void spd3_solve(const double A[9], const double r[3], double x[3])
{
    double l00 = sqrt(A[0]);
    double l10 = A[3] / l00, l20 = A[6] / l00;
    double l11 = sqrt(A[4] - l10 * l10);
    double l21 = (A[7] - l20 * l10) / l11;
    double l22 = sqrt(A[8] - l20 * l20 - l21 * l21);
    double y0 = r[0] / l00;
    double y1 = (r[1] - l10 * y0) / l11;
    double y2 = (r[2] - l20 * y0 - l21 * y1) / l22;
    x[2] = y2 / l22;
    x[1] = (y1 - l21 * x[2]) / l11;
    x[0] = (y0 - l10 * x[1] - l20 * x[2]) / l00;
}

/* -H restricted to the free coordinates 0..2: (c_j delta_jk - sum_i P_ij P_ik)/eps. */
static void birk_neg_hessian(const double P[16], double eps, double A[9])
{
    for (int j = 0; j < 3; ++j)
        for (int k = 0; k < 3; ++k) {
            double s = 0.0, c = 0.0;
            for (int i = 0; i < 4; ++i) {
                s += P[4 * i + j] * P[4 * i + k];
                c += P[4 * i + j];
            }
            A[3 * j + k] = ((j == k ? c : 0.0) - s) / eps;
        }
}

/*
 * Newton's method on F from g = 0, with a backtracking (Armijo) line search:
 * the step length halves until F rises by at least 1e-4 of the linear
 * prediction, less the rounding of F itself (1e-13 of the magnitude of its
 * terms), so that steps below the resolution of F are accepted as they are.
 * Before each step the plan of the current g is formed; with tol >= 0 the
 * loop stops when its worst column-sum error (rows are exact) is <= tol,
 * else after max_iters steps; tol < 0 runs exactly max_iters steps.
 * iters_out (nullable) gets the number of Newton steps taken; P the plan.
 */
void oracle_birkhoff4_newton(const double *L, int64_t B, double eps, int max_iters,
                             double tol, double *P, int32_t *iters_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < B; ++bi) {
        const double *Lb = L + 16 * bi;
        double g[4] = {0, 0, 0, 0}, Pc[16];
        int k = 0;
        for (;;) {
            double mag;
            double F = birk_rows(Lb, eps, g, Pc, &mag);
            double grad[3], err = 0.0;
            for (int j = 0; j < 4; ++j) {
                double c = Pc[j] + Pc[4 + j] + Pc[8 + j] + Pc[12 + j];
                if (fabs(c - 1.0) > err)
                    err = fabs(c - 1.0);
                if (j < 3)
                    grad[j] = 1.0 - c;
            }
            if ((tol >= 0.0 && err <= tol) || k >= max_iters)
                break;
            double A[9], step[3];
            birk_neg_hessian(Pc, eps, A);
            spd3_solve(A, grad, step); /* ascent direction: (-H)^-1 grad */
            double slope = grad[0] * step[0] + grad[1] * step[1] + grad[2] * step[2];
            double t = 1.0;
            for (int ls = 0; ls < 60; ++ls) {
                double gt[4] = {g[0] + t * step[0], g[1] + t * step[1], g[2] + t * step[2], 0.0};
                double tmp[16];
                if (birk_rows(Lb, eps, gt, tmp, NULL) >= F + 1e-4 * t * slope - 1e-13 * mag)
                    break;
                t *= 0.5;
            }
            for (int j = 0; j < 3; ++j)
                g[j] += t * step[j];
            ++k;
        }
        for (int e = 0; e < 16; ++e)
            P[16 * bi + e] = Pc[e];
        if (iters_out)
            iters_out[bi] = k;
    }
}

/*
 * Backward of the projection by implicit differentiation. With P the
 * projection of L, G = dl/dP and r_i = sum_j P_ij G_ij:
 *   direct part      dl/dL_ij |g fixed = P_ij (G_ij - r_i) / eps,
 *   through g        dl/dg_j = sum_i P_ij (G_ij - r_i) / eps   (j = 0..2),
 *   and the optimality 1 - c(g, L) = 0 gives dg = H^-1 (dc/dL) dL, so
 *   dl/dL_il = P_il (G_il - r_i + lam_l - (P lam)_i) / eps,
 * with -H lam = -dl/dg, i.e. lam = H^-1 dl/dg on coordinates 0..2, lam_3 = 0,
 * and H the Hessian of F at the solution (the matrix of the last Newton
 * step). gradL (B x 16) receives dl/dL.
 */
void oracle_birkhoff4_backward(const double *P, const double *G, int64_t B, double eps,
                               double *gradL)
{
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < B; ++bi) {
        const double *Pb = P + 16 * bi, *Gb = G + 16 * bi;
        double r[4];
        for (int i = 0; i < 4; ++i) {
            r[i] = 0.0;
            for (int j = 0; j < 4; ++j)
                r[i] += Pb[4 * i + j] * Gb[4 * i + j];
        }
        double w[3];
        for (int j = 0; j < 3; ++j) {
            w[j] = 0.0;
            for (int i = 0; i < 4; ++i)
                w[j] += Pb[4 * i + j] * (Gb[4 * i + j] - r[i]) / eps;
        }
        /* lam = H^-1 w = -(-H)^-1 w */
        double A[9], mlam[3];
        birk_neg_hessian(Pb, eps, A);
        spd3_solve(A, w, mlam);
        double lam[4] = {-mlam[0], -mlam[1], -mlam[2], 0.0};
        for (int i = 0; i < 4; ++i) {
            double pl = 0.0;
            for (int l = 0; l < 4; ++l)
                pl += Pb[4 * i + l] * lam[l];
            for (int l = 0; l < 4; ++l)
                gradL[16 * bi + 4 * i + l] =
                    Pb[4 * i + l] * (Gb[4 * i + l] - r[i] + lam[l] - pl) / eps;
        }
    }
}
