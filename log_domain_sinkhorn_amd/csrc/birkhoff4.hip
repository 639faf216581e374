// Batched projection of 4x4 matrices onto the doubly-stochastic matrices.
//
// "Aceleración de la Proyección de Birkhoff para Hiper-conexiones con
// Restricción de Variedad" (and its French twin), sections 1-2: the Birkhoff
// projection is entropic OT with unit marginals and cost -L, solved by
// Sinkhorn-Knopp; section 2.1 subtracts the maximum before exponentiating;
// section 1 names the common fixed budget of 20 iterations. In base 2, with
// l_ij = L_ij * log2(e)/eps and potentials in units of eps/log2(e):
//
//   f_i = -log2 sum_j 2^(g_j + l_ij),   g_j = -log2 sum_i 2^(f_i + l_ij)
//   out_ij = 2^(f_i + g_j + l_ij)
//
// One matrix per lane, everything in registers, no cross-lane traffic (the
// page's kernel puts two matrices in a 32-lane warp and exchanges values by
// shuffles; with one matrix per lane on 64-wide wavefronts there is nothing to
// exchange). The kernel carries the log-plan u_ij = f_i + g_j + l_ij instead
// of the potentials (see birkhoff4_kernel). Convergence test: after iteration
// k the row sums of the plan 2^u are the sums the next row step forms anyway;
// only when they are all within tol of 1 are the column sums of the same
// plan, exactly as it will be written, tested too. The decision is thus taken
// on the fp32 output, and a matrix that stops is written from those entries.
#include "ot_internal.h"

#include <math.h>

namespace otsk {

namespace {

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// max-subtracted base-2 log-sum-exp of 4 values: returns m, writes
// s = sum 2^(v-m). The maximum's term is 2^0 = 1 and is not exponentiated:
// with p = max(v0, v1, v2) the maximum is max(p, v3) and the other three
// values are min(p, v3), med(v0, v1, v2) and min(v0, v1, v2), so one LSE of 4
// takes 3 exp2 (used for the first row step, whose logits may be large, and
// when a row or column sum underflows).
__device__ __forceinline__ float lse4_parts(float v0, float v1, float v2, float v3, float &s) {
    const float p = fmaxf(fmaxf(v0, v1), v2);
    const float m = fmaxf(p, v3);
    const float o1 = fminf(p, v3);
    const float o2 = __builtin_amdgcn_fmed3f(v0, v1, v2);
    const float o3 = fminf(fminf(v0, v1), v2);
    s = 1.f + (hw_exp2(o1 - m) + (hw_exp2(o2 - m) + hw_exp2(o3 - m)));
    return m;
}

// Largest deviation of a row sum or a column sum of P from 1.
__device__ __forceinline__ float plan_error(const float P[4][4]) {
    float e = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        e = fmaxf(e, fabsf((P[i][0] + P[i][1]) + (P[i][2] + P[i][3]) - 1.f));
#pragma unroll
    for (int j = 0; j < 4; ++j)
        e = fmaxf(e, fabsf((P[0][j] + P[1][j]) + (P[2][j] + P[3][j]) - 1.f));
    return e;
}

// Normaliser of one row or column of the log-plan u (four entries): d with
// sum 2^(u - d) = 1. After a row or column step every entry is at most 0 and
// the sums are at most 4, so d = log2 of the plain sum; only when that sum
// falls below 2^-100 (entries near fp32's underflow, early iterations of
// extreme logits) is the maximum subtracted first. `e` holds 2^u on entry.
__device__ __forceinline__ float normaliser4(float u0, float u1, float u2, float u3,
                                             float e0, float e1, float e2, float e3) {
    const float s = (e0 + e1) + (e2 + e3);
    if (s >= 0x1p-100f)
        return hw_log2(s);
    float sm;
    const float m = lse4_parts(u0, u1, u2, u3, sm);
    return m + hw_log2(sm);
}

// The iteration on the log-plan u_ij = f_i + g_j + l_ij itself: a row step
// (the f update) subtracts from row i the base-2 LSE of the row, a column
// step (the g update) the LSE of the column; the potentials are implicit.
// This is the alternating update above, term for term: u_ij - LSE_j(u_ij) =
// f_i' + g_j + l_ij with f_i' = -LSE_j(g_j + l_ij). Carrying u instead of
// (f, g) saves forming f_i + l_ij for every entry at every step, and after
// the first (max-subtracted) row step the entries stay <= 0, so the plain
// sum of 2^u is safe without a maximum (see normaliser4).
__global__ __launch_bounds__(256) void birkhoff4_kernel(const float *logits, int64_t batch,
                                                        float scale, int max_iters, float tol,
                                                        float *out, int32_t *iters_out) {
    const int64_t bi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (bi >= batch)
        return;
    const float4 *src = reinterpret_cast<const float4 *>(logits) + 4 * bi;
    float u[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float4 v = src[r];
        u[r][0] = v.x * scale;
        u[r][1] = v.y * scale;
        u[r][2] = v.z * scale;
        u[r][3] = v.w * scale;
    }
    float P[4][4];
    bool have_plan = false;
    int k = 0;
    if (max_iters > 0) {
        const bool check = tol >= 0.f;
        // first row step (from g = 0), with the maximum subtracted: the
        // logits may be large
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float si;
            const float mi = lse4_parts(u[i][0], u[i][1], u[i][2], u[i][3], si);
            const float d = mi + hw_log2(si);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                u[i][j] -= d;
        }
        float e[4][4];
        for (k = 1;; ++k) {
            // column step: iterate k is complete afterwards
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    e[i][j] = hw_exp2(u[i][j]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float d = normaliser4(u[0][j], u[1][j], u[2][j], u[3][j], e[0][j], e[1][j],
                                            e[2][j], e[3][j]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    u[i][j] -= d;
            }
            if (k >= max_iters)
                break;
            // the next row step's sums: the row sums of iterate k's plan
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    e[i][j] = hw_exp2(u[i][j]);
            if (check) {
                float est = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    est = fmaxf(est,
                                fabsf(((e[i][0] + e[i][1]) + (e[i][2] + e[i][3])) - 1.f));
                if (est <= tol) {
                    // rows within tol: test the columns of the same plan
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            P[i][j] = e[i][j];
                    if (plan_error(P) <= tol) {
                        have_plan = true;
                        break;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float d = normaliser4(u[i][0], u[i][1], u[i][2], u[i][3], e[i][0], e[i][1],
                                            e[i][2], e[i][3]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    u[i][j] -= d;
            }
        }
    }
    if (!have_plan) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                P[i][j] = hw_exp2(u[i][j]);
    }
    float4 *dst = reinterpret_cast<float4 *>(out) + 4 * bi;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        dst[r] = make_float4(P[r][0], P[r][1], P[r][2], P[r][3]);
    if (iters_out)
        iters_out[bi] = k;
}

}  // namespace

hipError_t launch_birkhoff4(const float *logits, int64_t batch, float eps, int max_iters, float tol,
                            float *out, int32_t *iters_out, hipStream_t s) {
    if (batch == 0)
        return hipSuccess;
    const float scale = (float)(kLog2e / (double)eps);
    const unsigned blocks = (unsigned)((batch + 255) / 256);
    hipLaunchKernelGGL(birkhoff4_kernel, dim3(blocks), dim3(256), 0, s, logits, batch, scale,
                       max_iters, tol, out, iters_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Newton's method on the dual ("Aceleración de la Proyección de Birkhoff ...",
// section 2.1) and the implicit-differentiation backward (section 2.2).
//
// Semi-dual in base 2, with l_ij = L_ij log2(e)/eps and column potentials g
// (g_3 = 0 removes the shift (f + c, g - c); 3 free variables):
//   f_i(g) = -log2 sum_j 2^(g_j + l_ij),  P_ij = 2^(f_i + g_j + l_ij),
//   F(g)   = sum_i f_i(g) + sum_j g_j   (concave),
//   dF/dg_j = 1 - c_j,   d2F/dg_j dg_k = -ln2 (c_j delta_jk - sum_i P_ij P_ik),
// c_j the column sums (rows sum to 1 by construction). Each step solves the
// 3x3 system by Cholesky and backtracks (halving) until F rises by 1e-4 of
// the linear prediction, less the rounding of F. One matrix per lane; the
// exponents g_j + l_ij, the row maxima, F and the Hessian are fp64 (fp64
// VALU issues at the fp32 rate on gfx950) and 2^x is v_exp_f32 of the
// max-subtracted exponent, so P carries fp32 rounding only, not the rounding
// of exponents of size |l| (up to ~60 for N(0, 10^2) logits).
// ---------------------------------------------------------------------------
namespace {

// Longest Newton move per step in any dual coordinate (log2 units). Only a
// guard against overflow of g: a nearly flat direction (a column with almost
// no mass) asks for a long move, and the line search, not a short cap, has to
// find how much of it to take (a cap of 32..256 made such matrices oscillate
// between the cap's ends).
constexpr double kMaxStep = 1e4;
// Halvings of the line search (2^-60 of a 1e4 move is below fp64 resolution
// of g).
constexpr int kLineSearch = 60;

// Row softmax of t_ij = g_j + l_ij: P (fp32, rows as written), returns F.
__device__ __forceinline__ double newton_rows(const double l[4][4], const double g[4],
                                              float P[4][4], double &mag) {
    double F = g[0] + g[1] + g[2];
    mag = fabs(g[0]) + fabs(g[1]) + fabs(g[2]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            t[j] = g[j] + l[i][j];
        const double m = fmax(fmax(t[0], t[1]), fmax(t[2], t[3]));
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            e[j] = hw_exp2((float)(t[j] - m));
        const float sum = (e[0] + e[1]) + (e[2] + e[3]);
        const float inv = 1.f / sum;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            P[i][j] = e[j] * inv;
        const double fi = -(m + (double)hw_log2(sum));
        F += fi;
        mag += fabs(fi);
    }
    return F;
}

// F only (line-search trials).
__device__ __forceinline__ double newton_objective(const double l[4][4], const double g[4]) {
    double F = g[0] + g[1] + g[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            t[j] = g[j] + l[i][j];
        const double m = fmax(fmax(t[0], t[1]), fmax(t[2], t[3]));
        const float sum = (hw_exp2((float)(t[0] - m)) + hw_exp2((float)(t[1] - m))) +
                          (hw_exp2((float)(t[2] - m)) + hw_exp2((float)(t[3] - m)));
        F -= m + (double)hw_log2(sum);
    }
    return F;
}

// A = diag(c) - P^T P on the free coordinates 0..2 (fp64), A symmetric.
__device__ __forceinline__ void gram3(const float P[4][4], double A[3][3], double c[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        c[j] = ((double)P[0][j] + (double)P[1][j]) + ((double)P[2][j] + (double)P[3][j]);
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int k = 0; k <= j; ++k) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s = fma((double)P[i][j], (double)P[i][k], s);
            A[j][k] = (j == k ? c[j] : 0.0) - s;
            A[k][j] = A[j][k];
        }
}

// Solve A x = r for symmetric positive (semi)definite A by Cholesky. A is
// formed from an fp32 plan, so its entries carry ~1e-7 of rounding and a
// column with no mass (its entries below fp32's range) makes it singular;
// pivots are floored at 1e-13 of the largest diagonal entry, which keeps the
// solve finite and leaves well-conditioned systems untouched.
__device__ __forceinline__ void chol3_solve(const double A[3][3], const double r[3],
                                            double x[3]) {
    const double floor_ = 1e-300 + 1e-13 * fmax(fmax(A[0][0], A[1][1]), A[2][2]);
    const double l00 = sqrt(fmax(A[0][0], floor_));
    const double l10 = A[1][0] / l00, l20 = A[2][0] / l00;
    const double l11 = sqrt(fmax(A[1][1] - l10 * l10, floor_));
    const double l21 = (A[2][1] - l20 * l10) / l11;
    const double l22 = sqrt(fmax(A[2][2] - l20 * l20 - l21 * l21, floor_));
    const double y0 = r[0] / l00;
    const double y1 = (r[1] - l10 * y0) / l11;
    const double y2 = (r[2] - l20 * y0 - l21 * y1) / l22;
    x[2] = y2 / l22;
    x[1] = (y1 - l21 * x[2]) / l11;
    x[0] = (y0 - l10 * x[1] - l20 * x[2]) / l00;
}

__global__ __launch_bounds__(256) void birkhoff4_newton_kernel(const float *logits,
                                                               int64_t batch, double scale,
                                                               int max_iters, float tol,
                                                               float *out, int32_t *iters_out) {
    const int64_t bi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (bi >= batch)
        return;
    const float4 *src = reinterpret_cast<const float4 *>(logits) + 4 * bi;
    double l[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float4 v = src[r];
        l[r][0] = v.x * scale;
        l[r][1] = v.y * scale;
        l[r][2] = v.z * scale;
        l[r][3] = v.w * scale;
    }
    double g[4] = {0.0, 0.0, 0.0, 0.0};
    float P[4][4];
    int k = 0;
    for (;;) {
        double mag;
        const double F = newton_rows(l, g, P, mag);
        if ((tol >= 0.f && plan_error(P) <= tol) || k >= max_iters)
            break;
        double A[3][3], c[4];
        gram3(P, A, c);
        const double grad[3] = {1.0 - c[0], 1.0 - c[1], 1.0 - c[2]};
        double step[3];
        chol3_solve(A, grad, step);
        // (ln2 A)^-1 grad, at most kMaxStep log2 units in any coordinate.
        double len = 0.0;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            step[j] *= 1.4426950408889634;
            len = fmax(len, fabs(step[j]));
        }
        const double shrink = len > kMaxStep ? kMaxStep / len : 1.0;
#pragma unroll
        for (int j = 0; j < 3; ++j)
            step[j] *= shrink;
        const double slope = grad[0] * step[0] + grad[1] * step[1] + grad[2] * step[2];
        // F carries ~1e-7 of rounding per row from the fp32 log2 / exp2.
        const double slack = 4e-6 + 1e-12 * mag;
        double t = 1.0;
        bool accepted = false;
        for (int ls = 0; ls < kLineSearch; ++ls) {
            const double gt[4] = {g[0] + t * step[0], g[1] + t * step[1], g[2] + t * step[2],
                                  0.0};
            if (newton_objective(l, gt) >= F + 1e-4 * t * slope - slack) {
                accepted = true;
                break;
            }
            t *= 0.5;
        }
        // No acceptable step: the plan is as close as fp32 allows; stop here.
        if (!accepted)
            break;
#pragma unroll
        for (int j = 0; j < 3; ++j)
            g[j] += t * step[j];
        ++k;
    }
    float4 *dst = reinterpret_cast<float4 *>(out) + 4 * bi;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        dst[r] = make_float4(P[r][0], P[r][1], P[r][2], P[r][3]);
    if (iters_out)
        iters_out[bi] = k;
}

// dl/dL from the projection P and dl/dP = G by the implicit function theorem
// at the solution (section 2.2), in fp64 (the kernel is bound by its 192
// bytes of HBM traffic per matrix, and the 3x3 system is ill-conditioned for
// near-permutation plans):
//   r_i = sum_j P_ij G_ij,  w_j = sum_i P_ij (G_ij - r_i)  (j = 0..2),
//   A lam = -w (A = diag(c) - P^T P, the last Newton step's matrix), lam_3 = 0,
//   dl/dL_il = P_il (G_il - r_i + lam_l - sum_j P_ij lam_j) / eps.
__global__ __launch_bounds__(256) void birkhoff4_backward_kernel(const float *plan,
                                                                 const float *grad_plan,
                                                                 int64_t batch, double inv_eps,
                                                                 float *grad_logits) {
    const int64_t bi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (bi >= batch)
        return;
    const float4 *ps = reinterpret_cast<const float4 *>(plan) + 4 * bi;
    const float4 *gs = reinterpret_cast<const float4 *>(grad_plan) + 4 * bi;
    float P[4][4];
    double G[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float4 p = ps[r], q = gs[r];
        P[r][0] = p.x, P[r][1] = p.y, P[r][2] = p.z, P[r][3] = p.w;
        G[r][0] = q.x, G[r][1] = q.y, G[r][2] = q.z, G[r][3] = q.w;
    }
    double rr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s = fma((double)P[i][j], G[i][j], s);
        rr[i] = s;
    }
    double w[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s = fma((double)P[i][j], G[i][j] - rr[i], s);
        w[j] = -s;
    }
    double A[3][3], c[4], lam3[3];
    gram3(P, A, c);
    chol3_solve(A, w, lam3);
    const double lam[4] = {lam3[0], lam3[1], lam3[2], 0.0};
    float4 *dst = reinterpret_cast<float4 *>(grad_logits) + 4 * bi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double pl = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            pl = fma((double)P[i][j], lam[j], pl);
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = (float)((double)P[i][j] * (G[i][j] - rr[i] + lam[j] - pl) * inv_eps);
        dst[i] = make_float4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

hipError_t launch_birkhoff4_newton(const float *logits, int64_t batch, float eps, int max_iters,
                                   float tol, float *out, int32_t *iters_out, hipStream_t s) {
    if (batch == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((batch + 255) / 256);
    hipLaunchKernelGGL(birkhoff4_newton_kernel, dim3(blocks), dim3(256), 0, s, logits, batch,
                       kLog2e / (double)eps, max_iters, tol, out, iters_out);
    return hipGetLastError();
}

hipError_t launch_birkhoff4_backward(const float *plan, const float *grad_plan, int64_t batch,
                                     float eps, float *grad_logits, hipStream_t s) {
    if (batch == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((batch + 255) / 256);
    hipLaunchKernelGGL(birkhoff4_backward_kernel, dim3(blocks), dim3(256), 0, s, plan, grad_plan,
                       batch, 1.0 / (double)eps, grad_logits);
    return hipGetLastError();
}

}  // namespace otsk
