/*
 * ot_sinkhorn.h -- C ABI of the MI355X (gfx950) log-domain Sinkhorn library.
 *
 * Problem (page "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
 * technical summary, "Problemstellung" and "Methodik"): entropic optimal
 * transport between two weighted point clouds x (n points) and y (m points)
 * in R^d with weights a and b and squared Euclidean cost
 * C_ij = |x_i - y_j|^2, solved by stabilised log-domain Sinkhorn iterations.
 *
 * Convention used by every call below (the page's "Methodik" section 1 writes
 * the same update with log b_j inside the log-sum-exp instead; the two give
 * the same plan with f = f' + eps log a, g = g' + eps log b):
 *
 *   f_i <- eps*log a_i - eps*LSE_j((g_j - C_ij)/eps)
 *   g_j <- eps*log b_j - eps*LSE_i((f_i - C_ij)/eps)      (uses the new f)
 *   P_ij = exp((f_i + g_j - C_ij)/eps)                      (the plan)
 *
 * One iteration is one f update followed by one g update. C and P are never
 * stored in memory; they are formed tile by tile on chip (page section
 * "Methodik" 2).
 *
 * General rules
 *  - Every array argument is a DEVICE pointer to memory the caller owns.
 *    The library keeps no buffer between calls; temporary device memory is
 *    taken with hipMallocAsync on `stream` and released with hipFreeAsync on
 *    the same stream.
 *  - Point arrays are contiguous row-major fp32: x[i*d + k], y[j*d + k].
 *    Potentials and weights are contiguous fp32 vectors.  Pointers must be
 *    4-byte aligned.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    All work is enqueued on it and the call returns without synchronising,
 *    except where a result is stated to be written to host memory.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call returns OT_ERROR_INVALID_VALUE and enqueues nothing.
 *  - Preconditions that are NOT checked (checking would need a device read):
 *    finite inputs, a_i > 0, b_j > 0, and for d >= 32 the range of the
 *    split-f16 matrix-core products, (2 log2(e)/eps) * max_ik |x_ik - c_k| *
 *    max_jk |y_jk - c_k| < 2^30, where c = (mean_i x_i + mean_j y_j) / 2 is
 *    the centre the d >= 32 calls subtract from both clouds before forming
 *    products (the cost does not change; x and y are replaced by their
 *    unit-normalised rows and eps by 2 eps in the cosine calls). Violations
 *    give NaN or inf results, not an error code.
 *  - Outputs must not alias inputs unless a call says otherwise.
 *  - Calls are stateless; concurrent calls on different streams are safe.
 *  - Each call takes at most one temporary allocation, sized up front.
 *    When it cannot be had the call returns OT_ERROR_OUT_OF_MEMORY before
 *    anything is enqueued.
 *  - Graph capture: ot_sinkhorn_solve, ot_plan_stats, ot_transport_apply and
 *    ot_birkhoff_project_batched have been captured into HIP graphs on
 *    `stream` (their temporary memory becomes the graph's stream-ordered
 *    allocation) and replayed with results identical to direct calls. A
 *    graph that also held the cosine calls, ot_barycentric_map and
 *    ot_cost_gradient_x faulted on replay, cause unknown; those four calls
 *    return OT_ERROR_NOT_SUPPORTED, enqueueing nothing, when `stream` is
 *    capturing.
 */
#ifndef OT_SINKHORN_H
#define OT_SINKHORN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OT_SUCCESS = 0,
    OT_ERROR_INVALID_VALUE = 1,  /* bad argument; nothing was enqueued          */
    OT_ERROR_NOT_SUPPORTED = 2,  /* valid but unsupported (e.g. d > OT_MAX_DIM) */
    OT_ERROR_OUT_OF_MEMORY = 3,  /* a temporary device allocation failed         */
    OT_ERROR_LAUNCH_FAILURE = 4  /* a HIP call or kernel launch reported an error */
} ot_status;

/* Largest feature dimension d the point-cloud calls accept: up to 192 the
 * matrix-core kernels work on 32x32 tiles with a row's operands in registers,
 * from 193 to 448 on 16x16 tiles (half the row-operand registers per lane),
 * from 449 to 1024 tiled like a matrix product, both sides streamed through
 * LDS in 32-coordinate stages. */
#define OT_MAX_DIM 1024

/* Largest d of the transport calls (ot_transport_apply, ot_barycentric_map,
 * ot_cost_gradient_x): all of OT_MAX_DIM. Above d = 192, and from d = 129
 * with more than 128 value channels, one pass over the columns forms each
 * score once and applies it to every value channel (up to 1024). */
#define OT_MAX_TRANSPORT_DIM 1024

/* Human-readable name of a status code (static string, never NULL). */
const char *ot_status_string(ot_status s);

/*
 * ot_sinkhorn_solve -- `iters` alternating log-domain Sinkhorn iterations at
 * regularisation eps (page "FlashSinkhorn ...", "Methodik" section 1).
 *
 *   x      [n*d]  source points            y  [m*d]  target points
 *   a      [n]    source weights (> 0)     b  [m]    target weights (> 0)
 *   n, m   >= 1   d in [1, OT_MAX_DIM]     eps > 0 and finite
 *   iters  >= 0   (0 leaves f and g untouched)
 *   f      [n]    in/out; overwritten by the first f update
 *   g      [m]    in/out; read by the first f update (zeros = cold start),
 *                 holds the last g update on return
 *
 * Warm start (e.g. a decreasing eps schedule) is a second call with the f, g
 * of the first.  f and g must not overlap each other or any input.
 * Errors: INVALID_VALUE (null pointer, n or m < 1, d < 1, eps <= 0 or not
 * finite, iters < 0), NOT_SUPPORTED (d > OT_MAX_DIM, n or m > 2^34),
 * OUT_OF_MEMORY, LAUNCH_FAILURE.
 */
ot_status ot_sinkhorn_solve(const float *x, const float *y, const float *a,
                            const float *b, int64_t n, int64_t m, int32_t d,
                            float eps, int32_t iters, float *f, float *g,
                            void *stream);

/* Bytes of the static device array ot_sinkhorn_solve_no_alloc works in, per GPU. */
#define OT_NO_ALLOC_SCRATCH_BYTES (128ull << 20)

/*
 * ot_sinkhorn_solve_no_alloc -- for callers that cannot allocate device
 * memory: code under HIP graph capture that must not record allocation
 * nodes, tight serving loops, harnesses that forbid hipMalloc. It computes
 * exactly what ot_sinkhorn_solve computes (same kernels, same results) but
 * takes its scratch from a static device array of OT_NO_ALLOC_SCRATCH_BYTES
 * (128 MiB) that the library holds on every GPU it runs on until the process
 * ends, and calls no allocating routine.
 *
 * Scratch needed (n', m' = n, m rounded up to 256; kp = d rounded up to 32):
 * the records of both clouds, 32 (n' + m') bytes for d < 32 and
 * (8 kp + 8)(n' + m') bytes for d >= 32, plus 16 bytes per row and column
 * split of the larger half-step (plus about 4 KiB per coordinate for
 * d >= 32). n = m = 65536 needs 36 MiB at d = 3 and 69.25 MiB at d = 64,
 * 131072 x 98304 at d = 3 needs 40 MiB; 65536 x 65536 at d = 128 (133.5 MiB)
 * does not fit. A problem whose scratch exceeds the array returns
 * OT_ERROR_NOT_SUPPORTED and enqueues nothing.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (the solve writes every part it reads, so nothing needs
 * clearing): calls that overlap in time on one GPU (from other threads or on
 * other streams) race and must be serialised by the caller. The first call
 * on a GPU looks up the array's address on that GPU (stream's device).
 * Arguments, results and other errors as ot_sinkhorn_solve.
 */
ot_status ot_sinkhorn_solve_no_alloc(const float *x, const float *y,
                                     const float *a, const float *b,
                                     int64_t n, int64_t m, int32_t d, float eps,
                                     int32_t iters, float *f, float *g,
                                     void *stream);

/*
 * ot_sinkhorn_solve_eps_scaling -- `stages` calls of ot_sinkhorn_solve with
 * eps_s = eps0 * (eps_end/eps0)^(s/(stages-1)), s = 0..stages-1 (eps0 alone
 * when stages == 1), `iters_per_stage` iterations each, each stage starting
 * from the previous stage's f and g.  The schedule is not on the pages; it
 * is the usual warm-started decreasing-eps driver around the same update.
 * Arguments as ot_sinkhorn_solve; stages >= 1, eps0 and eps_end > 0 and
 * finite, iters_per_stage >= 0.
 */
ot_status ot_sinkhorn_solve_eps_scaling(const float *x, const float *y,
                                        const float *a, const float *b,
                                        int64_t n, int64_t m, int32_t d,
                                        float eps0, float eps_end,
                                        int32_t stages, int32_t iters_per_stage,
                                        float *f, float *g, void *stream);

/*
 * ot_plan_stats -- statistics of the plan P_ij = exp((f_i + g_j - C_ij)/eps)
 * without storing it (page "FlashSinkhorn ...", "Methodik" section 3: the
 * transport plan is applied by streaming, never materialised):
 *
 *   cost    = sum_ij P_ij * C_ij                       (device double [1])
 *   marg[0] = sum_i |sum_j P_ij - a_i|                   (device double [2])
 *   marg[1] = sum_j |sum_i P_ij - b_j|
 *
 * Either output may be NULL to skip it (both NULL is INVALID_VALUE); a, b
 * may be NULL when marg is NULL.  Per-pair terms are fp32 with fp64 partial
 * sums combined in a fixed order, so repeated calls give identical results.
 * Errors as ot_sinkhorn_solve.
 */
ot_status ot_plan_stats(const float *x, const float *y, const float *a,
                        const float *b, const float *f, const float *g,
                        int64_t n, int64_t m, int32_t d, float eps,
                        double *cost, double *marg, void *stream);

/* ot_plan_cost -- ot_plan_stats with cost only (device double [1]). */
ot_status ot_plan_cost(const float *x, const float *y, const float *f,
                       const float *g, int64_t n, int64_t m, int32_t d,
                       float eps, double *cost, void *stream);

/* ot_marginal_error -- ot_plan_stats with marg only (device double [2] =
 * {row L1 error, column L1 error}). */
ot_status ot_marginal_error(const float *x, const float *y, const float *a,
                            const float *b, const float *f, const float *g,
                            int64_t n, int64_t m, int32_t d, float eps,
                            double *marg, void *stream);

/* Largest number of value channels ot_transport_apply accepts. */
#define OT_MAX_VALUE_DIM 1024

/*
 * ot_transport_apply -- out_i = sum_j P_ij v_j for the plan
 * P_ij = exp((f_i + g_j - C_ij)/eps) of the given potentials, without storing
 * P (page "FlashSinkhorn ...", "Methodik" section 3: applying the transport
 * plan is an attention-like weighted average over the streamed tiles).
 *
 *   v    [m*dv]  values attached to the target points, row-major
 *   dv   in [1, OT_MAX_VALUE_DIM]
 *   out  [n*dv]  row-major; must not overlap any input
 *
 * Other arguments as ot_plan_stats. d < 32: the exponent of each P_ij is
 * formed in fp64 and exponentiated in fp32. d >= 32: log2 P_ij comes from the
 * split-f16 products of the solve (fp32 accumulation) and P.v from products
 * of three-part bf16 splits of P and v. Sums over j are fp32 within a column
 * range and fp64 across ranges, in a fixed order.
 * Errors: INVALID_VALUE (null pointer, sizes < 1, bad eps, overlap),
 * NOT_SUPPORTED (d > OT_MAX_TRANSPORT_DIM, dv > OT_MAX_VALUE_DIM),
 * OUT_OF_MEMORY, LAUNCH_FAILURE.
 */
ot_status ot_transport_apply(const float *x, const float *y, const float *f,
                             const float *g, int64_t n, int64_t m, int32_t d,
                             float eps, const float *v, int32_t dv, float *out,
                             void *stream);

/*
 * ot_barycentric_map -- out_i = sum_j P_ij y_j / a_i (n*d): the barycentric
 * projection of each source point under the plan (page "FlashSinkhorn ...",
 * "Methodik" section 3). a [n] are the source weights (> 0). d is limited to
 * OT_MAX_TRANSPORT_DIM, as for ot_transport_apply.
 */
ot_status ot_barycentric_map(const float *x, const float *y, const float *a,
                             const float *f, const float *g, int64_t n,
                             int64_t m, int32_t d, float eps, float *out,
                             void *stream);

/*
 * ot_cost_gradient_x -- out_i = 2 sum_j P_ij (x_i - y_j) (n*d): the gradient of
 * sum_ij P_ij C_ij with respect to x_i at the fixed plan of (f, g); at the
 * optimal potentials this is the gradient of the entropic OT cost with
 * respect to the source points (envelope theorem; page "FlashSinkhorn ...",
 * "Methodik" section 3, gradients as weighted averages). d is limited to
 * OT_MAX_TRANSPORT_DIM.
 */
ot_status ot_cost_gradient_x(const float *x, const float *y, const float *f,
                             const float *g, int64_t n, int64_t m, int32_t d,
                             float eps, float *out, void *stream);

/*
 * ot_birkhoff_project_batched -- project each 4x4 matrix of a batch onto the
 * doubly-stochastic matrices (page "Aceleración de la Proyección de Birkhoff
 * para Hiper-conexiones ...", sections 1-2: the projection is entropic OT
 * with unit marginals and cost -L, iterated by Sinkhorn-Knopp), here in the
 * log domain with the maximum subtracted before exponentiating (section 2.1):
 *
 *   g = 0; repeat:  f_i = -eps*LSE_j((g_j + L_ij)/eps)
 *                   g_j = -eps*LSE_i((f_i + L_ij)/eps)
 *   out_ij = exp((f_i + g_j + L_ij)/eps)
 *
 *   logits    [batch*16]  row-major 4x4 matrices L (fp32)
 *   batch     >= 0        (0 is a no-op)
 *   eps       > 0 and finite
 *   max_iters >= 0        iteration cap (0 returns exp(L/eps))
 *   tol       < 0: run exactly max_iters iterations;
 *             >= 0: stop a matrix after the first iteration k >= 1 whose
 *             plan, as written in fp32, has every row sum and every column
 *             sum within tol of 1 (evaluated in fp32), or at max_iters.
 *             NaN is invalid.
 *   out       [batch*16]  result; may alias logits exactly (in place)
 *   iters_out [batch]     nullable; iterations each matrix ran (int32)
 *
 * Errors: INVALID_VALUE (null logits/out, batch < 0, eps <= 0 or not finite,
 * max_iters < 0, NaN tol, partial overlap of out and logits), LAUNCH_FAILURE.
 */
ot_status ot_birkhoff_project_batched(const float *logits, int64_t batch,
                                      float eps, int32_t max_iters, float tol,
                                      float *out, int32_t *iters_out,
                                      void *stream);

/*
 * ot_sinkhorn_solve_cosine -- ot_sinkhorn_solve with the cosine cost
 * C_ij = 1 - x_i.y_j / (|x_i| |y_j|) (page "FlashSinkhorn ...", significance
 * section: the method covers the cosine distance after normalisation).
 * Computed as the squared Euclidean problem on x/|x|, y/|y| at 2*eps (on
 * unit vectors 1 - cos = |x - y|^2 / 2), with the potentials halved on the
 * way out and g doubled on the way in. Arguments, warm start and errors as
 * ot_sinkhorn_solve; every x_i and y_j must be nonzero (not checked).
 */
ot_status ot_sinkhorn_solve_cosine(const float *x, const float *y, const float *a,
                                   const float *b, int64_t n, int64_t m, int32_t d,
                                   float eps, int32_t iters, float *f, float *g,
                                   void *stream);

/*
 * ot_plan_stats_cosine -- ot_plan_stats for the cosine cost: cost =
 * sum_ij P_ij (1 - cos(x_i, y_j)) and the marginal L1 errors of
 * P_ij = exp((f_i + g_j - C_ij)/eps). Arguments and errors as ot_plan_stats.
 */
ot_status ot_plan_stats_cosine(const float *x, const float *y, const float *a,
                               const float *b, const float *f, const float *g,
                               int64_t n, int64_t m, int32_t d, float eps,
                               double *cost, double *marg, void *stream);

/*
 * ot_birkhoff_project_newton_batched -- the same projection as
 * ot_birkhoff_project_batched, computed by Newton's method on the dual (page
 * "Aceleración de la Proyección de Birkhoff ...", section 2.1): after fixing
 * g_4 = 0 (the dual is invariant under (f + c, g - c)) the row potentials are
 * eliminated, f_i(g) = -eps*LSE_j((g_j + L_ij)/eps), and the concave
 * F(g) = sum_i f_i(g) + sum_j g_j of the 3 free g_j is maximised with its
 * closed-form gradient 1 - c_j (c_j = column sums of the plan) and Hessian
 * -(c_j delta_jk - sum_i P_ij P_ik)/eps, each step halved until F rises by
 * 1e-4 of the linear prediction (less the rounding of F). The plan written
 * is the row softmax of the final g: rows sum to 1 up to rounding.
 *
 *   logits    [batch*16]  row-major 4x4 matrices L (fp32, 16-byte aligned)
 *   batch     >= 0        (0 is a no-op)
 *   eps       > 0 and finite
 *   max_iters >= 0        cap on Newton steps (0 returns the row softmax of L/eps)
 *   tol       < 0: take exactly max_iters steps;
 *             >= 0: stop before a step once the plan, as written in fp32, has
 *             every row and column sum within tol of 1. NaN is invalid.
 *   out       [batch*16]  result; may alias logits exactly (in place)
 *   iters_out [batch]     nullable; Newton steps each matrix took (int32)
 *
 * Errors: as ot_birkhoff_project_batched.
 */
ot_status ot_birkhoff_project_newton_batched(const float *logits, int64_t batch,
                                             float eps, int32_t max_iters,
                                             float tol, float *out,
                                             int32_t *iters_out, void *stream);

/*
 * ot_birkhoff_projection_backward_batched -- dl/dL of the projection by
 * implicit differentiation at the solution (page "Aceleración de la
 * Proyección de Birkhoff ...", section 2.2): with P the projection of L,
 * G = dl/dP and r_i = sum_j P_ij G_ij,
 *
 *   A lam = -w,  w_j = sum_i P_ij (G_ij - r_i),  A = diag(c) - P^T P
 *                (coordinates j, k < 3, lam_4 = 0; A is -eps times the
 *                Hessian of the last Newton step, recomputed from P),
 *   dl/dL_ij = P_ij (G_ij - r_i + lam_j - sum_k P_ik lam_k) / eps.
 *
 * Exact at a doubly-stochastic P; no forward iterate is stored or replayed.
 *
 *   plan        [batch*16]  the forward's output (fp32, 16-byte aligned)
 *   grad_plan   [batch*16]  dl/dP (fp32, 16-byte aligned)
 *   batch       >= 0
 *   eps         > 0 and finite, the forward's eps
 *   grad_logits [batch*16]  dl/dL; may alias plan or grad_plan exactly
 *
 * Errors: INVALID_VALUE (null pointers, batch < 0, eps <= 0 or not finite,
 * misaligned pointers, partial overlaps), LAUNCH_FAILURE.
 */
ot_status ot_birkhoff_projection_backward_batched(const float *plan,
                                                  const float *grad_plan,
                                                  int64_t batch, float eps,
                                                  float *grad_logits,
                                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* OT_SINKHORN_H */
