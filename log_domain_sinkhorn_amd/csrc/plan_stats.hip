// Statistics of the entropic plan P_ij = exp((f_i + g_j - C_ij)/eps) without
// storing it ("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
// Methodik section 3: the plan is applied by streaming, never materialised):
//
//   cost    = sum_ij P_ij C_ij
//   marg[0] = sum_i |sum_j P_ij - a_i|,   marg[1] = sum_j |sum_i P_ij - b_j|
//
// Two streaming passes of the same kernel: a row-stationary pass over the
// x side (row sums and cost) and a column-stationary pass over the y side
// (column sums), each over LDS-staged tiles of the other side's records.
//
// Accuracy: the exponent (f_i + g_j - C_ij)/eps cancels large terms at small
// eps, so it is formed in fp64 (C_ij by direct difference for d < 32, or from
// an fp32 dot product and fp64 norms for d >= 32); 2^t is evaluated as
// v_exp_f32 of the fp32-rounded t times (1 + residual*ln2). Per-row sums are
// fp64 and every reduction runs in a fixed order: no atomics, bitwise
// reproducible results.
#include "ot_internal.h"

#include <math.h>

namespace otsk {

namespace {

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kThreads = 256;

// fp64 squared norms of the first kp coordinates of each record.
__global__ __launch_bounds__(256) void norms_kernel(const float *__restrict__ rec, int64_t count,
                                                    int kp, int rs, double *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count)
        return;
    double s = 0.0;
    for (int k = 0; k < kp; ++k) {
        const double v = rec[i * rs + k];
        s = fma(v, v, s);
    }
    out[i] = s;
}

// One pass. Rows: records row_rec (raw potential in the bias slot). Columns:
// records col_rec. Writes part[split][row] = (sum_j P, sum_j P C) (COST) or
// sum_j P into part[split][row].x. Each lane owns R rows (kThreads apart), so
// the per-column loads and conversions are shared by R rows.
template <int KP, int RS, int TJ, bool DIRECT, bool COST, int R>
__global__ __launch_bounds__(kThreads) void plan_pass_kernel(
    const float *__restrict__ row_rec, const double *__restrict__ row_nrm,
    const float *__restrict__ col_rec, const double *__restrict__ col_nrm, int64_t rows,
    int64_t rows_pad, int tiles_per_split, int ntiles, double inv_eps_log2e,
    double2 *__restrict__ part) {
    constexpr int RS4 = RS / 4;
    constexpr int TILE4 = TJ * RS4;
    constexpr int PF = (TILE4 + kThreads - 1) / kThreads;
    __shared__ float4 lds[2][TILE4];
    __shared__ double lnrm[2][TJ];

    const int tid = threadIdx.x;
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const int64_t row0 = (int64_t)blockIdx.x * (kThreads * R);

    float xr[R][KP];
    double fi[R], nx[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row0 + tid + r * kThreads;
        const int64_t ic = i < rows ? i : rows - 1;
#pragma unroll
        for (int k = 0; k < KP; ++k)
            xr[r][k] = row_rec[ic * RS + k];
        fi[r] = row_rec[ic * RS + KP];
        nx[r] = DIRECT ? 0.0 : row_nrm[ic];
    }

    const float4 *col4 = reinterpret_cast<const float4 *>(col_rec);
    double rsum[R], csum[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        rsum[r] = csum[r] = 0.0;
#pragma unroll
    for (int q = 0; q < PF; ++q) {
        const int idx = tid + q * kThreads;
        if (TILE4 % kThreads == 0 || idx < TILE4)
            lds[0][idx] = col4[(int64_t)tbeg * TILE4 + idx];
    }
    if (!DIRECT && tid < TJ)
        lnrm[0][tid] = col_nrm[(int64_t)tbeg * TJ + tid];
    __syncthreads();
    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        // Next tile (the last iteration reloads its own tile; the copy into
        // the idle buffer is then unused). Unconditional, so the prefetch
        // stays in registers.
        const int tn = t + 1 < tend ? t + 1 : t;
        float4 pre[PF];
        double pn = 0.0;
        {
#pragma unroll
            for (int q = 0; q < PF; ++q) {
                const int idx = min(tid + q * kThreads, TILE4 - 1);
                pre[q] = col4[(int64_t)tn * TILE4 + idx];
            }
            if (!DIRECT && tid < TJ)
                pn = col_nrm[(int64_t)tn * TJ + tid];
        }
        const float *tile = reinterpret_cast<const float *>(lds[b]);
        for (int c = 0; c < TJ; ++c) {
            const float *rc = tile + c * RS;
            double cd[KP];
#pragma unroll
            for (int k = 0; k < KP; ++k)
                cd[k] = (double)rc[k];
            const double gj = (double)rc[KP];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                double C;
                if (DIRECT) {
                    C = 0.0;
#pragma unroll
                    for (int k = 0; k < KP; ++k) {
                        const double dlt = (double)xr[r][k] - cd[k];
                        C = fma(dlt, dlt, C);
                    }
                } else {
                    float dot = 0.f;
#pragma unroll
                    for (int k = 0; k < KP; ++k)
                        dot = fmaf(xr[r][k], rc[k], dot);
                    C = nx[r] + lnrm[b][c] - 2.0 * (double)dot;
                }
                double tt = (fi[r] + gj - C) * inv_eps_log2e;
                tt = fmax(tt, -2000.0);
                const float th = (float)tt;
                const float tl = (float)(tt - (double)th);
                const double p = (double)hw_exp2(th) * fma((double)tl, kLn2, 1.0);
                rsum[r] += p;
                if (COST)
                    csum[r] = fma(p, C, csum[r]);
            }
        }
        {
#pragma unroll
            for (int q = 0; q < PF; ++q) {
                const int idx = tid + q * kThreads;
                if (TILE4 % kThreads == 0 || idx < TILE4)
                    lds[b ^ 1][idx] = pre[q];
            }
            if (!DIRECT && tid < TJ)
                lnrm[b ^ 1][tid] = pn;
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row0 + tid + r * kThreads;
        if (i < rows)
            part[(int64_t)split * rows_pad + i] = make_double2(rsum[r], csum[r]);
    }
}

// Per block: sum over its rows of |sum_s part[s][i].x - w_i| and of
// sum_s part[s][i].y, tree-reduced in a fixed order.
__global__ __launch_bounds__(256) void reduce_rows_kernel(const double2 *__restrict__ part,
                                                          int nsplit, int64_t rows,
                                                          int64_t rows_pad,
                                                          const float *__restrict__ w,
                                                          double2 *__restrict__ block_out) {
    __shared__ double2 red[256];
    double m = 0.0, c = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows;
         i += (int64_t)gridDim.x * 256) {
        double r = 0.0, cc = 0.0;
        for (int s = 0; s < nsplit; ++s) {
            const double2 p = part[(int64_t)s * rows_pad + i];
            r += p.x;
            cc += p.y;
        }
        if (w)
            m += fabs(r - (double)w[i]);
        c += cc;
    }
    red[threadIdx.x] = make_double2(m, c);
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if ((int)threadIdx.x < st) {
            red[threadIdx.x].x += red[threadIdx.x + st].x;
            red[threadIdx.x].y += red[threadIdx.x + st].y;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0)
        block_out[blockIdx.x] = red[0];
}

// Single block: add the per-block partials in order and write the scalars.
__global__ __launch_bounds__(256) void stats_final_kernel(const double2 *__restrict__ row_blocks,
                                                          int nrb,
                                                          const double2 *__restrict__ col_blocks,
                                                          int ncb, double *cost, double *marg) {
    __shared__ double3 red[256];
    double mr = 0.0, cr = 0.0, mc = 0.0;
    for (int k = threadIdx.x; k < nrb; k += 256) {
        mr += row_blocks[k].x;
        cr += row_blocks[k].y;
    }
    for (int k = threadIdx.x; k < ncb; k += 256)
        mc += col_blocks[k].x;
    red[threadIdx.x] = make_double3(mr, cr, mc);
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if ((int)threadIdx.x < st) {
            red[threadIdx.x].x += red[threadIdx.x + st].x;
            red[threadIdx.x].y += red[threadIdx.x + st].y;
            red[threadIdx.x].z += red[threadIdx.x + st].z;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (cost)
            *cost = red[0].y;
        if (marg) {
            marg[0] = red[0].x;
            marg[1] = red[0].z;
        }
    }
}

constexpr int kTargetBlocks = 2048;
constexpr int kReduceBlocks = 512;

struct PassPlan {
    int TJ;
    int ntiles;
    int tiles_per_split;
    int nsplit;
    int R;
    int64_t row_blocks;
};

int pass_tile(int rs) { return rs <= 16 ? 64 : 32; }

// Rows per lane: up to 4 for 3-D records (65536^2: both passes 5.98 -> 5.31
// ms against 1), fewer while the grid would be short of kTargetBlocks
// workgroups.
PassPlan plan_pass(int rs, int64_t rows, int64_t cols_pad) {
    PassPlan p;
    p.TJ = pass_tile(rs);
    p.ntiles = (int)(cols_pad / p.TJ);
    const int max_r = rs <= 4 ? 4 : 1;
    p.R = 1;
    for (int R = max_r; R >= 1; R /= 2) {
        const int64_t rb = (rows + kThreads * R - 1) / (kThreads * R);
        if (rb * p.ntiles >= kTargetBlocks || R == 1) {
            p.R = R;
            break;
        }
    }
    p.row_blocks = (rows + kThreads * p.R - 1) / (kThreads * p.R);
    int64_t want = (kTargetBlocks + p.row_blocks - 1) / p.row_blocks;
    if (want > p.ntiles)
        want = p.ntiles;
    if (want > 65535)
        want = 65535;
    if (want < 1)
        want = 1;
    p.tiles_per_split = (int)((p.ntiles + want - 1) / want);
    p.nsplit = (p.ntiles + p.tiles_per_split - 1) / p.tiles_per_split;
    return p;
}

template <int KP, int RS, bool COST>
hipError_t launch_pass_t(const float *row_rec, const double *row_nrm, const float *col_rec,
                         const double *col_nrm, int64_t rows, int64_t rows_pad, const PassPlan &p,
                         double inv_eps_log2e, double2 *part, hipStream_t s) {
    constexpr bool DIRECT = KP < 32;
    constexpr int TJ = RS <= 16 ? 64 : 32;
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    if (p.R == 4 || p.R == 2) {
        if constexpr (RS <= 4) {
            if (p.R == 4)
                hipLaunchKernelGGL((plan_pass_kernel<KP, RS, TJ, DIRECT, COST, 4>), grid,
                                   dim3(kThreads), 0, s, row_rec, row_nrm, col_rec, col_nrm, rows,
                                   rows_pad, p.tiles_per_split, p.ntiles, inv_eps_log2e, part);
            else
                hipLaunchKernelGGL((plan_pass_kernel<KP, RS, TJ, DIRECT, COST, 2>), grid,
                                   dim3(kThreads), 0, s, row_rec, row_nrm, col_rec, col_nrm, rows,
                                   rows_pad, p.tiles_per_split, p.ntiles, inv_eps_log2e, part);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((plan_pass_kernel<KP, RS, TJ, DIRECT, COST, 1>), grid, dim3(kThreads), 0,
                       s, row_rec, row_nrm, col_rec, col_nrm, rows, rows_pad, p.tiles_per_split,
                       p.ntiles, inv_eps_log2e, part);
    return hipGetLastError();
}

template <bool COST>
hipError_t launch_pass(const Layout &L, const float *row_rec, const double *row_nrm,
                       const float *col_rec, const double *col_nrm, int64_t rows,
                       int64_t rows_pad, const PassPlan &p, double inv_eps_log2e, double2 *part,
                       hipStream_t s) {
#define OTSK_PASS(KPV, RSV)                                                                    \
    case KPV:                                                                                  \
        return launch_pass_t<KPV, RSV, COST>(row_rec, row_nrm, col_rec, col_nrm, rows,         \
                                             rows_pad, p, inv_eps_log2e, part, s);
    switch (L.kp) {
        OTSK_PASS(3, 4)
        OTSK_PASS(7, 8)
        OTSK_PASS(11, 12)
        OTSK_PASS(15, 16)
        OTSK_PASS(19, 20)
        OTSK_PASS(23, 24)
        OTSK_PASS(27, 28)
        OTSK_PASS(31, 32)
        OTSK_PASS(32, 36)
        OTSK_PASS(48, 52)
        OTSK_PASS(64, 68)
        OTSK_PASS(80, 84)
        OTSK_PASS(96, 100)
        OTSK_PASS(112, 116)
        OTSK_PASS(128, 132)
    default:
        return hipErrorInvalidValue;
    }
#undef OTSK_PASS
}

int reduce_blocks(int64_t rows) {
    int64_t b = (rows + 255) / 256;
    return (int)(b < kReduceBlocks ? b : kReduceBlocks);
}

}  // namespace

size_t plan_stats_scratch_doubles(const Layout &L, int64_t n, int64_t m, int64_t n_pad,
                                  int64_t m_pad) {
    const PassPlan pr = plan_pass(L.rs, n, m_pad);
    const PassPlan pc = plan_pass(L.rs, m, n_pad);
    size_t d = 0;
    d += (size_t)n_pad + (size_t)m_pad;          // norms
    d += 2 * (size_t)pr.nsplit * (size_t)n_pad;  // row partials (double2)
    d += 2 * (size_t)pc.nsplit * (size_t)m_pad;  // column partials (double2)
    d += 2 * 2 * (size_t)kReduceBlocks;          // per-block partials (double2)
    return d;
}

hipError_t launch_plan_stats(const float *x_rec, const float *y_rec, const float *a, const float *b,
                             int64_t n, int64_t m, int64_t n_pad,
                             int64_t m_pad, const Layout &L, float eps, double *cost, double *marg,
                             double *scratch, hipStream_t s) {
    hipError_t e;
    double *nx = scratch;
    double *ny = nx + n_pad;
    const bool direct = L.kp < 32;
    if (!direct) {
        // Over the padded counts: padding records have zero coordinates, so
        // their norms are written (0) and the passes never read stale memory.
        hipLaunchKernelGGL(norms_kernel, dim3((unsigned)((n_pad + 255) / 256)), dim3(256), 0, s,
                           x_rec, n_pad, L.kp, L.rs, nx);
        hipLaunchKernelGGL(norms_kernel, dim3((unsigned)((m_pad + 255) / 256)), dim3(256), 0, s,
                           y_rec, m_pad, L.kp, L.rs, ny);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    const double inv = kLog2e / (double)eps;
    const PassPlan pr = plan_pass(L.rs, n, m_pad);
    const PassPlan pc = plan_pass(L.rs, m, n_pad);
    double2 *prow = reinterpret_cast<double2 *>(ny + m_pad);
    double2 *pcol = prow + (size_t)pr.nsplit * n_pad;
    double2 *brow = pcol + (size_t)pc.nsplit * m_pad;
    double2 *bcol = brow + kReduceBlocks;

    // Row pass (row sums and cost), then column pass (column sums).
    if ((e = launch_pass<true>(L, x_rec, nx, y_rec, ny, n, n_pad, pr, inv, prow, s)) != hipSuccess)
        return e;
    const int nrb = reduce_blocks(n);
    hipLaunchKernelGGL(reduce_rows_kernel, dim3(nrb), dim3(256), 0, s, prow, pr.nsplit, n, n_pad,
                       marg ? a : nullptr, brow);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    int ncb = 0;
    if (marg) {
        if ((e = launch_pass<false>(L, y_rec, ny, x_rec, nx, m, m_pad, pc, inv, pcol, s)) !=
            hipSuccess)
            return e;
        ncb = reduce_blocks(m);
        hipLaunchKernelGGL(reduce_rows_kernel, dim3(ncb), dim3(256), 0, s, pcol, pc.nsplit, m,
                           m_pad, b, bcol);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(256), 0, s, brow, nrb, bcol, ncb, cost,
                       marg);
    return hipGetLastError();
}

size_t plan_stats_h3_scratch_doubles(int64_t n, int64_t m, int64_t n_pad, int64_t m_pad,
                                     int kp) {
    size_t d = 0;
    d += 2 * (size_t)plan_pass_h3_splits(n, m_pad, kp) * (size_t)n_pad;  // row partials
    d += 2 * (size_t)plan_pass_h3_splits(m, n_pad, kp) * (size_t)m_pad;  // column partials
    d += 2 * 2 * (size_t)kReduceBlocks;
    return d;
}

// d >= 32: the two passes on split-f16 records, then the same fp64
// reductions as the VALU passes.
hipError_t launch_plan_stats_h3(int kp, const void *xrow, const void *xcol, const float *xhat,
                                const float *xnrm, const void *yrow, const void *ycol,
                                const float *yhat, const float *ynrm, const float *a,
                                const float *b, int64_t n, int64_t m, int64_t n_pad,
                                int64_t m_pad, double scale, double *cost, double *marg,
                                double *scratch, hipStream_t s) {
    hipError_t e;
    double2 *prow = reinterpret_cast<double2 *>(scratch);
    double2 *pcol = prow + (size_t)plan_pass_h3_splits(n, m_pad, kp) * n_pad;
    double2 *brow = pcol + (size_t)plan_pass_h3_splits(m, n_pad, kp) * m_pad;
    double2 *bcol = brow + kReduceBlocks;
    if ((e = launch_plan_pass_h3(kp, true, xrow, xhat, xnrm, ycol, yhat, ynrm, n, n_pad, m_pad,
                                 scale, prow, s)) != hipSuccess)
        return e;
    const int nrb = reduce_blocks(n);
    hipLaunchKernelGGL(reduce_rows_kernel, dim3(nrb), dim3(256), 0, s, prow,
                       plan_pass_h3_splits(n, m_pad, kp), n, n_pad, marg ? a : nullptr, brow);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    int ncb = 0;
    if (marg) {
        if ((e = launch_plan_pass_h3(kp, false, yrow, yhat, ynrm, xcol, xhat, xnrm, m, m_pad,
                                     n_pad, scale, pcol, s)) != hipSuccess)
            return e;
        ncb = reduce_blocks(m);
        hipLaunchKernelGGL(reduce_rows_kernel, dim3(ncb), dim3(256), 0, s, pcol,
                           plan_pass_h3_splits(m, n_pad, kp), m, m_pad, b, bcol);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(256), 0, s, brow, nrb, bcol, ncb, cost,
                       marg);
    return hipGetLastError();
}

}  // namespace otsk
