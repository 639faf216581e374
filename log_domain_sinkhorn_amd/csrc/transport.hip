// Transport application: out_i = sum_j P_ij v_j for the plan
// P_ij = exp((f_i + g_j - C_ij)/eps) of given potentials, without storing P.
//
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodik
// section 3: the barycentric projection and the gradients are weighted
// averages under the plan (attention-like), computed by the same streaming
// traversal as the potential updates.
//
// In base 2, with the records of the half-step kernels (coordinates and the
// hat biases fhat_i = (f_i - |x_i|^2) log2(e)/eps, ghat_j likewise),
//
//   log2 P_ij = (2 log2(e)/eps) x_i . y_j + ghat_j + fhat_i,
//
// formed in fp64 (d fp64 FMAs + one add: the terms cancel from (2/eps)|x||y|
// down to log2 P, as in the half-step), rounded once for v_exp_f32, and
// multiplied into the values in fp32 within a tile, with fp64 totals across
// tiles. Unlike the half-step this needs no running maximum: P is a plan,
// not a normalised softmax, so its entries are at most min(a_i, b_j) for
// potentials produced by the solver.
//
// Layout: each lane owns R rows; column records (fp64) and the matching
// value rows (fp32, zero padded to DV) stream through double-buffered LDS
// tiles; columns are split across workgroups and the fp64 partials are added
// in split order by transport_reduce_kernel. No atomics.
#include "ot_internal.h"

#include <math.h>

namespace otsk {

namespace {

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kTargetBlocks = 2048;

template <int KP, int R, int TJ, int DV>
__global__ __launch_bounds__(256) void transport_valu_kernel(
    const double *__restrict__ row_rec, const double *__restrict__ col_rec,
    const float *__restrict__ v, int64_t m, int dv, int k0, int64_t rows, int64_t rows_pad,
    double scale, int tiles_per_split, int ntiles, double *__restrict__ part) {
    constexpr int RS = KP + 1;
    constexpr int RS2 = RS / 2;
    constexpr int TILE2 = TJ * RS2;
    constexpr int PF = (TILE2 + 255) / 256;
    __shared__ double2 lrec[2][TILE2];
    __shared__ float lv[2][TJ * DV];

    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * (256 * R);
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const double2 *col2 = reinterpret_cast<const double2 *>(col_rec);

    double xs[R][KP];
    double fh[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t i = row0 + tid + r * 256;
        i = i < rows ? i : rows - 1;
        const double *p = row_rec + i * RS;
#pragma unroll
        for (int k = 0; k < KP; ++k)
            xs[r][k] = p[k] * scale;
        fh[r] = p[KP];
    }

    // Values of column tile t (channels k0 .. k0 + DV of v), zero outside.
    auto stage_values = [&](int t, int buf) {
        for (int e = tid; e < TJ * DV; e += 256) {
            const int64_t j = (int64_t)t * TJ + e / DV;
            const int k = k0 + e % DV;
            lv[buf][e] = (j < m && k < dv) ? v[j * dv + k] : 0.f;
        }
    };

#pragma unroll
    for (int q = 0; q < PF; ++q) {
        const int idx = tid + q * 256;
        if (TILE2 % 256 == 0 || idx < TILE2)
            lrec[0][idx] = col2[(int64_t)tbeg * TILE2 + idx];
    }
    stage_values(tbeg, 0);
    __syncthreads();

    double tot[R][DV];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < DV; ++k)
            tot[r][k] = 0.0;

    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        const int tn = t + 1 < tend ? t + 1 : t;
        double2 pre[PF];
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int idx = min(tid + q * 256, TILE2 - 1);
            pre[q] = col2[(int64_t)tn * TILE2 + idx];
        }
        const double *tile = reinterpret_cast<const double *>(lrec[b]);
        const float *vt = lv[b];
        float acc[R][DV];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int k = 0; k < DV; ++k)
                acc[r][k] = 0.f;
        for (int c = 0; c < TJ; ++c) {
            const double *rec = tile + c * RS;
            float vv[DV];
#pragma unroll
            for (int k = 0; k < DV; ++k)
                vv[k] = vt[c * DV + k];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                double e = rec[KP] + fh[r];
#pragma unroll
                for (int k = KP - 1; k >= 0; --k)
                    e = fma(xs[r][k], rec[k], e);
                const float p = hw_exp2((float)e);
#pragma unroll
                for (int k = 0; k < DV; ++k)
                    acc[r][k] = fmaf(p, vv[k], acc[r][k]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int k = 0; k < DV; ++k)
                tot[r][k] += (double)acc[r][k];
        // Stage the next tile into the idle buffer (its last readers passed
        // the previous barrier).
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int idx = tid + q * 256;
            if (TILE2 % 256 == 0 || idx < TILE2)
                lrec[b ^ 1][idx] = pre[q];
        }
        if (t + 1 < tend)
            stage_values(t + 1, b ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row0 + tid + r * 256;
        if (i < rows)
#pragma unroll
            for (int k = 0; k < DV; ++k)
                part[((int64_t)split * rows_pad + i) * DV + k] = tot[r][k];
    }
}

// out[i*dv + k0 + k] = sum over splits of part[s][i][k], in split order.
template <int DV>
__global__ __launch_bounds__(256) void transport_reduce_kernel(const double *__restrict__ part,
                                                               int nsplit, int64_t rows,
                                                               int64_t rows_pad, int dv, int k0,
                                                               float *__restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= rows * DV)
        return;
    const int64_t i = e / DV;
    const int k = (int)(e % DV);
    if (k0 + k >= dv)
        return;
    double s = 0.0;
    for (int sp = 0; sp < nsplit; ++sp)
        s += part[((int64_t)sp * rows_pad + i) * DV + k];
    out[i * dv + k0 + k] = (float)s;
}

struct TPlan {
    int R, TJ, ntiles, tiles_per_split, nsplit;
    int64_t row_blocks;
};

constexpr int tcols(int rs) { return rs <= 4 ? 256 : (rs <= 8 ? 128 : (rs <= 16 ? 64 : 32)); }

// Rows per lane: up to 4 for 3-D records with at most 4 value channels per
// pass (more rows share each LDS read of a column; 65536^2 x 3: 1.26 -> 1.18 ms
// against 2 rows), fewer while the grid would otherwise be short of
// kTargetBlocks workgroups.
TPlan plan_transport(const Layout &L, int64_t rows, int64_t cols_pad, int dvc) {
    TPlan p;
    p.TJ = tcols(L.rs);
    p.ntiles = (int)(cols_pad / p.TJ);
    const int max_r = L.kp <= 3 ? (dvc <= 4 ? 4 : 2) : 1;
    p.R = 1;
    for (int R = max_r; R >= 1; R /= 2) {
        const int64_t rb = (rows + 256 * R - 1) / (256 * R);
        if (rb * p.ntiles >= kTargetBlocks || R == 1) {
            p.R = R;
            break;
        }
    }
    p.row_blocks = (rows + 256 * p.R - 1) / (256 * p.R);
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

template <int KP, int R, int DV>
hipError_t launch_tv(const double *xrec, const double *yrec, const float *v, int64_t m, int dv,
                     int k0, int64_t n, int64_t n_pad, double scale, const TPlan &p,
                     double *part, hipStream_t s) {
    constexpr int TJ = tcols(KP + 1);
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    hipLaunchKernelGGL((transport_valu_kernel<KP, R, TJ, DV>), grid, dim3(256), 0, s, xrec, yrec,
                       v, m, dv, k0, n, n_pad, scale, p.tiles_per_split, p.ntiles, part);
    return hipGetLastError();
}

template <int KP, int DV>
hipError_t launch_tk(const double *xrec, const double *yrec, const float *v, int64_t m, int dv,
                     int k0, int64_t n, int64_t n_pad, double scale, const TPlan &p,
                     double *part, hipStream_t s) {
    if (p.R == 4) {
        if constexpr (KP <= 3 && DV <= 4)
            return launch_tv<KP, 4, DV>(xrec, yrec, v, m, dv, k0, n, n_pad, scale, p, part, s);
        return hipErrorInvalidValue;
    }
    if (p.R == 2) {
        if constexpr (KP <= 3)
            return launch_tv<KP, 2, DV>(xrec, yrec, v, m, dv, k0, n, n_pad, scale, p, part, s);
        return hipErrorInvalidValue;
    }
    return launch_tv<KP, 1, DV>(xrec, yrec, v, m, dv, k0, n, n_pad, scale, p, part, s);
}

template <int DV>
hipError_t launch_t(const Layout &L, const double *xrec, const double *yrec, const float *v,
                    int64_t m, int dv, int k0, int64_t n, int64_t n_pad, double scale,
                    const TPlan &p, double *part, hipStream_t s) {
#define OTSK_T(KPV)                                                                            \
    case KPV:                                                                                  \
        return launch_tk<KPV, DV>(xrec, yrec, v, m, dv, k0, n, n_pad, scale, p, part, s);
    switch (L.kp) {
        OTSK_T(3)
        OTSK_T(7)
        OTSK_T(11)
        OTSK_T(15)
        OTSK_T(19)
        OTSK_T(23)
        OTSK_T(27)
        OTSK_T(31)
    default:
        return hipErrorInvalidValue;
    }
#undef OTSK_T
}

}  // namespace

// Value channels per pass: 3 exactly (the map and P.y of 3-D clouds), else
// the next of 1, 4, 8, 16 (zero-padded channels cost their FMAs).
int transport_value_chunk(int dv) {
    return dv <= 1 ? 1 : (dv == 3 ? 3 : (dv <= 4 ? 4 : (dv <= 8 ? 8 : 16)));
}

size_t transport_scratch_doubles(const Layout &L, int64_t n, int64_t m_pad, int dv) {
    const TPlan p = plan_transport(L, n, m_pad, transport_value_chunk(dv));
    return (size_t)p.nsplit * (size_t)pad_points(n) * (size_t)transport_value_chunk(dv);
}

hipError_t launch_transport_apply(const Layout &L, const void *xrec, const void *yrec,
                                  const float *v, int64_t n, int64_t n_pad, int64_t m,
                                  int64_t m_pad, int dv, double scale, double *part, float *out,
                                  hipStream_t s) {
    const int dvc = transport_value_chunk(dv);
    const TPlan p = plan_transport(L, n, m_pad, dvc);
    const double *xr = static_cast<const double *>(xrec);
    const double *yr = static_cast<const double *>(yrec);
    for (int k0 = 0; k0 < dv; k0 += dvc) {
        hipError_t e;
        switch (dvc) {
        case 1: e = launch_t<1>(L, xr, yr, v, m, dv, k0, n, n_pad, scale, p, part, s); break;
        case 3: e = launch_t<3>(L, xr, yr, v, m, dv, k0, n, n_pad, scale, p, part, s); break;
        case 4: e = launch_t<4>(L, xr, yr, v, m, dv, k0, n, n_pad, scale, p, part, s); break;
        case 8: e = launch_t<8>(L, xr, yr, v, m, dv, k0, n, n_pad, scale, p, part, s); break;
        default: e = launch_t<16>(L, xr, yr, v, m, dv, k0, n, n_pad, scale, p, part, s); break;
        }
        if (e != hipSuccess)
            return e;
        const int64_t total = n * dvc;
        const unsigned blocks = (unsigned)((total + 255) / 256);
        switch (dvc) {
        case 1:
            hipLaunchKernelGGL(transport_reduce_kernel<1>, dim3(blocks), dim3(256), 0, s, part,
                               p.nsplit, n, n_pad, dv, k0, out);
            break;
        case 3:
            hipLaunchKernelGGL(transport_reduce_kernel<3>, dim3(blocks), dim3(256), 0, s, part,
                               p.nsplit, n, n_pad, dv, k0, out);
            break;
        case 4:
            hipLaunchKernelGGL(transport_reduce_kernel<4>, dim3(blocks), dim3(256), 0, s, part,
                               p.nsplit, n, n_pad, dv, k0, out);
            break;
        case 8:
            hipLaunchKernelGGL(transport_reduce_kernel<8>, dim3(blocks), dim3(256), 0, s, part,
                               p.nsplit, n, n_pad, dv, k0, out);
            break;
        default:
            hipLaunchKernelGGL(transport_reduce_kernel<16>, dim3(blocks), dim3(256), 0, s, part,
                               p.nsplit, n, n_pad, dv, k0, out);
            break;
        }
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Helpers of the barycentric map and the x-gradient: the value matrix
// [y | 1] (whose last column gives the row sums r_i = sum_j P_ij on the VALU
// path) and the final elementwise combination.
// ---------------------------------------------------------------------------
namespace {

__global__ __launch_bounds__(256) void values_y1_kernel(const float *__restrict__ y, int64_t m,
                                                        int d, float *__restrict__ v) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= m * (d + 1))
        return;
    const int64_t j = e / (d + 1);
    const int k = (int)(e % (d + 1));
    v[e] = k < d ? y[j * d + k] : 1.f;
}

// mode 0: out_i = w_i / a_i; mode 1: out_i = 2 (r_i x_i - w_i); w_i is row i
// of w (stride ws), r_i = r[i] or, without r, the column after w_i.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ w, int ws,
                                                      const float *__restrict__ r,
                                                      const float *__restrict__ x,
                                                      const float *__restrict__ a, int64_t n,
                                                      int d, int mode, float *__restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n * d)
        return;
    const int64_t i = e / d;
    const int k = (int)(e % d);
    const float wk = w[i * ws + k];
    if (mode == 0) {
        out[e] = wk / a[i];
    } else {
        const float ri = r ? r[i] : w[i * ws + d];
        out[e] = 2.f * (ri * x[e] - wk);
    }
}

}  // namespace

hipError_t launch_values_y1(const float *y, int64_t m, int d, float *v, hipStream_t s) {
    const int64_t total = m * (d + 1);
    hipLaunchKernelGGL(values_y1_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       y, m, d, v);
    return hipGetLastError();
}

hipError_t launch_combine(const float *w, int ws, const float *r, const float *x, const float *a,
                          int64_t n, int d, int mode, float *out, hipStream_t s) {
    const int64_t total = n * d;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w,
                       ws, r, x, a, n, d, mode, out);
    return hipGetLastError();
}

}  // namespace otsk
