// Transport application on the matrix cores (feature dimension d >= 32):
// out_i = sum_j P_ij v_j with P_ij = exp((f_i + g_j - C_ij)/eps), P never
// stored ("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
// Methodik section 3: applying the plan is an attention-like weighted
// average over the streamed tiles).
//
// Per wave (32 rows) and 32-column subtile:
//  1. the split-f16 score chain of the half-step kernel (3*KP/16 f16 MFMAs
//     and one fp32 MFMA that adds ghat_j and fhat_i) gives log2 P_ij as
//     D[j][i], j on the per-lane register axis: lane l holds row i = l % 32
//     and the 16 columns j = 8*(v/4) + 4*(l/32) + v%4 of its registers v;
//  2. 16 v_exp_f32 turn them into P;
//  3. 16 fp32 MFMAs per 32 value channels accumulate O^T[k][i] += V[j][k] P_ij:
//     register v of every lane is exactly the B operand of one MFMA (its two
//     k-slots are the j's of the two lane halves), and the A operand is the
//     matching value row read from LDS, so P never leaves the VGPRs.
// No running maximum is needed: P is a plan, not a normalised softmax.
// With RSUM the row sums r_i = sum_j P_ij come out too (16 VALU adds per
// subtile), so the x-gradient 2(r_i x_i - sum_j P_ij y_j) needs one pass
// over the value channels of y instead of a pass over [y | 1].
// Accumulation is fp32 within a workgroup's column range; the column ranges'
// partials are added in fp64, in split order. No atomics.
#include "mfma_common.h"

#include <math.h>

namespace otsk {

namespace {

using namespace mfma;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;
constexpr int kTileCols = 64;
constexpr int kSub = kTileCols / 32;
constexpr int kBiasSlots = 2 * kTileCols;
constexpr int kTargetBlocks = 1024;

template <int KP, int NVB, bool RSUM>
__global__ __launch_bounds__(kThreads) void transport_mfma_kernel(
    const float4 *__restrict__ row_rec, const float *__restrict__ row_bias,
    const float4 *__restrict__ col4, const float *__restrict__ colb, const float *__restrict__ v,
    int64_t m, int dv, int k0, int64_t rows, int64_t rows_pad, int tiles_per_split,
    int ntiles, double *__restrict__ part, double *__restrict__ rpart) {
    constexpr int RC = KP / 4;
    constexpr int TILE4 = kTileCols * RC;
    constexpr int VC = 32 * NVB;                  // value channels per pass
    constexpr int VST = VC + 4;                   // LDS row stride of the values
    constexpr int VPT = kTileCols * VC / kThreads; // values staged per thread per tile
    static_assert(kTileCols * VC % kThreads == 0, "whole value tiles per thread");
    __shared__ float4 lrec[2][TILE4];
    __shared__ float lbias[2][kBiasSlots];
    __shared__ float lv[2][kTileCols * VST];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);

    for (int k = tid; k < 2 * kBiasSlots; k += kThreads) {
        const int e = k % kBiasSlots;
        if ((e / 32) & 1)
            lbias[k / kBiasSlots][e] = 1.f;
    }
    issue_tile<TILE4, kWaves, kSub>(col4, colb, tbeg, lrec[0], lbias[0], wave, lane);

    // Values of a column tile: channel block [k0, k0 + VC), zero outside.
    float pv[VPT];
    auto load_values = [&](int t) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int e = tid + q * kThreads;
            const int64_t j = (int64_t)t * kTileCols + e / VC;
            const int k = k0 + e % VC;
            pv[q] = (j < m && k < dv) ? v[j * dv + k] : 0.f;
        }
    };
    auto store_values = [&](int buf) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int e = tid + q * kThreads;
            lv[buf][(e / VC) * VST + e % VC] = pv[q];
        }
    };
    load_values(tbeg);
    store_values(0);

    const int64_t i = (int64_t)blockIdx.x * kRowsPerBlock + wave * 32 + li;
    const int64_t ic = i < rows ? i : rows - 1;
    half8 bh[KP / 16], bl[KP / 16];
    {
        const float4 *rr = row_rec + ic * RC;
#pragma unroll
        for (int c = 0; c < KP / 16; ++c) {
            bh[c] = as_half8(rr[2 * c + hl]);
            bl[c] = as_half8(rr[KP / 8 + 2 * c + hl]);
        }
    }
    // The bias MFMA adds ghat_j x 1 + 1 x (-Mu): Mu = -fhat_i puts fhat_i in.
    const float Mu = -row_bias[ic];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    floatx16 O[NVB];
#pragma unroll
    for (int nb = 0; nb < NVB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            O[nb][r] = 0.f;
    float rsum = 0.f;

    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        const bool more = t + 1 < tend;
        if (more) {
            issue_tile<TILE4, kWaves, kSub>(col4, colb, t + 1, lrec[b ^ 1], lbias[b ^ 1], wave,
                                            lane);
            load_values(t + 1);
        }
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) {
            floatx16 pr = score_h3<KP>(lrec[b], lbias[b], sub, lane, li, hl, bh, bl, Mu);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                pr[r] = hw_exp2(pr[r]);
            if (RSUM) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    rsum += pr[r];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = sub * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
#pragma unroll
                for (int nb = 0; nb < NVB; ++nb)
                    O[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(lv[b][j * VST + nb * 32 + li],
                                                                pr[r], O[nb], 0, 0, 0);
            }
        }
        if (more)
            store_values(b ^ 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // The two lane halves summed different columns of the same row.
    if (RSUM) {
        rsum += __shfl_xor(rsum, 32);
        if (hl == 0 && i < rows)
            rpart[(int64_t)split * rows_pad + i] = (double)rsum;
    }
    // Lane l holds O^T[k][i] for row i = l % 32 and the 16 channels
    // k = 8*(r/4) + 4*(l/32) + r%4 of each channel block.
    if (i < rows) {
#pragma unroll
        for (int nb = 0; nb < NVB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k = nb * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
                part[((int64_t)split * rows_pad + i) * VC + k] = (double)O[nb][r];
            }
    }
}

// out[i*dv + k0 + k] = sum over splits of part[s][i][k], in split order.
template <int VC>
__global__ __launch_bounds__(256) void transport_mfma_reduce_kernel(
    const double *__restrict__ part, int nsplit, int64_t rows, int64_t rows_pad, int dv, int k0,
    float *__restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= rows * VC)
        return;
    const int64_t i = e / VC;
    const int k = (int)(e % VC);
    if (k0 + k >= dv)
        return;
    double s = 0.0;
    for (int sp = 0; sp < nsplit; ++sp)
        s += part[((int64_t)sp * rows_pad + i) * VC + k];
    out[i * dv + k0 + k] = (float)s;
}

struct MPlan {
    int ntiles, tiles_per_split, nsplit;
    int64_t row_blocks;
};

MPlan plan_tm(int64_t rows, int64_t cols_pad) {
    MPlan p;
    p.ntiles = (int)(cols_pad / kTileCols);
    p.row_blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
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

int value_blocks(int dv) { return dv <= 32 ? 1 : 2; }

template <int KP, int NVB>
hipError_t launch_tm(const float4 *xrec, const float *xbias, const float4 *col4, const float *colb,
                     const float *v, int64_t m, int dv, int k0, int64_t n, int64_t n_pad,
                     const MPlan &p, double *part, double *rpart, hipStream_t s) {
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    if (rpart)
        hipLaunchKernelGGL((transport_mfma_kernel<KP, NVB, true>), grid, dim3(kThreads), 0, s,
                           xrec, xbias, col4, colb, v, m, dv, k0, n, n_pad, p.tiles_per_split,
                           p.ntiles, part, rpart);
    else
        hipLaunchKernelGGL((transport_mfma_kernel<KP, NVB, false>), grid, dim3(kThreads), 0, s,
                           xrec, xbias, col4, colb, v, m, dv, k0, n, n_pad, p.tiles_per_split,
                           p.ntiles, part, rpart);
    return hipGetLastError();
}

template <int NVB>
hipError_t launch_tm_kp(int kp, const float4 *xrec, const float *xbias, const float4 *col4,
                        const float *colb, const float *v, int64_t m, int dv, int k0, int64_t n,
                        int64_t n_pad, const MPlan &p, double *part, double *rpart,
                        hipStream_t s) {
#define OTSK_TM(KPV)                                                                           \
    case KPV:                                                                                  \
        return launch_tm<KPV, NVB>(xrec, xbias, col4, colb, v, m, dv, k0, n, n_pad, p, part,   \
                                   rpart, s);
    switch (kp) {
        OTSK_TM(32)
        OTSK_TM(64)
        OTSK_TM(96)
        OTSK_TM(128)
    default:
        return hipErrorInvalidValue;
    }
#undef OTSK_TM
}

}  // namespace

size_t transport_mfma_scratch_doubles(int64_t n, int64_t m_pad, int dv, bool rowsum) {
    const MPlan p = plan_tm(n, m_pad);
    const size_t per_row = (size_t)(32 * value_blocks(dv)) + (rowsum ? 1 : 0);
    return (size_t)p.nsplit * (size_t)pad_points(n) * per_row;
}

hipError_t launch_transport_apply_mfma(int kp, const void *xrow, const float *xhat,
                                       const void *ycol, const float *yhat, const float *v,
                                       int64_t n, int64_t n_pad, int64_t m, int64_t m_pad, int dv,
                                       double *part, float *out, float *rowsum, hipStream_t s) {
    const MPlan p = plan_tm(n, m_pad);
    const int nvb = value_blocks(dv);
    const int vc = 32 * nvb;
    const float4 *xr = static_cast<const float4 *>(xrow);
    const float4 *col4 = static_cast<const float4 *>(ycol);
    const float *xbias = xhat;
    const float *ybias = yhat;
    // Row-sum partials follow the value partials in the scratch.
    double *rpart = rowsum ? part + (size_t)p.nsplit * (size_t)n_pad * (size_t)vc : nullptr;
    for (int k0 = 0; k0 < dv; k0 += vc) {
        double *rp = k0 == 0 ? rpart : nullptr;
        hipError_t e = nvb == 1 ? launch_tm_kp<1>(kp, xr, xbias, col4, ybias, v, m, dv, k0, n,
                                                  n_pad, p, part, rp, s)
                                : launch_tm_kp<2>(kp, xr, xbias, col4, ybias, v, m, dv, k0, n,
                                                  n_pad, p, part, rp, s);
        if (e != hipSuccess)
            return e;
        const int64_t total = n * vc;
        const unsigned blocks = (unsigned)((total + 255) / 256);
        if (nvb == 1)
            hipLaunchKernelGGL(transport_mfma_reduce_kernel<32>, dim3(blocks), dim3(256), 0, s,
                               part, p.nsplit, n, n_pad, dv, k0, out);
        else
            hipLaunchKernelGGL(transport_mfma_reduce_kernel<64>, dim3(blocks), dim3(256), 0, s,
                               part, p.nsplit, n, n_pad, dv, k0, out);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        if (rp) {
            hipLaunchKernelGGL(transport_mfma_reduce_kernel<1>,
                               dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, rp, p.nsplit,
                               n, n_pad, 1, 0, rowsum);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

}  // namespace otsk
