// Log-domain Sinkhorn half-step and plan-statistics pass for the widest
// feature dimensions, 448 < d <= 1024 (the pages measure up to d = 1024,
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", "Experimentelle
// Ergebnisse").
//
// Same update and same split-f16 records as the other matrix-core kernels
// (lse_h3.hip, lse_wide.hip): s_ij = (2 log2(e)/eps) p_i.q_j + qhat_j, an
// online base-2 log-sum-exp over j, phat_i = log2 w_i - lse_i, with each dot
// product formed as three split f16 products (hi.hi + lo.hi + hi.lo, fp32
// accumulation). What changes is who holds the row operands. The 16x16-tile
// kernel keeps a row's hi and lo parts in KP/4 registers per lane, 256 at
// KP = 1024, more than a lane has (and spills from KP = 448 on). Here the
// coordinates are split in four:
// wave (rg, q) of a workgroup holds quarter q (KQ = KP/4 coordinates, KQ/4
// registers) of the 16 rows of row group rg and forms the partial dot
// products of that quarter for every 16-column tile. The four partial
// accumulators of a row group meet in LDS; wave q then takes register q of
// each, i.e. column 4g + q of the tile for lane group g, adds the four
// partials in a fixed order (fp32), the column bias (fp32) and folds the
// score into its own running (max, sum) with the exact two-exp2 online
// update (one score per lane and tile, so the lazy scheme of the other
// kernels buys nothing here). At the end the 16 (max, sum) pairs of a row
// (4 lane groups x 4 waves) are combined in a fixed order.
//
// One column tile (16 columns, 4 KP bytes each) per LDS buffer, two buffers;
// the exchange of partial accumulators is double-buffered too, so one
// barrier per tile both publishes the partials and releases the next tile.
// The epilogue of tile t runs after the chain of tile t+1 has been issued.
#include "mfma_common.h"

#include <math.h>

namespace otsk {

namespace {

using namespace mfma;

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTC = 16;  // columns per tile: one 16x16 subtile
constexpr int kQuarters = 4;
constexpr int kTargetBlocks = 1024;
constexpr int kLdsBytes = 160 * 1024;

// Bytes of LDS with rg row groups: two record tiles, two exchange buffers
// (a float4 per lane and wave), two bias and two norm tiles.
__host__ __device__ constexpr int ks_lds_bytes(int kp, int rg) {
    return 2 * kTC * (kp / 4) * 16 + 2 * rg * kQuarters * 64 * 16 + 4 * kTC * 4;
}

// Row groups per workgroup: 4 (64 rows, 16 waves: 4 per SIMD, 128 registers
// per lane) up to KP = 768, else 3 (48 rows, 12 waves, 168 registers): at
// KP = 1024 four row groups do not fit the LDS, at 896 the cost pass would
// spill registers.
__host__ __device__ constexpr int ks_row_groups(int kp) { return kp <= 768 ? 4 : 3; }

// Copy column tile t (16 records of KP/4 16-byte chunks, 16 biases and, for
// the statistics, 16 norms) into LDS with direct global->LDS loads.
template <int KP, int NW>
__device__ __forceinline__ void issue_ks_tile(const float4 *__restrict__ col4,
                                              const float *__restrict__ colb,
                                              const float *__restrict__ coln, int t, float4 *rec,
                                              float *bias, float *nrm, int wave, int lane) {
    constexpr int CH = kTC * (KP / 4) / 64;  // 64-lane chunks per tile
    const float4 *src = col4 + (int64_t)t * (kTC * (KP / 4));
#pragma unroll
    for (int c = 0; c < CH; c += NW) {
        const int chunk = c + wave;
        if (CH % NW == 0 || chunk < CH)
            __builtin_amdgcn_global_load_lds(src + chunk * 64 + lane,
                                             (lds_void *)(rec + chunk * 64), 16, 0, 0);
    }
    if (wave == NW - 1 && lane < kTC)
        __builtin_amdgcn_global_load_lds(colb + (int64_t)t * kTC + lane, (lds_void *)bias, 4, 0,
                                         0);
    if (coln && wave == NW - 2 && lane < kTC)
        __builtin_amdgcn_global_load_lds(coln + (int64_t)t * kTC + lane, (lds_void *)nrm, 4, 0, 0);
}

// Partial dot products of quarter q (coordinates q*KQ ... q*KQ + KQ - 1) of
// the tile's 16 columns (column j = lane % 16 of record array `rec`) against
// the lane's stationary row operands of that quarter: lo corrections first,
// hi x hi onto them (the order of the other kernels' chains); the column hi
// operands stay in registers for the hi x hi products.
template <int KP>
__device__ __forceinline__ floatx4 quarter_dot(const float4 *rec, int q, int lane, int g,
                                               const half8 (&bh)[KP / 128],
                                               const half8 (&bl)[KP / 128]) {
    constexpr int RC = KP / 4;
    constexpr int KC = KP / 128;  // k-steps of 32 coordinates per quarter
    constexpr int SW = swizzle_mask(RC);
    const int j = lane & 15;
    const float4 *ap = rec + j * RC;
    const int sw = j & SW;
    const int c0 = q * KC;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    half8 qh[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
        qh[c] = as_half8(ap[(4 * (c0 + c) + g) ^ sw]);
        const half8 ql = as_half8(ap[(KP / 8 + 4 * (c0 + c) + g) ^ sw]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, bh[c], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[c], bl[c], acc, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < KC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[c], bh[c], acc, 0, 0, 0);
    return acc;
}

// Sum of the four quarters' partials of register q for this lane, in
// quarter order: xb points at the row group's four float4-per-lane blocks.
__device__ __forceinline__ float quarter_sum(const float *xb, int q, int lane) {
    const float v0 = xb[(0 * 64 + lane) * 4 + q];
    const float v1 = xb[(1 * 64 + lane) * 4 + q];
    const float v2 = xb[(2 * 64 + lane) * 4 + q];
    const float v3 = xb[(3 * 64 + lane) * 4 + q];
    return ((v0 + v1) + v2) + v3;
}

// (M, S) <- the log-sum-exp pair of (M, S) and (Mo, So): max, rescaled sum.
__device__ __forceinline__ void lse_combine(float &M, float &S, float Mo, float So) {
    const float Mn = fmaxf(M, Mo);
    S = S * hw_exp2(M - Mn) + So * hw_exp2(Mo - Mn);
    M = Mn;
}

template <int KP, int RG>
__global__ __launch_bounds__(64 * kQuarters * RG) void lse_rows_ksplit_kernel(
    HalfStep h, int tiles_per_split, int ntiles, int nrb, int nsplit) {
    constexpr int NW = kQuarters * RG;
    constexpr int RC = KP / 4;
    constexpr int KC = KP / 128;
    static_assert(KP % 128 == 0, "quarters of whole k-steps");
    static_assert(ks_lds_bytes(KP, RG) <= kLdsBytes, "LDS budget");
    __shared__ float4 lrec[2][kTC * RC];
    __shared__ float4 xbuf[2][RG * kQuarters * 64];
    __shared__ float lbias[2][kTC];

    int rblk, split;
    xcd_block(nrb, nsplit, rblk, split);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = wave / kQuarters;
    const int q = wave % kQuarters;
    const int g = lane >> 4;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const float4 *col4 = static_cast<const float4 *>(h.col_rec);
    const float *colb = static_cast<const float *>(h.col_bias);

    issue_ks_tile<KP, NW>(col4, colb, nullptr, tbeg, lrec[0], lbias[0], nullptr, wave, lane);
    const int64_t i = (int64_t)rblk * (16 * RG) + rg * 16 + (lane & 15);
    const int64_t ic = i < h.rows ? i : h.rows - 1;
    half8 bh[KC], bl[KC];
    {
        const float4 *rr = static_cast<const float4 *>(h.row_rec) + ic * RC;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            bh[c] = as_half8(rr[4 * (q * KC + c) + g]);
            bl[c] = as_half8(rr[KP / 8 + 4 * (q * KC + c) + g]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Running maximum and sum of this lane's columns (4g + q of each tile).
    // The maximum starts at the padding bias, finite, so the first update
    // never forms (-inf) - (-inf).
    float M = kPadBias, S = 0.f;
    float bias_prev = 0.f;
    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        // Buffer b^1 was last read by the chain of tile t-1, before the
        // previous barrier; that tile's bias is already in bias_prev.
        if (t + 1 < tend)
            issue_ks_tile<KP, NW>(col4, colb, nullptr, t + 1, lrec[b ^ 1], lbias[b ^ 1], nullptr,
                                  wave, lane);
        const floatx4 acc = quarter_dot<KP>(lrec[b], q, lane, g, bh, bl);
        if (t > tbeg) {
            // Tile t-1: its partials were published by the previous barrier.
            const float *xb = reinterpret_cast<const float *>(&xbuf[b ^ 1][rg * kQuarters * 64]);
            const float s = quarter_sum(xb, q, lane) + bias_prev;
            const float Mn = fmaxf(M, s);
            S = S * hw_exp2(M - Mn) + hw_exp2(s - Mn);
            M = Mn;
        }
        bias_prev = lbias[b][4 * g + q];
        xbuf[b][(rg * kQuarters + q) * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    {
        const int b = (tend - 1 - tbeg) & 1;
        const float *xb = reinterpret_cast<const float *>(&xbuf[b][rg * kQuarters * 64]);
        const float s = quarter_sum(xb, q, lane) + bias_prev;
        const float Mn = fmaxf(M, s);
        S = S * hw_exp2(M - Mn) + hw_exp2(s - Mn);
        M = Mn;
    }
    // The row's 16 pairs: the four lane groups (butterfly, the same result on
    // every lane), then the four quarters in order through LDS (the exchange
    // buffer is free: every wave has read it before the last barrier... and
    // the barrier below orders the writes).
    lse_combine(M, S, __shfl_xor(M, 16), __shfl_xor(S, 16));
    lse_combine(M, S, __shfl_xor(M, 32), __shfl_xor(S, 32));
    __syncthreads();
    float2 *red = reinterpret_cast<float2 *>(&xbuf[0][0]);
    if (g == 0)
        red[(rg * kQuarters + q) * 16 + (lane & 15)] = make_float2(M, S);
    __syncthreads();
    if (q == 0 && g == 0) {
        float2 p = red[(rg * kQuarters + 0) * 16 + lane];
        float Mr = p.x, Sr = p.y;
#pragma unroll
        for (int o = 1; o < kQuarters; ++o) {
            p = red[(rg * kQuarters + o) * 16 + lane];
            lse_combine(Mr, Sr, p.x, p.y);
        }
        if (i < h.rows) {
            if (nsplit == 1) {
                const float lse = Mr + hw_log2(Sr);
                const float hat = log2f(h.row_w[i]) - lse;
                static_cast<float *>(h.row_bias)[i] = hat;
                h.pot_out[i] = fmaf((float)h.eps_ln2, hat, h.row_nrm[i]);
            } else {
                h.partials[(int64_t)split * h.rows_pad + i] = Partial{(double)Mr, Sr, 0.f};
            }
        }
    }
}

// One plan-statistics pass: part[split][row] = (sum_j P_ij, COST ?
// sum_j P_ij C_ij : 0) with log2 P_ij = dot + qhat_j + phat_i (fp32, in
// that order) and C_ij = |p_i|^2 + |q_j|^2 - 2 p_i.q_j from the same dot
// product; sums in fp64.
template <int KP, int RG, bool COST>
__global__ __launch_bounds__(64 * kQuarters * RG) void plan_rows_ksplit_kernel(
    const float4 *__restrict__ row_rec, const float *__restrict__ row_hat,
    const float *__restrict__ row_nrm, const float4 *__restrict__ col4,
    const float *__restrict__ colb, const float *__restrict__ col_nrm, int64_t rows,
    int64_t rows_pad, int tiles_per_split, int ntiles, float inv_scale,
    double2 *__restrict__ part) {
    constexpr int NW = kQuarters * RG;
    constexpr int RC = KP / 4;
    constexpr int KC = KP / 128;
    static_assert(ks_lds_bytes(KP, RG) <= kLdsBytes, "LDS budget");
    __shared__ float4 lrec[2][kTC * RC];
    __shared__ float4 xbuf[2][RG * kQuarters * 64];
    __shared__ float lbias[2][kTC];
    __shared__ float lnrm[2][kTC];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = wave / kQuarters;
    const int q = wave % kQuarters;
    const int g = lane >> 4;
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const float *cn = COST ? col_nrm : nullptr;

    issue_ks_tile<KP, NW>(col4, colb, cn, tbeg, lrec[0], lbias[0], lnrm[0], wave, lane);
    const int64_t i = (int64_t)blockIdx.x * (16 * RG) + rg * 16 + (lane & 15);
    const int64_t ic = i < rows ? i : rows - 1;
    half8 bh[KC], bl[KC];
    {
        const float4 *rr = row_rec + ic * RC;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            bh[c] = as_half8(rr[4 * (q * KC + c) + g]);
            bl[c] = as_half8(rr[KP / 8 + 4 * (q * KC + c) + g]);
        }
    }
    const float ph = row_hat[ic];
    const float nx = COST ? row_nrm[ic] : 0.f;
    const float m2 = -2.f * inv_scale;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    double rsum = 0.0, csum = 0.0;
    float bias_prev = 0.f, ny_prev = 0.f;
    auto fold_tile = [&](int bx) {
        const float *xb = reinterpret_cast<const float *>(&xbuf[bx][rg * kQuarters * 64]);
        const float dot = quarter_sum(xb, q, lane);
        const float pr = hw_exp2((dot + bias_prev) + ph);
        rsum += (double)pr;
        if (COST) {
            const float cij = fmaf(dot, m2, nx + ny_prev);
            csum = fma((double)pr, (double)cij, csum);
        }
    };
    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        if (t + 1 < tend)
            issue_ks_tile<KP, NW>(col4, colb, cn, t + 1, lrec[b ^ 1], lbias[b ^ 1], lnrm[b ^ 1],
                                  wave, lane);
        const floatx4 acc = quarter_dot<KP>(lrec[b], q, lane, g, bh, bl);
        if (t > tbeg)
            fold_tile(b ^ 1);
        bias_prev = lbias[b][4 * g + q];
        if (COST)
            ny_prev = lnrm[b][4 * g + q];
        xbuf[b][(rg * kQuarters + q) * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    fold_tile((tend - 1 - tbeg) & 1);
    // Lane groups (butterfly), then quarters in order through LDS.
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    csum += __shfl_xor(csum, 16);
    csum += __shfl_xor(csum, 32);
    __syncthreads();
    double2 *red = reinterpret_cast<double2 *>(&xbuf[0][0]);
    if (g == 0)
        red[(rg * kQuarters + q) * 16 + (lane & 15)] = make_double2(rsum, csum);
    __syncthreads();
    if (q == 0 && g == 0) {
        double2 acc = red[(rg * kQuarters + 0) * 16 + lane];
#pragma unroll
        for (int o = 1; o < kQuarters; ++o) {
            const double2 p = red[(rg * kQuarters + o) * 16 + lane];
            acc.x += p.x;
            acc.y += p.y;
        }
        if (i < rows)
            part[(int64_t)split * rows_pad + i] = acc;
    }
}

struct KPlan {
    int ntiles;
    int tiles_per_split;
    int nsplit;
    int64_t row_blocks;
};

KPlan plan_ksplit(int64_t rows, int64_t cols_pad, int kp) {
    KPlan p;
    p.ntiles = (int)(cols_pad / kTC);
    const int rows_per_block = 16 * ks_row_groups(kp);
    p.row_blocks = (rows + rows_per_block - 1) / rows_per_block;
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

template <int KP>
hipError_t launch_ksplit_kp(const HalfStep &h, const KPlan &p, hipStream_t s) {
    constexpr int RG = ks_row_groups(KP);
    dim3 grid((unsigned)(p.row_blocks * p.nsplit));
    hipLaunchKernelGGL((lse_rows_ksplit_kernel<KP, RG>), grid, dim3(64 * kQuarters * RG), 0, s, h,
                       p.tiles_per_split, p.ntiles, (int)p.row_blocks, p.nsplit);
    return hipGetLastError();
}

template <int KP, bool COST>
hipError_t launch_plan_ksplit_kp(const KPlan &p, const float4 *rr, const float *row_hat,
                                 const float *row_nrm, const float4 *cr, const float *col_hat,
                                 const float *col_nrm, int64_t rows, int64_t rows_pad, float inv,
                                 double2 *part, hipStream_t s) {
    constexpr int RG = ks_row_groups(KP);
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    hipLaunchKernelGGL((plan_rows_ksplit_kernel<KP, RG, COST>), grid, dim3(64 * kQuarters * RG), 0,
                       s, rr, row_hat, row_nrm, cr, col_hat, col_nrm, rows, rows_pad,
                       p.tiles_per_split, p.ntiles, inv, part);
    return hipGetLastError();
}

}  // namespace

bool ksplit_kp(int kp) {
    return kp == 512 || kp == 640 || kp == 768 || kp == 896 || kp == 1024;
}

size_t half_step_partials_ksplit(int64_t rows, int64_t cols_pad, int kp) {
    const KPlan p = plan_ksplit(rows, cols_pad, kp);
    return p.nsplit > 1 ? (size_t)p.nsplit * (size_t)pad_points(rows) : 0;
}

hipError_t launch_half_step_ksplit(const HalfStep &h, int kp, hipStream_t s) {
    const KPlan p = plan_ksplit(h.rows, h.cols_pad, kp);
    hipError_t e;
    switch (kp) {
    case 512: e = launch_ksplit_kp<512>(h, p, s); break;
    case 640: e = launch_ksplit_kp<640>(h, p, s); break;
    case 768: e = launch_ksplit_kp<768>(h, p, s); break;
    case 896: e = launch_ksplit_kp<896>(h, p, s); break;
    case 1024: e = launch_ksplit_kp<1024>(h, p, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.nsplit <= 1)
        return e;
    return launch_merge_h3(h, p.nsplit, s);
}

int plan_pass_ksplit_splits(int64_t rows, int64_t cols_pad, int kp) {
    return plan_ksplit(rows, cols_pad, kp).nsplit;
}

hipError_t launch_plan_pass_ksplit(int kp, bool cost, const void *row_rec, const float *row_hat,
                                   const float *row_nrm, const void *col_rec,
                                   const float *col_hat, const float *col_nrm, int64_t rows,
                                   int64_t rows_pad, int64_t cols_pad, double scale,
                                   double2 *part, hipStream_t s) {
    const KPlan p = plan_ksplit(rows, cols_pad, kp);
    const float4 *rr = static_cast<const float4 *>(row_rec);
    const float4 *cr = static_cast<const float4 *>(col_rec);
    const float inv = (float)(1.0 / scale);
#define OTSK_PK(KPV)                                                                           \
    case KPV:                                                                                  \
        return cost ? launch_plan_ksplit_kp<KPV, true>(p, rr, row_hat, row_nrm, cr, col_hat,   \
                                                       col_nrm, rows, rows_pad, inv, part, s)  \
                    : launch_plan_ksplit_kp<KPV, false>(p, rr, row_hat, row_nrm, cr, col_hat,  \
                                                        col_nrm, rows, rows_pad, inv, part, s);
    switch (kp) {
        OTSK_PK(512)
        OTSK_PK(640)
        OTSK_PK(768)
        OTSK_PK(896)
        OTSK_PK(1024)
    default:
        return hipErrorInvalidValue;
    }
#undef OTSK_PK
}

}  // namespace otsk
