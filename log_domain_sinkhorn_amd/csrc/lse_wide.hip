// Log-domain Sinkhorn half-step and plan-statistics pass for wide feature
// dimensions, 192 < d <= 448 (the pages measure up to d = 1024, "FlashSinkhorn:
// IO-Aware Entropic Optimal Transport on GPU", "Experimentelle Ergebnisse").
//
// The update is the one of the other half-step kernels ("Methodik" sections
// 1-2): s_ij = (2 log2(e)/eps) p_i.q_j + qhat_j, an online base-2 log-sum-exp
// over j, phat_i = log2 w_i - lse_i, with the dot products formed as three
// split f16 products (hi.hi + lo.hi + hi.lo, fp32 accumulation) on the same
// split-f16 records (see lse_h3.hip). What differs is the tile shape: the
// 32x32 kernels hold a row's hi and lo operands in KP/2 registers per lane,
// which spill above KP = 192. Here every wave owns 16 rows and runs
// v_mfma_f32_16x16x32_f16, whose stationary operand takes KP/4 registers per
// lane (112 at KP = 448): lane l holds row i = l % 16 and the 8-coordinate
// group g = l / 16 of every 32-coordinate k-step; the accumulator holds
// D[j][i] for the 4 columns j = 4g + r of the lane's 16-column subtile, so
// a row's running maximum and sum are shared by the 4 lane groups (lanes l,
// l ^ 16, l ^ 32, l ^ 48). The column bias and the row's running maximum
// enter through one v_mfma_f32_16x16x4f32 at the end of the chain (k-slot 0:
// bias_j x 1, k-slot 1: 1 x -M_i), as in the 32x32 kernels. Each column
// operand now feeds 16 rows instead of 32, so the LDS operand traffic per
// flop doubles; that is the price of the register budget.
#include "mfma_common.h"

#include <math.h>
#include <type_traits>

namespace otsk {

namespace {

using namespace mfma;

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 16 * kWaves;
constexpr int kTargetBlocks = 1024;

// Columns per LDS tile: one buffer, TC * KP * 4 bytes, stays at 64 KiB or
// less, so the double buffer fits one workgroup per CU.
__host__ __device__ constexpr int wide_tile_cols(int kp) { return kp <= 256 ? 64 : 32; }

// Copy column tile t (TILE4 16-byte chunks of records, TC biases) into LDS
// with direct global->LDS loads.
template <int TILE4, int TC>
__device__ __forceinline__ void issue_wide_tile(const float4 *__restrict__ col4,
                                                const float *__restrict__ colb, int t,
                                                float4 *rec, float *bias, int wave, int lane) {
    static_assert(TILE4 % (64 * kWaves) == 0, "whole chunk rounds per wave");
    const float4 *src = col4 + (int64_t)t * TILE4;
#pragma unroll
    for (int c = 0; c < TILE4 / 64; c += kWaves) {
        const int chunk = c + wave;
        __builtin_amdgcn_global_load_lds(src + chunk * 64 + lane, (lds_void *)(rec + chunk * 64),
                                         16, 0, 0);
    }
    if (wave == kWaves - 1 && lane < TC)
        __builtin_amdgcn_global_load_lds(colb + (int64_t)t * TC + lane, (lds_void *)bias, 4, 0,
                                         0);
}

// Dot products of the lane's 16-column subtile `sub` (columns j = sub*16 +
// l % 16 of the tile in `rec`) against the stationary row operands:
// D[j][i] = p_i.q_j (scaled), lo corrections first, hi x hi onto them.
template <int KP>
__device__ __forceinline__ floatx4 split_dot_wide(const float4 *rec, int sub, int lane, int g,
                                                  const half8 (&bh)[KP / 32],
                                                  const half8 (&bl)[KP / 32]) {
    constexpr int RC = KP / 4;
    constexpr int SW = swizzle_mask(RC);
    const int j = sub * 16 + (lane & 15);
    const float4 *ap = rec + j * RC;
    const int sw = j & SW;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KP <= 256) {
        half8 qh[KP / 32];
#pragma unroll
        for (int c = 0; c < KP / 32; ++c) {
            qh[c] = as_half8(ap[(4 * c + g) ^ sw]);
            const half8 ql = as_half8(ap[(KP / 8 + 4 * c + g) ^ sw]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, bh[c], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[c], bl[c], acc, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < KP / 32; ++c)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[c], bh[c], acc, 0, 0, 0);
    } else {
        // Above KP = 256 the hi operands are read a second time for the
        // hi x hi products instead of being held beside the row operands.
#pragma unroll
        for (int c = 0; c < KP / 32; ++c) {
            const half8 ql = as_half8(ap[(KP / 8 + 4 * c + g) ^ sw]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, bh[c], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(ap[(4 * c + g) ^ sw]), bl[c],
                                                         acc, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < KP / 32; ++c)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(ap[(4 * c + g) ^ sw]), bh[c],
                                                         acc, 0, 0, 0);
    }
    return acc;
}

// dot + bias_j - Mu_i through one fp32 MFMA: lanes 0-15 give A[j][0] = bias_j
// and B[0][i] = 1, lanes 16-31 give A[j][1] = 1 and B[1][i] = -Mu_i, lanes
// 32-63 the zero k-slots 2 and 3.
__device__ __forceinline__ floatx4 add_bias_wide(const floatx4 &dot, const float *bias, int sub,
                                                 int lane, float Mu) {
    const float a0 = lane < 16 ? bias[sub * 16 + lane] : (lane < 32 ? 1.f : 0.f);
    const float b0 = lane < 16 ? 1.f : (lane < 32 ? -Mu : 0.f);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, dot, 0, 0, 0);
}

template <int KP>
__device__ __forceinline__ floatx4 score_wide(const float4 *rec, const float *bias, int sub,
                                              int lane, int g, const half8 (&bh)[KP / 32],
                                              const half8 (&bl)[KP / 32], float Mu) {
    return add_bias_wide(split_dot_wide<KP>(rec, sub, lane, g, bh, bl), bias, sub, lane, Mu);
}

__device__ __forceinline__ float chunk_sum4(const floatx4 &u) {
    return (hw_exp2(u[0]) + hw_exp2(u[1])) + (hw_exp2(u[2]) + hw_exp2(u[3]));
}

// Fold a subtile (values u relative to Mu, sum c) into the row's (M, S); the
// four lane groups of a row keep the same M (the same rule as the 32x32
// kernels' epilogue, over 4 values per lane).
__device__ __forceinline__ void fold4(const floatx4 &u, float Mu, float c, float &M, float &S) {
    const bool need = !(c <= 0x1p16f) || !(S + c >= 0x1p-64f) || Mu != M;
    if (__builtin_amdgcn_ballot_w64(need)) {
        float mh = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
        mh = fmaxf(mh + Mu, M + hw_log2(S));
        mh = fmaxf(mh, __shfl_xor(mh, 16));
        const float Mn = fmaxf(mh, __shfl_xor(mh, 32));
        S = S == 0.f ? 0.f : S * hw_exp2(M - Mn);
        const float off = Mn - Mu;
        c = (hw_exp2(u[0] - off) + hw_exp2(u[1] - off)) +
            (hw_exp2(u[2] - off) + hw_exp2(u[3] - off));
        M = Mn;
    }
    S += c;
}

template <int KP>
__global__ __launch_bounds__(kThreads) void lse_rows_wide_kernel(HalfStep h, int tiles_per_split,
                                                                 int ntiles, int nrb,
                                                                 int nsplit) {
    int rblk, split;
    xcd_block(nrb, nsplit, rblk, split);
    constexpr int RC = KP / 4;
    constexpr int TC = wide_tile_cols(KP);
    constexpr int SUB = TC / 16;
    constexpr int TILE4 = TC * RC;
    static_assert(KP % 32 == 0, "whole k-steps");
    __shared__ float4 lrec[2][TILE4];
    __shared__ float lbias[2][TC];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const float4 *col4 = static_cast<const float4 *>(h.col_rec);
    const float *colb = static_cast<const float *>(h.col_bias);

    issue_wide_tile<TILE4, TC>(col4, colb, tbeg, lrec[0], lbias[0], wave, lane);
    const int64_t i = (int64_t)rblk * kRowsPerBlock + wave * 16 + (lane & 15);
    const int64_t ic = i < h.rows ? i : h.rows - 1;
    half8 bh[KP / 32], bl[KP / 32];
    {
        const float4 *rr = static_cast<const float4 *>(h.row_rec) + ic * RC;
#pragma unroll
        for (int c = 0; c < KP / 32; ++c) {
            bh[c] = as_half8(rr[4 * c + g]);
            bl[c] = as_half8(rr[KP / 8 + 4 * c + g]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    float M = 0.f;
    float S = 0.f;
    float Mu_prev = M;
    floatx4 acc_prev = score_wide<KP>(lrec[0], lbias[0], 0, lane, g, bh, bl, Mu_prev);
    auto tile = [&](int t, auto bc) {
        constexpr int b = decltype(bc)::value;
        if (t + 1 < tend)
            issue_wide_tile<TILE4, TC>(col4, colb, t + 1, lrec[b ^ 1], lbias[b ^ 1], wave, lane);
#pragma unroll
        for (int sub = 1; sub < SUB; ++sub) {
            const float Mu_cur = M;
            const floatx4 acc_cur =
                score_wide<KP>(lrec[b], lbias[b], sub, lane, g, bh, bl, Mu_cur);
            const float c = chunk_sum4(acc_prev);
            fold4(acc_prev, Mu_prev, c, M, S);
            pin(M, S);
            acc_prev = acc_cur;
            Mu_prev = Mu_cur;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // First subtile of the next tile (on the last tile: the idle buffer,
        // never folded).
        const float Mu_cur = M;
        const floatx4 acc_cur =
            score_wide<KP>(lrec[b ^ 1], lbias[b ^ 1], 0, lane, g, bh, bl, Mu_cur);
        const float c = chunk_sum4(acc_prev);
        fold4(acc_prev, Mu_prev, c, M, S);
        pin(M, S);
        acc_prev = acc_cur;
        Mu_prev = Mu_cur;
    };
    for (int t = tbeg; t < tend; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < tend)
            tile(t + 1, std::integral_constant<int, 1>{});
    }

    float Sm = S + __shfl_xor(S, 16);
    Sm += __shfl_xor(Sm, 32);
    if (g == 0 && i < h.rows) {
        if (nsplit == 1) {
            const float lse = M + hw_log2(Sm);
            const float hat = log2f(h.row_w[i]) - lse;
            static_cast<float *>(h.row_bias)[i] = hat;
            h.pot_out[i] = fmaf((float)h.eps_ln2, hat, h.row_nrm[i]);
        } else {
            h.partials[(int64_t)split * h.rows_pad + i] = Partial{(double)M, Sm, 0.f};
        }
    }
}

// One plan-statistics pass on the wide records: part[split][row] =
// (sum_j P_ij, COST ? sum_j P_ij C_ij : 0) with log2 P_ij from the split
// chain plus the fp32 bias MFMA (qhat_j and phat_i), and
// C_ij = |p_i|^2 + |q_j|^2 - 2 p_i.q_j from the chain's dot product. Sums are
// fp32 within a column tile and fp64 across tiles.
template <int KP, bool COST>
__global__ __launch_bounds__(kThreads) void plan_rows_wide_kernel(
    const float4 *__restrict__ row_rec, const float *__restrict__ row_hat,
    const float *__restrict__ row_nrm, const float4 *__restrict__ col4,
    const float *__restrict__ colb, const float *__restrict__ col_nrm, int64_t rows,
    int64_t rows_pad, int tiles_per_split, int ntiles, float inv_scale,
    double2 *__restrict__ part) {
    constexpr int RC = KP / 4;
    constexpr int TC = wide_tile_cols(KP);
    constexpr int SUB = TC / 16;
    constexpr int TILE4 = TC * RC;
    __shared__ float4 lrec[2][TILE4];
    __shared__ float lbias[2][TC];
    __shared__ __attribute__((aligned(16))) float lnrm[2][TC];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);

    auto issue_norms = [&](int t, float *dst) {
        if (COST && wave == 0 && lane < TC)
            __builtin_amdgcn_global_load_lds(col_nrm + (int64_t)t * TC + lane, (lds_void *)dst, 4,
                                             0, 0);
    };
    issue_wide_tile<TILE4, TC>(col4, colb, tbeg, lrec[0], lbias[0], wave, lane);
    issue_norms(tbeg, lnrm[0]);
    const int64_t i = (int64_t)blockIdx.x * kRowsPerBlock + wave * 16 + (lane & 15);
    const int64_t ic = i < rows ? i : rows - 1;
    half8 bh[KP / 32], bl[KP / 32];
    {
        const float4 *rr = row_rec + ic * RC;
#pragma unroll
        for (int c = 0; c < KP / 32; ++c) {
            bh[c] = as_half8(rr[4 * c + g]);
            bl[c] = as_half8(rr[KP / 8 + 4 * c + g]);
        }
    }
    // With Mu = -phat_i the bias MFMA adds qhat_j + phat_i.
    const float Mu = -row_hat[ic];
    const float nx = COST ? row_nrm[ic] : 0.f;
    const float m2 = -2.f * inv_scale;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    double rsum = 0.0, csum = 0.0;
    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        if (t + 1 < tend) {
            issue_wide_tile<TILE4, TC>(col4, colb, t + 1, lrec[b ^ 1], lbias[b ^ 1], wave, lane);
            issue_norms(t + 1, lnrm[b ^ 1]);
        }
        float rs = 0.f, cs = 0.f;
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
            const floatx4 dot = split_dot_wide<KP>(lrec[b], sub, lane, g, bh, bl);
            const floatx4 u = add_bias_wide(dot, lbias[b], sub, lane, Mu);
            float4 ny = make_float4(0.f, 0.f, 0.f, 0.f);
            if (COST)
                ny = *reinterpret_cast<const float4 *>(&lnrm[b][sub * 16 + 4 * g]);
            const float nyv[4] = {ny.x, ny.y, ny.z, ny.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pr = hw_exp2(u[r]);
                rs += pr;
                if (COST) {
                    const float cij = fmaf(dot[r], m2, nx + nyv[r]);
                    cs = fmaf(pr, cij, cs);
                }
            }
        }
        rsum += (double)rs;
        csum += (double)cs;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    double ro = rsum + __shfl_xor(rsum, 16);
    ro += __shfl_xor(ro, 32);
    double co = csum + __shfl_xor(csum, 16);
    co += __shfl_xor(co, 32);
    if (g == 0 && i < rows)
        part[(int64_t)split * rows_pad + i] = make_double2(ro, co);
}

struct WPlan {
    int ntiles;
    int tiles_per_split;
    int nsplit;
    int64_t row_blocks;
};

WPlan plan_wide(int64_t rows, int64_t cols_pad, int kp) {
    WPlan p;
    p.ntiles = (int)(cols_pad / wide_tile_cols(kp));
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

template <int KP>
hipError_t launch_wide_kp(const HalfStep &h, const WPlan &p, hipStream_t s) {
    dim3 grid((unsigned)(p.row_blocks * p.nsplit));
    hipLaunchKernelGGL((lse_rows_wide_kernel<KP>), grid, dim3(kThreads), 0, s, h,
                       p.tiles_per_split, p.ntiles, (int)p.row_blocks, p.nsplit);
    return hipGetLastError();
}

}  // namespace

bool wide_kp(int kp) { return kp == 224 || kp == 256 || kp == 320 || kp == 384 || kp == 448; }

size_t half_step_partials_wide(int64_t rows, int64_t cols_pad, int kp) {
    const WPlan p = plan_wide(rows, cols_pad, kp);
    return p.nsplit > 1 ? (size_t)p.nsplit * (size_t)pad_points(rows) : 0;
}

hipError_t launch_half_step_wide(const HalfStep &h, int kp, hipStream_t s) {
    const WPlan p = plan_wide(h.rows, h.cols_pad, kp);
    hipError_t e;
    switch (kp) {
    case 224: e = launch_wide_kp<224>(h, p, s); break;
    case 256: e = launch_wide_kp<256>(h, p, s); break;
    case 320: e = launch_wide_kp<320>(h, p, s); break;
    case 384: e = launch_wide_kp<384>(h, p, s); break;
    case 448: e = launch_wide_kp<448>(h, p, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.nsplit <= 1)
        return e;
    return launch_merge_h3(h, p.nsplit, s);
}

int plan_pass_wide_splits(int64_t rows, int64_t cols_pad, int kp) {
    return plan_wide(rows, cols_pad, kp).nsplit;
}

hipError_t launch_plan_pass_wide(int kp, bool cost, const void *row_rec, const float *row_hat,
                                 const float *row_nrm, const void *col_rec, const float *col_hat,
                                 const float *col_nrm, int64_t rows, int64_t rows_pad,
                                 int64_t cols_pad, double scale, double2 *part, hipStream_t s) {
    const WPlan p = plan_wide(rows, cols_pad, kp);
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    const float4 *rr = static_cast<const float4 *>(row_rec);
    const float4 *cr = static_cast<const float4 *>(col_rec);
    const float inv = (float)(1.0 / scale);
#define OTSK_PW(KPV)                                                                            \
    case KPV:                                                                                   \
        if (cost)                                                                               \
            hipLaunchKernelGGL((plan_rows_wide_kernel<KPV, true>), grid, dim3(kThreads), 0, s, \
                               rr, row_hat, row_nrm, cr, col_hat, col_nrm, rows, rows_pad,      \
                               p.tiles_per_split, p.ntiles, inv, part);                         \
        else                                                                                    \
            hipLaunchKernelGGL((plan_rows_wide_kernel<KPV, false>), grid, dim3(kThreads), 0,   \
                               s, rr, row_hat, row_nrm, cr, col_hat, col_nrm, rows, rows_pad,   \
                               p.tiles_per_split, p.ntiles, inv, part);                         \
        break;
    switch (kp) {
        OTSK_PW(224)
        OTSK_PW(256)
        OTSK_PW(320)
        OTSK_PW(384)
        OTSK_PW(448)
    default:
        return hipErrorInvalidValue;
    }
#undef OTSK_PW
    return hipGetLastError();
}

}  // namespace otsk
