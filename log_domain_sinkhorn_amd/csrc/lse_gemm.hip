// Log-domain Sinkhorn half-step and plan-statistics pass for the widest
// feature dimensions, 448 < d <= 1024 (the pages measure up to d = 1024,
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", "Experimentelle
// Ergebnisse"), tiled like a matrix product.
//
// Same update and same split-f16 records as the other matrix-core kernels
// (lse_h3.hip): s_ij = (2 log2(e)/eps) p_i.q_j + qhat_j, an online base-2
// log-sum-exp over j, phat_i = log2 w_i - lse_i, each dot product formed as
// three split f16 products (hi.hi + lo.hi + hi.lo) with fp32 accumulation.
//
// At these sizes a row's split operands (4 KP bytes) no longer fit a lane's
// registers, so neither side is stationary. A workgroup of 8 waves owns 256
// rows and walks its column split in blocks of 128 columns; for each block
// the coordinates go through LDS in stages of 32 (the 256 row and 128
// column records' 4 hi and 4 lo 16-byte chunks of that stage, 48 KiB),
// three stages deep, filled by gfx950's direct global->LDS loads two stages
// ahead of the one being multiplied. Wave (rw, cw) forms the 64 x 64 block of
// rows 64 rw .. 64 rw + 63 and columns 64 cw .. 64 cw + 63 as 2 x 2
// v_mfma_f32_32x32x16_f16 subtiles (D[j][i]: lane l holds row l mod 32 and
// 16 columns, as in lse_h3.hip). Per stage and subtile the chain starts from
// zero, takes the lo corrections of both 16-coordinate chunks and then the
// hi x hi products, and is added to an fp32 running sum: the matrix core's
// aligned sum loses about 2^-21 of its largest term, so no chain may grow
// past one stage's share of the dot product. After the last stage of a
// block the sums go to the block epilogue: for the half-step, the sums plus
// the column biases (fp32) are folded into each row's running (max, sum)
// with the lazy epilogue of the other kernels; for the statistics, P_ij and
// P_ij C_ij are added to fp64 row sums. The two waves that share rows
// combine their results through LDS at the end, in a fixed order.
//
// Workgroup order: the 1-D grid is dealt so that the column splits of one
// row block run on one XCD (workgroup L goes to XCD L mod 8), so that
// block's row records, re-read for every column block, stay in that XCD's L2.
//
// The stage pipeline, the workgroup order and the grid plan are in
// gemm_pipeline.h (shared with the transport application); these kernels run
// it with two row subtiles per wave.
#include "gemm_pipeline.h"

#include <math.h>

namespace otsk {

namespace {

using namespace mfma;
using namespace gemm;

constexpr int kGBM = GTile<2>::BM;         // rows per workgroup
constexpr int kGStage4 = GTile<2>::Stage4; // 16-byte chunks per stage

// Fold the finished column block (sums plus column biases) into the rows'
// running (M, S).
__device__ __forceinline__ void block_epilogue(const float *bias, int cw, int hl,
                                               floatx16 (&sum)[2][2], float (&M)[2],
                                               float (&S)[2]) {
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
        float bj[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 b4 =
                *reinterpret_cast<const float4 *>(bias + 64 * cw + 32 * cs + 8 * q + 4 * hl);
            bj[4 * q + 0] = b4.x;
            bj[4 * q + 1] = b4.y;
            bj[4 * q + 2] = b4.z;
            bj[4 * q + 3] = b4.w;
        }
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
            floatx16 u;
            const float Mu = M[rs];
#pragma unroll
            for (int v = 0; v < 16; ++v)
                u[v] = (sum[rs][cs][v] + bj[v]) - Mu;
            const float c = chunk_sum(u);
            fold(u, Mu, c, M[rs], S[rs]);
            pin(M[rs], S[rs]);
        }
    }
}

__device__ __forceinline__ void lse_combine2(float &M, float &S, float Mo, float So) {
    const float Mn = fmaxf(M, Mo);
    S = S * hw_exp2(M - Mn) + So * hw_exp2(Mo - Mn);
    M = Mn;
}

template <int KP>
__global__ __launch_bounds__(64 * kGW) void lse_rows_gemm_kernel(HalfStep h, int blocks_per_split,
                                                                 int nblocks, int nmap,
                                                                 int nrb, int nsplit) {
    __shared__ float4 st0[kGStage4 + kGTail4];
    __shared__ float4 st1[kGStage4 + kGTail4];
    __shared__ float4 st2[kGStage4 + kGTail4];

    int rblk, split;
    if (!gemm_block(nmap, nrb, nsplit, rblk, split))
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rw = wave & 3;
    const int cw = wave >> 2;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int bbeg = split * blocks_per_split;
    const int bend = min(bbeg + blocks_per_split, nblocks);
    const int64_t row0 = (int64_t)rblk * kGBM;

    float M[2] = {0.f, 0.f}, S[2] = {0.f, 0.f};
    gemm_stream<KP, false, 2>(st0, st1, st2, static_cast<const float4 *>(h.row_rec),
                           static_cast<const float4 *>(h.col_rec),
                           static_cast<const float *>(h.col_bias), nullptr, row0, bbeg, bend,
                           wave, lane, [&](const float *bias, const float *, floatx16(&sum)[2][2]) {
                               block_epilogue(bias, cw, hl, sum, M, S);
                           });

    // Each row's pair: the two lane halves (same M by construction), then
    // the two column waves through LDS in order cw = 0, 1.
    float2 *red = reinterpret_cast<float2 *>(st0);
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
        const float So = __shfl_xor(S[rs], 32);
        S[rs] = hl == 0 ? S[rs] + So : So + S[rs];
        if (cw == 1 && hl == 0)
            red[(rw * 2 + rs) * 32 + li] = make_float2(M[rs], S[rs]);
    }
    __syncthreads();
    if (cw == 0 && hl == 0) {
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
            const float2 o = red[(rw * 2 + rs) * 32 + li];
            float Mr = M[rs], Sr = S[rs];
            lse_combine2(Mr, Sr, o.x, o.y);
            const int64_t i = row0 + 64 * rw + 32 * rs + li;
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
}

// One plan-statistics pass: part[split][row] = (sum_j P_ij, COST ?
// sum_j P_ij C_ij : 0) with log2 P_ij = dot + qhat_j + phat_i (fp32, in
// that order) and C_ij = |p_i|^2 + |q_j|^2 - 2 p_i.q_j from the same dot
// product (dot / scale); sums in fp64, the two column waves added in order.
template <int KP, bool COST>
__global__ __launch_bounds__(64 * kGW) void plan_rows_gemm_kernel(
    const float4 *__restrict__ row_rec, const float *__restrict__ row_hat,
    const float *__restrict__ row_nrm, const float4 *__restrict__ col4,
    const float *__restrict__ colb, const float *__restrict__ col_nrm, int64_t rows,
    int64_t rows_pad, int blocks_per_split, int nblocks, int nmap, int nrb, int nsplit,
    float inv_scale, double2 *__restrict__ part) {
    __shared__ float4 st0[kGStage4 + kGTail4];
    __shared__ float4 st1[kGStage4 + kGTail4];
    __shared__ float4 st2[kGStage4 + kGTail4];
    // The rows' phat and |p|^2, read by the block epilogue (kept out of the
    // registers the stage pipeline needs).
    __shared__ float rowv[2][kGBM];

    int rblk, split;
    if (!gemm_block(nmap, nrb, nsplit, rblk, split))
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rw = wave & 3;
    const int cw = wave >> 2;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int bbeg = split * blocks_per_split;
    const int bend = min(bbeg + blocks_per_split, nblocks);
    const int64_t row0 = (int64_t)rblk * kGBM;
    {
        const int r = tid & (kGBM - 1);
        int64_t i = row0 + r;
        i = i < rows ? i : rows - 1;
        if (tid < kGBM)
            rowv[0][r] = row_hat[i];
        else
            rowv[1][r] = COST ? row_nrm[i] : 0.f;
    }
    __syncthreads();
    const float m2 = -2.f * inv_scale;

    double rsum[2] = {0.0, 0.0}, csum[2] = {0.0, 0.0};
    gemm_stream<KP, COST, 2>(
        st0, st1, st2, row_rec, col4, colb, col_nrm, row0, bbeg, bend, wave, lane,
        [&](const float *bias, const float *nrm, floatx16(&sum)[2][2]) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c0 = 64 * cw + 32 * cs + 8 * q + 4 * hl;
                    const float4 b4 = *reinterpret_cast<const float4 *>(bias + c0);
                    float4 n4 = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (COST)
                        n4 = *reinterpret_cast<const float4 *>(nrm + c0);
                    const float bj[4] = {b4.x, b4.y, b4.z, b4.w};
                    const float ny[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
#pragma unroll
                        for (int rs = 0; rs < 2; ++rs) {
                            const int r = 64 * rw + 32 * rs + li;
                            const float dot = sum[rs][cs][4 * q + e];
                            const float pr = hw_exp2((dot + bj[e]) + rowv[0][r]);
                            rsum[rs] += (double)pr;
                            if (COST) {
                                const float cij = fmaf(dot, m2, rowv[1][r] + ny[e]);
                                csum[rs] = fma((double)pr, (double)cij, csum[rs]);
                            }
                        }
                    }
                }
            }
        });

    double2 *red = reinterpret_cast<double2 *>(st0);
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
        const double ro = __shfl_xor(rsum[rs], 32);
        const double co = __shfl_xor(csum[rs], 32);
        rsum[rs] = hl == 0 ? rsum[rs] + ro : ro + rsum[rs];
        csum[rs] = hl == 0 ? csum[rs] + co : co + csum[rs];
        if (cw == 1 && hl == 0)
            red[(rw * 2 + rs) * 32 + li] = make_double2(rsum[rs], csum[rs]);
    }
    __syncthreads();
    if (cw == 0 && hl == 0) {
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
            const double2 o = red[(rw * 2 + rs) * 32 + li];
            const int64_t i = row0 + 64 * rw + 32 * rs + li;
            if (i < rows)
                part[(int64_t)split * rows_pad + i] = make_double2(rsum[rs] + o.x, csum[rs] + o.y);
        }
    }
}

template <int KP>
hipError_t launch_gemm_kp(const HalfStep &h, const GPlan &p, hipStream_t s) {
    hipLaunchKernelGGL((lse_rows_gemm_kernel<KP>), dim3((unsigned)(p.row_map * p.nsplit)),
                       dim3(64 * kGW), 0, s, h, p.blocks_per_split, p.nblocks, (int)p.row_map,
                       (int)p.row_blocks, p.nsplit);
    return hipGetLastError();
}

template <int KP, bool COST>
hipError_t launch_plan_gemm_kp(const GPlan &p, const float4 *rr, const float *row_hat,
                               const float *row_nrm, const float4 *cr, const float *col_hat,
                               const float *col_nrm, int64_t rows, int64_t rows_pad, float inv,
                               double2 *part, hipStream_t s) {
    hipLaunchKernelGGL((plan_rows_gemm_kernel<KP, COST>),
                       dim3((unsigned)(p.row_map * p.nsplit)), dim3(64 * kGW), 0, s, rr, row_hat,
                       row_nrm, cr, col_hat, col_nrm, rows, rows_pad, p.blocks_per_split,
                       p.nblocks, (int)p.row_map, (int)p.row_blocks, p.nsplit, inv, part);
    return hipGetLastError();
}

}  // namespace

size_t half_step_partials_gemm(int64_t rows, int64_t cols_pad) {
    const GPlan p = plan_gemm(rows, cols_pad, kGBM);
    return p.nsplit > 1 ? (size_t)p.nsplit * (size_t)pad_points(rows) : 0;
}

hipError_t launch_half_step_gemm(const HalfStep &h, int kp, hipStream_t s) {
    const GPlan p = plan_gemm(h.rows, h.cols_pad, kGBM);
    hipError_t e;
    switch (kp) {
    case 512: e = launch_gemm_kp<512>(h, p, s); break;
    case 640: e = launch_gemm_kp<640>(h, p, s); break;
    case 768: e = launch_gemm_kp<768>(h, p, s); break;
    case 896: e = launch_gemm_kp<896>(h, p, s); break;
    case 1024: e = launch_gemm_kp<1024>(h, p, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.nsplit <= 1)
        return e;
    return launch_merge_h3(h, p.nsplit, s);
}

int plan_pass_gemm_splits(int64_t rows, int64_t cols_pad) {
    return plan_gemm(rows, cols_pad, kGBM).nsplit;
}

hipError_t launch_plan_pass_gemm(int kp, bool cost, const void *row_rec, const float *row_hat,
                                 const float *row_nrm, const void *col_rec, const float *col_hat,
                                 const float *col_nrm, int64_t rows, int64_t rows_pad,
                                 int64_t cols_pad, double scale, double2 *part, hipStream_t s) {
    const GPlan p = plan_gemm(rows, cols_pad, kGBM);
    const float4 *rr = static_cast<const float4 *>(row_rec);
    const float4 *cr = static_cast<const float4 *>(col_rec);
    const float inv = (float)(1.0 / scale);
#define OTSK_PG(KPV)                                                                           \
    case KPV:                                                                                  \
        return cost ? launch_plan_gemm_kp<KPV, true>(p, rr, row_hat, row_nrm, cr, col_hat,     \
                                                     col_nrm, rows, rows_pad, inv, part, s)    \
                    : launch_plan_gemm_kp<KPV, false>(p, rr, row_hat, row_nrm, cr, col_hat,    \
                                                      col_nrm, rows, rows_pad, inv, part, s);
    switch (kp) {
        OTSK_PG(512)
        OTSK_PG(640)
        OTSK_PG(768)
        OTSK_PG(896)
        OTSK_PG(1024)
    default:
        return hipErrorInvalidValue;
    }
#undef OTSK_PG
}

}  // namespace otsk
