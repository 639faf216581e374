// Log-domain Sinkhorn half-step for feature dimension d >= 32 with the dot
// products on gfx950's f16 matrix cores, as three split products accumulated
// in fp32.
//
// The update is the one of the other half-step kernels ("FlashSinkhorn:
// IO-Aware Entropic Optimal Transport on GPU", Methodik sections 1-2):
// s_ij = (2 log2(e)/eps) p_i.q_j + qhat_j, an online base-2 log-sum-exp over
// j, phat_i = log2 w_i - lse_i. Only the way p_i.q_j is formed differs.
//
// Split products. Each fp32 coordinate v is written as hi + lo with
// hi = f16(v) and lo = f16(v - hi), so v - hi - lo is below 2^-22 |v|. Then
//   P.Q ~ Ph.Qh + Ph.Ql + Pl.Qh          (Pl.Ql, below 2^-22 |P||Q|, dropped)
// with every f16 x f16 product exact. The split loses about 2^-22 |P||Q|;
// the matrix core's aligned sums (below) lose about 2^-21 of the partial sum
// per instruction, comparable to fp32 accumulation over d terms. A tile of
// 32 columns x 32 rows takes 3*KP/16 v_mfma_f32_32x32x16_f16 (32 cycles each)
// instead of KP/2 v_mfma_f32_32x32x2f32 (64 cycles each): 2.7x fewer matrix
// cycles. On gfx950, f16 MFMAs also execute concurrently with vector-ALU
// work from the same SIMD (measured: an FMA stream hides completely under an
// f16 MFMA stream, an exp2 stream mostly), which fp32 MFMAs do not, so the
// exp2/add epilogue of the log-sum-exp largely overlaps the products.
//
// f16 range. The records hold the centred points p = x - c, q = y - c (c the
// mean of the two cloud means; the cost does not change, and |p| |q| stays
// near the size of the costs). To keep hi and lo inside f16's range, the
// column side stores (2 log2(e)/eps) q 2^-e and the row side p 2^e with one
// power of two e per direction, chosen so that both sides' largest magnitudes
// meet near T^(1/2), T = (2 log2(e)/eps) max|p| max|q|; the product is
// unchanged. With e
// rounded to an integer one side's largest magnitude is at most (2T)^(1/2),
// which stays below f16's largest finite value 65504 when T < 2^30 (near
// 2^32 the hi parts become inf; fp32 scores would carry no fractional bits
// there either).
//
// The column bias qhat_j and the row's running maximum M enter through one
// fp32 MFMA at the end of the chain (k-slot 0: bias_j x 1, k-slot 1:
// 1 x -M_i), so they keep full fp32 precision.
//
// Layout. Column records: 2*KP halves (hi then lo) in 16-byte chunks, chunk q
// of point j stored at position q ^ (j & SW), so the 16-byte operand reads of
// consecutive points fall in distinct LDS banks. Row records: hi then lo,
// unswizzled (read once per workgroup). Biases and norms are fp32 arrays.
// Workgroups of 8 waves own 256 rows and stream 128-column tiles (64 above
// KP = 128, see tile_cols) through double-buffered LDS with gfx950's direct
// global->LDS loads; the running maximum is shared lazily by the two lane
// halves of a row and moved only when a chunk sum leaves [2^-64, 2^16] (the
// epilogue in mfma_common.h).
#include "mfma_common.h"

#include <math.h>
#include <type_traits>

namespace otsk {

namespace {

using namespace mfma;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;
// Columns per LDS tile: 128 up to KP = 128; 64 above, so that the two tile
// buffers (2 * TC * KP * 4 bytes) still fit the LDS with one workgroup per CU.
__host__ __device__ constexpr int tile_cols(int kp) { return kp <= 128 ? 128 : 64; }
constexpr int kTargetBlocks = 1024;

template <int KP>
__global__ __launch_bounds__(kThreads) void lse_rows_h3_kernel(HalfStep h, int tiles_per_split,
                                                               int ntiles, int nrb, int nsplit) {
    int rblk, split;
    xcd_block(nrb, nsplit, rblk, split);
    constexpr int RC = KP / 4;
    constexpr int TC = tile_cols(KP);
    constexpr int SUB = TC / 32;
    constexpr int BS = 2 * TC;
    constexpr int TILE16 = TC * RC;
    static_assert(KP % 32 == 0, "records are whole groups of 8 chunks");
    static_assert(TILE16 % 64 == 0, "tiles are whole 64-lane chunks");
    static_assert(SUB <= kWaves, "one wave copies each subtile's biases");
    __shared__ float4 lrec[2][TILE16];
    __shared__ float lbias[2][BS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const float4 *col4 = static_cast<const float4 *>(h.col_rec);
    const float *colb = static_cast<const float *>(h.col_bias);

    for (int k = tid; k < 2 * BS; k += kThreads) {
        const int e = k % BS;
        if ((e / 32) & 1)
            lbias[k / BS][e] = 1.f;
    }
    issue_tile<TILE16, kWaves, SUB>(col4, colb, tbeg, lrec[0], lbias[0], wave, lane);
    // Stationary B operands: this lane's k-halves of its row's hi and lo parts.
    const int64_t i = (int64_t)rblk * kRowsPerBlock + wave * 32 + li;
    const int64_t ic = i < h.rows ? i : h.rows - 1;
    half8 bh[KP / 16], bl[KP / 16];
    {
        const float4 *rr = static_cast<const float4 *>(h.row_rec) + ic * RC;
#pragma unroll
        for (int c = 0; c < KP / 16; ++c) {
            bh[c] = as_half8(rr[2 * c + hl]);
            bl[c] = as_half8(rr[KP / 8 + 2 * c + hl]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    float M = 0.f;
    float S = 0.f;
    float Mu_prev = M;
    floatx16 acc_prev = score_h3<KP>(lrec[0], lbias[0], 0, lane, li, hl, bh, bl, Mu_prev);
    // One column tile from LDS buffer b (a compile-time constant, so every
    // LDS operand address is a per-lane register plus an immediate offset).
    auto tile = [&](int t, auto bc) {
        constexpr int b = decltype(bc)::value;
        if (t + 1 < tend)
            issue_tile<TILE16, kWaves, SUB>(col4, colb, t + 1, lrec[b ^ 1], lbias[b ^ 1], wave,
                                             lane);
#pragma unroll
        for (int sub = 1; sub < SUB; ++sub) {
            const float Mu_cur = M;
            const floatx16 acc_cur = score_h3<KP>(lrec[b], lbias[b], sub, lane, li, hl, bh, bl,
                                                  Mu_cur);
            const float c = chunk_sum(acc_prev);
            fold(acc_prev, Mu_prev, c, M, S);
            pin(M, S);
            acc_prev = acc_cur;
            Mu_prev = Mu_cur;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // First subtile of the next tile (on the last tile: the idle buffer,
        // never folded).
        const float Mu_cur = M;
        const floatx16 acc_cur =
            score_h3<KP>(lrec[b ^ 1], lbias[b ^ 1], 0, lane, li, hl, bh, bl, Mu_cur);
        const float c = chunk_sum(acc_prev);
        fold(acc_prev, Mu_prev, c, M, S);
        pin(M, S);
        acc_prev = acc_cur;
        Mu_prev = Mu_cur;
    };
    for (int t = tbeg; t < tend; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < tend)
            tile(t + 1, std::integral_constant<int, 1>{});
    }

    const float So = __shfl_xor(S, 32);
    const float Sm = hl == 0 ? S + So : So + S;
    if (hl == 0 && i < h.rows) {
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

// Combine the per-split (M, S) pairs of each row in split order.
__global__ __launch_bounds__(256) void lse_merge_h3_kernel(HalfStep h, int nsplit) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= h.rows)
        return;
    double M = h.partials[i].m;
    for (int s = 1; s < nsplit; ++s)
        M = fmax(M, h.partials[(int64_t)s * h.rows_pad + i].m);
    float S = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const Partial p = h.partials[(int64_t)s * h.rows_pad + i];
        S = fmaf(p.s, hw_exp2((float)(p.m - M)), S);
    }
    const float lse = (float)M + hw_log2(S);
    const float hat = log2f(h.row_w[i]) - lse;
    static_cast<float *>(h.row_bias)[i] = hat;
    h.pot_out[i] = fmaf((float)h.eps_ln2, hat, h.row_nrm[i]);
}

// ---------------------------------------------------------------------------
// Records.
// ---------------------------------------------------------------------------

// Centre of the two clouds, c = (mean(x) + mean(y)) / 2 (unweighted). The
// cost |x_i - y_j|^2 does not change when both clouds move by the same
// vector; records of x - c and y - c keep |p| |q| near the size of the costs
// themselves, so the expanded form |p|^2 + |q|^2 - 2 p.q does not cancel
// away the precision of the dot product when the clouds sit far from the
// origin. Per block: fp64 column sums over a strided set of rows of one side
// (blockIdx.y), 256 / d threads per coordinate.
__global__ __launch_bounds__(256) void center_partial_kernel(const float *__restrict__ x,
                                                             int64_t n,
                                                             const float *__restrict__ y,
                                                             int64_t m, int d,
                                                             double *__restrict__ part) {
    __shared__ double red[256];
    const float *p = blockIdx.y ? y : x;
    const int64_t cnt = blockIdx.y ? m : n;
    const int tid = threadIdx.x;
    if (d > 256) {
        // One row per block step; thread tid sums coordinates tid, tid + 256.
        for (int k = tid; k < d; k += 256) {
            double sum = 0.0;
            for (int64_t r = blockIdx.x; r < cnt; r += gridDim.x)
                sum += (double)p[r * d + k];
            part[((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * d + k] = sum;
        }
        return;
    }
    const int rows = 256 / d;
    const int k = tid % d, r0 = tid / d;
    double sum = 0.0;
    if (r0 < rows)
        for (int64_t r = (int64_t)blockIdx.x * rows + r0; r < cnt; r += (int64_t)gridDim.x * rows)
            sum += (double)p[r * d + k];
    red[tid] = sum;
    __syncthreads();
    if (tid < d) {
        double t = 0.0;
        for (int q = 0; q < rows; ++q)
            t += red[q * d + tid];
        part[((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * d + tid] = t;
    }
}

__global__ __launch_bounds__(256) void center_final_kernel(const double *__restrict__ part, int nb,
                                                           int d, int64_t n, int64_t m,
                                                           float *__restrict__ center) {
    for (int k = threadIdx.x; k < d; k += blockDim.x) {
        double sx = 0.0, sy = 0.0;
        for (int b = 0; b < nb; ++b) {
            sx += part[(int64_t)b * d + k];
            sy += part[((int64_t)nb + b) * d + k];
        }
        center[k] = (float)(0.5 * (sx / (double)n + sy / (double)m));
    }
}

// Largest |coordinate| of x - c (blockIdx.y == 0) or y - c (1), one value per
// block.
__global__ __launch_bounds__(256) void maxabs_kernel(const float *__restrict__ x, int64_t nx,
                                                     const float *__restrict__ y, int64_t ny,
                                                     const float *__restrict__ center, int d,
                                                     float *__restrict__ part) {
    __shared__ float red[4];
    const float *p = blockIdx.y ? y : x;
    const int64_t cnt = blockIdx.y ? ny : nx;
    float mx = 0.f;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < cnt;
         e += (int64_t)gridDim.x * 256)
        mx = fmaxf(mx, fabsf((float)((double)p[e] - (double)center[e % d])));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0)
        part[blockIdx.y * gridDim.x + blockIdx.x] =
            fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(64) void maxabs_final_kernel(const float *__restrict__ part, int nb,
                                                          float *__restrict__ out) {
    const int side = threadIdx.x >> 5;  // lanes 0-31: x, 32-63: y
    float mx = 0.f;
    for (int k = threadIdx.x & 31; k < nb; k += 32)
        mx = fmaxf(mx, part[side * nb + k]);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((threadIdx.x & 31) == 0)
        out[side] = mx;
}

// Power of two e with (scale * b_own) 2^-e ~ b_other 2^e; 0 for empty data.
__device__ __forceinline__ int balance_exp(double scale, double b_own, double b_other) {
    if (!(b_own > 0.0) || !(b_other > 0.0))
        return 0;
    double r = 0.5 * log2(scale * b_own / b_other);
    r = r < -100.0 ? -100.0 : (r > 100.0 ? 100.0 : r);
    return (int)rint(r);
}

// hi = f16(v), lo = f16(v - hi), each rounded once to nearest from an fp32
// value. The empty asm statements keep the compiler from fusing the product,
// the difference and the conversion into mixed-precision FMAs (v_fma_mix*),
// whose f16 results lose the subnormal lo parts of small coordinates.
__device__ __forceinline__ _Float16 split_hi(float v, _Float16 &lo) {
    asm volatile("" : "+v"(v));
    const _Float16 hi = (_Float16)v;
    float r = v - (float)hi;
    asm volatile("" : "+v"(r));
    lo = (_Float16)r;
    return hi;
}

__device__ __forceinline__ float4 pack8(const _Float16 (&v)[8]) {
    half8 h;
#pragma unroll
    for (int r = 0; r < 8; ++r)
        h[r] = v[r];
    return __builtin_bit_cast(float4, h);
}

// One side's records at one eps, of the centred points p = x - c: column
// record (scaled, split, swizzled; staged above kStagedRecordKP), row record
// (split; staged likewise), |p|^2 and the bias (zero, hat of pot, or
// padding).
__global__ __launch_bounds__(256) void prep_h3_kernel(
    const float *__restrict__ pts, const float *__restrict__ pot, const float *__restrict__ center,
    int64_t count, int64_t padded, int d, int kp, double scale, double hat_scale, int bias_mode,
    const float *__restrict__ maxabs, int own, float4 *__restrict__ colrec,
    float4 *__restrict__ rowrec, float *__restrict__ nrm_out, float *__restrict__ bias) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= padded)
        return;
    const double bo = maxabs[own], bt = maxabs[1 - own];
    const double cf = ldexp(scale, -balance_exp(scale, bo, bt));
    const double rf = ldexp(1.0, balance_exp(scale, bt, bo));
    const int rc = kp / 4;
    const int hc = kp / 8;
    const int sw = (int)(i & swizzle_mask(rc));
    const bool real = i < count;
    double nrm = 0.0;
    for (int q = 0; q < hc; ++q) {
        _Float16 ch[8], cl[8], rh[8], rl[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int k = 8 * q + r;
            const double v = (real && k < d) ? (double)pts[i * d + k] - (double)center[k] : 0.0;
            nrm = fma(v, v, nrm);
            ch[r] = split_hi((float)(v * cf), cl[r]);
            rh[r] = split_hi((float)(v * rf), rl[r]);
        }
        if (kp > kStagedRecordKP) {
            const int st = (q >> 2) * 8 + (q & 3);
            colrec[i * rc + st] = pack8(ch);
            colrec[i * rc + st + 4] = pack8(cl);
            rowrec[i * rc + st] = pack8(rh);
            rowrec[i * rc + st + 4] = pack8(rl);
        } else {
            colrec[i * rc + (q ^ sw)] = pack8(ch);
            colrec[i * rc + ((hc + q) ^ sw)] = pack8(cl);
            rowrec[i * rc + q] = pack8(rh);
            rowrec[i * rc + hc + q] = pack8(rl);
        }
    }
    nrm_out[i] = (float)nrm;
    float bv = kPadBias;
    if (real)
        bv = bias_mode == kBiasHat ? (float)(((double)pot[i] - nrm) * hat_scale)
                                   : (bias_mode == kBiasRaw ? pot[i] : 0.f);
    bias[i] = bv;
}

// ---------------------------------------------------------------------------
// Plan statistics on the same records: one pass over the columns for each row
// i gives r_i = sum_j P_ij and (COST) c_i = sum_j P_ij C_ij, with
// log2 P_ij = (2 log2(e)/eps) p_i.q_j + qhat_j + phat_i from the split-f16
// chain plus one fp32 MFMA (k-slot 0: qhat_j x 1, k-slot 1: 1 x phat_i), and
// C_ij = |p_i|^2 + |q_j|^2 - 2 p_i.q_j from the chain's dot product before the
// bias. Sums are fp32 within a column tile and fp64 across tiles; the
// two lane halves (disjoint columns of one row) are added at the end.
// ---------------------------------------------------------------------------
template <int KP, bool COST>
__global__ __launch_bounds__(kThreads) void plan_rows_h3_kernel(
    const float4 *__restrict__ row_rec, const float *__restrict__ row_hat,
    const float *__restrict__ row_nrm, const float4 *__restrict__ col4,
    const float *__restrict__ colb, const float *__restrict__ col_nrm, int64_t rows,
    int64_t rows_pad, int tiles_per_split, int ntiles, float inv_scale,
    double2 *__restrict__ part) {
    constexpr int RC = KP / 4;
    constexpr int TC = tile_cols(KP);
    constexpr int SUB = TC / 32;
    constexpr int BS = 2 * TC;
    constexpr int TILE16 = TC * RC;
    static_assert(SUB <= kWaves, "one wave copies each subtile's biases");
    __shared__ float4 lrec[2][TILE16];
    __shared__ float lbias[2][BS];
    __shared__ __attribute__((aligned(16))) float lnrm[2][TC];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);

    for (int k = tid; k < 2 * BS; k += kThreads) {
        const int e = k % BS;
        if ((e / 32) & 1)
            lbias[k / BS][e] = 1.f;
    }
    // Column norms of a tile: waves 0 and 1, one dword per lane.
    auto issue_norms = [&](int t, float *dst) {
        if (COST && wave < TC / 64)
            __builtin_amdgcn_global_load_lds(col_nrm + (int64_t)t * TC + wave * 64 + lane,
                                             (lds_void *)(dst + wave * 64), 4, 0, 0);
    };
    issue_tile<TILE16, kWaves, SUB>(col4, colb, tbeg, lrec[0], lbias[0], wave, lane);
    issue_norms(tbeg, lnrm[0]);
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
            issue_tile<TILE16, kWaves, SUB>(col4, colb, t + 1, lrec[b ^ 1], lbias[b ^ 1], wave,
                                             lane);
            issue_norms(t + 1, lnrm[b ^ 1]);
        }
        float rs = 0.f, cs = 0.f;
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
            constexpr int SW = swizzle_mask(RC);
            const int j = sub * 32 + li;
            const float4 *ap = lrec[b] + j * RC;
            const int sw = j & SW;
            const floatx16 dot = split_dot<KP>(ap, sw, hl, bh, bl);
            const float a0 = lbias[b][sub * 64 + lane];
            const float b0 = hl ? -Mu : 1.f;
            const floatx16 u = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, dot, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 ny = make_float4(0.f, 0.f, 0.f, 0.f);
                if (COST)
                    ny = *reinterpret_cast<const float4 *>(&lnrm[b][sub * 32 + 8 * q + 4 * hl]);
                const float nyv[4] = {ny.x, ny.y, ny.z, ny.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pr = hw_exp2(u[4 * q + r]);
                    rs += pr;
                    if (COST) {
                        const float cij = fmaf(dot[4 * q + r], m2, nx + nyv[r]);
                        cs = fmaf(pr, cij, cs);
                    }
                }
            }
        }
        rsum += (double)rs;
        csum += (double)cs;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    const double ro = __shfl_xor(rsum, 32);
    const double co = __shfl_xor(csum, 32);
    if (hl == 0 && i < rows)
        part[(int64_t)split * rows_pad + i] = make_double2(rsum + ro, csum + co);
}

struct H3Plan {
    int ntiles;
    int tiles_per_split;
    int nsplit;
    int64_t row_blocks;
};

H3Plan plan_h3(int64_t rows, int64_t cols_pad, int kp) {
    H3Plan p;
    p.ntiles = (int)(cols_pad / tile_cols(kp));
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
hipError_t launch_h3_kp(const HalfStep &h, const H3Plan &p, hipStream_t s) {
    dim3 grid((unsigned)(p.row_blocks * p.nsplit));
    hipLaunchKernelGGL((lse_rows_h3_kernel<KP>), grid, dim3(kThreads), 0, s, h, p.tiles_per_split,
                       p.ntiles, (int)p.row_blocks, p.nsplit);
    return hipGetLastError();
}

constexpr int kMaxabsBlocks = 256;
constexpr int kCenterBlocks = 256;

}  // namespace

// Coordinates per record: 32k up to 192 (the 32x32 kernels); above, the
// 16x16-tile kernels' sizes 224, 256, 320, 384, 448; above 448 the sizes of
// the kernels tiled like a matrix product, 512, 640, 768, 896, 1024 (whole
// 32-coordinate stages; at 512 the 16x16 kernel spills and measured 22.6 ms
// per 65536^2 half-step, the tiled one 13.3 ms).
int h3_kp(int d) {
    if (d <= 256)
        return (d + 31) / 32 * 32;
    return d <= 448 ? (d + 63) / 64 * 64 : (d + 127) / 128 * 128;
}

size_t h3_maxabs_floats() { return 2 * kMaxabsBlocks + 2; }

size_t h3_center_scratch_bytes(int d) {
    return (size_t)2 * kCenterBlocks * d * sizeof(double) + (size_t)d * sizeof(float);
}

hipError_t launch_center_maxabs(const float *x, int64_t n, const float *y, int64_t m, int d,
                                void *center_scratch, float *scratch, hipStream_t s) {
    if (d < 1 || d > 1024)
        return hipErrorInvalidValue;
    double *part = static_cast<double *>(center_scratch);
    float *center = reinterpret_cast<float *>(part + (size_t)2 * kCenterBlocks * d);
    hipLaunchKernelGGL(center_partial_kernel, dim3(kCenterBlocks, 2), dim3(256), 0, s, x, n, y, m,
                       d, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(center_final_kernel, dim3(1), dim3(256), 0, s, part, kCenterBlocks, d, n, m,
                       center);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(maxabs_kernel, dim3(kMaxabsBlocks, 2), dim3(256), 0, s, x, n * d, y, m * d,
                       center, d, scratch + 2);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(maxabs_final_kernel, dim3(1), dim3(64), 0, s, scratch + 2, kMaxabsBlocks,
                       scratch);
    return hipGetLastError();
}

hipError_t launch_prep_h3(const float *pts, const float *pot, int64_t count, int64_t padded, int d,
                          int kp, double scale, double hat_scale, int bias_mode,
                          const float *maxabs, const void *center_scratch, int own, void *colrec,
                          void *rowrec, float *nrm, float *bias, hipStream_t s) {
    const unsigned blocks = (unsigned)((padded + 255) / 256);
    const float *center = reinterpret_cast<const float *>(
        static_cast<const double *>(center_scratch) + (size_t)2 * kCenterBlocks * d);
    hipLaunchKernelGGL(prep_h3_kernel, dim3(blocks), dim3(256), 0, s, pts, pot, center, count,
                       padded, d, kp, scale, hat_scale, bias_mode, maxabs, own,
                       static_cast<float4 *>(colrec), static_cast<float4 *>(rowrec), nrm, bias);
    return hipGetLastError();
}

int plan_pass_h3_splits(int64_t rows, int64_t cols_pad, int kp) {
    if (kp > 448)
        return plan_pass_gemm_splits(rows, cols_pad);
    if (kp > 192)
        return plan_pass_wide_splits(rows, cols_pad, kp);
    return plan_h3(rows, cols_pad, kp).nsplit;
}

hipError_t launch_plan_pass_h3(int kp, bool cost, const void *row_rec, const float *row_hat,
                               const float *row_nrm, const void *col_rec, const float *col_hat,
                               const float *col_nrm, int64_t rows, int64_t rows_pad,
                               int64_t cols_pad, double scale, double2 *part, hipStream_t s) {
    if (kp > 448)
        return launch_plan_pass_gemm(kp, cost, row_rec, row_hat, row_nrm, col_rec, col_hat,
                                     col_nrm, rows, rows_pad, cols_pad, scale, part, s);
    if (kp > 192)
        return launch_plan_pass_wide(kp, cost, row_rec, row_hat, row_nrm, col_rec, col_hat,
                                     col_nrm, rows, rows_pad, cols_pad, scale, part, s);
    const H3Plan p = plan_h3(rows, cols_pad, kp);
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    const float4 *rr = static_cast<const float4 *>(row_rec);
    const float4 *cr = static_cast<const float4 *>(col_rec);
    const float inv = (float)(1.0 / scale);
#define OTSK_PR(KPV)                                                                           \
    case KPV:                                                                                  \
        if (cost)                                                                              \
            hipLaunchKernelGGL((plan_rows_h3_kernel<KPV, true>), grid, dim3(kThreads), 0, s,  \
                               rr, row_hat, row_nrm, cr, col_hat, col_nrm, rows, rows_pad,     \
                               p.tiles_per_split, p.ntiles, inv, part);                        \
        else                                                                                   \
            hipLaunchKernelGGL((plan_rows_h3_kernel<KPV, false>), grid, dim3(kThreads), 0, s, \
                               rr, row_hat, row_nrm, cr, col_hat, col_nrm, rows, rows_pad,     \
                               p.tiles_per_split, p.ntiles, inv, part);                        \
        break;
    switch (kp) {
        OTSK_PR(32)
        OTSK_PR(64)
        OTSK_PR(96)
        OTSK_PR(128)
        OTSK_PR(160)
        OTSK_PR(192)
    default:
        return hipErrorInvalidValue;
    }
#undef OTSK_PR
    return hipGetLastError();
}

size_t half_step_partials_h3(int64_t rows, int64_t cols_pad, int kp) {
    if (kp > 448)
        return half_step_partials_gemm(rows, cols_pad);
    if (kp > 192)
        return half_step_partials_wide(rows, cols_pad, kp);
    const H3Plan p = plan_h3(rows, cols_pad, kp);
    return p.nsplit > 1 ? (size_t)p.nsplit * (size_t)pad_points(rows) : 0;
}

hipError_t launch_merge_h3(const HalfStep &h, int nsplit, hipStream_t s) {
    hipLaunchKernelGGL(lse_merge_h3_kernel, dim3((unsigned)((h.rows + 255) / 256)), dim3(256), 0,
                       s, h, nsplit);
    return hipGetLastError();
}

hipError_t launch_half_step_h3(const HalfStep &h, int kp, hipStream_t s) {
    if (kp > 448)
        return launch_half_step_gemm(h, kp, s);
    if (kp > 192)
        return launch_half_step_wide(h, kp, s);
    const H3Plan p = plan_h3(h.rows, h.cols_pad, kp);
    hipError_t e;
    switch (kp) {
    case 32: e = launch_h3_kp<32>(h, p, s); break;
    case 64: e = launch_h3_kp<64>(h, p, s); break;
    case 96: e = launch_h3_kp<96>(h, p, s); break;
    case 128: e = launch_h3_kp<128>(h, p, s); break;
    case 160: e = launch_h3_kp<160>(h, p, s); break;
    case 192: e = launch_h3_kp<192>(h, p, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.nsplit <= 1)
        return e;
    return launch_merge_h3(h, p.nsplit, s);
}

}  // namespace otsk
