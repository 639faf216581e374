// Log-domain Sinkhorn half-step on the vector ALUs of gfx950 (feature
// dimension d < 32), plus the record preparation and the split merge.
//
// Method: "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU",
// Methodik section 1 (the update as a row-wise log-sum-exp of a biased
// dot-product score matrix, Proposition 1) and section 2 (tiles streamed
// through on-chip memory, online max / sum-exp statistics, whole update fused
// in one pass, row-stationary traversal).
//
// For a row point p_i (weights w_i) and column points q_j with bias
// qhat_j = (pot_j - |q_j|^2) * log2(e)/eps, in base 2:
//
//   s_ij   = (2*log2(e)/eps) * p_i . q_j + qhat_j
//   lse_i  = log2 sum_j 2^(s_ij)
//   phat_i = log2(w_i) - lse_i                 (the row side's new bias)
//   pot_i  = |p_i|^2 + eps*ln(2) * phat_i       (the potential itself)
//
// which is pot_i = eps*log w_i - eps*LSE_j((pot_j - C_ij)/eps) with
// C_ij = |p_i|^2 + |q_j|^2 - 2 p_i.q_j; the |p_i|^2 term leaves the sum.
//
// Precision: the score cancels terms of size (2/eps)|p||q| down to the few
// units that matter, so in fp32 its rounding error grows like 1/eps (about
// 3e-5 log2 units per term at eps = 0.01 with unit-size clouds). The score
// is therefore formed in fp64 -- d fp64 FMAs plus one fp64 add, which issue
// at the same rate as their fp32 forms on gfx950 -- relative to the row's
// running maximum, then rounded once to fp32 for v_exp_f32 and the fp32
// sums. The biases (the iteration state) are kept in fp64.
//
// Mapping onto the hardware:
//  * each lane owns R rows (their scaled fp64 coordinates, running max M and
//    running sum S live in VGPRs for the whole column sweep);
//  * a 256-lane workgroup streams column records through a double-buffered
//    LDS tile (coalesced 16-byte loads, one barrier per tile); every lane of a
//    wave reads the same record, so LDS reads are conflict-free broadcasts;
//  * per chunk of T columns: the T shifted scores u = s - M per row, their
//    maximum (v_max3_f32), and only when some lane's chunk maximum exceeds
//    kLazy a wave-uniform rescale branch (M moves up, S is scaled down, the
//    chunk is recomputed against the new M); every term therefore stays below
//    2^kLazy, the sum cannot overflow, and the common path is
//    fp64 FMAs + cvt + exp2 + add;
//  * blocked summation: each chunk is summed locally and then added to S;
//  * when the columns are split over several workgroups (grid.y > 1) each
//    writes its (M, S) pair and a merge kernel combines them in split order.
// No atomics: the result is bitwise reproducible.
#include "ot_internal.h"

#include <math.h>

namespace otsk {

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// Largest shifted score a term may have before the row's maximum is moved.
constexpr float kLazy = 8.0f;

// --------------------------------------------------------------------------
// Record preparation: copy coordinates (zero padded to kp), write the bias.
// --------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void prep_side_kernel(const float *__restrict__ pts,
                                                        const float *__restrict__ pot, int64_t count,
                                                        int64_t padded, int d, int kp, int rs,
                                                        double hat_scale, int bias_mode, E *rec,
                                                        E *bias, int bias_stride, int bias_off) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= padded)
        return;
    E *r = rec + i * rs;
    if (i < count) {
        double nrm = 0.0;
        for (int k = 0; k < kp; ++k) {
            const float v = k < d ? pts[i * d + k] : 0.f;
            r[k] = (E)v;
            nrm = fma((double)v, (double)v, nrm);
        }
        double bv = 0.0;
        if (bias_mode == kBiasHat)
            bv = ((double)pot[i] - nrm) * hat_scale;
        else if (bias_mode == kBiasRaw)
            bv = pot[i];
        for (int k = kp; k < rs; ++k)
            r[k] = (E)0;
        bias[i * bias_stride + bias_off] = (E)bv;
    } else {
        for (int k = 0; k < rs; ++k)
            r[k] = (E)0;
        bias[i * bias_stride + bias_off] = (E)kPadBias;
    }
}

hipError_t launch_prep_side(const float *pts, const float *pot, int64_t count, int64_t padded,
                            const Layout &L, double hat_scale, int bias_mode, void *rec,
                            void *bias, int bias_stride, int bias_off, hipStream_t s) {
    const unsigned blocks = (unsigned)((padded + 255) / 256);
    if (L.f64)
        hipLaunchKernelGGL(prep_side_kernel<double>, dim3(blocks), dim3(256), 0, s, pts, pot,
                           count, padded, L.d, L.kp, L.rs, hat_scale, bias_mode,
                           static_cast<double *>(rec), static_cast<double *>(bias), bias_stride,
                           bias_off);
    else
        hipLaunchKernelGGL(prep_side_kernel<float>, dim3(blocks), dim3(256), 0, s, pts, pot,
                           count, padded, L.d, L.kp, L.rs, hat_scale, bias_mode,
                           static_cast<float *>(rec), static_cast<float *>(bias), bias_stride,
                           bias_off);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Epilogue shared by the one-pass kernel and the merge: from the final
// (M, S) of row i write its fp64 bias slot and its potential.
// --------------------------------------------------------------------------
__device__ __forceinline__ void finish_row_f64(const HalfStep &h, int64_t i, double M, float S,
                                               double nrm) {
    const double lse = M + (double)hw_log2(S);
    const double hat = log2((double)h.row_w[i]) - lse;
    static_cast<double *>(h.row_bias)[i * h.bias_stride + h.bias_off] = hat;
    h.pot_out[i] = (float)fma(h.eps_ln2, hat, nrm);
}

// --------------------------------------------------------------------------
// The tiled half-step. KP coordinates per record (RS = KP + 1 doubles),
// R rows per lane, TJ columns per LDS tile.
// --------------------------------------------------------------------------
template <int KP, int R, int TJ>
__global__ __launch_bounds__(256) void lse_rows_valu_kernel(HalfStep h, int tiles_per_split,
                                                            int ntiles, int nrb, int nsplit) {
    int rblk, split;
    xcd_block(nrb, nsplit, rblk, split);
    constexpr int RS = KP + 1;
    static_assert(RS % 4 == 0, "record stride must be a multiple of 4 elements");
    constexpr int RS2 = RS / 2;          // 16-byte words per record
    constexpr int TILE2 = TJ * RS2;
    constexpr int PF = (TILE2 + 255) / 256;
    // Columns per chunk: the chunk's records are held in VGPRs, so longer
    // records get shorter chunks.
    constexpr int T = RS <= 4 ? 8 : (RS <= 8 ? 4 : (RS <= 16 ? 2 : 1));
    static_assert(TJ % T == 0, "tile must hold whole chunks");
    __shared__ double2 lds[2][TILE2];

    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)rblk * (256 * R);
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const double *row_rec = static_cast<const double *>(h.row_rec);
    const double2 *col2 = static_cast<const double2 *>(h.col_rec);

    double xs[R][KP];
    double nrm[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t i = row0 + tid + r * 256;
        i = i < h.rows ? i : h.rows - 1;
        const double *p = row_rec + i * RS;
        double q = 0.0;
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const double v = p[k];
            q = fma(v, v, q);
            xs[r][k] = v * h.scale;
        }
        nrm[r] = q;
    }

#pragma unroll
    for (int q = 0; q < PF; ++q) {
        const int idx = tid + q * 256;
        if (TILE2 % 256 == 0 || idx < TILE2)
            lds[0][idx] = col2[(int64_t)tbeg * TILE2 + idx];
    }
    __syncthreads();

    // Start every row's maximum at its score against the split's first
    // column, so M is finite from the start.
    double M[R];
    float S[R];
    {
        const double *rec = reinterpret_cast<const double *>(lds[0]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            double acc = rec[KP];
#pragma unroll
            for (int k = KP - 1; k >= 0; --k)
                acc = fma(xs[r][k], rec[k], acc);
            M[r] = acc;
            S[r] = 0.f;
        }
    }

    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        // Next tile (the last iteration reloads its own tile; the copy into
        // the idle buffer is then unused). Unconditional, so the prefetch
        // stays in registers.
        const int tn = t + 1 < tend ? t + 1 : t;
        double2 pre[PF];
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int idx = min(tid + q * 256, TILE2 - 1);
            pre[q] = col2[(int64_t)tn * TILE2 + idx];
        }
        const double *tile = reinterpret_cast<const double *>(lds[b]);
        for (int c0 = 0; c0 < TJ; c0 += T) {
            float u[R][T];
#pragma unroll
            for (int v = 0; v < T; ++v) {
                const double *rec = tile + (c0 + v) * RS;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    double acc = rec[KP] - M[r];
#pragma unroll
                    for (int k = KP - 1; k >= 0; --k)
                        acc = fma(xs[r][k], rec[k], acc);
                    u[r][v] = (float)acc;
                }
            }
            float mx[R];
            bool need = false;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float m = u[r][0];
#pragma unroll
                for (int v = 1; v < T; ++v)
                    m = fmaxf(m, u[r][v]);
                mx[r] = m;
                need |= m > kLazy;
            }
            if (__builtin_amdgcn_ballot_w64(need)) {
                // Rare: move the maximum up and recompute this chunk in fp64
                // against it, so no precision is lost on the rescaled terms.
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (mx[r] > kLazy) {
                        const double Mn = M[r] + (double)mx[r];
                        S[r] *= hw_exp2((float)(M[r] - Mn));
                        M[r] = Mn;
                    }
                }
#pragma unroll
                for (int v = 0; v < T; ++v) {
                    const double *rec = tile + (c0 + v) * RS;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        double acc = rec[KP] - M[r];
#pragma unroll
                        for (int k = KP - 1; k >= 0; --k)
                            acc = fma(xs[r][k], rec[k], acc);
                        u[r][v] = (float)acc;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float c = 0.f;
#pragma unroll
                for (int v = 0; v < T; ++v)
                    c += hw_exp2(u[r][v]);
                S[r] += c;
            }
        }
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int idx = tid + q * 256;
            if (TILE2 % 256 == 0 || idx < TILE2)
                lds[b ^ 1][idx] = pre[q];
        }
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row0 + tid + r * 256;
        if (i < h.rows) {
            if (nsplit == 1)
                finish_row_f64(h, i, M[r], S[r], nrm[r]);
            else
                h.partials[(int64_t)split * h.rows_pad + i] = Partial{M[r], S[r], 0.f};
        }
    }
}

// Combine the per-split (M, S) pairs of each row: G lanes per row (G = 32
// when there are at most 32 splits, else 64), lane s takes splits s, s + G,
// ...; the maximum and the rescaled sum are reduced across the G lanes in a
// fixed butterfly order (bitwise reproducible, and the same for both G: the
// extra butterfly step of G = 64 would only add zeros). A thread-per-row loop
// over the splits is bound by the latency of its dependent loads (25 us for
// 64 splits of 16384 rows); this takes one round of loads, and the first
// split's pair stays in registers between the two reductions.
template <int G>
__device__ __forceinline__ double group_max(double v) {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1)
        v = fmax(v, __shfl_xor(v, o));
    return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

template <int G>
__global__ __launch_bounds__(256) void lse_merge_kernel(HalfStep h, int nsplit, int kp, int rs) {
    constexpr int kRowsPerWave = 64 / G;
    const int lane = threadIdx.x & 63;
    const int gl = lane % G;
    const int64_t i =
        ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowsPerWave + lane / G;
    // Rows past the end take part in the shuffles with a valid row's data and
    // write nothing.
    const int64_t ir = i < h.rows ? i : h.rows - 1;
    const bool has = gl < nsplit;
    Partial first = {-INFINITY, 0.f, 0.f};
    if (has)
        first = h.partials[(int64_t)gl * h.rows_pad + ir];
    double M = first.m;
    for (int s = gl + G; s < nsplit; s += G)
        M = fmax(M, h.partials[(int64_t)s * h.rows_pad + ir].m);
    M = group_max<G>(M);
    float S = has ? first.s * hw_exp2((float)(first.m - M)) : 0.f;
    for (int s = gl + G; s < nsplit; s += G) {
        const Partial p = h.partials[(int64_t)s * h.rows_pad + ir];
        S = fmaf(p.s, hw_exp2((float)(p.m - M)), S);
    }
    S = group_sum<G>(S);
    if (gl == 0 && i < h.rows) {
        const double *p = static_cast<const double *>(h.row_rec) + i * rs;
        double q = 0.0;
        for (int k = 0; k < kp; ++k)
            q = fma(p[k], p[k], q);
        finish_row_f64(h, i, M, S, q);
    }
}

hipError_t launch_merge(const HalfStep &h, const Layout &L, int nsplit, hipStream_t s) {
    if (nsplit <= 32) {
        const unsigned blocks = (unsigned)((h.rows + 7) / 8);
        hipLaunchKernelGGL(lse_merge_kernel<32>, dim3(blocks), dim3(256), 0, s, h, nsplit, L.kp,
                           L.rs);
    } else {
        const unsigned blocks = (unsigned)((h.rows + 3) / 4);
        hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(blocks), dim3(256), 0, s, h, nsplit, L.kp,
                           L.rs);
    }
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Launch planning for the VALU path.
// --------------------------------------------------------------------------
namespace {

constexpr int kTargetBlocks = 2048;  // 8 waves per SIMD on 256 CUs x 4 SIMDs
constexpr int kMinTilesPerSplit = 2;
constexpr int kCUs = 256;

// Columns per LDS tile: 8 KB of fp64 records per buffer.
constexpr int tile_cols_for(int rs) { return rs <= 4 ? 256 : (rs <= 8 ? 128 : (rs <= 16 ? 64 : 32)); }

struct ValuPlan {
    int R;
    int TJ;
    int ntiles;
    int tiles_per_split;
    int nsplit;
    int64_t row_blocks;
};

// Narrow tiles for small problems with one-record-chunk records (d <= 3).
constexpr int kSmallTileCols = 32;

ValuPlan plan_valu(const Layout &L, int64_t rows, int64_t cols_pad) {
    ValuPlan p;
    p.TJ = tile_cols_for(L.rs);
    // When full-width tiles would leave fewer workgroups than CUs even at one
    // row per lane, narrower tiles give more column splits (1024^2 at d = 3:
    // 16 us per half-step with 256 columns, ~9.5 with 64, ~8 with 32); larger
    // problems keep the wide tiles, whose per-workgroup costs are lower
    // (16384^2: 85 us, against 110 us with 64-column tiles). Such plans
    // always end at one row per lane.
    if (L.rs <= 4 && (rows + 255) / 256 * (cols_pad / p.TJ) < kCUs)
        p.TJ = kSmallTileCols;
    p.ntiles = (int)(cols_pad / p.TJ);
    const int max_r = L.kp <= 3 ? 4 : (L.kp <= 15 ? 2 : 1);
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
    // At least kMinTilesPerSplit tiles per workgroup, so its fixed costs (row
    // records, the first tile's copy, the partial writes) are spread over
    // more work (16384^2 at d = 3: 95 -> 90 us per half-step) -- unless that
    // leaves fewer workgroups than CUs (1024^2: 16 -> 25 us per half-step).
    if (p.ntiles / want < kMinTilesPerSplit &&
        p.row_blocks * (p.ntiles / kMinTilesPerSplit) >= kCUs)
        want = p.ntiles / kMinTilesPerSplit > 0 ? p.ntiles / kMinTilesPerSplit : 1;
    if (want > 65535)
        want = 65535;
    if (want < 1)
        want = 1;
    p.tiles_per_split = (int)((p.ntiles + want - 1) / want);
    p.nsplit = (p.ntiles + p.tiles_per_split - 1) / p.tiles_per_split;
    return p;
}

template <int KP, int R, int TJ = tile_cols_for(KP + 1)>
hipError_t launch_kr(const HalfStep &h, const ValuPlan &p, hipStream_t s) {
    if (p.TJ != TJ)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)(p.row_blocks * p.nsplit));
    hipLaunchKernelGGL((lse_rows_valu_kernel<KP, R, TJ>), grid, dim3(256), 0, s, h,
                       p.tiles_per_split, p.ntiles, (int)p.row_blocks, p.nsplit);
    return hipGetLastError();
}

template <int KP>
hipError_t launch_k(const HalfStep &h, const ValuPlan &p, hipStream_t s) {
    switch (p.R) {
    case 4:
        if constexpr (KP <= 3)
            return launch_kr<KP, 4>(h, p, s);
        return hipErrorInvalidValue;
    case 2:
        if constexpr (KP <= 15)
            return launch_kr<KP, 2>(h, p, s);
        return hipErrorInvalidValue;
    default:
        if constexpr (KP <= 3)
            if (p.TJ == kSmallTileCols)
                return launch_kr<KP, 1, kSmallTileCols>(h, p, s);
        return launch_kr<KP, 1>(h, p, s);
    }
}

}  // namespace

size_t half_step_partials(const Layout &L, int64_t rows, int64_t cols_pad) {
    const ValuPlan p = plan_valu(L, rows, cols_pad);
    return p.nsplit > 1 ? (size_t)p.nsplit * (size_t)pad_points(rows) : 0;
}

hipError_t launch_half_step_valu(const HalfStep &h, const Layout &L, hipStream_t s) {
    const ValuPlan p = plan_valu(L, h.rows, h.cols_pad);
    hipError_t e;
    switch (L.kp) {
    case 3: e = launch_k<3>(h, p, s); break;
    case 7: e = launch_k<7>(h, p, s); break;
    case 11: e = launch_k<11>(h, p, s); break;
    case 15: e = launch_k<15>(h, p, s); break;
    case 19: e = launch_k<19>(h, p, s); break;
    case 23: e = launch_k<23>(h, p, s); break;
    case 27: e = launch_k<27>(h, p, s); break;
    case 31: e = launch_k<31>(h, p, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    if (p.nsplit > 1)
        return launch_merge(h, L, p.nsplit, s);
    return hipSuccess;
}

}  // namespace otsk
