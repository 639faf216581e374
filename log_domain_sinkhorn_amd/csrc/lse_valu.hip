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
// Mapping onto the hardware:
//  * each lane owns R rows (their scaled coordinates, running max M and
//    running sum S live in VGPRs for the whole column sweep);
//  * a 256-lane workgroup streams column records through a double-buffered
//    LDS tile (one coalesced 16-byte load per lane per tile, one barrier per
//    tile); every lane of a wave reads the same record, so the LDS read is a
//    conflict-free broadcast;
//  * per chunk of T columns: the scores, one max per row, a rescale only when
//    the chunk maximum exceeds M by more than 64 (so every term stays below
//    2^64 and the sum cannot overflow), then exp2 and a chunk-local sum that
//    is added to S (blocked summation);
//  * when the columns are split over several workgroups (grid.y > 1) each
//    writes its (M, S) pair and a merge kernel combines them in split order.
// No atomics: the result is bitwise reproducible.
#include "ot_internal.h"

#include <math.h>

namespace otsk {

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// --------------------------------------------------------------------------
// Record preparation: copy coordinates (zero padded to kp), write the bias.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_side_kernel(const float *__restrict__ pts,
                                                        const float *__restrict__ pot, int64_t count,
                                                        int64_t padded, int d, int kp, int rs,
                                                        float hat_scale, int bias_mode,
                                                        float *__restrict__ rec) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= padded)
        return;
    float *r = rec + i * rs;
    if (i < count) {
        float nrm = 0.f;
        for (int k = 0; k < kp; ++k) {
            const float v = k < d ? pts[i * d + k] : 0.f;
            r[k] = v;
            nrm = fmaf(v, v, nrm);
        }
        float bias = 0.f;
        if (bias_mode == kBiasHat)
            bias = (pot[i] - nrm) * hat_scale;
        else if (bias_mode == kBiasRaw)
            bias = pot[i];
        r[kp] = bias;
    } else {
        for (int k = 0; k < kp; ++k)
            r[k] = 0.f;
        r[kp] = kPadBias;
    }
    for (int k = kp + 1; k < rs; ++k)
        r[k] = 0.f;
}

hipError_t launch_prep_side(const float *pts, const float *pot, int64_t count, int64_t padded,
                            const Layout &L, float hat_scale, int bias_mode, float *rec,
                            hipStream_t s) {
    const unsigned blocks = (unsigned)((padded + 255) / 256);
    hipLaunchKernelGGL(prep_side_kernel, dim3(blocks), dim3(256), 0, s, pts, pot, count, padded,
                       L.d, L.kp, L.rs, hat_scale, bias_mode, rec);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Epilogue shared by the one-pass kernels and the merge: from the final
// (M, S) of row i write its bias slot and its potential.
// --------------------------------------------------------------------------
__device__ __forceinline__ void finish_row(const HalfStep &h, int kp, int rs, int64_t i, float M,
                                           float S, float nrm) {
    const float lse = M + hw_log2(S);
    const float hat = log2f(h.row_w[i]) - lse;
    h.row_bias[i * rs + kp] = hat;
    h.pot_out[i] = fmaf(h.eps_ln2, hat, nrm);
}

// --------------------------------------------------------------------------
// The tiled half-step. KP coordinates per record (RS = KP + 1 floats),
// R rows per lane, TJ columns per LDS tile.
// --------------------------------------------------------------------------
template <int KP, int R, int TJ>
__global__ __launch_bounds__(256) void lse_rows_valu_kernel(HalfStep h, int tiles_per_split,
                                                            int ntiles) {
    constexpr int RS = KP + 1;
    static_assert(RS % 4 == 0, "record stride must be a multiple of 4 floats");
    constexpr int RS4 = RS / 4;
    constexpr int TILE4 = TJ * RS4;
    constexpr int PF = (TILE4 + 255) / 256;
    constexpr int T = 8;
    static_assert(TJ % T == 0, "tile must hold whole chunks");
    __shared__ float4 lds[2][TILE4];

    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * (256 * R);
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);

    float xs[R][KP];
    float nrm[R], M[R], S[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t i = row0 + tid + r * 256;
        i = i < h.rows ? i : h.rows - 1;
        const float *p = h.row_rec + i * RS;
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const float v = p[k];
            q = fmaf(v, v, q);
            xs[r][k] = v * h.scale;
        }
        nrm[r] = q;
        M[r] = -INFINITY;
        S[r] = 0.f;
    }

    const float4 *col4 = reinterpret_cast<const float4 *>(h.col_rec);
#pragma unroll
    for (int q = 0; q < PF; ++q) {
        const int idx = tid + q * 256;
        if (TILE4 % 256 == 0 || idx < TILE4)
            lds[0][idx] = col4[(int64_t)tbeg * TILE4 + idx];
    }
    __syncthreads();
    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        // Next tile (the last iteration reloads its own tile; the copy into
        // the idle buffer is then unused). Unconditional, so the prefetch
        // stays in registers.
        const int tn = t + 1 < tend ? t + 1 : t;
        float4 pre[PF];
        {
#pragma unroll
            for (int q = 0; q < PF; ++q) {
                const int idx = min(tid + q * 256, TILE4 - 1);
                pre[q] = col4[(int64_t)tn * TILE4 + idx];
            }
        }
        const float4 *tile = lds[b];
        for (int c0 = 0; c0 < TJ; c0 += T) {
            float s[R][T];
#pragma unroll
            for (int u = 0; u < T; ++u) {
                float rec[RS];
#pragma unroll
                for (int q = 0; q < RS4; ++q) {
                    const float4 v = tile[(c0 + u) * RS4 + q];
                    rec[4 * q + 0] = v.x;
                    rec[4 * q + 1] = v.y;
                    rec[4 * q + 2] = v.z;
                    rec[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float acc = rec[KP];
#pragma unroll
                    for (int k = KP - 1; k >= 0; --k)
                        acc = fmaf(xs[r][k], rec[k], acc);
                    s[r][u] = acc;
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float mx = s[r][0];
#pragma unroll
                for (int u = 1; u < T; ++u)
                    mx = fmaxf(mx, s[r][u]);
                if (mx > M[r] + 64.f) {
                    S[r] *= hw_exp2(M[r] - mx);
                    M[r] = mx;
                }
                float c = 0.f;
#pragma unroll
                for (int u = 0; u < T; ++u)
                    c += hw_exp2(s[r][u] - M[r]);
                S[r] += c;
            }
        }
        {
#pragma unroll
            for (int q = 0; q < PF; ++q) {
                const int idx = tid + q * 256;
                if (TILE4 % 256 == 0 || idx < TILE4)
                    lds[b ^ 1][idx] = pre[q];
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = row0 + tid + r * 256;
        if (i < h.rows) {
            if (gridDim.y == 1)
                finish_row(h, KP, RS, i, M[r], S[r], nrm[r]);
            else
                h.partials[(int64_t)split * h.rows_pad + i] = make_float2(M[r], S[r]);
        }
    }
}

// Combine the per-split (M, S) pairs of each row in split order.
__global__ __launch_bounds__(256) void lse_merge_kernel(HalfStep h, int nsplit, int kp, int rs) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= h.rows)
        return;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s)
        M = fmaxf(M, h.partials[(int64_t)s * h.rows_pad + i].x);
    float S = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float2 p = h.partials[(int64_t)s * h.rows_pad + i];
        S = fmaf(p.y, hw_exp2(p.x - M), S);
    }
    const float *p = h.row_rec + i * rs;
    float q = 0.f;
    for (int k = 0; k < kp; ++k)
        q = fmaf(p[k], p[k], q);
    finish_row(h, kp, rs, i, M, S, q);
}

hipError_t launch_merge(const HalfStep &h, const Layout &L, int nsplit, hipStream_t s) {
    const unsigned blocks = (unsigned)((h.rows + 255) / 256);
    hipLaunchKernelGGL(lse_merge_kernel, dim3(blocks), dim3(256), 0, s, h, nsplit, L.kp, L.rs);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Launch planning for the VALU path.
// --------------------------------------------------------------------------
namespace {

constexpr int kTargetBlocks = 2048;  // 8 waves per SIMD on 256 CUs x 4 SIMDs

int tile_cols(int rs) { return rs <= 8 ? 256 : (rs <= 16 ? 128 : 64); }

struct ValuPlan {
    int R;
    int TJ;
    int ntiles;
    int tiles_per_split;
    int nsplit;
    int64_t row_blocks;
};

ValuPlan plan_valu(const Layout &L, int64_t rows, int64_t cols_pad) {
    ValuPlan p;
    p.TJ = tile_cols(L.rs);
    p.ntiles = (int)(cols_pad / p.TJ);
    const int max_r = L.kp <= 7 ? 4 : 2;
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

template <int KP, int R>
hipError_t launch_kr(const HalfStep &h, const ValuPlan &p, hipStream_t s) {
    constexpr int TJ = (KP + 1) <= 8 ? 256 : ((KP + 1) <= 16 ? 128 : 64);
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    hipLaunchKernelGGL((lse_rows_valu_kernel<KP, R, TJ>), grid, dim3(256), 0, s, h,
                       p.tiles_per_split, p.ntiles);
    return hipGetLastError();
}

template <int KP>
hipError_t launch_k(const HalfStep &h, const ValuPlan &p, hipStream_t s) {
    switch (p.R) {
    case 4:
        if constexpr (KP <= 7)
            return launch_kr<KP, 4>(h, p, s);
        return hipErrorInvalidValue;
    case 2:
        return launch_kr<KP, 2>(h, p, s);
    default:
        return launch_kr<KP, 1>(h, p, s);
    }
}

}  // namespace

size_t half_step_partials(const Layout &L, int64_t rows, int64_t cols_pad) {
    if (L.mfma)
        return 0;  // sized by the MFMA planner
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
