// Log-domain Sinkhorn half-step with the dot products on the fp32 matrix
// cores of gfx950 (feature dimension d >= 32).
//
// Same update as the VALU kernel ("FlashSinkhorn: IO-Aware Entropic Optimal
// Transport on GPU", Methodik sections 1-2): s_ij = (2 log2(e)/eps) p_i.q_j +
// qhat_j, an online base-2 log-sum-exp over j, phat_i = log2 w_i - lse_i.
// The page's kernels form the score tile as Q K^T on tensor cores; here a
// tile of 32 columns x 32 rows is one chain of KP/2 v_mfma_f32_32x32x2f32:
//
//   D[j][i] = sum_k A[j][k] B[k][i] + Cinit[j][i]
//   A = column coordinates q_j (raw),  B = scaled row coordinates,
//   Cinit[j][i] = qhat_j (the bias enters through the accumulator).
//
// The reduced index j is put on the output's per-lane register axis: lane l
// holds column i = l % 32 and the 16 rows j = 8*(v/4) + 4*(l/32) + v%4 of
// its accumulator registers v, so every lane keeps a private running
// (max, sum) for its row i and the two lane halves merge once at the end.
// The k index of each MFMA is split between lane halves (half h supplies
// k = h*KP/2 + q for the q-th MFMA) so a lane's A and B operands for the whole
// chain are KP/2 contiguous floats: 16-byte LDS reads and loads.
//
// A workgroup of 8 waves owns 256 rows (32 per wave, the B operands stay in
// VGPRs for the whole sweep) and streams the column records of its split
// through a double-buffered LDS tile of 64 columns, shared by all 8 waves.
// Record stride KP + 4 floats rotates LDS banks by 4 per record, so the
// per-lane 16-byte operand reads of 32 consecutive records do not conflict.
#include "ot_internal.h"

#include <math.h>

namespace otsk {

hipError_t launch_merge(const HalfStep &h, const Layout &L, int nsplit, hipStream_t s);

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr int kThreads = 512;   // 8 waves
constexpr int kRowsPerBlock = 256;
constexpr int kTileCols = 64;

template <int KP>
__global__ __launch_bounds__(kThreads) void lse_rows_mfma_kernel(HalfStep h, int tiles_per_split,
                                                                 int ntiles) {
    constexpr int RS = KP + 4;
    constexpr int RS4 = RS / 4;
    constexpr int TILE4 = kTileCols * RS4;
    constexpr int PF = (TILE4 + kThreads - 1) / kThreads;
    constexpr int KH = KP / 2;
    static_assert(KP % 8 == 0, "each lane half reads whole float4s");
    __shared__ float4 lrec[2][TILE4];
    __shared__ float4 lbias[2][kTileCols / 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);

    // Stationary B operands: this lane's half of its row's scaled coordinates.
    const float scale = (float)h.scale;
    const int64_t i = (int64_t)blockIdx.x * kRowsPerBlock + wave * 32 + li;
    const int64_t ic = i < h.rows ? i : h.rows - 1;
    float bx[KH];
    float nrm_half = 0.f;
    {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(h.row_rec) +
                                                         ic * RS + hl * KH);
#pragma unroll
        for (int q = 0; q < KH / 4; ++q) {
            const float4 v = p[q];
            nrm_half = fmaf(v.x, v.x, nrm_half);
            nrm_half = fmaf(v.y, v.y, nrm_half);
            nrm_half = fmaf(v.z, v.z, nrm_half);
            nrm_half = fmaf(v.w, v.w, nrm_half);
            bx[4 * q + 0] = v.x * scale;
            bx[4 * q + 1] = v.y * scale;
            bx[4 * q + 2] = v.z * scale;
            bx[4 * q + 3] = v.w * scale;
        }
    }

    const float4 *col4 = static_cast<const float4 *>(h.col_rec);
    float M = -INFINITY;
    float S = 0.f;

#pragma unroll
    for (int q = 0; q < PF; ++q) {
        const int idx = tid + q * kThreads;
        if (TILE4 % kThreads == 0 || idx < TILE4) {
            const float4 v = col4[(int64_t)tbeg * TILE4 + idx];
            lrec[0][idx] = v;
            const int c = idx / RS4;
            if (idx - c * RS4 == KP / 4)
                reinterpret_cast<float *>(lbias[0])[c] = v.x;
        }
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
                const int idx = min(tid + q * kThreads, TILE4 - 1);
                pre[q] = col4[(int64_t)tn * TILE4 + idx];
            }
        }
#pragma unroll
        for (int sub = 0; sub < kTileCols / 32; ++sub) {
            floatx16 acc;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 bv = lbias[b][sub * 8 + 2 * g4 + hl];
                acc[4 * g4 + 0] = bv.x;
                acc[4 * g4 + 1] = bv.y;
                acc[4 * g4 + 2] = bv.z;
                acc[4 * g4 + 3] = bv.w;
            }
            const float4 *ap = &lrec[b][(sub * 32 + li) * RS4 + hl * (KH / 4)];
#pragma unroll
            for (int q4 = 0; q4 < KH / 4; ++q4) {
                const float4 av = ap[q4];
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bx[4 * q4 + 0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bx[4 * q4 + 1], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bx[4 * q4 + 2], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bx[4 * q4 + 3], acc, 0, 0, 0);
            }
            float mx = acc[0];
#pragma unroll
            for (int v = 1; v < 16; ++v)
                mx = fmaxf(mx, acc[v]);
            if (mx > M + 64.f) {
                S *= hw_exp2(M - mx);
                M = mx;
            }
            float c = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v)
                c += hw_exp2(acc[v] - M);
            S += c;
        }
        {
#pragma unroll
            for (int q = 0; q < PF; ++q) {
                const int idx = tid + q * kThreads;
                if (TILE4 % kThreads == 0 || idx < TILE4) {
                    lrec[b ^ 1][idx] = pre[q];
                    const int c = idx / RS4;
                    if (idx - c * RS4 == KP / 4)
                        reinterpret_cast<float *>(lbias[b ^ 1])[c] = pre[q].x;
                }
            }
        }
        __syncthreads();
    }

    // Merge the two lane halves (same row i, disjoint columns). Both halves
    // form the same sums in the same order, so they agree bitwise.
    const float Mo = __shfl_xor(M, 32);
    const float So = __shfl_xor(S, 32);
    const float no = __shfl_xor(nrm_half, 32);
    const float Mm = fmaxf(M, Mo);
    const float e0 = S * hw_exp2(M - Mm);
    const float e1 = So * hw_exp2(Mo - Mm);
    const float Sm = hl == 0 ? e0 + e1 : e1 + e0;
    const float nrm = hl == 0 ? nrm_half + no : no + nrm_half;
    if (hl == 0 && i < h.rows) {
        if (gridDim.y == 1) {
            const float lse = Mm + hw_log2(Sm);
            const float hat = log2f(h.row_w[i]) - lse;
            static_cast<float *>(h.row_bias)[i * RS + KP] = hat;
            h.pot_out[i] = fmaf((float)h.eps_ln2, hat, nrm);
        } else {
            h.partials[(int64_t)split * h.rows_pad + i] = Partial{(double)Mm, Sm, 0.f};
        }
    }
}

constexpr int kTargetBlocks = 1024;  // x 8 waves = 8 waves per SIMD

struct MfmaPlan {
    int ntiles;
    int tiles_per_split;
    int nsplit;
    int64_t row_blocks;
};

MfmaPlan plan_mfma(int64_t rows, int64_t cols_pad) {
    MfmaPlan p;
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

template <int KP>
hipError_t launch_kp(const HalfStep &h, const MfmaPlan &p, hipStream_t s) {
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    hipLaunchKernelGGL((lse_rows_mfma_kernel<KP>), grid, dim3(kThreads), 0, s, h,
                       p.tiles_per_split, p.ntiles);
    return hipGetLastError();
}

}  // namespace

size_t half_step_partials_mfma(int64_t rows, int64_t cols_pad) {
    const MfmaPlan p = plan_mfma(rows, cols_pad);
    return p.nsplit > 1 ? (size_t)p.nsplit * (size_t)pad_points(rows) : 0;
}

hipError_t launch_half_step_mfma(const HalfStep &h, const Layout &L, hipStream_t s) {
    const MfmaPlan p = plan_mfma(h.rows, h.cols_pad);
    hipError_t e;
    switch (L.kp) {
    case 32: e = launch_kp<32>(h, p, s); break;
    case 48: e = launch_kp<48>(h, p, s); break;
    case 64: e = launch_kp<64>(h, p, s); break;
    case 80: e = launch_kp<80>(h, p, s); break;
    case 96: e = launch_kp<96>(h, p, s); break;
    case 112: e = launch_kp<112>(h, p, s); break;
    case 128: e = launch_kp<128>(h, p, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    if (p.nsplit > 1)
        return launch_merge(h, L, p.nsplit, s);
    return hipSuccess;
}

}  // namespace otsk
