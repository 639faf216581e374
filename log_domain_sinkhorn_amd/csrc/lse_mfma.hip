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
// VGPRs for the whole sweep) and streams the column records and biases of
// its split through a double-buffered LDS tile of 128 columns, shared by all 8
// waves. Record stride KP + 4 floats rotates LDS banks by 4 per record, so the
// per-lane 16-byte operand reads of 32 consecutive records do not conflict.
//
// Tiles are copied with gfx950's direct global->LDS loads
// (global_load_lds_dwordx4 for coordinates, _dword for biases): each wave
// issues whole chunks for the next tile at the top of an iteration and only
// waits for them at the tile's barrier, so no VGPRs hold the prefetch and the
// load latency hides behind a tile's worth of MFMAs.
//
// On gfx950 fp32 MFMAs and vector-ALU instructions do not execute
// concurrently on a SIMD (measured: an MFMA stream plus an FMA or exp2 stream
// takes the sum of their times, in one wave or spread over several), so a
// half-step costs MFMA cycles plus epilogue cycles and the epilogue is kept
// minimal:
//  * the column bias and the row's running maximum M enter through one extra
//    MFMA per subtile (k-slot 0: bias_j x 1, k-slot 1: 1 x -M_i) on a zero
//    accumulator, so the MFMA chain yields u_ji = s_ij - M_i directly;
//  * M is shared by the two lane halves holding row i and moves lazily: the
//    common epilogue is one exp2 and one add per value; only when a chunk's
//    sum leaves [2^-64, 2^16] (a term above 2^16, or no mass yet) does a
//    wave-uniform branch recompute the row maximum and rescale.
// The loop is software-pipelined over 32-column subtiles with two
// accumulators so a subtile's MFMA chain and the previous subtile's epilogue
// sit next to each other in one basic block.
#include "mfma_common.h"

#include <math.h>

namespace otsk {

hipError_t launch_merge(const HalfStep &h, const Layout &L, int nsplit, hipStream_t s);

namespace {

using namespace mfma;

constexpr int kWaves = 8;                 // waves per workgroup, 32 rows each
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;
constexpr int kTileCols = 128;            // columns per LDS tile
constexpr int kSub = kTileCols / 32;      // 32-column subtiles per tile
static_assert(kSub <= kWaves, "one wave copies each subtile's biases");
constexpr int kBiasSlots = 2 * kTileCols;

// Common part of the epilogue: the sum of 2^u over the lane's 16 values.
__device__ __forceinline__ float chunk_sum(const floatx16 &u) {
    float c0 = hw_exp2(u[0]), c1 = hw_exp2(u[1]);
#pragma unroll
    for (int v = 2; v < 16; v += 2) {
        c0 += hw_exp2(u[v]);
        c1 += hw_exp2(u[v + 1]);
    }
    return c0 + c1;
}

// Fold a subtile (values u relative to Mu, sum c) into the row's (M, S).
// Lanes l and l^32 hold the same row and keep the same M.
__device__ __forceinline__ void fold(const floatx16 &u, float Mu, float c, float &M, float &S) {
    const bool need = !(c <= 0x1p16f) || !(S + c >= 0x1p-64f) || Mu != M;
    if (__builtin_amdgcn_ballot_w64(need)) {
        // Rare (wave-uniform): move M to the larger of this subtile's row
        // maximum and the mass already accumulated, rescale, recompute c.
        float mh = u[0];
#pragma unroll
        for (int v = 1; v < 16; ++v)
            mh = fmaxf(mh, u[v]);
        mh = fmaxf(mh + Mu, M + hw_log2(S));
        const float Mn = fmaxf(mh, __shfl_xor(mh, 32));
        // S is 0 or >= 2^-64 (the common path only adds when S + c >= 2^-64)
        // and Mn >= M + log2 S, so the factor stays below 2^64; S = 0 is kept
        // apart because M may move down by ~1e30 past a padding-only chunk.
        S = S > 0.f ? S * hw_exp2(M - Mn) : 0.f;
        const float off = Mn - Mu;
        float c0 = 0.f, c1 = 0.f;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
            c0 += hw_exp2(u[v] - off);
            c1 += hw_exp2(u[v + 1] - off);
        }
        c = c0 + c1;
        M = Mn;
    }
    S += c;
}

// Keep the running (M, S) computed here: the fold above it may not be moved
// past this point (in particular not past the tile barrier that follows).
__device__ __forceinline__ void pin(float &M, float &S) { asm volatile("" : "+v"(M), "+v"(S)); }

template <int KP>
__global__ __launch_bounds__(kThreads) void lse_rows_mfma_kernel(HalfStep h, int tiles_per_split,
                                                                 int ntiles) {
    constexpr int RS = KP + 4;
    constexpr int RS4 = RS / 4;
    constexpr int TILE4 = kTileCols * RS4;
    constexpr int KH = KP / 2;
    static_assert(KP % 8 == 0, "each lane half reads whole float4s");
    static_assert(TILE4 % 64 == 0, "tiles are whole 64-lane chunks");
    __shared__ float4 lrec[2][TILE4];
    __shared__ float lbias[2][kBiasSlots];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int split = blockIdx.y;
    const int tbeg = split * tiles_per_split;
    const int tend = min(tbeg + tiles_per_split, ntiles);
    const float4 *col4 = static_cast<const float4 *>(h.col_rec);
    const float *colb = static_cast<const float *>(h.col_bias);

    // The ones of the extra MFMA's operand (never overwritten by the copies).
    for (int k = tid; k < 2 * kBiasSlots; k += kThreads) {
        const int e = k % kBiasSlots;
        if ((e / 32) & 1)
            lbias[k / kBiasSlots][e] = 1.f;
    }
    // Start the first tile's copy, then load the stationary B operands: this
    // lane's half of its row's scaled coordinates.
    issue_tile<TILE4, kWaves, kSub>(col4, colb, tbeg, lrec[0], lbias[0], wave, lane);
    const float scale = (float)h.scale;
    const int64_t i = (int64_t)blockIdx.x * kRowsPerBlock + wave * 32 + li;
    const int64_t ic = i < h.rows ? i : h.rows - 1;
    float bx[KH];
    float nrm_half = 0.f;
    {
        const float4 *p = reinterpret_cast<const float4 *>(
            static_cast<const float *>(h.row_rec) + ic * RS + hl * KH);
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
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Running reference M (shared by the row's two lane halves) and sum S.
    // Software pipeline over subtiles: the MFMA chain of one subtile is
    // issued before the previous subtile is folded.
    float M = 0.f;
    float S = 0.f;
    float Mu_prev = M;
    floatx16 acc_prev = score_tile<KP>(lrec[0], lbias[0], 0, lane, li, hl, bx, Mu_prev);
    for (int t = tbeg; t < tend; ++t) {
        const int b = (t - tbeg) & 1;
        if (t + 1 < tend)
            issue_tile<TILE4, kWaves, kSub>(col4, colb, t + 1, lrec[b ^ 1], lbias[b ^ 1], wave,
                                            lane);
#pragma unroll
        for (int sub = 1; sub < kSub; ++sub) {
            const float Mu_cur = M;
            const floatx16 acc_cur =
                score_tile<KP>(lrec[b], lbias[b], sub, lane, li, hl, bx, Mu_cur);
            const float c = chunk_sum(acc_prev);
            fold(acc_prev, Mu_prev, c, M, S);
            pin(M, S);
            acc_prev = acc_cur;
            Mu_prev = Mu_cur;
        }
        // The next tile has landed for every wave, and every wave is done
        // reading this one.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // First subtile of the next tile. On the last iteration this reads
        // the idle buffer and the result is never folded.
        const float Mu_cur = M;
        const floatx16 acc_cur =
            score_tile<KP>(lrec[b ^ 1], lbias[b ^ 1], 0, lane, li, hl, bx, Mu_cur);
        const float c = chunk_sum(acc_prev);
        fold(acc_prev, Mu_prev, c, M, S);
        pin(M, S);
        acc_prev = acc_cur;
        Mu_prev = Mu_cur;
    }

    // Merge the two lane halves (same row i, same M, disjoint columns). Both
    // halves add the same two numbers, so they agree bitwise.
    const float So = __shfl_xor(S, 32);
    const float no = __shfl_xor(nrm_half, 32);
    const float Sm = hl == 0 ? S + So : So + S;
    const float nrm = hl == 0 ? nrm_half + no : no + nrm_half;
    if (hl == 0 && i < h.rows) {
        if (gridDim.y == 1) {
            const float lse = M + hw_log2(Sm);
            const float hat = log2f(h.row_w[i]) - lse;
            static_cast<float *>(h.row_bias)[i] = hat;
            h.pot_out[i] = fmaf((float)h.eps_ln2, hat, nrm);
        } else {
            h.partials[(int64_t)split * h.rows_pad + i] = Partial{(double)M, Sm, 0.f};
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
