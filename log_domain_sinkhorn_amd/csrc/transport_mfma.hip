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
//  3. P.V on the bf16 matrix cores: P (fp32, in registers) and V are each
//     split into three bf16 parts h + m + l (8 + 8 + 8 significand bits, the
//     fp32 exponent range, so no scaling is needed), and
//       P.V ~ h.h + h.m + m.h + h.l + l.h + m.m     (dropped terms ~2^-24)
//     take 6 v_mfma_f32_32x32x16_bf16 (32 cycles) per 16 columns and 32
//     channels, against 8 v_mfma_f32_32x32x2f32 (64 cycles) for the same
//     work in fp32: 2.7x fewer matrix cycles. The B operand of an MFMA is 8
//     of a lane's 16 P registers: half h of lane (i, h) holds columns
//     j = 8*(v/4) + 4h + v%4, so registers 8u..8u+7 are the k-slots of
//     chunk u; the values are stored transposed in LDS with the columns of
//     each 16-block permuted to the same order, so the A operand is one
//     16-byte read. Each subtile's products start from a zero accumulator
//     (the matrix core's aligned sums lose ~2^-21 of their largest term) and
//     are added to the running sums by vector adds.
// No running maximum is needed: P is a plan, not a normalised softmax.
// With RSUM the row sums r_i = sum_j P_ij come out too (16 VALU adds per
// subtile), so the x-gradient 2(r_i x_i - sum_j P_ij y_j) needs one pass
// over the value channels of y instead of a pass over [y | 1].
// Accumulation is fp32 within a workgroup's column range; the column ranges'
// partials are added in fp64, in split order. No atomics.
//
// Up to kp = 192; larger records go to transport_rows_kernel
// (transport_rows.hip), every value channel in one pass.
#include "mfma_common.h"

#include <type_traits>

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
// bf16 per transposed value row in LDS and in the staged value buffer: the
// 64 columns of a tile and 8 of padding (row stride 36 dwords: the 16-byte
// operand reads of 16 consecutive channels hit distinct banks).
constexpr int kVRow = 72;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8(float4 v) { return __builtin_bit_cast(bf16x8, v); }

// Column position q (0..15) of a 16-block in the staged values holds column
// jmap(q): the k-slot order of the P registers (lane half q / 8, register
// q % 8 of the chunk).
__host__ __device__ constexpr int jmap(int q) { return 8 * ((q % 8) / 4) + 4 * (q / 8) + q % 4; }

// v = h + m + l with h, m, l bf16, each rounded once from an fp32 value (the
// asm statements keep the compiler from fusing the differences).
__device__ __forceinline__ void split3_bf16(float v, __bf16 &h, __bf16 &m, __bf16 &l) {
    asm volatile("" : "+v"(v));
    h = (__bf16)v;
    float r = v - (float)h;
    asm volatile("" : "+v"(r));
    m = (__bf16)r;
    float r2 = r - (float)m;
    asm volatile("" : "+v"(r2));
    l = (__bf16)r2;
}

// The same split for two values at once: each rounding is a lane of one
// v_cvt_pk_bf16_f32, and the pair lands packed as the MFMA operand wants it.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split3_bf16x2(float2v v, bf16x2v &h, bf16x2v &m, bf16x2v &l) {
    asm volatile("" : "+v"(v));
    h = __builtin_convertvector(v, bf16x2v);
    float2v r = v - __builtin_convertvector(h, float2v);
    asm volatile("" : "+v"(r));
    m = __builtin_convertvector(r, bf16x2v);
    float2v r2 = r - __builtin_convertvector(m, float2v);
    asm volatile("" : "+v"(r2));
    l = __builtin_convertvector(r2, bf16x2v);
}

// Copy n16 16-byte chunks from src to LDS dst with direct global->LDS loads.
template <int WAVES>
__device__ __forceinline__ void issue_copy(const float4 *__restrict__ src, float4 *dst, int n16,
                                           int wave, int lane) {
    for (int c = wave; c * 64 < n16; c += WAVES) {
        const int idx = c * 64 + lane;
        if (idx < n16)
            __builtin_amdgcn_global_load_lds(src + idx, (lds_void *)(dst + c * 64), 16, 0, 0);
    }
}

template <int KP, int NVB, bool RSUM>
__global__ __launch_bounds__(kThreads) void transport_mfma_kernel(
    const float4 *__restrict__ row_rec, const float *__restrict__ row_bias,
    const float4 *__restrict__ col4, const float *__restrict__ colb,
    const float4 *__restrict__ vt, int dv_pad, int k0, int64_t rows, int64_t rows_pad,
    int tiles_per_split, int ntiles, double *__restrict__ part, double *__restrict__ rpart) {
    constexpr int RC = KP / 4;
    constexpr int TILE4 = kTileCols * RC;
    constexpr int VC = 32 * NVB;                  // value channels per pass
    constexpr int PART16 = VC * kVRow / 8;        // 16-byte chunks of one bf16 part
    __shared__ float4 lrec[2][TILE4];
    __shared__ float lbias[2][kBiasSlots];
    __shared__ float4 lvt[2][3 * PART16];

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
    // Staged values: tile t, part p, channel c at vt[((t*3 + p)*dv_pad + c)*kVRow / 8].
    auto issue_values = [&](int t, float4 *dst) {
#pragma unroll
        for (int p = 0; p < 3; ++p)
            issue_copy<kWaves>(vt + ((int64_t)(t * 3 + p) * dv_pad + k0) * (kVRow / 8),
                               dst + p * PART16, PART16, wave, lane);
    };
    issue_tile<TILE4, kWaves, kSub>(col4, colb, tbeg, lrec[0], lbias[0], wave, lane);
    issue_values(tbeg, lvt[0]);

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

    // One column tile from LDS buffer b (a compile-time constant, so the
    // operand addresses are per-lane registers plus immediate offsets).
    auto tile = [&](int t, auto bc) {
        constexpr int b = decltype(bc)::value;
        if (t + 1 < tend) {
            issue_tile<TILE4, kWaves, kSub>(col4, colb, t + 1, lrec[b ^ 1], lbias[b ^ 1], wave,
                                            lane);
            issue_values(t + 1, lvt[b ^ 1]);
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
            // B operands: chunk u = registers 8u..8u+7, three bf16 parts.
            bf16x8 ph[2], pm[2], plo[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                bf16x2v h, mm, l;
                float2v pv = {pr[r], pr[r + 1]};
                split3_bf16x2(pv, h, mm, l);
                ph[r / 8][r % 8] = h[0];
                ph[r / 8][r % 8 + 1] = h[1];
                pm[r / 8][r % 8] = mm[0];
                pm[r / 8][r % 8 + 1] = mm[1];
                plo[r / 8][r % 8] = l[0];
                plo[r / 8][r % 8 + 1] = l[1];
            }
#pragma unroll
            for (int nb = 0; nb < NVB; ++nb) {
                floatx16 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                                0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                const int row = nb * 32 + li;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int at = (row * kVRow + sub * 32 + 16 * u + 8 * hl) / 8;
                    const bf16x8 vh = as_bf16x8(lvt[b][at]);
                    const bf16x8 vm = as_bf16x8(lvt[b][PART16 + at]);
                    const bf16x8 vl = as_bf16x8(lvt[b][2 * PART16 + at]);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vm, pm[u], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, ph[u], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, plo[u], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vm, ph[u], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, pm[u], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, ph[u], acc, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    O[nb][r] += acc[r];
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int t = tbeg; t < tend; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < tend)
            tile(t + 1, std::integral_constant<int, 1>{});
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

// Stage the values for the kernel above: for every column tile t (64
// columns), part p (h, m, l) and channel c < dv_pad, the row of kVRow bf16
// vt[((t*3 + p)*dv_pad + c)*kVRow + q] = part p of v[t*64 + 16*(q/16) +
// jmap(q % 16)][c] for q < 64 (zero for missing columns or channels and for
// the padding q >= 64).
__global__ __launch_bounds__(256) void values_bf16x3_kernel(const float *__restrict__ v,
                                                            int64_t m, int dv, int dv_pad,
                                                            int ntiles,
                                                            __bf16 *__restrict__ vt) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)ntiles * dv_pad * kVRow;
    if (e >= total)
        return;
    const int q = (int)(e % kVRow);
    const int c = (int)((e / kVRow) % dv_pad);
    const int64_t t = e / ((int64_t)kVRow * dv_pad);
    float x = 0.f;
    if (q < 64) {
        const int64_t j = t * 64 + 16 * (q / 16) + jmap(q % 16);
        if (j < m && c < dv)
            x = v[j * dv + c];
    }
    __bf16 h, mm, l;
    split3_bf16(x, h, mm, l);
    const int64_t base = (t * 3 * dv_pad + c) * kVRow + q;
    vt[base] = h;
    vt[base + (int64_t)dv_pad * kVRow] = mm;
    vt[base + 2 * (int64_t)dv_pad * kVRow] = l;
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

// Value channels per pass: 64 (two 32-channel blocks) when there are more
// than 32, except above KP = 128, where the second block's accumulators and
// operands do not fit beside the row operands.
int value_blocks(int dv, int kp) { return dv <= 32 || kp > 128 ? 1 : 2; }

// Whether the one-pass kernel of transport_rows.hip takes the call: always
// above kp = 192; at kp = 160 and 192 when this kernel's passes (each forming
// the score again, 3 kp / 16 f16 and 12 bf16 matrix instructions per 32
// channels per 32x32 subtile) cost more than one pass over dv rounded up to
// 256 channels, at the measured efficiencies (about 0.5 of the matrix-pipe
// time here, 0.33 there; d = 192, dv = 192: 31.6 ms here).
bool one_pass(int dv, int kp) {
    if (kp > 192)
        return true;
    if (kp < 160)
        return false;
    const int64_t vc = 32 * value_blocks(dv, kp);
    const int64_t passes = (dv + vc - 1) / vc;
    const int64_t here = passes * (3 * kp / 16 + 12 * vc / 32);
    const int64_t there = 3 * kp / 16 + 12 * ((dv + 255) / 256 * 256) / 32;
    return 2 * here > 3 * there;
}

template <int KP, int NVB>
hipError_t launch_tm(const float4 *xrec, const float *xbias, const float4 *col4, const float *colb,
                     const float4 *vt, int dv_pad, int k0, int64_t n, int64_t n_pad,
                     const MPlan &p, double *part, double *rpart, hipStream_t s) {
    dim3 grid((unsigned)p.row_blocks, (unsigned)p.nsplit);
    if (rpart)
        hipLaunchKernelGGL((transport_mfma_kernel<KP, NVB, true>), grid, dim3(kThreads), 0, s,
                           xrec, xbias, col4, colb, vt, dv_pad, k0, n, n_pad, p.tiles_per_split,
                           p.ntiles, part, rpart);
    else
        hipLaunchKernelGGL((transport_mfma_kernel<KP, NVB, false>), grid, dim3(kThreads), 0, s,
                           xrec, xbias, col4, colb, vt, dv_pad, k0, n, n_pad, p.tiles_per_split,
                           p.ntiles, part, rpart);
    return hipGetLastError();
}

template <int NVB>
hipError_t launch_tm_kp(int kp, const float4 *xrec, const float *xbias, const float4 *col4,
                        const float *colb, const float4 *vt, int dv_pad, int k0, int64_t n,
                        int64_t n_pad, const MPlan &p, double *part, double *rpart,
                        hipStream_t s) {
#define OTSK_TM(KPV)                                                                           \
    case KPV:                                                                                  \
        return launch_tm<KPV, NVB>(xrec, xbias, col4, colb, vt, dv_pad, k0, n, n_pad, p, part, \
                                   rpart, s);
    switch (kp) {
        OTSK_TM(32)
        OTSK_TM(64)
        OTSK_TM(96)
        OTSK_TM(128)
    default:
        break;
    }
    if constexpr (NVB == 1) {
        switch (kp) {
            OTSK_TM(160)
            OTSK_TM(192)
        default:
            break;
        }
    }
    return hipErrorInvalidValue;
#undef OTSK_TM
}

// Doubles of scratch ahead of the staged values (partials and row sums),
// rounded to a 256-byte boundary.
size_t partial_doubles(int64_t n, int64_t m_pad, int dv, bool rowsum, int kp) {
    const MPlan p = plan_tm(n, m_pad);
    const size_t per_row = (size_t)(32 * value_blocks(dv, kp)) + (rowsum ? 1 : 0);
    const size_t d = (size_t)p.nsplit * (size_t)pad_points(n) * per_row;
    return (d + 31) / 32 * 32;
}

int padded_channels(int dv, int kp) {
    const int vc = 32 * value_blocks(dv, kp);
    return (dv + vc - 1) / vc * vc;
}

}  // namespace

size_t transport_mfma_scratch_doubles(int64_t n, int64_t m_pad, int dv, bool rowsum, int kp) {
    if (one_pass(dv, kp))
        return transport_rows_scratch_doubles(n, m_pad, dv, rowsum);
    const size_t vt_bytes = (size_t)(m_pad / kTileCols) * 3 * (size_t)padded_channels(dv, kp) *
                            kVRow * sizeof(__bf16);
    return partial_doubles(n, m_pad, dv, rowsum, kp) + (vt_bytes + 7) / 8;
}

hipError_t launch_transport_apply_mfma(int kp, const void *xrow, const float *xhat,
                                       const void *ycol, const float *yhat, const float *v,
                                       int64_t n, int64_t n_pad, int64_t m, int64_t m_pad, int dv,
                                       double *part, float *out, float *rowsum, hipStream_t s) {
    if (one_pass(dv, kp))
        return launch_transport_rows(kp, xrow, xhat, ycol, yhat, v, n, n_pad, m, m_pad, dv, part,
                                     out, rowsum, s);
    const MPlan p = plan_tm(n, m_pad);
    const int nvb = value_blocks(dv, kp);
    const int vc = 32 * nvb;
    const int dv_pad = padded_channels(dv, kp);
    const float4 *xr = static_cast<const float4 *>(xrow);
    const float4 *col4 = static_cast<const float4 *>(ycol);
    // Row-sum partials follow the value partials; the staged values follow both.
    double *rpart = rowsum ? part + (size_t)p.nsplit * (size_t)n_pad * (size_t)vc : nullptr;
    __bf16 *vt =
        reinterpret_cast<__bf16 *>(part + partial_doubles(n, m_pad, dv, rowsum != nullptr, kp));
    {
        const int64_t total = (int64_t)p.ntiles * dv_pad * kVRow;
        hipLaunchKernelGGL(values_bf16x3_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                           0, s, v, m, dv, dv_pad, p.ntiles, vt);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const float4 *vt4 = reinterpret_cast<const float4 *>(vt);
    for (int k0 = 0; k0 < dv; k0 += vc) {
        double *rp = k0 == 0 ? rpart : nullptr;
        hipError_t e = nvb == 1 ? launch_tm_kp<1>(kp, xr, xhat, col4, yhat, vt4, dv_pad, k0, n,
                                                  n_pad, p, part, rp, s)
                                : launch_tm_kp<2>(kp, xr, xhat, col4, yhat, vt4, dv_pad, k0, n,
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
