// Transport application above 192 coordinates with every value channel in one
// pass over the columns: out_i = sum_j P_ij v_j, P never stored
// ("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodik
// section 3: applying the plan is an attention-like weighted average over
// the streamed tiles).
//
// A workgroup of 8 waves owns 32 rows and all dv_pad = 256 NB value channels
// (wave w holds channels 32 NB w .. 32 NB w + 32 NB - 1 of its 32 rows as NB
// 32x32 accumulators). It walks its column split in blocks of 256 columns.
// Per block the split-f16 score goes through LDS in 32-coordinate stages of
// the records (the 32 row records and the 256 column records; above
// kStagedRecordKP one 128-byte line each, below it the 4 hi and 4 lo chunks of
// the stage, columns with their chunk swizzle), three stages deep, filled by
// direct global->LDS loads two stages ahead (the waits, barriers and clamped
// reloads of the pipeline in gemm_pipeline.h); wave w forms the 32x32 subtile
// of columns 32w .. 32w + 31
// (chains from zero per stage, flushed into fp32 sums, as in the other
// kernels). After the block's last stage each wave splits its P_ij =
// 2^((dot + ghat_j) + fhat_i) into three bf16 parts (h + m + l, each rounded
// once) and writes them to three LDS planes of 32 rows x 256 columns; then
// every wave multiplies the whole tile by its channels of the block's values:
// B operand 8 consecutive columns of P (one row), A operand 8 consecutive
// columns of one channel of v, both in three parts (h.h + h.m + m.h + h.l +
// l.h + m.m, each 16-column product from a zero accumulator, added to the
// running fp32 sums). The values are split the same way once per call
// (values_split_kernel) and read from L2 in blocks of 16 columns x dv_pad
// channels x 3 parts (a wave's 32 channels x 16 columns of one part are 1 KiB
// in a row), kTVD six-product steps ahead of their use. With RSUM the row sums come
// out too. Partials per column split in fp64, added in split order.
//
// It replaced a kernel on the same stage pipeline with 128-row workgroups,
// which had to form the score again for every 64 value channels.
#include "mfma_common.h"

#include <type_traits>

namespace otsk {

namespace {

using namespace mfma;

constexpr int kTW = 8;                // waves per workgroup
constexpr int kTR = 32;               // rows per workgroup
constexpr int kTN = 256;              // columns per block (32 per wave)
constexpr int kTStage4 = (kTR + kTN) * 8;  // 16-byte chunks per stage
constexpr int kTPP = kTN / 8 + 1;     // 16-byte chunks per row of a P plane (padded)
constexpr int kTLoads = 5;            // direct loads per wave and stage
constexpr int kTVD = 4;               // value loads in flight, in 6-product steps
constexpr int kTKS = 32;              // coordinates per stage
constexpr int kTTargetBlocks = 4096;

typedef __bf16 bf16x8t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2t __attribute__((ext_vector_type(2)));
typedef float float2t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int tslot(int r, int t) { return r * 8 + (t ^ ((r ^ (r >> 3)) & 7)); }

// Split two fp32 values into three bf16 parts (h + m + l, each rounded once:
// h = bf16(x), m = bf16(x - h), l = bf16(x - h - m)).
__device__ __forceinline__ void split2(float2t x, bf16x2t &h, bf16x2t &m, bf16x2t &l) {
    asm volatile("" : "+v"(x));
    h = __builtin_convertvector(x, bf16x2t);
    float2t r = x - __builtin_convertvector(h, float2t);
    asm volatile("" : "+v"(r));
    m = __builtin_convertvector(r, bf16x2t);
    float2t r2 = r - __builtin_convertvector(m, float2t);
    asm volatile("" : "+v"(r2));
    l = __builtin_convertvector(r2, bf16x2t);
}

__device__ __forceinline__ void split4(float4 a, bf16x4t &h, bf16x4t &m, bf16x4t &l) {
    bf16x2t h0, m0, l0, h1, m1, l1;
    split2(float2t{a.x, a.y}, h0, m0, l0);
    split2(float2t{a.z, a.w}, h1, m1, l1);
    h = bf16x4t{h0[0], h0[1], h1[0], h1[1]};
    m = bf16x4t{m0[0], m0[1], m1[0], m1[1]};
    l = bf16x4t{l0[0], l0[1], l1[0], l1[1]};
}

// Direct loads of stage s of the block at col0 into buf: row record r
// (0 .. 31) and column record 32 + c fill slots 8r .. 8r + 7 with the read
// swizzle of tslot. Rows: wave w fills slots 32w .. 32w + 31 (lanes 0-31);
// columns: wave w fills 4 x 64 slots; 5 loads per wave and stage. Records
// above kStagedRecordKP hold each stage's 8 chunks at 8s .. 8s + 7; below it
// the stage's hi chunks are 4s .. 4s + 3 and its lo chunks KP/8 + 4s ..,
// column chunk q of point j stored at q ^ (j & SW). With the last stage,
// waves 0-3 also load the block's 256 column biases into bias.
template <int KP>
__device__ __forceinline__ void t_issue(const float4 *__restrict__ row4,
                                        const float4 *__restrict__ col4,
                                        const float *__restrict__ colb, int64_t row0,
                                        int64_t col0, int s, bool last, float4 *buf,
                                        float *bias, int wave, int lane) {
    constexpr int RC = KP / 4;
    constexpr bool STAGED = KP > kStagedRecordKP;
    if (lane < 32) {
        const int c = 32 * wave + lane;
        const int r = c >> 3;
        const int t = (c & 7) ^ ((r ^ (r >> 3)) & 7);
        const int q = STAGED ? 8 * s + t : (t < 4 ? 0 : KP / 8) + 4 * s + (t & 3);
        __builtin_amdgcn_global_load_lds(row4 + (row0 + r) * RC + q,
                                         (lds_void *)(buf + 32 * wave), 16, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int g = 4 * wave + k;
        const int c = g * 64 + lane;  // column slot, 0 .. 2047
        const int rl = c >> 3;        // column within the block
        const int r = kTR + rl;
        const int t = (c & 7) ^ ((r ^ (r >> 3)) & 7);
        const int q = STAGED ? 8 * s + t
                             : ((t < 4 ? 0 : KP / 8) + 4 * s + (t & 3)) ^ (rl & swizzle_mask(RC));
        __builtin_amdgcn_global_load_lds(col4 + (col0 + rl) * RC + q,
                                         (lds_void *)(buf + kTR * 8 + g * 64), 16, 0, 0);
    }
    if (last && wave < kTN / 64)
        __builtin_amdgcn_global_load_lds(
            colb + col0 + 64 * wave + lane,
            (lds_void *)(bias + 64 * wave), 4, 0, 0);
}

template <int KP, int NB, bool RSUM>
__global__ __launch_bounds__(64 * kTW) void transport_rows_kernel(
    const float4 *__restrict__ row_rec, const float *__restrict__ row_bias,
    const float4 *__restrict__ col4, const float *__restrict__ colb,
    const bf16x8t *__restrict__ vb, int dv_pad, int64_t rows, int64_t rows_pad, int nrb,
    int blocks_per_split, int nblocks, double *__restrict__ part, double *__restrict__ rpart) {
    constexpr int NS = KP / kTKS;
    static_assert(KP % kTKS == 0 && NS >= 2, "whole stages");
    __shared__ float4 st0[kTStage4];
    __shared__ float4 st1[kTStage4];
    __shared__ float4 st2[kTStage4];
    // The column biases of the block in flight: loaded with its last stage,
    // at least two stages after the previous block's epilogue read them.
    __shared__ float4 bias4[kTN / 4];
    float *const biasb = reinterpret_cast<float *>(bias4);
    __shared__ bf16x8t pp[3 * kTR * kTPP];  // P in 3 planes of 32 rows x kTPP chunks
    __shared__ float rowv[kTR];
    float4 *const stg[3] = {st0, st1, st2};

    const int L = (int)blockIdx.x;
    const int split = L / nrb;
    const int rb = L - split * nrb;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int bbeg = split * blocks_per_split;
    const int bend = min(bbeg + blocks_per_split, nblocks);
    const int64_t row0 = (int64_t)rb * kTR;
    // This wave's first value channel (wave-uniform, so that the value
    // addresses are a scalar base plus one per-lane offset).
    const int c0 = 32 * NB * __builtin_amdgcn_readfirstlane(wave);
    if (tid < kTR) {
        const int64_t i = row0 + tid;
        rowv[tid] = row_bias[i < rows ? i : rows - 1];
    }
    __syncthreads();

    floatx16 O[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            O[nb][r] = 0.f;
    float rsum = 0.f;

    const int T = (bend - bbeg) * NS;
    auto issue = [&](int t, auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value;
        const int cb = bbeg + t / NS;
        t_issue<KP>(row_rec, col4, colb, row0, (int64_t)cb * kTN, t % NS, t % NS == NS - 1,
                    stg[b], biasb, wave, lane);
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1>{});

    floatx16 sum;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        sum[v] = 0.f;

    // The block's P tile times this wave's channels of the block's values.
    auto epilogue = [&](const float *bias, int cb) __attribute__((always_inline)) {
        const float fh = rowv[li];
        bf16x4t *pw = reinterpret_cast<bf16x4t *>(pp);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = 32 * wave + 8 * q + 4 * hl;
            const float4 b4 = *reinterpret_cast<const float4 *>(bias + col);
            float4 p4;
            p4.x = hw_exp2((sum[4 * q + 0] + b4.x) + fh);
            p4.y = hw_exp2((sum[4 * q + 1] + b4.y) + fh);
            p4.z = hw_exp2((sum[4 * q + 2] + b4.z) + fh);
            p4.w = hw_exp2((sum[4 * q + 3] + b4.w) + fh);
            if (RSUM)
                rsum += (p4.x + p4.y) + (p4.z + p4.w);
            bf16x4t h4, m4, l4;
            split4(p4, h4, m4, l4);
            const int slot = (li * kTPP + 4 * wave + q) * 2 + hl;
            pw[slot] = h4;
            pw[kTR * kTPP * 2 + slot] = m4;
            pw[2 * kTR * kTPP * 2 + slot] = l4;
        }
        __syncthreads();  // the whole P tile is in LDS
        // 96 bytes per (16-column block, channel): 3 parts x 2 halves.
        const char *vblk =
            reinterpret_cast<const char *>(vb) + ((int64_t)cb * (kTN / 16) * dv_pad + c0) * 96;
        const unsigned voff = (unsigned)(li * 96 + hl * 16);
        // Step st = kc * NB + nb: the three parts of channel c0 + 32 nb + li,
        // columns 16 kc + 8 hl .. + 7; loaded kTVD steps ahead of their use.
        auto load_v = [&](int st, bf16x8t (&dst)[3]) __attribute__((always_inline)) {
            const int kc = st / NB, nb = st % NB;
            const char *u = vblk + ((int64_t)kc * dv_pad + 32 * nb) * 96;
            dst[0] = *reinterpret_cast<const bf16x8t *>(u + voff);
            dst[1] = *reinterpret_cast<const bf16x8t *>(u + voff + 32);
            dst[2] = *reinterpret_cast<const bf16x8t *>(u + voff + 64);
        };
        constexpr int NST = (kTN / 16) * NB;
        bf16x8t ring[kTVD + 1][3];
#pragma unroll
        for (int st = 0; st < kTVD; ++st)
            load_v(st, ring[st]);
        bf16x8t ph, pm, plo;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            // Keep each step's loads and products where they are written:
            // hoisted loads would hold every step's values at once.
            __builtin_amdgcn_sched_barrier(0);
            if (st + kTVD < NST)
                load_v(st + kTVD, ring[(st + kTVD) % (kTVD + 1)]);
            const int kc = st / NB, nb = st % NB;
            if (nb == 0) {
                const int slot = li * kTPP + 2 * kc + hl;
                ph = pp[slot];
                pm = pp[kTR * kTPP + slot];
                plo = pp[2 * kTR * kTPP + slot];
            }
            const bf16x8t vh = ring[st % (kTVD + 1)][0];
            const bf16x8t vm = ring[st % (kTVD + 1)][1];
            const bf16x8t vl = ring[st % (kTVD + 1)][2];
            floatx16 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                            0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vm, pm, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, ph, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, plo, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vm, ph, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, pm, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, ph, acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                O[nb][r] += acc[r];
        }
    };

    auto step = [&](int t, auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70 | kTLoads);  // vmcnt(kTLoads)
        __builtin_amdgcn_s_barrier();
        const float4 *buf = stg[b];
        half8 ah[2], al[2], bh[2], bl[2];
        const int rc = kTR + 32 * wave + li;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            al[c] = as_half8(buf[tslot(rc, 4 + 2 * c + hl)]);
            bh[c] = as_half8(buf[tslot(li, 2 * c + hl)]);
            ah[c] = as_half8(buf[tslot(rc, 2 * c + hl)]);
            bl[c] = as_half8(buf[tslot(li, 4 + 2 * c + hl)]);
        }
        issue(min(t + 2, T - 1), std::integral_constant<int, (b + 2) % 3>{});
        floatx16 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                        0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[0], bh[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0], bl[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[1], bh[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1], bl[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[0], bh[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[1], bh[1], acc, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v)
            sum[v] += acc[v];
        if (t % NS == NS - 1) {
            epilogue(biasb, bbeg + t / NS);
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sum[v] = 0.f;
        }
    };
    for (int t = 0; t < T; t += 3) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < T) {
            step(t + 1, std::integral_constant<int, 1>{});
            if (t + 2 < T)
                step(t + 2, std::integral_constant<int, 2>{});
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Lane l of wave w holds row l mod 32 and the channels
    // c0 + 32 nb + 8 (r / 4) + 4 (l / 32) + r mod 4 of its registers (nb, r).
    const int64_t i = row0 + li;
    if (i < rows) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k = c0 + 32 * nb + 8 * (r / 4) + 4 * hl + (r % 4);
                part[((int64_t)split * rows_pad + i) * dv_pad + k] = (double)O[nb][r];
            }
    }
    if (RSUM) {
        // Each lane summed its 16 columns of every block; the lane halves,
        // then the waves in order.
        float rs = rsum + __shfl_xor(rsum, 32);
        float *red = reinterpret_cast<float *>(st0);
        if (hl == 0)
            red[wave * 32 + li] = rs;
        __syncthreads();
        if (wave == 0 && hl == 0) {
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < kTW; ++w)
                tot += red[w * 32 + li];
            if (i < rows)
                rpart[(int64_t)split * rows_pad + i] = (double)tot;
        }
    }
}

// The values in three bf16 parts, in blocks of 16 columns: part p of
// v[16 jb + 8 h + k][c] (k < 8; 0 beyond m or dv) is element k of
// vb[((jb * dv_pad + c) * 3 + p) * 2 + h]. One thread per (jb, c, h).
__global__ __launch_bounds__(256) void values_split_kernel(const float *__restrict__ v,
                                                           int64_t m, int dv, int dv_pad,
                                                           int64_t m_pad,
                                                           bf16x8t *__restrict__ vb) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= m_pad / 8 * dv_pad)
        return;
    const int h = (int)(e & 1);
    const int c = (int)((e >> 1) % dv_pad);
    const int64_t jb = (e >> 1) / dv_pad;
    const int64_t j0 = jb * 16 + 8 * h;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        x[k] = (j0 + k < m && c < dv) ? v[(j0 + k) * dv + c] : 0.f;
    bf16x8t ph, pm, pl;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        bf16x2t xh, xm, xl;
        split2(float2t{x[k], x[k + 1]}, xh, xm, xl);
        ph[k] = xh[0];
        ph[k + 1] = xh[1];
        pm[k] = xm[0];
        pm[k + 1] = xm[1];
        pl[k] = xl[0];
        pl[k + 1] = xl[1];
    }
    bf16x8t *o = vb + ((jb * dv_pad + c) * 3) * 2 + h;
    o[0] = ph;
    o[2] = pm;
    o[4] = pl;
}

// out[i * dv + k] = sum over splits of part[s][i][k] (k < dv), in split order.
__global__ __launch_bounds__(256) void rows_reduce_kernel(const double *__restrict__ part,
                                                          int nsplit, int64_t rows,
                                                          int64_t rows_pad, int dv, int stride,
                                                          float *__restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= rows * dv)
        return;
    const int64_t i = e / dv;
    const int k = (int)(e % dv);
    double s = 0.0;
    for (int sp = 0; sp < nsplit; ++sp)
        s += part[((int64_t)sp * rows_pad + i) * stride + k];
    out[e] = (float)s;
}

struct RPlan {
    int nrb, nblocks, blocks_per_split, nsplit;
};

// One workgroup fits a CU (its LDS), so the launch runs in rounds of kTCUs
// workgroups. The split count is at least ceil(kTTargetBlocks / row blocks)
// (measured at 65536 rows and d = 512: one split 53.9 ms, two 48.2); from
// there up to twice that (at least 8) it takes the count with the fewest
// rounds x blocks per workgroup, the smaller on a tie (50000 rows x 196
// blocks: 7 splits, 43 rounds x 28 blocks; 2 splits took 63.0 ms, 7 55.4).
constexpr int64_t kTCUs = 256;

RPlan plan_rows(int64_t rows, int64_t cols_pad) {
    RPlan p;
    p.nrb = (int)((rows + kTR - 1) / kTR);
    p.nblocks = (int)(cols_pad / kTN);
    int64_t lo = (kTTargetBlocks + p.nrb - 1) / p.nrb;
    if (lo > p.nblocks)
        lo = p.nblocks;
    if (lo < 1)
        lo = 1;
    int64_t hi = 2 * lo < 8 ? 8 : 2 * lo;
    if (hi > p.nblocks)
        hi = p.nblocks;
    int64_t best = -1;
    p.blocks_per_split = p.nblocks;
    p.nsplit = 1;
    for (int64_t ns = lo; ns <= hi; ++ns) {
        const int64_t bps = (p.nblocks + ns - 1) / ns;
        const int64_t nsp = (p.nblocks + bps - 1) / bps;
        const int64_t cost = (p.nrb * nsp + kTCUs - 1) / kTCUs * bps;
        if (best < 0 || cost < best) {
            best = cost;
            p.blocks_per_split = (int)bps;
            p.nsplit = (int)nsp;
        }
    }
    return p;
}

int rows_channels(int dv) { return (dv + 255) / 256 * 256; }

size_t rows_partial_doubles(int64_t n, int64_t m_pad, int dv, bool rowsum) {
    const RPlan p = plan_rows(n, m_pad);
    const size_t d = (size_t)p.nsplit * (size_t)pad_points(n) *
                     (size_t)(rows_channels(dv) + (rowsum ? 1 : 0));
    return (d + 31) / 32 * 32;
}

template <int KP, int NB>
hipError_t launch_tr(const RPlan &p, const float4 *xr, const float *xhat, const float4 *col4,
                     const float *yhat, const bf16x8t *vb, int dv_pad, int64_t n, int64_t n_pad,
                     double *part, double *rpart, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)p.nrb * p.nsplit));
    if (rpart)
        hipLaunchKernelGGL((transport_rows_kernel<KP, NB, true>), grid, dim3(64 * kTW), 0, s, xr,
                           xhat, col4, yhat, vb, dv_pad, n, n_pad, p.nrb, p.blocks_per_split,
                           p.nblocks, part, rpart);
    else
        hipLaunchKernelGGL((transport_rows_kernel<KP, NB, false>), grid, dim3(64 * kTW), 0, s,
                           xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, p.nrb, p.blocks_per_split,
                           p.nblocks, part, rpart);
    return hipGetLastError();
}

template <int KP>
hipError_t launch_tr_nb(int nb, const RPlan &p, const float4 *xr, const float *xhat,
                        const float4 *col4, const float *yhat, const bf16x8t *vb, int dv_pad,
                        int64_t n, int64_t n_pad, double *part, double *rpart, hipStream_t s) {
    switch (nb) {
    case 1: return launch_tr<KP, 1>(p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s);
    case 2: return launch_tr<KP, 2>(p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s);
    case 3: return launch_tr<KP, 3>(p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s);
    case 4: return launch_tr<KP, 4>(p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t transport_rows_scratch_doubles(int64_t n, int64_t m_pad, int dv, bool rowsum) {
    const size_t vb = (size_t)m_pad * (size_t)rows_channels(dv) * 6;  // bytes, 3 bf16 parts
    return rows_partial_doubles(n, m_pad, dv, rowsum) + (vb + 7) / 8;
}

hipError_t launch_transport_rows(int kp, const void *xrow, const float *xhat, const void *ycol,
                                 const float *yhat, const float *v, int64_t n, int64_t n_pad,
                                 int64_t m, int64_t m_pad, int dv, double *part, float *out,
                                 float *rowsum, hipStream_t s) {
    const int dv_pad = rows_channels(dv);
    const int nb = dv_pad / 256;
    if (nb < 1 || nb > 4)
        return hipErrorInvalidValue;
    const RPlan p = plan_rows(n, m_pad);
    double *rpart = rowsum ? part + (size_t)p.nsplit * (size_t)n_pad * (size_t)dv_pad : nullptr;
    bf16x8t *vb = reinterpret_cast<bf16x8t *>(part + rows_partial_doubles(n, m_pad, dv, rowsum));
    {
        const int64_t total = m_pad / 8 * dv_pad;
        hipLaunchKernelGGL(values_split_kernel, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, s, v, m, dv, dv_pad, m_pad, vb);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const float4 *xr = static_cast<const float4 *>(xrow);
    const float4 *col4 = static_cast<const float4 *>(ycol);
    hipError_t e;
    switch (kp) {
    case 160: e = launch_tr_nb<160>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 192: e = launch_tr_nb<192>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 224: e = launch_tr_nb<224>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 256: e = launch_tr_nb<256>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 320: e = launch_tr_nb<320>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 384: e = launch_tr_nb<384>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 448: e = launch_tr_nb<448>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 512: e = launch_tr_nb<512>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 640: e = launch_tr_nb<640>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 768: e = launch_tr_nb<768>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 896: e = launch_tr_nb<896>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    case 1024: e = launch_tr_nb<1024>(nb, p, xr, xhat, col4, yhat, vb, dv_pad, n, n_pad, part, rpart, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(rows_reduce_kernel, dim3((unsigned)((n * dv + 255) / 256)), dim3(256), 0,
                       s, part, p.nsplit, n, n_pad, dv, dv_pad, out);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    if (rpart) {
        hipLaunchKernelGGL(rows_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           rpart, p.nsplit, n, n_pad, 1, 1, rowsum);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace otsk
