// The stage pipeline of the kernels tiled like a matrix product: the
// half-step and the plan statistics for 448 < d <= 1024 (lse_gemm.hip).
//
// A workgroup of 8 waves owns 128 RS rows (RS = 1 or 2 row subtiles of 32
// per wave) and walks its column split in blocks of 128 columns. For each
// block the coordinates go through LDS in stages of 32 (the block's row and
// column records' 4 hi and 4 lo 16-byte chunks of that stage), three stages
// deep, filled by gfx950's direct global->LDS loads two stages ahead of the
// one being multiplied. Wave (rw, cw) = (wave mod 4, wave / 4) forms the
// block of rows 32 RS rw .. 32 RS rw + 32 RS - 1 and columns 64 cw .. 64 cw
// + 63 as RS x 2 v_mfma_f32_32x32x16_f16 subtiles (D[j][i]: lane l holds row
// l mod 32 and 16 columns j = 8 (v / 4) + 4 (l / 32) + v mod 4 of its
// registers v, as in lse_h3.hip). Per stage and subtile the chain starts
// from zero, takes the lo corrections of both 16-coordinate chunks and then
// the hi x hi products, and is added to an fp32 running sum: the matrix
// core's aligned sum loses about 2^-21 of its largest term, so no chain may
// grow past one stage's share of the dot product. After the last stage of a
// block the sums go to the caller's block epilogue.
#pragma once

#include "mfma_common.h"

#include <type_traits>

namespace otsk {
namespace gemm {

using namespace mfma;

constexpr int kGW = 8;                    // waves per workgroup
constexpr int kGBN = 128;                 // columns per column block
constexpr int kGKS = 32;                  // coordinates per stage
constexpr int kGTail4 = 2 * kGBN / 4;     // behind the records: biases, norms
constexpr int kGTargetBlocks = 2048;
constexpr int kGColLoads = kGBN * 8 / 64 / kGW;  // column loads per wave and stage

// Sizes for RS row subtiles per wave.
template <int RS>
struct GTile {
    static constexpr int BM = 128 * RS;                      // rows per workgroup
    static constexpr int Stage4 = (BM + kGBN) * 8;           // 16-byte chunks per stage
    static constexpr int RowLoads = BM * 8 / 64 / kGW;       // per wave and stage
    static constexpr int Loads = RowLoads + kGColLoads;      // direct loads per wave and stage
    static_assert(Stage4 == Loads * 64 * kGW, "every slot loaded once");
};

// LDS slot of logical chunk t (0-3 hi, 4-7 lo) of stage record r. The XOR
// keeps the 16-byte reads of 8 (and of 16) consecutive lanes, which take
// consecutive records, on distinct banks.
__device__ __forceinline__ int gslot(int r, int t) { return r * 8 + (t ^ ((r ^ (r >> 3)) & 7)); }

// Workgroup L -> (row block, column split) over nmap row blocks: the splits
// of row block rb run on XCD rb mod 8 when nmap is a multiple of 8 (the grid
// then rounds the row-block count up to it), otherwise in split-minor order,
// so that a block's row records, re-read for every column block, stay in
// one XCD's L2. Returns false for the rounding's extra workgroups (rb >= nrb).
__device__ __forceinline__ bool gemm_block(int nmap, int nrb, int nsplit, int &rb, int &split) {
    const int L = (int)blockIdx.x;
    if (nmap % 8 == 0) {
        const int q = L / 8;
        split = q % nsplit;
        rb = (q / nsplit) * 8 + L % 8;
    } else {
        split = L % nsplit;
        rb = L / nsplit;
    }
    return rb < nrb;
}

// Issue the direct loads of stage s of column block cb into `buf`. Stage
// record r (the BM rows, then the columns) fills slots 8r .. 8r + 7; slot
// 8r + p holds logical chunk t = p ^ ((r ^ (r >> 3)) & 7) (the read swizzle
// of gslot). Each 64-lane load fills 64 consecutive slots, i.e. 8 records:
// wave w issues row loads RowLoads w .. RowLoads (w + 1) - 1 and column
// loads 2w, 2w + 1, so lane l of load g serves record 8g + l/8 and position
// l mod 8. Column records carry the global layout's chunk swizzle (16-byte
// chunk q of point j at q ^ (j & SW), SW = swizzle_mask(KP / 4); column
// blocks start at multiples of 128, so j & SW is the record's index in the
// block, masked); row records are unswizzled. Above kStagedRecordKP both
// sides' records are staged (a stage's 8 chunks side by side at 8s .. 8s + 7,
// unswizzled), so a record's stage is one 128-byte line. With the last stage
// of a block, waves 0 and 1 also load the block's 128 column biases behind
// the stage's records, where the block's epilogue reads them, and with NRM
// waves 2 and 3 the columns' squared norms after those.
template <int KP, bool NRM, int RS>
__device__ __forceinline__ void issue_stage(const float4 *__restrict__ row4,
                                            const float4 *__restrict__ col4,
                                            const float *__restrict__ colb,
                                            const float *__restrict__ coln, int64_t row0,
                                            int64_t col0, int s, bool last, float4 *buf,
                                            int wave, int lane) {
    using G = GTile<RS>;
    constexpr int RC = KP / 4;
    const int lr = lane >> 3, lp = lane & 7;
#pragma unroll
    for (int k = 0; k < G::RowLoads; ++k) {
        const int g = wave * G::RowLoads + k;
        const int t = lp ^ ((lr ^ g) & 7);
        const int q = KP > kStagedRecordKP ? 8 * s + t : (t < 4 ? 0 : KP / 8) + 4 * s + (t & 3);
        __builtin_amdgcn_global_load_lds(row4 + (row0 + g * 8 + lr) * RC + q,
                                         (lds_void *)(buf + g * 64), 16, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kGColLoads; ++k) {
        const int g = wave * kGColLoads + k;
        const int rl = g * 8 + lr;  // column within the block
        const int t = lp ^ ((lr ^ g) & 7);
        const int q = KP > kStagedRecordKP
                          ? 8 * s + t
                          : ((t < 4 ? 0 : KP / 8) + 4 * s + (t & 3)) ^ (rl & swizzle_mask(RC));
        __builtin_amdgcn_global_load_lds(col4 + (col0 + rl) * RC + q,
                                         (lds_void *)(buf + G::BM * 8 + g * 64), 16, 0, 0);
    }
    if (last && wave < kGBN / 64)
        __builtin_amdgcn_global_load_lds(
            colb + col0 + wave * 64 + lane,
            (lds_void *)(reinterpret_cast<float *>(buf + G::Stage4) + wave * 64), 4, 0, 0);
    if (NRM && last && wave >= kGBN / 64 && wave < kGBN / 32)
        __builtin_amdgcn_global_load_lds(
            coln + col0 + (wave - kGBN / 64) * 64 + lane,
            (lds_void *)(reinterpret_cast<float *>(buf + G::Stage4) + kGBN +
                         (wave - kGBN / 64) * 64),
            4, 0, 0);
}

// The wave's operands of one stage: hi and lo chunks of both 16-coordinate
// k-steps for its two column subtiles (a) and RS row subtiles (b).
template <int RS>
struct StageOps {
    half8 ah[2][2], al[2][2], bh[RS][2], bl[RS][2];
};

template <int RS>
__device__ __forceinline__ void stage_operands(const float4 *buf, int rw, int cw, int li, int hl,
                                               StageOps<RS> &o) {
    // In the order the chains consume them: the first layer's operands
    // (lo of the columns, hi of the rows, k-step 0) first.
    int rc[2], rr[RS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
        rc[u] = GTile<RS>::BM + 64 * cw + 32 * u + li;
#pragma unroll
    for (int u = 0; u < RS; ++u)
        rr[u] = 32 * RS * rw + 32 * u + li;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            o.al[u][c] = as_half8(buf[gslot(rc[u], 4 + 2 * c + hl)]);
            if (u < RS)
                o.bh[u][c] = as_half8(buf[gslot(rr[u], 2 * c + hl)]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            o.ah[u][c] = as_half8(buf[gslot(rc[u], 2 * c + hl)]);
            if (u < RS)
                o.bl[u][c] = as_half8(buf[gslot(rr[u], 4 + 2 * c + hl)]);
        }
    }
}

// One stage of the wave's RS x 2 subtiles: chains from zero (corrections,
// then hi x hi) added to the fp32 sums. The chains advance together, one
// product each in turn, on their own accumulators; layers [l0, l1) of the
// six (al0.bh0, ah0.bl0, al1.bh1, ah1.bl1, ah0.bh0, ah1.bh1).
template <int L0, int L1, int RS>
__device__ __forceinline__ void stage_layers(const StageOps<RS> &o, floatx16 (&acc)[RS][2]) {
#pragma unroll
    for (int l = L0; l < L1; ++l) {
        const int c = (l == 0 || l == 1 || l == 4) ? 0 : 1;
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                const half8 a = (l == 0 || l == 2) ? o.al[cs][c] : o.ah[cs][c];
                const half8 b = (l == 1 || l == 3) ? o.bl[rs][c] : o.bh[rs][c];
                acc[rs][cs] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    a, b,
                    l == 0 ? floatx16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                                      0.f, 0.f, 0.f, 0.f}
                           : acc[rs][cs],
                    0, 0, 0);
            }
    }
}

template <int RS>
__device__ __forceinline__ void add_sums(const floatx16 (&acc)[RS][2], floatx16 (&sum)[RS][2]) {
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sum[rs][cs][v] += acc[rs][cs][v];
}

// The stage pipeline of one workgroup: column blocks bbeg .. bend - 1 of its
// split against its BM rows; after the last stage of each block,
// epi(bias, nrm, sum) consumes the block (bias and norms in LDS) and the
// sums restart from zero. st0 .. st2 are three separate __shared__ arrays of
// at least GTile<RS>::Stage4 + kGTail4 chunks: each gets its own alias
// scope, so the compiler sees that reading stage t does not wait for the
// direct loads into the other two buffers. Returns with every load landed
// and the workgroup synchronised.
template <int KP, bool NRM, int RS, class Epi>
__device__ __forceinline__ void gemm_stream(float4 *st0, float4 *st1, float4 *st2,
                                            const float4 *row4, const float4 *col4,
                                            const float *colb, const float *coln, int64_t row0,
                                            int bbeg, int bend, int wave, int lane, Epi &&epi) {
    using G = GTile<RS>;
    constexpr int NS = KP / kGKS;  // stages per column block
    static_assert(KP % kGKS == 0 && NS >= 2, "whole stages, at least two per block");
    float4 *const stg[3] = {st0, st1, st2};
    const int rw = wave & 3;
    const int cw = wave >> 2;
    const int hl = lane >> 5;
    const int li = lane & 31;
    const int T = (bend - bbeg) * NS;  // stages of this workgroup (>= NS)

    auto issue = [&](int t, auto bc) {
        constexpr int b = decltype(bc)::value;
        const int cb = bbeg + t / NS;
        issue_stage<KP, NRM, RS>(row4, col4, colb, coln, row0, (int64_t)cb * kGBN, t % NS,
                                 t % NS == NS - 1, stg[b], wave, lane);
    };
    issue(0, std::integral_constant<int, 0>{});
    issue(1, std::integral_constant<int, 1>{});

    floatx16 sum[RS][2];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sum[rs][cs][v] = 0.f;

    // Stage t: wait for its loads (those of stage t + 1, issued later, may
    // still be in flight), then the barrier makes every wave's loads
    // visible and tells that every wave is done with stage t - 1, whose
    // buffer then takes stage t + 2. A bare s_barrier: the direct loads are
    // ordered by the explicit vmcnt wait, and __syncthreads()'s fence would
    // wait for the loads of stage t + 1 as well. Every step issues one
    // stage (past the end, a reload of the last one into the free buffer,
    // never read), so the count of loads behind stage t is always the same
    // and the compiler adds no wait of its own before the LDS reads.
    auto step = [&](int t, auto bc) {
        constexpr int b = decltype(bc)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70 | G::Loads);  // vmcnt(Loads)
        __builtin_amdgcn_s_barrier();
        StageOps<RS> o;
        stage_operands<RS>(stg[b], rw, cw, li, hl, o);
        issue(min(t + 2, T - 1), std::integral_constant<int, (b + 2) % 3>{});
        floatx16 acc[RS][2];
        stage_layers<0, 6, RS>(o, acc);
        add_sums<RS>(acc, sum);
        if (t % NS == NS - 1) {
            const float *tail = reinterpret_cast<const float *>(stg[b] + G::Stage4);
            epi(tail, tail + kGBN, sum);
#pragma unroll
            for (int rs = 0; rs < RS; ++rs)
#pragma unroll
                for (int cs = 0; cs < 2; ++cs)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        sum[rs][cs][v] = 0.f;
        }
    };
    for (int t = 0; t < T; t += 3) {
        // Nested, so that no path reaches step t + 2 without step t + 1.
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < T) {
            step(t + 1, std::integral_constant<int, 1>{});
            if (t + 2 < T)
                step(t + 2, std::integral_constant<int, 2>{});
        }
    }
    // The last reloads land before the caller reuses stage buffer 0.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Grid of a pass: the row-block count rounded up to a multiple of 8 when
// there are at least 8, so that the XCD order of gemm_block applies, times
// the column splits. One workgroup fits a CU, so the grid runs in rounds of
// 256 workgroups (the padded rows' workgroups included); the split count is
// the one between ceil(kGTargetBlocks / row blocks) and twice that (at least
// 8) with the fewest rounds x blocks per workgroup, the smaller on a tie. At
// 50000 rows x 392 blocks that is 14 splits (11 rounds x 28 blocks): 14.8 ms
// per half-step at d = 1024, against 15.6 with 11 splits (9 rounds x 36).
struct GPlan {
    int nblocks;
    int blocks_per_split;
    int nsplit;
    int64_t row_blocks;
    int64_t row_map;  // row blocks of the grid's mapping (>= row_blocks)
};

inline GPlan plan_gemm(int64_t rows, int64_t cols_pad, int bm) {
    GPlan p;
    p.nblocks = (int)(cols_pad / kGBN);
    p.row_blocks = (rows + bm - 1) / bm;
    p.row_map = p.row_blocks >= 8 ? (p.row_blocks + 7) / 8 * 8 : p.row_blocks;
    int64_t lo = (kGTargetBlocks + p.row_blocks - 1) / p.row_blocks;
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
        const int64_t cost = (p.row_map * nsp + 255) / 256 * bps;
        if (best < 0 || cost < best) {
            best = cost;
            p.blocks_per_split = (int)bps;
            p.nsplit = (int)nsp;
        }
    }
    return p;
}

}  // namespace gemm
}  // namespace otsk
