// Device helpers shared by the matrix-core kernels (the half-steps, the plan
// statistics and the transport application): tile copies with gfx950's
// direct global->LDS loads, the 32x32 split-f16 score tile with the bias and
// a per-row offset folded into one extra v_mfma_f32_32x32x2f32, and the lazy
// online log-sum-exp epilogue over the 16 accumulator values a lane holds.
#pragma once

#include "ot_internal.h"

namespace otsk {
namespace mfma {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }


// Start the copy of column tile t into LDS buffers (rec, bias). Coordinates:
// whole 64-lane chunks of 16 bytes; lane l lands 16 bytes after lane l-1 at
// the wave-uniform chunk base. Biases: two 32-lane dword loads, one per
// subtile, each into the first half of that subtile's slot pair.
template <int TILE4, int WAVES, int SUB>
__device__ __forceinline__ void issue_tile(const float4 *__restrict__ col4,
                                           const float *__restrict__ colb, int t, float4 *rec,
                                           float *bias, int wave, int lane) {
    const float4 *src = col4 + (int64_t)t * TILE4;
#pragma unroll
    for (int c = 0; c < TILE4 / 64; c += WAVES) {
        const int chunk = c + wave;
        if (TILE4 / 64 % WAVES == 0 || chunk < TILE4 / 64)
            __builtin_amdgcn_global_load_lds(src + chunk * 64 + lane,
                                             (lds_void *)(rec + chunk * 64), 16, 0, 0);
    }
    if (wave >= WAVES - SUB && lane < 32) {
        const int sub = wave - (WAVES - SUB);
        __builtin_amdgcn_global_load_lds(colb + (int64_t)t * (32 * SUB) + sub * 32 + lane,
                                         (lds_void *)(bias + sub * 64), 4, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// Split-f16 score tile. Each fp32 coordinate is hi + lo, hi = f16(v),
// lo = f16(v - hi); the column record holds the 2*KP halves of
// (2 log2(e)/eps) q 2^-e (hi chunks then lo chunks, 16-byte chunk q of point
// j stored at q ^ (j & SW)), the row side holds p 2^e's hi and lo parts as
// the stationary B operands. p.q ~ ph.qh + pl.qh + ph.ql.
// ---------------------------------------------------------------------------
// Swizzle mask of a record of RC 16-byte chunks (RC a multiple of 8).
__host__ __device__ constexpr int swizzle_mask(int rc) { return rc % 16 == 0 ? 15 : 7; }

__device__ __forceinline__ half8 as_half8(float4 v) { return __builtin_bit_cast(half8, v); }

// The chain alone: D[j][i] = p_i.q_j (scaled) for the column record ap of
// column j (swizzle sw) against the stationary row operands bh, bl.
//
// Order of the chain. The f16 MFMA adds its 16 products and the accumulator
// in one aligned sum whose error is about 2^-21 of the largest term
// (measured on gfx950; a lone product is exact), so the accumulator should be
// small while the products go in: first the lo corrections (2^-11 of the
// rest), then the hi x hi products onto them, and the bias and -M last (in
// score_h3), through the fp32 MFMA, whose sum is rounded like fp32
// arithmetic.
template <int KP>
__device__ __forceinline__ floatx16 split_dot(const float4 *ap, int sw, int hl,
                                              const half8 (&bh)[KP / 16],
                                              const half8 (&bl)[KP / 16]) {
    floatx16 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                    0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (KP <= 128) {
        half8 qh[KP / 16];
#pragma unroll
        for (int c = 0; c < KP / 16; ++c) {
            qh[c] = as_half8(ap[(2 * c + hl) ^ sw]);
            const half8 ql = as_half8(ap[(KP / 8 + 2 * c + hl) ^ sw]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ql, bh[c], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qh[c], bl[c], acc, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < KP / 16; ++c)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qh[c], bh[c], acc, 0, 0, 0);
    } else {
        // Above KP = 128 the hi operands are read from LDS a second time for
        // the hi x hi products instead of being held: KP/4 more registers do
        // not fit beside the stationary row operands (KP/2 registers). Up to
        // KP = 192 the kernels then compile without register spills; at 224
        // and 256 they would spill, so the point-cloud calls stop at 192.
#pragma unroll
        for (int c = 0; c < KP / 16; ++c) {
            const half8 ql = as_half8(ap[(KP / 8 + 2 * c + hl) ^ sw]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ql, bh[c], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_half8(ap[(2 * c + hl) ^ sw]), bl[c],
                                                         acc, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < KP / 16; ++c)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_half8(ap[(2 * c + hl) ^ sw]), bh[c],
                                                         acc, 0, 0, 0);
    }
    return acc;
}

// u[j][i] = s_ij - Mu_i for subtile `sub` of the tile in `rec` / `bias`.
template <int KP>
__device__ __forceinline__ floatx16 score_h3(const float4 *rec, const float *bias, int sub,
                                             int lane, int li, int hl, const half8 (&bh)[KP / 16],
                                             const half8 (&bl)[KP / 16], float Mu) {
    constexpr int RC = KP / 4;
    constexpr int SW = swizzle_mask(RC);
    const int j = sub * 32 + li;
    const floatx16 acc = split_dot<KP>(rec + j * RC, j & SW, hl, bh, bl);
    const float a0 = bias[sub * 64 + lane];
    const float b0 = hl ? -Mu : 1.f;
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc, 0, 0, 0);
}

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
        // A NaN sum (from NaN inputs) stays NaN.
        S = S == 0.f ? 0.f : S * hw_exp2(M - Mn);
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

}  // namespace mfma
}  // namespace otsk
