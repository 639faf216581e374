// Device helpers shared by the MFMA kernels (the half-steps and the
// transport application): tile copies with gfx950's direct global->LDS
// loads, the 32x32 score tile with the bias and a per-row offset folded into
// one extra v_mfma_f32_32x32x2f32, and the lazy online log-sum-exp epilogue
// over the 16 accumulator values a lane holds.
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

// u[j][i] = s_ij - Mu_i for the 32 columns of subtile `sub`: the extra MFMA
// (bias and -Mu) on a zero accumulator, then KP/2 MFMAs over k.
template <int KP>
__device__ __forceinline__ floatx16 score_tile(const float4 *rec, const float *bias, int sub,
                                               int lane, int li, int hl, const float (&bx)[KP / 2],
                                               float Mu) {
    constexpr int RS4 = (KP + 4) / 4;
    constexpr int KH = KP / 2;
    const floatx16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                           0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float a0 = bias[sub * 64 + lane];
    const float b0 = hl ? -Mu : 1.f;
    floatx16 acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, zero, 0, 0, 0);
    const float4 *ap = rec + (sub * 32 + li) * RS4 + hl * (KH / 4);
#pragma unroll
    for (int q4 = 0; q4 < KH / 4; ++q4) {
        const float4 av = ap[q4];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bx[4 * q4 + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bx[4 * q4 + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bx[4 * q4 + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bx[4 * q4 + 3], acc, 0, 0, 0);
    }
    return acc;
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

}  // namespace mfma
}  // namespace otsk
