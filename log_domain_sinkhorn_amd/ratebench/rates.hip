// Instruction-rate microbenchmarks of gfx950, used by the benchmark to turn
// per-pair operation counts into ALU and matrix-core ceilings measured on
// the GPU it runs on (not part of the solver library).
//
// Each kernel keeps 8 independent dependency chains per lane (enough to
// hide the instruction latencies) over 8 waves per CU-slot of a grid of
// 2048 workgroups of 256 lanes, and stores its chains so nothing is removed.
// The rates are lane-operations (or matrix flops) per second of the whole
// chip at whatever clock it holds under that stream:
//   0  v_fma_f32                 v = v * a + b
//   1  v_exp_f32                 v = 2^(-|v|)          (stays in (0, 1])
//   2  v_log_f32                 v = log2(|v| + 1)
//   3  v_exp_f32 on 8 chains and v_fma_f32 on 8 other chains, interleaved
//      (does exp issue beside FMA? at the sum of the two costs it does not)
//   4  v_fma_f64                 w = w * a + w (a = -2^-10: decays, no denormals)
//   5  v_mfma_f32_32x32x16_f16   f16 matrix-core flops (4 accumulators)
//   6  v_mfma_f32_32x32x2f32     fp32 matrix-core flops (4 accumulators)
//   7  v_add_f32                 v = v + c
//   8  v_mfma_f32_32x32x16_f16   as 5, but with operands of random f16
//                                mantissas in +-[1, 2) whose bits change every
//                                step, run long enough (~0.4 s) for the board's
//                                power management to settle: the matrix-core
//                                rate a data-carrying f16 product sustains
// Lane 0 of every workgroup also reads the shader-clock counter and the
// constant-rate wall counter when it starts and ends, so the average shader
// clock under each stream is known and the rates can be put per clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;
constexpr int kBlocks = 2048;
constexpr int kThreads = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Clock readings of lane 0 of a workgroup: (shader cycles, wall ticks).
__device__ __forceinline__ void clock_mark(long long *clk, int slot) {
    if (threadIdx.x == 0) {
        clk[4 * blockIdx.x + 2 * slot] = clock64();
        clk[4 * blockIdx.x + 2 * slot + 1] = wall_clock64();
    }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_rate_kernel(int iters, float *out,
                                                             long long *clk) {
    clock_mark(clk, 0);
    const int tid = blockIdx.x * kThreads + threadIdx.x;
    float v[kChains], u[kChains];
    double w[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        v[k] = 0.25f + 0.01f * (float)((tid + k) & 31);
        u[k] = v[k] + 0.5f;
        w[k] = (double)v[k];
    }
    const float a = 0.9990234375f, b = 0.0009765625f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) {
            if (KIND == 0)
                v[k] = fmaf(v[k], a, b);
            else if (KIND == 1)
                v[k] = __builtin_amdgcn_exp2f(-fabsf(v[k]));
            else if (KIND == 2)
                v[k] = __builtin_amdgcn_logf(fabsf(v[k]) + 1.0f);
            else if (KIND == 3) {
                v[k] = __builtin_amdgcn_exp2f(-fabsf(v[k]));
                u[k] = fmaf(u[k], a, b);
            } else if (KIND == 7)
                v[k] = v[k] + b;
            else
                w[k] = fma(w[k], -0x1p-10, w[k]);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k)
        s += v[k] + u[k] + (float)w[k];
    out[tid] = s;
    clock_mark(clk, 1);
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(int iters, float *out,
                                                             long long *clk) {
    clock_mark(clk, 0);
    const int tid = blockIdx.x * kThreads + threadIdx.x;
    floatx16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[c][r] = 0.f;
    half8 ah, bh;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        ah[r] = (_Float16)(0.001f * (float)((tid + r) & 7));
        bh[r] = (_Float16)(0.002f * (float)((tid + 2 * r) & 7));
    }
    // KIND 8: xorshift32 bits with the exponent fixed (halves in +-[1, 2)).
    u32x4 ua, ub;
    unsigned x = (unsigned)tid * 2654435761u + 12345u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        x ^= x << 13; x ^= x >> 17; x ^= x << 5;
        ua[r] = (x & 0x83FF83FFu) | 0x3C003C00u;
        x ^= x << 13; x ^= x >> 17; x ^= x << 5;
        ub[r] = (x & 0x83FF83FFu) | 0x3C003C00u;
    }
    const float af = 0.001f * (float)(tid & 7), bf = 0.002f * (float)(tid & 3);
    for (int i = 0; i < iters; ++i) {
        if (KIND == 8) {
            const unsigned flip = (0x02AB02ABu * (unsigned)((i & 7) + 1)) & 0x03FF03FFu;
            ua ^= flip;
            ub ^= flip >> 1;
            ah = __builtin_bit_cast(half8, ua);
            bh = __builtin_bit_cast(half8, ub);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (KIND == 5 || KIND == 8)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[c], 0, 0, 0);
            else
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(af, bf, acc[c], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s += acc[c][r];
    out[tid] = s;
    clock_mark(clk, 1);
}

}  // namespace

extern "C" {

// Measure rate `kind` (table above) with `iters` chain steps per lane; writes
// operations per second to *rate and the average shader clock of the
// workgroups (Hz) to *clock_hz. Returns 0 or the HIP error code.
int otr_measure(int kind, int iters, double *rate, double *clock_hz) {
    if (kind < 0 || kind > 8 || iters < 1 || !rate || !clock_hz)
        return (int)hipErrorInvalidValue;
    int dev = 0, wall_khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess)
        return (int)e;
    float *out = nullptr;
    long long *clk = nullptr;
    e = hipMalloc(&out, sizeof(float) * kBlocks * kThreads);
    if (e == hipSuccess)
        e = hipMalloc(&clk, sizeof(long long) * 4 * kBlocks);
    if (e != hipSuccess) {
        (void)hipFree(out);
        return (int)e;
    }
    hipEvent_t t0, t1;
    (void)hipEventCreate(&t0);
    (void)hipEventCreate(&t1);
    float ms = 0.f;
    for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {  // rep 0 warms up
        (void)hipEventRecord(t0, nullptr);
        const dim3 g(kBlocks), b(kThreads);
        switch (kind) {
        case 0: hipLaunchKernelGGL(valu_rate_kernel<0>, g, b, 0, nullptr, iters, out, clk); break;
        case 1: hipLaunchKernelGGL(valu_rate_kernel<1>, g, b, 0, nullptr, iters, out, clk); break;
        case 2: hipLaunchKernelGGL(valu_rate_kernel<2>, g, b, 0, nullptr, iters, out, clk); break;
        case 3: hipLaunchKernelGGL(valu_rate_kernel<3>, g, b, 0, nullptr, iters, out, clk); break;
        case 4: hipLaunchKernelGGL(valu_rate_kernel<4>, g, b, 0, nullptr, iters, out, clk); break;
        case 5: hipLaunchKernelGGL(mfma_rate_kernel<5>, g, b, 0, nullptr, iters, out, clk); break;
        case 6: hipLaunchKernelGGL(mfma_rate_kernel<6>, g, b, 0, nullptr, iters, out, clk); break;
        case 8: hipLaunchKernelGGL(mfma_rate_kernel<8>, g, b, 0, nullptr, iters, out, clk); break;
        default: hipLaunchKernelGGL(valu_rate_kernel<7>, g, b, 0, nullptr, iters, out, clk); break;
        }
        e = hipGetLastError();
        (void)hipEventRecord(t1, nullptr);
        if (e == hipSuccess)
            e = hipEventSynchronize(t1);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, t0, t1);
    }
    long long *h = new long long[4 * kBlocks];
    if (e == hipSuccess)
        e = hipMemcpy(h, clk, sizeof(long long) * 4 * kBlocks, hipMemcpyDeviceToHost);
    (void)hipEventDestroy(t0);
    (void)hipEventDestroy(t1);
    (void)hipFree(out);
    (void)hipFree(clk);
    if (e != hipSuccess) {
        delete[] h;
        return (int)e;
    }
    double cycles = 0.0, ticks = 0.0;
    for (int blk = 0; blk < kBlocks; ++blk) {
        cycles += (double)(h[4 * blk + 2] - h[4 * blk]);
        ticks += (double)(h[4 * blk + 3] - h[4 * blk + 1]);
    }
    delete[] h;
    *clock_hz = ticks > 0.0 ? cycles / ticks * (double)wall_khz * 1e3 : 0.0;
    const double lanes = (double)kBlocks * kThreads;
    double ops;
    if (kind <= 4 || kind == 7)
        ops = lanes * iters * kChains * (kind == 3 ? 2.0 : 1.0);
    else  // per wave and instruction: 32*32*16*2 (f16) or 32*32*2*2 (fp32) flops
        ops = (lanes / 64.0) * iters * 4.0 * (kind == 6 ? 4096.0 : 32768.0);
    *rate = ops / (ms / 1e3);
    return 0;
}

}  // extern "C"
