// Cosine cost after normalisation ("FlashSinkhorn: IO-Aware Entropic Optimal
// Transport on GPU", significance section: the streaming method applies to
// the squared Euclidean cost and to the cosine distance once the points are
// normalised). On unit vectors 1 - cos(x, y) = |x - y|^2 / 2, so
//   exp((f + g - (1 - cos))/eps) = exp((2f + 2g - |x^ - y^|^2)/(2 eps)):
// the cosine problem at eps is the squared Euclidean problem on the
// normalised points at 2 eps with potentials 2f, 2g. These kernels
// normalise the points and scale the potentials; the squared Euclidean
// kernels do the rest.
#include "ot_internal.h"

#include <math.h>

namespace otsk {

namespace {

// out_i = p_i / |p_i| (norm in fp64); one thread per point.
__global__ __launch_bounds__(256) void normalize_kernel(const float *__restrict__ pts,
                                                        int64_t count, int d,
                                                        float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count)
        return;
    const float *p = pts + i * d;
    double s = 0.0;
    for (int k = 0; k < d; ++k)
        s = fma((double)p[k], (double)p[k], s);
    const double inv = 1.0 / sqrt(s);
    for (int k = 0; k < d; ++k)
        out[i * d + k] = (float)((double)p[k] * inv);
}

__global__ __launch_bounds__(256) void scale_kernel(const float *__restrict__ in, int64_t count,
                                                    float s, float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        out[i] = in[i] * s;
}

__global__ void scale_double_kernel(double *v, double s) { *v *= s; }

}  // namespace

hipError_t launch_normalize(const float *pts, int64_t count, int d, float *out, hipStream_t s) {
    hipLaunchKernelGGL(normalize_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                       pts, count, d, out);
    return hipGetLastError();
}

hipError_t launch_scale(const float *in, int64_t count, float factor, float *out, hipStream_t s) {
    hipLaunchKernelGGL(scale_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, in,
                       count, factor, out);
    return hipGetLastError();
}

hipError_t launch_scale_double(double *v, double factor, hipStream_t s) {
    hipLaunchKernelGGL(scale_double_kernel, dim3(1), dim3(1), 0, s, v, factor);
    return hipGetLastError();
}

}  // namespace otsk
