// Host side of the C ABI declared in include/ot_sinkhorn.h: argument checks,
// stream-ordered scratch, and the launch sequence of each call.
#include "ot_sinkhorn.h"
#include "ot_internal.h"

#include <math.h>
#include <stdint.h>

namespace otsk {

Layout choose_layout(int d) {
    Layout L;
    L.d = d;
    if (d < 32) {
        // VALU kernels: coordinates padded to 4k-1 so coordinates + bias fill
        // whole float4s (d = 3: one 16-byte record).
        L.kp = (d + 1 + 3) / 4 * 4 - 1;
        L.rs = L.kp + 1;
        L.mfma = false;
        L.f64 = true;
    } else {
        // MFMA kernels: coordinates padded to a multiple of 16 (each lane
        // half reads KP/2 floats as whole float4s); bias at KP; stride KP + 4.
        L.kp = (d + 15) / 16 * 16;
        L.rs = L.kp + 4;
        L.mfma = true;
        L.f64 = false;
    }
    return L;
}

}  // namespace otsk

using namespace otsk;

namespace {

ot_status map_error(hipError_t e) {
    if (e == hipSuccess)
        return OT_SUCCESS;
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
        return OT_ERROR_OUT_OF_MEMORY;
    return OT_ERROR_LAUNCH_FAILURE;
}

bool overlaps(const void *p, size_t pb, const void *q, size_t qb) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + qb && b < a + pb;
}

bool finite_pos(float v) { return isfinite(v) && v > 0.f; }

// Arguments every point-cloud call shares. Invalid values first, then
// what is valid but not supported.
ot_status check_clouds(const float *x, const float *y, int64_t n, int64_t m, int32_t d,
                       float eps) {
    if (!x || !y || n < 1 || m < 1 || d < 1 || !finite_pos(eps))
        return OT_ERROR_INVALID_VALUE;
    return OT_SUCCESS;
}

ot_status check_supported(int64_t n, int64_t m, int32_t d) {
    if (d > OT_MAX_DIM)
        return OT_ERROR_NOT_SUPPORTED;
    // 64-bit index arithmetic everywhere; keep point counts well inside it.
    if (n > ((int64_t)1 << 40) || m > ((int64_t)1 << 40))
        return OT_ERROR_NOT_SUPPORTED;
    return OT_SUCCESS;
}

// A block of device scratch memory taken and released on the call's stream.
struct Scratch {
    void *ptr = nullptr;
    hipStream_t s;
    explicit Scratch(hipStream_t st) : s(st) {}
    hipError_t alloc(size_t bytes) { return hipMallocAsync(&ptr, bytes < 256 ? 256 : bytes, s); }
    ~Scratch() {
        if (ptr)
            (void)hipFreeAsync(ptr, s);
    }
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// d >= 32: split-f16 matrix-core half-steps. Per side: column record and row
// record (4*kp bytes per point each), |p|^2 and the fp32 bias.
ot_status run_schedule_h3(const float *x, const float *y, const float *a, const float *b,
                          int64_t n, int64_t m, int32_t d, const double *eps_list, int stages,
                          int iters, float *f, float *g, hipStream_t s) {
    const int kp = h3_kp(d);
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    size_t part = half_step_partials_h3(n, m_pad, kp);
    const size_t part2 = half_step_partials_h3(m, n_pad, kp);
    if (part2 > part)
        part = part2;
    const size_t xr = align_up((size_t)n_pad * 4 * kp, 256);
    const size_t yr = align_up((size_t)m_pad * 4 * kp, 256);
    const size_t xv = align_up((size_t)n_pad * sizeof(float), 256);
    const size_t yv = align_up((size_t)m_pad * sizeof(float), 256);
    const size_t pb = align_up(part * sizeof(Partial), 256);
    const size_t mb = align_up(h3_maxabs_floats() * sizeof(float), 256);
    const size_t cb = align_up(h3_center_scratch_bytes(d), 256);
    Scratch sc(s);
    hipError_t e = sc.alloc(2 * xr + 2 * yr + 2 * xv + 2 * yv + pb + mb + cb);
    if (e != hipSuccess)
        return map_error(e);
    char *p = static_cast<char *>(sc.ptr);
    void *xcol = p, *xrow = p + xr;
    p += 2 * xr;
    void *ycol = p, *yrow = p + yr;
    p += 2 * yr;
    float *xnrm = reinterpret_cast<float *>(p), *xbias = reinterpret_cast<float *>(p + xv);
    p += 2 * xv;
    float *ynrm = reinterpret_cast<float *>(p), *ybias = reinterpret_cast<float *>(p + yv);
    p += 2 * yv;
    Partial *partials = reinterpret_cast<Partial *>(p);
    float *maxabs = reinterpret_cast<float *>(p + pb);
    void *csc = p + pb + mb;

    if ((e = launch_center_maxabs(x, n, y, m, d, csc, maxabs, s)) != hipSuccess)
        return map_error(e);
    for (int st = 0; st < stages; ++st) {
        const double eps = eps_list[st];
        const double scale = 2.0 * kLog2e / eps;
        const double hat_scale = kLog2e / eps;
        if ((e = launch_prep_h3(x, nullptr, n, n_pad, d, kp, scale, hat_scale, kBiasZero, maxabs,
                                csc, 0, xcol, xrow, xnrm, xbias, s)) != hipSuccess)
            return map_error(e);
        if ((e = launch_prep_h3(y, g, m, m_pad, d, kp, scale, hat_scale, kBiasHat, maxabs, csc,
                                1, ycol, yrow, ynrm, ybias, s)) != hipSuccess)
            return map_error(e);
        HalfStep hf{xrow, xbias, a, ycol, ybias, 1, 0, f, n, m_pad, scale, eps * kLn2,
                    partials, n_pad, xnrm};
        HalfStep hg{yrow, ybias, b, xcol, xbias, 1, 0, g, m, n_pad, scale, eps * kLn2,
                    partials, m_pad, ynrm};
        for (int it = 0; it < iters; ++it) {
            if ((e = launch_half_step_h3(hf, kp, s)) != hipSuccess)
                return map_error(e);
            if ((e = launch_half_step_h3(hg, kp, s)) != hipSuccess)
                return map_error(e);
        }
    }
    return OT_SUCCESS;
}

// The whole schedule: stages of eps, each warm-started from the previous
// stage's potentials; d < 32 on the VALU kernels (fp64 records with the bias
// in the record), d >= 32 on the split-f16 matrix-core kernels.
ot_status run_schedule(const float *x, const float *y, const float *a, const float *b, int64_t n,
                       int64_t m, int32_t d, const double *eps_list, int stages, int iters,
                       float *f, float *g, hipStream_t s) {
    if (d >= 32)
        return run_schedule_h3(x, y, a, b, n, m, d, eps_list, stages, iters, f, g, s);
    const Layout L = choose_layout(d);
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    size_t part = half_step_partials(L, n, m_pad);
    const size_t part2 = half_step_partials(L, m, n_pad);
    if (part2 > part)
        part = part2;
    const size_t xb = align_up((size_t)n_pad * L.record_bytes(), 256);
    const size_t yb = align_up((size_t)m_pad * L.record_bytes(), 256);
    const size_t pb = align_up(part * sizeof(Partial), 256);
    Scratch sc(s);
    hipError_t e = sc.alloc(xb + yb + pb);
    if (e != hipSuccess)
        return map_error(e);
    char *base = static_cast<char *>(sc.ptr);
    void *xrec = base;
    void *yrec = base + xb;
    Partial *partials = reinterpret_cast<Partial *>(base + xb + yb);

    if ((e = launch_prep_side(x, nullptr, n, n_pad, L, 0.0, kBiasZero, xrec, xrec, L.rs, L.kp,
                              s)) != hipSuccess)
        return map_error(e);
    for (int st = 0; st < stages; ++st) {
        const double eps = eps_list[st];
        const double hat_scale = kLog2e / eps;
        // Column bias of the first f update, from the caller's (or the
        // previous stage's) g at this stage's eps.
        if ((e = launch_prep_side(y, g, m, m_pad, L, hat_scale, kBiasHat, yrec, yrec, L.rs, L.kp,
                                  s)) != hipSuccess)
            return map_error(e);
        HalfStep hf{xrec, xrec, a, yrec, yrec, L.rs, L.kp, f, n, m_pad,
                    2.0 * kLog2e / eps, eps * kLn2, partials, n_pad, nullptr};
        HalfStep hg{yrec, yrec, b, xrec, xrec, L.rs, L.kp, g, m, n_pad,
                    2.0 * kLog2e / eps, eps * kLn2, partials, m_pad, nullptr};
        for (int it = 0; it < iters; ++it) {
            if ((e = launch_half_step_valu(hf, L, s)) != hipSuccess)
                return map_error(e);
            if ((e = launch_half_step_valu(hg, L, s)) != hipSuccess)
                return map_error(e);
        }
    }
    return OT_SUCCESS;
}

ot_status check_solve_outputs(const float *x, const float *y, const float *a, const float *b,
                              int64_t n, int64_t m, int32_t d, const float *f, const float *g) {
    if (!a || !b || !f || !g)
        return OT_ERROR_INVALID_VALUE;
    const size_t fb = (size_t)n * 4, gb = (size_t)m * 4;
    if (overlaps(f, fb, g, gb))
        return OT_ERROR_INVALID_VALUE;
    const void *ins[4] = {x, y, a, b};
    const size_t inb[4] = {(size_t)n * d * 4, (size_t)m * d * 4, fb, gb};
    for (int k = 0; k < 4; ++k)
        if (overlaps(f, fb, ins[k], inb[k]) || overlaps(g, gb, ins[k], inb[k]))
            return OT_ERROR_INVALID_VALUE;
    return OT_SUCCESS;
}

// d >= 32: plan statistics on split-f16 records with the hat biases of f
// and g (the records of the solver at this eps).
ot_status plan_stats_h3(const float *x, const float *y, const float *a, const float *b,
                        const float *f, const float *g, int64_t n, int64_t m, int32_t d,
                        float eps, double *cost, double *marg, hipStream_t s) {
    const int kp = h3_kp(d);
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    const size_t xr = align_up((size_t)n_pad * 4 * kp, 256);
    const size_t yr = align_up((size_t)m_pad * 4 * kp, 256);
    const size_t xv = align_up((size_t)n_pad * sizeof(float), 256);
    const size_t yv = align_up((size_t)m_pad * sizeof(float), 256);
    const size_t mb = align_up(h3_maxabs_floats() * sizeof(float), 256);
    const size_t db = plan_stats_h3_scratch_doubles(n, m, n_pad, m_pad, kp) * sizeof(double);
    const size_t cb = align_up(h3_center_scratch_bytes(d), 256);
    Scratch sc(s);
    hipError_t e = sc.alloc(2 * xr + 2 * yr + 2 * xv + 2 * yv + mb + db + cb);
    if (e != hipSuccess)
        return map_error(e);
    char *p = static_cast<char *>(sc.ptr);
    void *xcol = p, *xrow = p + xr;
    p += 2 * xr;
    void *ycol = p, *yrow = p + yr;
    p += 2 * yr;
    float *xnrm = reinterpret_cast<float *>(p), *xhat = reinterpret_cast<float *>(p + xv);
    p += 2 * xv;
    float *ynrm = reinterpret_cast<float *>(p), *yhat = reinterpret_cast<float *>(p + yv);
    p += 2 * yv;
    float *maxabs = reinterpret_cast<float *>(p);
    double *dsc = reinterpret_cast<double *>(p + mb);
    void *csc = p + mb + db;
    const double scale = 2.0 * kLog2e / (double)eps;
    const double hat_scale = kLog2e / (double)eps;
    if ((e = launch_center_maxabs(x, n, y, m, d, csc, maxabs, s)) != hipSuccess)
        return map_error(e);
    if ((e = launch_prep_h3(x, f, n, n_pad, d, kp, scale, hat_scale, kBiasHat, maxabs, csc, 0,
                            xcol, xrow, xnrm, xhat, s)) != hipSuccess)
        return map_error(e);
    if ((e = launch_prep_h3(y, g, m, m_pad, d, kp, scale, hat_scale, kBiasHat, maxabs, csc, 1,
                            ycol, yrow, ynrm, yhat, s)) != hipSuccess)
        return map_error(e);
    e = launch_plan_stats_h3(kp, xrow, xcol, xhat, xnrm, yrow, ycol, yhat, ynrm, a, b, n, m, n_pad,
                             m_pad, scale, cost, marg, dsc, s);
    return map_error(e);
}

}  // namespace

extern "C" {

const char *ot_status_string(ot_status s) {
    switch (s) {
    case OT_SUCCESS: return "OT_SUCCESS";
    case OT_ERROR_INVALID_VALUE: return "OT_ERROR_INVALID_VALUE";
    case OT_ERROR_NOT_SUPPORTED: return "OT_ERROR_NOT_SUPPORTED";
    case OT_ERROR_OUT_OF_MEMORY: return "OT_ERROR_OUT_OF_MEMORY";
    case OT_ERROR_LAUNCH_FAILURE: return "OT_ERROR_LAUNCH_FAILURE";
    default: return "OT_ERROR_UNKNOWN";
    }
}

ot_status ot_sinkhorn_solve(const float *x, const float *y, const float *a, const float *b,
                            int64_t n, int64_t m, int32_t d, float eps, int32_t iters, float *f,
                            float *g, void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps);
    if (st == OT_SUCCESS && iters < 0)
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS)
        st = check_solve_outputs(x, y, a, b, n, m, d, f, g);
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st != OT_SUCCESS || iters == 0)
        return st;
    const double e = eps;
    return run_schedule(x, y, a, b, n, m, d, &e, 1, iters, f, g, (hipStream_t)stream);
}

ot_status ot_sinkhorn_solve_eps_scaling(const float *x, const float *y, const float *a,
                                        const float *b, int64_t n, int64_t m, int32_t d,
                                        float eps0, float eps_end, int32_t stages,
                                        int32_t iters_per_stage, float *f, float *g,
                                        void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps0);
    if (st == OT_SUCCESS && (!finite_pos(eps_end) || stages < 1 || iters_per_stage < 0))
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS)
        st = check_solve_outputs(x, y, a, b, n, m, d, f, g);
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st == OT_SUCCESS && stages > 4096)
        st = OT_ERROR_NOT_SUPPORTED;
    if (st != OT_SUCCESS || iters_per_stage == 0)
        return st;
    double eps_list[4096];
    for (int s = 0; s < stages; ++s)
        eps_list[s] = stages == 1 ? (double)eps0
                                  : (double)eps0 * pow((double)eps_end / (double)eps0,
                                                       (double)s / (double)(stages - 1));
    return run_schedule(x, y, a, b, n, m, d, eps_list, stages, iters_per_stage, f, g,
                        (hipStream_t)stream);
}

ot_status ot_plan_stats(const float *x, const float *y, const float *a, const float *b,
                        const float *f, const float *g, int64_t n, int64_t m, int32_t d, float eps,
                        double *cost, double *marg, void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps);
    if (st == OT_SUCCESS && (!f || !g || (!cost && !marg) || (marg && (!a || !b))))
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st != OT_SUCCESS)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (d >= 32)
        return plan_stats_h3(x, y, a, b, f, g, n, m, d, eps, cost, marg, s);
    // The statistics passes read fp32 records (raw potentials in the bias slot).
    Layout L = choose_layout(d);
    L.f64 = false;
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    const size_t xb = align_up((size_t)n_pad * L.record_bytes(), 256);
    const size_t yb = align_up((size_t)m_pad * L.record_bytes(), 256);
    const size_t db = plan_stats_scratch_doubles(L, n, m, n_pad, m_pad) * sizeof(double);
    Scratch sc(s);
    hipError_t e = sc.alloc(xb + yb + db);
    if (e != hipSuccess)
        return map_error(e);
    float *xrec = static_cast<float *>(sc.ptr);
    float *yrec = reinterpret_cast<float *>(static_cast<char *>(sc.ptr) + xb);
    double *dsc = reinterpret_cast<double *>(static_cast<char *>(sc.ptr) + xb + yb);
    if ((e = launch_prep_side(x, f, n, n_pad, L, 0.0, kBiasRaw, xrec, xrec, L.rs, L.kp, s)) !=
        hipSuccess)
        return map_error(e);
    if ((e = launch_prep_side(y, g, m, m_pad, L, 0.0, kBiasRaw, yrec, yrec, L.rs, L.kp, s)) !=
        hipSuccess)
        return map_error(e);
    e = launch_plan_stats(xrec, yrec, a, b, n, m, n_pad, m_pad, L, eps, cost, marg, dsc, s);
    return map_error(e);
}

ot_status ot_plan_cost(const float *x, const float *y, const float *f, const float *g, int64_t n,
                       int64_t m, int32_t d, float eps, double *cost, void *stream) {
    if (!cost)
        return OT_ERROR_INVALID_VALUE;
    return ot_plan_stats(x, y, nullptr, nullptr, f, g, n, m, d, eps, cost, nullptr, stream);
}

ot_status ot_marginal_error(const float *x, const float *y, const float *a, const float *b,
                            const float *f, const float *g, int64_t n, int64_t m, int32_t d,
                            float eps, double *marg, void *stream) {
    if (!marg)
        return OT_ERROR_INVALID_VALUE;
    return ot_plan_stats(x, y, a, b, f, g, n, m, d, eps, nullptr, marg, stream);
}

// out_i = sum_j P_ij v_j: records with hat biases of f and g, then the
// VALU (d < 32) or matrix-core (d >= 32, split-f16 records) streaming
// kernel. rowsum (matrix-core path only, nullable) also receives
// r_i = sum_j P_ij.
static ot_status transport_apply_impl(const float *x, const float *y, const float *f,
                                      const float *g, int64_t n, int64_t m, int32_t d, float eps,
                                      const float *v, int32_t dv, float *out, float *rowsum,
                                      hipStream_t s) {
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    const double hat_scale = kLog2e / (double)eps;
    const double scale = 2.0 * kLog2e / (double)eps;
    hipError_t e;
    if (d >= 32) {
        const int kp = h3_kp(d);
        const size_t xr = align_up((size_t)n_pad * 4 * kp, 256);
        const size_t yr = align_up((size_t)m_pad * 4 * kp, 256);
        const size_t xv = align_up((size_t)n_pad * sizeof(float), 256);
        const size_t yv = align_up((size_t)m_pad * sizeof(float), 256);
        const size_t mb = align_up(h3_maxabs_floats() * sizeof(float), 256);
        const size_t pd = transport_mfma_scratch_doubles(n, m_pad, dv, rowsum != nullptr, kp);
        const size_t cb = align_up(h3_center_scratch_bytes(d), 256);
        Scratch sc(s);
        if ((e = sc.alloc(2 * xr + 2 * yr + 2 * xv + 2 * yv + mb + cb +
                          pd * sizeof(double))) != hipSuccess)
            return map_error(e);
        char *p = static_cast<char *>(sc.ptr);
        void *xcol = p, *xrow = p + xr;
        p += 2 * xr;
        void *ycol = p, *yrow = p + yr;
        p += 2 * yr;
        float *xnrm = reinterpret_cast<float *>(p), *xhat = reinterpret_cast<float *>(p + xv);
        p += 2 * xv;
        float *ynrm = reinterpret_cast<float *>(p), *yhat = reinterpret_cast<float *>(p + yv);
        p += 2 * yv;
        float *maxabs = reinterpret_cast<float *>(p);
        void *csc = p + mb;
        double *part = reinterpret_cast<double *>(p + mb + cb);
        if ((e = launch_center_maxabs(x, n, y, m, d, csc, maxabs, s)) != hipSuccess ||
            (e = launch_prep_h3(x, f, n, n_pad, d, kp, scale, hat_scale, kBiasHat, maxabs, csc,
                                0, xcol, xrow, xnrm, xhat, s)) != hipSuccess ||
            (e = launch_prep_h3(y, g, m, m_pad, d, kp, scale, hat_scale, kBiasHat, maxabs, csc,
                                1, ycol, yrow, ynrm, yhat, s)) != hipSuccess)
            return map_error(e);
        return map_error(launch_transport_apply_mfma(kp, xrow, xhat, ycol, yhat, v, n, n_pad, m,
                                                     m_pad, dv, part, out, rowsum, s));
    }
    if (rowsum)
        return OT_ERROR_INVALID_VALUE;
    const Layout L = choose_layout(d);
    const size_t xb = align_up((size_t)n_pad * L.record_bytes(), 256);
    const size_t yb = align_up((size_t)m_pad * L.record_bytes(), 256);
    const size_t pd = transport_scratch_doubles(L, n, m_pad, dv);
    Scratch sc(s);
    if ((e = sc.alloc(xb + yb + pd * sizeof(double))) != hipSuccess)
        return map_error(e);
    char *base = static_cast<char *>(sc.ptr);
    void *xrec = base, *yrec = base + xb;
    double *part = reinterpret_cast<double *>(base + xb + yb);
    if ((e = launch_prep_side(x, f, n, n_pad, L, hat_scale, kBiasHat, xrec, xrec, L.rs, L.kp,
                              s)) != hipSuccess)
        return map_error(e);
    if ((e = launch_prep_side(y, g, m, m_pad, L, hat_scale, kBiasHat, yrec, yrec, L.rs, L.kp,
                              s)) != hipSuccess)
        return map_error(e);
    e = launch_transport_apply(L, xrec, yrec, v, n, n_pad, m, m_pad, dv, scale, part, out, s);
    return map_error(e);
}

ot_status ot_transport_apply(const float *x, const float *y, const float *f, const float *g,
                             int64_t n, int64_t m, int32_t d, float eps, const float *v,
                             int32_t dv, float *out, void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps);
    if (st == OT_SUCCESS && (!f || !g || !v || !out || dv < 1))
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS) {
        const size_t ob = (size_t)n * dv * 4;
        const void *ins[5] = {x, y, f, g, v};
        const size_t inb[5] = {(size_t)n * d * 4, (size_t)m * d * 4, (size_t)n * 4,
                               (size_t)m * 4, (size_t)m * dv * 4};
        for (int k = 0; k < 5; ++k)
            if (overlaps(out, ob, ins[k], inb[k]))
                st = OT_ERROR_INVALID_VALUE;
    }
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st == OT_SUCCESS && dv > OT_MAX_VALUE_DIM)
        st = OT_ERROR_NOT_SUPPORTED;
    if (st != OT_SUCCESS)
        return st;
    return transport_apply_impl(x, y, f, g, n, m, d, eps, v, dv, out, nullptr,
                                (hipStream_t)stream);
}

// The barycentric map (mode 0) and the x-gradient (mode 1) from one
// application. The map applies the plan to y and divides by a. The gradient
// also needs the row sums r_i: the MFMA kernel forms them beside its value
// channels; the VALU path applies the plan to [y | 1] instead.
static ot_status map_or_grad(const float *x, const float *y, const float *a, const float *f,
                             const float *g, int64_t n, int64_t m, int32_t d, float eps,
                             float *out, int mode, void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps);
    if (st == OT_SUCCESS && (!f || !g || !out || (mode == 0 && !a)))
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS) {
        const size_t ob = (size_t)n * d * 4;
        const void *ins[5] = {x, y, f, g, a};
        const size_t inb[5] = {(size_t)n * d * 4, (size_t)m * d * 4, (size_t)n * 4,
                               (size_t)m * 4, a ? (size_t)n * 4 : 0};
        for (int k = 0; k < 5; ++k)
            if (ins[k] && overlaps(out, ob, ins[k], inb[k]))
                st = OT_ERROR_INVALID_VALUE;
    }
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st != OT_SUCCESS)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const bool mfma = choose_layout(d).mfma;
    const bool ones = mode == 1 && !mfma;  // values [y | 1]
    const int dv = ones ? d + 1 : d;
    const size_t vb = ones ? align_up((size_t)m * dv * sizeof(float), 256) : 0;
    const size_t wb = align_up((size_t)n * dv * sizeof(float), 256);
    const size_t rb = mode == 1 && mfma ? align_up((size_t)n * sizeof(float), 256) : 0;
    Scratch sc(s);
    hipError_t e = sc.alloc(vb + wb + rb);
    if (e != hipSuccess)
        return map_error(e);
    char *base = static_cast<char *>(sc.ptr);
    const float *v = y;
    if (ones) {
        if ((e = launch_values_y1(y, m, d, reinterpret_cast<float *>(base), s)) != hipSuccess)
            return map_error(e);
        v = reinterpret_cast<const float *>(base);
    }
    float *w = reinterpret_cast<float *>(base + vb);
    float *r = rb ? reinterpret_cast<float *>(base + vb + wb) : nullptr;
    st = transport_apply_impl(x, y, f, g, n, m, d, eps, v, dv, w, r, s);
    if (st != OT_SUCCESS)
        return st;
    return map_error(launch_combine(w, dv, r, x, a, n, d, mode, out, s));
}

ot_status ot_barycentric_map(const float *x, const float *y, const float *a, const float *f,
                             const float *g, int64_t n, int64_t m, int32_t d, float eps,
                             float *out, void *stream) {
    return map_or_grad(x, y, a, f, g, n, m, d, eps, out, 0, stream);
}

ot_status ot_cost_gradient_x(const float *x, const float *y, const float *f, const float *g,
                             int64_t n, int64_t m, int32_t d, float eps, float *out,
                             void *stream) {
    return map_or_grad(x, y, nullptr, f, g, n, m, d, eps, out, 1, stream);
}

ot_status ot_birkhoff_project_batched(const float *logits, int64_t batch, float eps,
                                      int32_t max_iters, float tol, float *out,
                                      int32_t *iters_out, void *stream) {
    if (!logits || !out || batch < 0 || !finite_pos(eps) || max_iters < 0 || isnan(tol))
        return OT_ERROR_INVALID_VALUE;
    if (((uintptr_t)logits & 15) || ((uintptr_t)out & 15))
        return OT_ERROR_INVALID_VALUE;
    const size_t bytes = (size_t)batch * 16 * sizeof(float);
    if (logits != out && overlaps(logits, bytes, out, bytes))
        return OT_ERROR_INVALID_VALUE;
    if (iters_out && (overlaps(iters_out, (size_t)batch * 4, out, bytes) ||
                      overlaps(iters_out, (size_t)batch * 4, logits, bytes)))
        return OT_ERROR_INVALID_VALUE;
    if (batch == 0)
        return OT_SUCCESS;
    return map_error(launch_birkhoff4(logits, batch, eps, max_iters, tol, out, iters_out,
                                      (hipStream_t)stream));
}

ot_status ot_sinkhorn_solve_cosine(const float *x, const float *y, const float *a, const float *b,
                                   int64_t n, int64_t m, int32_t d, float eps, int32_t iters,
                                   float *f, float *g, void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps);
    if (st == OT_SUCCESS && iters < 0)
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS)
        st = check_solve_outputs(x, y, a, b, n, m, d, f, g);
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st == OT_SUCCESS && !isfinite(2.0f * eps))
        st = OT_ERROR_NOT_SUPPORTED;
    if (st != OT_SUCCESS || iters == 0)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t xb = align_up((size_t)n * d * sizeof(float), 256);
    const size_t yb = align_up((size_t)m * d * sizeof(float), 256);
    const size_t fb = align_up((size_t)n * sizeof(float), 256);
    const size_t gb = align_up((size_t)m * sizeof(float), 256);
    Scratch sc(s);
    hipError_t e = sc.alloc(xb + yb + fb + gb);
    if (e != hipSuccess)
        return map_error(e);
    char *p = static_cast<char *>(sc.ptr);
    float *xn = reinterpret_cast<float *>(p), *yn = reinterpret_cast<float *>(p + xb);
    float *f2 = reinterpret_cast<float *>(p + xb + yb);
    float *g2 = reinterpret_cast<float *>(p + xb + yb + fb);
    if ((e = launch_normalize(x, n, d, xn, s)) != hipSuccess ||
        (e = launch_normalize(y, m, d, yn, s)) != hipSuccess ||
        (e = launch_scale(g, m, 2.f, g2, s)) != hipSuccess)
        return map_error(e);
    const double e2 = 2.0 * (double)eps;
    st = run_schedule(xn, yn, a, b, n, m, d, &e2, 1, iters, f2, g2, s);
    if (st != OT_SUCCESS)
        return st;
    if ((e = launch_scale(f2, n, 0.5f, f, s)) != hipSuccess ||
        (e = launch_scale(g2, m, 0.5f, g, s)) != hipSuccess)
        return map_error(e);
    return OT_SUCCESS;
}

ot_status ot_plan_stats_cosine(const float *x, const float *y, const float *a, const float *b,
                               const float *f, const float *g, int64_t n, int64_t m, int32_t d,
                               float eps, double *cost, double *marg, void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps);
    if (st == OT_SUCCESS && (!f || !g || (!cost && !marg) || (marg && (!a || !b))))
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st == OT_SUCCESS && !isfinite(2.0f * eps))
        st = OT_ERROR_NOT_SUPPORTED;
    if (st != OT_SUCCESS)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t xb = align_up((size_t)n * d * sizeof(float), 256);
    const size_t yb = align_up((size_t)m * d * sizeof(float), 256);
    const size_t fb = align_up((size_t)n * sizeof(float), 256);
    const size_t gb = align_up((size_t)m * sizeof(float), 256);
    Scratch sc(s);
    hipError_t e = sc.alloc(xb + yb + fb + gb);
    if (e != hipSuccess)
        return map_error(e);
    char *p = static_cast<char *>(sc.ptr);
    float *xn = reinterpret_cast<float *>(p), *yn = reinterpret_cast<float *>(p + xb);
    float *f2 = reinterpret_cast<float *>(p + xb + yb);
    float *g2 = reinterpret_cast<float *>(p + xb + yb + fb);
    if ((e = launch_normalize(x, n, d, xn, s)) != hipSuccess ||
        (e = launch_normalize(y, m, d, yn, s)) != hipSuccess ||
        (e = launch_scale(f, n, 2.f, f2, s)) != hipSuccess ||
        (e = launch_scale(g, m, 2.f, g2, s)) != hipSuccess)
        return map_error(e);
    st = ot_plan_stats(xn, yn, a, b, f2, g2, n, m, d, 2.0f * eps, cost, marg, stream);
    if (st != OT_SUCCESS || !cost)
        return st;
    return map_error(launch_scale_double(cost, 0.5, s));
}

ot_status ot_birkhoff_project_newton_batched(const float *logits, int64_t batch, float eps,
                                             int32_t max_iters, float tol, float *out,
                                             int32_t *iters_out, void *stream) {
    if (!logits || !out || batch < 0 || !finite_pos(eps) || max_iters < 0 || isnan(tol))
        return OT_ERROR_INVALID_VALUE;
    if (((uintptr_t)logits & 15) || ((uintptr_t)out & 15))
        return OT_ERROR_INVALID_VALUE;
    const size_t bytes = (size_t)batch * 16 * sizeof(float);
    if (logits != out && overlaps(logits, bytes, out, bytes))
        return OT_ERROR_INVALID_VALUE;
    if (iters_out && (overlaps(iters_out, (size_t)batch * 4, out, bytes) ||
                      overlaps(iters_out, (size_t)batch * 4, logits, bytes)))
        return OT_ERROR_INVALID_VALUE;
    if (batch == 0)
        return OT_SUCCESS;
    return map_error(launch_birkhoff4_newton(logits, batch, eps, max_iters, tol, out, iters_out,
                                             (hipStream_t)stream));
}

ot_status ot_birkhoff_projection_backward_batched(const float *plan, const float *grad_plan,
                                                  int64_t batch, float eps, float *grad_logits,
                                                  void *stream) {
    if (!plan || !grad_plan || !grad_logits || batch < 0 || !finite_pos(eps))
        return OT_ERROR_INVALID_VALUE;
    if (((uintptr_t)plan & 15) || ((uintptr_t)grad_plan & 15) || ((uintptr_t)grad_logits & 15))
        return OT_ERROR_INVALID_VALUE;
    const size_t bytes = (size_t)batch * 16 * sizeof(float);
    if ((grad_logits != plan && overlaps(grad_logits, bytes, plan, bytes)) ||
        (grad_logits != grad_plan && overlaps(grad_logits, bytes, grad_plan, bytes)))
        return OT_ERROR_INVALID_VALUE;
    if (batch == 0)
        return OT_SUCCESS;
    return map_error(launch_birkhoff4_backward(plan, grad_plan, batch, eps, grad_logits,
                                               (hipStream_t)stream));
}

}  // extern "C"
