// Host side of the C ABI declared in include/ot_sinkhorn.h: argument checks,
// stream-ordered scratch, and the launch sequence of each call.
#include "ot_sinkhorn.h"
#include "ot_internal.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

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

constexpr int64_t kMaxPoints = (int64_t)1 << 34;

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
    // Tile counts are int (up to 2^34 / 32 = 2^29); 2^34 points of even one
    // fp32 coordinate are 64 GiB, past what the calls can hold in HBM.
    if (n > kMaxPoints || m > kMaxPoints)
        return OT_ERROR_NOT_SUPPORTED;
    return OT_SUCCESS;
}

// A block of device scratch memory taken and released on the call's stream.
struct Scratch {
    void *ptr = nullptr;
    hipStream_t s;
    explicit Scratch(hipStream_t st) : s(st) {}
    // A failed allocation also leaves its error as the thread's last error;
    // it is cleared here so that the next call's launch checks do not report
    // it again.
    hipError_t alloc(size_t bytes) {
        const hipError_t e = hipMallocAsync(&ptr, bytes < 256 ? 256 : bytes, s);
        if (e != hipSuccess) {
            ptr = nullptr;
            (void)hipGetLastError();
        }
        return e;
    }
    ~Scratch() {
        if (ptr)
            (void)hipFreeAsync(ptr, s);
    }
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Sub-buffers of one scratch block, each starting on a 256-byte boundary.
// With a null base only the total size is accumulated, so one carve function
// both sizes a call's scratch and splits it: the two cannot disagree.
struct Carve {
    char *base;
    size_t off = 0;
    explicit Carve(void *b) : base(static_cast<char *>(b)) {}
    template <class T> T *take(size_t bytes) {
        const size_t o = off;
        off += align_up(bytes ? bytes : 1, 256);
        return base ? static_cast<T *>(static_cast<void *>(base + o)) : nullptr;
    }
};

// d >= 32: split-f16 records of both sides. Per side: column record and row
// record (4*kp bytes per point each), |p|^2 and the fp32 bias; plus the
// per-direction maxima and the centre scratch.
struct H3Side {
    void *col, *row;
    float *nrm, *bias;
};
struct H3Records {
    int kp;
    H3Side x, y;
    float *maxabs;
    void *csc;
};

H3Side carve_h3_side(Carve &c, int64_t padded, int kp) {
    H3Side s;
    s.col = c.take<void>((size_t)padded * 4 * kp);
    s.row = c.take<void>((size_t)padded * 4 * kp);
    s.nrm = c.take<float>((size_t)padded * sizeof(float));
    s.bias = c.take<float>((size_t)padded * sizeof(float));
    return s;
}

H3Records carve_h3(Carve &c, int64_t n, int64_t m, int32_t d) {
    H3Records r;
    r.kp = h3_kp(d);
    r.x = carve_h3_side(c, pad_points(n), r.kp);
    r.y = carve_h3_side(c, pad_points(m), r.kp);
    r.maxabs = c.take<float>(h3_maxabs_floats() * sizeof(float));
    r.csc = c.take<void>(h3_center_scratch_bytes(d));
    return r;
}

// Centre and maxima of both clouds, then the records of both sides with the
// given bias modes (potentials xpot / ypot read only for kBiasHat/kBiasRaw).
hipError_t prep_h3_both(const float *x, const float *xpot, int xmode, const float *y,
                        const float *ypot, int ymode, int64_t n, int64_t m, int32_t d,
                        double eps, bool center, const H3Records &r, hipStream_t s) {
    hipError_t e;
    const double scale = 2.0 * kLog2e / eps, hat_scale = kLog2e / eps;
    if (center && (e = launch_center_maxabs(x, n, y, m, d, r.csc, r.maxabs, s)) != hipSuccess)
        return e;
    if ((e = launch_prep_h3(x, xpot, n, pad_points(n), d, r.kp, scale, hat_scale, xmode, r.maxabs,
                            r.csc, 0, r.x.col, r.x.row, r.x.nrm, r.x.bias, s)) != hipSuccess)
        return e;
    return launch_prep_h3(y, ypot, m, pad_points(m), d, r.kp, scale, hat_scale, ymode, r.maxabs,
                          r.csc, 1, r.y.col, r.y.row, r.y.nrm, r.y.bias, s);
}

// Scratch of a solve (any number of eps stages).
struct SolveBufs {
    H3Records h3;          // d >= 32
    void *xrec, *yrec;     // d < 32: fp64 records with the bias inside
    Partial *partials;     // split-column partials of either path
};

SolveBufs carve_solve(Carve &c, int64_t n, int64_t m, int32_t d) {
    SolveBufs B{};
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    size_t part;
    if (d >= 32) {
        B.h3 = carve_h3(c, n, m, d);
        part = half_step_partials_h3(n, m_pad, B.h3.kp);
        const size_t p2 = half_step_partials_h3(m, n_pad, B.h3.kp);
        part = p2 > part ? p2 : part;
    } else {
        const Layout L = choose_layout(d);
        B.xrec = c.take<void>((size_t)n_pad * L.record_bytes());
        B.yrec = c.take<void>((size_t)m_pad * L.record_bytes());
        part = half_step_partials(L, n, m_pad);
        const size_t p2 = half_step_partials(L, m, n_pad);
        part = p2 > part ? p2 : part;
    }
    B.partials = c.take<Partial>(part * sizeof(Partial));
    return B;
}

size_t solve_scratch_bytes(int64_t n, int64_t m, int32_t d) {
    Carve c(nullptr);
    carve_solve(c, n, m, d);
    return c.off;
}

// The whole schedule: stages of eps, each warm-started from the previous
// stage's potentials; d < 32 on the VALU kernels (fp64 records with the bias
// in the record), d >= 32 on the split-f16 matrix-core kernels. B is carved
// from scratch of solve_scratch_bytes(n, m, d) bytes.
ot_status run_schedule(const float *x, const float *y, const float *a, const float *b, int64_t n,
                       int64_t m, int32_t d, const double *eps_list, int stages, int iters,
                       float *f, float *g, const SolveBufs &B, hipStream_t s) {
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    hipError_t e;
    if (d >= 32) {
        const H3Records &r = B.h3;
        for (int st = 0; st < stages; ++st) {
            const double eps = eps_list[st];
            const double scale = 2.0 * kLog2e / eps;
            if ((e = prep_h3_both(x, nullptr, kBiasZero, y, g, kBiasHat, n, m, d, eps, st == 0, r,
                                  s)) != hipSuccess)
                return map_error(e);
            HalfStep hf{r.x.row, r.x.bias, a, r.y.col, r.y.bias, 1, 0, f, n, m_pad, scale,
                        eps * kLn2, B.partials, n_pad, r.x.nrm};
            HalfStep hg{r.y.row, r.y.bias, b, r.x.col, r.x.bias, 1, 0, g, m, n_pad, scale,
                        eps * kLn2, B.partials, m_pad, r.y.nrm};
            for (int it = 0; it < iters; ++it) {
                if ((e = launch_half_step_h3(hf, r.kp, s)) != hipSuccess)
                    return map_error(e);
                if ((e = launch_half_step_h3(hg, r.kp, s)) != hipSuccess)
                    return map_error(e);
            }
        }
        return OT_SUCCESS;
    }
    const Layout L = choose_layout(d);
    if ((e = launch_prep_side(x, nullptr, n, n_pad, L, 0.0, kBiasZero, B.xrec, B.xrec, L.rs, L.kp,
                              s)) != hipSuccess)
        return map_error(e);
    for (int st = 0; st < stages; ++st) {
        const double eps = eps_list[st];
        const double hat_scale = kLog2e / eps;
        // Column bias of the first f update, from the caller's (or the
        // previous stage's) g at this stage's eps.
        if ((e = launch_prep_side(y, g, m, m_pad, L, hat_scale, kBiasHat, B.yrec, B.yrec, L.rs,
                                  L.kp, s)) != hipSuccess)
            return map_error(e);
        HalfStep hf{B.xrec, B.xrec, a, B.yrec, B.yrec, L.rs, L.kp, f, n, m_pad,
                    2.0 * kLog2e / eps, eps * kLn2, B.partials, n_pad, nullptr};
        HalfStep hg{B.yrec, B.yrec, b, B.xrec, B.xrec, L.rs, L.kp, g, m, n_pad,
                    2.0 * kLog2e / eps, eps * kLn2, B.partials, m_pad, nullptr};
        for (int it = 0; it < iters; ++it) {
            if ((e = launch_half_step_valu(hf, L, s)) != hipSuccess)
                return map_error(e);
            if ((e = launch_half_step_valu(hg, L, s)) != hipSuccess)
                return map_error(e);
        }
    }
    return OT_SUCCESS;
}

// One allocation for the schedule, then the schedule.
ot_status solve_alloc(const float *x, const float *y, const float *a, const float *b, int64_t n,
                      int64_t m, int32_t d, const double *eps_list, int stages, int iters,
                      float *f, float *g, hipStream_t s) {
    Scratch sc(s);
    hipError_t e = sc.alloc(solve_scratch_bytes(n, m, d));
    if (e != hipSuccess)
        return map_error(e);
    Carve c(sc.ptr);
    const SolveBufs B = carve_solve(c, n, m, d);
    return run_schedule(x, y, a, b, n, m, d, eps_list, stages, iters, f, g, B, s);
}

// Scratch of ot_sinkhorn_solve_no_alloc: a static device array, one copy on
// every GPU the library runs on, kept until the process ends. Host code uses
// only the per-device address that hipGetSymbolAddress returns for it (the
// array's name on the host side is a stand-in, not a device address).
constexpr size_t kNoAllocBytes = (size_t)OT_NO_ALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Address of the array on the device of stream s; looked up once per device
// with that device current.
hipError_t no_alloc_scratch(hipStream_t s, void **out) {
    int dev = 0, cur = 0;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e == hipSuccess)
        e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess)
                e = r;
        }
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
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

// Scratch of the plan statistics.
struct StatsBufs {
    H3Records h3;          // d >= 32
    float *xrec, *yrec;    // d < 32: fp32 records with the raw potential inside
    double *dsc;           // partials and reductions of the passes
};

// The d < 32 statistics passes read fp32 records (raw potentials in the
// bias slot).
Layout stats_layout(int32_t d) {
    Layout L = choose_layout(d);
    L.f64 = false;
    return L;
}

StatsBufs carve_stats(Carve &c, int64_t n, int64_t m, int32_t d) {
    StatsBufs B{};
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    if (d >= 32) {
        B.h3 = carve_h3(c, n, m, d);
        B.dsc = c.take<double>(plan_stats_h3_scratch_doubles(n, m, n_pad, m_pad, B.h3.kp) *
                               sizeof(double));
    } else {
        const Layout L = stats_layout(d);
        B.xrec = c.take<float>((size_t)n_pad * L.record_bytes());
        B.yrec = c.take<float>((size_t)m_pad * L.record_bytes());
        B.dsc = c.take<double>(plan_stats_scratch_doubles(L, n, m, n_pad, m_pad) * sizeof(double));
    }
    return B;
}

ot_status plan_stats_impl(const float *x, const float *y, const float *a, const float *b,
                          const float *f, const float *g, int64_t n, int64_t m, int32_t d,
                          float eps, double *cost, double *marg, const StatsBufs &B,
                          hipStream_t s) {
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    hipError_t e;
    if (d >= 32) {
        // Hat biases of f and g: the records of the solver at this eps.
        const H3Records &r = B.h3;
        if ((e = prep_h3_both(x, f, kBiasHat, y, g, kBiasHat, n, m, d, eps, true, r, s)) !=
            hipSuccess)
            return map_error(e);
        return map_error(launch_plan_stats_h3(r.kp, r.x.row, r.x.col, r.x.bias, r.x.nrm, r.y.row,
                                              r.y.col, r.y.bias, r.y.nrm, a, b, n, m, n_pad, m_pad,
                                              2.0 * kLog2e / (double)eps, cost, marg, B.dsc, s));
    }
    const Layout L = stats_layout(d);
    if ((e = launch_prep_side(x, f, n, n_pad, L, 0.0, kBiasRaw, B.xrec, B.xrec, L.rs, L.kp, s)) !=
        hipSuccess)
        return map_error(e);
    if ((e = launch_prep_side(y, g, m, m_pad, L, 0.0, kBiasRaw, B.yrec, B.yrec, L.rs, L.kp, s)) !=
        hipSuccess)
        return map_error(e);
    return map_error(
        launch_plan_stats(B.xrec, B.yrec, a, b, n, m, n_pad, m_pad, L, eps, cost, marg, B.dsc, s));
}

// Scratch of the transport application.
struct TransportBufs {
    H3Records h3;          // d >= 32
    void *xrec, *yrec;     // d < 32: fp64 records with the hat biases
    double *part;          // split partials (and, d >= 32, the staged values)
};

TransportBufs carve_transport(Carve &c, int64_t n, int64_t m, int32_t d, int32_t dv,
                              bool rowsum) {
    TransportBufs B{};
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    if (d >= 32) {
        B.h3 = carve_h3(c, n, m, d);
        B.part = c.take<double>(transport_mfma_scratch_doubles(n, m_pad, dv, rowsum, B.h3.kp) *
                                sizeof(double));
    } else {
        const Layout L = choose_layout(d);
        B.xrec = c.take<void>((size_t)n_pad * L.record_bytes());
        B.yrec = c.take<void>((size_t)m_pad * L.record_bytes());
        B.part = c.take<double>(transport_scratch_doubles(L, n, m_pad, dv) * sizeof(double));
    }
    return B;
}

// out_i = sum_j P_ij v_j: records with hat biases of f and g, then the
// VALU (d < 32) or matrix-core (d >= 32, split-f16 records) streaming
// kernel. rowsum (matrix-core path only, nullable) also receives
// r_i = sum_j P_ij.
ot_status transport_apply_impl(const float *x, const float *y, const float *f, const float *g,
                               int64_t n, int64_t m, int32_t d, float eps, const float *v,
                               int32_t dv, float *out, float *rowsum, const TransportBufs &B,
                               hipStream_t s) {
    const int64_t n_pad = pad_points(n), m_pad = pad_points(m);
    hipError_t e;
    if (d >= 32) {
        const H3Records &r = B.h3;
        if ((e = prep_h3_both(x, f, kBiasHat, y, g, kBiasHat, n, m, d, eps, true, r, s)) !=
            hipSuccess)
            return map_error(e);
        return map_error(launch_transport_apply_mfma(r.kp, r.x.row, r.x.bias, r.y.col, r.y.bias, v,
                                                     n, n_pad, m, m_pad, dv, B.part, out, rowsum,
                                                     s));
    }
    if (rowsum)
        return OT_ERROR_INVALID_VALUE;
    const Layout L = choose_layout(d);
    const double hat_scale = kLog2e / (double)eps;
    if ((e = launch_prep_side(x, f, n, n_pad, L, hat_scale, kBiasHat, B.xrec, B.xrec, L.rs, L.kp,
                              s)) != hipSuccess)
        return map_error(e);
    if ((e = launch_prep_side(y, g, m, m_pad, L, hat_scale, kBiasHat, B.yrec, B.yrec, L.rs, L.kp,
                              s)) != hipSuccess)
        return map_error(e);
    return map_error(launch_transport_apply(L, B.xrec, B.yrec, v, n, n_pad, m, m_pad, dv,
                                            2.0 * kLog2e / (double)eps, B.part, out, s));
}

// A graph captured from the cosine calls, the barycentric map and the
// x-gradient faulted on its first replay (illegal address reported in the
// record preparation) after the same sequence ran correctly without capture;
// no out-of-range access was found in the kernels or in the scratch layout.
// Until the cause is known those calls refuse to run on a capturing stream.
// An error from the query itself is treated as a capture in progress.
bool stream_capturing(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
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
    return solve_alloc(x, y, a, b, n, m, d, &e, 1, iters, f, g, (hipStream_t)stream);
}

ot_status ot_sinkhorn_solve_no_alloc(const float *x, const float *y, const float *a,
                                     const float *b, int64_t n, int64_t m, int32_t d, float eps,
                                     int32_t iters, float *f, float *g, void *stream) {
    ot_status st = check_clouds(x, y, n, m, d, eps);
    if (st == OT_SUCCESS && iters < 0)
        st = OT_ERROR_INVALID_VALUE;
    if (st == OT_SUCCESS)
        st = check_solve_outputs(x, y, a, b, n, m, d, f, g);
    if (st == OT_SUCCESS)
        st = check_supported(n, m, d);
    if (st == OT_SUCCESS && solve_scratch_bytes(n, m, d) > kNoAllocBytes)
        st = OT_ERROR_NOT_SUPPORTED;
    if (st != OT_SUCCESS || iters == 0)
        return st;
    hipStream_t s = (hipStream_t)stream;
    void *base = nullptr;
    const hipError_t e = no_alloc_scratch(s, &base);
    if (e != hipSuccess)
        return map_error(e);
    Carve c(base);
    const SolveBufs B = carve_solve(c, n, m, d);
    const double ed = eps;
    return run_schedule(x, y, a, b, n, m, d, &ed, 1, iters, f, g, B, s);
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
    return solve_alloc(x, y, a, b, n, m, d, eps_list, stages, iters_per_stage, f, g,
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
    Carve size(nullptr);
    carve_stats(size, n, m, d);
    Scratch sc(s);
    hipError_t e = sc.alloc(size.off);
    if (e != hipSuccess)
        return map_error(e);
    Carve c(sc.ptr);
    const StatsBufs B = carve_stats(c, n, m, d);
    return plan_stats_impl(x, y, a, b, f, g, n, m, d, eps, cost, marg, B, s);
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
    if (st == OT_SUCCESS && (d > OT_MAX_TRANSPORT_DIM || dv > OT_MAX_VALUE_DIM))
        st = OT_ERROR_NOT_SUPPORTED;
    if (st != OT_SUCCESS)
        return st;
    hipStream_t s = (hipStream_t)stream;
    Carve size(nullptr);
    carve_transport(size, n, m, d, dv, false);
    Scratch sc(s);
    hipError_t e = sc.alloc(size.off);
    if (e != hipSuccess)
        return map_error(e);
    Carve c(sc.ptr);
    const TransportBufs B = carve_transport(c, n, m, d, dv, false);
    return transport_apply_impl(x, y, f, g, n, m, d, eps, v, dv, out, nullptr, B, s);
}

}  // extern "C"

namespace {

// The barycentric map (mode 0) and the x-gradient (mode 1) from one
// application. The map applies the plan to y and divides by a. The gradient
// also needs the row sums r_i: the MFMA kernel forms them beside its value
// channels; the VALU path applies the plan to [y | 1] instead. One
// allocation holds the values, the applied sums and the application's own
// scratch.
ot_status map_or_grad(const float *x, const float *y, const float *a, const float *f,
                      const float *g, int64_t n, int64_t m, int32_t d, float eps, float *out,
                      int mode, void *stream) {
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
    if (st == OT_SUCCESS && d > OT_MAX_TRANSPORT_DIM)
        st = OT_ERROR_NOT_SUPPORTED;
    if (st != OT_SUCCESS)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (stream_capturing(s))
        return OT_ERROR_NOT_SUPPORTED;
    const bool mfma = choose_layout(d).mfma;
    const bool ones = mode == 1 && !mfma;  // values [y | 1]
    const bool rows = mode == 1 && mfma;   // row sums beside the values
    const int dv = ones ? d + 1 : d;
    auto carve = [&](Carve &c, float *&v1, float *&w, float *&r) {
        v1 = ones ? c.take<float>((size_t)m * dv * sizeof(float)) : nullptr;
        w = c.take<float>((size_t)n * dv * sizeof(float));
        r = rows ? c.take<float>((size_t)n * sizeof(float)) : nullptr;
        return carve_transport(c, n, m, d, dv, rows);
    };
    float *v1, *w, *r;
    Carve size(nullptr);
    carve(size, v1, w, r);
    Scratch sc(s);
    hipError_t e = sc.alloc(size.off);
    if (e != hipSuccess)
        return map_error(e);
    Carve c(sc.ptr);
    const TransportBufs B = carve(c, v1, w, r);
    const float *v = y;
    if (ones) {
        if ((e = launch_values_y1(y, m, d, v1, s)) != hipSuccess)
            return map_error(e);
        v = v1;
    }
    st = transport_apply_impl(x, y, f, g, n, m, d, eps, v, dv, w, r, B, s);
    if (st != OT_SUCCESS)
        return st;
    return map_error(launch_combine(w, dv, r, x, a, n, d, mode, out, s));
}

// Normalised copies of both clouds and the potentials scaled by `scale`
// (cosine calls: the squared Euclidean problem on unit vectors at 2 eps).
struct CosineBufs {
    float *xn, *yn, *f2, *g2;
};

CosineBufs carve_cosine(Carve &c, int64_t n, int64_t m, int32_t d) {
    CosineBufs B;
    B.xn = c.take<float>((size_t)n * d * sizeof(float));
    B.yn = c.take<float>((size_t)m * d * sizeof(float));
    B.f2 = c.take<float>((size_t)n * sizeof(float));
    B.g2 = c.take<float>((size_t)m * sizeof(float));
    return B;
}

}  // namespace

extern "C" {

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
    if (stream_capturing(s))
        return OT_ERROR_NOT_SUPPORTED;
    Carve size(nullptr);
    carve_cosine(size, n, m, d);
    carve_solve(size, n, m, d);
    Scratch sc(s);
    hipError_t e = sc.alloc(size.off);
    if (e != hipSuccess)
        return map_error(e);
    Carve c(sc.ptr);
    const CosineBufs C = carve_cosine(c, n, m, d);
    const SolveBufs B = carve_solve(c, n, m, d);
    if ((e = launch_normalize(x, n, d, C.xn, s)) != hipSuccess ||
        (e = launch_normalize(y, m, d, C.yn, s)) != hipSuccess ||
        (e = launch_scale(g, m, 2.f, C.g2, s)) != hipSuccess)
        return map_error(e);
    const double e2 = 2.0 * (double)eps;
    st = run_schedule(C.xn, C.yn, a, b, n, m, d, &e2, 1, iters, C.f2, C.g2, B, s);
    if (st != OT_SUCCESS)
        return st;
    if ((e = launch_scale(C.f2, n, 0.5f, f, s)) != hipSuccess ||
        (e = launch_scale(C.g2, m, 0.5f, g, s)) != hipSuccess)
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
    if (stream_capturing(s))
        return OT_ERROR_NOT_SUPPORTED;
    Carve size(nullptr);
    carve_cosine(size, n, m, d);
    carve_stats(size, n, m, d);
    Scratch sc(s);
    hipError_t e = sc.alloc(size.off);
    if (e != hipSuccess)
        return map_error(e);
    Carve c(sc.ptr);
    const CosineBufs C = carve_cosine(c, n, m, d);
    const StatsBufs B = carve_stats(c, n, m, d);
    if ((e = launch_normalize(x, n, d, C.xn, s)) != hipSuccess ||
        (e = launch_normalize(y, m, d, C.yn, s)) != hipSuccess ||
        (e = launch_scale(f, n, 2.f, C.f2, s)) != hipSuccess ||
        (e = launch_scale(g, m, 2.f, C.g2, s)) != hipSuccess)
        return map_error(e);
    st = plan_stats_impl(C.xn, C.yn, a, b, C.f2, C.g2, n, m, d, 2.0f * eps, cost, marg, B, s);
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
