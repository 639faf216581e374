// Internal declarations shared by the host code and the kernels of the
// gfx950 log-domain Sinkhorn library. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace otsk {

// Bias of padding records. Finite on purpose: with -inf, an all-padding
// chunk would give (-inf) - (-inf) = NaN in the running-max update.
constexpr float kPadBias = -1.0e30f;

// Every side's record array is padded to a multiple of this many points, so
// the column loops of all kernels run over whole tiles with no tail code.
constexpr int kPointPad = 256;

// log2(e) and ln(2).
constexpr double kLog2e = 1.4426950408889634074;
constexpr double kLn2 = 0.69314718055994530942;

// How one side of the problem is laid out in device scratch memory: one
// record of rs elements (fp64 when f64, else fp32) per point.
//
// rec[i*rs + k], k < kp : raw coordinate k of point i (zero for k >= d and for
//                         padding points i >= count)
// rec[i*rs + kp]        : the point's log2-domain bias ("hat" potential)
//                         (f_i - |x_i|^2) * log2(e)/eps, kPadBias for padding
// rec[i*rs + k], k > kp : zero
struct Layout {
    int d;        // feature dimension
    int kp;       // coordinates stored per record (>= d)
    int rs;       // elements per record (multiple of 4, > kp)
    bool mfma;    // true: the MFMA kernels; false: the VALU kernels
    bool f64;     // record elements are fp64 (VALU solve) or fp32
    size_t record_bytes() const { return (size_t)rs * (f64 ? 8 : 4); }
};

// Per-split partial of a row's streamed log-sum-exp: running max (log2
// units) and the sum of 2^(s - m) over the split's columns.
struct Partial {
    double m;
    float s;
    float pad;
};

Layout choose_layout(int d);

inline int64_t pad_points(int64_t count) {
    return (count + kPointPad - 1) / kPointPad * kPointPad;
}

// Arguments of one half-step: update the potentials of the "row" side from
// the records (coordinates) and biases of the "column" side.
//
// Where a side's bias lives: element i*bias_stride + bias_off of its bias
// base. VALU layout: inside the fp64 record (base = records, stride rs,
// offset kp). MFMA layout: a separate contiguous fp32 array (stride 1,
// offset 0), so whole bias tiles load with one instruction.
struct HalfStep {
    const void *row_rec;    // rows' own records (coordinates read)
    void *row_bias;         // rows' bias base: new biases written here
    const float *row_w;     // row weights (count rows)
    const void *col_rec;    // columns' records (coordinates read)
    const void *col_bias;   // columns' bias base (read)
    int bias_stride;        // elements between consecutive points' biases
    int bias_off;           // offset of a point's bias from its base element
    float *pot_out;         // row potentials written (count rows)
    int64_t rows;           // real row count
    int64_t cols_pad;       // padded column count (multiple of kPointPad)
    double scale;           // 2*log2(e)/eps, applied to the rows' coordinates
    double eps_ln2;         // eps*ln(2)
    Partial *partials;      // split-column scratch, >= nsplit * rows_pad entries
    int64_t rows_pad;
    const float *row_nrm;   // |p_i|^2 of the rows (split-f16 kernel only)
};

// Launch helpers (each returns hipSuccess or the first HIP error).
// Write the records of one side and its biases (bias of point i at
// bias[i*bias_stride + bias_off], in the records' element type).
hipError_t launch_prep_side(const float *pts, const float *pot, int64_t count, int64_t padded,
                            const Layout &L, double hat_scale, int bias_mode, void *rec,
                            void *bias, int bias_stride, int bias_off, hipStream_t s);
hipError_t launch_half_step_valu(const HalfStep &h, const Layout &L, hipStream_t s);
size_t half_step_partials(const Layout &L, int64_t rows, int64_t cols_pad);
hipError_t launch_merge(const HalfStep &h, const Layout &L, int nsplit, hipStream_t s);

// x_rec / y_rec: records whose bias slot holds the raw potential (f or g).
hipError_t launch_plan_stats(const float *x_rec, const float *y_rec, const float *a, const float *b,
                             int64_t n, int64_t m, int64_t n_pad, int64_t m_pad, const Layout &L,
                             float eps, double *cost, double *marg, double *scratch,
                             hipStream_t s);
size_t plan_stats_scratch_doubles(const Layout &L, int64_t n, int64_t m, int64_t n_pad,
                                  int64_t m_pad);

// Transport application (records from launch_prep_side with kBiasHat of f
// and g; out_i = sum_j P_ij v_j).
int transport_value_chunk(int dv);
size_t transport_scratch_doubles(const Layout &L, int64_t n, int64_t m_pad, int dv);
hipError_t launch_transport_apply(const Layout &L, const void *xrec, const void *yrec,
                                  const float *v, int64_t n, int64_t n_pad, int64_t m,
                                  int64_t m_pad, int dv, double scale, double *part, float *out,
                                  hipStream_t s);
// Matrix-core variant on split-f16 records (launch_prep_h3 with the hat
// biases of f and g): x's row records and y's column records; rowsum
// (nullable) also receives r_i = sum_j P_ij, with rowsum = true in the
// scratch size.
// Above kp = 192, and at kp = 160 and 192 for wide enough dv (dv <= 1024),
// in transport_rows.hip, with the same records and arguments.
size_t transport_rows_scratch_doubles(int64_t n, int64_t m_pad, int dv, bool rowsum);
hipError_t launch_transport_rows(int kp, const void *xrow, const float *xhat, const void *ycol,
                                 const float *yhat, const float *v, int64_t n, int64_t n_pad,
                                 int64_t m, int64_t m_pad, int dv, double *part, float *out,
                                 float *rowsum, hipStream_t s);
size_t transport_mfma_scratch_doubles(int64_t n, int64_t m_pad, int dv, bool rowsum,
                                      int kp);
hipError_t launch_transport_apply_mfma(int kp, const void *xrow, const float *xhat,
                                       const void *ycol, const float *yhat, const float *v,
                                       int64_t n, int64_t n_pad, int64_t m, int64_t m_pad, int dv,
                                       double *part, float *out, float *rowsum, hipStream_t s);
hipError_t launch_values_y1(const float *y, int64_t m, int d, float *v, hipStream_t s);
// mode 0: out_i = w_i / a_i; mode 1: out_i = 2 (r_i x_i - w_i), where w_i is
// row i of w (row stride ws >= d) and r_i = r[i], or w[i*ws + d] if r is null.
hipError_t launch_combine(const float *w, int ws, const float *r, const float *x, const float *a,
                          int64_t n, int d, int mode, float *out, hipStream_t s);

// Half-step with split-f16 matrix-core products (d >= 32): records from
// launch_prep_h3 (column record, row record, |p|^2, fp32 bias per side) of
// the centred points p = x - c, after launch_center_maxabs has written the
// centre c = (mean(x) + mean(y)) / 2 into center_scratch
// (h3_center_scratch_bytes(d) bytes) and max|x - c|, max|y - c| to
// maxabs[0..1] (scratch of h3_maxabs_floats() floats).
int h3_kp(int d);
size_t h3_maxabs_floats();
size_t h3_center_scratch_bytes(int d);
hipError_t launch_center_maxabs(const float *x, int64_t n, const float *y, int64_t m, int d,
                                void *center_scratch, float *maxabs, hipStream_t s);
hipError_t launch_prep_h3(const float *pts, const float *pot, int64_t count, int64_t padded, int d,
                          int kp, double scale, double hat_scale, int bias_mode,
                          const float *maxabs, const void *center_scratch, int own, void *colrec,
                          void *rowrec, float *nrm, float *bias, hipStream_t s);
size_t half_step_partials_h3(int64_t rows, int64_t cols_pad, int kp);
// One plan-statistics pass on split-f16 records (hat biases of the
// potentials): part[split][row] = (sum_j P_ij, cost ? sum_j P_ij C_ij : 0).
int plan_pass_h3_splits(int64_t rows, int64_t cols_pad, int kp);
hipError_t launch_plan_pass_h3(int kp, bool cost, const void *row_rec, const float *row_hat,
                               const float *row_nrm, const void *col_rec, const float *col_hat,
                               const float *col_nrm, int64_t rows, int64_t rows_pad,
                               int64_t cols_pad, double scale, double2 *part, hipStream_t s);
// Reductions of the two passes' partials into cost and marginal errors
// (scratch of plan_stats_h3_scratch_doubles doubles).
size_t plan_stats_h3_scratch_doubles(int64_t n, int64_t m, int64_t n_pad, int64_t m_pad,
                                     int kp);
hipError_t launch_plan_stats_h3(int kp, const void *xrow, const void *xcol, const float *xhat,
                                const float *xnrm, const void *yrow, const void *ycol,
                                const float *yhat, const float *ynrm, const float *a,
                                const float *b, int64_t n, int64_t m, int64_t n_pad,
                                int64_t m_pad, double scale, double *cost, double *marg,
                                double *scratch, hipStream_t s);
hipError_t launch_half_step_h3(const HalfStep &h, int kp, hipStream_t s);
// Merge of the column splits' (max, sum) partials of a split-f16 half-step.
hipError_t launch_merge_h3(const HalfStep &h, int nsplit, hipStream_t s);
// The same half-step and statistics pass for kp in {224, 256, 320, 384, 448}
// on 16x16 matrix-core tiles (lse_wide.hip); the h3 entry points above
// dispatch to them for 192 < kp <= 448.
bool wide_kp(int kp);
size_t half_step_partials_wide(int64_t rows, int64_t cols_pad, int kp);
hipError_t launch_half_step_wide(const HalfStep &h, int kp, hipStream_t s);
int plan_pass_wide_splits(int64_t rows, int64_t cols_pad, int kp);
hipError_t launch_plan_pass_wide(int kp, bool cost, const void *row_rec, const float *row_hat,
                                 const float *row_nrm, const void *col_rec, const float *col_hat,
                                 const float *col_nrm, int64_t rows, int64_t rows_pad,
                                 int64_t cols_pad, double scale, double2 *part, hipStream_t s);
// Above this many coordinates per record the split-f16 records are staged:
// each 32-coordinate stage's 4 hi and 4 lo 16-byte chunks side by side (one
// 128-byte line per record and stage, chunk q of stage s at 8s + q for hi and
// 8s + 4 + q for lo), unswizzled, on both sides; only the kernels that stream
// both sides through LDS in coordinate stages read them (the widest half-step
// and statistics pass, and the transport application above 192 coordinates).
constexpr int kStagedRecordKP = 512;
// For kp in {512, 640, 768, 896, 1024} (448 < d <= 1024) the half-step and
// the statistics pass are tiled like a matrix product, both sides streamed
// through LDS in coordinate stages (lse_gemm.hip); the h3 entry points
// dispatch to these for kp > 448.
size_t half_step_partials_gemm(int64_t rows, int64_t cols_pad);
hipError_t launch_half_step_gemm(const HalfStep &h, int kp, hipStream_t s);
int plan_pass_gemm_splits(int64_t rows, int64_t cols_pad);
hipError_t launch_plan_pass_gemm(int kp, bool cost, const void *row_rec, const float *row_hat,
                                 const float *row_nrm, const void *col_rec, const float *col_hat,
                                 const float *col_nrm, int64_t rows, int64_t rows_pad,
                                 int64_t cols_pad, double scale, double2 *part, hipStream_t s);

// Cosine cost: normalised copies of the points, scaled potentials.
hipError_t launch_normalize(const float *pts, int64_t count, int d, float *out, hipStream_t s);
hipError_t launch_scale(const float *in, int64_t count, float factor, float *out, hipStream_t s);
hipError_t launch_scale_double(double *v, double factor, hipStream_t s);

hipError_t launch_birkhoff4(const float *logits, int64_t batch, float eps, int max_iters, float tol,
                            float *out, int32_t *iters_out, hipStream_t s);
hipError_t launch_birkhoff4_newton(const float *logits, int64_t batch, float eps, int max_iters,
                                   float tol, float *out, int32_t *iters_out, hipStream_t s);
hipError_t launch_birkhoff4_backward(const float *plan, const float *grad_plan, int64_t batch,
                                     float eps, float *grad_logits, hipStream_t s);

// bias_mode values of launch_prep_side
enum { kBiasZero = 0, kBiasHat = 1, kBiasRaw = 2 };

// Workgroup -> (row block, column split) for a 1-D grid of nrb * nsplit
// workgroups. The dispatcher deals workgroups to the 8 XCDs round robin; with
// the split-major order below each XCD gets a contiguous run of (split, row
// block) pairs, so it streams as few column splits through its L2 as
// possible (at 65536^2, d = 64: one split per XCD pair, 17% less HBM traffic).
__device__ __forceinline__ void xcd_block(int nrb, int nsplit, int &rb, int &split) {
    const int L = (int)blockIdx.x, T = nrb * nsplit;
    const int q = (T % 8 == 0) ? (L % 8) * (T / 8) + L / 8 : L;
    split = q / nrb;
    rb = q % nrb;
}

}  // namespace otsk
