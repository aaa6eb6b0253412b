// Rotation fitting on calibration residuals (host code; an offline step, not
// part of the decode path).
//
// The pages give the rotation's role -- a per-(layer, head, K|V) channel
// rotation of the residual before its low-bit quantization (ResidualQuant,
// arXiv 2610.10381 abstract; rit.work summary, section on how each pass is
// restored) -- but no rule for choosing it. This fits one by alternating
//   (1) quantize the rotated samples with the method's group quantizer
//       (step (max-min)/(2^b-1) and offset min rounded to the metadata dtype,
//       codes rounded to nearest even and clamped), and
//   (2) the orthogonal Procrustes step: the orthogonal R that best maps the
//       samples onto their quantized values, R = U V^T for the SVD
//       M = sum_i yhat_i d_i^T = U S V^T,
// keeping the R with the lowest mean squared quantization error seen (the
// starting rotation included). Everything is float64; the SVD is a one-sided
// (Hestenes) Jacobi iteration.
#include <math.h>
#include <string.h>

#include <vector>

#include "rq_internal.h"

namespace rq {
namespace {

// float64 -> float16 -> float64, round to nearest even: the value is scaled
// by a power of two onto the fp16 grid of its binade (exact), rounded with
// rint (nearest even in the default rounding mode) and scaled back.
double round_f16(double x) {
    if (!isfinite(x) || x == 0.0) return x;
    const double ax = fabs(x);
    if (ax >= 65520.0) return copysign(INFINITY, x);   // rounds past the largest fp16
    int e;
    frexp(ax, &e);                                      // ax in [2^(e-1), 2^e)
    int q = e - 1 - 10;                                 // exponent of the fp16 quantum in this binade
    if (q < -24) q = -24;                               // subnormal quantum 2^-24
    const double r = rint(ldexp(ax, -q));
    return copysign(ldexp(r, q), x);
}

double meta_round(double x, int meta) { return meta == RQ_DTYPE_F32 ? (double)(float)x : round_f16(x); }

// y [D] -> its quantized reconstruction yh [D]
void quantize_row(const double *y, double *yh, int D, int G, int bits, int meta) {
    const double qmax = (double)((1 << bits) - 1);
    for (int g0 = 0; g0 < D; g0 += G) {
        double lo = y[g0], hi = y[g0];
        for (int c = g0 + 1; c < g0 + G; ++c) {
            lo = fmin(lo, y[c]);
            hi = fmax(hi, y[c]);
        }
        const double s = meta_round((hi - lo) / qmax, meta);
        const double z = meta_round(lo, meta);
        for (int c = g0; c < g0 + G; ++c) {
            double code = 0.0;
            if (s != 0.0) code = fmin(fmax(rint((y[c] - z) / s), 0.0), qmax);
            yh[c] = code * s + z;
        }
    }
}

// Y = rows of samples rotated by R (row-major R, y_i = R d_i); returns the mean
// squared quantization error and, if M is given, accumulates M += yhat_i d_i^T.
double quant_error(const std::vector<double> &X, int64_t n, int D, const std::vector<double> &R, int G, int bits,
                   int meta, std::vector<double> *M) {
    std::vector<double> y(D), yh(D);
    double err = 0.0;
    if (M) M->assign((size_t)D * D, 0.0);
    for (int64_t i = 0; i < n; ++i) {
        const double *d = &X[(size_t)i * D];
        for (int r = 0; r < D; ++r) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c) acc += R[(size_t)r * D + c] * d[c];
            y[r] = acc;
        }
        quantize_row(y.data(), yh.data(), D, G, bits, meta);
        for (int r = 0; r < D; ++r) err += (yh[r] - y[r]) * (yh[r] - y[r]);
        if (M)
            for (int r = 0; r < D; ++r)
                for (int c = 0; c < D; ++c) (*M)[(size_t)r * D + c] += yh[r] * d[c];
    }
    return err / (double)n;
}

// Orthogonal polar factor R = U V^T of M (row-major D x D) by one-sided Jacobi:
// rotate column pairs of W = M V until they are mutually orthogonal; then
// W = U S and R = U V^T.
void procrustes(const std::vector<double> &M, int D, std::vector<double> &R) {
    std::vector<double> W(M), V((size_t)D * D, 0.0);
    for (int i = 0; i < D; ++i) V[(size_t)i * D + i] = 1.0;
    auto col = [&](std::vector<double> &A, int r, int c) -> double & { return A[(size_t)r * D + c]; };
    for (int sweep = 0; sweep < 60; ++sweep) {
        double off = 0.0;
        for (int p = 0; p < D - 1; ++p) {
            for (int q = p + 1; q < D; ++q) {
                double a = 0.0, b = 0.0, g = 0.0;
                for (int r = 0; r < D; ++r) {
                    const double wp = col(W, r, p), wq = col(W, r, q);
                    a += wp * wp;
                    b += wq * wq;
                    g += wp * wq;
                }
                if (a == 0.0 || b == 0.0) continue;
                const double rel = fabs(g) / sqrt(a * b);
                off = fmax(off, rel);
                if (rel < 1e-15) continue;
                const double zeta = (b - a) / (2.0 * g);
                const double t = (zeta >= 0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
                const double cs = 1.0 / sqrt(1.0 + t * t), sn = cs * t;
                for (int r = 0; r < D; ++r) {
                    const double wp = col(W, r, p), wq = col(W, r, q);
                    col(W, r, p) = cs * wp - sn * wq;
                    col(W, r, q) = sn * wp + cs * wq;
                    const double vp = col(V, r, p), vq = col(V, r, q);
                    col(V, r, p) = cs * vp - sn * vq;
                    col(V, r, q) = sn * vp + cs * vq;
                }
            }
        }
        if (off < 1e-15) break;
    }
    // U = W S^-1 column by column. Columns whose singular value is zero (M of
    // rank < D: fewer samples than channels, or channels that are zero in every
    // sample) have no direction of their own; U is completed there with unit
    // vectors orthogonal to every other column (Gram-Schmidt over the standard
    // basis), so that R stays orthogonal. The samples have no component along
    // the matching columns of V, so the completion does not change R d.
    std::vector<double> nrm(D, 0.0);
    double nmax = 0.0;
    for (int c = 0; c < D; ++c) {
        for (int r = 0; r < D; ++r) nrm[c] += col(W, r, c) * col(W, r, c);
        nrm[c] = sqrt(nrm[c]);
        nmax = fmax(nmax, nrm[c]);
    }
    std::vector<char> null_col(D, 0);
    for (int c = 0; c < D; ++c) {
        null_col[c] = !(nrm[c] > 1e-13 * nmax);
        const double inv = null_col[c] ? 0.0 : 1.0 / nrm[c];
        for (int r = 0; r < D; ++r) col(W, r, c) *= inv;
    }
    // each null column: the standard basis vector with the largest component
    // outside the span of the columns set so far (at least 1/sqrt(D) of it,
    // since that span has dimension < D), projected out twice and normalized
    std::vector<double> v(D), best_v(D);
    for (int c = 0; c < D; ++c) {
        if (!null_col[c]) continue;
        double best_n = -1.0;
        for (int k = 0; k < D; ++k) {
            for (int r = 0; r < D; ++r) v[r] = r == k ? 1.0 : 0.0;
            for (int pass = 0; pass < 2; ++pass)
                for (int j = 0; j < D; ++j) {
                    if (j == c) continue;      // unset null columns are zero and change nothing
                    double dot = 0.0;
                    for (int r = 0; r < D; ++r) dot += col(W, r, j) * v[r];
                    for (int r = 0; r < D; ++r) v[r] -= dot * col(W, r, j);
                }
            double vn = 0.0;
            for (int r = 0; r < D; ++r) vn += v[r] * v[r];
            if (vn > best_n) { best_n = vn; best_v = v; }
        }
        const double inv = 1.0 / sqrt(best_n);
        for (int r = 0; r < D; ++r) col(W, r, c) = best_v[r] * inv;
    }
    R.assign((size_t)D * D, 0.0);
    for (int r = 0; r < D; ++r)
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int k = 0; k < D; ++k) acc += col(W, r, k) * col(V, c, k);
            R[(size_t)r * D + c] = acc;
        }
}

}  // namespace
}  // namespace rq

using namespace rq;

namespace rq {
namespace {

// Workspace of the device fit: R, M and the error, then the per-workgroup
// partials (float64 throughout).
size_t fit_ws_off_m(int D) { return (size_t)D * D * 8; }
size_t fit_ws_off_err(int D) { return 2 * (size_t)D * D * 8; }
size_t fit_ws_off_mpart(int D) { return 2 * (size_t)D * D * 8 + 256; }
size_t fit_ws_off_epart(int D) { return fit_ws_off_mpart(D) + (size_t)kFitBlocks * D * D * 8; }
size_t fit_ws_bytes(int D) { return fit_ws_off_epart(D) + (size_t)kFitBlocks * 8; }

}  // namespace
}  // namespace rq

extern "C" size_t rq_fit_workspace_bytes(int32_t head_dim) {
    if (head_dim != 64 && head_dim != 96 && head_dim != 128) return 0;
    return rq::fit_ws_bytes(head_dim);
}

extern "C" rq_status rq_fit_rotation_device(const float *samples, int64_t n, int32_t head_dim, int32_t bits,
                                            int32_t group_size, int32_t meta_dtype, const float *rot0,
                                            int32_t iters, float *rot_out, double *objective, void *workspace,
                                            size_t workspace_bytes, void *stream) {
    using namespace rq;
    if (!samples || !rot0 || !rot_out || !workspace) return RQ_ERR_NULL;
    const int D = head_dim, G = group_size;
    if (n < 1 || G < 1 || D % G != 0 || iters < 0 || iters > 10000) return RQ_ERR_SHAPE;
    if (D != 64 && D != 96 && D != 128) return RQ_ERR_UNSUPPORTED;
    if (bits != 2 && bits != 4) return RQ_ERR_UNSUPPORTED;
    if (meta_dtype != RQ_DTYPE_F16 && meta_dtype != RQ_DTYPE_F32) return RQ_ERR_UNSUPPORTED;
    if (workspace_bytes < fit_ws_bytes(D)) return RQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0 || ((uintptr_t)samples & 3) != 0) return RQ_ERR_SHAPE;
    uint8_t *ws = (uint8_t *)workspace;
    const hipStream_t st = (hipStream_t)stream;
    FitPass p;
    p.x = samples; p.n = n; p.D = D; p.bits = bits; p.G = G; p.meta = meta_dtype;
    p.r = (const double *)ws;
    p.m = (double *)(ws + fit_ws_off_m(D));
    p.err = (double *)(ws + fit_ws_off_err(D));
    p.mpart = (double *)(ws + fit_ws_off_mpart(D));
    p.epart = (double *)(ws + fit_ws_off_epart(D));
    p.stream = st;
    std::vector<double> R((size_t)D * D), M((size_t)D * D);
    for (size_t i = 0; i < R.size(); ++i) R[i] = (double)rot0[i];
    std::vector<double> best(R);
    double best_err = 0.0;
    // one pass per rotation: its error, and M for the next Procrustes step
    auto pass = [&](double *err) -> bool {
        double e = 0.0;
        if (hipMemcpyAsync((void *)p.r, R.data(), R.size() * 8, hipMemcpyHostToDevice, st) != hipSuccess) return false;
        if (launch_fit_pass(p) != hipSuccess) return false;
        if (hipMemcpyAsync(M.data(), p.m, M.size() * 8, hipMemcpyDeviceToHost, st) != hipSuccess) return false;
        if (hipMemcpyAsync(&e, p.err, 8, hipMemcpyDeviceToHost, st) != hipSuccess) return false;
        if (hipStreamSynchronize(st) != hipSuccess) return false;
        *err = e / (double)n;
        return true;
    };
    if (!pass(&best_err)) return RQ_ERR_HIP;
    if (objective) objective[0] = best_err;
    for (int it = 0; it < iters; ++it) {
        procrustes(M, D, R);
        double err = 0.0;
        if (!pass(&err)) return RQ_ERR_HIP;
        if (objective) objective[it + 1] = err;
        if (err < best_err) {
            best_err = err;
            best = R;
        }
    }
    for (size_t i = 0; i < best.size(); ++i) rot_out[i] = (float)best[i];
    return RQ_OK;
}

extern "C" rq_status rq_fit_rotation(const float *samples, int64_t n, int32_t head_dim, int32_t bits,
                                     int32_t group_size, int32_t meta_dtype, const float *rot0, int32_t iters,
                                     float *rot_out, double *objective) {
    if (!samples || !rot0 || !rot_out) return RQ_ERR_NULL;
    const int D = head_dim, G = group_size;
    if (n < 1 || D < 1 || D > 128 || G < 1 || D % G != 0 || iters < 0 || iters > 10000) return RQ_ERR_SHAPE;
    if (bits != 2 && bits != 4) return RQ_ERR_UNSUPPORTED;
    if (meta_dtype != RQ_DTYPE_F16 && meta_dtype != RQ_DTYPE_F32) return RQ_ERR_UNSUPPORTED;
    std::vector<double> X((size_t)n * D), R((size_t)D * D), M;
    for (size_t i = 0; i < X.size(); ++i) X[i] = (double)samples[i];
    for (size_t i = 0; i < R.size(); ++i) R[i] = (double)rot0[i];
    std::vector<double> best(R);
    double best_err = quant_error(X, n, D, R, G, bits, meta_dtype, nullptr);
    if (objective) objective[0] = best_err;
    for (int it = 0; it < iters; ++it) {
        quant_error(X, n, D, R, G, bits, meta_dtype, &M);
        procrustes(M, D, R);
        const double err = quant_error(X, n, D, R, G, bits, meta_dtype, nullptr);
        if (objective) objective[it + 1] = err;
        if (err < best_err) {
            best_err = err;
            best = R;
        }
    }
    for (size_t i = 0; i < best.size(); ++i) rot_out[i] = (float)best[i];
    return RQ_OK;
}
