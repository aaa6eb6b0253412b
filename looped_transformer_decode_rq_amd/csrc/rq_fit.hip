// Rotation fitting on the GPU: one pass of the alternation (see rq_fit.cpp)
// over the calibration rows in float64 -- rotate every row (y = R d), quantize
// it with the method's group quantizer (step (max-min)/(2^b-1) and offset min
// rounded to the metadata dtype, codes rounded to nearest even and clamped;
// ResidualQuant, arXiv 2610.10381 abstract and the rit.work summary, section
// on how each pass's KV cache is restored: rotated residuals in low-bit
// asymmetric quantization), and accumulate the squared quantization error and
// the Procrustes matrix M = sum_i yhat_i d_i^T. The orthogonal polar factor
// of M (a 128 x 128 SVD) stays on the host.
//
// Two kernels per pass, deterministic (no atomics: fixed partition and
// summation order):
//   rq_fit_pass    kFitBlocks workgroups, each over a contiguous run of rows
//                  in chunks of kFitRows; thread (c, kq) holds row c of R and
//                  of its partial M over the k-part kq of the channels, so
//                  both products run from registers against LDS rows
//   rq_fit_reduce  M and the error: the partials summed in workgroup order
#include "rq_device.h"
#include "rq_internal.h"

namespace rq {
namespace {

constexpr int kFitThreads = 512;
constexpr int kFitRows = 8;

struct FitPassArgs {
    const float *x;      // [n][D] calibration rows
    const double *r;     // [D][D] rotation, y = R d
    double *mpart;       // [nb][D][D] per-workgroup M
    double *epart;       // [nb] per-workgroup squared error
    int64_t n, rows_per_wg;
    int bits, G, meta;
};

__device__ __forceinline__ double meta_round_d(double x, int meta) {
    if (meta == RQ_DTYPE_F32) return (double)(float)x;
    return f16_bits_to_f64(f64_to_f16_bits(x));
}

template <int D>
__global__ __launch_bounds__(kFitThreads) void rq_fit_pass_kernel(FitPassArgs a) {
    constexpr int KQ = kFitThreads / D >= 8 ? 8 : 4;    // threads per channel (k-parts)
    constexpr int KL = D / KQ;                           // channels of one k-part
    static_assert(KQ >= 2 && KQ * kFitRows * D >= kFitThreads, "the k-part area also holds S, Z and the reduction");
    __shared__ double X[kFitRows][D];
    __shared__ double YP[KQ][kFitRows][D];               // partial y per k-part
    __shared__ double Y[kFitRows][D];                    // y, then yhat
    // once y is summed, the k-part area holds the step and offset of each
    // (row, group) (D / G per row), and at the end the error reduction
    auto S = YP[0];
    auto Z = YP[1];
    double *red = &YP[0][0][0];
    const int t = threadIdx.x;
    const bool act = t < KQ * D;
    const int c = t % D, kq = act ? t / D : 0;
    const double qmax = (double)((1 << a.bits) - 1);
    const int ng = D / a.G;
    double rr[KL], mm[KL];
#pragma unroll
    for (int k = 0; k < KL; ++k) {
        rr[k] = act ? a.r[(int64_t)c * D + kq * KL + k] : 0.0;
        mm[k] = 0.0;
    }
    double err = 0.0;
    const int64_t row0 = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row1 = min(a.n, row0 + a.rows_per_wg);
    for (int64_t c0 = row0; c0 < row1; c0 += kFitRows) {
        for (int i = t; i < kFitRows * D; i += kFitThreads) {
            const int r = i / D, k = i % D;
            X[r][k] = c0 + r < row1 ? (double)a.x[(c0 + r) * D + k] : 0.0;
        }
        __syncthreads();
        if (act) {
#pragma unroll
            for (int r = 0; r < kFitRows; ++r) {
                double s = 0.0;
#pragma unroll
                for (int k = 0; k < KL; ++k) s = fma(rr[k], X[r][kq * KL + k], s);
                YP[kq][r][c] = s;
            }
        }
        __syncthreads();
        for (int i = t; i < kFitRows * D; i += kFitThreads) {
            const int r = i / D, cc = i % D;
            double s = YP[0][r][cc];
#pragma unroll
            for (int q = 1; q < KQ; ++q) s += YP[q][r][cc];
            Y[r][cc] = s;
        }
        __syncthreads();
        for (int i = t; i < kFitRows * ng; i += kFitThreads) {
            const int r = i / ng, g = i % ng;
            double lo = Y[r][g * a.G], hi = lo;
            for (int j = 1; j < a.G; ++j) {
                lo = fmin(lo, Y[r][g * a.G + j]);
                hi = fmax(hi, Y[r][g * a.G + j]);
            }
            S[r][g] = meta_round_d((hi - lo) / qmax, a.meta);
            Z[r][g] = meta_round_d(lo, a.meta);
        }
        __syncthreads();
        for (int i = t; i < kFitRows * D; i += kFitThreads) {
            const int r = i / D, cc = i % D, g = cc / a.G;
            const double y = Y[r][cc], s = S[r][g], z = Z[r][g];
            const double code = s != 0.0 ? fmin(fmax(rint((y - z) / s), 0.0), qmax) : 0.0;
            const double yh = code * s + z;
            const bool live = c0 + r < row1;
            if (live) err = fma(yh - y, yh - y, err);
            Y[r][cc] = live ? yh : 0.0;
        }
        __syncthreads();
        if (act) {
#pragma unroll
            for (int r = 0; r < kFitRows; ++r) {
                const double yv = Y[r][c];
#pragma unroll
                for (int k = 0; k < KL; ++k) mm[k] = fma(yv, X[r][kq * KL + k], mm[k]);
            }
        }
        __syncthreads();
    }
    if (act) {
        double *mp = a.mpart + (int64_t)blockIdx.x * D * D + (int64_t)c * D + kq * KL;
#pragma unroll
        for (int k = 0; k < KL; ++k) mp[k] = mm[k];
    }
    red[t] = err;
    __syncthreads();
    for (int w = kFitThreads / 2; w > 0; w >>= 1) {
        if (t < w) red[t] += red[t + w];
        __syncthreads();
    }
    if (t == 0) a.epart[blockIdx.x] = red[0];
}

// m[i] = sum_b mpart[b][i] (i < D*D), err = sum_b epart[b], in workgroup order
__global__ __launch_bounds__(256) void rq_fit_reduce_kernel(const double *mpart, const double *epart, int nb,
                                                            int dd, double *m, double *err) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < dd) {
        double s = 0.0;
        for (int b = 0; b < nb; ++b) s += mpart[(int64_t)b * dd + i];
        m[i] = s;
    }
    if (i == 0) {
        double s = 0.0;
        for (int b = 0; b < nb; ++b) s += epart[b];
        *err = s;
    }
}

}  // namespace

hipError_t launch_fit_pass(const FitPass &p) {
    FitPassArgs a;
    a.x = p.x; a.r = p.r; a.mpart = p.mpart; a.epart = p.epart; a.n = p.n;
    a.rows_per_wg = ((p.n + kFitBlocks - 1) / kFitBlocks + kFitRows - 1) / kFitRows * kFitRows;
    a.bits = p.bits; a.G = p.G; a.meta = p.meta;
    const dim3 grid(kFitBlocks);
    switch (p.D) {
        case 64: hipLaunchKernelGGL(rq_fit_pass_kernel<64>, grid, dim3(kFitThreads), 0, p.stream, a); break;
        case 96: hipLaunchKernelGGL(rq_fit_pass_kernel<96>, grid, dim3(kFitThreads), 0, p.stream, a); break;
        case 128: hipLaunchKernelGGL(rq_fit_pass_kernel<128>, grid, dim3(kFitThreads), 0, p.stream, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int dd = p.D * p.D;
    hipLaunchKernelGGL(rq_fit_reduce_kernel, dim3((dd + 255) / 256), dim3(256), 0, p.stream, p.mpart, p.epart,
                       kFitBlocks, dd, p.m, p.err);
    return hipGetLastError();
}

}  // namespace rq
