// Encoder / packer: compresses tokens once their final loop has run and
// scatters them into the paged pool.
//
// Method: ResidualQuant (arXiv 2610.10381, abstract) and the rit.work summary,
// section on how each pass is restored -- final-loop reference in INT4; for
// every other loop the least-squares scale of the reference, subtraction,
// channel-space rotation and low-bit asymmetric quantization with tunable step
// and offset; the compressed write is deferred until after the final pass.
//
// Everything that decides a code is computed in float64 so that codes and
// metadata are a deterministic function of the inputs up to the summation
// order of two dot products and one rotation: alpha = <x,ref>/<ref,ref>,
// d = fma(-alpha_stored, ref, x), r = R d on the f64 matrix cores, group
// min/max, step = (max-min)/(2^b-1), all casts round-to-nearest-even.
//
// One workgroup (4 waves) per (tile of 16 tokens, head, K|V, residual loop);
// the workgroup of residual loop 0 also writes the reference record. Lanes
// own two adjacent channels. The rotation of the 16 residual rows is a
// [16 x D] x [D x D]^T product on v_mfma_f64_16x16x4f64; R is read from
// global memory (L2-resident), the rows live in LDS.
#include "rq_encode_body.h"

namespace rq {
namespace {

using namespace enc;

template <bool KV_F32, bool META_F32>
__global__ __launch_bounds__(kThreads) void rq_encode_pack_kernel(EncArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kEncLdsBytes];
    encode_item<KV_F32, META_F32>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds, kThreads / 64);
}

}  // namespace

hipError_t launch_encode(const EncodeCall &c) {
    const Geom &g = *c.g;
    if (c.T <= 0) return hipSuccess;
    EncArgs a;
    fill_args(a, g, c.pool, c.kv_new, c.rot, c.slots, c.T);
    dim3 grid((c.T + kTT - 1) / kTT, g.H, 2 * (g.L > 1 ? g.L - 1 : 1));
    const bool kvf = g.kvdt == RQ_DTYPE_F32, mf = g.meta == RQ_DTYPE_F32;
    if (kvf && mf) hipLaunchKernelGGL((rq_encode_pack_kernel<true, true>), grid, dim3(kThreads), 0, c.stream, a);
    else if (kvf) hipLaunchKernelGGL((rq_encode_pack_kernel<true, false>), grid, dim3(kThreads), 0, c.stream, a);
    else if (mf) hipLaunchKernelGGL((rq_encode_pack_kernel<false, true>), grid, dim3(kThreads), 0, c.stream, a);
    else hipLaunchKernelGGL((rq_encode_pack_kernel<false, false>), grid, dim3(kThreads), 0, c.stream, a);
    return hipGetLastError();
}

}  // namespace rq
