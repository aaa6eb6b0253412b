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

// Direct per-loop baseline (layout mode RQ_MODE_DIRECT): one workgroup per
// (tile of 16 tokens, head, K|V x loop); each wave quantizes its tokens' rows
// of loop l at the loop's own bit width into loop l's record (no alpha).
template <bool KV_F32, bool META_F32>
__global__ __launch_bounds__(kThreads) void rq_direct_encode_kernel(EncArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = blockIdx.x, h = blockIdx.y;
    const int kv = blockIdx.z / a.L, l = blockIdx.z % a.L;
    const int D = a.D, H = a.H;
    const int c0 = 2 * lane, c1 = 2 * lane + 1;
    const bool active = c0 < D;
    for (int t = wave; t < kTT; t += kThreads / 64) {
        const int tg = tile * kTT + t;
        const bool tok = tg < a.T;
        const int64_t slot = tok ? a.slots[tg] : -1;
        const bool write = slot >= 0 && slot < (int64_t)a.nblk * 16;
        const int64_t blk = write ? slot / 16 : 0;
        const int off = write ? (int)(slot % 16) : 0;
        double x0 = 0.0, x1 = 0.0;
        if (tok && active) {
            const int64_t base = ((((int64_t)l * 2 + kv) * a.T + tg) * H + h) * D;
            x0 = (double)load_kv<KV_F32>(a.kv, base + c0);
            x1 = (double)load_kv<KV_F32>(a.kv, base + c1);
        }
        uint8_t *rec = a.pool + (blk * H + h) * a.slab + a.loop_off[l] + (int64_t)kv * a.rec[l];
        quantize_row<META_F32>(x0, x1, active, lane, D, a.G, a.bits[l], rec, a.code_bytes[l], off, write, kv == 1);
    }
}

}  // namespace

hipError_t launch_encode(const EncodeCall &c) {
    const Geom &g = *c.g;
    if (c.T <= 0) return hipSuccess;
    EncArgs a;
    fill_args(a, g, c.pool, c.kv_new, c.rot, c.slots, c.T);
    const bool kvf = g.kvdt == RQ_DTYPE_F32, mf = g.meta == RQ_DTYPE_F32;
    if (g.direct) {
        dim3 dgrid((c.T + kTT - 1) / kTT, g.H, 2 * g.L);
        if (kvf && mf) hipLaunchKernelGGL((rq_direct_encode_kernel<true, true>), dgrid, dim3(kThreads), 0, c.stream, a);
        else if (kvf) hipLaunchKernelGGL((rq_direct_encode_kernel<true, false>), dgrid, dim3(kThreads), 0, c.stream, a);
        else if (mf) hipLaunchKernelGGL((rq_direct_encode_kernel<false, true>), dgrid, dim3(kThreads), 0, c.stream, a);
        else hipLaunchKernelGGL((rq_direct_encode_kernel<false, false>), dgrid, dim3(kThreads), 0, c.stream, a);
        return hipGetLastError();
    }
    dim3 grid((c.T + kTT - 1) / kTT, g.H, 2 * (g.L > 1 ? g.L - 1 : 1));
    if (kvf && mf) hipLaunchKernelGGL((rq_encode_pack_kernel<true, true>), grid, dim3(kThreads), 0, c.stream, a);
    else if (kvf) hipLaunchKernelGGL((rq_encode_pack_kernel<true, false>), grid, dim3(kThreads), 0, c.stream, a);
    else if (mf) hipLaunchKernelGGL((rq_encode_pack_kernel<false, true>), grid, dim3(kThreads), 0, c.stream, a);
    else hipLaunchKernelGGL((rq_encode_pack_kernel<false, false>), grid, dim3(kThreads), 0, c.stream, a);
    return hipGetLastError();
}

}  // namespace rq
