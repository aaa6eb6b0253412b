// Contiguous-read bandwidth reference (rq_read_probe): the rate at which plain
// 16-byte vector loads stream a contiguous buffer from HBM, the roof against
// which the decode kernels' page pattern (rq_decode_stream_probe) and the
// decode kernels themselves are compared.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq.h"
#include "rq_device.h"

namespace rq {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeUnroll = 8;          // 16-byte loads in flight per lane
constexpr int kProbeWgPerCu = 8;

// Grid-stride over n 16-byte units: each lane keeps kProbeUnroll
// non-temporal loads in flight and folds every word into an XOR; the wave's
// XOR goes into sink word (4 * workgroup + wave) mod nsink with one atomic
// (order-independent: the XOR of all sink words is the XOR of all 32-bit
// words of the buffer). One word per wave keeps the atomics apart: thousands
// of them on one word serialize at the end of the kernel.
__global__ __launch_bounds__(256) void rq_read_probe_kernel(const u32x4 *__restrict__ p, size_t n, uint32_t *sink,
                                                            uint32_t nsink) {
    uint32_t acc = 0;
    const size_t block = (size_t)256 * kProbeUnroll;
    const size_t stride = (size_t)gridDim.x * block;
    size_t i = (size_t)blockIdx.x * block + threadIdx.x;
    for (; i + 256 * (kProbeUnroll - 1) < n; i += stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + 256 * u);
        // all loads issued before the first use (else the compiler waits for
        // the first ones while the rest are not yet in flight)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // the units of a last, partial block of this lane's stride
    for (; i < n; i += 256) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    int a[1] = {(int)acc};
    wave_reduce_n<1>(a, [](int x, int y) { return x ^ y; });
    if ((threadIdx.x & 63) == 0) atomicXor(sink + (blockIdx.x * 4u + (threadIdx.x >> 6)) % nsink, (uint32_t)a[0]);
}

int probe_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

}  // namespace
}  // namespace rq

extern "C" rq_status rq_read_probe(const void *buf, size_t bytes, uint32_t *sink, int32_t sink_words,
                                   const rq_decode_opts *opts, void *stream) {
    if (!sink || (bytes > 0 && !buf)) return RQ_ERR_NULL;
    if (bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0 || sink_words < 1) return RQ_ERR_SHAPE;
    const size_t n = bytes / 16;
    const int64_t want = (int64_t)rq::kProbeWgPerCu * rq::probe_cus();
    const int64_t need = (int64_t)((n + 256 * rq::kProbeUnroll - 1) / (256 * rq::kProbeUnroll));
    const int grid = (int)(need < want ? (need > 0 ? need : 1) : want);
    hipEvent_t e0 = opts ? (hipEvent_t)opts->event_main_begin : nullptr;
    hipEvent_t e1 = opts ? (hipEvent_t)opts->event_main_end : nullptr;
    hipExtLaunchKernelGGL(rq::rq_read_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, e0, e1, 0,
                          (const rq::u32x4 *)buf, n, sink, (uint32_t)sink_words);
    return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}
