// Uncompressed bf16 decode-attention baseline over a paged cache
// [num_blocks][H][16][D], one loop, with the same split-K structure as the
// packed path: one wave per (split of pages, head, sequence), four (D=96: two)
// lanes per token, scores with v_dot2_f32_bf16 (exact bf16 products), online
// softmax, V accumulated in fp32 registers, log-sum-exp combine with the
// current token.
#include <hip/hip_ext.h>

#include "rq_device.h"
#include "rq_internal.h"

namespace rq {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kWaves = 4;
constexpr float kRescaleThresh = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

struct Bf16SplitArgs {
    const uint16_t *kc, *vc, *q;
    const int32_t *block_table, *seq_lens;
    int H, nblk, max_blocks, nsplit, split_pages;
    float score_scale;
    float *partials;    // [B][H][nsplit][2 + D]
};

template <int NB>
__device__ __forceinline__ void load_words(const uint16_t *p, uint32_t *out) {
    static_assert(NB % 16 == 0, "");
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
        const uint4 v = ((const uint4 *)p)[i];
        out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
}

template <int D>
__global__ __launch_bounds__(256) void rq_bf16_split_kernel(Bf16SplitArgs a) {
    constexpr int LPT = (D == 96) ? 2 : 4, CPL = D / LPT, PPI = (64 / LPT) / 16;
    constexpr int NW = CPL / 2;   // 32-bit words (bf16 pairs) per lane
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x * kWaves + wave, h = blockIdx.y, b = blockIdx.z;
    if (split >= a.nsplit) return;
    const int H = a.H;
    int seq = a.seq_lens[b];
    seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
    const int npages = (seq + 15) >> 4;
    const int p0 = split * a.split_pages, p1 = min(npages, p0 + a.split_pages);
    if (p0 >= p1) return;
    const int tok_i = lane / LPT, q4 = lane % LPT, page_in_step = tok_i >> 4, tok = tok_i & 15;

    uint32_t qw[NW];
    load_words<CPL * 2>(a.q + ((int64_t)b * H + h) * D + q4 * CPL, qw);
    const int32_t *table = a.block_table + (int64_t)b * a.max_blocks;

    float m = kNegInf, lsum = 0.f, acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;

    for (int p = p0; p < p1; p += PPI) {
        const int pp = p + page_in_step;
        bool valid = pp < p1;
        int64_t blk = valid ? (int64_t)table[pp] : 0;
        if (blk < 0 || blk >= a.nblk) { blk = 0; valid = false; }
        valid = valid && (pp * 16 + tok < seq);
        const int64_t off = ((blk * H + h) * 16 + tok) * D + q4 * CPL;
        uint32_t kw[NW], vw[NW];
        load_words<CPL * 2>(a.kc + off, kw);
        load_words<CPL * 2>(a.vc + off, vw);
        float d = 0.f;
#pragma unroll
        for (int k = 0; k < NW; ++k)
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[k]), __builtin_bit_cast(bf16x2, kw[k]), d, false);
        float score = group_sum<LPT>(d) * a.score_scale;
        score = valid ? score : kNegInf;
        if (__any(score > m + kRescaleThresh)) {
            const float mn = fmaxf(m, wave_max(score));
            const float f = fast_exp2(m - mn);
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc[i] *= f;
            lsum *= f;
            m = mn;
        }
        // a masked token weighs 0 (also while m is still -inf)
        const float w = valid ? fast_exp2(score - m) : 0.f;
        lsum += w;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            acc[2 * k] = fmaf(w, __uint_as_float(vw[k] << 16), acc[2 * k]);
            acc[2 * k + 1] = fmaf(w, __uint_as_float(vw[k] & 0xFFFF0000u), acc[2 * k + 1]);
        }
    }
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[i] += __shfl_xor(acc[i], off, 64);
        lsum += __shfl_xor(lsum, off, 64);
    }
    if (lane < LPT) {
        float *out = a.partials + (((int64_t)b * H + h) * a.nsplit + split) * (2 + D);
        if (lane == 0) { out[0] = m; out[1] = lsum; }
#pragma unroll
        for (int i = 0; i < CPL; ++i) out[2 + q4 * CPL + i] = acc[i];
    }
}

struct Bf16CombineArgs {
    const float *partials;
    int nsplit, split_pages, max_blocks, H;
    const int32_t *seq_lens;
    const uint16_t *q, *tail_k, *tail_v;
    float *out;
    float score_scale;
};

// one wave per (head, sequence)
template <int D>
__global__ __launch_bounds__(64) void rq_bf16_combine_kernel(Bf16CombineArgs a) {
    const int lane = threadIdx.x, h = blockIdx.x, b = blockIdx.y, H = a.H;
    const int64_t row = (int64_t)b * H + h;
    int seq = a.seq_lens[b];
    seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
    const int ns = (((seq + 15) >> 4) + a.split_pages - 1) / a.split_pages;
    const float *P = a.partials + row * a.nsplit * (2 + D);
    const int c0 = lane, c1 = lane + 64;
    float st = kNegInf;
    if (a.tail_k) {
        float d = 0.f;
        if (c0 < D) d += bf16_to_f32(a.q[row * D + c0]) * bf16_to_f32(a.tail_k[row * D + c0]);
        if (c1 < D) d += bf16_to_f32(a.q[row * D + c1]) * bf16_to_f32(a.tail_k[row * D + c1]);
        st = wave_sum(d) * a.score_scale;
    }
    float mloc = kNegInf;
    for (int s = lane; s < ns; s += 64) mloc = fmaxf(mloc, P[(int64_t)s * (2 + D)]);
    const float M = fmaxf(wave_max(mloc), st);
    float o0 = 0.f, o1 = 0.f;
    if (M != kNegInf) {
        float lloc = 0.f;
        for (int s = lane; s < ns; s += 64) lloc += fast_exp2(P[(int64_t)s * (2 + D)] - M) * P[(int64_t)s * (2 + D) + 1];
        float lsum = wave_sum(lloc);
        // eight partials per round with their loads in flight together
        // (indices past the last partial re-read it with weight 0; columns
        // beyond D read column D-1 and are never stored)
        const int k0 = min(c0, D - 1), k1 = min(c1, D - 1);
        for (int s0 = 0; s0 < ns; s0 += 8) {
            float e[8], v0[8], v1[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float *ps = P + (int64_t)min(s0 + u, ns - 1) * (2 + D);
                const float eu = fast_exp2(ps[0] - M);
                e[u] = s0 + u < ns ? eu : 0.f;
                v0[u] = ps[2 + k0];
                v1[u] = ps[2 + k1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                o0 = fmaf(e[u], v0[u], o0);
                o1 = fmaf(e[u], v1[u], o1);
            }
        }
        if (a.tail_k) {
            const float pt = fast_exp2(st - M);
            lsum += pt;
            if (c0 < D) o0 = fmaf(pt, bf16_to_f32(a.tail_v[row * D + c0]), o0);
            if (c1 < D) o1 = fmaf(pt, bf16_to_f32(a.tail_v[row * D + c1]), o1);
        }
        const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
        o0 *= inv; o1 *= inv;
    }
    if (c0 < D) a.out[row * D + c0] = o0;
    if (c1 < D) a.out[row * D + c1] = o1;
}

// kv_new [2][T][H][D] -> caches at their slots; 16-byte chunks
__global__ __launch_bounds__(256) void rq_bf16_write_kernel(uint16_t *kc, uint16_t *vc, const uint16_t *kv,
                                                            const int64_t *slots, int T, int H, int D, int nblk) {
    const int t = blockIdx.x;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= (int64_t)nblk * 16) return;
    const int64_t blk = slot / 16, off = slot % 16;
    const int chunks = H * D / 8;
    for (int e = threadIdx.x; e < 2 * chunks; e += blockDim.x) {
        const int kvi = e / chunks, rem = e % chunks;
        const int h = rem / (D / 8), c8 = rem % (D / 8);
        const uint4 v = *(const uint4 *)(kv + (((int64_t)kvi * T + t) * H + h) * D + 8 * c8);
        uint16_t *dst = (kvi ? vc : kc) + ((blk * H + h) * 16 + off) * D + 8 * c8;
        *(uint4 *)dst = v;
    }
}

template <int D>
hipError_t launch_bf16_d(const Bf16Call &c) {
    Bf16SplitArgs s;
    s.kc = c.kc; s.vc = c.vc; s.q = c.q; s.block_table = c.block_table; s.seq_lens = c.seq_lens;
    s.H = c.H; s.nblk = c.nblk; s.max_blocks = c.max_blocks; s.nsplit = c.nsplit; s.split_pages = c.split_pages;
    s.score_scale = c.softmax_scale * kLog2e;
    s.partials = c.partials;
    dim3 grid((c.nsplit + kWaves - 1) / kWaves, c.H, c.B);
    // the optional events are stamped by the kernel's own dispatch
    hipExtLaunchKernelGGL((rq_bf16_split_kernel<D>), grid, dim3(256), 0, c.stream, c.ev_begin, c.ev_end, 0, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    Bf16CombineArgs ca;
    ca.partials = c.partials; ca.nsplit = c.nsplit; ca.split_pages = c.split_pages; ca.max_blocks = c.max_blocks;
    ca.H = c.H; ca.seq_lens = c.seq_lens; ca.q = c.q; ca.tail_k = c.tail_k; ca.tail_v = c.tail_v;
    ca.out = c.out; ca.score_scale = s.score_scale;
    hipLaunchKernelGGL((rq_bf16_combine_kernel<D>), dim3(c.H, c.B), dim3(64), 0, c.stream, ca);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_decode(const Bf16Call &c) {
    if (c.B <= 0) return hipSuccess;
    switch (c.D) {
        case 64: return launch_bf16_d<64>(c);
        case 96: return launch_bf16_d<96>(c);
        case 128: return launch_bf16_d<128>(c);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bf16_write(int H, int D, int nblk, uint16_t *kc, uint16_t *vc, const uint16_t *kv_new,
                             const int64_t *slots, int T, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(rq_bf16_write_kernel, dim3(T), dim3(256), 0, stream, kc, vc, kv_new, slots, T, H, D, nblk);
    return hipGetLastError();
}

}  // namespace rq
