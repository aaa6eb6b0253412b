// Decode attention over the packed, paged ResidualQuant cache.
//
// Reconstruction of loop l (ResidualQuant, arXiv 2610.10381 abstract; rit.work
// summary, section on how each pass is restored): x_hat = alpha*ref_hat +
// R^T res_hat, ref_hat = c*s + z (INT4), res_hat = c*s + z (INT2/INT4).
// Attention never materializes x_hat (the summary: reference and differences
// are rebuilt in small blocks inside attention, nothing decompressed is written
// back). It uses two exact identities of that formula:
//   q . x_hat = alpha*(q . ref_hat) + (R q) . res_hat
//   sum_t p_t x_hat_t = sum_t p_t alpha_t ref_hat_t + R^T sum_t p_t res_hat_t
// so the query is rotated once, V is accumulated in the rotated space, and
// R_V^T is applied once per output row.
//
// Three kernels per request:
//   rq_qprep     per (loop call, head, 16 sequences): q' = R_K q on the f32
//                matrix cores; q and q' are turned into fixed point with one
//                power-of-two scale per lane slice of channels (24 bits for q,
//                20 for q'), split into signed 4-bit limbs laid out for
//                v_dot8_i32_i4.
//   rq_split     per (split of pages, head, sequence) one wave: walks the
//                block table, loads each page's packed codes and metadata with
//                wide coalesced loads, scores tokens with integer dot products
//                of codes x query limbs (exact integer sums), runs the online
//                softmax, accumulates V in registers and writes a partial
//                (m, l, acc_ref[D], acc_res[D]).
//   rq_combine   per (head, loop call, 16 sequences): log-sum-exp merge of the
//                partials and the uncompressed tail token, then
//                out = acc_ref/l + R_V^T (acc_res/l) on the f32 matrix cores.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "rq_device.h"
#include "rq_encode_body.h"
#include "rq_internal.h"
#include "rq_vmfma.h"

namespace rq {
namespace {

constexpr int kWaves = 4;
constexpr float kRescaleThresh = 8.0f;   // log2 units: rescale when a score beats m by 2^8
constexpr float kLog2e = 1.4426950408889634f;

// Largest magnitude of nl balanced base-16 digits (each -8..7): 7 * (16^nl - 1) / 15.
// A fixed-point value v is stored as the nibbles of v + 8 * (16^nl - 1) / 15
// (every nibble u_d of that sum gives the digit u_d - 8, i.e. the 4-bit
// two's-complement nibble u_d ^ 8).
__host__ __device__ constexpr int qmax_fixed(int nl) { return 7 * (int)(((1u << (4 * nl)) - 1u) / 15u); }
__host__ __device__ constexpr int digit_offset(int nl) { return 8 * (int)(((1u << (4 * nl)) - 1u) / 15u); }
static_assert(kQueryLimbs == 6 && kRotLimbs == 5, "limb planes below: 4 + 2 (q) and 4 + 1 (q')");

template <int D> struct Lanes {
    static constexpr int LPT = (D == 96) ? 2 : 4;   // lanes per token
    static constexpr int CPL = D / LPT;             // channels per lane
    static constexpr int TPW = 64 / LPT;            // tokens per wave step
    static constexpr int PPI = TPW / 16;            // pages per wave step
    static constexpr int NDW = CPL / 8;             // limb dwords per lane per limb
};

// ---------------------------------------------------------------- qprep
struct QPrepArgs {
    const void *q;          // [n][B][H][D]
    const float *rot;       // [H][2][D][D]
    uint8_t *qpack;         // [n][B][H][qpack_bytes]
    int B, H;
    int rb[RQ_MAX_LOOPS];   // residual bits of call i, 0 = reference loop
    int ro[RQ_MAX_LOOPS];   // limb order of q itself for call i: 4, or 2 for a direct INT2 loop
};

// Channel covered by nibble n of limb dword (q4, k) in the order the split
// kernel consumes codes: INT4 words hold 8 consecutive channels; an INT2 word
// (16 channels) is consumed as its even then its odd channels.
template <int D>
__device__ __forceinline__ int limb_channel(int q4, int k, int n, int rb) {
    constexpr int CPL = Lanes<D>::CPL;
    if (rb == 2) return q4 * CPL + 16 * (k >> 1) + 2 * n + (k & 1);
    return q4 * CPL + 8 * k + n;
}

// Sequences per workgroup of the query prep and of the combine (one wave
// each): small workgroups spread these latency-bound kernels over more CUs.
constexpr int kPrepRows = 4;

// One workgroup per (head, loop call, kPrepRows sequences); one wave per sequence.
template <int D, bool KV_F32>
__global__ __launch_bounds__(64 * kPrepRows) void rq_qprep_kernel(QPrepArgs a) {
    using Ln = Lanes<D>;
    constexpr int QS = D + 1, RW = kPrepRows;
    constexpr int NT = (D / 16 + RW - 1) / RW;    // column tiles of the rotation per wave
    __shared__ float Q[16 * QS];                  // rows RW..15 zero: the A operand has 16 rows
    __shared__ float QR[RW * QS];
    __shared__ int QI[RW][2][D];

    const int lane = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int h = blockIdx.x, i = blockIdx.y, tile = blockIdx.z;
    const int rb = a.rb[i];
    const int B = a.B, H = a.H;
    const int b = tile * RW + r;
    const bool row_ok = b < B;

    // q' = R_K q for the RW rows: [16 x D] x R_K^T. v_mfma_f32_16x16x4f32:
    // lane l supplies A[l%16][k], B[k][l%16] for its k-slot l/16 and receives
    // D[4*(l/16)+v][l%16]; wave r computes the column tiles r, r + RW, ...
    // Step kk gives slot k0 = l/16 the channel k = (D/4) k0 + kk, so that a
    // lane's B operands are D/4 consecutive floats of row n of R_K (vector
    // loads). They are loaded first, so that their latency overlaps the
    // query loads.
    float rk[NT][D / 4];
    if (rb != 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int ct = r + RW * j;
            if (ct < D / 16) {
                const float4 *RK = (const float4 *)(a.rot + ((int64_t)h * 2 + 0) * D * D +
                                                    (int64_t)(ct * 16 + (lane & 15)) * D + (lane >> 4) * (D / 4));
#pragma unroll
                for (int k4 = 0; k4 < D / 16; ++k4) {
                    const float4 v = RK[k4];
                    rk[j][4 * k4] = v.x; rk[j][4 * k4 + 1] = v.y; rk[j][4 * k4 + 2] = v.z; rk[j][4 * k4 + 3] = v.w;
                }
            }
        }
    }
    for (int c = lane; c < D; c += 64)
        Q[r * QS + c] = row_ok ? load_kv<KV_F32>(a.q, (((int64_t)i * B + b) * H + h) * D + c) : 0.0f;
    for (int e = threadIdx.x; e < (16 - RW) * QS; e += 64 * RW) Q[RW * QS + e] = 0.0f;
    __syncthreads();
    if (rb != 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int ct = r + RW * j;
            if (ct < D / 16) {
                // four independent accumulation chains (the products' latency overlaps)
                floatx4 c4[4] = {};
#pragma unroll
                for (int kk = 0; kk < D / 4; ++kk) {
                    const int k = (lane >> 4) * (D / 4) + kk;
                    c4[kk & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(Q[(lane & 15) * QS + k], rk[j][kk], c4[kk & 3],
                                                                      0, 0, 0);
                }
                const floatx4 c = (c4[0] + c4[1]) + (c4[2] + c4[3]);
                for (int v = 0; v < 4; ++v)
                    if (4 * (lane >> 4) + v < RW) QR[(4 * (lane >> 4) + v) * QS + ct * 16 + (lane & 15)] = c[v];
            }
        }
    }
    __syncthreads();

    // Fixed point per lane slice (the CPL channels one lane of the split
    // kernels holds): v = rint(x * 2^s) with the largest s that keeps every
    // |v| of the slice within the range of the limbs. A large channel then
    // coarsens only its own slice, and 24 bits (q) / 20 bits (q') keep the
    // small channels of that slice: bf16 values of q are exact down to
    // 2^-15 of their slice's largest magnitude.
    // All 2 LPT maxima (q and q' per slice) in one reduction, likewise the
    // slices' sums of the fixed-point values below.
    constexpr int LPT = Ln::LPT;
    const int t0 = lane / Ln::CPL, t1 = (lane + 64) / Ln::CPL;
    float x[2][2], am[2 * LPT];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const float *src = which == 0 ? Q : QR;
        const bool on = which == 0 || rb != 0;
        x[which][0] = (on && lane < D) ? src[r * QS + lane] : 0.f;
        x[which][1] = (on && lane + 64 < D) ? src[r * QS + lane + 64] : 0.f;
#pragma unroll
        for (int t = 0; t < LPT; ++t)
            am[which * LPT + t] = fmaxf(t0 == t ? fabsf(x[which][0]) : 0.f, t1 == t ? fabsf(x[which][1]) : 0.f);
    }
    wave_max_n(am);
    int S[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    int ps[2 * LPT];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const int qmax = qmax_fixed(which == 0 ? kQueryLimbs : kRotLimbs);
        int s0 = 0, s1 = 0;
#pragma unroll
        for (int t = 0; t < LPT; ++t) {
            const float amax = am[which * LPT + t];
            int sh = 0;
            if (amax > 0.f) {
                int e;
                frexpf(amax, &e);                       // amax in [2^(e-1), 2^e)
                sh = 31 - __builtin_clz((unsigned)qmax) - e;   // amax * 2^sh < 2^floor(log2 qmax)
                if (ldexpf(amax, sh + 1) <= (float)qmax) sh += 1;
            }
            S[which][t] = sh;
            s0 = t0 == t ? sh : s0;
            s1 = t1 == t ? sh : s1;
        }
        const int v0 = (int)rintf(ldexpf(x[which][0], s0)), v1 = (int)rintf(ldexpf(x[which][1], s1));
        if (lane < D) QI[r][which][lane] = v0;
        if (lane + 64 < D) QI[r][which][lane + 64] = v1;
#pragma unroll
        for (int t = 0; t < LPT; ++t) ps[which * LPT + t] = (t0 == t ? v0 : 0) + (t1 == t ? v1 : 0);
    }
    wave_sum_n(ps);                                     // |sum| < 2^31
    __syncthreads();
    if (!row_ok) return;
    uint8_t *qp = a.qpack + (((int64_t)i * B + b) * H + h) * qpack_bytes(D);
    // per (which, slice): the sum of the slice's fixed-point values and the
    // slice's scale 2^-s
    if (lane == 0) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const bool on = which == 0 || rb != 0;
#pragma unroll
            for (int t = 0; t < LPT; ++t) {
                ((int *)(qp + 16 + 16 * which))[t] = ps[which * LPT + t];
                ((float *)(qp + 48 * which))[t] = on ? ldexpf(1.0f, -S[which][t]) : 0.0f;
            }
        }
    }
    // Limb words. Per quantity (q, then q'), plane A holds limbs 0..3 as one
    // 16-byte entry per (slice q4, dword k) and plane B the remaining limbs
    // (2 for q, 1 for q') as one 8- or 4-byte entry per (q4, k). Nibble n of
    // the word of (limb, q4, k) is the digit of channel limb_channel(q4, k, n).
    for (int which = 0; which < 2; ++which) {
        if (which == 1 && rb == 0) break;
        const int nl = which == 0 ? kQueryLimbs : kRotLimbs;
        const int order = which == 0 ? a.ro[i] : rb;
        const int off = digit_offset(nl);
        uint32_t *base = (uint32_t *)(qp + 64 + (which == 0 ? 0 : kQueryLimbs * D / 2));
        for (int dw = lane; dw < nl * D / 8; dw += 64) {
            int limb, e;
            if (dw < D / 2) {
                limb = dw & 3; e = dw >> 2;
            } else {
                const int nb = nl - 4, j = dw - D / 2;
                limb = 4 + j % nb; e = j / nb;
            }
            const int k = e % Ln::NDW, q4 = e / Ln::NDW;
            uint32_t word = 0;
            for (int nn = 0; nn < 8; ++nn) {
                const uint32_t u = (uint32_t)(QI[r][which][limb_channel<D>(q4, k, nn, order)] + off);
                word |= (((u >> (4 * limb)) & 15u) ^ 8u) << (4 * nn);
            }
            base[dw] = word;
        }
    }
}

// ------------------------------------------------------------------ split
struct SplitArgs {
    const uint8_t *pool;
    int64_t slab;
    int H, nblk, G;
    int ref_off, ref_rec, ref_code_bytes;
    int res_off, res_rec, res_code_bytes;
    int meta_bytes;
    const int32_t *block_table;
    int max_blocks;
    const int32_t *seq_lens;
    const uint8_t *qpack;   // this call: [B][H][qpack_bytes]
    float *partials;        // this call: [B][H][nwg][2 + 2D]
    int nsplit, split_pages;
    int nwg;                // split workgroups per (sequence, head): the partials' row stride
    float score_scale;      // softmax_scale * log2(e)
    // encode work items riding in this launch (reference-loop kernel only):
    // workgroups with blockIdx.x >= enc_x0 run item (blockIdx.x - enc_x0) *
    // gridDim.z + blockIdx.z of enc_items, for head blockIdx.y
    int enc_x0, enc_items, enc_kvf;
    enc::EncArgs enc;
};

template <int NB>
__device__ __forceinline__ void load_bytes(const uint8_t *p, uint32_t *out) {
    // NB bytes, 4-byte granules; widest aligned vector loads the offsets allow
    static_assert(NB % 4 == 0, "");
    if constexpr (NB % 16 == 0) {
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            uint4 v = ((const uint4 *)p)[i];
            out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
        }
    } else if constexpr (NB % 8 == 0) {
#pragma unroll
        for (int i = 0; i < NB / 8; ++i) {
            uint2 v = ((const uint2 *)p)[i];
            out[2 * i] = v.x; out[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NB / 4; ++i) out[i] = ((const uint32_t *)p)[i];
    }
}

template <bool META_F32>
__device__ __forceinline__ void load_sz(const uint8_t *p, float &s, float &z) {
    if constexpr (META_F32) {
        const float2 v = *(const float2 *)p;
        s = v.x; z = v.y;
    } else {
        const uint32_t v = *(const uint32_t *)p;
        s = f16_to_f32((uint16_t)(v & 0xFFFF));
        z = f16_to_f32((uint16_t)(v >> 16));
    }
}

template <bool META_F32>
__device__ __forceinline__ float load_meta1(const uint8_t *p) {
    if constexpr (META_F32) return *(const float *)p;
    else return f16_to_f32(*(const uint16_t *)p);
}

__device__ __forceinline__ float ubyte(uint32_t x, int j) { return (float)((x >> (8 * j)) & 0xFFu); }

// sum of the 8 products of signed nibbles of a and b, plus c: the
// three-operand v_dot8_i32_i4, written out so that a chain can start from
// the inline constant 0 (the builtin is lowered to the accumulate-in-place
// form, which needs a register zeroed first)
__device__ __forceinline__ int sdot8(int a, int b, int c) {
    int r;
    __asm__("v_dot8_i32_i4 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ int sdot8_0(int a, int b) {
    int r;
    __asm__("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Query limbs of one lane slice as the split kernels hold them: per dword k
// of channels, limbs 0..3 in `lo[k]` and the remaining NL - 4 limbs in
// `hi[k]` (uint2 for the query, one uint for the rotated query).
template <int NL> struct HiLimbs;
template <> struct HiLimbs<6> { using T = uint2; };
template <> struct HiLimbs<5> { using T = uint32_t; };

__device__ __forceinline__ int hi_limb(uint2 v, int j) { return (int)(j == 0 ? v.x : v.y); }
__device__ __forceinline__ int hi_limb(uint32_t v, int) { return (int)v; }

// Sum of the digit sums a_d weighted by 16^d, as a float: exact in int32 up to
// five limbs (|a_d| <= 8 * 8 * 48); six limbs are combined as two exact
// three-limb halves (one fp32 rounding, relative 2^-24).
template <int NL>
__device__ __forceinline__ float combine_limbs(const int (&a)[NL]) {
    if constexpr (NL == 6) {
        const int lo = a[0] + 16 * a[1] + 256 * a[2];
        const int hi = a[3] + 16 * a[4] + 256 * a[5];
        return fmaf(4096.f, (float)hi, (float)lo);
    } else {
        return (float)(a[0] + 16 * a[1] + 256 * a[2] + 4096 * a[3] + 65536 * a[4]);
    }
}

// Dot of 4-bit codes (XOR 8 turns 0..15 into signed -8..7) with the query
// limbs: returns sum_i v_i * (c_i - 8) over the lane's channels, v_i the
// fixed-point query.
template <int NW, int NL>
__device__ __forceinline__ float dot_int4(const uint32_t *codes, const uint4 *lo,
                                          const typename HiLimbs<NL>::T *hi) {
    int a[NL];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const int w = (int)(codes[k] ^ 0x88888888u);
        const uint4 q = lo[k];
        const int l4[4] = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
#pragma unroll
        for (int d = 0; d < NL; ++d) {
            const int ql = d < 4 ? l4[d & 3] : hi_limb(hi[k], d - 4);
            a[d] = k == 0 ? sdot8_0(ql, w) : sdot8(ql, w, a[d]);
        }
    }
    return combine_limbs<NL>(a);
}

// Same for 2-bit codes: a word of 16 crumbs is split into its even and odd
// channels, each widened to nibbles (values 0..3 need no offset); returns
// sum_i v_i * c_i.
template <int NW, int NL>
__device__ __forceinline__ float dot_int2(const uint32_t *codes, const uint4 *lo,
                                          const typename HiLimbs<NL>::T *hi) {
    int a[NL];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const int ev = (int)(codes[k] & 0x33333333u);
        const int od = (int)((codes[k] >> 2) & 0x33333333u);
        const uint4 qe = lo[2 * k], qo = lo[2 * k + 1];
        const int le[4] = {(int)qe.x, (int)qe.y, (int)qe.z, (int)qe.w};
        const int lodd[4] = {(int)qo.x, (int)qo.y, (int)qo.z, (int)qo.w};
#pragma unroll
        for (int d = 0; d < NL; ++d) {
            const int qle = d < 4 ? le[d & 3] : hi_limb(hi[2 * k], d - 4);
            const int qlo = d < 4 ? lodd[d & 3] : hi_limb(hi[2 * k + 1], d - 4);
            a[d] = k == 0 ? sdot8_0(qle, ev) : sdot8(qle, ev, a[d]);
            a[d] = sdot8(qlo, od, a[d]);
        }
    }
    return combine_limbs<NL>(a);
}

// Sum over each group of LPT consecutive lanes (LPT = 2 or 4, all lanes
// active), with the DPP swizzle on the add's first operand. The s_nop covers
// the wait states a DPP read needs after the VALU write of its source.
template <int LPT>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(LPT == 2 || LPT == 4, "");
    float r;
    __asm__("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
            : "=v"(r) : "v"(v));
    if constexpr (LPT == 4) {
        float t;
        __asm__("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                : "=v"(t) : "v"(r));
        r = t;
    }
    return r;
}

__device__ __forceinline__ void sz_of(float2 v, float &s, float &z) { s = v.x; z = v.y; }
__device__ __forceinline__ void sz_of(uint32_t v, float &s, float &z) {
    s = f16_to_f32((uint16_t)(v & 0xFFFF));
    z = f16_to_f32((uint16_t)(v >> 16));
}

// ---- shared per-token arithmetic of the split kernels

// Query state of one (loop call, sequence, head) held by each lane for its
// slice of channels: the fixed-point scales and value sums of q and of
// q' = R_K q, and their limbs (planes A and B of the query record).
template <int D>
struct QueryRegs {
    float sc_ref, sc_res;
    int qs_ref, qs_res;
    uint4 lrv[Lanes<D>::NDW], lsv[Lanes<D>::NDW];
    uint2 lrh[Lanes<D>::NDW];
    uint32_t lsh[Lanes<D>::NDW];
};

// Online-softmax state of one wave: running max (log2 units) and, per lane,
// its token slots' sum of weights and per-group zero terms; the V sums of
// the whole wave in matrix accumulators: rows 4g, 4g+1 of column group m
// sum the reference term, rows 4g+2, 4g+3 the rotated residual (the A
// operand of the reference codes is zero in the residual rows and vice
// versa, so both share one accumulator).
template <int D>
struct SplitState {
    float m, lsum, zr, zs;
    floatx4 v[D / 16];
};

// Bytes of the per-wave weight scratch (A operand rows) of one page.
constexpr int kWScratch = 16 * 16 * 2;

template <int D, bool RES>
__device__ __forceinline__ void load_query(const uint8_t *qp, int q4, QueryRegs<D> &q) {
    using Ln = Lanes<D>;
    q.sc_ref = ((const float *)qp)[q4];
    q.sc_res = ((const float *)(qp + 48))[q4];
    q.qs_ref = ((const int *)(qp + 16))[q4];
    q.qs_res = ((const int *)(qp + 32))[q4];
    const uint4 *qa = (const uint4 *)(qp + 64);
    const uint2 *qb = (const uint2 *)(qp + 64 + 2 * D);
    const uint4 *ra = (const uint4 *)(qp + 64 + kQueryLimbs * D / 2);
    const uint32_t *rbp = (const uint32_t *)(qp + 64 + kQueryLimbs * D / 2 + 2 * D);
#pragma unroll
    for (int k = 0; k < Ln::NDW; ++k) {
        q.lrv[k] = qa[q4 * Ln::NDW + k];
        q.lrh[k] = qb[q4 * Ln::NDW + k];
    }
    if constexpr (RES) {
#pragma unroll
        for (int k = 0; k < Ln::NDW; ++k) {
            q.lsv[k] = ra[q4 * Ln::NDW + k];
            q.lsh[k] = rbp[q4 * Ln::NDW + k];
        }
    }
    // Make the compiler complete these loads here: its wait-count tracking
    // does not see the direct-to-LDS loads issued later, so a wait it placed
    // at a first use inside the page loop would also drain the ring.
#pragma unroll
    for (int k = 0; k < Ln::NDW; ++k)
        __asm__ volatile("" ::"v"(q.lrv[k].x), "v"(q.lrv[k].y), "v"(q.lrv[k].z), "v"(q.lrv[k].w),
                         "v"(q.lrh[k].x), "v"(q.lrh[k].y));
    if constexpr (RES) {
#pragma unroll
        for (int k = 0; k < Ln::NDW; ++k)
            __asm__ volatile("" ::"v"(q.lsv[k].x), "v"(q.lsv[k].y), "v"(q.lsv[k].z), "v"(q.lsv[k].w),
                             "v"(q.lsh[k]));
    }
    __asm__ volatile("" ::"v"(q.qs_ref), "v"(q.qs_res), "v"(q.sc_ref), "v"(q.sc_res));
}

template <int D>
__device__ __forceinline__ void init_state(SplitState<D> &s) {
    s.m = kNegInf; s.lsum = 0.f; s.zr = 0.f; s.zs = 0.f;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) s.v[i] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// One page step of one wave (LPT lanes per token, PPI pages): score this
// lane's token from the K codes in LDS, fold it into the online softmax, and
// add every token's V to the matrix accumulators.
//   ck, mkr, mvr  this lane's reference K code bytes and (scale, zero) of K / V
//   rk            this lane's residual K code bytes (RB != 0)
//   mks, mvs      residual (scale, zero); aks, avs residual alphas (RB != 0)
//   vref, vres    V code blocks of page 0 of the step (page pg at + pg*stride)
//   wsc           this wave's weight scratch (PPI pages of kWScratch bytes);
//                 may alias the step's code bytes, which are all read first
//   SHR           shared reference rows (multi-loop): the reference weights go
//                 to rows 2*(sha_pair + g) + {hi, lo} of `sha` instead of the
//                 wave's own product; the reference product and the rescale
//                 of those rows are done by the wave that owns them, which
//                 reads this step's factor from `fr` (1 without a rescale).
//                 The accumulators are then rescaled only when RB != 0.
template <int D, int RB, bool META_F32, int G, int REFB = 4, bool SHR = false>
__device__ __forceinline__ void token_step(const uint8_t *ck, const uint8_t *mkr, const uint8_t *mvr,
                                           const uint8_t *rk, const uint8_t *mks, const uint8_t *aks,
                                           const uint8_t *mvs, const uint8_t *avs, const uint8_t *vref,
                                           const uint8_t *vres, uint8_t *wsc, int lane, bool valid,
                                           float score_scale, const QueryRegs<D> &q, SplitState<D> &s, uint8_t *sha = nullptr, int sha_pair = 0,
                                           float *fr = nullptr) {
    using Ln = Lanes<D>;
    constexpr int LPT = Ln::LPT, CPL = Ln::CPL, PPI = Ln::PPI;
    constexpr int REF_NB = CPL * REFB / 8;          // first record's K code bytes per lane (INT4, or INT2 direct)
    constexpr int RES_NB = RB ? CPL * RB / 8 : 4;   // residual K code bytes per lane
    constexpr int REF_NW = REF_NB / 4, RES_NW = RES_NB / 4;
    constexpr int NPG = G / CPL;                    // lanes of one token in one group
    constexpr int VREF_STRIDE = 16 * D * REFB / 8, VRES_STRIDE = 16 * D * (RB ? RB : 2) / 8;
    using SZ = typename std::conditional<META_F32, float2, uint32_t>::type;
    const int tok_i = lane / LPT, q4 = lane % LPT;
    uint32_t ckw[REF_NW], rkw[RES_NW];
    load_bytes<REF_NB>(ck, ckw);
    if constexpr (RB != 0) load_bytes<RES_NB>(rk, rkw);
    VWords<D, REFB> vw_ref[PPI];
    VWords<D, RB ? RB : 2> vw_res[PPI];
#pragma unroll
    for (int pg = 0; pg < PPI; ++pg) {
        if constexpr (!SHR) load_v<D, REFB>(vw_ref[pg], vref + pg * VREF_STRIDE, lane);
        if constexpr (RB != 0) load_v<D, RB>(vw_res[pg], vres + pg * VRES_STRIDE, lane);
    }
    // every code byte of the step is read before the weight scratch (which
    // may overlap them) is written
    __asm__ volatile("" ::: "memory");
    float skr, zkr, svr, zvr;
    sz_of(*(const SZ *)mkr, skr, zkr);
    sz_of(*(const SZ *)mvr, svr, zvr);
    // score: q.x_hat = alpha*(s*sum q c + z*sum q) + (s_r*sum q' c_r + z_r*sum q'),
    // per lane slice in its own fixed-point scale; INT4 codes are centred,
    // s*sum q c + z*sum q = s*sum q (c - 8) + (8 s + z)*sum q
    float part;
    if constexpr (REFB == 4)
        part = fmaf(skr, dot_int4<REF_NW, kQueryLimbs>(ckw, q.lrv, q.lrh), fmaf(8.f, skr, zkr) * (float)q.qs_ref);
    else
        part = fmaf(skr, dot_int2<REF_NW, kQueryLimbs>(ckw, q.lrv, q.lrh), zkr * (float)q.qs_ref);
    part *= q.sc_ref;
    float av = 1.f, svs = 0.f, zvs = 0.f;
    if constexpr (RB != 0) {
        float sks, zks;
        sz_of(*(const SZ *)mks, sks, zks);
        sz_of(*(const SZ *)mvs, svs, zvs);
        const float ak = load_meta1<META_F32>(aks);
        av = load_meta1<META_F32>(avs);
        float pres;
        if constexpr (RB == 2)
            pres = fmaf(sks, dot_int2<RES_NW, kRotLimbs>(rkw, q.lsv, q.lsh), zks * (float)q.qs_res);
        else
            pres = fmaf(sks, dot_int4<RES_NW, kRotLimbs>(rkw, q.lsv, q.lsh), fmaf(8.f, sks, zks) * (float)q.qs_res);
        part = fmaf(ak, part, pres * q.sc_res);
    }
    float score = lane_group_sum<LPT>(part) * score_scale;
    score = valid ? score : kNegInf;
    // online softmax, rescaled only when a score beats m by 2^8
    float fstep = 1.f;
    if (__any(score > s.m + kRescaleThresh)) {
        const float mn = fmaxf(s.m, wave_max(score));
        const float f = fast_exp2(s.m - mn);
        if constexpr (!SHR || RB != 0) {
#pragma unroll
            for (int i = 0; i < D / 16; ++i) s.v[i] *= f;
        }
        s.zr *= f; s.zs *= f; s.lsum *= f;
        s.m = mn;
        fstep = f;
    }
    if constexpr (SHR) {
        if (lane == 0) *fr = fstep;
    }
    // a masked token weighs 0 (also while every score so far is masked and
    // s.m is still -inf, where score - s.m would be NaN)
    const float pr = valid ? fast_exp2(score - s.m) : 0.f;
    s.lsum += pr;
    // weights of this token (group of this lane); the zero terms carry z - 16 s
    const float pa = pr * av;
    float wr = valid ? pa * svr : 0.f;
    float ws = valid ? pr * svs : 0.f;
    // pin the weights as fp32 values, so that the fp16 terms below and the
    // zero terms split and use the same numbers
    __asm__ volatile("" : "+v"(wr), "+v"(ws));
    // fp16 terms, both rounded to nearest (unbiased): hi = RNE(w), lo = RNE(w - hi)
    const halfx2 hi = {(_Float16)wr, (_Float16)ws};
    const uint32_t hib = __builtin_bit_cast(uint32_t, hi);
    // lo: one mixed-precision FMA per weight (-1 * hi + w in fp32, exact,
    // rounded once to fp16 into the low or the high half)
    uint32_t lob;
    __asm__("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(lob) : "v"(hib), "v"(wr));
    __asm__("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(lob) : "v"(hib), "v"(ws));
    // zero terms: p*alpha*z minus the offset 16 times the weight. The matrix
    // cores see hi + lo instead of w: the offset then leaves 16 (hi + lo - w)
    // per token, an unbiased rounding error of the same size as the one the
    // split already makes on the code term (c (hi + lo - w), c <= 15).
    s.zr += valid ? fmaf(pa, zvr, -16.f * wr) : 0.f;
    if constexpr (RB != 0) s.zs += valid ? fmaf(pr, zvs, -16.f * ws) : 0.f;
    // rows 4g + r of this token's column: lane k of the group's NPG lanes writes rows k, k + NPG, ...
    {
        const int g = (q4 * CPL) / G, k = q4 % NPG;
        uint16_t *wrow = (uint16_t *)(wsc + (tok_i >> 4) * kWScratch) + (tok_i & 15);
        uint16_t *srow = nullptr;
        if constexpr (SHR) srow = (uint16_t *)(sha + (tok_i >> 4) * kWScratch) + (tok_i & 15) + 32 * (sha_pair + g);
#pragma unroll
        for (int e = 0; e < 4 / NPG; ++e) {
            const int r = k + NPG * e;
            if (RB != 0 || r < 2) {
                const uint32_t pair = (r & 1) ? lob : hib;
                const uint16_t h16 = (uint16_t)((r >> 1) ? pair >> 16 : pair);
                if (SHR && r < 2) srow[16 * r] = h16;
                else wrow[(4 * g + r) * 16] = h16;
            }
        }
    }
    // the rows are read back by other lanes of this wave: LDS keeps one wave's
    // accesses in order; keep the compiler from reordering them
    __asm__ volatile("" ::: "memory");
    // A row of this lane: 4g + r with r = lane%4; the reference codes take
    // rows r < 2, the residual codes rows r >= 2 (unwritten rows are masked)
    const bool ref_row = (lane & 2) == 0;
#pragma unroll
    for (int pg = 0; pg < PPI; ++pg) {
        const uint2 a2 = *(const uint2 *)(wsc + pg * kWScratch + (lane & 15) * 32 + (lane >> 4) * 8);
        if constexpr (!SHR) {
            const uint2 ar = make_uint2(ref_row ? a2.x : 0u, ref_row ? a2.y : 0u);
            v_mfma<D, REFB>(s.v, vw_ref[pg], ar);
        }
        if constexpr (RB != 0) {
            const uint2 as = make_uint2(ref_row ? 0u : a2.x, ref_row ? 0u : a2.y);
            v_mfma<D, RB>(s.v, vw_res[pg], as);
        }
    }
    __asm__ volatile("" ::: "memory");
}

// End of a split: sum the weights and zero terms over the wave's token slots
// and write (m, l, acc_ref[D], acc_res[D]) of the wave to `out` (acc_res
// only when RES). Lanes 16g..16g+15 hold rows 4g..4g+3 of the products of the
// column groups of group g.
template <int D, bool RES, int G>
__device__ __forceinline__ void finish_split(SplitState<D> &s, int lane, float *out) {
    constexpr int LPT = Lanes<D>::LPT, CPL = Lanes<D>::CPL, NPG = G / CPL;
    {
        float t[3] = {s.zr, RES ? s.zs : 0.f, s.lsum};
        strided_sum_n<LPT>(t);
        s.zr = t[0]; s.zs = t[1]; s.lsum = t[2];
    }
    // lane q4 = g*NPG (token slot 0) holds group g's zero terms
    const int gl = lane >> 4, col = lane & 15;
    const float zr = __shfl(s.zr, gl * NPG, 64);
    const float zs = RES ? __shfl(s.zs, gl * NPG, 64) : 0.f;
    if (lane == 0) { out[0] = s.m; out[1] = s.lsum; }
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        if (gl == (16 * m) / G) {
            out[2 + 16 * m + col] = s.v[m][0] + s.v[m][1] + zr;
            if constexpr (RES) out[2 + D + 16 * m + col] = s.v[m][2] + s.v[m][3] + zs;
        }
    }
}

// ---- shared reference rows (multi-loop)
//
// The reference V codes of a page are the same B operand for every loop of a
// multi-loop workgroup; only the weights differ. One wave (the reference
// loop's, which has no residual of its own) therefore multiplies the
// reference V codes by an A operand whose row pairs 2P, 2P+1 (P = call*NG +
// g) hold the (hi, lo) weights that wave `call` wrote for group g, and keeps
// every loop's reference sums in its accumulators. The rows of a step are
// consumed one step later, after the workgroup barrier that publishes them.

// Fold one step's shared rows into the owner's accumulators: rescale the
// rows of each loop by the factor that loop applied at that step, then add
// the products with the step's reference V codes.
template <int D, int G>
__device__ __forceinline__ void shared_ref_step(SplitState<D> &s, const uint8_t *sha, const float *fr,
                                                const uint8_t *vref, int lane, int nl) {
    constexpr int NG = D / G, PPI = Lanes<D>::PPI;
    constexpr int VREF_STRIDE = 16 * D * 4 / 8;
    // rows 4(lane/16) + i of this lane's accumulators: pairs P0 (i < 2), P0 + 1
    const int p0 = 2 * (lane >> 4), c0 = p0 / NG, c1 = (p0 + 1) / NG;
    const float f0 = c0 < nl ? fr[c0] : 1.f, f1 = c1 < nl ? fr[c1] : 1.f;
    if (__any(f0 != 1.f || f1 != 1.f)) {
        // in place (tied registers): a plain product lets the compiler move
        // every accumulator into new registers on both paths of this branch
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
            __asm__("v_mul_f32 %0, %0, %1" : "+v"(s.v[m][0]) : "v"(f0));
            __asm__("v_mul_f32 %0, %0, %1" : "+v"(s.v[m][1]) : "v"(f0));
            __asm__("v_mul_f32 %0, %0, %1" : "+v"(s.v[m][2]) : "v"(f1));
            __asm__("v_mul_f32 %0, %0, %1" : "+v"(s.v[m][3]) : "v"(f1));
        }
    }
#pragma unroll
    for (int pg = 0; pg < PPI; ++pg) {
        VWords<D, 4> vw;
        load_v<D, 4>(vw, vref + pg * VREF_STRIDE, lane);
        const uint2 a = *(const uint2 *)(sha + pg * kWScratch + (lane & 15) * 32 + (lane >> 4) * 8);
        v_mfma<D, 4>(s.v, vw, a);
    }
}

// The owner's reference sums of every loop into `gath` ([nl][D] floats):
// pair P = call*NG + g of column group m belongs to call P/NG when g is the
// group of m's channels.
template <int D, int G>
__device__ __forceinline__ void shared_ref_gather(const SplitState<D> &s, float *gath, int lane, int nl) {
    constexpr int NG = D / G;
    const int p0 = 2 * (lane >> 4), col = lane & 15;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        const int gm = (16 * m) / G;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int P = p0 + j, c = P / NG;
            if (c < nl && P % NG == gm) gath[c * D + 16 * m + col] = s.v[m][2 * j] + s.v[m][2 * j + 1];
        }
    }
}

// End of a split with shared reference rows: as finish_split, with the
// reference sums of this wave's loop taken from `gref` (its row of the
// gather area) and the residual sums from the wave's own accumulators (none
// for the reference loop, RES = false).
template <int D, bool RES, int G>
__device__ __forceinline__ void finish_split_shared(SplitState<D> &s, int lane, const float *gref, float *out) {
    constexpr int LPT = Lanes<D>::LPT, CPL = Lanes<D>::CPL, NPG = G / CPL;
    {
        float t[3] = {s.zr, RES ? s.zs : 0.f, s.lsum};
        strided_sum_n<LPT>(t);
        s.zr = t[0]; s.zs = t[1]; s.lsum = t[2];
    }
    const int gl = lane >> 4, col = lane & 15;
    const float zr = __shfl(s.zr, gl * NPG, 64);
    const float zs = RES ? __shfl(s.zs, gl * NPG, 64) : 0.f;
    if (lane == 0) { out[0] = s.m; out[1] = s.lsum; }
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
        if (gl == (16 * m) / G) {
            out[2 + 16 * m + col] = gref[16 * m + col] + zr;
            out[2 + D + 16 * m + col] = RES ? s.v[m][2] + s.v[m][3] + zs : 0.f;
        }
    }
}

// ---- per-loop split kernel

// One LDS stage holds one page step's packed bytes exactly as stored, in the
// order [ref K codes][ref V codes][res K codes][res V codes] (each for the
// step's PPI pages) and then, per page, [ref K meta][ref V meta][res K meta +
// alpha][res V meta + alpha]. It is filled by direct-to-LDS loads
// (global_load_lds_dwordx4): each instruction moves 64 pieces of 16 bytes.
template <int D, int RB, bool META_F32, int G, int REFB = 4>
struct StageGeom {
    static constexpr int PPI = Lanes<D>::PPI;
    static constexpr int MSZ = META_F32 ? 4 : 2;
    static constexpr int NG = D / G;
    static constexpr int CB_REF = 16 * D * REFB / 8;    // codes of one reference (or direct) record
    static constexpr int CB_RES = 16 * D * RB / 8;      // codes of one residual record
    static constexpr int MB = 16 * NG * 2 * MSZ;        // (scale, zero) of one record
    static constexpr int AB = RB ? 16 * MSZ : 0;        // alpha of one residual record
    static constexpr int MP = 2 * MB + (RB ? 2 * (MB + AB) : 0);   // metadata of one page
    static constexpr int O_RK = 0;
    static constexpr int O_RV = PPI * CB_REF;
    static constexpr int O_SK = 2 * PPI * CB_REF;
    static constexpr int O_SV = O_SK + PPI * CB_RES;
    static constexpr int O_M = O_SV + PPI * CB_RES;
    static constexpr int BYTES = O_M + PPI * MP;
    static constexpr int NP = BYTES / 16;               // 16-byte pieces
    static constexpr int NI = (NP + 63) / 64;           // direct-to-LDS instructions per stage
    static constexpr int LIVE_LAST = NP - 64 * (NI - 1);
    // ring depth per wave: as deep as four 4-wave workgroups (the register
    // bound's occupancy) allow in the CU's 160 KB of LDS, up to four stages,
    // else three when three workgroups fit, else two; the end-of-loop merge
    // reuses each wave's own stages
    static constexpr int NST = 4 * kWaves * 4 * BYTES <= 160 * 1024   ? 4
                               : 4 * kWaves * 3 * BYTES <= 160 * 1024 ? 3
                               : 3 * kWaves * 3 * BYTES <= 160 * 1024 ? 3
                                                                      : 2;
    // the step's weight scratch reuses the start of its own slot (the code
    // bytes, read into registers first)
    static_assert(PPI * kWScratch <= O_M, "weight scratch fits in the slot's code bytes");
    static_assert(BYTES % 16 == 0, "stage pieces are 16 bytes");
    static_assert(NST * BYTES >= partial_floats(D) * 4, "a wave's partial fits in its stages");
};

// This lane's piece of each of a stage's direct-to-LDS instructions: the page
// of the step it belongs to and its byte offset in that page's slab.
template <class SG, int RB>
__device__ __forceinline__ void stage_pieces(const SplitArgs &a, int lane, int *doff, int *dpg) {
#pragma unroll
    for (int i = 0; i < SG::NI; ++i) {
        const int byte = 16 * (64 * i + lane);
        int off = 0, pg = 0;
        if (byte < SG::O_RV) {
            pg = byte / SG::CB_REF; off = a.ref_off + byte % SG::CB_REF;
        } else if (byte < SG::O_SK) {
            const int w = byte - SG::O_RV; pg = w / SG::CB_REF; off = a.ref_off + a.ref_rec + w % SG::CB_REF;
        } else if (RB != 0 && byte < SG::O_SV) {
            const int w = byte - SG::O_SK; pg = w / SG::CB_RES; off = a.res_off + w % SG::CB_RES;
        } else if (RB != 0 && byte < SG::O_M) {
            const int w = byte - SG::O_SV; pg = w / SG::CB_RES; off = a.res_off + a.res_rec + w % SG::CB_RES;
        } else if (byte < SG::BYTES) {
            const int w0 = byte - SG::O_M; pg = w0 / SG::MP;
            const int w = w0 % SG::MP;
            if (w < SG::MB) off = a.ref_off + SG::CB_REF + w;
            else if (w < 2 * SG::MB) off = a.ref_off + a.ref_rec + SG::CB_REF + (w - SG::MB);
            else if (w < 3 * SG::MB + SG::AB) off = a.res_off + SG::CB_RES + (w - 2 * SG::MB);
            else off = a.res_off + a.res_rec + SG::CB_RES + (w - 3 * SG::MB - SG::AB);
        }
        doff[i] = off;
        dpg[i] = pg;
    }
}

// Split-K decode of one loop over packed pages. One wave per split (4 per
// workgroup, the same (sequence, head)); each wave streams its pages through
// a ring of NST LDS stages with NST-1 page steps in flight while one is
// consumed. The direct-to-LDS loads and their wait counts are issued
// explicitly (the data never occupies registers while in flight, and no wait
// is more conservative than the ring needs).
template <int D, int RB, bool META_F32, int G, int REFB = 4>
// (at most 128 registers: four waves per SIMD, four workgroups per CU)
__global__ __launch_bounds__(256, 4) void rq_split_kernel(SplitArgs a) {
    using Ln = Lanes<D>;
    using SG = StageGeom<D, RB, META_F32, G, REFB>;
    constexpr int LPT = Ln::LPT, CPL = Ln::CPL, PPI = Ln::PPI;
    constexpr int REF_NB = CPL * REFB / 8;
    constexpr int RES_NB = RB ? CPL * RB / 8 : 4;
    constexpr int MSZ = SG::MSZ, NG = SG::NG, NST = SG::NST, NI = SG::NI;
    constexpr int PF = partial_floats(D);
    // the LDS stages; in the reference-loop kernel also the scratch of an encode work item
    constexpr int STAGE_BYTES = kWaves * NST * SG::BYTES;
    constexpr int LDS_BYTES = (RB == 0 && enc::kEncLdsBytes > STAGE_BYTES) ? enc::kEncLdsBytes : STAGE_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t stage_mem[LDS_BYTES];
    auto stage = reinterpret_cast<uint8_t (*)[NST][SG::BYTES]>(stage_mem);
    // after the page loop: wave w's partial (m, l, acc_ref, acc_res) in its own stages
    auto wp = [&](int w) -> float * { return (float *)&stage[w][0][0]; };

    if constexpr (RB == 0) {
        if ((int)blockIdx.x >= a.enc_x0) {
            // an encode work item of the current tokens, run in the LDS stages
            const int e = ((int)blockIdx.x - a.enc_x0) * (int)gridDim.z + (int)blockIdx.z;
            if (e < a.enc_items) {
                const int nz = 2 * (a.enc.L > 1 ? a.enc.L - 1 : 1);
                if (a.enc_kvf) enc::encode_item<true, META_F32>(a.enc, e / nz, blockIdx.y, e % nz, stage_mem, kWaves);
                else enc::encode_item<false, META_F32>(a.enc, e / nz, blockIdx.y, e % nz, stage_mem, kWaves);
            }
            return;
        }
    }
    // wave index made provably wave-uniform, so the page loop is a scalar loop
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x * kWaves + wave;
    const int h = blockIdx.y, b = blockIdx.z;
    const int H = a.H;
    int seq = a.seq_lens[b];
    seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
    const int npages = (seq + 15) >> 4;
    // a workgroup none of whose splits has a page writes nothing (the combine
    // reads only the partials of workgroups that have pages)
    if (blockIdx.x * kWaves * a.split_pages >= npages) return;
    const int p0 = split * a.split_pages;
    const int p1 = min(npages, p0 + a.split_pages);   // p0 >= p1: this wave has no pages
    const int cnt = p1 - p0;
    const int steps = cnt > 0 ? (cnt + PPI - 1) / PPI : 0;

    const int tok_i = lane / LPT, q4 = lane % LPT;
    const int page_in_step = tok_i >> 4, tok = tok_i & 15;
    const int g = (q4 * CPL) / G;

    // the split's block-table entries, one per lane (at most 64 pages per
    // split), loaded together with the query (one memory latency, not two,
    // before the first page's loads can be issued)
    int tbl = -1;
    if (lane < cnt) tbl = a.block_table[(int64_t)b * a.max_blocks + p0 + lane];
    QueryRegs<D> q;
    const uint8_t *qp = a.qpack + ((int64_t)b * H + h) * qpack_bytes(D);
    load_query<D, RB != 0>(qp, q4, q);
    if (tbl < 0 || tbl >= a.nblk) tbl = -1;

    // this lane's piece of each direct-to-LDS instruction: (page of the step, byte offset in the slab)
    int doff[NI], dpg[NI];
    stage_pieces<SG, RB>(a, lane, doff, dpg);

    // this lane's reads inside a stage: four lane offsets; the other reads
    // sit at compile-time distances from them (immediate LDS offsets)
    const int o_ck = tok_i * (D * REFB / 8) + q4 * REF_NB;           // + O_RK / O_RV
    const int o_rk = tok_i * (D * RB / 8) + q4 * RES_NB;             // + O_SK / O_SV
    const int o_mkr = page_in_step * SG::MP + (tok * NG + g) * 2 * MSZ;   // + O_M (+ MB, ...)
    const int o_aks = page_in_step * SG::MP + tok * MSZ;             // + O_M + 3 MB (+ MB + AB)

    SplitState<D> s;
    init_state<D>(s);

    auto blk_of = [&](int st, int pg) -> int { return __builtin_amdgcn_readlane(tbl, st * PPI + pg); };

    // issue the NI direct-to-LDS loads of page step `st` into ring slot `slot`
    // (a missing page reads block 0; its tokens are masked)
    auto issue = [&](int st, int slot) {
        // the slot's previous contents must have been read out before the
        // loads can land on it
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int b0 = max(blk_of(st, 0), 0);
        const uint8_t *base0 = a.pool + ((int64_t)b0 * H + h) * a.slab;
        const uint8_t *base1 = base0;
        if constexpr (PPI == 2) base1 = a.pool + ((int64_t)max(blk_of(st, 1), 0) * H + h) * a.slab;
        const uint32_t lds = lds_addr(&stage[wave][slot][0]);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if (i < NI - 1 || SG::LIVE_LAST == 64 || lane < SG::LIVE_LAST) {
                if constexpr (PPI == 1) dma16(lds + 1024u * i, base0, (uint32_t)doff[i]);
                else dma16(lds + 1024u * i, (dpg[i] ? base1 : base0) + doff[i]);
            }
        }
    };

    if (steps > 0) {
#pragma unroll
        for (int j = 0; j < NST - 1; ++j)
            if (j < steps) issue(j, j);
        for (int cur = 0; cur < steps; ++cur) {
            if (cur + NST - 1 < steps) issue(cur + NST - 1, (cur + NST - 1) % NST);
            wait_steps<NST - 1, NI>(min(NST - 1, steps - 1 - cur));
            const int pp = p0 + cur * PPI + page_in_step;
            int blk = blk_of(cur, 0);
            if constexpr (PPI == 2) blk = page_in_step ? blk_of(cur, 1) : blk;
            const bool valid = blk >= 0 && pp < p1 && pp * 16 + tok < seq;
            uint8_t *S = &stage[wave][cur % NST][0];
            const uint8_t *M = S + SG::O_M + o_mkr, *A = S + SG::O_M + o_aks;
            token_step<D, RB, META_F32, G, REFB>(S + SG::O_RK + o_ck, M, M + SG::MB, S + SG::O_SK + o_rk,
                                                 M + 2 * SG::MB, A + 3 * SG::MB, M + 3 * SG::MB + SG::AB,
                                                 A + 4 * SG::MB + SG::AB, S + SG::O_RV, S + SG::O_SV, S, lane,
                                                 valid, a.score_scale, q, s);
        }
    }

    // ---- merge the workgroup's 4 wave partials (log-sum-exp), one partial per workgroup
    finish_split<D, RB != 0, G>(s, lane, wp(wave));
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wp(w)[0]);
    // every token of the workgroup masked (invalid block ids): an empty partial
    float e[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) e[w] = M == kNegInf ? 0.f : fast_exp2(wp(w)[0] - M);
    float *out = a.partials + (((int64_t)b * H + h) * a.nwg + blockIdx.x) * PF;
    constexpr int NV = RB ? 2 * D : D;
    for (int v = threadIdx.x; v < NV; v += 256) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc = fmaf(e[w], wp(w)[2 + v], acc);
        out[2 + v] = acc;
    }
    if (threadIdx.x == 0) {
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) l = fmaf(e[w], wp(w)[1], l);
        out[0] = M;
        out[1] = l;
    }
}

// ---- streaming reference of the per-loop split kernel
//
// The same grid, ring, block-table walk and direct-to-LDS loads as
// rq_split_kernel, with no attention arithmetic: each lane folds one word of
// every landed stage into a checksum (one per workgroup, written to
// a.partials as uint32). Its duration is the rate at which this access
// pattern streams the page records from HBM, the reference the split
// kernel's bandwidth is measured against.
template <int D, int RB, bool META_F32, int G, int REFB = 4>
__global__ __launch_bounds__(256, 4) void rq_stream_kernel(SplitArgs a) {
    using Ln = Lanes<D>;
    using SG = StageGeom<D, RB, META_F32, G, REFB>;
    constexpr int PPI = Ln::PPI, NST = SG::NST, NI = SG::NI;
    __shared__ __attribute__((aligned(16))) uint8_t stage_mem[kWaves * NST * SG::BYTES];
    auto stage = reinterpret_cast<uint8_t (*)[NST][SG::BYTES]>(stage_mem);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x * kWaves + wave;
    const int h = blockIdx.y, b = blockIdx.z;
    const int H = a.H;
    int seq = a.seq_lens[b];
    seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
    const int npages = (seq + 15) >> 4;
    if (blockIdx.x * kWaves * a.split_pages >= npages) return;
    const int p0 = split * a.split_pages;
    const int p1 = min(npages, p0 + a.split_pages);
    const int cnt = p1 - p0;
    const int steps = cnt > 0 ? (cnt + PPI - 1) / PPI : 0;
    int tbl = -1;
    if (lane < cnt) {
        tbl = a.block_table[(int64_t)b * a.max_blocks + p0 + lane];
        if (tbl < 0 || tbl >= a.nblk) tbl = -1;
    }
    int doff[NI], dpg[NI];
    stage_pieces<SG, RB>(a, lane, doff, dpg);
    auto blk_of = [&](int st, int pg) -> int { return __builtin_amdgcn_readlane(tbl, st * PPI + pg); };
    auto issue = [&](int st, int slot) {
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int b0 = max(blk_of(st, 0), 0);
        const uint8_t *base0 = a.pool + ((int64_t)b0 * H + h) * a.slab;
        const uint8_t *base1 = base0;
        if constexpr (PPI == 2) base1 = a.pool + ((int64_t)max(blk_of(st, 1), 0) * H + h) * a.slab;
        const uint32_t lds = lds_addr(&stage[wave][slot][0]);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if (i < NI - 1 || SG::LIVE_LAST == 64 || lane < SG::LIVE_LAST) {
                if constexpr (PPI == 1) dma16(lds + 1024u * i, base0, (uint32_t)doff[i]);
                else dma16(lds + 1024u * i, (dpg[i] ? base1 : base0) + doff[i]);
            }
        }
    };
    uint32_t sum = 0;
    if (steps > 0) {
#pragma unroll
        for (int j = 0; j < NST - 1; ++j)
            if (j < steps) issue(j, j);
        for (int cur = 0; cur < steps; ++cur) {
            if (cur + NST - 1 < steps) issue(cur + NST - 1, (cur + NST - 1) % NST);
            wait_steps<NST - 1, NI>(min(NST - 1, steps - 1 - cur));
            sum ^= ((const uint32_t *)&stage[wave][cur % NST][0])[lane] + (uint32_t)cur;
            __asm__ volatile("" ::: "memory");
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum ^= (uint32_t)__shfl_xor((int)sum, o, 64);
    if (lane == 0) ((uint32_t *)a.partials)[(((int64_t)b * H + h) * a.nwg + blockIdx.x) * kWaves + wave] = sum;
}

// ---- multi-loop split kernel

struct MultiArgs {
    const uint8_t *pool;
    int64_t slab;
    int H, nblk;
    int ref_off, ref_rec;
    int nl;                                   // loop calls of this group = waves per workgroup
    int nres;                                 // calls with a residual (rb != 0): private residual rings
    int res_off[kMaxMultiLoops], res_rec[kMaxMultiLoops], rb[kMaxMultiLoops];   // rb 0: reference loop
    const int32_t *block_table;
    int max_blocks;
    const int32_t *seq_lens;
    const uint8_t *qpack;     // group's first call: [nl][B][H][qpack_bytes]
    float *partials;          // group's first call: [nl][B][H][nsplit][2 + 2D]
    int B, nsplit, split_pages, nst;
    float score_scale;
    int enc_x0, enc_items, enc_kvf;   // encode work items riding in this launch (as in SplitArgs)
    enc::EncArgs enc;
};

// Stage layout of the multi-loop kernel. The reference stage is shared by the
// workgroup: [ref K codes][ref V codes] for the step's PPI pages, then per
// page [ref K meta][ref V meta]. Each wave has a private residual stage for
// its own loop's bits rb: [res K codes][res V codes], then per page
// [res K meta][K alpha][res V meta][V alpha] (each record's tail as stored).
template <int D, bool META_F32, int G, int RBMAX>
struct MultiGeom {
    static constexpr int PPI = Lanes<D>::PPI;
    static constexpr int MSZ = META_F32 ? 4 : 2;
    static constexpr int NG = D / G;
    static constexpr int CB_REF = 16 * D / 2;
    static constexpr int MB = 16 * NG * 2 * MSZ;
    static constexpr int AB = 16 * MSZ;
    static constexpr int R_CV = PPI * CB_REF;
    static constexpr int R_M = 2 * PPI * CB_REF;
    static constexpr int REF_BYTES = R_M + PPI * 2 * MB;
    static constexpr int P_REF = REF_BYTES / 16;
    __host__ __device__ static constexpr int cb_res(int rb) { return 16 * D * rb / 8; }
    __host__ __device__ static constexpr int smp() { return 2 * (MB + AB); }
    __host__ __device__ static constexpr int res_bytes(int rb) { return rb ? 2 * PPI * cb_res(rb) + PPI * smp() : 0; }
    static constexpr int RES_MAX = 2 * PPI * (16 * D * RBMAX / 8) + PPI * 2 * (MB + AB);
    // loads per wave and step: the wave's share of the reference (at least
    // two waves share it) and its residual, padded to fixed counts
    static constexpr int NIR = ((P_REF + 1) / 2 + 63) / 64;
    static constexpr int NIS = (RES_MAX / 16 + 63) / 64;
    static constexpr int NIW = NIR + NIS;
    static_assert(REF_BYTES % 16 == 0 && RES_MAX % 16 == 0, "stage pieces are 16 bytes");
};

// Split-K decode of several loops at once (the same sequences and heads, one
// query per loop): one workgroup per (split, head, sequence) with one wave per
// loop call. Each reference page is loaded once into the shared stage and
// scored by every wave; each wave adds its own loop's residual. The ring has
// nst stages; every wave issues exactly NIW direct-to-LDS loads per step
// (short shares are padded with a one-lane load into the wave's scratch
// slot), so its waits are fixed counts, and one barrier per step publishes
// the landed stage to all waves and frees the slot for reuse.
// SH: the group holds the reference loop and its wave owns the reference
// rows of every loop (shared_ref_step); the rows of step cur are consumed in
// step cur + 1, so loads run nst - 2 steps ahead instead of nst - 1 and the
// stage of step cur stays intact until then.
template <int D, bool META_F32, int G, int RBMAX, bool SH>
__global__ __launch_bounds__(64 * kMaxMultiLoops) void rq_multi_kernel(MultiArgs a) {
    using Ln = Lanes<D>;
    using MG = MultiGeom<D, META_F32, G, RBMAX>;
    constexpr int LPT = Ln::LPT, CPL = Ln::CPL, PPI = Ln::PPI;
    constexpr int REF_NB = CPL / 2;
    constexpr int MSZ = MG::MSZ, NG = MG::NG, NIR = MG::NIR, NIS = MG::NIS, NIW = MG::NIW;
    constexpr int PF = partial_floats(D);
    constexpr int NST_MAX = 8;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    if ((int)blockIdx.x >= a.enc_x0) {
        // an encode work item of the current tokens (LDS sized for it by the host)
        const int e = ((int)blockIdx.x - a.enc_x0) * (int)gridDim.z + (int)blockIdx.z;
        if (e < a.enc_items) {
            const int nz = 2 * (a.enc.L > 1 ? a.enc.L - 1 : 1);
            if (a.enc_kvf) enc::encode_item<true, META_F32>(a.enc, e / nz, blockIdx.y, e % nz, smem, a.nl);
            else enc::encode_item<false, META_F32>(a.enc, e / nz, blockIdx.y, e % nz, smem, a.nl);
        }
        return;
    }
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int H = a.H, nl = a.nl, nst = a.nst;
    int seq = a.seq_lens[b];
    seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
    const int npages = (seq + 15) >> 4;
    const int p0 = split * a.split_pages;
    if (p0 >= npages) return;                     // the whole workgroup: no page in this split
    const int p1 = min(npages, p0 + a.split_pages);
    const int cnt = p1 - p0;
    const int steps = (cnt + PPI - 1) / PPI;

    // Loop call of this wave. The calls do unequal work (the reference loop has
    // no residual), so the wave -> call assignment rotates from workgroup to
    // workgroup: the waves a SIMD hosts from different workgroups then carry a
    // mix of calls instead of always the same one.
    const uint32_t lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int call = __builtin_amdgcn_readfirstlane((int)((wave + (lin ^ (lin >> 8))) % (uint32_t)nl));
    const int rb = __builtin_amdgcn_readfirstlane(a.rb[call]);
    const int res_off = a.res_off[call], res_rec = a.res_rec[call];
    const int tok_i = lane / LPT, q4 = lane % LPT;
    const int page_in_step = tok_i >> 4, tok = tok_i & 15;
    const int g = (q4 * CPL) / G;

    // the split's block ids, loaded together with the query (one memory latency)
    int tbl = -1;
    if (lane < cnt) tbl = a.block_table[(int64_t)b * a.max_blocks + p0 + lane];
    QueryRegs<D> q;
    load_query<D, true>(a.qpack + (((int64_t)call * a.B + b) * H + h) * qpack_bytes(D), q4, q);
    if (tbl < 0 || tbl >= a.nblk) tbl = -1;

    // LDS: nst shared reference stages, then nst private residual stages per
    // wave, then one 16-byte scratch slot per wave for the padding loads, the
    // weight scratch of each wave and (SH) two buffers of shared reference
    // rows and two of rescale factors
    const int ref_stage = MG::REF_BYTES, res_stage = MG::RES_MAX;
    uint8_t *ref_base = smem;
    // residual rings only for the calls with a residual (index ri among them)
    int ri = 0;
    for (int c = 0; c < call; ++c) ri += a.rb[c] != 0 ? 1 : 0;
    uint8_t *res_base = smem + nst * ref_stage + ri * nst * res_stage;
    const int ring_bytes = nst * (ref_stage + a.nres * res_stage);
    const uint32_t junk = lds_addr(smem + ring_bytes + 16 * wave);

    // this wave's share of the reference pieces [r0, r0 + rcount)
    const int rq = (MG::P_REF + nl - 1) / nl;
    const int r0 = wave * rq;
    const int rcount = max(0, min(MG::P_REF, r0 + rq) - r0);
    const int cbr = MG::cb_res(rb);
    const int pres = MG::res_bytes(rb) / 16;

    // per instruction: destination offset in the stage (-1: padding), and
    // this lane's (page of the step, byte offset in the slab)
    int rdst[NIR], rdoff[NIR], rdpg[NIR];
    bool rlive[NIR];
#pragma unroll
    for (int j = 0; j < NIR; ++j) {
        const bool pad = 64 * j >= rcount;
        rdst[j] = pad ? -1 : 16 * (r0 + 64 * j);
        rlive[j] = pad ? lane == 0 : 64 * j + lane < rcount;
        const int byte = 16 * (r0 + 64 * j + lane);
        int off = 0, pg = 0;
        if (!pad && rlive[j]) {
            if (byte < MG::R_CV) {
                pg = byte / MG::CB_REF; off = a.ref_off + byte % MG::CB_REF;
            } else if (byte < MG::R_M) {
                const int w = byte - MG::R_CV; pg = w / MG::CB_REF; off = a.ref_off + a.ref_rec + w % MG::CB_REF;
            } else {
                const int w0 = byte - MG::R_M; pg = w0 / (2 * MG::MB);
                const int w = w0 % (2 * MG::MB);
                off = w < MG::MB ? a.ref_off + MG::CB_REF + w : a.ref_off + a.ref_rec + MG::CB_REF + (w - MG::MB);
            }
        }
        rdoff[j] = off; rdpg[j] = pg;
    }
    int sdst[NIS], sdoff[NIS], sdpg[NIS];
    bool slive[NIS];
#pragma unroll
    for (int j = 0; j < NIS; ++j) {
        const bool pad = 64 * j >= pres;
        sdst[j] = pad ? -1 : 16 * 64 * j;
        slive[j] = pad ? lane == 0 : 64 * j + lane < pres;
        const int byte = 16 * (64 * j + lane);
        int off = 0, pg = 0;
        if (!pad && slive[j]) {
            const int s_cv = PPI * cbr, s_m = 2 * PPI * cbr;
            if (byte < s_cv) {
                pg = byte / cbr; off = res_off + byte % cbr;
            } else if (byte < s_m) {
                const int w = byte - s_cv; pg = w / cbr; off = res_off + res_rec + w % cbr;
            } else {
                const int w0 = byte - s_m; pg = w0 / MG::smp();
                const int w = w0 % MG::smp();
                off = w < MG::MB + MG::AB ? res_off + cbr + w : res_off + res_rec + cbr + (w - MG::MB - MG::AB);
            }
        }
        sdoff[j] = off; sdpg[j] = pg;
    }

    // this lane's reads inside the stages
    const int o_ck = tok_i * (D / 2) + q4 * REF_NB;
    const int o_mkr = MG::R_M + page_in_step * 2 * MG::MB + (tok * NG + g) * 2 * MSZ;
    const int o_mvr = o_mkr + MG::MB;
    const int res_nb = CPL * rb / 8;
    const int o_rk = tok_i * (D * rb / 8) + q4 * res_nb;
    const int o_m = 2 * PPI * cbr + page_in_step * MG::smp();
    const int o_mks = o_m + (tok * NG + g) * 2 * MSZ;
    const int o_aks = o_m + MG::MB + tok * MSZ;
    const int o_mvs = o_mks + MG::MB + MG::AB;
    const int o_avs = o_aks + MG::MB + MG::AB;

    SplitState<D> s;
    init_state<D>(s);
    // this wave's weight scratch (after the padding slots)
    uint8_t *wsc = smem + ring_bytes + 16 * nl + wave * PPI * kWScratch;
    uint8_t *sha = smem + ring_bytes + nl * (16 + PPI * kWScratch);
    float *fbuf = (float *)(sha + 2 * PPI * kWScratch);
    if constexpr (SH) {
        // rows past the last loop's pairs are never written: zero them once
        // (visible to the owner after the first barrier)
        for (int i = threadIdx.x; i < 2 * PPI * kWScratch / 4; i += 64 * nl) ((uint32_t *)sha)[i] = 0u;
    }
    const int la = SH ? nst - 2 : nst - 1;   // steps in flight ahead of the current one

    auto blk_of = [&](int st, int pg) -> int { return __builtin_amdgcn_readlane(tbl, st * PPI + pg); };

    // byte offset of slab (block, h): block * H + h and the slab size fit 32 bits
    const uint32_t slab32 = (uint32_t)a.slab;
    auto slab_at = [&](int blk) -> const uint8_t * {
        return a.pool + (uint64_t)(uint32_t)(max(blk, 0) * H + h) * slab32;
    };
    auto issue = [&](int st, int slot) {
        const uint8_t *base0 = slab_at(blk_of(st, 0));
        const uint8_t *base1 = base0;
        if constexpr (PPI == 2) base1 = slab_at(blk_of(st, 1));
        const uint32_t rl = lds_addr(ref_base + slot * ref_stage);
        const uint32_t sl = lds_addr(res_base + slot * res_stage);
#pragma unroll
        for (int j = 0; j < NIR; ++j) {
            const uint32_t dst = rdst[j] < 0 ? junk : rl + (uint32_t)rdst[j];
            if (rlive[j]) {
                if constexpr (PPI == 1) dma16(dst, base0, (uint32_t)rdoff[j]);
                else dma16(dst, (rdpg[j] ? base1 : base0) + rdoff[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NIS; ++j) {
            const uint32_t dst = sdst[j] < 0 ? junk : sl + (uint32_t)sdst[j];
            if (slive[j]) {
                if constexpr (PPI == 1) dma16(dst, base0, (uint32_t)sdoff[j]);
                else dma16(dst, (sdpg[j] ? base1 : base0) + sdoff[j]);
            }
        }
    };

    for (int j = 0; j < la; ++j)
        if (j < steps) issue(j, j);
    // ring slots of the current, the previous and the issued step, kept as
    // running counters (nst is a launch value: no division per step)
    int slot = 0, pslot = nst - 1, islot = la;
    // The page loop, one copy per residual width RBW of this wave's loop: the
    // accumulators then stay in the same registers from step to step.
    auto page_loop = [&](auto rbw_tag) {
        constexpr int RBW = decltype(rbw_tag)::value;
        for (int cur = 0; cur < steps; ++cur) {
            // this wave's loads of step `cur` have landed ...
            wait_steps<NST_MAX - 2, NIW>(min(la - 1, steps - 1 - cur));
            // ... and so have every other wave's; all waves are done with step
            // cur-1 (SH: except the owner's use of its reference stage, which
            // ends before the next barrier, and the stage is refilled only after it)
            __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (cur + la < steps) issue(cur + la, islot);
            const int pp = p0 + cur * PPI + page_in_step;
            int blk = blk_of(cur, 0);
            if constexpr (PPI == 2) blk = page_in_step ? blk_of(cur, 1) : blk;
            const bool valid = blk >= 0 && pp < p1 && pp * 16 + tok < seq;
            const uint8_t *R = ref_base + slot * ref_stage;
            const uint8_t *S = res_base + slot * res_stage;
            uint8_t *shc = sha + (cur & 1) * PPI * kWScratch;
            float *fc = fbuf + (cur & 1) * kMaxMultiLoops + call;
            if constexpr (RBW != 0) {
                token_step<D, RBW, META_F32, G, 4, SH>(R + o_ck, R + o_mkr, R + o_mvr, S + o_rk, S + o_mks,
                                                       S + o_aks, S + o_mvs, S + o_avs, R + MG::R_CV,
                                                       S + PPI * MG::cb_res(RBW), wsc, lane, valid, a.score_scale,
                                                       q, s, shc, call * NG, fc);
            } else {
                token_step<D, 0, META_F32, G, 4, SH>(R + o_ck, R + o_mkr, R + o_mvr, S, S, S, S, S, R + MG::R_CV, S,
                                                     wsc, lane, valid, a.score_scale, q, s, shc, call * NG,
                                                     fc);
                // SH: the previous step's rows of every loop
                if (SH && cur > 0)
                    shared_ref_step<D, G>(s, sha + ((cur - 1) & 1) * PPI * kWScratch,
                                          fbuf + ((cur - 1) & 1) * kMaxMultiLoops,
                                          ref_base + pslot * ref_stage + MG::R_CV, lane, nl);
            }
            pslot = slot;
            slot = slot + 1 == nst ? 0 : slot + 1;
            islot = islot + 1 == nst ? 0 : islot + 1;
        }
    };
    if (rb == 2) page_loop(std::integral_constant<int, 2>{});
    else if (RBMAX == 4 && rb == 4) page_loop(std::integral_constant<int, RBMAX>{});
    else page_loop(std::integral_constant<int, 0>{});

    float *part = a.partials + ((((int64_t)call * a.B + b) * H + h) * a.nsplit + split) * PF;
    if constexpr (SH) {
        // the last step's rows, then every loop's reference sums through LDS
        // (the ring is free: every load has landed and every read is done)
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        float *gath = (float *)smem;
        if (rb == 0) {
            const int last = steps - 1;
            shared_ref_step<D, G>(s, sha + (last & 1) * PPI * kWScratch, fbuf + (last & 1) * kMaxMultiLoops,
                                  ref_base + pslot * ref_stage + MG::R_CV, lane, nl);
            __asm__ volatile("" ::: "memory");
            shared_ref_gather<D, G>(s, gath, lane, nl);
        }
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (rb == 0) finish_split_shared<D, false, G>(s, lane, gath + call * D, part);
        else finish_split_shared<D, true, G>(s, lane, gath + call * D, part);
    } else {
        finish_split<D, true, G>(s, lane, part);
    }
}

// --------------------------------------------------------------- combine
struct CombineArgs {
    const float *partials;  // [n][B][H][nparts][2 + 2D]
    int nparts, spp;        // partials per row; splits merged into one partial (4, or 1 for multi-loop)
    int split_pages, max_blocks;
    const int32_t *seq_lens;
    const void *q, *tail_k, *tail_v;   // [n][B][H][D]
    const float *rot;
    float *out;                        // [n][B][H][D]
    int B, H;
    float score_scale;
    int is_res[RQ_MAX_LOOPS];
};

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// One workgroup per (head, loop call, kPrepRows sequences); one wave per sequence.
template <int D, bool KV_F32>
__global__ __launch_bounds__(64 * kPrepRows) void rq_combine_kernel(CombineArgs a) {
    constexpr int QS = D + 1, RW = kPrepRows;
    constexpr int NT = (D / 16 + RW - 1) / RW;    // column tiles of the rotation per wave
    constexpr int PF = partial_floats(D);
    __shared__ float A[16 * QS];                  // rows RW..15 zero: the A operand has 16 rows
    __shared__ float O[RW * QS];
    const int lane = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int h = blockIdx.x, i = blockIdx.y, tile = blockIdx.z;
    const int B = a.B, H = a.H;
    const bool has_res = a.is_res[i] != 0;
    const int b = tile * RW + r;
    const int c0 = lane, c1 = lane + 64;
    float ar0 = 0.f, ar1 = 0.f, as0 = 0.f, as1 = 0.f;
    // this lane's R_V operands of the output rotation (column tiles r, r +
    // RW, ...), loaded before the partials so that the two latencies overlap
    // (see the MFMA below)
    float rv[NT][D / 4];
    if (has_res) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int ct = r + RW * j;
            if (ct < D / 16) {
                const float *RV = a.rot + ((int64_t)h * 2 + 1) * D * D + (int64_t)(lane >> 4) * D + ct * 16 + (lane & 15);
#pragma unroll
                for (int kk = 0; kk < D / 4; ++kk) rv[j][kk] = RV[(int64_t)4 * kk * D];
            }
        }
        for (int e = threadIdx.x; e < (16 - RW) * QS; e += 64 * RW) A[RW * QS + e] = 0.0f;
    }
    if (b < B) {
        int seq = a.seq_lens[b];
        seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
        const int npages = (seq + 15) >> 4;
        const int nsw = (npages + a.split_pages - 1) / a.split_pages;   // splits with pages
        const int ns = (nsw + a.spp - 1) / a.spp;                        // their partials
        const int64_t row = ((int64_t)i * B + b) * H + h;
        const float *P = a.partials + row * a.nparts * PF;
        float st = kNegInf, tv0 = 0.f, tv1 = 0.f;
        if (a.tail_k) {
            float d = 0.f;
            if (c0 < D) d += load_kv<KV_F32>(a.q, row * D + c0) * load_kv<KV_F32>(a.tail_k, row * D + c0);
            if (c1 < D) d += load_kv<KV_F32>(a.q, row * D + c1) * load_kv<KV_F32>(a.tail_k, row * D + c1);
            if (c0 < D) tv0 = load_kv<KV_F32>(a.tail_v, row * D + c0);
            if (c1 < D) tv1 = load_kv<KV_F32>(a.tail_v, row * D + c1);
            st = wave_sum(d) * a.score_scale;
        }
        // One round of loads for what the merge needs first: (m, l) of the
        // partials lane, lane + 64, ... and this lane's columns c0 and c1
        // (clamped: the weight of a column beyond D is never used) of the
        // first NPRE partials (indices past the last partial re-read it with
        // weight 0)
        constexpr int NPRE = 24;
        const int k0 = min(c0, D - 1), k1 = min(c1, D - 1);
        const float m_l = lane < ns ? P[(int64_t)lane * PF] : kNegInf;
        const float l_l = lane < ns ? P[(int64_t)lane * PF + 1] : 0.f;
        float pv0[NPRE], pv1[NPRE], pw0[NPRE], pw1[NPRE];
        if (ns > 0) {
#pragma unroll
            for (int j = 0; j < NPRE; ++j) {
                const float *ps = P + (int64_t)min(j, ns - 1) * PF + 2;
                pv0[j] = ps[k0];
                pv1[j] = D > 64 ? ps[k1] : 0.f;
                pw0[j] = has_res ? ps[D + k0] : 0.f;
                pw1[j] = (has_res && D > 64) ? ps[D + k1] : 0.f;
            }
        }
        float mloc = m_l;
        for (int s = lane + 64; s < ns; s += 64) mloc = fmaxf(mloc, P[(int64_t)s * PF]);
        const float M = fmaxf(wave_max(mloc), st);
        if (M != kNegInf) {
            float lloc = 0.f;
            for (int cb = 0; cb < ns; cb += 64) {
                const int s = cb + lane;
                const float e_l = s < ns ? fast_exp2((cb == 0 ? m_l : P[(int64_t)s * PF]) - M) : 0.f;
                if (s < ns) lloc = fmaf(e_l, cb == 0 ? l_l : P[(int64_t)s * PF + 1], lloc);
                const int cnt = min(64, ns - cb);
                int j0 = 0;
                if (cb == 0) {
#pragma unroll
                    for (int j = 0; j < NPRE; ++j) {
                        const float e = j < cnt ? readlane_f(e_l, j) : 0.f;
                        ar0 = fmaf(e, pv0[j], ar0);
                        ar1 = fmaf(e, pv1[j], ar1);
                        as0 = fmaf(e, pw0[j], as0);
                        as1 = fmaf(e, pw1[j], as1);
                    }
                    j0 = NPRE;
                }
                // the rest in groups of 8 partials with unconditional loads,
                // so that all the group's loads are in flight together
                for (; j0 < cnt; j0 += 8) {
                    float e[8], v0[8], v1[8], w0[8], w1[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int jj = min(j0 + j, cnt - 1);
                        e[j] = j0 + j < cnt ? readlane_f(e_l, j0 + j) : 0.f;
                        const float *ps = P + (int64_t)(cb + jj) * PF + 2;
                        v0[j] = ps[k0];
                        v1[j] = ps[k1];
                        w0[j] = has_res ? ps[D + k0] : 0.f;
                        w1[j] = has_res ? ps[D + k1] : 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        ar0 = fmaf(e[j], v0[j], ar0);
                        ar1 = fmaf(e[j], v1[j], ar1);
                        as0 = fmaf(e[j], w0[j], as0);
                        as1 = fmaf(e[j], w1[j], as1);
                    }
                }
            }
            float lsum = wave_sum(lloc);
            if (a.tail_k) {
                const float pt = fast_exp2(st - M);
                lsum += pt;
                if (c0 < D) ar0 = fmaf(pt, tv0, ar0);
                if (c1 < D) ar1 = fmaf(pt, tv1, ar1);
            }
            const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
            ar0 *= inv; ar1 *= inv; as0 *= inv; as1 *= inv;
        }
    }
    if (c0 < D) { O[r * QS + c0] = ar0; A[r * QS + c0] = as0; }
    if (c1 < D) { O[r * QS + c1] = ar1; A[r * QS + c1] = as1; }
    __syncthreads();

    if (has_res) {
        // out = O + A * R_V (row vector times R_V = R_V^T applied to the column),
        // v_mfma_f32_16x16x4f32: lane l supplies A[l%16][k0 + l/16], B[k0 + l/16][l%16]
        // and receives D[4*(l/16)+v][l%16]; wave r computes the output column
        // tiles r, r + RW, ...
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int ct = r + RW * j;
            if (ct < D / 16) {
                const int n = ct * 16 + (lane & 15);
                // four independent accumulation chains (the products' latency overlaps)
                floatx4 c4[4] = {};
#pragma unroll
                for (int kk = 0; kk < D / 4; ++kk) {
                    const int k = 4 * kk + (lane >> 4);
                    c4[kk & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(lane & 15) * QS + k], rv[j][kk], c4[kk & 3],
                                                                      0, 0, 0);
                }
                const floatx4 c = (c4[0] + c4[1]) + (c4[2] + c4[3]);
                for (int v = 0; v < 4; ++v) {
                    const int rr = 4 * (lane >> 4) + v;
                    const int bb = tile * RW + rr;
                    if (rr < RW && bb < B) a.out[(((int64_t)i * B + bb) * H + h) * D + n] = c[v] + O[rr * QS + n];
                }
            }
        }
    } else if (b < B) {
        if (c0 < D) a.out[(((int64_t)i * B + b) * H + h) * D + c0] = O[r * QS + c0];
        if (c1 < D) a.out[(((int64_t)i * B + b) * H + h) * D + c1] = O[r * QS + c1];
    }
}

// ------------------------------------------------------------- dispatch
// ev0 / ev1 (may be null) are stamped by the kernel's own dispatch at its
// start and end (no separate event packets in the stream)
// rb: residual bits (0: one record only); refb: bits of the first record
// (4: the INT4 reference; 2: a direct INT2 loop, with rb == 0)
template <int D>
hipError_t launch_split_d(const SplitArgs &s, int rb, int refb, bool mf, dim3 grid, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
#define RQ_SPLIT(RB_, MF_, G_, REFB_) \
    hipExtLaunchKernelGGL((rq_split_kernel<D, RB_, MF_, G_, REFB_>), grid, dim3(256), 0, st, ev0, ev1, 0, s)
#define RQ_SPLIT_RB(MF_, G_)                          \
    do {                                              \
        if (rb == 0 && refb == 2) RQ_SPLIT(0, MF_, G_, 2); \
        else if (rb == 0) RQ_SPLIT(0, MF_, G_, 4);    \
        else if (rb == 2) RQ_SPLIT(2, MF_, G_, 4);    \
        else RQ_SPLIT(4, MF_, G_, 4);                 \
    } while (0)
#define RQ_SPLIT_G(G_)                                \
    do {                                              \
        if (mf) RQ_SPLIT_RB(true, G_);                \
        else RQ_SPLIT_RB(false, G_);                  \
    } while (0)
    // group sizes per head dim as accepted by the layout check
    if constexpr (D == 128) {
        if (s.G == 32) RQ_SPLIT_G(32); else if (s.G == 64) RQ_SPLIT_G(64); else RQ_SPLIT_G(128);
    } else if constexpr (D == 96) {
        RQ_SPLIT_G(96);
    } else {
        if (s.G == 16) RQ_SPLIT_G(16); else if (s.G == 32) RQ_SPLIT_G(32); else RQ_SPLIT_G(64);
    }
#undef RQ_SPLIT_G
#undef RQ_SPLIT_RB
#undef RQ_SPLIT
    return hipGetLastError();
}

// The streaming reference of launch_split_d's kernel (same variants).
template <int D>
hipError_t launch_stream_d(const SplitArgs &s, int rb, int refb, bool mf, dim3 grid, hipStream_t st, hipEvent_t ev0,
                           hipEvent_t ev1) {
#define RQ_STREAM(RB_, MF_, G_, REFB_) \
    hipExtLaunchKernelGGL((rq_stream_kernel<D, RB_, MF_, G_, REFB_>), grid, dim3(256), 0, st, ev0, ev1, 0, s)
#define RQ_STREAM_RB(MF_, G_)                          \
    do {                                               \
        if (rb == 0 && refb == 2) RQ_STREAM(0, MF_, G_, 2); \
        else if (rb == 0) RQ_STREAM(0, MF_, G_, 4);    \
        else if (rb == 2) RQ_STREAM(2, MF_, G_, 4);    \
        else RQ_STREAM(4, MF_, G_, 4);                 \
    } while (0)
#define RQ_STREAM_G(G_)                                \
    do {                                               \
        if (mf) RQ_STREAM_RB(true, G_);                \
        else RQ_STREAM_RB(false, G_);                  \
    } while (0)
    if constexpr (D == 128) {
        if (s.G == 32) RQ_STREAM_G(32); else if (s.G == 64) RQ_STREAM_G(64); else RQ_STREAM_G(128);
    } else if constexpr (D == 96) {
        RQ_STREAM_G(96);
    } else {
        if (s.G == 16) RQ_STREAM_G(16); else if (s.G == 32) RQ_STREAM_G(32); else RQ_STREAM_G(64);
    }
#undef RQ_STREAM_G
#undef RQ_STREAM_RB
#undef RQ_STREAM
    return hipGetLastError();
}

template <int D, bool MF, int G, int RBMAX>
hipError_t launch_multi_k(const MultiArgs &m, bool sh, dim3 grid, size_t lds, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
    if (sh)
        hipExtLaunchKernelGGL((rq_multi_kernel<D, MF, G, RBMAX, true>), grid, dim3(64 * m.nl), (uint32_t)lds, st, ev0,
                              ev1, 0, m);
    else
        hipExtLaunchKernelGGL((rq_multi_kernel<D, MF, G, RBMAX, false>), grid, dim3(64 * m.nl), (uint32_t)lds, st,
                              ev0, ev1, 0, m);
    return hipGetLastError();
}

template <int D, bool MF, int RBMAX>
hipError_t launch_multi_g(const MultiArgs &m, bool sh, int G, dim3 grid, size_t lds, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
    if constexpr (D == 128) {
        if (G == 32) return launch_multi_k<D, MF, 32, RBMAX>(m, sh, grid, lds, st, ev0, ev1);
        if (G == 64) return launch_multi_k<D, MF, 64, RBMAX>(m, sh, grid, lds, st, ev0, ev1);
        return launch_multi_k<D, MF, 128, RBMAX>(m, sh, grid, lds, st, ev0, ev1);
    } else if constexpr (D == 96) {
        return launch_multi_k<D, MF, 96, RBMAX>(m, sh, grid, lds, st, ev0, ev1);
    } else {
        if (G == 16) return launch_multi_k<D, MF, 16, RBMAX>(m, sh, grid, lds, st, ev0, ev1);
        if (G == 32) return launch_multi_k<D, MF, 32, RBMAX>(m, sh, grid, lds, st, ev0, ev1);
        return launch_multi_k<D, MF, 64, RBMAX>(m, sh, grid, lds, st, ev0, ev1);
    }
}

// LDS bytes of one multi-loop ring slot (shared reference stage plus one
// residual stage per call with a residual, nres of them)
template <int D, bool MF, int RBMAX>
int multi_slot_bytes(int G, int nres) {
    const int msz = MF ? 4 : 2, ppi = Lanes<D>::PPI;
    const int mb = 16 * (D / G) * 2 * msz, ab = 16 * msz;
    const int ref = 2 * ppi * (16 * D / 2) + ppi * 2 * mb;
    const int res = 2 * ppi * (16 * D * RBMAX / 8) + ppi * 2 * (mb + ab);
    return ref + nres * res;
}

// LDS bytes of the multi-loop kernel outside its ring: one 16-byte padding
// slot and one weight scratch per wave, and with shared reference rows two
// row buffers and two factor buffers
template <int D>
int multi_fixed_bytes(int nl, bool sh) {
    return nl * (16 + Lanes<D>::PPI * kWScratch) + (sh ? 2 * Lanes<D>::PPI * kWScratch + 2 * kMaxMultiLoops * 4 : 0);
}

// LDS of one CU of the current device (queried once per device; 160 KB if
// the query fails)
static int lds_per_cu() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 160 * 1024;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || n <= 0)
        n = 160 * 1024;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workgroups of one multi-loop kernel variant with nl waves that its
// registers and wave slots let one CU hold (queried once per variant and nl)
template <int D, bool MF, int G, int RBMAX, bool SH>
int multi_occ_k(int nl) {
    static std::atomic<int> cache[kMaxMultiLoops + 1];
    int n = cache[nl].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rq_multi_kernel<D, MF, G, RBMAX, SH>, 64 * nl, 0) !=
            hipSuccess || n <= 0)
        n = 1;
    cache[nl].store(n, std::memory_order_relaxed);
    return n;
}

template <int D, bool MF, int RBMAX>
int multi_occ(int G, int nl, bool sh) {
    auto k = [&](auto gt) {
        constexpr int GG = decltype(gt)::value;
        return sh ? multi_occ_k<D, MF, GG, RBMAX, true>(nl) : multi_occ_k<D, MF, GG, RBMAX, false>(nl);
    };
    if constexpr (D == 128) {
        if (G == 32) return k(std::integral_constant<int, 32>{});
        if (G == 64) return k(std::integral_constant<int, 64>{});
        return k(std::integral_constant<int, 128>{});
    } else if constexpr (D == 96) {
        return k(std::integral_constant<int, 96>{});
    } else {
        if (G == 16) return k(std::integral_constant<int, 16>{});
        if (G == 32) return k(std::integral_constant<int, 32>{});
        return k(std::integral_constant<int, 64>{});
    }
}

// Ring depth of the multi-loop kernel, at most 8: as deep as the LDS share
// of one workgroup allows when the CU holds as many workgroups as the
// kernel's registers and wave slots admit (LDS then never lowers the
// occupancy), at most 64 KB; a ring of fewer than 3 stages takes 64 KB.
template <int D, bool MF, int RBMAX>
int multi_ring_depth(int G, int nl, int nres, bool sh) {
    const int fixed = multi_fixed_bytes<D>(nl, sh), slot = multi_slot_bytes<D, MF, RBMAX>(G, nres);
    const int budget = std::min(64 * 1024, lds_per_cu() / multi_occ<D, MF, RBMAX>(G, nl, sh));
    const int d = (budget - fixed) / slot;
    return std::min(8, d >= 3 ? d : (64 * 1024 - fixed) / slot);
}

template <int D>
hipError_t launch_decode_d(const DecodeCall &c) {
    const Geom &g = *c.g;
    const bool kvf = g.kvdt == RQ_DTYPE_F32, mf = g.meta == RQ_DTYPE_F32;
    const int tiles = (c.B + kPrepRows - 1) / kPrepRows;

    QPrepArgs qa;
    qa.q = c.q; qa.rot = c.rot; qa.qpack = c.qpack; qa.B = c.B; qa.H = g.H;
    CombineArgs ca;
    for (int i = 0; i < RQ_MAX_LOOPS; ++i) {
        const bool res = i < c.n && c.loops[i] != g.L - 1 && !g.direct;
        qa.rb[i] = res ? g.bits[c.loops[i]] : 0;
        qa.ro[i] = (g.direct && i < c.n) ? g.bits[c.loops[i]] : 4;
        ca.is_res[i] = res ? 1 : 0;
    }
    dim3 pgrid(g.H, c.n, tiles);
    hipError_t err = hipSuccess;
    if (!c.stream_probe) {
        if (kvf) hipLaunchKernelGGL((rq_qprep_kernel<D, true>), pgrid, dim3(64 * kPrepRows), 0, c.stream, qa);
        else hipLaunchKernelGGL((rq_qprep_kernel<D, false>), pgrid, dim3(64 * kPrepRows), 0, c.stream, qa);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }

    const float score_scale = c.softmax_scale * kLog2e;
    const int ref = g.L - 1;
    const bool multi = c.n >= 2 && !g.direct;   // direct loops share nothing: one kernel per call
    if (multi) {
        // multi-loop mode: loop calls in balanced groups of at least 2 and at
        // most nl_max waves, each group reading every reference page once
        bool any4 = false;
        for (int i = 0; i < c.n; ++i) any4 = any4 || (c.loops[i] != ref && g.bits[c.loops[i]] == 4);
        auto depth = [&](int nl) {
            if (mf) return any4 ? multi_ring_depth<D, true, 4>(g.G, nl, nl, false)
                                : multi_ring_depth<D, true, 2>(g.G, nl, nl, false);
            return any4 ? multi_ring_depth<D, false, 4>(g.G, nl, nl, false)
                        : multi_ring_depth<D, false, 2>(g.G, nl, nl, false);
        };
        int nl_max = 3;
        for (int nl = std::min(c.n, kMaxMultiLoops); nl > 3; --nl)
            if (depth(nl) >= 3) { nl_max = nl; break; }
        const int ngroups = (c.n + nl_max - 1) / nl_max;
        int first = 0;
        for (int k = 0; k < ngroups; ++k) {
            const int nl = c.n / ngroups + (k < c.n % ngroups ? 1 : 0);
            MultiArgs m;
            m.pool = c.pool; m.slab = g.slab; m.H = g.H; m.nblk = g.nblk;
            m.ref_off = (int)g.loop_off[ref]; m.ref_rec = g.rec[ref];
            m.nl = nl;
            bool g4 = false;
            int nref = 0;
            for (int w = 0; w < kMaxMultiLoops; ++w) {
                const int l = w < nl ? c.loops[first + w] : ref;
                m.rb[w] = (l == ref) ? 0 : g.bits[l];
                m.res_off[w] = (int)g.loop_off[l];
                m.res_rec[w] = g.rec[l];
                g4 = g4 || m.rb[w] == 4;
                nref += (w < nl && l == ref) ? 1 : 0;
            }
            m.block_table = c.block_table; m.max_blocks = c.max_blocks; m.seq_lens = c.seq_lens;
            m.qpack = c.qpack + (int64_t)first * c.B * g.H * qpack_bytes(D);
            m.partials = c.partials + (int64_t)first * c.B * g.H * c.nparts * partial_floats(D);
            m.B = c.B; m.nsplit = c.nsplit; m.split_pages = c.split_pages;
            m.score_scale = score_scale;
            const int nres = nl - nref;
            m.nres = nres;
            int slot;
            auto ring = [&](bool sh) {
                if (mf) return g4 ? multi_ring_depth<D, true, 4>(g.G, nl, nres, sh)
                                  : multi_ring_depth<D, true, 2>(g.G, nl, nres, sh);
                return g4 ? multi_ring_depth<D, false, 4>(g.G, nl, nres, sh)
                          : multi_ring_depth<D, false, 2>(g.G, nl, nres, sh);
            };
            if (mf) slot = g4 ? multi_slot_bytes<D, true, 4>(g.G, nres) : multi_slot_bytes<D, true, 2>(g.G, nres);
            else slot = g4 ? multi_slot_bytes<D, false, 4>(g.G, nres) : multi_slot_bytes<D, false, 2>(g.G, nres);
            // shared reference rows: the group holds the reference loop (whose
            // wave owns the rows), every (call, group) row pair fits the
            // 16 rows of the A operand, and the ring keeps a stage in flight
            // besides the current and the previous one
            const bool sh = nref == 1 && nl * (D / g.G) <= 8 && ring(true) >= 3;
            m.nst = ring(sh);
            if (m.nst < 2) return hipErrorInvalidConfiguration;
            size_t lds = (size_t)m.nst * slot + multi_fixed_bytes<D>(nl, sh);
            const bool last = k == ngroups - 1;
            // the current tokens' encode rides in the last group's launch
            m.enc_x0 = c.nsplit; m.enc_items = 0; m.enc_kvf = kvf ? 1 : 0;
            int ex = 0;
            if (last && c.enc_T > 0) {
                enc::fill_args(m.enc, g, c.enc_pool, c.enc_kv, c.rot, c.enc_slots, c.enc_T);
                m.enc_items = (c.enc_T + enc::kTT - 1) / enc::kTT * 2 * (g.L > 1 ? g.L - 1 : 1);
                ex = (m.enc_items + c.B - 1) / c.B;
                lds = std::max(lds, (size_t)enc::kEncLdsBytes);
            }
            dim3 grid(c.nsplit + ex, g.H, c.B);
            hipEvent_t e0 = last ? c.ev_begin : nullptr, e1 = last ? c.ev_end : nullptr;
            if (mf) err = g4 ? launch_multi_g<D, true, 4>(m, sh, g.G, grid, lds, c.stream, e0, e1)
                             : launch_multi_g<D, true, 2>(m, sh, g.G, grid, lds, c.stream, e0, e1);
            else err = g4 ? launch_multi_g<D, false, 4>(m, sh, g.G, grid, lds, c.stream, e0, e1)
                          : launch_multi_g<D, false, 2>(m, sh, g.G, grid, lds, c.stream, e0, e1);
            if (err != hipSuccess) return err;
            first += nl;
        }
    }
    bool enc_done = multi;   // multi-loop mode: attached to the last group above
    if (c.stream_probe && (multi || c.n != 1)) return hipErrorInvalidValue;
    for (int i = 0; i < (multi ? 0 : c.n); ++i) {
        const int l = c.loops[i];
        SplitArgs s;
        s.pool = c.pool; s.slab = g.slab; s.H = g.H; s.nblk = g.nblk; s.G = g.G;
        const int first = g.direct ? l : ref;   // the record read in full: the reference, or loop l itself
        s.ref_off = (int)g.loop_off[first]; s.ref_rec = g.rec[first]; s.ref_code_bytes = g.code_bytes[first];
        s.res_off = (int)g.loop_off[l]; s.res_rec = g.rec[l]; s.res_code_bytes = g.code_bytes[l];
        s.meta_bytes = g.meta_bytes;
        s.block_table = c.block_table; s.max_blocks = c.max_blocks; s.seq_lens = c.seq_lens;
        s.qpack = c.qpack + (int64_t)i * c.B * g.H * qpack_bytes(D);
        s.partials = c.partials + (int64_t)i * c.B * g.H * c.nparts * partial_floats(D);
        s.nsplit = c.nsplit; s.split_pages = c.split_pages;
        s.score_scale = score_scale;
        const int rb = (l == ref || g.direct) ? 0 : g.bits[l];
        const int refb = g.direct ? g.bits[l] : 4;
        const int nwg = (c.nsplit + kWaves - 1) / kWaves;
        s.nwg = nwg;
        // the current tokens' encode rides in the first reference-loop launch
        s.enc_x0 = nwg; s.enc_items = 0; s.enc_kvf = kvf ? 1 : 0;
        int ex = 0;
        if (l == ref && c.enc_T > 0 && !enc_done && !g.direct) {
            enc::fill_args(s.enc, g, c.enc_pool, c.enc_kv, c.rot, c.enc_slots, c.enc_T);
            s.enc_items = (c.enc_T + enc::kTT - 1) / enc::kTT * 2 * (g.L > 1 ? g.L - 1 : 1);
            ex = (s.enc_items + c.B - 1) / c.B;
            enc_done = true;
        }
        dim3 grid(nwg + ex, g.H, c.B);
        const bool last = i == c.n - 1;
        if (c.stream_probe)   // the streaming reference alone: no query prep, merge or encode
            return launch_stream_d<D>(s, rb, refb, mf, dim3(nwg, g.H, c.B), c.stream, c.ev_begin, c.ev_end);
        err = launch_split_d<D>(s, rb, refb, mf, grid, c.stream, last ? c.ev_begin : nullptr, last ? c.ev_end : nullptr);
        if (err != hipSuccess) return err;
    }

    if (c.enc_T > 0 && !enc_done) {
        // no reference-loop call to ride in: the encoder's own launch
        EncodeCall ec;
        ec.g = &g; ec.pool = c.enc_pool; ec.kv_new = c.enc_kv; ec.rot = c.rot; ec.slots = c.enc_slots;
        ec.T = c.enc_T; ec.stream = c.stream;
        err = launch_encode(ec);
        if (err != hipSuccess) return err;
    }
    ca.partials = c.partials; ca.nparts = c.nparts; ca.spp = multi ? 1 : kWaves;
    ca.split_pages = c.split_pages;
    ca.max_blocks = c.max_blocks; ca.seq_lens = c.seq_lens;
    ca.q = c.q; ca.tail_k = c.tail_k; ca.tail_v = c.tail_v; ca.rot = c.rot; ca.out = c.out;
    ca.B = c.B; ca.H = g.H; ca.score_scale = score_scale;
    if (kvf) hipLaunchKernelGGL((rq_combine_kernel<D, true>), pgrid, dim3(64 * kPrepRows), 0, c.stream, ca);
    else hipLaunchKernelGGL((rq_combine_kernel<D, false>), pgrid, dim3(64 * kPrepRows), 0, c.stream, ca);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeCall &c) {
    if (c.B <= 0 || c.n <= 0) return hipSuccess;
    switch (c.g->D) {
        case 64: return launch_decode_d<64>(c);
        case 96: return launch_decode_d<96>(c);
        case 128: return launch_decode_d<128>(c);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rq
