// Encoder work item shared by the stand-alone encode kernel and the decode
// kernels that run the encode in the same launch (see rq_encode.hip for the
// method and its citations).
#pragma once

#include "rq_device.h"
#include "rq_internal.h"

namespace rq {
namespace enc {

constexpr int kTT = 16;
constexpr int kThreads = 256;
constexpr int kMaxD = 128;
constexpr int kRowStride = kMaxD + 1;   // doubles; +1 keeps MFMA operand reads bank-conflict free
constexpr int kEncLdsBytes = (kTT * kRowStride + 2 * kTT) * 8;

struct EncArgs {
    uint8_t *pool;
    int64_t slab;
    int H, nblk, D, G, L, meta_bytes;
    int bits[RQ_MAX_LOOPS];
    int rec[RQ_MAX_LOOPS];
    int code_bytes[RQ_MAX_LOOPS];
    int64_t loop_off[RQ_MAX_LOOPS];
    const void *kv;
    const float *rot;
    const int64_t *slots;
    int T;
};

template <bool META_F32>
__device__ __forceinline__ double meta_round(double x) {
    if constexpr (META_F32) return (double)(float)x;
    else return f16_bits_to_f64(f64_to_f16_bits(x));
}

template <bool META_F32>
__device__ __forceinline__ void store_meta(uint8_t *p, double v) {
    if constexpr (META_F32) *(float *)p = (float)v;
    else *(uint16_t *)p = f64_to_f16_bits(v);
}

// Min/max over the lanes of one quantization group. Lanes hold 2 adjacent
// channels; a group of G channels spans G/2 aligned lanes, or the whole wave
// when the group is the whole head (inactive lanes carry neutral values).
__device__ __forceinline__ void group_minmax(double &lo, double &hi, int span) {
    for (int off = 1; off < span; off <<= 1) {
        lo = fmin(lo, __shfl_xor(lo, off, 64));
        hi = fmax(hi, __shfl_xor(hi, off, 64));
    }
}

// Place one V code of token offset `off` (0..15) and channel c into a V
// record's code block (the record format in rq.h): lane 16*(off/4) + c%16,
// word plane p = (c/16)/W (W = 8/bits column groups per 32-bit word, every
// earlier plane full: 64 lanes x 4 bytes), field 2*W_p*(v%2) + W_p*(v/2) + i
// with v = off%4, i = (c/16)%W and W_p the groups in word p (the last word
// of D = 96 INT2 holds 2 and is a 16-bit unit). Codes of the four tokens of
// a quad share words, and tokens are written by different waves and
// launches, so the field is cleared and set with atomic and/or on the
// aligned 32-bit word (other tokens' bits are untouched).
__device__ __forceinline__ void put_v_code(uint8_t *rec, int D, int bits, int off, int c, uint32_t code) {
    const int u = off >> 2, v = off & 3;
    const int m = c >> 4, j = c & 15;
    const int lam = 16 * u + j;
    const int W = 8 / bits, M = D >> 4;
    const int p = m / W, i = m % W;
    const int wp = min(W, M - W * p);
    const int f = 2 * wp * (v & 1) + wp * (v >> 1) + i;
    const int byte = 256 * p + lam * wp * bits / 2;
    uint32_t *word = (uint32_t *)(rec + (byte & ~3));
    const int sh = (byte & 3) * 8 + f * bits;
    atomicAnd(word, ~(((1u << bits) - 1u) << sh));
    atomicOr(word, code << sh);
}

// Quantize the row held by this wave (two channels per lane) and write codes
// and (scale, zero) into the record at `rec` for token offset `off`: K
// records token-major, V records (vorder) in the column-lane order of
// put_v_code. `write` and `vorder` are wave-uniform.
template <bool META_F32>
__device__ void quantize_row(double y0, double y1, bool active, int lane, int D, int G, int bits,
                             uint8_t *rec, int code_bytes, int off, bool write, bool vorder) {
    const int span = (G == D) ? 64 : G / 2;
    double lo = active ? fmin(y0, y1) : __builtin_inf();
    double hi = active ? fmax(y0, y1) : -__builtin_inf();
    group_minmax(lo, hi, span);
    const int qmax = (1 << bits) - 1;
    const double s = meta_round<META_F32>((hi - lo) / (double)qmax);
    const double z = meta_round<META_F32>(lo);
    uint32_t c0 = 0, c1 = 0;
    if (s != 0.0) {
        c0 = (uint32_t)fmin(fmax(rint((y0 - z) / s), 0.0), (double)qmax);
        c1 = (uint32_t)fmin(fmax(rint((y1 - z) / s), 0.0), (double)qmax);
    }
    if (vorder) {
        if (write && active) {
            put_v_code(rec, D, bits, off, 2 * lane, c0);
            put_v_code(rec, D, bits, off, 2 * lane + 1, c1);
        }
    }
    // pack (K records): each lane contributes its two codes; OR-reduce inside
    // the lanes that share one 32-bit word (4 lanes for INT4, 8 lanes for INT2)
    uint32_t word;
    int lanes_per_word;
    if (bits == 4) {
        word = (active ? (c0 | (c1 << 4)) : 0u) << (8 * (lane & 3));
        lanes_per_word = 4;
    } else {
        word = (active ? (c0 | (c1 << 2)) : 0u) << (4 * (lane & 7));
        lanes_per_word = 8;
    }
    for (int off2 = 1; off2 < lanes_per_word; off2 <<= 1) word |= __shfl_xor(word, off2, 64);
    if (!write) return;
    const int row_bytes = D * bits / 8;
    if (!vorder && (lane % lanes_per_word) == 0 && active) {
        const int w = lane / lanes_per_word;
        *(uint32_t *)(rec + (int64_t)off * row_bytes + 4 * w) = word;
    }
    const int ng = D / G;
    const int msz = META_F32 ? 4 : 2;
    const int first = 2 * lane;                 // first channel of this lane
    if (active && (first % G) == 0) {
        const int g = first / G;
        uint8_t *m = rec + code_bytes + (int64_t)(off * ng + g) * 2 * msz;
        store_meta<META_F32>(m, s);
        store_meta<META_F32>(m + msz, z);
    }
}

// One work item of the encoder: (tile of 16 tokens, head h, item z = kv * nres
// + l) with nres = max(L-1, 1), run by a 256-thread workgroup. `lds` is the
// workgroup's scratch of at least kEncLdsBytes (8-byte aligned): one
// [16][kRowStride] float64 array that first holds the reference rows and is
// then overwritten in place by the residual rows (each element is read and
// rewritten by the same thread), plus <ref,ref> and alpha per token. The
// workgroup's nw waves (2 <= nw <= 16; the caller's whole workgroup) share the
// rows and rotation tiles.
template <bool KV_F32, bool META_F32>
__device__ void encode_item(const EncArgs &a, int tile, int h, int z, uint8_t *lds, int nw) {
    double *rows = (double *)lds;                 // x_ref, then d = x - alpha x_ref, then R d
    double *xref = rows;
    double *refsq = rows + kTT * kRowStride;
    double *alph = refsq + kTT;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nres = a.L > 1 ? a.L - 1 : 1;
    const int kv = z / nres, l = z % nres;        // l: this item's residual loop
    const int D = a.D, L = a.L, H = a.H;
    const int c0 = 2 * lane, c1 = 2 * lane + 1;
    const bool active = c0 < D;
    const int msz = META_F32 ? 4 : 2;

    // ---- reference loop: quantize in INT4, keep x_ref and <x_ref, x_ref>
    for (int t = wave; t < kTT; t += nw) {
        const int tg = tile * kTT + t;
        const bool tok = tg < a.T;
        int64_t slot = tok ? a.slots[tg] : -1;
        const bool write = slot >= 0 && slot < (int64_t)a.nblk * 16;
        const int64_t blk = write ? slot / 16 : 0;
        const int off = write ? (int)(slot % 16) : 0;
        double x0 = 0.0, x1 = 0.0;
        if (tok && active) {
            const int64_t base = ((((int64_t)(L - 1) * 2 + kv) * a.T + tg) * H + h) * D;
            x0 = (double)load_kv<KV_F32>(a.kv, base + c0);
            x1 = (double)load_kv<KV_F32>(a.kv, base + c1);
        }
        xref[t * kRowStride + c0] = x0;
        if (active) xref[t * kRowStride + c1] = x1;
        const double sq = wave_sum_f64(x0 * x0 + x1 * x1);
        if (lane == 0) refsq[t] = sq;
        uint8_t *rec = a.pool + (blk * H + h) * a.slab + a.loop_off[L - 1] + (int64_t)kv * a.rec[L - 1];
        quantize_row<META_F32>(x0, x1, active, lane, D, a.G, 4, rec, a.code_bytes[L - 1], off, write && l == 0,
                               kv == 1);
    }
    __syncthreads();

    // ---- residual loop l
    if (L > 1) {
        // alpha (least squares), rounded to the meta dtype; d = x_l - alpha*x_ref
        for (int t = wave; t < kTT; t += nw) {
            const int tg = tile * kTT + t;
            const bool tok = tg < a.T;
            double x0 = 0.0, x1 = 0.0;
            if (tok && active) {
                const int64_t base = ((((int64_t)l * 2 + kv) * a.T + tg) * H + h) * D;
                x0 = (double)load_kv<KV_F32>(a.kv, base + c0);
                x1 = (double)load_kv<KV_F32>(a.kv, base + c1);
            }
            const double r0 = xref[t * kRowStride + c0];    // read, then overwritten below
            const double r1 = active ? xref[t * kRowStride + c1] : 0.0;
            const double num = wave_sum_f64(x0 * r0 + x1 * r1);
            const double den = refsq[t];
            const double a64 = (den == 0.0) ? 0.0 : num / den;
            const double al = meta_round<META_F32>(a64);
            if (lane == 0) alph[t] = al;
            rows[t * kRowStride + c0] = active ? fma(-al, r0, x0) : 0.0;
            if (active) rows[t * kRowStride + c1] = fma(-al, r1, x1);
        }
        __syncthreads();

        // r = R d for the 16 rows: [16 x D] x R^T on the f64 matrix cores.
        // v_mfma_f64_16x16x4f64: lane l supplies A[l%16][k0 + l/16] and
        // B[k0 + l/16][l%16]; its four results are D[4*i + l/16][l%16],
        // i = 0..3 (rows strided by 4, unlike the f32 16x16x4 form).
        const float *R = a.rot + ((int64_t)h * 2 + kv) * D * D;
        // column tiles nt = wave + i*nw: at most kMaxTiles per wave (nw >= 2)
        constexpr int kMaxTiles = kMaxD / 16 / 2;
        doublex4 acc[kMaxTiles];
#pragma unroll
        for (int i = 0; i < kMaxTiles; ++i) {
            const int nt = wave + i * nw;
            doublex4 c = {0.0, 0.0, 0.0, 0.0};
            if (nt < D / 16) {
                const int n = nt * 16 + (lane & 15);
#pragma unroll 8
                for (int kk = 0; kk < D / 4; ++kk) {
                    const int k = 4 * kk + (lane >> 4);
                    const double av = rows[(lane & 15) * kRowStride + k];
                    const double bv = (double)R[(int64_t)n * D + k];
                    c = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, c, 0, 0, 0);
                }
            }
            acc[i] = c;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kMaxTiles; ++i) {
            const int nt = wave + i * nw;
            if (nt < D / 16) {
                const int col = nt * 16 + (lane & 15);
                for (int v = 0; v < 4; ++v) rows[(4 * v + (lane >> 4)) * kRowStride + col] = acc[i][v];
            }
        }
        __syncthreads();

        // quantize each rotated row and write codes, (scale, zero) and alpha
        for (int t = wave; t < kTT; t += nw) {
            const int tg = tile * kTT + t;
            int64_t slot = (tg < a.T) ? a.slots[tg] : -1;
            const bool write = slot >= 0 && slot < (int64_t)a.nblk * 16;
            const int64_t blk = write ? slot / 16 : 0;
            const int off = write ? (int)(slot % 16) : 0;
            const double y0 = rows[t * kRowStride + c0];
            const double y1 = active ? rows[t * kRowStride + c1] : 0.0;
            uint8_t *rec = a.pool + (blk * H + h) * a.slab + a.loop_off[l] + (int64_t)kv * a.rec[l];
            quantize_row<META_F32>(y0, y1, active, lane, D, a.G, a.bits[l], rec, a.code_bytes[l], off, write,
                                   kv == 1);
            if (write && lane == 0)
                store_meta<META_F32>(rec + a.code_bytes[l] + a.meta_bytes + (int64_t)off * msz, alph[t]);
        }
        __syncthreads();
    }
}


// Fill the encoder arguments from a layout geometry.
inline void fill_args(EncArgs &a, const Geom &g, uint8_t *pool, const void *kv_new, const float *rot,
                      const int64_t *slots, int T) {
    a.pool = pool;
    a.slab = g.slab;
    a.H = g.H;
    a.nblk = g.nblk;
    a.D = g.D;
    a.G = g.G;
    a.L = g.L;
    a.meta_bytes = g.meta_bytes;
    for (int l = 0; l < RQ_MAX_LOOPS; ++l) {
        a.bits[l] = g.bits[l];
        a.rec[l] = g.rec[l];
        a.code_bytes[l] = g.code_bytes[l];
        a.loop_off[l] = g.loop_off[l];
    }
    a.kv = kv_new;
    a.rot = rot;
    a.slots = slots;
    a.T = T;
}

// Work items of an encode of T tokens: tiles x (K|V x residual loops) per head.
inline int items_per_head(const Geom &g, int T) { return (T + kTT - 1) / kTT * 2 * (g.L > 1 ? g.L - 1 : 1); }

}  // namespace enc
}  // namespace rq
