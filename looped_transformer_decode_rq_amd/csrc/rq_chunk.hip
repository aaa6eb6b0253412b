// Chunked prefill attention over the packed, paged ResidualQuant cache.
//
// A chunk of C new tokens per sequence, for one loop, attends every cached
// token of that loop (reconstructed from the INT4 reference and the loop's
// rotated residual, arXiv 2610.10381 abstract; rit.work summary, section on
// how each pass is restored: reference and differences rebuilt inside
// attention, nothing decompressed written back) and, causally, the chunk's own
// uncompressed K/V (query i sees chunk tokens 0..i).
//
// Unlike decode, sixteen queries share every page, so both products run on
// the matrix cores, with tokens as the 16 rows of one operand:
//   scores^T = Kcodes x Q on the int8 matrix cores (v_mfma_i32_16x16x64_i8):
//     A = the K codes of 16 tokens, one code per byte (K records are
//     token-major: a lane's codes of one step are one or two words, unpacked
//     by two masks and a shift per word, in the order that leaves them);
//     B = a fixed-point copy of each query, round(q 2^e) with one power of
//     two per query row and |round(q 2^e)| < 2^22, as three signed base-256
//     digits in the same channel order (q' = R_K q likewise for the
//     residual, under the same power of two): exact integer dot products per
//     digit, joined in fp32. The scores stay in units of 2^-e until the
//     exponent, where the scale joins the subtraction of the running max. The
//     output leaves each lane with four tokens of one query, which is exactly
//     the A operand of the next product, so no transpose is needed;
//   out = P x Vcodes on the fp16 matrix cores (v_mfma_f32_16x16x32_f16):
//     A = fp16 hi/lo of p * alpha * s (reference) and p * s (residual),
//     B = the V codes as fp16 (16 + c) in their stored operand order.
// Per token and group: q . k_hat = alpha * (s * sum q c + z * sum q) +
// (s_r * sum q' c_r + z_r * sum q'), one group per token-head (group_size ==
// head_dim).
//
// Three kernels per call:
//   rq_chunk_qprep    per (head, 16 query rows): the digits of q and of
//                     q' = R_K q (computed on the f32 matrix cores) under one
//                     scale 2^-e per row, and their sums
//   rq_chunk_split    per (head, split of pages, sequence x 64 queries): four
//                     waves of 16 queries walk the split's pages, online
//                     softmax per query, one partial per (split, query)
//   rq_chunk_combine  per (head, sequence, 16 queries): merge the partials,
//                     the chunk's causal part on the bf16 matrix cores,
//                     out = acc_ref/l + R_V^T acc_res/l on the f32 matrix cores
#include <hip/hip_ext.h>

#include "rq_device.h"
#include "rq_internal.h"
#include "rq_vmfma.h"

namespace rq {
namespace {

constexpr float kLog2eC = 1.4426950408889634f;
constexpr float kThreshC = 8.0f;         // rescale when a score beats the running max by 2^8
// The running max before the first unmasked score: finite, so that a masked
// score's weight exp2(-inf - m) is 0 without a test; written out as -inf.
constexpr float kFloorC = -1e30f;
// LDS offset of the per-page token tables: after the ring (ring_bytes), the
// padding slots and the split's block ids, 16-byte aligned; two buffers of two
// pages x 8 entries x 16 tokens (floats)
__host__ __device__ constexpr int chunk_tab_offset(int ring_bytes, int split_pages) {
    return (ring_bytes + 64 + 4 * split_pages + 15) & ~15;
}
constexpr int kChunkTabBytes = 2 * 2 * 8 * 16 * 4;
constexpr int kChunkFold = 16;           // pages between folds of the zero terms into the accumulators

// ---------------------------------------------------- int8 score operands
// A lane of the score product holds one token's (K) or one query's (B)
// channels kb*D/4 .. kb*D/4 + D/4 - 1; step s of the 16x16x64 product takes
// sixteen of them, as bytes in the order the unpacking of the stored codes
// leaves them (byte e of the operand's four words):
//   4-bit codes, words w0, w1 = channels 16s + 0..7, 16s + 8..15 (nibble j =
//   channel j): operand (w0 & M, w0 >> 4 & M, w1 & M, w1 >> 4 & M), so byte
//   i of word d is channel 16s + 8 (d / 2) + 2 i + d % 2;
//   2-bit codes, word w = channels 16s + 0..15: operand (w >> 2d & M), byte i
//   of word d is channel 16s + 4 i + d.
// Channels past D/4 (the second step of D = 96) are zero in the query.
template <int D>
__host__ __device__ constexpr int chunk_steps8() { return (D / 4 + 15) / 16; }

template <int D, int BITS>
__device__ __forceinline__ uint4 chunk_kbytes(const uint32_t *w, int s) {
    if constexpr (BITS == 4) {
        constexpr int NW = (D * 4 / 32 + 3) / 4;
        const uint32_t w0 = w[2 * s], w1 = 2 * s + 1 < NW ? w[2 * s + 1] : 0u;
        return make_uint4(w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu);
    } else {
        const uint32_t v = w[s];
        return make_uint4(v & 0x03030303u, (v >> 2) & 0x03030303u, (v >> 4) & 0x03030303u, (v >> 6) & 0x03030303u);
    }
}

// Maxima of scores, which are never NaN: the plain instructions. (fmaxf
// makes the compiler quiet possible signaling NaNs first, one extra
// instruction per operand it cannot prove canonical.)
__device__ __forceinline__ float vmax2(float a, float b) {
    float r;
    __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Max of x over lanes l, l^16, l^32, l^48 (the four lanes that share a query)
// with the gfx950 row and half swaps (v_permlane16_swap, v_permlane32_swap):
// no LDS round trip, unlike a bpermute shuffle
__device__ __forceinline__ float max_lanes4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = vmax2(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return vmax2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum of x over the same four lanes, as (x_l + x_l^16) + (x_l^32 + x_l^48)
__device__ __forceinline__ float sum_lanes4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef int intx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ intx4 mfma_i8(uint4 a, uint4 b, intx4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(intx4, a), __builtin_bit_cast(intx4, b), c, 0, 0,
                                                 0);
}

// Fixed point of a query row: exponent e with |round(x 2^e)| < 2^22 for
// every |x| <= mx (clamped so that 2^-e stays a normal float), the rounded
// integer, and its signed base-256 digits d0 + 256 d1 + 65536 d2 (d0, d1 in
// -128..127; |d2| <= 64)
__device__ __forceinline__ int fix_exp(float mx) {
    if (!(mx > 0.f)) return 0;
    const int e = 21 - ilogbf(mx);
    return e < -126 ? -126 : (e > 126 ? 126 : e);
}
__device__ __forceinline__ int fix_int(float x, int e) {
    const float y = rintf(ldexpf(x, e));
    return (int)fminf(fmaxf(y, -4194303.f), 4194303.f);
}
__device__ __forceinline__ int fix_digit(int v, int l) {
    const int d0 = ((v + 128) & 255) - 128;
    const int v1 = (v - d0) >> 8;
    const int d1 = ((v1 + 128) & 255) - 128;
    return l == 0 ? d0 : (l == 1 ? d1 : (v1 - d1) >> 8);
}

// Byte of channel c (0..D-1) in the digit words of a query row: the words
// are [step s][digit l][lane slot kb][4 words d], byte i of word d holding
// the slot's channel 16s + 8 (d / 2) + 2 i + d % 2 (INT4 operand order) or
// 16s + 4 i + d (INT2), slot kb covering channels kb D/4 ..; this returns
// the byte of digit 0 (digit l: + 64 l).
template <int D, int BITS>
__device__ __forceinline__ int digit_byte(int c) {
    const int kb = c / (D / 4), ch = c % (D / 4), st = ch >> 4, rem = ch & 15;
    const int d = BITS == 4 ? 2 * (rem >> 3) + (rem & 1) : rem & 3;
    const int i = BITS == 4 ? (rem & 7) >> 1 : rem >> 2;
    return st * 192 + kb * 16 + d * 4 + i;
}

// ------------------------------------------------------------------ qprep
struct ChunkPrepArgs {
    const uint16_t *q;      // [R][H][D] bf16, R = B*C rows
    const float *rot;       // [H][2][D][D]
    uint8_t *qrec;          // [R][H][chunk_qrec_bytes]
    int R, H, res;          // res: bits of the residual codes (0: reference loop)
};

// One workgroup per (head, 16 rows); one wave per row.
template <int D>
__global__ __launch_bounds__(1024) void rq_chunk_qprep_kernel(ChunkPrepArgs a) {
    constexpr int QS = D + 1;
    __shared__ float Q[16 * QS];
    __shared__ float QR[16 * QS];
    __shared__ uint32_t DW[16 * 2 * chunk_steps8<D>() * 48];   // per row: the digit words of q and q'
    const int lane = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int h = blockIdx.x, tile = blockIdx.y;
    const int row = tile * 16 + r;
    const bool row_ok = row < a.R;
    const bool rot_wave = a.res && r < D / 16;
    const int n = r * 16 + (lane & 15);
    // this lane's B operands: D/4 consecutive floats of row n of R_K (vector
    // loads); step kk gives k-slot l/16 the channel k = (D/4)(l/16) + kk
    float rk[D / 4];
    if (rot_wave) {
        const float4 *RK = (const float4 *)(a.rot + ((int64_t)h * 2 + 0) * D * D + (int64_t)n * D +
                                            (lane >> 4) * (D / 4));
#pragma unroll
        for (int k4 = 0; k4 < D / 16; ++k4) {
            const float4 v = RK[k4];
            rk[4 * k4] = v.x; rk[4 * k4 + 1] = v.y; rk[4 * k4 + 2] = v.z; rk[4 * k4 + 3] = v.w;
        }
    }
    for (int c = lane; c < D; c += 64)
        Q[r * QS + c] = row_ok ? bf16_to_f32(a.q[((int64_t)row * a.H + h) * D + c]) : 0.0f;
    __syncthreads();
    if (rot_wave) {
        // q' = R_K q for the 16 rows: [16 x D] x R_K^T; v_mfma_f32_16x16x4f32:
        // lane l supplies A[l%16][k], B[k][l%16] for its k-slot l/16, receives
        // D[4*(l/16)+v][l%16]; wave r computes columns 16r..16r+15; four
        // independent accumulation chains (the products' latency overlaps)
        floatx4 c4[4] = {};
#pragma unroll
        for (int kk = 0; kk < D / 4; ++kk) {
            const int k = (lane >> 4) * (D / 4) + kk;
            c4[kk & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(Q[(lane & 15) * QS + k], rk[kk], c4[kk & 3], 0, 0, 0);
        }
        const floatx4 c = (c4[0] + c4[1]) + (c4[2] + c4[3]);
        for (int v = 0; v < 4; ++v) QR[(4 * (lane >> 4) + v) * QS + n] = c[v];
    }
    __syncthreads();
    if (!row_ok) return;
    // record: sum round(q 2^e), sum round(q' 2^e), 2^-e, 2^-e (floats), then
    // the digit words of q and of q' in operand order [step][digit][lane
    // slot kb][4 words]
    uint8_t *rec = a.qrec + ((int64_t)row * a.H + h) * chunk_qrec_bytes(D);
    const float *qrow = Q + r * QS, *rrow = QR + r * QS;
    const bool has1 = lane + 64 < D;
    const float x0 = qrow[lane], x1 = has1 ? qrow[lane + 64] : 0.f;
    const float y0 = a.res ? rrow[lane] : 0.f, y1 = (a.res && has1) ? rrow[lane + 64] : 0.f;
    // one exponent for q and q' (that of the larger magnitude), so that the
    // two sums of a score share the scale 2^-e
    float mx[2] = {fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(y0), fabsf(y1))};
    wave_max_n(mx);
    const int eq0 = fix_exp(mx[0]), er0 = fix_exp(mx[1]);
    const int eq = a.res ? min(eq0, er0) : eq0;
    // the fixed-point values (each channel converted once) and their sums
    // (exact: |sum| < 2^29)
    const int vq0 = fix_int(x0, eq), vq1 = has1 ? fix_int(x1, eq) : 0;
    const int vr0 = fix_int(y0, eq), vr1 = has1 ? fix_int(y1, eq) : 0;
    int sums[2] = {vq0 + vq1, vr0 + vr1};
    wave_sum_n(sums);
    // the digit words of this row, assembled byte by byte in LDS (zero
    // bytes for the padding channels), then stored as words
    constexpr int NS = chunk_steps8<D>();
    constexpr int NW = NS * 48;                 // words per quantity
    uint32_t *img = DW + r * 2 * NW;
    for (int j = lane; j < 2 * NW; j += 64) img[j] = 0u;
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's zeros land before its bytes
    uint8_t *bq = (uint8_t *)img, *br = (uint8_t *)(img + NW);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = lane + 64 * u;
        if (c < D) {
            const int vq = u ? vq1 : vq0, vr = u ? vr1 : vr0;
            const int oq = digit_byte<D, 4>(c);
#pragma unroll
            for (int l = 0; l < 3; ++l) bq[oq + 64 * l] = (uint8_t)fix_digit(vq, l);
            if (a.res) {
                const int orr = a.res == 4 ? digit_byte<D, 4>(c) : digit_byte<D, 2>(c);
#pragma unroll
                for (int l = 0; l < 3; ++l) br[orr + 64 * l] = (uint8_t)fix_digit(vr, l);
            }
        }
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // LDS keeps one wave's accesses in order
    uint32_t *wq = (uint32_t *)(rec + 16), *wr = wq + NW;
    for (int j = lane; j < NW; j += 64) {
        wq[j] = img[j];
        if (a.res) wr[j] = img[NW + j];
    }
    const int sq = sums[0], sr = sums[1];
    if (lane == 0) {
        float *hd = (float *)rec;
        hd[0] = (float)sq;
        hd[1] = (float)sr;
        hd[2] = ldexpf(1.f, -eq);
        hd[3] = hd[2];
    }
}

// ------------------------------------------------------------------ split
struct ChunkArgs {
    const uint8_t *pool;
    int64_t slab;
    int H, nblk;
    int ref_off, ref_rec, res_off, res_rec;   // slab offsets of the K records; V at + rec
    int meta_bytes;                           // (scale, zero) bytes of one record
    const int32_t *block_table;
    int max_blocks;
    const int32_t *seq_lens;
    const uint16_t *q;                        // [B][C][H][D] bf16
    const uint8_t *qrec;                      // [B*C][H][chunk_qrec_bytes]
    float *partials;                          // [B*C][H][nsplit][2 + 2D]
    int C, nqg, nsplit, split_pages;
    float score_scale;                        // softmax_scale * log2(e)
    int stage;                                // bytes of one ring stage: 2*ref_rec (+ 2*res_rec)
};

constexpr int kChunkStages = 8;               // ring depth in pages: two pairs in flight, one tabulated, one used
constexpr int kChunkMaxSplit = 1024;          // pages per split (block ids preloaded into LDS)

// 16x16x32 products: a lane's eight k values of A and of B are two 16x16x16
// operands side by side (the matrix cores pair element e of A with element e
// of B within a lane group, so any split of k between the halves works)
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ floatx4 mfma_f16x32(uint4 a, uint4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c, 0,
                                                  0, 0);
}

// This lane's K codes of one token: D*BITS/32 bytes (channels kb*D/4 ..
// kb*D/4 + D/4 - 1), as 32-bit words (the last one partial for D = 96 INT2)
template <int D, int BITS>
struct KChunk {
    static constexpr int NB = D * BITS / 32;
    static constexpr int NW = (NB + 3) / 4;
    uint32_t w[NW];
};

template <int D, int BITS>
__device__ __forceinline__ void load_k(KChunk<D, BITS> &k, const uint8_t *p) {
    using K = KChunk<D, BITS>;
    if constexpr (K::NB % 4 == 0) {
#pragma unroll
        for (int i = 0; i < K::NW; ++i) k.w[i] = ((const uint32_t *)p)[i];
    } else {
        // 6 bytes (D = 96, INT2), 2-byte aligned
        const uint16_t *h = (const uint16_t *)p;
        k.w[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        k.w[1] = h[2];
    }
}

// Where the K codes of a page record sit in an LDS stage. The record is token
// major (token t's D*BITS/8 bytes, then token t+1's), and the 16 lanes that
// read one channel chunk of 16 tokens would address pieces one token record
// apart (a 4-way LDS bank conflict for D = 128). The direct-to-LDS loads
// therefore transpose the code area at 16-byte granularity on the way in:
// piece c of token t lands at piece 16c + t, so those 16 lanes read 16
// consecutive pieces. Only where a lane's chunk lies inside one piece (D = 64
// and 128); for D = 96 the area is copied as stored.
template <int D, int BITS>
struct KSwz {
    static constexpr int CB = D * BITS / 32;          // bytes of one lane's chunk
    static constexpr int TB = D * BITS / 8;           // bytes of one token's codes
    static constexpr bool ON = 16 % CB == 0 && TB % 16 == 0;
    static constexpr int TP = TB / 16;                // pieces per token (when ON)
    static constexpr int PIECES = ON ? 16 * TP : 0;   // pieces of the code area that move
    // LDS byte offset of chunk kb of token x from the start of the codes
    __device__ static int off(int x, int kb) {
        if constexpr (ON) {
            const int o = kb * CB;
            return ((o >> 4) * 16 + x) * 16 + (o & 15);
        } else {
            return x * TB + kb * CB;
        }
    }
    // the record's piece that LDS piece j (< PIECES) holds
    __host__ __device__ static constexpr int src(int j) { return (j & 15) * TP + (j >> 4); }
};

// (scale, zero) of four consecutive tokens of one record
template <bool MF>
__device__ __forceinline__ void load_sz4(const uint8_t *p, float *s, float *z) {
    if constexpr (MF) {
        const float4 a = ((const float4 *)p)[0], b = ((const float4 *)p)[1];
        s[0] = a.x; z[0] = a.y; s[1] = a.z; z[1] = a.w; s[2] = b.x; z[2] = b.y; s[3] = b.z; z[3] = b.w;
    } else {
        const uint4 v = *(const uint4 *)p;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = f16_to_f32((uint16_t)(w[r] & 0xFFFF));
            z[r] = f16_to_f32((uint16_t)(w[r] >> 16));
        }
    }
}

template <bool MF>
__device__ __forceinline__ void load_a4(const uint8_t *p, float *al) {
    if constexpr (MF) {
        const float4 a = *(const float4 *)p;
        al[0] = a.x; al[1] = a.y; al[2] = a.z; al[3] = a.w;
    } else {
        const uint2 v = *(const uint2 *)p;
        al[0] = f16_to_f32((uint16_t)(v.x & 0xFFFF)); al[1] = f16_to_f32((uint16_t)(v.x >> 16));
        al[2] = f16_to_f32((uint16_t)(v.y & 0xFFFF)); al[3] = f16_to_f32((uint16_t)(v.y >> 16));
    }
}

// fp16 hi/lo of four weights as two A operands (token order 0..3), and their
// sum before the split (`used`, for the zero term: the matrix cores see hi +
// lo, and the offset then leaves 16 (hi + lo - w) per token, an unbiased
// rounding error the size of the split's own error on the code term). Each
// weight is first pinned as an fp32 register value: otherwise the compiler
// may fuse the product that forms it into some of the fp16 conversions and
// not into others (one rounding against two), and lo would then be formed
// against a different hi than the one the matrix cores see.
__device__ __forceinline__ void split4(const float *win, uint2 &hi, uint2 &lo, float &used) {
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[i] = win[i];
        __asm__ volatile("" : "+v"(w[i]));
    }
    halfx2 h01 = {(_Float16)w[0], (_Float16)w[1]}, h23 = {(_Float16)w[2], (_Float16)w[3]};
    hi = make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
    // lo = RNE_f16(w - hi), one mixed-precision FMA per weight (-1 * hi + w in
    // fp32, exact, rounded once to fp16 into the low or the high half)
    uint32_t l01, l23;
    __asm__("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l01) : "v"(hi.x), "v"(w[0]));
    __asm__("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(l01) : "v"(hi.x), "v"(w[1]));
    __asm__("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l23) : "v"(hi.y), "v"(w[2]));
    __asm__("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(l23) : "v"(hi.y), "v"(w[3]));
    lo = make_uint2(l01, l23);
    used = (w[0] + w[1]) + (w[2] + w[3]);
}

// acc[m] += Ahi x B_m + Alo x B_m for every column group m of a page pair:
// B_m = the fp16 (16 + c) codes of this lane group's four tokens of the first
// page, then of the second (the order of the A operands' weights); two
// 16x16x32 products per group against the same operand
template <int WP, int BITS, int I>
__device__ __forceinline__ void v_mfma_pair_word(floatx4 *acc, uint32_t w0, uint32_t w1, uint4 ahi, uint4 alo,
                                                 uint32_t vmask, uint32_t exp16) {
    if constexpr (I < WP) {
        const uint4 bv = make_uint4(vpair<BITS * I>(w0, vmask, exp16), vpair<BITS * (WP + I)>(w0, vmask, exp16),
                                    vpair<BITS * I>(w1, vmask, exp16), vpair<BITS * (WP + I)>(w1, vmask, exp16));
        acc[I] = mfma_f16x32(ahi, bv, acc[I]);
        acc[I] = mfma_f16x32(alo, bv, acc[I]);
        v_mfma_pair_word<WP, BITS, I + 1>(acc, w0, w1, ahi, alo, vmask, exp16);
    }
}

template <int D, int BITS>
__device__ __forceinline__ void v_mfma_pair(floatx4 *acc, const VWords<D, BITS> &va, const VWords<D, BITS> &vb,
                                            uint4 ahi, uint4 alo) {
    using V = VWords<D, BITS>;
    uint32_t vmask, exp16;
    vpair_consts<BITS>(vmask, exp16);
#pragma unroll
    for (int p = 0; p < V::NFULL; ++p)
        v_mfma_pair_word<V::W, BITS, 0>(acc + V::W * p, va.w[p], vb.w[p], ahi, alo, vmask, exp16);
    if constexpr (V::REM > 0)
        v_mfma_pair_word<V::REM, BITS, 0>(acc + V::W * V::NFULL, va.w[V::NFULL], vb.w[V::NFULL], ahi, alo, vmask,
                                          exp16);
}

// element i of a record's metadata area (fp16 or fp32 values)
template <bool MF>
__device__ __forceinline__ float meta_at(const uint8_t *p, int i) {
    if constexpr (MF) return ((const float *)p)[i];
    else return f16_to_f32(((const uint16_t *)p)[i]);
}

// One workgroup per (head, split, sequence x group of 64 queries); wave w
// holds queries 16*(4*qg + w) + 0..15. Lane l = 16*kb + x: as the query
// operand it holds the digits of query x's channels kb*D/4 + 16s + 0..15 of
// step s; as the K operand token x's codes of the same channels; after the
// score product it holds tokens 4*kb..4*kb+3 of query x; in the output
// accumulators queries 4*kb..4*kb+3 at channel 16m + x.
//
// The four waves share every page: each slot of an LDS ring holds one page's
// reference K and V records and the loop's residual K and V records as
// stored (two runs of the slab; only the K code areas transposed, see KSwz),
// filled by direct-to-LDS loads that the waves issue in equal shares. Pages
// go in pairs (the V product takes k = four tokens of each page of a pair, so
// its operand is never duplicated), three pairs ahead. The per-token factors
// of a pair (metadata as f32, times alpha and the softmax scale where they
// apply) are tabulated once per workgroup, each wave one record, one pair
// ahead of their use. One barrier per pair publishes the landed slots and the
// tables and frees the oldest ones. The split's block ids are preloaded into
// LDS. Two waves per SIMD: with three (at most 168 registers) the pair's
// scores, weights and operands spill to scratch, which measured slower.
template <int D, int RB, bool MF, int NI>
__global__ __launch_bounds__(256, 2) void rq_chunk_split_kernel(ChunkArgs a) {
    constexpr int NK = D / 16;                 // k-steps of the score product = column groups of V
    constexpr int PF = partial_floats(D);
    constexpr int MSZ = MF ? 4 : 2;
    constexpr int NST = kChunkStages;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kb = lane >> 4, x = lane & 15;
    const int h = blockIdx.x, split = blockIdx.y;
    const int b = blockIdx.z / a.nqg, qg = blockIdx.z % a.nqg;
    const int H = a.H, C = a.C;
    const int q0 = 16 * (4 * qg + wave);       // first query row of this wave (>= C: loads only)
    int seq = a.seq_lens[b];
    seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
    const int npages = (seq + 15) >> 4;
    const int p0 = split * a.split_pages;
    const int p1 = min(npages, p0 + a.split_pages);
    const int steps = p1 > p0 ? p1 - p0 : 0;

    // LDS: ring of NST stages, one 16-byte padding slot per wave, block ids of the split
    const int stage = a.stage;
    uint8_t *ring = smem;
    const uint32_t junk = lds_addr(smem + NST * stage + 16 * wave);
    int *tbl = (int *)(smem + NST * stage + 64);
    for (int i = threadIdx.x; i < steps; i += 256) {
        int blk = a.block_table[(int64_t)b * a.max_blocks + p0 + i];
        tbl[i] = (blk >= 0 && blk < a.nblk) ? blk : -1;
    }
    __syncthreads();

    // this lane's pieces: instruction j of wave w covers pieces 64*(NI*w + j) + lane
    const int np = stage >> 4, nref = a.ref_rec >> 3;          // 16-byte pieces; of them in the reference run
    using KR = KSwz<D, 4>;
    using KS = KSwz<D, RB ? RB : 2>;
    int doff[NI], live[NI], dst[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int start = 64 * (NI * wave + j);
        live[j] = max(0, min(64, np - start));
        dst[j] = start * 16;
        const int k = start + lane;
        if (k < nref) {
            doff[j] = a.ref_off + 16 * (k < KR::PIECES ? KR::src(k) : k);
        } else {
            const int kk = k - nref;
            doff[j] = a.res_off + 16 * (RB != 0 && kk < KS::PIECES ? KS::src(kk) : kk);
        }
    }
    auto issue = [&](int st, int slot) {
        const int blk = max(__builtin_amdgcn_readfirstlane(tbl[st]), 0);
        const uint8_t *base = a.pool + ((int64_t)blk * H + h) * a.slab;
        const uint32_t l0 = lds_addr(ring + slot * stage);
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            if (live[j] > 0) {
                if (lane < live[j]) dma16(l0 + dst[j], base, (uint32_t)doff[j]);
            } else if (lane == 0) {
                dma16(junk, base, 0u);
            }
        }
    };

    // this lane's query (operand role): row q0 + x
    const int qi = q0 + x;
    const bool qok = qi < C;
    const int64_t qrow = ((int64_t)b * C + (qok ? qi : 0)) * H + h;
    // the digits of q and of q' in registers
    constexpr int NS = chunk_steps8<D>();
    uint4 qd[NS][3], qe[RB ? NS : 1][3];
    const uint8_t *qr = a.qrec + qrow * chunk_qrec_bytes(D);
    {
        const uint4 *dq = (const uint4 *)(qr + 16) + kb, *dr = dq + NS * 12;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int l = 0; l < 3; ++l) {
                qd[s][l] = qok ? dq[(s * 3 + l) * 4] : make_uint4(0u, 0u, 0u, 0u);
                if constexpr (RB != 0) qe[s][l] = qok ? dr[(s * 3 + l) * 4] : make_uint4(0u, 0u, 0u, 0u);
            }
    }
    // sums of the fixed-point q and q', 2^-e twice (the softmax scale is in
    // the token tables); a missing query: zero sums, scale 1 (no NaN from -inf * 0)
    const float4 hd = qok ? *(const float4 *)qr : make_float4(0.f, 0.f, 1.f, 1.f);
    // the query registers are complete before the ring's loads are counted
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int l = 0; l < 3; ++l) {
            __asm__ volatile("" ::"v"(qd[s][l].x), "v"(qd[s][l].y), "v"(qd[s][l].z), "v"(qd[s][l].w));
            if constexpr (RB != 0)
                __asm__ volatile("" ::"v"(qe[s][l].x), "v"(qe[s][l].y), "v"(qe[s][l].z), "v"(qe[s][l].w));
        }
    __asm__ volatile("" ::"v"(hd.x), "v"(hd.y), "v"(hd.z), "v"(hd.w));
    wait_vmcnt<0>();

    float m = kFloorC, lsum = 0.f, zr = 0.f, zs = 0.f;
    floatx4 vacc_r[NK], vacc_s[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        vacc_r[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        vacc_s[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // pages in pairs: pair i = split pages 2i, 2i+1 in slots 2i % NST,
    // (2i+1) % NST, issued three pairs ahead; a split with an odd page count
    // loads its last page twice (the copy is masked)
    const int npair = (steps + 1) >> 1;
    auto issue_pair = [&](int i) {
        issue(2 * i, (2 * i) % NST);
        issue(min(2 * i + 1, steps - 1), (2 * i + 1) % NST);
    };

    // token tables of pair i in buffer i % 2: [page][entry][token] with the
    // entries (tau = softmax scale * log2 e; alpha from the residual record)
    //   0, 1: tau alpha s, tau alpha z of the reference K record
    //   2, 3: tau s, tau z of the residual K record
    //   4, 5: alpha s, alpha z of the reference V record
    //   6, 7: s, z of the residual V record
    // wave w fills the entries of record w, lanes 0..31 = (page, token)
    float *tabs = (float *)(smem + chunk_tab_offset(NST * stage, a.split_pages));
    const int code_ref = 16 * D / 2, code_res = 16 * D * (RB ? RB : 2) / 8;
    auto make_tables = [&](int i) {
        if (lane < 32 && (RB != 0 || (wave & 1) == 0)) {
            const int j = lane >> 4, t = lane & 15;
            const uint8_t *S = ring + ((2 * i + j) % NST) * stage;
            const bool vrec = wave >= 2, resrec = (wave & 1) != 0;
            const uint8_t *rec = resrec ? S + 2 * a.ref_rec + (vrec ? a.res_rec : 0) : S + (vrec ? a.ref_rec : 0);
            const uint8_t *meta = rec + (resrec ? code_res : code_ref);
            float f = vrec ? 1.f : a.score_scale;
            if (RB != 0 && !resrec) f *= meta_at<MF>(S + 2 * a.ref_rec + (vrec ? a.res_rec : 0) + code_res + a.meta_bytes, t);
            float *T = tabs + ((i & 1) * 2 + j) * 128 + 2 * wave * 16 + t;
            T[0] = f * meta_at<MF>(meta, 2 * t);
            T[16] = f * meta_at<MF>(meta, 2 * t + 1);
        }
    };

    // scores (log2 domain, in units of 2^-e; masked: -inf) of the four
    // tokens 4kb..4kb+3 of split page c held by this lane, for query x
    auto page_scores = [&](int c, const uint8_t *S, const float *T, float *sc) {
        const uint8_t *rk = S, *sk = S + 2 * a.ref_rec;
        KChunk<D, 4> kr;
        load_k<D, 4>(kr, rk + KR::off(x, kb));
        intx4 dr[3] = {}, ds[3] = {};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint4 kk = chunk_kbytes<D, 4>(kr.w, s);
#pragma unroll
            for (int l = 0; l < 3; ++l) dr[l] = mfma_i8(kk, qd[s][l], dr[l]);
        }
        if constexpr (RB != 0) {
            KChunk<D, RB> ks;
            load_k<D, RB>(ks, sk + KS::off(x, kb));
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 kk = chunk_kbytes<D, RB>(ks.w, s);
#pragma unroll
                for (int l = 0; l < 3; ++l) ds[l] = mfma_i8(kk, qe[s][l], ds[l]);
            }
        }
        const float *tt = T + 4 * kb;
        const float4 e0 = *(const float4 *)tt, e1 = *(const float4 *)(tt + 16);
        float4 e2 = {0.f, 0.f, 0.f, 0.f}, e3 = e2;
        if constexpr (RB != 0) {
            e2 = *(const float4 *)(tt + 32);
            e3 = *(const float4 *)(tt + 48);
        }
        const float a0[4] = {e0.x, e0.y, e0.z, e0.w}, a1[4] = {e1.x, e1.y, e1.z, e1.w};
        const float a2[4] = {e2.x, e2.y, e2.z, e2.w}, a3[4] = {e3.x, e3.y, e3.z, e3.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // sum q c = 65536 S2 + 256 S1 + S0 (256 S2 + S1 is exact in int32)
            const float sr = fmaf((float)((dr[2][r] << 8) + dr[1][r]), 256.f, (float)dr[0][r]);
            float u = fmaf(a0[r], sr, a1[r] * hd.x);
            if constexpr (RB != 0) {
                const float ss = fmaf((float)((ds[2][r] << 8) + ds[1][r]), 256.f, (float)ds[0][r]);
                u = fmaf(a2[r], ss, fmaf(a3[r], hd.y, u));
            }
            sc[r] = u;
        }
        // masks only on a page not wholly valid for the wave's 16 queries
        const int blk = __builtin_amdgcn_readfirstlane(tbl[min(c, steps - 1)]);
        const bool whole = c < steps && blk >= 0 && 16 * (p0 + c) + 16 <= seq && q0 + 16 <= C;
        if (!whole) {
            const bool ok = (c < steps) & (blk >= 0) & qok;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * (p0 + c) + 4 * kb + r;
                sc[r] = (ok & (t < seq)) ? sc[r] : kNegInf;
            }
        }
    };
    // the weights of the four tokens: reference (p alpha s_v, p alpha z_v)
    // and residual (p s_v, p z_v); zero for masked tokens
    auto page_weights = [&](const float *T, const float *pr, float *wr, float *ws, float &zsr, float &zss) {
        const float *tt = T + 64 + 4 * kb;
        const float4 e4 = *(const float4 *)tt, e5 = *(const float4 *)(tt + 16);
        float4 e6 = {0.f, 0.f, 0.f, 0.f}, e7 = e6;
        if constexpr (RB != 0) {
            e6 = *(const float4 *)(tt + 32);
            e7 = *(const float4 *)(tt + 48);
        }
        const float a4[4] = {e4.x, e4.y, e4.z, e4.w}, a5[4] = {e5.x, e5.y, e5.z, e5.w};
        const float a6[4] = {e6.x, e6.y, e6.z, e6.w}, a7[4] = {e7.x, e7.y, e7.z, e7.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            wr[r] = pr[r] * a4[r];
            zsr = fmaf(pr[r], a5[r], zsr);
            if constexpr (RB != 0) {
                ws[r] = pr[r] * a6[r];
                zss = fmaf(pr[r], a7[r], zss);
            }
        }
    };

    for (int i = 0; i < 3; ++i)
        if (i < npair) issue_pair(i);
    if (npair > 0) {
        wait_steps<2, 2 * NI>(min(2, npair - 1));          // this wave's loads of pair 0
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        make_tables(0);
    }
    // pairs in blocks of kChunkFold/2; the zero terms are folded into the
    // accumulators after each block (see below)
    for (int cb = 0; cb < npair; cb += kChunkFold / 2) {
        const int ce = min(npair, cb + kChunkFold / 2);
        for (int ci = cb; ci < ce; ++ci) {
            // this wave's loads of pair ci+1 have landed (of pair ci, the last) ...
            wait_steps<1, 2 * NI>(min(ci + 2, npair - 1) - min(ci + 1, npair - 1));
            // ... and every other wave's; the tables of pair ci are complete;
            // all waves are done with pair ci-1 and its tables
            __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (ci + 3 < npair) issue_pair(ci + 3);
            if (ci + 1 < npair) make_tables(ci + 1);
            if (q0 >= C) continue;                 // a wave without queries only loads and tabulates
            const uint8_t *S0 = ring + ((2 * ci) % NST) * stage, *S1 = ring + ((2 * ci + 1) % NST) * stage;
            const float *T0 = tabs + (ci & 1) * 256, *T1 = T0 + 128;
            float sc0[4], sc1[4];
            // The two workgroups on a CU run out of phase: each SIMD holds one
            // wave of each. Raising this wave's priority over its matrix-core
            // sections (the score products here, the V products below) lets
            // the other wave's VALU work fill the cycles around them
            // (measured: residual 1.300 -> 1.278 ms, reference 0.672 -> 0.624 ms).
            __builtin_amdgcn_s_setprio(1);
            page_scores(2 * ci, S0, T0, sc0);
            page_scores(2 * ci + 1, S1, T1, sc1);
            __builtin_amdgcn_s_setprio(0);
            // ---- online softmax per query (lanes x, x+16, x+32, x+48 share query x)
            float pmax = vmax2(vmax3(sc0[0], sc0[1], sc0[2]),
                               vmax3(sc0[3], sc1[0], vmax3(sc1[1], sc1[2], sc1[3])));
            pmax = max_lanes4(pmax) * hd.z;        // log2 units
            if (__any(pmax > m + kThreshC)) {
                const float mn = fmaxf(m, pmax);
                const float f = fast_exp2(m - mn);
                lsum *= f; zr *= f; zs *= f;
                m = mn;
                // accumulator rows are queries 4kb + v: their factors come from lanes 4kb + v
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float fv = __shfl(f, 4 * kb + v, 64);
#pragma unroll
                    for (int i = 0; i < NK; ++i) {
                        vacc_r[i][v] *= fv;
                        if constexpr (RB != 0) vacc_s[i][v] *= fv;
                    }
                }
            }
            // weights exp2(score - m), the scale 2^-e joined with the subtraction
            float p0w[4], p1w[4];
            const float nm = -m;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p0w[r] = fast_exp2(fmaf(sc0[r], hd.z, nm));
                p1w[r] = fast_exp2(fmaf(sc1[r], hd.z, nm));
                lsum += p0w[r] + p1w[r];
            }
            float wr0[4], ws0[4], wr1[4], ws1[4];
            float zsum_r = 0.f, zsum_s = 0.f;
            page_weights(T0, p0w, wr0, ws0, zsum_r, zsum_s);
            page_weights(T1, p1w, wr1, ws1, zsum_r, zsum_s);
            // ---- out += P x V: k = this lane group's four tokens of page
            // 2ci, then the same four of page 2ci+1; hi and lo weights in two
            // products against the same V operand
            __builtin_amdgcn_s_setprio(1);
            // the compiler's interleaving strategy for the V products and
            // their operand expansion (measured: 1.260 -> 1.236 ms)
            __builtin_amdgcn_iglp_opt(0);
            const uint8_t *rv0 = S0 + a.ref_rec, *rv1 = S1 + a.ref_rec;
            uint2 h0, l0, h1, l1;
            float u0, u1;
            split4(wr0, h0, l0, u0);
            split4(wr1, h1, l1, u1);
            zr += zsum_r - 16.f * (u0 + u1);
            {
                VWords<D, 4> va, vb;
                load_v<D, 4>(va, rv0, lane);
                load_v<D, 4>(vb, rv1, lane);
                v_mfma_pair<D, 4>(vacc_r, va, vb, make_uint4(h0.x, h0.y, h1.x, h1.y), make_uint4(l0.x, l0.y, l1.x, l1.y));
            }
            if constexpr (RB != 0) {
                const uint8_t *sv0 = S0 + 2 * a.ref_rec + a.res_rec, *sv1 = S1 + 2 * a.ref_rec + a.res_rec;
                split4(ws0, h0, l0, u0);
                split4(ws1, h1, l1, u1);
                zs += zsum_s - 16.f * (u0 + u1);
                VWords<D, RB> va, vb;
                load_v<D, RB>(va, sv0, lane);
                load_v<D, RB>(vb, sv1, lane);
                v_mfma_pair<D, RB>(vacc_s, va, vb, make_uint4(h0.x, h0.y, h1.x, h1.y), make_uint4(l0.x, l0.y, l1.x, l1.y));
            }
            __builtin_amdgcn_s_setprio(0);
        }
        // After every block of kChunkFold pages the zero terms go into the
        // accumulators. The products carry the offset 16 of every code, so the
        // running sums grow (16 + c) s / |value| times faster than the result
        // and their fp32 rounding would otherwise build up over the whole split
        // (thousands of tokens); folded, it builds up over one block only.
        if (q0 < C) {
            const float zq = sum_lanes4(zr);
            const float zsq = RB != 0 ? sum_lanes4(zs) : 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float zrv = __shfl(zq, 4 * kb + v, 64);       // accumulator row v: query 4kb + v
                const float zsv = RB != 0 ? __shfl(zsq, 4 * kb + v, 64) : 0.f;
#pragma unroll
                for (int i = 0; i < NK; ++i) {
                    vacc_r[i][v] += zrv;
                    if constexpr (RB != 0) vacc_s[i][v] += zsv;
                }
            }
            zr = 0.f;
            zs = 0.f;
        }
    }

    // ---- partials: sums over the four token lanes of each query
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    zr += __shfl_xor(zr, 16, 64);
    zr += __shfl_xor(zr, 32, 64);
    zs += __shfl_xor(zs, 16, 64);
    zs += __shfl_xor(zs, 32, 64);
    if (kb == 0 && qok) {
        float *o = a.partials + (qrow * a.nsplit + split) * PF;
        o[0] = m == kFloorC ? kNegInf : m;
        o[1] = lsum;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int qv = 4 * kb + v;                  // query of accumulator row v
        const float zrv = __shfl(zr, qv, 64), zsv = __shfl(zs, qv, 64);
        const int qiv = q0 + qv;
        if (qiv < C) {
            float *o = a.partials + ((((int64_t)b * C + qiv) * H + h) * a.nsplit + split) * PF;
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                o[2 + 16 * i + x] = vacc_r[i][v] + zrv;
                if constexpr (RB != 0) o[2 + D + 16 * i + x] = vacc_s[i][v] + zsv;
            }
        }
    }
}

// --------------------------------------------------------------- combine
struct ChunkCombineArgs {
    const float *partials;          // [R][H][nsplit][2 + 2D]
    int nsplit, split_pages, max_blocks;
    const int32_t *seq_lens;
    const uint16_t *q, *chunk_k, *chunk_v;   // [B][C][H][D] bf16 (chunk K/V may be NULL)
    const float *rot;
    float *out;                     // [B][C][H][D]
    int R, C, H, res;
    float score_scale;
};

// bf16 RNE of a float, and the bf16 hi/lo pair of a weight (hi = RNE(w),
// lo = RNE(w - hi): relative error <= 2^-16)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ floatx4 mfma_bf16x32(uint4 a, uint4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// One workgroup per (head, sequence, 16 consecutive queries of the chunk);
// wave r holds query i = 16t + r. The chunk's own causal part runs on the
// bf16 matrix cores (v_mfma_f32_16x16x32_bf16: lane l supplies row l%16 of A
// and column l%16 of B for its eight k values 8(l/16)..8(l/16)+7, and
// receives rows 4(l/16)..4(l/16)+3 of column l%16):
//   scores S = Q K^T of the tile's 16 queries and its tokens j < 16t + 16,
//     one 16-token tile per wave (exact bf16 products, fp32 sums);
//   after each wave has merged its row's split partials and turned its
//     scores into weights, O += P V_chunk, one 16-channel tile per wave,
//     with the weights as bf16 hi/lo terms and the V rows as stored.
// At most 64 registers (eight waves per SIMD), so that two workgroups share a
// CU and one's loads overlap the other's work: the rotation's R_V operands are
// therefore loaded in the rotation phase, not held across the merge.
template <int D>
__global__ __launch_bounds__(1024, 8) void rq_chunk_combine_kernel(ChunkCombineArgs a) {
    constexpr int QS = D + 1;
    constexpr int PF = partial_floats(D);
    constexpr int SS = kMaxChunk + 4;              // row stride of the score / weight tile
    __shared__ float A[16 * QS];
    __shared__ float O[16 * QS];
    __shared__ float S[16 * SS];
    const int lane = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int h = blockIdx.x;
    const int H = a.H, C = a.C;
    const int nt = (C + 15) >> 4;
    const int b = blockIdx.y / nt, t = blockIdx.y % nt;
    const int i = 16 * t + r;
    const bool row_ok = i < C;
    const int64_t qrow = ((int64_t)b * C + (row_ok ? i : 0)) * H + h;
    // the tile's chunk tokens (causal: up to its last query) in 16-token tiles
    const int jmax = a.chunk_k ? min(C, 16 * t + 16) : 0;
    const int ntt = (jmax + 15) >> 4;
    if (r < ntt) {
        const int qi = 16 * t + (lane & 15), tj = 16 * r + (lane & 15);
        const uint16_t *qa = a.q + (((int64_t)b * C + min(qi, C - 1)) * H + h) * D + 8 * (lane >> 4);
        const uint16_t *kb = a.chunk_k + (((int64_t)b * C + min(tj, jmax - 1)) * H + h) * D + 8 * (lane >> 4);
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const uint4 av = *(const uint4 *)(qa + 32 * kk), bv = *(const uint4 *)(kb + 32 * kk);
            acc = mfma_bf16x32(av, bv, acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) S[(4 * (lane >> 4) + v) * SS + tj] = acc[v] * a.score_scale;
    }
    __syncthreads();

    const int c0 = lane, c1 = lane + 64;
    float ar0 = 0.f, ar1 = 0.f, as0 = 0.f, as1 = 0.f, inv = 0.f;
    if (row_ok) {
        int seq = a.seq_lens[b];
        seq = seq < 0 ? 0 : (seq > a.max_blocks * 16 ? a.max_blocks * 16 : seq);
        const int npages = (seq + 15) >> 4;
        const int ns = (npages + a.split_pages - 1) / a.split_pages;     // splits with pages
        const float *P = a.partials + qrow * a.nsplit * PF;
        // this row's chunk scores (tokens 0..i), lanes lane + 64k
        const int nj = a.chunk_k ? i + 1 : 0;
        float mloc = kNegInf;
        for (int s = lane; s < ns; s += 64) mloc = fmaxf(mloc, P[(int64_t)s * PF]);
        float sj[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = lane + 64 * k;
            sj[k] = j < nj ? S[r * SS + j] : kNegInf;
            mloc = fmaxf(mloc, sj[k]);
        }
        const float M = wave_max(mloc);
        float lloc = 0.f;
        float pj[4] = {0.f, 0.f, 0.f, 0.f};
        if (M != kNegInf) {
            const int k0 = min(c0, D - 1), k1 = min(c1, D - 1);
            // four partials per round with their loads in flight together
            // (indices past the last partial re-read it with weight 0)
            for (int s0 = 0; s0 < ns; s0 += 4) {
                float e[4], l[4], v0[4], v1[4], w0[4], w1[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float *ps = P + (int64_t)min(s0 + u, ns - 1) * PF;
                    const float mu = ps[0];
                    e[u] = (s0 + u >= ns || mu == kNegInf) ? 0.f : fast_exp2(mu - M);
                    l[u] = ps[1];
                    v0[u] = ps[2 + k0];
                    v1[u] = ps[2 + k1];
                    w0[u] = a.res ? ps[2 + D + k0] : 0.f;
                    w1[u] = a.res ? ps[2 + D + k1] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (lane == 0) lloc = fmaf(e[u], l[u], lloc);
                    ar0 = fmaf(e[u], v0[u], ar0);
                    ar1 = fmaf(e[u], v1[u], ar1);
                    as0 = fmaf(e[u], w0[u], as0);
                    as1 = fmaf(e[u], w1[u], as1);
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                pj[k] = sj[k] == kNegInf ? 0.f : fast_exp2(sj[k] - M);
                lloc += pj[k];
            }
            const float lsum = wave_sum(lloc);
            inv = lsum > 0.f ? 1.0f / lsum : 0.f;
        }
        as0 *= inv; as1 *= inv;
#pragma unroll
        for (int k = 0; k < 4; ++k) pj[k] *= inv;        // normalized weights of the chunk tokens
        // this row's weights for the P V product (0 past token i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (lane + 64 * k < 16 * ntt) S[r * SS + lane + 64 * k] = pj[k];
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (lane + 64 * k < 16 * ntt) S[r * SS + lane + 64 * k] = 0.f;
    }
    // merged partials, normalized: O (reference sums; the chunk's part is
    // added below) and A (residual sums)
    if (c0 < D) { O[r * QS + c0] = ar0 * inv; A[r * QS + c0] = as0; }
    if (c1 < D) { O[r * QS + c1] = ar1 * inv; A[r * QS + c1] = as1; }
    const bool rot_wave = a.res && r < D / 16;
    const int n = r * 16 + (lane & 15);
    __syncthreads();

    // O += P V_chunk: wave r computes channels 16r..16r+15 over the tile's
    // tokens, 32 per product (tokens past the tile's last one weigh 0)
    if (ntt > 0 && r < D / 16) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t *vcol = a.chunk_v + ((int64_t)b * C * H + h) * D + n;
        for (int j0 = 0; j0 < 16 * ntt; j0 += 32) {
            const int jb = j0 + 8 * (lane >> 4);
            uint32_t hi[4], lo[4], vv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ja = jb + 2 * e, jc = ja + 1;
                const float wa = ja < 16 * ntt ? S[(lane & 15) * SS + ja] : 0.f;
                const float wc = jc < 16 * ntt ? S[(lane & 15) * SS + jc] : 0.f;
                const uint32_t ha = bf16_rne(wa), hc = bf16_rne(wc);
                const uint32_t la = bf16_rne(wa - __uint_as_float(ha << 16)), lc = bf16_rne(wc - __uint_as_float(hc << 16));
                hi[e] = ha | (hc << 16);
                lo[e] = la | (lc << 16);
                const uint32_t va = ja < jmax ? vcol[(int64_t)ja * H * D] : 0u;
                const uint32_t vc = jc < jmax ? vcol[(int64_t)jc * H * D] : 0u;
                vv[e] = va | (vc << 16);
            }
            const uint4 bv = make_uint4(vv[0], vv[1], vv[2], vv[3]);
            acc = mfma_bf16x32(make_uint4(hi[0], hi[1], hi[2], hi[3]), bv, acc);
            acc = mfma_bf16x32(make_uint4(lo[0], lo[1], lo[2], lo[3]), bv, acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) O[(4 * (lane >> 4) + v) * QS + n] += acc[v];
    }
    __syncthreads();

    if (a.res) {
        // out = O + A * R_V (R_V^T applied to each row's residual sum), as in decode
        if (rot_wave) {
            // this lane's R_V operands (rows 4kk + lane/16 of column n)
            float rv[D / 4];
            const float *RV = a.rot + ((int64_t)h * 2 + 1) * D * D + (int64_t)(lane >> 4) * D + n;
#pragma unroll
            for (int kk = 0; kk < D / 4; ++kk) rv[kk] = RV[(int64_t)4 * kk * D];
            floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 4; ++kk) {
                const int k = 4 * kk + (lane >> 4);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(lane & 15) * QS + k], rv[kk], c, 0, 0, 0);
            }
            for (int v = 0; v < 4; ++v) {
                const int rr = 4 * (lane >> 4) + v;
                const int ir = 16 * t + rr;
                if (ir < C) a.out[(((int64_t)b * C + ir) * H + h) * D + n] = c[v] + O[rr * QS + n];
            }
        }
    } else if (row_ok) {
        if (c0 < D) a.out[qrow * D + c0] = O[r * QS + c0];
        if (c1 < D) a.out[qrow * D + c1] = O[r * QS + c1];
    }
}

template <int D, int RB>
hipError_t launch_chunk_split(const ChunkArgs &s, bool mf, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    // ring, padding slots, block ids of one split, token tables (<= 64 KB:
    // stage <= 4736 bytes for the supported layouts, split_pages <= 1024)
    const size_t lds = (size_t)chunk_tab_offset(kChunkStages * s.stage, s.split_pages) + kChunkTabBytes;
    if (lds > 65536) return hipErrorInvalidValue;
    const bool two = s.stage > 4096;           // two direct-to-LDS instructions per wave and page
    if (mf) {
        if (two) hipExtLaunchKernelGGL((rq_chunk_split_kernel<D, RB, true, 2>), grid, dim3(256), (uint32_t)lds, st, e0, e1, 0, s);
        else hipExtLaunchKernelGGL((rq_chunk_split_kernel<D, RB, true, 1>), grid, dim3(256), (uint32_t)lds, st, e0, e1, 0, s);
    } else {
        if (two) hipExtLaunchKernelGGL((rq_chunk_split_kernel<D, RB, false, 2>), grid, dim3(256), (uint32_t)lds, st, e0, e1, 0, s);
        else hipExtLaunchKernelGGL((rq_chunk_split_kernel<D, RB, false, 1>), grid, dim3(256), (uint32_t)lds, st, e0, e1, 0, s);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_chunk_d(const ChunkCall &c) {
    const Geom &g = *c.g;
    const int R = c.B * c.C;
    const int ref = g.L - 1;
    const bool res = c.loop != ref;
    const int rb = res ? g.bits[c.loop] : 0;

    ChunkPrepArgs pa;
    pa.q = (const uint16_t *)c.q; pa.rot = c.rot; pa.qrec = c.qrec; pa.R = R; pa.H = g.H; pa.res = rb;
    const int tiles = (R + 15) / 16;
    hipLaunchKernelGGL((rq_chunk_qprep_kernel<D>), dim3(g.H, tiles), dim3(1024), 0, c.stream, pa);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    ChunkArgs s;
    s.pool = c.pool; s.slab = g.slab; s.H = g.H; s.nblk = g.nblk;
    s.ref_off = (int)g.loop_off[ref]; s.ref_rec = g.rec[ref];
    s.res_off = (int)g.loop_off[c.loop]; s.res_rec = g.rec[c.loop];
    s.meta_bytes = g.meta_bytes;
    s.block_table = c.block_table; s.max_blocks = c.max_blocks; s.seq_lens = c.seq_lens;
    s.q = (const uint16_t *)c.q; s.qrec = c.qrec; s.partials = c.partials;
    s.C = c.C; s.nqg = (c.C + 63) / 64; s.nsplit = c.nsplit; s.split_pages = c.split_pages;
    s.score_scale = c.softmax_scale * kLog2eC;
    s.stage = 2 * g.rec[ref] + (res ? 2 * g.rec[c.loop] : 0);
    if (s.stage > 8192 || c.split_pages > kChunkMaxSplit) return hipErrorInvalidValue;
    const bool mf = g.meta == RQ_DTYPE_F32;
    dim3 grid(g.H, c.nsplit, c.B * s.nqg);
    if (rb == 0) err = launch_chunk_split<D, 0>(s, mf, grid, c.stream, c.ev_begin, c.ev_end);
    else if (rb == 2) err = launch_chunk_split<D, 2>(s, mf, grid, c.stream, c.ev_begin, c.ev_end);
    else err = launch_chunk_split<D, 4>(s, mf, grid, c.stream, c.ev_begin, c.ev_end);
    if (err != hipSuccess) return err;

    ChunkCombineArgs ca;
    ca.partials = c.partials; ca.nsplit = c.nsplit; ca.split_pages = c.split_pages; ca.max_blocks = c.max_blocks;
    ca.seq_lens = c.seq_lens; ca.q = (const uint16_t *)c.q;
    ca.chunk_k = (const uint16_t *)c.chunk_k; ca.chunk_v = (const uint16_t *)c.chunk_v;
    ca.rot = c.rot; ca.out = c.out; ca.R = R; ca.C = c.C; ca.H = g.H; ca.res = res ? 1 : 0;
    ca.score_scale = s.score_scale;
    hipLaunchKernelGGL((rq_chunk_combine_kernel<D>), dim3(g.H, c.B * ((c.C + 15) / 16)), dim3(1024), 0, c.stream, ca);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk(const ChunkCall &c) {
    if (c.B <= 0 || c.C <= 0) return hipSuccess;
    switch (c.g->D) {
        case 64: return launch_chunk_d<64>(c);
        case 96: return launch_chunk_d<96>(c);
        case 128: return launch_chunk_d<128>(c);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rq
