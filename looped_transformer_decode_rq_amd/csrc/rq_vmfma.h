// V codes on the matrix cores: operand expansion shared by the decode and
// the chunked-prefill kernels.
#pragma once

#include "rq_device.h"

namespace rq {

// ---- V on the matrix cores
//
// The V codes of a page record are stored for the B operand of
// v_mfma_f32_16x16x16_f16 (the record format in rq.h): lane l = 16u + j
// holds, for column group m = 0..D/16-1, the codes of tokens 4u..4u+3 at
// channel 16m + j, packed in 32-bit word planes (plane p of lane l at byte
// 256p + 4l of the code block; the one partial word, D = 96 INT2, is a 16-bit
// unit at 256p + 2l). Inside word p, the code of (group W*p + i, token 4u+v)
// is field 2W(v%2) + W(v/2) + i (W = 8/bits groups per word; W_p for the
// partial word), so one shift and one and-or turn two codes of the same group
// into the fp16 pair (16 + c_v, 16 + c_{v+1}): 16 + c is exact in fp16 as
// 0x4C00 | c << 6.
//
// The per-token weights (p*alpha*s for the reference, p*s for the residual)
// form the A operand: rows 4g + r of group g hold (reference hi, lo, residual
// hi, lo) of the weight split into two fp16 terms (hi = RNE(w), lo = RNE(w -
// hi): relative error <= 2^-22 while w is a normal fp16 number, absolute
// <= 2^-25 below; w <= 256*alpha*s by the lazy softmax rescale), tokens
// along k. Row 4g+r of the product is then sum_t w_t (16 + c_t) for every
// column, lanes 16g..16g+15 receiving the rows of group g. The offset 16 is
// taken out again in the zero term:
// value sum = sum_t w_t (16 + c_t) + sum_t (p alpha z_t - 16 w'_t),
// with w' the weight as the matrix cores see it (chunked prefill) or before
// the split (decode: then 16 (w - w') joins the split's own error c (w - w'),
// unbiased and of the same size).
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp16 pair (16 + c, 16 + c') of the BITS-bit fields at bit SH and at bit
// SH + 16 of w: one shift to bit 6, then (x & mask) | 0x4C004C00. The mask and
// the exponent bits come in as opaque registers (vmask: SGPR, exp16: VGPR),
// so that the compiler selects a single v_and_or_b32 (a VOP3 takes no literal
// and reads at most one scalar operand) and still tracks its hazards.
template <int SH>
__device__ __forceinline__ uint32_t vpair(uint32_t w, uint32_t vmask, uint32_t exp16) {
    uint32_t x = w;
    if constexpr (SH > 6) x = w >> (SH - 6);
    else if constexpr (SH < 6) x = w << (6 - SH);
    return (x & vmask) | exp16;
}

// The opaque operands of vpair for BITS-bit codes.
template <int BITS>
__device__ __forceinline__ void vpair_consts(uint32_t &vmask, uint32_t &exp16) {
    if constexpr (BITS == 4) __asm__("s_mov_b32 %0, 0x03c003c0" : "=s"(vmask));
    else __asm__("s_mov_b32 %0, 0x00c000c0" : "=s"(vmask));
    __asm__("v_mov_b32 %0, 0x4c004c00" : "=v"(exp16));
}

__device__ __forceinline__ floatx4 mfma_f16(uint2 a, uint32_t b0, uint32_t b1, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(halfx4, a),
                                                 __builtin_bit_cast(halfx4, make_uint2(b0, b1)), c, 0, 0, 0);
}

// This lane's words of one page's V code block `vb` (BITS-bit codes, D
// channels): the full 32-bit words, then the 16-bit partial unit (D = 96
// INT2) with its upper fields moved 8 bits up so that every word is read the
// same way
template <int D, int BITS>
struct VWords {
    static constexpr int NM = D / 16, W = 8 / BITS;
    static constexpr int NFULL = NM / W, REM = NM - NFULL * W;
    static constexpr int N = NFULL + (REM > 0 ? 1 : 0);
    uint32_t w[N];
};

template <int D, int BITS>
__device__ __forceinline__ void load_v(VWords<D, BITS> &v, const uint8_t *vb, int lane) {
    using V = VWords<D, BITS>;
#pragma unroll
    for (int p = 0; p < V::NFULL; ++p) v.w[p] = ((const uint32_t *)vb)[64 * p + lane];
    if constexpr (V::REM > 0) {
        const uint32_t u = ((const uint16_t *)(vb + 256 * V::NFULL))[lane];
        v.w[V::NFULL] = u | (u << (16 - 2 * V::REM * BITS));
    }
}

// acc[m] += A x B_m for every column group m of the page
template <int WP, int BITS, int I>
__device__ __forceinline__ void v_mfma_word(floatx4 *acc, uint32_t w, uint2 a, uint32_t vmask, uint32_t exp16) {
    if constexpr (I < WP) {
        const uint32_t b0 = vpair<BITS * I>(w, vmask, exp16);
        const uint32_t b1 = vpair<BITS * (WP + I)>(w, vmask, exp16);
        acc[I] = mfma_f16(a, b0, b1, acc[I]);
        v_mfma_word<WP, BITS, I + 1>(acc, w, a, vmask, exp16);
    }
}

template <int D, int BITS>
__device__ __forceinline__ void v_mfma(floatx4 *acc, const VWords<D, BITS> &v, uint2 a) {
    using V = VWords<D, BITS>;
    uint32_t vmask, exp16;
    vpair_consts<BITS>(vmask, exp16);
#pragma unroll
    for (int p = 0; p < V::NFULL; ++p) v_mfma_word<V::W, BITS, 0>(acc + V::W * p, v.w[p], a, vmask, exp16);
    if constexpr (V::REM > 0)
        v_mfma_word<V::REM, BITS, 0>(acc + V::W * V::NFULL, v.w[V::NFULL], a, vmask, exp16);
}

}  // namespace rq
