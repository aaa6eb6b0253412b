// Device helpers for the gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------ dtype access
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// Element i of a [.. D] row whose dtype is bf16 (IS_F32 = false) or fp32.
template <bool IS_F32>
__device__ __forceinline__ float load_kv(const void *base, int64_t i) {
    if constexpr (IS_F32) return ((const float *)base)[i];
    else return bf16_to_f32(((const uint16_t *)base)[i]);
}

// Round a float64 to IEEE binary16, nearest-even, directly from the double
// (a float64 -> float32 -> float16 chain can round twice).
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    int e = (int)((u >> 52) & 0x7FF);
    uint64_t m = u & 0xFFFFFFFFFFFFFull;
    if (e == 0x7FF) return (uint16_t)(sign | 0x7C00u | (m ? 0x200u : 0u));
    if (e == 0) return (uint16_t)sign;                 // |x| < 2^-1022
    int E = e - 1023;
    if (E >= 16) return (uint16_t)(sign | 0x7C00u);    // |x| >= 2^16
    uint64_t sig = m | (1ull << 52);
    int Q = (E < -14 ? -14 : E) - 10;                  // exponent of one fp16 quantum
    int shift = 52 + Q - E;                            // >= 42
    if (shift >= 64) return (uint16_t)sign;            // below half the smallest subnormal
    uint64_t k = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (k & 1))) k++;
    uint32_t bits = (E < -14) ? (uint32_t)k                               // subnormal (1024 = min normal)
                              : (uint32_t)(((E + 15) << 10) + (int)(k - 1024));  // carry moves the exponent
    if (bits >= 0x7C00u) bits = 0x7C00u;
    return (uint16_t)(sign | bits);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t b) {
    return (double)__builtin_bit_cast(_Float16, b);
}

// --------------------------------------------------------- cross-lane ops
// DPP quad permutations: xor 1 and xor 2 inside each group of 4 lanes.
__device__ __forceinline__ float dpp_quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Sum over groups of LPT consecutive lanes (LPT in {1, 2, 4}); every lane of
// the group gets the sum.
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPT >= 2) v += dpp_quad_xor1(v);
    if constexpr (LPT >= 4) v += dpp_quad_xor2(v);
    return v;
}

// Butterfly partners of a whole-wave reduction without LDS: quad xor 1 and
// xor 2 and row rotations by 4 and 8 (DPP) leave the row's reduction in each
// of its 16 lanes; the gfx950 row swap (v_permlane16_swap) then pairs rows
// 0-1 and 2-3, the half swap (v_permlane32_swap) the two halves. A bpermute
// shuffle per step would cost an LDS round trip and its address arithmetic.
// These read other lanes' registers unconditionally: call them with every
// lane of the wave active (all call sites are wave-uniform).
__device__ __forceinline__ uint32_t dpp_row_ror4(uint32_t v) { return __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_row_ror8(uint32_t v) { return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }

template <int N, typename T, typename Op>
__device__ __forceinline__ void wave_reduce_n(T (&v)[N], Op op) {
    static_assert(sizeof(T) == 4, "32-bit values");
    auto u = [](T x) { return __builtin_bit_cast(uint32_t, x); };
    auto t = [](uint32_t x) { return __builtin_bit_cast(T, x); };
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = op(v[j], t(dpp_xor1(u(v[j]))));
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = op(v[j], t(dpp_xor2(u(v[j]))));
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = op(v[j], t(dpp_row_ror4(u(v[j]))));
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = op(v[j], t(dpp_row_ror8(u(v[j]))));
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const auto a = __builtin_amdgcn_permlane16_swap(u(v[j]), u(v[j]), false, false);
        v[j] = op(t(a[0]), t(a[1]));
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const auto a = __builtin_amdgcn_permlane32_swap(u(v[j]), u(v[j]), false, false);
        v[j] = op(t(a[0]), t(a[1]));
    }
}

// Sums over the lanes that share lane % LPT (LPT in {1, 2, 4}), every such
// lane receiving its sum: the steps of wave_reduce_n from the first partner
// distance LPT on.
template <int LPT, int N>
__device__ __forceinline__ void strided_sum_n(float (&v)[N]) {
    auto u = [](float x) { return __builtin_bit_cast(uint32_t, x); };
    auto f = [](uint32_t x) { return __builtin_bit_cast(float, x); };
    if constexpr (LPT == 1) {
#pragma unroll
        for (int j = 0; j < N; ++j) v[j] += f(dpp_xor1(u(v[j])));
    }
    if constexpr (LPT <= 2) {
#pragma unroll
        for (int j = 0; j < N; ++j) v[j] += f(dpp_xor2(u(v[j])));
    }
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] += f(dpp_row_ror4(u(v[j])));
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] += f(dpp_row_ror8(u(v[j])));
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const auto a = __builtin_amdgcn_permlane16_swap(u(v[j]), u(v[j]), false, false);
        v[j] = f(a[0]) + f(a[1]);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const auto a = __builtin_amdgcn_permlane32_swap(u(v[j]), u(v[j]), false, false);
        v[j] = f(a[0]) + f(a[1]);
    }
}

__device__ __forceinline__ float wave_max(float v) {
    float a[1] = {v};
    wave_reduce_n<1>(a, [](float x, float y) { return fmaxf(x, y); });
    return a[0];
}
__device__ __forceinline__ float wave_sum(float v) {
    float a[1] = {v};
    wave_reduce_n<1>(a, [](float x, float y) { return x + y; });
    return a[0];
}
// The same over N values at once (independent chains, issued together).
template <int N>
__device__ __forceinline__ void wave_max_n(float (&v)[N]) {
    wave_reduce_n<N>(v, [](float x, float y) { return fmaxf(x, y); });
}
template <int N>
__device__ __forceinline__ void wave_sum_n(int (&v)[N]) {
    wave_reduce_n<N>(v, [](int x, int y) { return x + y; });
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------- direct-to-LDS loads and waits
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `ahead` page steps of NI loads each are still in flight
// (ahead is wave-uniform, 0 <= ahead <= K).
template <int K, int NI>
__device__ __forceinline__ void wait_steps(int ahead) {
    if constexpr (K == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= K) wait_vmcnt<K * NI>();
        else wait_steps<K - 1, NI>(ahead);
    }
}

// One direct-to-LDS load of 16 bytes per active lane: lane i's bytes land at
// lds + 16*i (lds is wave-uniform).
// The packed cache is streamed: every byte is read once per call, so the
// loads carry the non-temporal hint (nt), which keeps them from displacing
// reused lines in the caches (measured on MI355X: the decode kernels' page
// records stream about 10% faster than with the default policy).
__device__ __forceinline__ void dma16(uint32_t lds, const uint8_t *base, uint32_t off) {
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma16(uint32_t lds, const uint8_t *src) {
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                     ::"s"(lds), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}


}  // namespace rq
