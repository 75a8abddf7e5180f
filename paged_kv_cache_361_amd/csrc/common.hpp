// common.hpp - storage types, conversions and wavefront helpers shared by the
// gfx950 kernels of libpagedkv.  Device code targets CDNA4 only (64-lane
// wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Storage formats.  Each tag gives the stored element type, its byte size and
// exact widening to fp32 (every f16/bf16/E4M3 value is an fp32 value).
// ---------------------------------------------------------------------------

struct F32 {
    using T = float;
    static constexpr int kBytes = 4;
    __device__ static inline float widen(T x) { return x; }
    __device__ static inline T narrow(float x) { return x; }
};

struct F16 {
    using T = _Float16;
    static constexpr int kBytes = 2;
    __device__ static inline float widen(T x) { return (float)x; }
    __device__ static inline T narrow(float x) { return (_Float16)x; }  // RNE
};

struct BF16 {
    using T = __bf16;
    static constexpr int kBytes = 2;
    __device__ static inline float widen(T x) { return (float)x; }
    __device__ static inline T narrow(float x) { return (__bf16)x; }     // RNE
};

// OCP E4M3: bias 7, no infinity, S.1111.111 = NaN, max 448, min subnormal 2^-9.
struct FP8 {
    using T = uint8_t;
    static constexpr int kBytes = 1;
    // Decode: placing the 7 magnitude bits at fp32 bit 20 yields
    // 2^(e-127) * (1 + m/8) for e >= 1 and the fp32 subnormal m * 2^-129 for
    // e == 0; one multiply by 2^120 rebiases both exactly.
    __device__ static inline float widen(uint32_t c) {
        uint32_t mag = c & 0x7Fu;
        float v = __builtin_bit_cast(float, (mag << 20) | ((c & 0x80u) << 24)) *
                  0x1p120f;
        return mag == 0x7Fu ? __builtin_nanf("") : v;
    }
};

// fp32 -> E4M3, round to nearest even, finite overflow saturates to +-448,
// NaN -> S.1111.111.  Bit-level: the 3 kept fraction bits of a normal value
// are rounded with the usual add-half-minus-one-plus-lsb trick (a carry
// ripples into the exponent); the subnormal range uses the exact fp32
// product by 2^9 and the hardware round-to-nearest-even.
__device__ inline uint32_t e4m3_encode(float y) {
    uint32_t u = __builtin_bit_cast(uint32_t, y);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;            // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;           // >= 448 (and inf)
    if (a >= 0x3C800000u) {                              // >= 2^-6: normal
        uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        return sign | (r - (120u << 3));
    }
    float f = __builtin_bit_cast(float, a) * 512.0f;     // exact
    return sign | (uint32_t)__builtin_rintf(f);          // 0..8
}

// ---------------------------------------------------------------------------
// Wavefront reductions (64 lanes).
// ---------------------------------------------------------------------------

// Sum / max over aligned groups of W consecutive lanes (W a power of two,
// W <= 64); every lane of a group receives the group's result.
template <int W>
__device__ inline float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int W>
__device__ inline float group_max(float x) {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Integer sum over the 64 lanes of a wavefront (every lane gets it).
__device__ inline int group_sum_int(int x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Sum / max across lanes that differ only in bits >= log2(STRIDE): combines
// the 64/STRIDE lanes {l, l+STRIDE, ...} that hold the same column.
// Stride 16 uses the gfx950 lane-swap instructions instead of LDS
// permutes: v_permlane16_swap / v_permlane32_swap of a value with itself
// return, in one order or the other, this lane's value and that of lane
// l ^ 16 (resp. l ^ 32), so the max or the two-term sum of the pair is the
// exchange's result, bit for bit (IEEE addition is commutative).
__device__ inline float swap_sum16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float swap_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float swap_max16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap_max32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int STRIDE>
__device__ inline float strided_sum(float x) {
    if constexpr (STRIDE == 16) return swap_sum32(swap_sum16(x));
#pragma unroll
    for (int o = STRIDE; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int STRIDE>
__device__ inline float strided_max(float x) {
    if constexpr (STRIDE == 16) return swap_max32(swap_max16(x));
#pragma unroll
    for (int o = STRIDE; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// Compact partial entries (the balanced split of multi-query calls, whose
// split streams leave 16 rows per cut).  A row is stored as D f16 values
// x_d = (o_d / l) 2^(15 - e), e the frexp exponent of the row's largest
// |o_d / l| (that value lies in [2^(e-1), 2^e)), so every |x_d| < 2^15
// keeps 11 significant bits whatever the magnitude of V.  e + 127 rides in
// the low 8 bits of the stored l, which moves l by less than 2^-15 of
// itself; the reader takes the sums o_d = x_d 2^(e - 15) l.
__device__ inline int compact_exponent(float amax) {
    const int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
    return e < -127 ? -127 : (e > 128 ? 128 : e);
}
__device__ inline float compact_l(float l, int e) {
    return __uint_as_float((__float_as_uint(l) & ~0xFFu) | (uint32_t)(e + 127));
}
// the factor that turns a stored x_d back into the sum o_d, from the stored l
__device__ inline float compact_scale(float l) {
    return __builtin_ldexpf(l, (int)(__float_as_uint(l) & 0xFFu) - 127 - 15);
}

}  // namespace pkv
