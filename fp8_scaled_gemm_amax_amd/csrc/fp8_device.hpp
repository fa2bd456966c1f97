// fp8_device.hpp - device-side FP8 encoding, bf16 unpacking and wavefront
// reductions shared by the quantizer and GEMM kernels (gfx950 only).
//
// Encodings ("FP8 Training on MI300X", section on the AMD FP8 dtype difference):
// OCP e4m3 (max 448) / e5m2 (max 57344) and the fnuz variants (e4m3 max 240,
// bias 8; e5m2 bias 16), which have a single zero and NaN = 0x80.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8amax {

enum Fmt : int { kE4M3 = 0, kE5M2 = 1, kE4M3Fnuz = 2, kE5M2Fnuz = 3 };

template <int F> struct FmtTraits;
template <> struct FmtTraits<kE4M3> {
    static constexpr int mbits = 3, bias = 7;
    static constexpr bool fnuz = false;
    static constexpr float fmax = 448.0f;
    static constexpr float min_normal = 0.015625f;      // 2^-6
    static constexpr float sub_magic = 16384.0f;        // 2^(1-bias-mbits+23): ulp = subnormal spacing
};
template <> struct FmtTraits<kE5M2> {
    static constexpr int mbits = 2, bias = 15;
    static constexpr bool fnuz = false;
    static constexpr float fmax = 57344.0f;
    static constexpr float min_normal = 6.103515625e-05f;  // 2^-14
    static constexpr float sub_magic = 128.0f;
};
template <> struct FmtTraits<kE4M3Fnuz> {
    static constexpr int mbits = 3, bias = 8;
    static constexpr bool fnuz = true;
    static constexpr float fmax = 240.0f;
    static constexpr float min_normal = 0.0078125f;     // 2^-7
    static constexpr float sub_magic = 8192.0f;
};
template <> struct FmtTraits<kE5M2Fnuz> {
    static constexpr int mbits = 2, bias = 16;
    static constexpr bool fnuz = true;
    static constexpr float fmax = 57344.0f;
    static constexpr float min_normal = 3.0517578125e-05f; // 2^-15
    static constexpr float sub_magic = 64.0f;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Saturating clamp for inputs known not to be NaN (the compiler folds it into
// v_med3_f32; Inf saturates to +-fmax).
template <int F>
__device__ __forceinline__ float sat(float p) {
    constexpr float m = FmtTraits<F>::fmax;
    return fminf(fmaxf(p, -m), m);
}

// Bit-level saturating round-to-nearest-even encode of one fp32 value; the
// code is in the low 8 bits. Normal range: round the fp32 mantissa to mbits
// (carry into the exponent is the next binade), then rebias the exponent.
// Subnormal range: adding 2^(1-bias-mbits+23) makes the fp32 adder round |p|
// onto the FP8 subnormal grid (its ulp equals the grid spacing).
template <int F>
__device__ __forceinline__ uint32_t encode_sw(float p) {
    using T = FmtTraits<F>;
    constexpr int m = T::mbits;
    const uint32_t u = __float_as_uint(p);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t au = u & 0x7fffffffu;
    const float a = fminf(__uint_as_float(au), T::fmax);
    const uint32_t ab = __float_as_uint(a);
    const uint32_t rnd = ((1u << (22 - m)) - 1u) + ((ab >> (23 - m)) & 1u);
    const uint32_t normal = ((ab + rnd) >> (23 - m)) - ((uint32_t)(127 - T::bias) << m);
    const uint32_t sub = __float_as_uint(a + T::sub_magic) - __float_as_uint(T::sub_magic);
    uint32_t code = (a < T::min_normal) ? sub : normal;
    if (T::fnuz) {
        code = (code == 0u) ? 0u : (code | sign);
        code = (au > 0x7f800000u) ? 0x80u : code;
    } else {
        code |= sign;
        code = (au > 0x7f800000u) ? (sign | 0x7fu) : code;
    }
    return code;
}

// Encode four fp32 values (already multiplied by the scale) into one 32-bit
// word, byte i = code of v_i.
//  - NAN_FREE: the caller knows none of the inputs is NaN (it checked the
//    amax of the data). OCP encodings then use gfx950's conversion
//    instructions (round to nearest even) on clamped inputs; their results
//    equal encode_sw for every non-NaN input. (For NaN the instructions
//    return one canonical code whatever the sign, while the cast defined here
//    keeps the sign: sign|0x7F.)
//  - otherwise, and for fnuz (which the conversion instructions do not
//    produce), the bit-level encoder.
template <int F, bool NAN_FREE>
__device__ __forceinline__ uint32_t encode4(float v0, float v1, float v2, float v3) {
    if constexpr (NAN_FREE && F == kE4M3) {
        int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat<F>(v0), sat<F>(v1), 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(sat<F>(v2), sat<F>(v3), r, true);
        return (uint32_t)r;
    } else if constexpr (NAN_FREE && F == kE5M2) {
        int r = __builtin_amdgcn_cvt_pk_bf8_f32(sat<F>(v0), sat<F>(v1), 0, false);
        r = __builtin_amdgcn_cvt_pk_bf8_f32(sat<F>(v2), sat<F>(v3), r, true);
        return (uint32_t)r;
    } else {
        return encode_sw<F>(v0) | (encode_sw<F>(v1) << 8) | (encode_sw<F>(v2) << 16) | (encode_sw<F>(v3) << 24);
    }
}

// A bf16 magnitude (16 bits) above the Inf pattern is a NaN.
__device__ __forceinline__ bool nan_bits16(uint32_t mag16) { return mag16 > 0x7f80u; }

// Scale from amax for current scaling: fl32(fmax / amax) * 2^-margin, FLT_MAX if
// the quotient overflows, 1 if amax is zero or not finite. The division is the
// correctly rounded fp32 one (the build keeps -fhip-fp32-correctly-rounded-divide-sqrt).
template <int F>
__device__ __forceinline__ float scale_from_amax(float amax, int margin) {
    if (!(amax > 0.0f) || !__builtin_isfinite(amax)) return 1.0f;
    float s = FmtTraits<F>::fmax / amax;
    if (__builtin_isinf(s)) s = 3.402823466e+38f;
    return ldexpf(s, -margin);
}

// Same rule for the delayed update, which keeps the old scale instead of 1:
// returns false when amax is zero or not finite.
template <int F>
__device__ __forceinline__ bool delayed_scale(float amax, int margin, float* s_out) {
    if (!(amax > 0.0f) || !__builtin_isfinite(amax)) return false;
    float s = FmtTraits<F>::fmax / amax;
    if (__builtin_isinf(s)) s = 3.402823466e+38f;
    *s_out = ldexpf(s, -margin);
    return true;
}

// |bf16| magnitude bits of the two halves of a word, packed max. The unsigned
// order of magnitude bits is the numeric order of |x|, with NaN above Inf,
// so a NaN anywhere makes the maximum NaN.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_absmax(uint32_t acc, uint32_t w) {
    u16x2 a = __builtin_bit_cast(u16x2, acc);
    u16x2 b = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}
__device__ __forceinline__ uint32_t pk_fold(uint32_t acc) {
    uint32_t lo = acc & 0xffffu, hi = acc >> 16;
    return lo > hi ? lo : hi;
}

// 16-byte load of streamed input (read once by a single-pass kernel): a
// nontemporal load, so the input does not push out of the caches what the
// next kernel reads (the codes this kernel writes). Measured between GEMMs:
// the rowwise cast at 8192 x 4096 and 14336 x 4096 went from 4.1-4.3 to
// 4.8-5.4 TB/s.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
    const u32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

// Running packed max of the 8 bf16 magnitudes of one 16-byte chunk.
__device__ __forceinline__ uint32_t word_absmax(uint32_t acc, uint4 v) {
    acc = pk_absmax(acc, v.x);
    acc = pk_absmax(acc, v.y);
    acc = pk_absmax(acc, v.z);
    return pk_absmax(acc, v.w);
}

// Wavefront (64 lanes) maximum of an unsigned value; every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// bf16 magnitude bits -> fp32 amax value.
__device__ __forceinline__ float amax_from_bits16(uint32_t b) { return __uint_as_float(b << 16); }

// Relaxed device-scope max on the bits of a non-negative float (NaN above Inf).
__device__ __forceinline__ void atomic_max_bits(float* addr, uint32_t bits32) {
    __hip_atomic_fetch_max(reinterpret_cast<unsigned int*>(addr), bits32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// fp32 -> bf16 round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return __builtin_isnan(f) ? ((u >> 16) | 0x40u) : r;
}

// Eight bf16 values (one 16-byte chunk) times s -> eight codes.
template <int F, bool NAN_FREE>
__device__ __forceinline__ uint2 encode8(uint4 v, float s) {
    uint2 o;
    o.x = encode4<F, NAN_FREE>(bf16_lo(v.x) * s, bf16_hi(v.x) * s, bf16_lo(v.y) * s, bf16_hi(v.y) * s);
    o.y = encode4<F, NAN_FREE>(bf16_lo(v.z) * s, bf16_hi(v.z) * s, bf16_lo(v.w) * s, bf16_hi(v.w) * s);
    return o;
}

}  // namespace fp8amax
