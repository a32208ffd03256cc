// Per-token activation quantization inside the fused linear kernels
// (internal to libiqd): the same result as the quantize kernel,
//   s = fl(amax / 127),  q = clamp(rint_half_even(fl(x / s)), -127, 127),
//   s == 0 -> q = 0,
// with the division replaced by a multiply by fl(1 / s) wherever that
// provably gives the same integer.
// Source: "why speculative decoding changed my output", section "the mat-vec
// kernel" (int8 activations with a float scale); the absmax / 127 scale and
// the rounding rule are the plain reading stated in iqd.h.
#pragma once

#include "device.hpp"

namespace iqd {

// Per-token quantization of 8 bf16 values (one 16-byte vector), the same
// result as the quantize kernel: q = clamp(rint_half_even(fl(x / s)), -127,
// 127), 0 when s == 0.
//
// Fast path, per value, with r = fl(1 / s) and M = 1.5 * 2^23 (in [2^23,
// 2^24) floats are spaced by 1, so adding M rounds to an integer):
//   z = fma(x, r, M)      = M + rint_half_even(x * r)   (exact product, one rounding)
//   d = fma(x, r, M - z)  = x * r - n rounded once     (n = z - M, exact)
// and n is the low byte of z's bit pattern (two's complement, |n| <= 127).
// Error: |x * r - x / s| <= |x / s| 2^-24 and |fl(x / s) - x / s| <= 2^-17
// (|x / s| <= 127 (1 + 2^-24)), together below 1.6e-5.  So when |d| < 0.5 -
// 2^-14 (d is within 2^-25 relative of x * r - n), x * r and fl(x / s) lie
// more than 4.5e-5 from the same side of every half-integer and rint(fl(x /
// s)) == n.  A vector with a value that fails the test (or any vector when
// 1 / s overflows) is redone with the correctly rounded division; the test
// fails for values within 2^-14 of a half-integer, about 1.2e-4 of them when
// the fractions are spread evenly.  The clamp only matters for the slow
// path's non-finite inputs.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Low bytes of four dwords, in order, as one dword (v_perm_b32: selector
// bytes 0-3 pick bytes of the second operand, 4-7 of the first, 12 gives 0).
__device__ __forceinline__ uint32_t pack_lo4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

__device__ __forceinline__ uint2 act_quant8(const v4i &v, float s, float rcp, bool fast_ok) {
    if (s == 0.0f) return make_uint2(0u, 0u);
    constexpr float kMagic = 0x1.8p23f;
    float e[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e[2 * i] = bf16_lo(static_cast<uint32_t>(v[i]));
        e[2 * i + 1] = bf16_hi(static_cast<uint32_t>(v[i]));
    }
    uint32_t z[8];
    bool near = !fast_ok;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float zi = __builtin_fmaf(e[i], rcp, kMagic);
        const float d = __builtin_fmaf(e[i], rcp, kMagic - zi);
        near |= !(__builtin_fabsf(d) < 0.5f - 0x1p-14f);  // NaN (1 / s overflowed) fails too
        z[i] = __float_as_uint(zi);
    }
    if (__builtin_expect(near, 0)) {  // one branch per vector
#pragma unroll
        for (int i = 0; i < 8; ++i)
            z[i] = static_cast<uint32_t>(static_cast<int32_t>(fminf(fmaxf(__builtin_rintf(e[i] / s), -127.0f), 127.0f)));
    }
    return make_uint2(pack_lo4(z[0], z[1], z[2], z[3]), pack_lo4(z[4], z[5], z[6], z[7]));
}

// Largest |x| of 8 bf16 values.  With the sign bit cleared, bf16 bit
// patterns of finite values order as their magnitudes, so the maximum is
// taken on the 16-bit halves in pairs (v_pk_max_u16) and widened once.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t amax_pk8(const v4i &v) {
    u16x2_t m = __builtin_bit_cast(u16x2_t, static_cast<uint32_t>(v[0]) & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 4; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, static_cast<uint32_t>(v[i]) & 0x7FFF7FFFu));
    return __builtin_bit_cast(uint32_t, m);
}

__device__ __forceinline__ float act_amax8(const v4i &v) {
    const uint32_t p = amax_pk8(v);
    return fmaxf(__uint_as_float(p << 16), __uint_as_float(p & 0xFFFF0000u));
}

}  // namespace iqd
