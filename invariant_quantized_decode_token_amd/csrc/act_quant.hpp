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
// 127), 0 when s == 0.  The quotient is formed as y = fl(x * fl(1 / s)) first:
// |y - fl(x / s)| <= |x / s| (3 u + u^2) < 2.3e-5 (u = 2^-24, |x / s| <= 127
// (1 + u)), so rint(y) == rint(fl(x / s)) unless y lies within 2^-14 of a
// half-integer.  A vector with such a value (or any vector when 1 / s
// overflows) is redone with the correctly rounded division.  |x / s| never
// exceeds 127 (1 + u) for finite x, so the clamp only matters for the slow
// path's non-finite inputs.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack4(int32_t a, int32_t b, int32_t c, int32_t d) {
    return (static_cast<uint32_t>(a) & 0xFFu) | ((static_cast<uint32_t>(b) & 0xFFu) << 8) |
           ((static_cast<uint32_t>(c) & 0xFFu) << 16) | (static_cast<uint32_t>(d) << 24);
}

__device__ __forceinline__ uint2 act_quant8(const v4i &v, float s, float rcp, bool fast_ok) {
    if (s == 0.0f) return make_uint2(0u, 0u);
    float e[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e[2 * i] = bf16_lo(static_cast<uint32_t>(v[i]));
        e[2 * i + 1] = bf16_hi(static_cast<uint32_t>(v[i]));
    }
    int32_t q[8];
    bool near = !fast_ok;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float y = e[i] * rcp;
        near |= __builtin_fabsf(__builtin_amdgcn_fractf(y) - 0.5f) <= 0x1p-14f;
        q[i] = static_cast<int32_t>(__builtin_rintf(y));
    }
    if (__builtin_expect(near, 0)) {  // one branch per vector
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = static_cast<int32_t>(fminf(fmaxf(__builtin_rintf(e[i] / s), -127.0f), 127.0f));
    }
    return make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
}

__device__ __forceinline__ float act_amax8(const v4i &v) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, __builtin_fabsf(bf16_lo(static_cast<uint32_t>(v[i]))));
        m = fmaxf(m, __builtin_fabsf(bf16_hi(static_cast<uint32_t>(v[i]))));
    }
    return m;
}

}  // namespace iqd
