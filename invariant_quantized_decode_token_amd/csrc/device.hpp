// Device-side building blocks shared by the gfx950 kernels of libiqd.
//
// Floating point: every kernel is compiled with -ffp-contract=off, no fast
// math and no denormal flushing, so each C++ float operator below is one
// IEEE-754 binary32 operation rounded to nearest even.  Integer sums are
// exact (the K bound keeps |sum| < 2^31), so their order is free.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqd {

constexpr int kWave = 64;

// Native 4 x int32 vector (16 bytes): the unit of every weight and
// activation load.
typedef int32_t v4i __attribute__((ext_vector_type(4)));

// binary32 -> bfloat16 bits, round to nearest even.  NaN stays NaN (quiet,
// sign kept); overflow carries into the exponent and gives +-Inf; no flush.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// IEEE binary16 bits -> binary32 (exact widening via the hardware convert).
__device__ __forceinline__ float fp16_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return static_cast<float>(v);
}

// The canonical W8A8 epilogue: bf16( fl( fl(fl32(acc) * s_a) * s_w ) ).
// Two separate multiplies (no fused multiply-add: -ffp-contract=off).
__device__ __forceinline__ uint16_t w8a8_epilogue(int32_t acc, float s_a, float s_w) {
    float a = static_cast<float>(acc);   // v_cvt_f32_i32, round to nearest even
    float t = a * s_a;
    float y = t * s_w;
    return bf16_rne(y);
}

// Four int8 x int8 products summed into an int32 accumulator.
__device__ __forceinline__ int32_t dot4(int32_t a, int32_t b, int32_t c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

__device__ __forceinline__ int32_t dot16(const v4i &a, const v4i &b, int32_t c) {
    c = dot4(a.x, b.x, c);
    c = dot4(a.y, b.y, c);
    c = dot4(a.z, b.z, c);
    c = dot4(a.w, b.w, c);
    return c;
}

// 16-byte streaming load of weights that are read exactly once.
__device__ __forceinline__ v4i load_stream16(const int8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

__device__ __forceinline__ v4i load16(const int8_t *p) { return *reinterpret_cast<const v4i *>(p); }

__device__ __forceinline__ v4i zero16() { return v4i{0, 0, 0, 0}; }

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// --- cross-lane exchange with a compile-time lane mask ------------------------
// xor_lane<M>(v) returns v from lane (lane ^ M).  Chosen per mask for gfx950:
// DPP quad permutes for 1 and 2, DPP row rotate for 8, two bank-masked DPP
// row shifts for 4, ds_swizzle (no memory access) for 16, ds_bpermute for 32.
// Every lane of the wave must be active.
__device__ __forceinline__ int32_t as_i32(int32_t v) { return v; }
__device__ __forceinline__ int32_t as_i32(float v) { return __float_as_int(v); }
template <typename T>
__device__ __forceinline__ T from_i32(int32_t v);
template <>
__device__ __forceinline__ int32_t from_i32<int32_t>(int32_t v) { return v; }
template <>
__device__ __forceinline__ float from_i32<float>(int32_t v) { return __int_as_float(v); }

template <int M>
__device__ __forceinline__ int32_t xor_lane_i32(int32_t v) {
    if constexpr (M == 1) {
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        int32_t t = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);  // row_shl:4 -> banks 0, 2
        return __builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false);      // row_shr:4 -> banks 1, 3
    } else if constexpr (M == 8) {
        return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (M == 16) {
        return __builtin_amdgcn_ds_swizzle(v, (16 << 10) | 0x1F);  // bit mode: xor 16 within 32 lanes
    } else {
        static_assert(M == 32, "lane mask");
        return __builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, v);
    }
}

template <int M, typename T>
__device__ __forceinline__ T xor_lane(T v) {
    return from_i32<T>(xor_lane_i32<M>(as_i32(v)));
}

// Branch-free value select (no select of addresses, so arrays stay in registers).
__device__ __forceinline__ int32_t sel(bool c, int32_t x, int32_t y) {
    const int32_t m = -static_cast<int32_t>(c);
    return y ^ ((x ^ y) & m);
}
__device__ __forceinline__ float sel(bool c, float x, float y) {
    return __int_as_float(sel(c, __float_as_int(x), __float_as_int(y)));
}

// Argmax key of a bf16 logit h at index idx: the value mapped to an
// order-preserving integer in the high word (-0 and +0 both map to 0x8000),
// the complemented index in the low word.  The largest key of a row is its
// maximum at the smallest index, and a maximum of keys is order-free.  Every
// key of a real logit is >= 2^32, so 0 never wins.
__device__ __forceinline__ uint64_t argmax_key(uint32_t h, uint32_t idx) {
    const int32_t o = (h & 0x8000u) ? -static_cast<int32_t>(h & 0x7FFFu) : static_cast<int32_t>(h & 0x7FFFu);
    const uint32_t hi = static_cast<uint32_t>(o + 0x8000);
    return (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }
constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

// One reduce-scatter step over lane mask M on the first C values of v: the
// lane whose mask bit is 0 keeps the lower half of the values, the other the
// upper half, and each adds its partner's copy of the half it keeps (results
// in v[0, C/2)).  `add(mine, partner's)`; for float sums the single rounded
// add is commutative, so both partners compute the same bits.
template <int M, int C, typename T, typename Add>
__device__ __forceinline__ void rs_step(T *v, int lane, Add add) {
    const bool hi = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
        const T lo_v = v[i];
        const T hi_v = v[i + C / 2];
        const T send = sel(hi, lo_v, hi_v);
        const T keep = sel(hi, hi_v, lo_v);
        v[i] = add(keep, xor_lane<M>(send));
    }
}

// Reduce-scatter over lane masks M, 2M, ... on C values until one is left,
// then all-reduce the last value over the remaining masks up to 32.  After
// it, lane l holds the full sum of value index
//     idx = sum_j bit(lane, log2(M) + j) << (log2(C) - 1 - j)
// over the lanes it was combined with.
template <int M, int C, typename T, typename Add>
__device__ __forceinline__ T rs_chain(T *v, int lane, Add add) {
    if constexpr (M > 32) {
        return v[0];
    } else if constexpr (C >= 2) {
        rs_step<M, C>(v, lane, add);
        return rs_chain<M * 2, C / 2>(v, lane, add);
    } else {
        v[0] = add(v[0], xor_lane<M>(v[0]));
        return rs_chain<M * 2, 1>(v, lane, add);
    }
}

// Reduce-scatter of NP (a power of two, <= 64) values across all 64 lanes.
template <int NP, typename T, typename Add>
__device__ __forceinline__ T reduce_scatter(T (&v)[NP], int lane, Add add) {
    return rs_chain<1, NP>(v, lane, add);
}

// Value index a lane holds after reduce_scatter<NP> (masks from 1 upwards).
template <int NP>
__device__ __forceinline__ int reduce_scatter_index(int lane) {
    constexpr int LG = ilog2(NP);
    int idx = 0;
#pragma unroll
    for (int j = 0; j < LG; ++j) idx |= ((lane >> j) & 1) << (LG - 1 - j);
    return idx;
}

}  // namespace iqd
