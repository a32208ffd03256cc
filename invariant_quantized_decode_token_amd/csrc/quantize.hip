// Activation quantization kernels (gfx950).
//
// Per group (a token row, or an aligned 32-element block):
//   amax = max |x|, s = fl(amax / 127), q = clamp(rint_half_even(fl(x / s)), -127, 127),
//   s == 0 -> q = 0.
// Source: "why speculative decoding changed my output", section "the mat-vec
// kernel" (int8 activations, blocks of 32, float scales); the absmax / 127
// scale and the rounding rule are the plain reading stated in iqd.h.
// The division is IEEE correctly rounded (hipcc's default for '/', no fast
// math); rintf is v_rndne_f32 (ties to even); max and fabs are exact, so
// the reduction order of amax is free.
#include "act_quant.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

struct Bf16x8 {
    uint32_t w[4];
};

__device__ __forceinline__ float lo16(uint32_t v) { return bf16_to_f32(v & 0xFFFFu); }
__device__ __forceinline__ float hi16(uint32_t v) { return bf16_to_f32(v >> 16); }

__device__ __forceinline__ float amax8(const Bf16x8 &x) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fabsf(lo16(x.w[i])));
        m = fmaxf(m, fabsf(hi16(x.w[i])));
    }
    return m;
}

__device__ __forceinline__ int32_t q1(float x, float s) {
    float r = __builtin_rintf(x / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int32_t>(r) & 0xFF;
}

// 8 bf16 -> 8 int8 packed in two dwords (byte i = element i).
__device__ __forceinline__ int2 quant8(const Bf16x8 &x, float s) {
    if (s == 0.0f) return make_int2(0, 0);
    int32_t b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b[2 * i] = q1(lo16(x.w[i]), s);
        b[2 * i + 1] = q1(hi16(x.w[i]), s);
    }
    int2 r;
    r.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    r.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    return r;
}

__device__ __forceinline__ Bf16x8 load8(const uint16_t *p) {
    int4 v = *reinterpret_cast<const int4 *>(p);
    Bf16x8 r;
    r.w[0] = static_cast<uint32_t>(v.x);
    r.w[1] = static_cast<uint32_t>(v.y);
    r.w[2] = static_cast<uint32_t>(v.z);
    r.w[3] = static_cast<uint32_t>(v.w);
    return r;
}

constexpr int kQuantThreads = 256;

template <int NT>
__device__ __forceinline__ float block_amax(float m) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) m = fmaxf(m, shfl_xor(m, mask));
    __shared__ float wmax[NT / kWave];
    if (lane_id() == 0) wmax[threadIdx.x / kWave] = m;
    __syncthreads();
    float amax = wmax[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) amax = fmaxf(amax, wmax[i]);
    return amax;
}

// One workgroup of NT threads per token row, the row held in registers (VPT
// 16-byte vectors per thread): one read of x, then the quantized write.  The
// quotient is formed as x * fl(1 / s), redone with the correctly rounded
// division only for a vector with a value near a half-integer (act_quant8:
// the same integers as fl(x / s), proved there); against a division per
// value this took the quantize + mat-vec chain at 12288 -> 4096 from 14.9
// and 15.6 to 14.2 and 14.9 us at b = 5 and 8 (measured on MI355X).
template <int NT, int VPT>
__global__ __launch_bounds__(NT) void k_quant_token_reg(const uint16_t *__restrict__ x, int K,
                                                        int8_t *__restrict__ q, float *__restrict__ s_out) {
    const int t = blockIdx.x;
    const uint16_t *xr = x + static_cast<int64_t>(t) * K;
    int8_t *qr = q + static_cast<int64_t>(t) * K;
    const int nvec = K / 8;
    v4i xv[VPT];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = threadIdx.x + i * NT;
        xv[i] = v4i{0, 0, 0, 0};
        if (v < nvec) xv[i] = *reinterpret_cast<const v4i *>(xr + 8 * v);
        m = fmaxf(m, act_amax8(xv[i]));
    }
    const float s = block_amax<NT>(m) / 127.0f;
    if (threadIdx.x == 0) s_out[t] = s;
    const float rc = 1.0f / s;
    const bool fast_ok = __builtin_isfinite(rc);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = threadIdx.x + i * NT;
        if (v < nvec) *reinterpret_cast<uint2 *>(qr + 8 * v) = act_quant8(xv[i], s, rc, fast_ok);
    }
}

// Rows too long for registers: two passes over x.
__global__ __launch_bounds__(kQuantThreads) void k_quant_token(const uint16_t *__restrict__ x, int K,
                                                               int8_t *__restrict__ q,
                                                               float *__restrict__ s_out) {
    const int t = blockIdx.x;
    const uint16_t *xr = x + static_cast<int64_t>(t) * K;
    int8_t *qr = q + static_cast<int64_t>(t) * K;
    const int nvec = K / 8;
    float m = 0.0f;
    for (int v = threadIdx.x; v < nvec; v += kQuantThreads) m = fmaxf(m, amax8(load8(xr + 8 * v)));
    const float s = block_amax<kQuantThreads>(m) / 127.0f;
    if (threadIdx.x == 0) s_out[t] = s;
    for (int v = threadIdx.x; v < nvec; v += kQuantThreads)
        *reinterpret_cast<int2 *>(qr + 8 * v) = quant8(load8(xr + 8 * v), s);
}

// Four lanes per 32-element block, 8 elements per lane.
__global__ __launch_bounds__(kQuantThreads) void k_quant_block32(const uint16_t *__restrict__ x,
                                                                 int64_t nvec,
                                                                 int8_t *__restrict__ q,
                                                                 float *__restrict__ d) {
    const int64_t v = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x;
    const bool live = v < nvec;  // nvec is a multiple of 4: a block is all live or all dead
    Bf16x8 xv = {};
    if (live) xv = load8(x + 8 * v);
    float m = amax8(xv);
    m = fmaxf(m, shfl_xor(m, 1));
    m = fmaxf(m, shfl_xor(m, 2));
    const float s = m / 127.0f;
    if (live) {
        *reinterpret_cast<int2 *>(q + 8 * v) = quant8(xv, s);
        if ((v & 3) == 0) d[v / 4] = s;
    }
}

}  // namespace

hipError_t launch_quantize_token(const uint16_t *x, int b, int K, int8_t *q, float *s, hipStream_t st) {
    const int nvec = K / 8;
    if (nvec <= 256)
        hipLaunchKernelGGL((k_quant_token_reg<256, 1>), dim3(b), dim3(256), 0, st, x, K, q, s);
    else if (nvec <= 512)
        hipLaunchKernelGGL((k_quant_token_reg<512, 1>), dim3(b), dim3(512), 0, st, x, K, q, s);
    else if (nvec <= 1024)
        hipLaunchKernelGGL((k_quant_token_reg<1024, 1>), dim3(b), dim3(1024), 0, st, x, K, q, s);
    else if (nvec <= 2048)
        hipLaunchKernelGGL((k_quant_token_reg<1024, 2>), dim3(b), dim3(1024), 0, st, x, K, q, s);
    else if (nvec <= 4096)
        hipLaunchKernelGGL((k_quant_token_reg<1024, 4>), dim3(b), dim3(1024), 0, st, x, K, q, s);
    else if (nvec <= 8192)
        hipLaunchKernelGGL((k_quant_token_reg<1024, 8>), dim3(b), dim3(1024), 0, st, x, K, q, s);
    else
        hipLaunchKernelGGL(k_quant_token, dim3(b), dim3(kQuantThreads), 0, st, x, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quantize_block32(const uint16_t *x, int b, int K, int8_t *q, float *d, hipStream_t st) {
    const int64_t nvec = static_cast<int64_t>(b) * K / 8;
    const int64_t grid = (nvec + kQuantThreads - 1) / kQuantThreads;
    hipLaunchKernelGGL(k_quant_block32, dim3(static_cast<unsigned>(grid)), dim3(kQuantThreads), 0, st, x,
                       nvec, q, d);
    return hipGetLastError();
}

}  // namespace iqd
