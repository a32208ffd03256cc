// Power-of-two weight-scale requantization (gfx950), offline weight prep.
//
// Source: "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
// Quantization Scales and the Limits of Tolerance-Based Conformance",
// Abstract: move each weight scale to its nearest power of two and re-round
// the weights to it (rewriting scales alone was the artefact).  "Nearest" is
// read as linear distance with a tie at mantissa 1.5 going up:
//   |s| = m * 2^E, m in [1, 2):  s' = sign(s) * (m < 1.5 ? 2^E : 2^(E+1))
//   w'  = clamp(rint_half_even(w * s / s'), -127, 127)
// w * s has at most 8 + 24 significant bits and s' is a power of two, so in
// binary64 the product and the quotient are exact; rint is the only rounding.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kRqThreads = 256;

__device__ __forceinline__ float nearest_pow2(float s) {
    if (s == 0.0f) return 0.0f;
    int e;
    const float f = frexpf(fabsf(s), &e);  // |s| = f * 2^e, f in [0.5, 1)
    const float p = (f < 0.75f) ? ldexpf(1.0f, e - 1) : ldexpf(1.0f, e);
    return s < 0.0f ? -p : p;
}

__global__ __launch_bounds__(kRqThreads) void k_pow2_requant(const int8_t *__restrict__ w,
                                                             const float *__restrict__ s, int K,
                                                             int8_t *__restrict__ w_out,
                                                             float *__restrict__ s_out) {
    const int n = blockIdx.x;
    const float sn = s[n];
    const float sp = nearest_pow2(sn);
    if (threadIdx.x == 0) s_out[n] = sp;
    const int8_t *wr = w + static_cast<int64_t>(n) * K;
    int8_t *wo = w_out + static_cast<int64_t>(n) * K;
    for (int k = threadIdx.x; k < K; k += kRqThreads) {
        int8_t r8 = 0;
        if (sp != 0.0f) {
            double r = __builtin_rint((static_cast<double>(wr[k]) * static_cast<double>(sn)) / static_cast<double>(sp));
            r = r > 127.0 ? 127.0 : (r < -127.0 ? -127.0 : r);
            r8 = static_cast<int8_t>(r);
        }
        wo[k] = r8;
    }
}

}  // namespace

hipError_t launch_pow2_requant(const int8_t *w, const float *s, int N, int K, int8_t *w_out, float *s_out,
                               hipStream_t st) {
    hipLaunchKernelGGL(k_pow2_requant, dim3(N), dim3(kRqThreads), 0, st, w, s, K, w_out, s_out);
    return hipGetLastError();
}

}  // namespace iqd
