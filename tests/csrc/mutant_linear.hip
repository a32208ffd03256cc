// Test-only candidate kernel for the conformance suite: a plain W8A8 linear
// layer (int32 accumulation, fp32 epilogue, bf16 output) into which one of
// the epilogue faults of "Deterministic LLM Inference Across GPU Kernels:
// Power-of-Two INT8 Quantization Scales and the Limits of Tolerance-Based
// Conformance" (Table II, F1-F5) can be switched.  It stands for a second,
// independently written kernel behind the same interface; it shares no
// source with the library under test or with the CPU oracle.  One thread per
// output, speed is of no concern.
//
// Built with -ffp-contract=off: every product and sum below is one rounded
// binary32 operation.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

enum Fault { kNull = 0, kF1 = 1, kF2 = 2, kF3 = 3, kF4 = 4, kF5 = 5 };

// binary32 -> bfloat16, nearest even; NaN stays a quiet NaN.
__device__ uint16_t bf16_nearest_even(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ float bf16_value(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

__global__ void k_mutant_linear(int fault, const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b,
                                int N, int K, uint16_t *y, int32_t *acc_out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<int64_t>(b) * N) return;
    const int t = static_cast<int>(i / N), n = static_cast<int>(i % N);
    const int8_t *qa = q + static_cast<int64_t>(t) * K;
    const int8_t *wr = w + static_cast<int64_t>(n) * K;
    const float sa = s_a[t], sw = s_w[n];
    uint32_t acc = 0;     // wraps modulo 2^32 like any int32 accumulator
    float folded = 0.0f;  // F5: the column scale folded into a float sum, k in order
    for (int k = 0; k < K; ++k) {
        const int32_t a = qa[k], v = wr[k];
        acc += static_cast<uint32_t>(a * v);
        if (fault == kF5) folded = folded + static_cast<float>(a) * (static_cast<float>(v) * sw);
    }
    const int32_t acc_i = static_cast<int32_t>(acc);
    const float fa = static_cast<float>(acc_i);
    uint16_t out;
    switch (fault) {
    case kF1:  // both scales cast to bfloat16 first
        out = bf16_nearest_even((fa * bf16_value(bf16_nearest_even(sa))) * bf16_value(bf16_nearest_even(sw)));
        break;
    case kF2:  // an extra bfloat16 rounding between the two multiplies
        out = bf16_nearest_even(bf16_value(bf16_nearest_even(fa * sa)) * sw);
        break;
    case kF3:  // acc * (s_a * s_w)
        out = bf16_nearest_even(fa * (sa * sw));
        break;
    case kF4:  // the output cast truncates
        out = static_cast<uint16_t>(__float_as_uint((fa * sa) * sw) >> 16);
        break;
    case kF5:
        out = bf16_nearest_even(folded * sa);
        break;
    default:  // no fault: (acc * s_a) * s_w, nearest even
        out = bf16_nearest_even((fa * sa) * sw);
        break;
    }
    y[i] = out;
    if (acc_out != nullptr) acc_out[i] = acc_i;
}

}  // namespace

// y [b, N] bf16 bits, acc_out [b, N] int32 (may be null).  Returns 0, -1 on
// bad arguments (nothing launched), or the HIP error of the launch.
extern "C" int mutant_linear(int fault, const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b,
                             int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, void *stream) {
    if (fault < kNull || fault > kF5 || b < 1 || N < 1 || K < 1 || b * N > (int64_t{1} << 31) - 256 ||
        K > (int64_t{1} << 30) || q == nullptr || s_a == nullptr || w == nullptr || s_w == nullptr || y == nullptr)
        return -1;
    const int64_t total = b * N;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(k_mutant_linear, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                       static_cast<hipStream_t>(stream), fault, q, s_a, w, s_w, static_cast<int>(b),
                       static_cast<int>(N), static_cast<int>(K), y, acc_out);
    return static_cast<int>(hipGetLastError());
}
