// Per-row argmax over bf16 logits (gfx950): the smallest index whose value
// equals the row maximum, compared as real numbers (+0 == -0).
//
// Source: "My speculative decoder got slower", section "We're nowhere near
// SOL" (a vocab head that returns only the winning token).  The tie rule
// (lowest index) is the reading stated in iqd.h.
//
// Each candidate is packed into a 64-bit key: the bf16 value mapped to an
// order-preserving integer in the high word, the complement of the index in
// the low word.  The row maximum of the keys is unique and does not depend on
// the order in which keys are compared, so the reduction tree is free.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kArgThreads = 1024;

__device__ __forceinline__ uint64_t argmax_key(uint32_t h, uint32_t idx) {
    // -0 and +0 both map to 0; negative values below, positive above.
    const int32_t o = (h & 0x8000u) ? -static_cast<int32_t>(h & 0x7FFFu) : static_cast<int32_t>(h & 0x7FFFu);
    const uint32_t hi = static_cast<uint32_t>(o + 0x8000);
    return (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// One workgroup per token row.
__global__ __launch_bounds__(kArgThreads) void k_argmax_rows(const uint16_t *__restrict__ logits, int N,
                                                             int32_t *__restrict__ out) {
    const int t = blockIdx.x;
    const uint16_t *row = logits + static_cast<int64_t>(t) * N;
    uint64_t best = 0;
    for (int n = threadIdx.x; n < N; n += kArgThreads) best = umax64(best, argmax_key(row[n], static_cast<uint32_t>(n)));
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) best = umax64(best, shfl_xor(best, mask));
    __shared__ uint64_t wbest[kArgThreads / kWave];
    if (lane_id() == 0) wbest[threadIdx.x / kWave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t k = wbest[0];
        for (int i = 1; i < kArgThreads / kWave; ++i) k = umax64(k, wbest[i]);
        out[t] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFu));
    }
}

}  // namespace

hipError_t launch_argmax_rows(const uint16_t *logits, int b, int N, int32_t *out, hipStream_t st) {
    hipLaunchKernelGGL(k_argmax_rows, dim3(b), dim3(kArgThreads), 0, st, logits, N, out);
    return hipGetLastError();
}

}  // namespace iqd
