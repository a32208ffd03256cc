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
// the order in which keys are compared, so the reduction tree is free: many
// workgroups reduce chunks of a row, a second kernel folds the chunk keys.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kArgThreads = 256;
constexpr int kArgPerThread = 16;

__device__ __forceinline__ uint64_t argmax_key(uint32_t h, uint32_t idx) {
    // -0 and +0 both map to 0; negative values below, positive above.  Every
    // key of a real logit is >= 2^32, so 0 never wins.
    const int32_t o = (h & 0x8000u) ? -static_cast<int32_t>(h & 0x7FFFu) : static_cast<int32_t>(h & 0x7FFFu);
    const uint32_t hi = static_cast<uint32_t>(o + 0x8000);
    return (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t block_max(uint64_t best) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) best = umax64(best, shfl_xor(best, mask));
    __shared__ uint64_t wbest[kArgThreads / kWave];
    if (lane_id() == 0) wbest[threadIdx.x / kWave] = best;
    __syncthreads();
    uint64_t k = wbest[0];
#pragma unroll
    for (int i = 1; i < kArgThreads / kWave; ++i) k = umax64(k, wbest[i]);
    return k;
}

// Phase 1: workgroup (c, t) reduces logits [c * C, (c + 1) * C) of token t,
// C = kArgThreads * kArgPerThread, to one key.  All of a thread's loads are
// issued before the first is used.
__global__ __launch_bounds__(kArgThreads) void k_argmax_partial(const uint16_t *__restrict__ logits, int N,
                                                                int nchunk, uint64_t *__restrict__ part) {
    const int c = blockIdx.x, t = blockIdx.y;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(logits + static_cast<int64_t>(t) * N), 0, 2 * N, 0x00020000);
    const int n0 = c * kArgThreads * kArgPerThread + static_cast<int>(threadIdx.x);
    uint32_t h[kArgPerThread];
#pragma unroll
    for (int j = 0; j < kArgPerThread; ++j) h[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * (n0 + j * kArgThreads), 0, 0);
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kArgPerThread; ++j) {
        const int n = n0 + j * kArgThreads;
        if (n < N) best = umax64(best, argmax_key(h[j], static_cast<uint32_t>(n)));
    }
    const uint64_t k = block_max(best);
    if (threadIdx.x == 0) part[static_cast<int64_t>(t) * nchunk + c] = k;
}

// Phase 2: one workgroup per token folds its chunk keys.
__global__ __launch_bounds__(kArgThreads) void k_argmax_final(const uint64_t *__restrict__ part, int nchunk,
                                                              int32_t *__restrict__ out) {
    const int t = blockIdx.x;
    uint64_t best = 0;
    for (int i = static_cast<int>(threadIdx.x); i < nchunk; i += kArgThreads)
        best = umax64(best, part[static_cast<int64_t>(t) * nchunk + i]);
    const uint64_t k = block_max(best);
    if (threadIdx.x == 0) out[t] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFu));
}

}  // namespace

int argmax_chunks(int N) { return (N + kArgThreads * kArgPerThread - 1) / (kArgThreads * kArgPerThread); }

hipError_t launch_argmax_rows(const uint16_t *logits, int b, int N, int32_t *out, uint64_t *part, hipStream_t st) {
    const int nchunk = argmax_chunks(N);
    for (int t0 = 0; t0 < b; t0 += 65535) {  // grid y is at most 65535
        const int bt = b - t0 < 65535 ? b - t0 : 65535;
        hipLaunchKernelGGL(k_argmax_partial, dim3(nchunk, bt), dim3(kArgThreads), 0, st,
                           logits + static_cast<int64_t>(t0) * N, N, nchunk, part + static_cast<int64_t>(t0) * nchunk);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_argmax_final, dim3(b), dim3(kArgThreads), 0, st, part, nchunk, out);
    return hipGetLastError();
}

}  // namespace iqd
