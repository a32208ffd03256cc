// Per-row argmax of the LM head's bf16 logits (gfx950): the smallest index
// whose value equals the row maximum, compared as real numbers (+0 == -0).
//
// Source: "My speculative decoder got slower", section "We're nowhere near
// SOL" (a vocab head that returns only the winning token).  The tie rule
// (lowest index) is the reading stated in iqd.h.
//
// Each candidate is a 64-bit key (argmax_key in device.hpp): the bf16 value
// mapped to an order-preserving integer, then the complemented index.  The
// row maximum of the keys is unique and does not depend on the order in
// which keys are compared, so any reduction tree gives it.  Two ways in:
//  * the logits mat-vec (launch_w8a8_matvec_keys) leaves one key per
//    workgroup and token, the largest of the outputs that workgroup wrote, so
//    the logits are not read back;
//  * k_argmax_partial reduces chunks of stored logits to one key each.
// k_argmax_fold then folds a token's keys.  Measured on MI355X with the
// Qwen3-8B head (151936 x 4096): from b = 2 the keyed mat-vec saves 2-4 us
// per call; at b = 1 the mat-vec is fastest with one workgroup per row group
// (19k workgroups), whose keys take longer to fold than the chunked re-read
// of 300 KB of logits (a persistent keyed grid cost 4 us more), so one token
// re-reads its logits.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kFoldThreads = 1024;
constexpr int kFoldPerThread = (kArgKeysMaxGrid + kFoldThreads - 1) / kFoldThreads;  // all key loads in flight at once
constexpr int kArgThreads = 256;
constexpr int kArgPerThread = 16;

template <int NT>
__device__ __forceinline__ uint64_t block_max(uint64_t best) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) best = umax64(best, shfl_xor(best, mask));
    __shared__ uint64_t wbest[NT / kWave];
    if (lane_id() == 0) wbest[threadIdx.x / kWave] = best;
    __syncthreads();
    uint64_t k = wbest[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) k = umax64(k, wbest[i]);
    return k;
}

// Workgroup (c, t) reduces logits [c * C, (c + 1) * C) of token t,
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
    const uint64_t k = block_max<kArgThreads>(best);
    if (threadIdx.x == 0) part[static_cast<int64_t>(t) * nchunk + c] = k;
}

// One workgroup per token folds its nkeys (<= kArgKeysMaxGrid) keys.
__global__ __launch_bounds__(kFoldThreads) void k_argmax_fold(const uint64_t *__restrict__ keys, int nkeys,
                                                              int32_t *__restrict__ out) {
    const int t = blockIdx.x;
    const uint64_t *kt = keys + static_cast<int64_t>(t) * nkeys;
    uint64_t k[kFoldPerThread];
#pragma unroll
    for (int j = 0; j < kFoldPerThread; ++j) {
        const int i = static_cast<int>(threadIdx.x) + j * kFoldThreads;
        k[j] = i < nkeys ? kt[i] : 0;
    }
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kFoldPerThread; ++j) best = umax64(best, k[j]);
    best = block_max<kFoldThreads>(best);
    if (threadIdx.x == 0) out[t] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
}

}  // namespace

int argmax_chunks(int N) { return (N + kArgThreads * kArgPerThread - 1) / (kArgThreads * kArgPerThread); }

hipError_t launch_argmax_partial(const uint16_t *logits, int b, int N, uint64_t *keys, hipStream_t st) {
    const int nchunk = argmax_chunks(N);
    if (nchunk > kArgKeysMaxGrid || b < 1 || b > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_argmax_partial, dim3(nchunk, b), dim3(kArgThreads), 0, st, logits, N, nchunk, keys);
    return hipGetLastError();
}

hipError_t launch_argmax_fold(const uint64_t *keys, int b, int nkeys, int32_t *out, hipStream_t st) {
    if (nkeys < 1 || nkeys > kArgKeysMaxGrid || b < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_argmax_fold, dim3(b), dim3(kFoldThreads), 0, st, keys, nkeys, out);
    return hipGetLastError();
}

}  // namespace iqd
