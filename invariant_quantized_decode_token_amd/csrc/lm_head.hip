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
// which keys are compared, so any reduction tree gives it.  The logits
// mat-vec (launch_w8a8_matvec_keys) leaves one key per workgroup and token,
// the largest of the outputs that workgroup wrote, so the logits are never
// read back; k_argmax_fold folds a token's keys.  Measured on MI355X with the
// Qwen3-8B head (151936 x 4096), against a chunked re-read of the stored
// logits: 2-4 us faster per call from b = 2, the same at b = 1 (the dot4
// mat-vec's 18,992 workgroups each leave a key; a persistent keyed grid of
// 1024-4096 workgroups cost 4-7 us, its last row groups ending unevenly).
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kFoldThreads = 1024;

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

// One workgroup per token folds its nkeys (<= PT * kFoldThreads) keys; every
// key load is in flight at once (buffer loads: keys past nkeys read zeros,
// which never win).
template <int PT>
__global__ __launch_bounds__(kFoldThreads) void k_argmax_fold(const uint64_t *__restrict__ keys, int nkeys,
                                                              int32_t *__restrict__ out) {
    const int t = blockIdx.x;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint64_t *>(keys + static_cast<int64_t>(t) * nkeys), 0, 8 * nkeys, 0x00020000);
    uint64_t k[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j)
        k[j] = __builtin_bit_cast(
            uint64_t, __builtin_amdgcn_raw_buffer_load_b64(kr, 8 * (static_cast<int>(threadIdx.x) + j * kFoldThreads), 0, 0));
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) best = umax64(best, k[j]);
    best = block_max<kFoldThreads>(best);
    if (threadIdx.x == 0) out[t] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
}

}  // namespace

hipError_t launch_argmax_fold(const uint64_t *keys, int b, int nkeys, int32_t *out, hipStream_t st) {
    static_assert(kArgKeysMaxGrid <= 32 * kFoldThreads, "fold capacity");
    if (nkeys < 1 || nkeys > kArgKeysMaxGrid || b < 1) return hipErrorInvalidValue;
    if (nkeys <= 2 * kFoldThreads)
        hipLaunchKernelGGL((k_argmax_fold<2>), dim3(b), dim3(kFoldThreads), 0, st, keys, nkeys, out);
    else if (nkeys <= 8 * kFoldThreads)
        hipLaunchKernelGGL((k_argmax_fold<8>), dim3(b), dim3(kFoldThreads), 0, st, keys, nkeys, out);
    else
        hipLaunchKernelGGL((k_argmax_fold<32>), dim3(b), dim3(kFoldThreads), 0, st, keys, nkeys, out);
    return hipGetLastError();
}

}  // namespace iqd
