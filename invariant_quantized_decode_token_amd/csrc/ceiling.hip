// Read-ceiling kernel (gfx950): streams a buffer of device memory with the
// same 16-byte non-temporal loads the mat-vec kernels use and keeps nothing.
// Timed over a launch of the same byte count as a linear layer's weights, it
// gives the practical HBM ceiling for one launch of that size: the dispatch,
// the first memory round trip and the drain that every launch pays, with no
// arithmetic and no output.  It is a measurement helper, not a step of the
// linear layer.
//
// Mapping: block-cyclic over units of NT * U 16-byte vectors, every thread
// issuing its U loads before it consumes any.  Launch shapes from a sweep on
// MI355X over 16-100 MB (256-1024 threads, 2-8 loads in flight per thread,
// 256-4096 workgroups): up to 32 MB many small workgroups (256 threads, 2
// loads, 2048 workgroups) lead; above, 512 threads with 4 loads on 512
// workgroups.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

template <int NT, int U>
__global__ __launch_bounds__(NT) void k_read_ceiling(const v4i *__restrict__ src, int64_t nvec, int32_t *sink) {
    const int64_t G = gridDim.x, g = blockIdx.x, t = threadIdx.x;
    int32_t acc = 0;
    for (int64_t i = g * NT * U + t; i < nvec; i += G * NT * U) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + static_cast<int64_t>(u) * NT;
            v[u] = j < nvec ? __builtin_nontemporal_load(src + j) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    // The loaded values must look used, so the loads are kept; the store
    // happens only for one 32-bit pattern of the xor of all of them, into the
    // caller's 4-byte sink.
    if (acc == 0x5EED1E55 && sink != nullptr) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_ceiling(const void *p, int64_t bytes, int32_t *sink, hipStream_t st) {
    const int64_t nvec = bytes / 16;
    const v4i *src = static_cast<const v4i *>(p);
    if (bytes <= (int64_t{32} << 20)) {
        constexpr int NT = 256, U = 2;
        const int64_t units = (nvec + NT * U - 1) / (NT * U);
        const unsigned grid = static_cast<unsigned>(units < 2048 ? units : 2048);
        hipLaunchKernelGGL((k_read_ceiling<NT, U>), dim3(grid), dim3(NT), 0, st, src, nvec, sink);
    } else {
        constexpr int NT = 512, U = 4;
        const int64_t units = (nvec + NT * U - 1) / (NT * U);
        const unsigned grid = static_cast<unsigned>(units < 512 ? units : 512);
        hipLaunchKernelGGL((k_read_ceiling<NT, U>), dim3(grid), dim3(NT), 0, st, src, nvec, sink);
    }
    return hipGetLastError();
}

}  // namespace iqd
