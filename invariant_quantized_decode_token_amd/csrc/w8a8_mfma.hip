// W8A8 linear for b > 16 (prefill).  Interim implementation: token chunks of
// at most 16 through the mat-vec kernel; every token's row is computed
// exactly as in a decode pass, so the bits are the same.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {

hipError_t launch_w8a8_mfma(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N,
                            int K, uint16_t *y, hipStream_t st) {
    for (int t0 = 0; t0 < b; t0 += 16) {
        const int bc = b - t0 < 16 ? b - t0 : 16;
        hipError_t e = launch_w8a8_matvec(q + static_cast<int64_t>(t0) * K, s_a + t0, w, s_w, bc, N, K,
                                          y + static_cast<int64_t>(t0) * N, 1, nullptr, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace iqd
