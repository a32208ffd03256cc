// W8A8 mat-vec for decode and speculative verify (1 <= b <= 16), gfx950.
//
//   y[t, n] = bf16( fl( fl( fl32(acc[t, n]) * s_a[t] ) * s_w[n] ) ),
//   acc[t, n] = sum_k q[t, k] * w[n, k]   (int32, exact)
//
// Sources: "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
// Quantization Scales and the Limits of Tolerance-Based Conformance"
// (Abstract, Fig. 1: exact, order-free int32 accumulation under a
// no-overflow bound; Table II: the epilogue is the negation of faults
// F1-F5).  "why speculative decoding changed my output", section "the mat-vec
// kernel": the integer dot products are exact, the float order is what a
// token-count-dependent launch geometry breaks.
//
// Because the K reduction is exact integer arithmetic, the decomposition of
// K over lanes, waves and workgroups is chosen for speed alone (and may
// depend on b); the epilogue runs once per output on the fully reduced
// int32, so no result depends on b or on the launch shape.
//
// Mapping (64-lane waves):
//  * a wave owns RS consecutive weight rows and a contiguous range of 16-byte
//    K vectors; lane l reads vector v0 + l + 64 i of each row with a 16-byte
//    non-temporal buffer load (1 KiB contiguous per row per wave
//    instruction).  Row starts live in scalar buffer resources whose range
//    ends at the wave's K range, token starts in scalar offsets, so the loads
//    need no per-lane address arithmetic and lanes past the range read zeros;
//  * the wave walks its work as a flat sequence of chunks (U vectors per lane
//    per row) and keeps the next chunk's weights in flight while it computes
//    the current one (a ring of D register buffers, D - 1 chunks in flight);
//  * each 16-byte weight vector meets the same K vector of all B tokens
//    (read through L1/L2) through four
//    v_dot4_i32_i8 per token, tokens in the outer loop so that only one
//    activation vector per chunk step is live;
//  * RS*B int32 accumulators per lane are reduce-scattered across the wave,
//    then the `ks` waves that split the same rows along K add their partials
//    through LDS; the owning lane applies the epilogue;
//  * a workgroup may be persistent over several row groups.
#include "device.hpp"
#include "kernels.hpp"
#include "w8a8_matvec_impl.hpp"

namespace iqd {
namespace {

// Launch configurations, chosen by a sweep on MI355X (rows per wave, chunk
// size, waves per workgroup, ring depth, K split, LDS staging, grid) over the
// Qwen3-8B decode shapes; the numerics are the same for every configuration.
//  * small b: activations read through L1/L2, one workgroup per row group;
//  * b >= 5 on large matrices: activations staged once per workgroup in LDS
//    (16-wave workgroups, persistent over row groups), which keeps the
//    per-lane activation reads off the vector-memory path.
struct MvConfig {
    int rs, u, nw, d, ks;
    bool lds;
};

constexpr int64_t kLdsMinWeightBytes = 32ll << 20;

template <int B, int RS, int U, int NW, int D, bool KEYS>
hipError_t launch_cfg(const MvArgs &a, hipStream_t st, int ks, bool lds, int *grid_out) {
    const int kvec = a.K / 16;
    if (ks > kvec / a.split) ks = 1;
    return mv_launch<B, RS, U, NW, D, 0, KEYS>(a, st, device_info().cus, ks, /*grid*/ 0, lds, grid_out);
}

template <int B, bool KEYS = false>
hipError_t launch_b(const MvArgs &a, hipStream_t st, int *grid_out = nullptr) {
    const int64_t wbytes = static_cast<int64_t>(a.N) * a.K;
    // Past 8 tokens the LDS-staged configuration pays only while the
    // activations leave room for a second workgroup (12288 -> 4096 at b = 10,
    // 120 KiB of activations: 21.1 us staged against 15.7 read through L1);
    // up to 8 tokens its 16-wave workgroups pay up to 128 KiB (Qwen3-14B down,
    // 17408 -> 5120 at b = 7: 25.0 against 28.8 us).
    const int64_t act_bytes = static_cast<int64_t>(B) * a.K / a.split;
    const bool big = wbytes >= kLdsMinWeightBytes && act_bytes <= (B <= 8 ? 128 : 64) * 1024;
    if constexpr (B <= 4) {
        // K split over all four waves of a row group past K = 4096 (b = 1:
        // 12288 -> 4096 10.3 against 11.0 us with two; 5120 -> 5120 7.1
        // against 7.3; 5120 -> 7168 8.6 against 9.0)
        return launch_cfg<B, 4, 2, 4, 3, KEYS>(a, st, a.K > 4096 ? 4 : 2, false, grid_out);
    } else if constexpr (B <= 8) {
        if (big) return launch_cfg<B, 2, 1, 16, 2, KEYS>(a, st, 2, true, grid_out);
        return launch_cfg<B, 4, 1, 4, 3, KEYS>(a, st, 2, false, grid_out);
    } else {
        if (big) return launch_cfg<B, 4, 1, 8, 2, KEYS>(a, st, 1, true, grid_out);
        return launch_cfg<B, 4, 2, 4, 4, KEYS>(a, st, 2, false, grid_out);
    }
}

// The matrix-core kernel (w8a8_mfvec.hip) costs about the same for any
// b <= 16, while the dot4 kernel's work grows with b: on MI355X the dot4
// kernel wins at b = 1 and, on matrices of at most 384 tiles of 16 rows with
// K <= 8192 (the Qwen3-8B o and qkv), at b = 2; the matrix-core kernel wins
// everywhere else (the Qwen3-14B qkv, 448 tiles, at b = 2: 9.6 against
// 10.7 us).
bool use_mfvec(int b, int N, int K) {
    if (b == 1) return false;
    if (b == 2 && (N + 15) / 16 <= 384 && K <= 8192) return false;
    return w8a8_mfvec_fits(b, N, K);
}

}  // namespace

hipError_t launch_w8a8_matvec(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w,
                              int b, int N, int K, uint16_t *y, int split, int32_t *part,
                              hipStream_t st) {
    if (split == 1 && use_mfvec(b, N, K))
        return launch_w8a8_mfvec(q, s_a, w, s_w, b, N, K, y, st);
    MvArgs a{};
    a.q = q;
    a.s_a = s_a;
    a.w = w;
    a.s_w = s_w;
    a.N = N;
    a.K = K;
    a.y = y;
    a.part = part;
    a.split = split;
    switch (b) {
        case 1: return launch_b<1>(a, st);
        case 2: return launch_b<2>(a, st);
        case 3: return launch_b<3>(a, st);
        case 4: return launch_b<4>(a, st);
        case 5: return launch_b<5>(a, st);
        case 6: return launch_b<6>(a, st);
        case 7: return launch_b<7>(a, st);
        case 8: return launch_b<8>(a, st);
        case 9: return launch_b<9>(a, st);
        case 10: return launch_b<10>(a, st);
        case 11: return launch_b<11>(a, st);
        case 12: return launch_b<12>(a, st);
        case 13: return launch_b<13>(a, st);
        case 14: return launch_b<14>(a, st);
        case 15: return launch_b<15>(a, st);
        case 16: return launch_b<16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

// Quantization fused in, one token: every workgroup quantizes the bf16 row
// into its LDS activations while its first weight chunks are in flight, on a
// grid of two workgroups per CU that walks the row groups (so that each
// workgroup quantizes once).  Measured against the fused matrix-core kernel
// on the Qwen3 layers it wins only for rows longer than 8192 (and loses at
// b = 2 everywhere), so the entry point takes it there alone.
namespace {

template <int B, int XB>
hipError_t launch_fused_xb(const MvArgs &a, hipStream_t st) {
    const int cus = device_info().cus;
    return mv_launch<B, 4, 2, 4, 3, XB>(a, st, cus, a.K > 4096 ? 4 : 2, 2 * cus, true);
}

template <int B>
hipError_t launch_fused_b(const MvArgs &a, hipStream_t st) {
    const int per_thread = (B * (a.K / 8) + 4 * kWave - 1) / (4 * kWave);  // 16-byte bf16 vectors per thread
    if (per_thread <= 2) return launch_fused_xb<B, 2>(a, st);
    if (per_thread <= 4) return launch_fused_xb<B, 4>(a, st);
    if (per_thread <= 8) return launch_fused_xb<B, 8>(a, st);
    return launch_fused_xb<B, 16>(a, st);
}

}  // namespace

bool w8a8_matvec_fused_ok(int b, int N, int K) {
    (void)N;
    return b == 1 && K / 8 <= 16 * 4 * kWave;
}

hipError_t launch_w8a8_matvec_fused(const uint16_t *x, const int8_t *w, const float *s_w, int b, int N, int K,
                                    uint16_t *y, int8_t *q_out, float *s_out, hipStream_t st) {
    if (!w8a8_matvec_fused_ok(b, N, K)) return hipErrorInvalidValue;
    MvArgs a{};
    a.x = x;
    a.q_out = q_out;
    a.s_out = s_out;
    a.w = w;
    a.s_w = s_w;
    a.N = N;
    a.K = K;
    a.y = y;
    a.split = 1;
    return launch_fused_b<1>(a, st);
}

hipError_t launch_w8a8_matvec_keys(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N,
                                   int K, uint16_t *y, uint64_t *keys, int keys_cap, int *grid, hipStream_t st) {
    if (keys_cap < 1) return hipErrorInvalidValue;
    if (use_mfvec(b, N, K)) return launch_w8a8_mfvec_keys(q, s_a, w, s_w, b, N, K, y, keys, keys_cap, grid, st);
    MvArgs a{};
    a.q = q;
    a.s_a = s_a;
    a.w = w;
    a.s_w = s_w;
    a.N = N;
    a.K = K;
    a.y = y;
    a.keys = keys;
    a.keys_cap = keys_cap;
    a.split = 1;
    switch (b) {
        case 1: return launch_b<1, true>(a, st, grid);
        case 2: return launch_b<2, true>(a, st, grid);
        case 3: return launch_b<3, true>(a, st, grid);
        case 4: return launch_b<4, true>(a, st, grid);
        case 5: return launch_b<5, true>(a, st, grid);
        case 6: return launch_b<6, true>(a, st, grid);
        case 7: return launch_b<7, true>(a, st, grid);
        case 8: return launch_b<8, true>(a, st, grid);
        case 9: return launch_b<9, true>(a, st, grid);
        case 10: return launch_b<10, true>(a, st, grid);
        case 11: return launch_b<11, true>(a, st, grid);
        case 12: return launch_b<12, true>(a, st, grid);
        case 13: return launch_b<13, true>(a, st, grid);
        case 14: return launch_b<14, true>(a, st, grid);
        case 15: return launch_b<15, true>(a, st, grid);
        case 16: return launch_b<16, true>(a, st, grid);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_w8a8_combine(const int32_t *part, const float *s_a, const float *s_w, int b, int N,
                               int split, uint16_t *y, hipStream_t st) {
    const int64_t total = static_cast<int64_t>(b) * N;
    const unsigned grid = static_cast<unsigned>((total + 255) / 256);
    hipLaunchKernelGGL(k_w8a8_combine, dim3(grid), dim3(256), 0, st, part, s_a, s_w, b, N, split, y);
    return hipGetLastError();
}

}  // namespace iqd
