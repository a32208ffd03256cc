// W8A8 linear for wide passes (b > 16, prefill) on the gfx950 int8 matrix
// cores, with the same canonical epilogue as the mat-vec.
//
//   y[t, n] = bf16( fl( fl( fl32(acc[t, n]) * s_a[t] ) * s_w[n] ) ),
//   acc[t, n] = sum_k q[t, k] * w[n, k]   (int32, exact)
//
// Sources: "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
// Quantization Scales and the Limits of Tolerance-Based Conformance"
// (Abstract, Fig. 1: the int32 dot product is exact and order-independent, so
// a tiled matrix-core kernel and a mat-vec agree bit for bit; Table II: the
// epilogue).  "why speculative decoding changed my output", section "the
// mat-vec kernel": past a handful of tokens the stock path moved to a tiled
// matmul with its own add order; here the integer sums make the order moot.
//
// Tiling: a workgroup of 4 waves computes a BM x 128 tile of y (BM tokens,
// 128 weight rows); waves are 2 x 2, each owning a (BM/2) x 64 sub-tile of
// v_mfma_i32_16x16x64_i8 accumulators.  K advances 64 bytes per stage; both
// operand tiles are staged in LDS (rows padded to 80 bytes, so that the 16
// rows a fragment read touches fall on distinct banks), double-buffered, with
// the next stage's global loads in flight during the current stage's MFMAs.
// Operand layout of the instruction (checked on MI355X): lane l holds 16
// bytes of A row (l % 16) and of B column (l % 16) at the same K offset
// 16 * (l / 16); result register i of lane l is D[4 * (l / 16) + i][l % 16].
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kRowPad = 80;  // bytes per staged row
constexpr int kMfThreads = 256;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
    const int nr = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nr, 0x00020000);
}

template <int BM>
__global__ __launch_bounds__(kMfThreads) void k_w8a8_mfma(const int8_t *__restrict__ q, const float *__restrict__ s_a,
                                                          const int8_t *__restrict__ w, const float *__restrict__ s_w,
                                                          int M, int N, int K, uint16_t *__restrict__ y) {
    constexpr int WM = BM / 2;        // wave sub-tile rows (tokens)
    constexpr int FM = WM / 16;       // fragments along M per wave
    constexpr int FN = 64 / 16;       // fragments along N per wave
    constexpr int A_PIECES = BM * (kBK / 16);
    constexpr int B_PIECES = kBN * (kBK / 16);
    constexpr int PIECES = (A_PIECES + B_PIECES) / kMfThreads;
    static_assert((A_PIECES + B_PIECES) % kMfThreads == 0, "whole pieces per thread");
    __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + kBN) * kRowPad];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * kBN;
    const int nst = (K + kBK - 1) / kBK;

    // Loads: every row of A (token) and B (weight) is a K-long byte row; the
    // resources end at the matrix ends (rows past M or N read zeros) and a
    // piece whose K offset is past K is redirected out of range as well.
    const __amdgpu_buffer_rsrc_t ra = rsrc(q, static_cast<int64_t>(M) * K);
    const __amdgpu_buffer_rsrc_t rb = rsrc(w, static_cast<int64_t>(N) * K);
    int piece_row[PIECES], piece_chunk[PIECES];
    bool piece_is_a[PIECES];
#pragma unroll
    for (int p = 0; p < PIECES; ++p) {
        const int id = tid + p * kMfThreads;
        piece_is_a[p] = id < A_PIECES;
        const int j = piece_is_a[p] ? id : id - A_PIECES;
        piece_row[p] = j >> 2;
        piece_chunk[p] = j & 3;
    }
    auto gload = [&](int st, v4i(&regs)[PIECES]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const int k = st * kBK + piece_chunk[p] * 16;
            const int row = (piece_is_a[p] ? m0 : n0) + piece_row[p];
            const int lim = piece_is_a[p] ? M : N;
            int off = row * K + k;
            if (k >= K || row >= lim) off = 0x7FFFFFF0;  // out of range: zeros
            regs[p] = piece_is_a[p] ? __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0)
                                    : __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 2);
        }
    };
    auto lstore = [&](int buf, const v4i(&regs)[PIECES]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const int row = piece_is_a[p] ? piece_row[p] : BM + piece_row[p];
            *reinterpret_cast<v4i *>(&lds[buf][row * kRowPad + piece_chunk[p] * 16]) = regs[p];
        }
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    v4i regs[PIECES];
    gload(0, regs);
    lstore(0, regs);
    __syncthreads();
    const int fr = lane & 15;           // fragment row (A) / column (B)
    const int fk = (lane >> 4) * 16;    // K byte offset of this lane's 16 bytes
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) gload(st + 1, regs);
        v4i af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = *reinterpret_cast<const v4i *>(&lds[buf][(wm * WM + i * 16 + fr) * kRowPad + fk]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bfr[j] = *reinterpret_cast<const v4i *>(&lds[buf][(BM + wn * 64 + j * 16 + fr) * kRowPad + fk]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
        if (st + 1 < nst) lstore(buf ^ 1, regs);
        __syncthreads();
    }

    // Epilogue: lane l, register r of fragment (i, j) is token
    // m0 + wm*WM + 16 i + 4 (l / 16) + r and weight row n0 + 64 wn + 16 j + l % 16.
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * 64 + j * 16 + fr;
        if (n >= N) continue;
        const float sw = s_w[n];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + r;
                if (m < M) y[static_cast<int64_t>(m) * N + n] = w8a8_epilogue(acc[i][j][r], s_a[m], sw);
            }
        }
    }
}

}  // namespace

hipError_t launch_w8a8_mfma(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N, int K,
                            uint16_t *y, hipStream_t st) {
    // Buffer offsets are 32-bit: matrices past 2 GB take token chunks of 16
    // through the mat-vec instead (same bits, every row is independent).
    if (static_cast<int64_t>(N) * K > 0x7FFF0000ll || static_cast<int64_t>(b) * K > 0x7FFF0000ll) {
        for (int t0 = 0; t0 < b; t0 += 16) {
            const int bc = b - t0 < 16 ? b - t0 : 16;
            hipError_t e = launch_w8a8_matvec(q + static_cast<int64_t>(t0) * K, s_a + t0, w, s_w, bc, N, K,
                                              y + static_cast<int64_t>(t0) * N, 1, nullptr, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int nt = (N + kBN - 1) / kBN;
    // 128-token tiles when they leave enough workgroups for the chip, else 64.
    if (static_cast<int64_t>((b + 127) / 128) * nt >= 2 * device_info().cus) {
        hipLaunchKernelGGL(k_w8a8_mfma<128>, dim3(nt, (b + 127) / 128), dim3(kMfThreads), 0, st, q, s_a, w, s_w, b, N, K, y);
    } else {
        hipLaunchKernelGGL(k_w8a8_mfma<64>, dim3(nt, (b + 63) / 64), dim3(kMfThreads), 0, st, q, s_a, w, s_w, b, N, K, y);
    }
    return hipGetLastError();
}

}  // namespace iqd
