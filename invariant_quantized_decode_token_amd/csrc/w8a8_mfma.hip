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
// Tiling: a workgroup computes a BM x 128 tile of y (BM tokens, 128 weight
// rows) with KG groups of 4 waves; group g takes the K stages g, g + KG, ...
// and its waves are 2 x 2, each owning a (BM/2) x 64 sub-tile of
// v_mfma_i32_16x16x64_i8 accumulators.  K advances BK bytes per stage; both
// operand tiles are staged in LDS (rows padded by 16 bytes, so that the 16
// rows a fragment read touches fall on distinct banks), double-buffered per
// group, with two stages of global loads in flight ahead of the stage being
// multiplied.  The groups' partial tiles are added through LDS at the end
// (exact int32).  At b = 512 the kernel is bound by load latency: more K
// groups keep more bytes in flight per CU.
// Tiles are mapped to workgroups XCD by XCD so that the M tiles sharing a
// weight tile run on one XCD and reuse it from its L2.
// Operand layout of the instruction (checked on MI355X): lane l holds 16
// bytes of A row (l % 16) and of B column (l % 16) at the same K offset
// 16 * (l / 16); result register i of lane l is D[4 * (l / 16) + i][l % 16].
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kBN = 128;
constexpr int kGroupThreads = 256;  // one K group: 4 waves, 2 x 2 over the tile
constexpr int kXcds = 8;      // workgroups are dealt round-robin to the 8 XCDs (L2 domains)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
    const int nr = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nr, 0x00020000);
}

// Staged row: BK bytes plus 16 of padding, so that the 16 rows one fragment
// read touches fall on distinct LDS banks.
template <int BK>
constexpr int row_pad() { return BK + 16; }

template <int BM, int BK, int KG>
__global__ __launch_bounds__(KG * kGroupThreads) void k_w8a8_mfma(const int8_t *__restrict__ q,
                                                                  const float *__restrict__ s_a,
                                                                  const int8_t *__restrict__ w,
                                                                  const float *__restrict__ s_w, int M, int N, int K,
                                                                  uint16_t *__restrict__ y) {
    constexpr int WM = BM / 2;        // wave sub-tile rows (tokens)
    constexpr int FM = WM / 16;       // fragments along M per wave
    constexpr int FN = 64 / 16;       // fragments along N per wave
    constexpr int kBK = BK;
    constexpr int kRowPad = row_pad<BK>();
    constexpr int CPR = kBK / 16;     // 16-byte pieces per staged row
    constexpr int A_PIECES = BM * CPR;
    constexpr int B_PIECES = kBN * CPR;
    constexpr int PIECES = (A_PIECES + B_PIECES) / kGroupThreads;
    static_assert((A_PIECES + B_PIECES) % kGroupThreads == 0, "whole pieces per thread");
    extern __shared__ __attribute__((aligned(16))) int8_t lds_all[];  // [KG][2][(BM + kBN) * kRowPad]
    constexpr int STAGE = (BM + kBN) * kRowPad;

    // Tile of this workgroup.  The M tiles of one N tile (which read the same
    // weight rows) are given consecutive slots of one XCD, so that the
    // weight tile is fetched into that XCD's L2 once and reused from there.
    const int mt = (M + BM - 1) / BM;
    const int nt = (N + kBN - 1) / kBN;
    const int L = blockIdx.x;
    const int xcd = L % kXcds, slot = L / kXcds;
    const int ntile = (slot / mt) * kXcds + xcd;
    const int mtile = slot % mt;
    if (ntile >= nt) return;  // padding slots of the last XCD round
    const int m0 = mtile * BM;
    const int n0 = ntile * kBN;

    // K group kg takes the stages st = kg, kg + KG, ... of K; its 4 waves
    // split the tile 2 x 2.  The groups' partial tiles are added at the end
    // (exact int32), so the split does not change a bit.
    const int kg = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kGroupThreads);
    const int tid = static_cast<int>(threadIdx.x) - kg * kGroupThreads;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave >> 1, wn = wave & 1;
    const int nst_all = (K + kBK - 1) / kBK;
    // Every group walks the same number of stages (the workgroup shares its
    // barriers); a stage past K loads zeros.
    const int nst = (nst_all + KG - 1) / KG;
    int8_t *lds = lds_all + kg * 2 * STAGE;

    // Every row of A (token) and B (weight) is a K-long byte row; the
    // resources end at the matrix ends and a piece past K or past the last row
    // is redirected out of range, so it reads zeros.
    const __amdgpu_buffer_rsrc_t ra = rsrc(q, static_cast<int64_t>(M) * K);
    const __amdgpu_buffer_rsrc_t rb = rsrc(w, static_cast<int64_t>(N) * K);
    auto gload = [&](int st, v4i(&regs)[PIECES]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const int id = tid + p * kGroupThreads;
            const bool is_a = id < A_PIECES;
            const int j = is_a ? id : id - A_PIECES;
            const int k = (st * KG + kg) * kBK + (j % CPR) * 16;
            const int row = (is_a ? m0 : n0) + j / CPR;
            int off = row * K + k;
            if (k >= K || row >= (is_a ? M : N)) off = 0x7FFFFFF0;
            regs[p] = is_a ? __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0)
                           : __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 2);
        }
    };
    auto lstore = [&](int buf, const v4i(&regs)[PIECES]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const int id = tid + p * kGroupThreads;
            const bool is_a = id < A_PIECES;
            const int j = is_a ? id : id - A_PIECES;
            const int row = (is_a ? 0 : BM) + j / CPR;
            *reinterpret_cast<v4i *>(&lds[buf * STAGE + row * kRowPad + (j % CPR) * 16]) = regs[p];
        }
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // Two stages of global loads in flight ahead of the one being computed.
    v4i r0[PIECES], r1[PIECES];
    gload(0, r0);
    if (nst > 1) gload(1, r1);
    lstore(0, r0);
    __syncthreads();
    const int fr = lane & 15;         // fragment row (A) / column (B)
    const int fk = (lane >> 4) * 16;  // K byte offset of this lane's 16 bytes within 64
    auto stage = [&](int st, v4i(&next)[PIECES], v4i(&cur_in)[PIECES]) __attribute__((always_inline)) {
        const int buf = st & 1;
        if (st + 1 < nst) lstore(buf ^ 1, cur_in);          // stage st+1, loaded one stage ago
        if (st + 2 < nst) gload(st + 2, next);               // stage st+2 into the registers just freed
        const int8_t *base = lds + buf * STAGE;
#pragma unroll
        for (int kk = 0; kk < kBK / 64; ++kk) {
            v4i af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const v4i *>(base + (wm * WM + i * 16 + fr) * kRowPad + kk * 64 + fk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const v4i *>(base + (BM + wn * 64 + j * 16 + fr) * kRowPad + kk * 64 + fk);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    };
    // r0 is free after stage 0's store; stage st stores st+1 from the other set.
    for (int st = 0; st < nst; st += 2) {
        stage(st, r0, r1);
        if (st + 1 < nst) stage(st + 1, r1, r0);
    }

    // The other K groups hand their partial tiles to group 0 through LDS
    // (their stage buffers are free after the loop's last barrier).
    if constexpr (KG > 1) {
        v4i *xch = reinterpret_cast<v4i *>(lds_all);  // [KG - 1][4 waves][FM * FN][64 lanes]
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    xch[(((kg - 1) * 4 + wave) * FM * FN + i * FN + j) * kWave + lane] = acc[i][j];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int g = 1; g < KG; ++g)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] += xch[(((g - 1) * 4 + wave) * FM * FN + i * FN + j) * kWave + lane];
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

template <int BM, int BK, int KG>
hipError_t launch_tiles(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N, int K,
                        uint16_t *y, hipStream_t st) {
    constexpr int WM = BM / 2, FM = WM / 16, FN = 4;
    const size_t stages = static_cast<size_t>(KG) * 2 * (BM + kBN) * row_pad<BK>();
    const size_t xch = static_cast<size_t>(KG - 1) * 4 * FM * FN * kWave * 16;
    const size_t smem = stages > xch ? stages : xch;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_w8a8_mfma<BM, BK, KG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    const int mt = (b + BM - 1) / BM;
    const int nt = (N + kBN - 1) / kBN;
    const int nt_pad = (nt + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((k_w8a8_mfma<BM, BK, KG>), dim3(mt * nt_pad), dim3(KG * kGroupThreads), smem, st, q, s_a, w,
                       s_w, b, N, K, y);
    return hipGetLastError();
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
    // Two K groups per workgroup (8 waves) keep twice the loads in flight
    // per CU; the tile shape follows the tile count (measured at b = 512 on
    // the Qwen3-8B layers, against 1 or 4 groups, 32- to 128-token tiles and
    // 64- or 128-byte stages): up to one 64 x 128 tile per CU, 128-byte
    // stages; up to two, 64-byte stages; past that, 128 x 128 tiles.
    const int64_t tiles = static_cast<int64_t>((b + 63) / 64) * ((N + kBN - 1) / kBN);
    const int cus = device_info().cus;
    if (tiles <= cus) return launch_tiles<64, 128, 2>(q, s_a, w, s_w, b, N, K, y, st);
    if (tiles <= 2 * cus) return launch_tiles<64, 64, 2>(q, s_a, w, s_w, b, N, K, y, st);
    return launch_tiles<128, 64, 2>(q, s_a, w, s_w, b, N, K, y, st);
}

}  // namespace iqd
