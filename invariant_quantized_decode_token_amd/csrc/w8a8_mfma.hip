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
// Tiling: a workgroup computes a BM x BN tile of y (BM tokens, BN weight
// rows) with KG groups of 4 waves; group g takes the K stages g, g + KG, ...
// and its waves are 2 x 2, each owning a (BM/2) x (BN/2) sub-tile of
// v_mfma_i32_16x16x64_i8 accumulators.  K advances BK bytes per stage; both
// operand tiles are staged in LDS (rows padded by 16 bytes, so that the 16
// rows a fragment read touches fall on distinct banks), double-buffered per
// group, and a ring of R register sets keeps the global loads of R - 1
// stages in flight.  The groups' partial tiles are added through LDS at the
// end (exact int32), and the bf16 tile leaves through LDS as 16-byte stores.
// Measured on MI355X (per-stage timestamps and kernels with parts removed):
// a stage costs its barrier, its global loads, its LDS traffic and its
// matrix-core work nearly one after the other, so overlap comes from a
// second workgroup on the CU rather than from a deeper ring.
// Tiles are mapped to workgroups XCD by XCD so that the M tiles sharing a
// weight tile run on one XCD and reuse it from its L2.
// Operand layout of the instruction (checked on MI355X): lane l holds 16
// bytes of A row (l % 16) and of B column (l % 16) at the same K offset
// 16 * (l / 16); result register i of lane l is D[4 * (l / 16) + i][l % 16].
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

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

// Row stride (elements) of the bf16 output tile staged in LDS: 16-byte
// aligned rows, and rows four apart fall 16 banks apart for the 2-byte
// writes of the epilogue.
template <int BN>
constexpr int out_stride() { return BN + 8; }

template <int BM, int BN, int BK, int KG, int R>
__global__ __launch_bounds__(KG * kGroupThreads) void k_w8a8_mfma(const int8_t *__restrict__ q,
                                                                  const float *__restrict__ s_a,
                                                                  const int8_t *__restrict__ w,
                                                                  const float *__restrict__ s_w, int M, int N, int K,
                                                                  uint16_t *__restrict__ y) {
    constexpr int WM = BM / 2;        // wave sub-tile rows (tokens)
    constexpr int FM = WM / 16;       // fragments along M per wave
    constexpr int WN = BN / 2;        // wave sub-tile columns (weight rows)
    constexpr int FN = WN / 16;       // fragments along N per wave
    constexpr int kBK = BK;
    constexpr int kRowPad = row_pad<BK>();
    constexpr int CPR = kBK / 16;     // 16-byte pieces per staged row
    constexpr int A_PIECES = BM * CPR;
    constexpr int B_PIECES = BN * CPR;
    constexpr int PIECES = (A_PIECES + B_PIECES) / kGroupThreads;
    static_assert((A_PIECES + B_PIECES) % kGroupThreads == 0, "whole pieces per thread");
    extern __shared__ __attribute__((aligned(16))) int8_t lds_all[];  // [KG][2][(BM + BN) * kRowPad]
    constexpr int STAGE = (BM + BN) * kRowPad;

    // Tile of this workgroup.  The M tiles of one N tile (which read the same
    // weight rows) are given consecutive slots of one XCD, so that the
    // weight tile is fetched into that XCD's L2 once and reused from there.
    const int mt = (M + BM - 1) / BM;
    const int nt = (N + BN - 1) / BN;
    const int L = blockIdx.x;
    const int xcd = L % kXcds, slot = L / kXcds;
    const int ntile = (slot / mt) * kXcds + xcd;
    const int mtile = slot % mt;
    if (ntile >= nt) return;  // padding slots of the last XCD round
    const int m0 = mtile * BM;
    const int n0 = ntile * BN;

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
    // Piece p of a thread is an activation piece for p < A_PIECES / 256 and a
    // weight piece after that, the same for every lane: no lane-dependent
    // branch surrounds a load (such branches make the compiler wait for all
    // loads in flight before the next LDS store).
    static_assert(A_PIECES % kGroupThreads == 0, "whole activation pieces per thread");
    auto gload = [&](int st, v4i(&regs)[PIECES]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            constexpr int AP = A_PIECES / kGroupThreads;
            const bool is_a = p < AP;
            const int j = tid + (is_a ? p : p - AP) * kGroupThreads;
            const int k = (st * KG + kg) * kBK + (j % CPR) * 16;
            const int row = (is_a ? m0 : n0) + j / CPR;
            const bool in = k < K && row < (is_a ? M : N);
            const int off = in ? row * K + k : 0x7FFFFFF0;
            if (is_a)
                regs[p] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
            else
                regs[p] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 2);
        }
    };
    auto lstore = [&](int buf, const v4i(&regs)[PIECES]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            constexpr int AP = A_PIECES / kGroupThreads;
            const bool is_a = p < AP;
            const int j = tid + (is_a ? p : p - AP) * kGroupThreads;
            const int row = (is_a ? 0 : BM) + j / CPR;
            *reinterpret_cast<v4i *>(&lds[buf * STAGE + row * kRowPad + (j % CPR) * 16]) = regs[p];
        }
    };

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // A ring of R register sets holds the global loads of the next R - 1
    // stages while one stage is multiplied out of LDS.  Loads of stages past
    // K read zeros (their buffer offsets are out of range), so no branch
    // guards a load.
    v4i ring[R][PIECES];
#pragma unroll
    for (int d = 0; d < R; ++d) gload(d, ring[d]);
    lstore(0, ring[0]);
    __syncthreads();
    const int fr = lane & 15;         // fragment row (A) / column (B)
    const int fk = (lane >> 4) * 16;  // K byte offset of this lane's 16 bytes within 64
    for (int st0 = 0; st0 < nst; st0 += R) {
#pragma unroll
        for (int d = 0; d < R; ++d) {
            const int st = st0 + d;
            if (st >= nst) break;  // uniform: the last round may be short
            lstore((st + 1) & 1, ring[(d + 1) % R]);  // stage st + 1, loaded R - 1 stages ago
            gload(st + R, ring[d]);                  // stage st + R into the set stage st used
            const int8_t *base = lds + (st & 1) * STAGE;
#pragma unroll
            for (int kk = 0; kk < kBK / 64; ++kk) {
                v4i af[FM], bfr[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = *reinterpret_cast<const v4i *>(base + (wm * WM + i * 16 + fr) * kRowPad + kk * 64 + fk);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bfr[j] = *reinterpret_cast<const v4i *>(base + (BM + wn * WN + j * 16 + fr) * kRowPad + kk * 64 + fk);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
            __syncthreads();
        }
    }

    // Scales of the tile, loaded before the first store: one counter tracks
    // both loads and stores, so a load issued after stores would wait for
    // them to complete.  Lane l, register r of fragment (i, j) is token
    // m0 + wm*WM + 16 i + 4 (l / 16) + r and weight row n0 + 64 wn + 16 j + l % 16.
    float sw[FN], sa[FM][4];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WN + j * 16 + fr;
        sw[j] = n < N ? s_w[n] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + r;
            sa[i][r] = m < M ? s_a[m] : 0.0f;
        }

    // The other K groups hand their partial tiles to group 0 through LDS
    // (the stage buffers are free after the loop's last barrier).
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
        if (kg == 0) {
#pragma unroll
            for (int g = 1; g < KG; ++g)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] += xch[(((g - 1) * 4 + wave) * FM * FN + i * FN + j) * kWave + lane];
        }
        __syncthreads();  // the exchange is read before the output tile reuses its space
    }

    // Epilogue into a bf16 tile in LDS, then stores of 16 contiguous bytes
    // (8 outputs of one token) by every thread of the workgroup.
    constexpr int OTS = out_stride<BN>();
    uint16_t *ot = reinterpret_cast<uint16_t *>(lds_all);  // [BM][OTS]
    if (kg == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ot[(wm * WM + i * 16 + (lane >> 4) * 4 + r) * OTS + wn * WN + j * 16 + fr] =
                        w8a8_epilogue(acc[i][j][r], sa[i][r], sw[j]);
    }
    __syncthreads();
    constexpr int PPR = BN / 8;  // 16-byte pieces per tile row
    for (int p = static_cast<int>(threadIdx.x); p < BM * PPR; p += KG * kGroupThreads) {
        const int row = p / PPR, c = (p % PPR) * 8;
        const int m = m0 + row, n = n0 + c;
        if (m >= M || n >= N) continue;
        const v4i v = *reinterpret_cast<const v4i *>(&ot[row * OTS + c]);
        uint16_t *dst = y + static_cast<int64_t>(m) * N + n;
        if ((N & 7) == 0) {  // n + 8 <= N and the row start is 16-byte aligned
            *reinterpret_cast<v4i *>(dst) = v;
        } else {
            uint16_t e[8];
            __builtin_memcpy(e, &v, sizeof(e));
            for (int t = 0; t < 8 && n + t < N; ++t) dst[t] = e[t];
        }
    }
}

template <int BM, int BN, int BK, int KG, int R>
hipError_t launch_tiles(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N, int K,
                        uint16_t *y, hipStream_t st) {
    constexpr int WM = BM / 2, FM = WM / 16, FN = BN / 32;
    const size_t stages = static_cast<size_t>(KG) * 2 * (BM + BN) * row_pad<BK>();
    const size_t xch = static_cast<size_t>(KG - 1) * 4 * FM * FN * kWave * 16;
    const size_t otile = static_cast<size_t>(BM) * out_stride<BN>() * 2;
    size_t smem = stages > xch ? stages : xch;
    if (otile > smem) smem = otile;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_w8a8_mfma<BM, BN, BK, KG, R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    const int mt = (b + BM - 1) / BM;
    const int nt = (N + BN - 1) / BN;
    const int nt_pad = (nt + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((k_w8a8_mfma<BM, BN, BK, KG, R>), dim3(mt * nt_pad), dim3(KG * kGroupThreads), smem, st, q, s_a, w,
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
    // Tile choice, measured at b = 512 on the Qwen3-8B layers against 32- to
    // 128-token and 64- or 128-row tiles, 64- or 128-byte stages, 1, 2 or 4 K
    // groups and ring depths 2 to 8: while the 64 x 128 tiles fit one per CU,
    // two K groups (8 waves) share each tile; past that, tiles with one K
    // group, two or more workgroups per CU, whose barriers do not wait for
    // each other: 128 x 128 when there are at least as many as CUs, else
    // 64 x 64.
    const int cus = device_info().cus;
    const int64_t tiles = static_cast<int64_t>((b + 63) / 64) * ((N + 127) / 128);
    const int64_t big = static_cast<int64_t>((b + 127) / 128) * ((N + 127) / 128);
    if (tiles <= cus) return launch_tiles<64, 128, 128, 2, 4>(q, s_a, w, s_w, b, N, K, y, st);
    if (big < cus) return launch_tiles<64, 64, 128, 1, 3>(q, s_a, w, s_w, b, N, K, y, st);
    return launch_tiles<128, 128, 128, 1, 3>(q, s_a, w, s_w, b, N, K, y, st);
}

}  // namespace iqd
