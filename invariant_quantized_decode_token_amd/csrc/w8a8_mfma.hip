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
// Tiling: a workgroup of GM x GN waves computes a BM x BN tile of y (BM
// tokens, BN weight rows); each wave owns a (BM/GM) x (BN/GN) sub-tile of
// v_mfma_i32_16x16x64_i8 accumulators.  K advances 128 bytes per stage.
//  * Operands go from global memory straight into LDS (buffer loads with the
//    LDS destination, 16 bytes per lane): an S-stage ring, one barrier per
//    stage, no registers spent on staging.
//  * The fragment reads of stage st + 1 are issued between the matrix
//    operations of stage st, so that LDS reads and products overlap within
//    a wave (two fragment register sets); loads run S - 2 stages ahead.
//  * A load instruction fills 1 KiB of LDS in lane order.  Each lane picks
//    the global 16 bytes that belong at its LDS slot: chunk c of row r is
//    kept at slot c ^ ((r >> 1) & 7) of the row, so the 16 rows a fragment
//    read touches fall on 16 distinct bank groups, and the 8 lanes that fill
//    a row still read one contiguous 128-byte segment.
//  * The compiler waits for every load in flight before any LDS read that
//    follows such a load (it cannot tell the ring slots apart).  The fragment
//    reads are therefore issued as inline ds_read_b128, tied to their
//    lgkmcnt wait, and the stage waits are explicit vmcnt counts.
//  * Weights are loaded as ordinary cached data: the M tiles that share a
//    weight tile run on one XCD (tiles are mapped XCD by XCD) and read it
//    from its L2.  The non-temporal hint of the mat-vec cost 20-40 % here.
//  * The epilogue loads every scale of the tile before its first store (one
//    counter tracks loads and stores), writes the bf16 tile to LDS and
//    leaves it as 16-byte stores.
// Operand layout of the instruction (checked on MI355X): lane l holds 16
// bytes of A row (l % 16) and of B column (l % 16) at the same K offset
// 16 * (l / 16); result register i of lane l is D[4 * (l / 16) + i][l % 16].
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kXcds = 8;       // workgroups are dealt round-robin to the 8 XCDs (L2 domains)
constexpr int kBK = 128;       // K bytes per stage
constexpr int kCPR = kBK / 16; // 16-byte chunks per staged row
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every range: the load returns zeros

typedef __attribute__((address_space(3))) int8_t lds_i8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
    const int nr = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nr, 0x00020000);
}

// s_waitcnt vmcnt(n), no wait on the other counters.
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte LDS read the compiler does not track; lgkm_tie() waits for it.
__device__ __forceinline__ v4i lds_read(uint32_t addr) {
    v4i r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
    return r;
}

// Wait for the outstanding LDS reads and mark the fragments as written by the
// wait, so that no use of them is scheduled before it.
template <int N>
__device__ __forceinline__ void lgkm_tie(v4i (&f)[2][N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int x = 0; x < N; ++x) asm volatile("" : "+v"(f[h][x]));
}

// Byte offset, within a stage, of logical chunk c of staged row `row`.
__device__ __forceinline__ uint32_t slot_of(int row, int c) {
    return static_cast<uint32_t>(row * kCPR + (c ^ ((row >> 1) & 7))) * 16;
}

// Row stride (elements) of the bf16 output tile staged in LDS: 16-byte
// aligned rows, and rows four apart fall 16 banks apart for the 2-byte
// writes of the epilogue.
template <int BN>
constexpr int out_stride() { return BN + 8; }

template <int BM, int BN, int S, int GM, int GN>
__global__ __launch_bounds__(64 * GM * GN) void k_w8a8_mfma(const int8_t *__restrict__ q, const float *__restrict__ s_a,
                                                        const int8_t *__restrict__ w, const float *__restrict__ s_w,
                                                        int M, int N, int K, uint16_t *__restrict__ y,
                                                        int32_t *__restrict__ part, int split) {
    constexpr int NWV = GM * GN, NTH = kWave * NWV;  // waves, GM x GN over the tile
    constexpr int WM = BM / GM, WN = BN / GN;        // wave sub-tile
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int PA = BM / (8 * NWV), PB = BN / (8 * NWV);  // 1 KiB load instructions per wave per stage
    constexpr int STAGE = (BM + BN) * kBK;
    static_assert(BM % (8 * NWV) == 0 && BN % (8 * NWV) == 0 && S >= 2, "tile and ring");
    extern __shared__ __attribute__((aligned(16))) int8_t lds_all[];  // [S][STAGE], then the output tile

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

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = lane_id();
    const int wm = wave / GN, wn = wave % GN;
    // Split s of `split` (blockIdx.y) owns the stages [st0, st1); K bytes at or
    // past k_hi load as zeros.  A split with no stage writes zero partials.
    const int nst_all = (K + kBK - 1) / kBK;
    const int per = (nst_all + split - 1) / split;
    const int st0 = min(nst_all, static_cast<int>(blockIdx.y) * per);
    const int nst = min(nst_all, st0 + per) - st0;
    const int k_hi = min(K, (st0 + nst) * kBK);
    const __amdgpu_buffer_rsrc_t ra = rsrc(q, static_cast<int64_t>(M) * K);
    const __amdgpu_buffer_rsrc_t rb = rsrc(w, static_cast<int64_t>(N) * K);
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_all));

    // Load instruction p of this wave fills LDS slots 64 (NWV p + wave) ..
    // + 63 of a stage: lane -> (row, slot) -> the logical chunk stored there.
    // Instructions p < PA hold activation rows, the rest weight rows.
    uint32_t goff[PA + PB];
    int gk[PA + PB];  // byte offset of the lane's chunk within the stage's K range
#pragma unroll
    for (int p = 0; p < PA + PB; ++p) {
        const int u = (NWV * p + wave) * kWave + lane;
        const int row = u / kCPR;
        const int c = (u % kCPR) ^ ((row >> 1) & 7);
        gk[p] = 16 * c;
        const int gr = p < PA ? m0 + row : n0 + row - BM;
        const bool in = gr < (p < PA ? M : N);
        goff[p] = in ? static_cast<uint32_t>(gr) * static_cast<uint32_t>(K) + 16 * c : kOob;
    }
    auto stage_load = [&](int st, int buf) __attribute__((always_inline)) {
        const int k0 = (st0 + st) * kBK;  // past k_hi (stages beyond the last) every lane reads zeros
#pragma unroll
        for (int p = 0; p < PA + PB; ++p) {
            const bool in = goff[p] != kOob && k0 + gk[p] < k_hi;
            const uint32_t off = in ? goff[p] + static_cast<uint32_t>(k0) : kOob;
            lds_i8 *dst = (lds_i8 *)(lds_all + buf * STAGE + (NWV * p + wave) * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(p < PA ? ra : rb, dst, 16, off, 0, 0, 0);
        }
    };

    // Fragment addresses within a stage for the two 64-byte K steps.
    const int fr = lane & 15, fc = lane >> 4;
    uint32_t fa[2][FM + FN];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[kk][i] = slot_of(wm * WM + 16 * i + fr, 4 * kk + fc);
#pragma unroll
        for (int j = 0; j < FN; ++j) fa[kk][FM + j] = slot_of(BM + wn * WN + 16 * j + fr, 4 * kk + fc);
    }

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    static_assert(S >= 3, "stage st + 1 is read while stage st is multiplied");
#pragma unroll
    for (int s = 0; s < S - 1; ++s) stage_load(s, s);
    // Stage 0 in LDS for every wave, then its fragments.
    wait_vm<(PA + PB) * (S - 2)>();
    __builtin_amdgcn_s_barrier();
    auto read_frags = [&](v4i (&f)[2][FM + FN], int st) __attribute__((always_inline)) {
        const uint32_t sb = lds_base + static_cast<uint32_t>((st % S) * STAGE);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int x = 0; x < FM + FN; ++x) f[h][x] = lds_read(sb + fa[h][x]);
    };
    v4i fx[2][FM + FN], fy[2][FM + FN];
    read_frags(fx, 0);
    // Step st: wait for the fragments of stage st (read during step st - 1)
    // and for this wave's loads of stage st + 1; the barrier then tells that
    // every wave's loads of stage st + 1 have landed and that every wave has
    // its fragments of stage st - 1, whose slot takes stage st + S - 1.  The
    // products of stage st follow, each with one fragment read of stage
    // st + 1 behind it.
    auto step = [&](v4i (&cur)[2][FM + FN], v4i (&nxt)[2][FM + FN], int st) __attribute__((always_inline)) {
        lgkm_tie<FM + FN>(cur);
        wait_vm<(PA + PB) * (S - 3)>();
        __builtin_amdgcn_s_barrier();
        stage_load(st + S - 1, (st + S - 1) % S);
        const uint32_t sb = lds_base + static_cast<uint32_t>(((st + 1) % S) * STAGE);
        constexpr int NR = 2 * (FM + FN), NM = 2 * FM * FN;
        static_assert(NM >= NR, "one fragment read per product at most");
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int h = m / (FM * FN), i = (m % (FM * FN)) / FN, j = m % FN;
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur[h][i], cur[h][FM + j], acc[i][j], 0, 0, 0);
            if (m < NR) nxt[m / (FM + FN)][m % (FM + FN)] = lds_read(sb + fa[m / (FM + FN)][m % (FM + FN)]);
            __builtin_amdgcn_sched_barrier(0);  // keep the product / read order
        }
    };
    int st = 0;
    for (; st + 1 < nst; st += 2) {
        step(fx, fy, st);
        step(fy, fx, st + 1);
    }
    if (st < nst) step(fx, fy, st);
    // The last step read stage nst (zeros or a tile edge), which nothing uses;
    // its registers must land before they are reused.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    if (part) {
        // Exact int32 partial sums of this split, part[split][M][N]; the
        // combine adds the splits and applies the epilogue.  Lane l, register
        // r of fragment (i, j) holds the element named below.
        wait_vm<0>();
        int32_t *ps = part + static_cast<int64_t>(blockIdx.y) * M * N;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * WM + i * 16 + fc * 4 + r;
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = n0 + wn * WN + j * 16 + fr;
                    if (n < N) ps[static_cast<int64_t>(m) * N + n] = acc[i][j][r];
                }
            }
        return;
    }

    // Scales of the tile, loaded before the first store.  Lane l, register r
    // of fragment (i, j) is token m0 + wm*WM + 16 i + 4 (l / 16) + r and weight
    // row n0 + wn*WN + 16 j + l % 16.
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
            const int m = m0 + wm * WM + i * 16 + fc * 4 + r;
            sa[i][r] = m < M ? s_a[m] : 0.0f;
        }
    // The loads issued past the last stage still write zeros into the ring:
    // they land before the output tile reuses its space.
    wait_vm<0>();
    __syncthreads();

    // Epilogue into a bf16 tile in LDS, then stores of 16 contiguous bytes
    // (8 outputs of one token) by every thread of the workgroup.
    constexpr int OTS = out_stride<BN>();
    uint16_t *ot = reinterpret_cast<uint16_t *>(lds_all);  // [BM][OTS]
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ot[(wm * WM + i * 16 + fc * 4 + r) * OTS + wn * WN + j * 16 + fr] =
                    w8a8_epilogue(acc[i][j][r], sa[i][r], sw[j]);
    __syncthreads();
    constexpr int PPR = BN / 8;  // 16-byte pieces per tile row
    for (int p = static_cast<int>(threadIdx.x); p < BM * PPR; p += NTH) {
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

template <int BM, int BN, int S, int GM, int GN>
hipError_t launch_tiles(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N, int K,
                        uint16_t *y, int split, int32_t *part, hipStream_t st) {
    const size_t ring = static_cast<size_t>(S) * (BM + BN) * kBK;
    const size_t otile = static_cast<size_t>(BM) * out_stride<BN>() * 2;
    const size_t smem = ring > otile ? ring : otile;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_w8a8_mfma<BM, BN, S, GM, GN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    const int mt = (b + BM - 1) / BM;
    const int nt = (N + BN - 1) / BN;
    const int nt_pad = (nt + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((k_w8a8_mfma<BM, BN, S, GM, GN>), dim3(mt * nt_pad, split), dim3(kWave * GM * GN), smem, st, q,
                       s_a, w, s_w, b, N, K, y, split > 1 ? part : nullptr, split);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_w8a8_mfma(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N, int K,
                            uint16_t *y, int split, int32_t *part, hipStream_t st) {
    // Buffer offsets are 32-bit: matrices past 2 GB take token chunks of 16
    // through the mat-vec instead (same bits, every row is independent, and
    // the split does not change them).
    if (static_cast<int64_t>(N) * K > 0x7FFF0000ll || static_cast<int64_t>(b) * K > 0x7FFF0000ll) {
        for (int t0 = 0; t0 < b; t0 += 16) {
            const int bc = b - t0 < 16 ? b - t0 : 16;
            hipError_t e = launch_w8a8_matvec(q + static_cast<int64_t>(t0) * K, s_a + t0, w, s_w, bc, N, K,
                                              y + static_cast<int64_t>(t0) * N, 1, nullptr, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // Tile choice, measured at b = 512 on the Qwen3-8B layers (weights read
    // from HBM, eight copies in rotation), 8 waves throughout, one workgroup
    // per CU (the rings take 96-128 KiB of LDS):
    //  * 64 x 128 tiles (4 stages) when they, times the K splits, fill at
    //    most one round of CUs and K <= 8192 (o: 17.0 us against 17.9 with
    //    the 128 x 64 tiles);
    //  * 128 x 64 tiles (5 stages) for such shapes with longer rows (down,
    //    K = 12288: 45.8 against 49.0 us);
    //  * else 128 x 128 tiles (4 stages; qkv 22.7 and gate_up 73.6 us, 384
    //    and 1536 narrow tiles would take 1.5 and 6 rounds).
    const int cus = device_info().cus;
    const int64_t narrow = static_cast<int64_t>((b + 63) / 64) * ((N + 127) / 128) * split;
    hipError_t e = narrow > cus ? launch_tiles<128, 128, 4, 2, 4>(q, s_a, w, s_w, b, N, K, y, split, part, st)
                   : K <= 8192  ? launch_tiles<64, 128, 4, 2, 4>(q, s_a, w, s_w, b, N, K, y, split, part, st)
                                : launch_tiles<128, 64, 5, 4, 2>(q, s_a, w, s_w, b, N, K, y, split, part, st);
    if (e != hipSuccess || split == 1) return e;
    return launch_w8a8_combine(part, s_a, s_w, b, N, split, y, st);
}

}  // namespace iqd
