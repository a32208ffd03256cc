// Block-quantized mat-vec, 1 <= b <= 16, gfx950: q8_0-style blocks, and the
// kq6 / kq4 superblock formats decoded into the same block structure.
//
// Per 32-element block j of a row:  isum_j = sum q*w (int32, exact) and the
// leaf  p_j = fl( fl( fl32(isum_j) * d_a[t,j] ) * fl32(d_w[n,j]) ).
// kq6: w = sc * c (sub-scale per 16 weights) and d_w the superblock's scale;
// kq4: the leaf is that of sc * sum q*a with d, minus that of m * sum a with
// dmin (the superblock's pair).
// The m = K/32 leaves are summed by the canonical tree: zero-padded to
// L = 2^ceil(log2 m) leaves, adjacent pairs added level by level, so the root
// is the same for every b, grid, wave count and split.  y = bf16(root).
//
// Sources: "why speculative decoding changed my output", opening (the decode
// workload at q4_k_m and q6_k) and section "the mat-vec kernel" (q6_k rows as
// 256-weight blocks against int8 activation blocks of 32; each block's exact
// integer result is scaled into fp32; the stock
// kernel dealt blocks to warps by a token-count-dependent table, changing
// the float order).  "My speculative decoder got slower", section "Two
// matmul schedules that survived" (split-K moved the rounding points); here
// every split owns an aligned subtree of the one fixed tree.
//
// Mapping (64-lane waves).  A "chunk" is 32 consecutive blocks (1 KiB of a
// row).  Lane l reads the 16-byte half (l & 1) of block (l >> 1) of the chunk
// with one coalesced 16-byte load per row, so a wave instruction covers the
// chunk of one row.  The lane pairs (2i, 2i+1) add their int32 halves (the
// first step of an integer reduce-scatter), the lanes form the fp32 leaves,
// and fp32 reduce-scatter steps over lane masks 2, 4, 8, 16, 32 combine
// adjacent blocks, then adjacent pairs of pairs, ... : exactly the tree
// levels 1..5 over the chunk.  Chunk roots are combined with a binary carry
// stack (the same tree, built left to right), the waves of a workgroup own
// aligned sub-ranges of chunks and fold them in tree order, and API splits
// own aligned subtrees folded by k_blockq8_combine (a subtree smaller than a
// chunk is a window of lanes; the others give -0 leaves).
// A wave takes RS rows at once, so that each activation load serves RS
// weight rows, and issues the loads of U chunks before it uses any; loads of
// blocks past m read zeros from out-of-range buffer offsets, so no branch
// surrounds a load (such branches make the compiler wait for every load in
// flight).
// Leaves of blocks in [m, L) are +0 (the canonical padding).  When L < 32
// the chunk has lanes beyond the tree; their leaves are -0, the exact
// identity of binary32 addition, so they do not disturb the root.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kBqWaves = 4;
constexpr int kBqThreads = kBqWaves * kWave;
constexpr int kMaxLevels = 8;  // chunk-slot tree depth: K <= 131071 -> at most 128 slots
constexpr int kBqOob = 0x7FFFFFF0;  // a buffer offset past every range: the load returns zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int64_t bytes) {
    const int nr = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nr, 0x00020000);
}

struct BqArgs {
    const int8_t *q;
    const float *d_a;
    const int8_t *w;       // q8_0: int8 weights [N, K]
    const uint16_t *d_w;   // q8_0: fp16 [N, K/32]; kq6: superblock scales fp16 [N, K/256];
                           // kq4: (d, dmin) fp16 pairs [N, K/256, 2]
    const uint8_t *ql;     // kq6: low plane [N, K/2]
    const uint8_t *qh;     // kq6: high plane [N, K/4]
    const int8_t *sc;      // kq6: sub-scales [N, K/16]; kq4: (sub-scale, minimum) byte pairs [N, K/32, 2]
    int N, K, m, L;
    uint16_t *y;
    float *part;  // [split, B, N] subtree roots when split > 1
    int split;
    int nslots;  // max(1, L / 32) chunk slots in the whole tree
    int ks;      // waves sharing a row group (aligned sub-ranges of slots)
    int nsteps;
    int nb;      // tokens: at most the kernel's B (tokens past nb read zeros and write nothing)
};

// Insert the root of slot i (0-based within an aligned power-of-two range)
// into a binary carry stack; returns the value the insertion ends with,
// which after the last slot of the range is the root of the whole range.
__device__ __forceinline__ float carry_insert(float (&stk)[kMaxLevels], int i, float v) {
    bool open = true;
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) {
        if (open) {
            if ((i >> l) & 1) {
                v = stk[l] + v;  // left subtree + right subtree
            } else {
                stk[l] = v;
                open = false;
            }
        }
    }
    return v;
}

// kq6: the 16 codes of one group of 16 weights from its 8 bytes of the low
// plane (lo0, lo1) and 4 bytes of the high plane (hi).  The planes hold weight
// i of the group at byte i % 8, nibble i / 8, and at byte i % 4, bit pair
// i / 4, so output word w (weights 4w .. 4w+3, one per byte) takes one shift
// and one mask per plane; u = lo | hi << 4 in [0, 63], and the int8 code
// u - 32 for four bytes at once: (u | 0x80) - 0x20 = u + 0x60 borrows nothing
// from the next byte, and flipping bit 7 back gives u - 32 in two's
// complement.
__device__ __forceinline__ v4i kq6_codes(uint32_t lo0, uint32_t lo1, uint32_t hi) {
    v4i c;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t l = ((w & 1 ? lo1 : lo0) >> (4 * (w >> 1))) & 0x0F0F0F0Fu;
        const uint32_t h = (hi >> (2 * w)) & 0x03030303u;
        const uint32_t u = l | (h << 4);
        c[w] = static_cast<int32_t>(((u | 0x80808080u) - 0x20202020u) ^ 0x80808080u);
    }
    return c;
}

// kq4: the 16 codes (0..15) of a group of 16 weights from its 8 bytes of the
// low plane, laid out as kq6's.
__device__ __forceinline__ v4i kq4_codes(uint32_t lo0, uint32_t lo1) {
    v4i c;
#pragma unroll
    for (int w = 0; w < 4; ++w) c[w] = static_cast<int32_t>(((w & 1 ? lo1 : lo0) >> (4 * (w >> 1))) & 0x0F0F0F0Fu);
    return c;
}

constexpr int kFmtQ8 = 0, kFmtKq6 = 1, kFmtKq4 = 2;  // weight formats of k_blockq8_matvec

struct AddI {
    __device__ int32_t operator()(int32_t a, int32_t b) const { return a + b; }
};
struct AddF {
    __device__ float operator()(float a, float b) const { return a + b; }
};

// FMT: the weight format.  q8_0 blocks; kq6 superblocks (two bit planes, a
// sub-scale per 16 weights, an fp16 scale per 256): the lane's 16 weights are
// one sub-block, whose integer dot is multiplied by its sub-scale before the
// lane pair adds its halves, so the pair forms isum_j = sum of (sc * c) * q
// over the block, and the block's weight scale is its superblock's; kq4
// superblocks (4-bit codes, a sub-scale and a minimum per block, d and dmin per
// 256): the pair forms isum_j = sc * sum q * a and msum_j = m * sum a, and the
// leaf is fl(fl(fl(fl32(isum_j) * d_a) * d) - fl(fl(fl32(msum_j) * d_a) * dmin)).
template <int B, int RS, int U, int FMT>
__global__ __launch_bounds__(kBqThreads) void k_blockq8_matvec(BqArgs a) {
    __shared__ float red[kBqWaves][kWave];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int s = blockIdx.y;
    const int K = a.K, N = a.N, m = a.m, L = a.L;
    const int ks = a.ks;
    const int rg = wave / ks;
    const int kp = wave - rg * ks;
    const int rgs = kBqWaves / ks;
    // Split s owns the aligned subtree of LS = L / split leaves.  When LS < 32
    // the subtree is a window [wlo, wlo + LS) of one chunk: the lanes outside
    // it read nothing and give -0 leaves, the exact identity of binary32
    // addition, so the chunk's root is the window's root.
    const int LS = L / a.split;
    const bool window = LS < 32;
    const int nss = window ? 1 : LS / 32;  // slots per split
    const int nsw = nss / ks;              // slots per wave
    const int slot0 = window ? (s * LS) >> 5 : s * nss + kp * nsw;
    const int wlo = window ? (s * LS) & 31 : 0;
    const bool inwin = (lane >> 1) >= wlo && (lane >> 1) < wlo + (window ? LS : 32);
    const int half = lane & 1;

    constexpr int NV = RS * B;
    constexpr int NP = pow2_ceil(NV);
    constexpr int NPH = NP >= 2 ? NP / 2 : 1;

    // Activations and their scales: one buffer for all tokens (b * K < 2^31).
    const __amdgpu_buffer_rsrc_t qr = buf_rsrc(a.q, static_cast<int64_t>(a.nb) * K);
    const __amdgpu_buffer_rsrc_t dar = buf_rsrc(a.d_a, static_cast<int64_t>(a.nb) * m * 4);

    for (int step = blockIdx.x; step < a.nsteps; step += gridDim.x) {
        const int row0 = (step * rgs + rg) * RS;
        // Weights and block scales of the RS rows from buffers based at the
        // first row (offsets stay below 2 * K whatever N is); rows past N
        // re-read the last row and their results are dropped.
        const int rfirst = min(row0, N - 1);
        const int rlast = min(row0 + RS - 1, N - 1);
        const int nrows = rlast - rfirst + 1;
        constexpr bool KQ = FMT != kFmtQ8;
        const int dstride = FMT == kFmtQ8 ? m : FMT == kFmtKq6 ? K / 256 : 2 * (K / 256);  // fp16 scales per row
        const __amdgpu_buffer_rsrc_t wr =
            KQ ? buf_rsrc(a.ql + static_cast<int64_t>(rfirst) * (K / 2), static_cast<int64_t>(nrows) * (K / 2))
               : buf_rsrc(a.w + static_cast<int64_t>(rfirst) * K, static_cast<int64_t>(nrows) * K);
        const __amdgpu_buffer_rsrc_t hr = buf_rsrc(FMT == kFmtKq6 ? a.qh + static_cast<int64_t>(rfirst) * (K / 4) : nullptr,
                                                   FMT == kFmtKq6 ? static_cast<int64_t>(nrows) * (K / 4) : 0);
        // kq6 sub-scales and kq4 (sub-scale, minimum) pairs are both K/16 bytes per row
        const __amdgpu_buffer_rsrc_t scr = buf_rsrc(KQ ? a.sc + static_cast<int64_t>(rfirst) * (K / 16) : nullptr,
                                                    KQ ? static_cast<int64_t>(nrows) * (K / 16) : 0);
        const __amdgpu_buffer_rsrc_t dwr =
            buf_rsrc(a.d_w + static_cast<int64_t>(rfirst) * dstride, static_cast<int64_t>(nrows) * dstride * 2);
        int roff[RS];
#pragma unroll
        for (int r = 0; r < RS; ++r) roff[r] = min(row0 + r, N - 1) - rfirst;
        float stk[kMaxLevels];
#pragma unroll
        for (int l = 0; l < kMaxLevels; ++l) stk[l] = 0.0f;
        float root = 0.0f;
        for (int i0 = 0; i0 < nsw; i0 += U) {
            // All loads of U slots go out before any is used, and no branch
            // surrounds them: blocks past m (or slots past the wave's range)
            // read zeros from out-of-range offsets.
            v4i wv[U][RS], av[U][B];  // kq6: low plane in words 0-1, high plane in word 2
            uint32_t dwb[U][RS], scb[KQ ? U : 1][RS];
            float dav[U][B];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = (slot0 + i0 + u) * 32 + (lane >> 1);  // this lane's block
                const bool live = i0 + u < nsw && j < m && inwin;
                const int kb = j * 32 + 16 * half;
#pragma unroll
                for (int r = 0; r < RS; ++r) {
                    if constexpr (FMT == kFmtKq4) {
                        // weights kb .. kb + 15: 8 bytes of the low plane; the block's
                        // (sub-scale, minimum) pair and the superblock's (d, dmin) pair
                        const auto lo = __builtin_amdgcn_raw_buffer_load_b64(
                            wr, live ? roff[r] * (K / 2) + kb / 2 : kBqOob, 0, 2);
                        wv[u][r][0] = static_cast<int32_t>(lo[0]);
                        wv[u][r][1] = static_cast<int32_t>(lo[1]);
                        wv[u][r][2] = 0;
                        wv[u][r][3] = 0;
                        scb[u][r] = __builtin_amdgcn_raw_buffer_load_b16(scr, live ? roff[r] * (K / 16) + 2 * j : kBqOob, 0, 0);
                        dwb[u][r] =
                            __builtin_amdgcn_raw_buffer_load_b32(dwr, live ? 2 * (roff[r] * dstride + 2 * (j >> 3)) : kBqOob, 0, 0);
                    } else if constexpr (FMT == kFmtKq6) {
                        // weights kb .. kb + 15: 8 bytes of the low plane, 4 of the high
                        const auto lo = __builtin_amdgcn_raw_buffer_load_b64(
                            wr, live ? roff[r] * (K / 2) + kb / 2 : kBqOob, 0, 2);
                        wv[u][r][0] = static_cast<int32_t>(lo[0]);
                        wv[u][r][1] = static_cast<int32_t>(lo[1]);
                        wv[u][r][2] = static_cast<int32_t>(
                            __builtin_amdgcn_raw_buffer_load_b32(hr, live ? roff[r] * (K / 4) + kb / 4 : kBqOob, 0, 2));
                        wv[u][r][3] = 0;
                        scb[u][r] = __builtin_amdgcn_raw_buffer_load_b8(scr, live ? roff[r] * (K / 16) + 2 * j + half : kBqOob,
                                                                        0, 0);
                        dwb[u][r] =
                            __builtin_amdgcn_raw_buffer_load_b16(dwr, live ? 2 * (roff[r] * dstride + (j >> 3)) : kBqOob, 0, 0);
                    } else {
                        wv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wr, live ? roff[r] * K + kb : kBqOob, 0, 2);
                        dwb[u][r] =
                            __builtin_amdgcn_raw_buffer_load_b16(dwr, live ? 2 * (roff[r] * dstride + j) : kBqOob, 0, 0);
                    }
                }
#pragma unroll
                for (int t = 0; t < B; ++t) {
                    av[u][t] = __builtin_amdgcn_raw_buffer_load_b128(qr, live ? t * K + kb : kBqOob, 0, 0);
                    dav[u][t] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(dar, live ? 4 * (t * m + j) : kBqOob, 0, 0));
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int slot = slot0 + i0 + u;
                if (i0 + u >= nsw) break;  // uniform: past the wave's slots
                const int j = slot * 32 + (lane >> 1);
                const bool live = j < m && inwin;  // blocks in [m, L) are +0 leaves, beyond L or the window -0
                const bool pad = j < L && inwin;    // (a slot made only of padding gives +0)
                float cr = 0.0f;          // a slot made only of padding leaves
                if (slot * 32 < m) {      // uniform
                    int32_t isum[NP], msum[FMT == kFmtKq4 ? NP : 1];
#pragma unroll
                    for (int v = 0; v < NP; ++v) isum[v] = 0;
                    if constexpr (FMT == kFmtKq4) {
#pragma unroll
                        for (int v = 0; v < NP; ++v) msum[v] = 0;
                        int32_t asum[B];  // the half block's activation sum per token
#pragma unroll
                        for (int t = 0; t < B; ++t) asum[t] = dot16(v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101}, av[u][t], 0);
#pragma unroll
                        for (int r = 0; r < RS; ++r) {
                            const v4i c = kq4_codes(static_cast<uint32_t>(wv[u][r][0]), static_cast<uint32_t>(wv[u][r][1]));
                            const int32_t scv = static_cast<int32_t>(scb[u][r] & 0xFFu);
                            const int32_t mnv = static_cast<int32_t>((scb[u][r] >> 8) & 0xFFu);
#pragma unroll
                            for (int t = 0; t < B; ++t) {
                                isum[r * B + t] = dot16(c, av[u][t], 0) * scv;
                                msum[r * B + t] = asum[t] * mnv;
                            }
                        }
                    } else if constexpr (FMT == kFmtKq6) {
#pragma unroll
                        for (int r = 0; r < RS; ++r) {
                            const v4i c = kq6_codes(static_cast<uint32_t>(wv[u][r][0]), static_cast<uint32_t>(wv[u][r][1]),
                                                    static_cast<uint32_t>(wv[u][r][2]));
                            const int32_t scv = static_cast<int8_t>(scb[u][r]);
#pragma unroll
                            for (int t = 0; t < B; ++t) isum[r * B + t] = dot16(c, av[u][t], 0) * scv;
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < B; ++t)
#pragma unroll
                            for (int r = 0; r < RS; ++r) isum[r * B + t] = dot16(wv[u][r], av[u][t], isum[r * B + t]);
                    }
                    float dwv[RS], dmv[RS];  // the block's weight scale (kq4: d) and kq4's dmin
#pragma unroll
                    for (int r = 0; r < RS; ++r) {
                        dwv[r] = fp16_to_f32(static_cast<uint16_t>(dwb[u][r] & 0xFFFFu));
                        dmv[r] = fp16_to_f32(static_cast<uint16_t>(dwb[u][r] >> 16));
                    }
                    // tree level 0 -> block sums: integer reduce-scatter over the lane pair
                    float leaf[NPH];
                    if constexpr (NP >= 2) {
                        rs_step<1, NP>(isum, lane, AddI());
                        if constexpr (FMT == kFmtKq4) rs_step<1, NP>(msum, lane, AddI());
#pragma unroll
                        for (int v = 0; v < NPH; ++v) {
                            const int vlo = v, vhi = v + NPH;
                            const float da_lo = vlo < NV ? dav[u][vlo % B] : 0.0f;
                            const float dw_lo = vlo < NV ? dwv[vlo / B] : 0.0f;
                            const float da_hi = vhi < NV ? dav[u][vhi % B] : 0.0f;
                            const float dw_hi = vhi < NV ? dwv[vhi / B] : 0.0f;
                            const float da = sel(half != 0, da_hi, da_lo);
                            const float dw = sel(half != 0, dw_hi, dw_lo);
                            float p = (static_cast<float>(isum[v]) * da) * dw;
                            if constexpr (FMT == kFmtKq4) {
                                const float dm_lo = vlo < NV ? dmv[vlo / B] : 0.0f;
                                const float dm_hi = vhi < NV ? dmv[vhi / B] : 0.0f;
                                p = p - (static_cast<float>(msum[v]) * da) * sel(half != 0, dm_hi, dm_lo);
                            }
                            leaf[v] = live ? p : (pad ? 0.0f : -0.0f);
                        }
                    } else {
                        const int32_t tot = isum[0] + xor_lane<1>(isum[0]);
                        float p = (static_cast<float>(tot) * dav[u][0]) * dwv[0];
                        if constexpr (FMT == kFmtKq4) {
                            const int32_t mt = msum[0] + xor_lane<1>(msum[0]);
                            p = p - (static_cast<float>(mt) * dav[u][0]) * dmv[0];
                        }
                        leaf[0] = live ? p : (pad ? 0.0f : -0.0f);
                    }
                    // tree levels 1..5 inside the chunk: lane masks 2..32
                    cr = rs_chain<2, NPH>(leaf, lane, AddF());
                }
                root = carry_insert(stk, i0 + u, cr);
            }
        }
        if (ks > 1) {
            red[wave][lane] = root;
            __syncthreads();
            if (kp == 0) {
                if (ks == 2) {
                    root = root + red[wave + 1][lane];
                } else {  // ks == 4
                    root = (root + red[wave + 1][lane]) + (red[wave + 2][lane] + red[wave + 3][lane]);
                }
            }
        }
        const int idx = reduce_scatter_index<NP>(lane);
        if (kp == 0 && lane < NP && idx < NV) {
            const int r = idx / B;
            const int t = idx - r * B;
            const int row = row0 + r;
            if (row < N && t < a.nb) {
                if (a.split == 1)
                    a.y[static_cast<int64_t>(t) * N + row] = bf16_rne(root);
                else
                    a.part[(static_cast<int64_t>(s) * a.nb + t) * N + row] = root;
            }
        }
        if (ks > 1) __syncthreads();
    }
}

// Top log2(split) tree levels over the split roots, then bf16.
__global__ __launch_bounds__(256) void k_blockq8_combine(const float *__restrict__ part, int b, int N,
                                                         int split, uint16_t *__restrict__ y) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = static_cast<int64_t>(b) * N;
    if (i >= total) return;
    float stk[kMaxLevels];
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) stk[l] = 0.0f;
    float root = 0.0f;
    for (int s = 0; s < split; ++s) root = carry_insert(stk, s, part[static_cast<int64_t>(s) * total + i]);
    y[i] = bf16_rne(root);
}

template <int B, int RS, int U, int FMT>
hipError_t launch_rs(const BqArgs &a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_blockq8_matvec<B, RS, U, FMT>), dim3(grid, a.split), dim3(kBqThreads), 0, st, a);
    return hipGetLastError();
}

// Four rows per wave: each activation load serves four weight rows (measured
// on MI355X at 4096 -> 4096 and 12288 -> 4096 against 1, 2 and 8 rows).  At
// b = 1 a wave with at least four slots keeps two slots of loads in flight.
template <int B, int FMT>
hipError_t launch_b(const BqArgs &base, hipStream_t st) {
    constexpr int RS = 4;
    BqArgs a = base;
    const int row_groups = (a.N + RS - 1) / RS;
    const int target = device_info().cus * 16;
    const int nss = a.nslots >= a.split ? a.nslots / a.split : 1;  // whole chunk slots per split (or one window)
    int ks = 1;
    while (ks < kBqWaves && ks * 2 <= nss && static_cast<int64_t>(row_groups) * ks * a.split < target) ks *= 2;
    a.ks = ks;
    const int rows_per_step = (kBqWaves / ks) * RS;
    a.nsteps = (a.N + rows_per_step - 1) / rows_per_step;
    int grid = device_info().cus * 8;
    if (grid > a.nsteps) grid = a.nsteps;
    if constexpr (B == 1) {
        if (nss / ks >= 4) return launch_rs<B, RS, 2, FMT>(a, grid, st);
    }
    return launch_rs<B, RS, 1, FMT>(a, grid, st);
}

// q8_0 at 11 <= b <= 15 runs the 16-token kernel (the other tokens read
// zeros and are not written): measured on MI355X at 12288 -> 4096, 28.4-29.1
// us against 32.0-35.1 with the b-token kernels (the same bits); the kq6 and
// kq4 kernels at those b are as fast as or faster than their 16-token ones.
template <int FMT>
hipError_t launch_any_b(const BqArgs &base, int b, hipStream_t st) {
    BqArgs a = base;
    a.nb = b;
    if (FMT == kFmtQ8 && b >= 11 && b <= 15) b = 16;
    switch (b) {
        case 1: return launch_b<1, FMT>(a, st);
        case 2: return launch_b<2, FMT>(a, st);
        case 3: return launch_b<3, FMT>(a, st);
        case 4: return launch_b<4, FMT>(a, st);
        case 5: return launch_b<5, FMT>(a, st);
        case 6: return launch_b<6, FMT>(a, st);
        case 7: return launch_b<7, FMT>(a, st);
        case 8: return launch_b<8, FMT>(a, st);
        case 9: return launch_b<9, FMT>(a, st);
        case 10: return launch_b<10, FMT>(a, st);
        case 11: return launch_b<11, FMT>(a, st);
        case 12: return launch_b<12, FMT>(a, st);
        case 13: return launch_b<13, FMT>(a, st);
        case 14: return launch_b<14, FMT>(a, st);
        case 15: return launch_b<15, FMT>(a, st);
        case 16: return launch_b<16, FMT>(a, st);
        default: return hipErrorInvalidValue;
    }
}

BqArgs bq_args(int N, int K, uint16_t *y, int split, float *part) {
    const int m = K / 32;
    int L = 1;
    while (L < m) L *= 2;
    BqArgs a{};
    a.N = N;
    a.K = K;
    a.m = m;
    a.L = L;
    a.y = y;
    a.part = part;
    a.split = split;
    a.nslots = L >= 32 ? L / 32 : 1;
    a.ks = 1;
    return a;
}

}  // namespace

hipError_t launch_blockq8_matvec(const int8_t *q, const float *d_a, const int8_t *w,
                                 const uint16_t *d_w, int b, int N, int K, uint16_t *y, int split,
                                 float *part, hipStream_t st) {
    // The matrix-core kernel forms the leaves of all 16 token columns of its
    // instruction whatever b is, so its cost is flat in b; measured on MI355X
    // (4096 -> 4096 and 12288 -> 4096) it is ahead of this kernel only from
    // b = 9 on, where its activations fit in LDS.
    if (b >= 9 && blockq8_mfvec_fits(b, N, K, split))
        return launch_blockq8_mfvec(q, d_a, w, d_w, b, N, K, y, split, part, st);
    BqArgs a = bq_args(N, K, y, split, part);
    a.q = q;
    a.d_a = d_a;
    a.w = w;
    a.d_w = d_w;
    return launch_any_b<kFmtQ8>(a, b, st);
}

hipError_t launch_kq6_matvec(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
                             const uint16_t *d, int b, int N, int K, uint16_t *y, int split, float *part,
                             hipStream_t st) {
    BqArgs a = bq_args(N, K, y, split, part);
    a.q = q;
    a.d_a = d_a;
    a.ql = ql;
    a.qh = qh;
    a.sc = sc;
    a.d_w = d;
    return launch_any_b<kFmtKq6>(a, b, st);
}

hipError_t launch_kq4_matvec(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *scm, const uint16_t *dm,
                             int b, int N, int K, uint16_t *y, int split, float *part, hipStream_t st) {
    BqArgs a = bq_args(N, K, y, split, part);
    a.q = q;
    a.d_a = d_a;
    a.ql = ql;
    a.sc = reinterpret_cast<const int8_t *>(scm);
    a.d_w = dm;
    return launch_any_b<kFmtKq4>(a, b, st);
}

hipError_t launch_blockq8_combine(const float *part, int b, int N, int split, uint16_t *y,
                                  hipStream_t st) {
    const int64_t total = static_cast<int64_t>(b) * N;
    const unsigned grid = static_cast<unsigned>((total + 255) / 256);
    hipLaunchKernelGGL(k_blockq8_combine, dim3(grid), dim3(256), 0, st, part, b, N, split, y);
    return hipGetLastError();
}

}  // namespace iqd
