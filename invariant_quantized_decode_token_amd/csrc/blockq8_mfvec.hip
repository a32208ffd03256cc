// Block-quantized (q8_0-style) mat-vec on the int8 matrix cores, for decode
// and verify passes (1 <= b <= 16), gfx950.  Same results as
// k_blockq8_matvec bit for bit:
//
//   isum_j = sum over block j of q * w (int32, exact),
//   p_j    = fl( fl( fl32(isum_j) * d_a[t, j] ) * fl32(d_w[n, j]) ),
//   y      = bf16( canonical tree over p_0 .. p_{m-1} ): zero-padded to
//            L = 2^ceil(log2 m) leaves, adjacent pairs added level by level.
//
// Sources: "why speculative decoding changed my output", section "the mat-vec
// kernel" (exact block dot products scaled into fp32, then a float sum whose
// order must not depend on the token count).  "My speculative decoder got
// slower", section "Two matmul schedules that survived" (split-K moves the
// rounding points; here every split owns an aligned subtree of the one tree).
//
// Mapping (64-lane waves; v_mfma_i32_16x16x32_i8: A = 16 weight rows, B = 16
// token columns, K = 32 bytes = exactly one block, so one instruction yields
// the exact block sums of 16 rows x 16 tokens):
//  * weights are cut into tiles of 16 rows and K into units of 8 blocks
//    (256 bytes).  The tree is cut the same way: a unit is an aligned subtree
//    of 8 leaves, each of the KS waves of a tile slot owns an aligned subtree
//    of units, each API split an aligned subtree of those;
//  * per unit a wave loads its 16 rows x 256 bytes with four 16-byte buffer
//    loads per lane (4 rows x 256 contiguous bytes per instruction) and its
//    16 x 8 fp16 block scales with two 2-byte loads per lane, writes both to
//    a wave-private LDS tile, and reads back the operand layout: lane
//    l = r + 16 g takes row r, bytes 32 j + 8 g for block j of the unit;
//  * activations and their block scales are staged once per workgroup in LDS
//    (row strides padded for conflict-free 16-token reads); lane l reads
//    token l % 16 (clamped to b - 1; columns of tokens >= b are dropped);
//  * result register i of lane l is the block sum of row 4 (l / 16) + i and
//    token l % 16, so every leaf of a (row, token) pair lands in one lane:
//    the 8-leaf unit tree is three levels of in-register adds, units fold
//    with a binary carry stack (the same tree, built left to right), the KS
//    wave roots fold in tree order through LDS, and split roots fold in
//    k_blockq8_combine;
//  * leaves of blocks in [m, L) are +0, the canonical padding; when L < 8 the
//    unit has leaves beyond the tree, fed as -0, the exact identity of
//    binary32 addition.
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kTileRows = 16;
constexpr int kUnitBlocks = 8;
constexpr int kUnit = 32 * kUnitBlocks;       // K bytes per unit
constexpr int kTRow = kUnit + 16;             // padded LDS row of the transposed weight tile
constexpr int kTBytes = kTileRows * kTRow;    // one wave's staged weights
constexpr int kDwBytes = kTileRows * 16;      // one wave's staged block scales (16 rows x 8 fp16)
constexpr int kWaveLds = kTBytes + kDwBytes;
constexpr int kOob = 0x7FFFFFF0;
constexpr int kMaxLds = 160 * 1024;
constexpr int kMaxLevels = 7;  // chunks per wave slice: at most 64 (K <= 131071, 8 waves per slot)

typedef int64_t i64x1;
typedef float v4f __attribute__((ext_vector_type(4)));

struct Bq8Args {
    const int8_t *q;
    const float *d_a;
    const int8_t *w;
    const uint16_t *d_w;
    int b, N, K, m, L;
    uint16_t *y;
    float *part;  // [split, b, N] subtree roots when split > 1
    int split;
    int ks;       // waves per tile slot (a power of two)
    int units;    // units per wave slice (a power of two)
    int ntiles;
    int nch;      // chunks per tile per wave
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

__host__ __device__ constexpr int act_stride(int K) { return (K + kUnit - 1) / kUnit * kUnit + 16; }
__host__ __device__ constexpr int da_stride(int m) { return (m + 7) / 8 * 8 + 4; }  // floats

template <int U>
struct QChunk {
    v4i w[U][4];        // unit u, load i: rows 4 i + l / 16, bytes 16 (l % 16)
    uint32_t dw[U][2];  // unit u: fp16 scale of (row v / 8, block v % 8), v = l and 64 + l
};

// Insert the root of unit i of an aligned power-of-two range into a binary
// carry stack (one per row held by the lane); after the range's last unit the
// returned value is the root of the whole range.
template <int LV>
__device__ __forceinline__ v4f carry_insert(v4f (&stk)[LV], int i, v4f v) {
    bool open = true;
#pragma unroll
    for (int l = 0; l < LV; ++l) {
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

template <int NW, int U, int D, int XB>
__global__ __launch_bounds__(NW * kWave) void k_blockq8_mfvec(Bq8Args a) {
    static_assert(D >= 2 && (U == 1 || U == 2), "ring, chunk of one or two units");
    __shared__ v4f red[2][NW][kWave];
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];  // [NW][kWaveLds], x[b][KP], d_a[b][DAS]
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int ks = a.ks;
    const int slot = wave / ks, kp = wave - slot * ks;
    const int NT = NW / ks;
    const int r = lane & 15, g = lane >> 4;
    const int K = a.K, N = a.N, m = a.m, L = a.L;
    const int s = blockIdx.y;
    const int KP = act_stride(K), DAS = da_stride(m);
    const int units = a.units;
    const int blk0 = (L >= kUnitBlocks ? s * (L / a.split) : 0) + kp * units * kUnitBlocks;  // first block of the slice
    const int gx = static_cast<int>(gridDim.x), bx = static_cast<int>(blockIdx.x);
    const int ngroups = (a.ntiles + NT - 1) / NT;
    const int nch = a.nch;
    const int total = ((ngroups - bx + gx - 1) / gx) * nch;
    int8_t *tt = smem + wave * kWaveLds;
    int8_t *dws = tt + kTBytes;
    int8_t *xs = smem + NW * kWaveLds;
    float *das = reinterpret_cast<float *>(xs + a.b * KP);
    const __amdgpu_buffer_rsrc_t wr = rsrc(a.w, N * K);
    const __amdgpu_buffer_rsrc_t dwr = rsrc(a.d_w, N * m * 2);
    const __amdgpu_buffer_rsrc_t qr = rsrc(a.q, a.b * K);
    const __amdgpu_buffer_rsrc_t dar = rsrc(a.d_a, a.b * m * 4);
    const int tr = min(r, a.b - 1);
    const int8_t *xrow = xs + tr * KP + 8 * g;
    const float *darow = das + tr * DAS;
    const int lrow = lane >> 4, lcol = 16 * (lane & 15);

    auto tile_of = [&](int c) __attribute__((always_inline)) { return (bx + (c / nch) * gx) * NT + slot; };
    auto unit_of = [&](int c, int u) __attribute__((always_inline)) { return (c % nch) * U + u; };
    auto unit_live = [&](int c, int u) __attribute__((always_inline)) {
        const int ui = unit_of(c, u);
        return ui < units && blk0 + ui * kUnitBlocks < m;
    };
    // No branch surrounds a load (such branches make the compiler wait for
    // every load in flight before the data are used): a dead unit, or a chunk
    // past the wave's last one (its tile lies past the last row), reads zeros
    // from out-of-range buffer offsets and is never used.
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
        QChunk<U> ch;
        const int tile = tile_of(c);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = unit_live(c, u);  // uniform
            const int ublk = blk0 + unit_of(c, u) * kUnitBlocks;
            const int k = 32 * ublk + lcol;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = tile * kTileRows + 4 * i + lrow;
                const unsigned lin = static_cast<unsigned>(row) * static_cast<unsigned>(K) + static_cast<unsigned>(k);
                const int off = (live && row < N && k < K) ? static_cast<int>(lin) : kOob;
                ch.w[u][i] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2);  // nt: read once
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int v = 64 * h + lane;
                const int row = tile * kTileRows + (v >> 3), blk = ublk + (v & 7);
                const unsigned dl = 2u * (static_cast<unsigned>(row) * static_cast<unsigned>(m) + static_cast<unsigned>(blk));
                const int off = (live && row < N && blk < m) ? static_cast<int>(dl) : kOob;
                ch.dw[u][h] = __builtin_amdgcn_raw_buffer_load_b16(dwr, off, 0, 0);
            }
        }
        return ch;
    };

    // Activations and their block scales go out first (vector memory loads
    // return in issue order), then the prologue weight chunks.
    constexpr int NTH = NW * kWave;
    const int tid = static_cast<int>(threadIdx.x);
    const int kv = K / 16;
    const int nv = a.b * kv;      // 16-byte activation vectors
    const int nd = a.b * m;       // block scales
    v4i xa[XB];
    float da[XB];
#pragma unroll
    for (int j = 0; j < XB; ++j) {
        const int v = j * NTH + tid;
        xa[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, v < nv ? 16 * v : kOob, 0, 0);
        da[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dar, v < nd ? 4 * v : kOob, 0, 0));
    }
    QChunk<U> ring[D];
    // Every wave's activation loads go out before any wave's weight loads:
    // behind the weights (HBM misses) they took 4-7 us to land; with the
    // barrier the call at 4096 -> 4096, b = 9..16 took 10.8-11.1 against
    // 12.4-13.1 us (per-wave timestamps showed the staging shrink from about
    // 9000-15000 to 5000-9600 clocks).
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < D - 1; ++i) ring[i] = load_chunk(i);
    auto put = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < XB; ++j) {
            const int v = base + j * NTH + tid;
            if (v < nv) {
                const int t = v / kv;
                *reinterpret_cast<v4i *>(xs + t * KP + 16 * (v - t * kv)) = xa[j];
            }
            if (v < nd) {
                const int t = v / m;
                das[t * DAS + (v - t * m)] = da[j];
            }
        }
    };
    put(0);
    for (int base = XB * NTH; base < nv || base < nd; base += XB * NTH) {  // only for large b x K
#pragma unroll
        for (int j = 0; j < XB; ++j) {
            const int v = base + j * NTH + tid;
            xa[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, v < nv ? 16 * v : kOob, 0, 0);
            da[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dar, v < nd ? 4 * v : kOob, 0, 0));
        }
        put(base);
    }
    __syncthreads();

    v4f stk[kMaxLevels];
    v4f root = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < total; c0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int c = c0 + i;
            if (c >= total) break;
            ring[(i + D - 1) % D] = load_chunk(c + D - 1);  // past the end: zeros, unused
            // The U units of a chunk are an aligned subtree (U divides the
            // slice, or the slice is one unit): their roots fold pairwise and
            // the chunk root goes into the carry stack.
            v4f ch_root[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ui = unit_of(c, u);
                if (ui >= units) break;  // past the slice (U does not divide it)
                v4f ur = v4f{0.0f, 0.0f, 0.0f, 0.0f};  // a unit made only of padding leaves
                if (blk0 + ui * kUnitBlocks < m) {
                    const int ublk = blk0 + ui * kUnitBlocks;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<v4i *>(tt + (4 * j + lrow) * kTRow + lcol) = ring[i].w[u][j];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        *reinterpret_cast<uint16_t *>(dws + 2 * (64 * h + lane)) =
                            static_cast<uint16_t>(ring[i].dw[u][h]);
                    __builtin_amdgcn_wave_barrier();
                    v4i dwv[4];  // fp16 scales of rows 4 g + e, blocks 0..7 of the unit
#pragma unroll
                    for (int e = 0; e < 4; ++e) dwv[e] = *reinterpret_cast<const v4i *>(dws + 16 * (4 * g + e));
                    const v4f da_lo = *reinterpret_cast<const v4f *>(darow + ublk);
                    const v4f da_hi = *reinterpret_cast<const v4f *>(darow + ublk + 4);
                    // Leaf j of rows 4 g .. 4 g + 3 for token l % 16, folded into
                    // the unit's 8-leaf tree as soon as its sibling exists.  Units
                    // past the end of the real blocks (at most one per slice)
                    // take the padded variant; the test is uniform, so it is a
                    // branch around the whole unit, not per leaf.
                    auto leaf = [&](int j, auto padded) __attribute__((always_inline)) {
                        const i64x1 wa = *reinterpret_cast<const i64x1 *>(tt + r * kTRow + 32 * j + 8 * g);
                        const i64x1 xb = *reinterpret_cast<const i64x1 *>(xrow + 32 * ublk + 32 * j);
                        const v4i isum = __builtin_amdgcn_mfma_i32_16x16x32_i8(wa, xb, v4i{0, 0, 0, 0}, 0, 0, 0);
                        const float dav = j < 4 ? da_lo[j] : da_hi[j - 4];
                        v4f p;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t word = static_cast<uint32_t>(dwv[e][j >> 1]);
                            const float dw = fp16_to_f32(static_cast<uint16_t>((j & 1) ? word >> 16 : word & 0xFFFFu));
                            p[e] = (static_cast<float>(isum[e]) * dav) * dw;
                        }
                        if constexpr (decltype(padded)::value) {
                            const int blk = ublk + j;
                            const float pad = blk < L ? 0.0f : -0.0f;
                            if (blk >= m) p = v4f{pad, pad, pad, pad};
                        }
                        return p;
                    };
                    auto unit_tree = [&](auto padded) __attribute__((always_inline)) {
                        const v4f p01 = leaf(0, padded) + leaf(1, padded);
                        const v4f p23 = leaf(2, padded) + leaf(3, padded);
                        const v4f p45 = leaf(4, padded) + leaf(5, padded);
                        const v4f p67 = leaf(6, padded) + leaf(7, padded);
                        return (p01 + p23) + (p45 + p67);
                    };
                    if (ublk + kUnitBlocks <= m)
                        ur = unit_tree(std::false_type{});
                    else
                        ur = unit_tree(std::true_type{});
                    __builtin_amdgcn_wave_barrier();
                }
                ch_root[u] = ur;
            }
            {
                v4f cr = ch_root[0];
                if constexpr (U == 2) {
                    if (units >= 2) cr = ch_root[0] + ch_root[1];
                }
                root = carry_insert(stk, c % nch, cr);
            }
            if (c % nch == nch - 1) {  // tile done: fold the KS wave roots in tree order, epilogue
                if (ks > 1) {
                    const int buf = (c / nch) & 1;
                    red[buf][wave][lane] = root;
                    __syncthreads();
                    if (kp == 0) {
                        v4f st2[4];  // ks <= 8 wave roots
                        for (int j = 0; j < ks; ++j) root = carry_insert(st2, j, red[buf][wave + j][lane]);
                    }
                }
                if (kp == 0 && r < a.b) {
                    const int row0 = tile_of(c) * kTileRows + 4 * g;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = row0 + e;
                        if (row < N) {
                            if (a.split == 1)
                                a.y[static_cast<int64_t>(r) * N + row] = bf16_rne(root[e]);
                            else
                                a.part[(static_cast<int64_t>(s) * a.b + r) * N + row] = root[e];
                        }
                    }
                }
            }
        }
    }
}

template <int NW, int U, int D, int XB>
hipError_t launch_x(const Bq8Args &a, int smem, hipStream_t st) {
    const int NT = NW / a.ks;
    const int ngroups = (a.ntiles + NT - 1) / NT;
    const void *fn = reinterpret_cast<const void *>(&k_blockq8_mfvec<NW, U, D, XB>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NW * kWave, smem);
    if (e != hipSuccess) return e;
    const int lds_blk = (smem + static_cast<int>(sizeof(v4f)) * 2 * NW * kWave + 1023) / 1024 * 1024;
    if (per_cu > kMaxLds / lds_blk) per_cu = kMaxLds / lds_blk;
    int grid = (per_cu < 1 ? 1 : per_cu) * device_info().cus / a.split;
    if (grid < 1) grid = 1;
    if (grid > ngroups) grid = ngroups;
    hipLaunchKernelGGL((k_blockq8_mfvec<NW, U, D, XB>), dim3(grid, a.split), dim3(NW * kWave), smem, st, a);
    return hipGetLastError();
}

template <int NW, int U, int D>
hipError_t launch_d(const Bq8Args &a, int smem, hipStream_t st) {
    const int per_thread = (a.b * (a.K / 16) + NW * kWave - 1) / (NW * kWave);
    if (per_thread <= 2) return launch_x<NW, U, D, 2>(a, smem, st);
    if (per_thread <= 4) return launch_x<NW, U, D, 4>(a, smem, st);
    if (per_thread <= 8) return launch_x<NW, U, D, 8>(a, smem, st);
    return launch_x<NW, U, D, 12>(a, smem, st);
}

constexpr int kNW = 8;

int lds_bytes(int b, int K) {
    const int m = K / 32;
    return kNW * kWaveLds + b * act_stride(K) + b * da_stride(m) * 4 + 2 * kNW * kWave * 16;
}

}  // namespace

bool blockq8_mfvec_fits(int b, int N, int K, int split) {
    if (b < 1 || b > 16 || K % 32 != 0) return false;
    if (static_cast<int64_t>(N + 3 * kTileRows) * K >= kOob) return false;
    if (static_cast<int64_t>(N) * (K / 32) * 2 >= kOob) return false;
    // A split subtree must hold whole 8-leaf units (smaller ones: the lane-pair kernel).
    int L = 1;
    while (L < K / 32) L *= 2;
    if (split > 1 && L / split < kUnitBlocks) return false;
    return lds_bytes(b, K) <= kMaxLds;
}

// The tree of one split is cut into KS wave slices of a power-of-two number
// of 8-leaf units; 8 waves per workgroup, KS chosen so that a wave slice
// holds at least two units where the tree allows it.
hipError_t launch_blockq8_mfvec(const int8_t *q, const float *d_a, const int8_t *w, const uint16_t *d_w, int b,
                                int N, int K, uint16_t *y, int split, float *part, hipStream_t st) {
    if (!blockq8_mfvec_fits(b, N, K, split)) return hipErrorInvalidValue;
    Bq8Args a{};
    a.q = q;
    a.d_a = d_a;
    a.w = w;
    a.d_w = d_w;
    a.b = b;
    a.N = N;
    a.K = K;
    a.m = K / 32;
    a.L = 1;
    while (a.L < a.m) a.L *= 2;
    a.y = y;
    a.part = part;
    a.split = split;
    const int sub = a.L >= kUnitBlocks ? a.L / split : kUnitBlocks;  // blocks per split subtree
    const int sub_units = sub >= kUnitBlocks ? sub / kUnitBlocks : 1;
    int ks = kNW;
    while (ks > 1 && sub_units / ks < 2) ks /= 2;
    a.ks = ks;
    a.units = sub_units / ks;
    if (a.units > (1 << (kMaxLevels - 1))) return hipErrorInvalidValue;
    a.ntiles = (N + kTileRows - 1) / kTileRows;
    constexpr int U = 2;
    a.nch = (a.units + U - 1) / U;
    const int smem = lds_bytes(b, K) - 2 * kNW * kWave * 16;
    return launch_d<kNW, U, 2>(a, smem, st);
}

}  // namespace iqd
