// W8A8 mat-vec on the int8 matrix cores, for decode and verify passes with a
// few tokens (1 <= b <= 16), gfx950.
//
//   y[t, n] = bf16( fl( fl( fl32(acc[t, n]) * s_a[t] ) * s_w[n] ) ),
//   acc[t, n] = sum_k q[t, k] * w[n, k]   (int32, exact)
//
// Sources: "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
// Quantization Scales and the Limits of Tolerance-Based Conformance"
// (Abstract, Fig. 1: the int32 dot product is exact and order-free, so a
// matrix-core kernel, the dot4 mat-vec and the prefill GEMM agree bit for bit;
// Table II: the epilogue).  "why speculative decoding changed my output",
// section "the mat-vec kernel": the stock multi-token path pays for extra
// tokens in registers per column; here the token dimension rides in the
// matrix instruction's N dimension, so 1 and 16 tokens cost the same work.
//
// Mapping (64-lane waves; v_mfma_i32_16x16x64_i8 with A = 16 weight rows,
// B = 16 token columns, both 64 bytes of K per step):
//  * weights are cut into tiles of 16 rows and K into 256-byte units; the KS
//    waves of a tile slot split the units of K, and a workgroup holds NW/KS
//    tile slots, walking tiles with a grid stride;
//  * per unit a wave loads its 16 rows x 256 bytes with four 16-byte buffer
//    loads per lane, each instruction covering 4 rows x 256 contiguous bytes
//    (whole cache lines: instructions that cover 16 rows x 64 bytes stream
//    about 15 % slower on MI355X), writes them to a wave-private LDS tile and
//    reads back the operand layout: lane l = r + 16 g takes row r, bytes
//    64 s + 16 g of the unit for step s.  Rows of the LDS tile are padded by
//    16 bytes, so both the row-wise writes and the transposed reads touch 64
//    distinct banks per quarter-wave;
//  * the activations of all b tokens are staged once per workgroup in LDS
//    (row stride 16 mod 256 bytes, conflict-free for the 16-token fragment
//    read); lane l reads token l % 16 (clamped to b - 1: the columns of
//    tokens >= b are computed and dropped);
//  * weights move through a ring of D register chunks of U units, D - 1
//    chunks in flight while one is multiplied; the weight scales of a tile
//    are fetched with its last chunk;
//  * result register i of lane l is D[4 (l / 16) + i][l % 16]: rows
//    4 (l / 16) .. + 3 of token l % 16.  The KS partial tiles are added
//    through LDS (exact int32) and the epilogue is applied once per output.
#include "act_quant.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kTileRows = 16;
constexpr int kUnit = 256;                  // K bytes per unit
constexpr int kTRow = kUnit + 16;           // padded LDS row of the transposed tile
constexpr int kTBytes = kTileRows * kTRow;  // one wave's staged unit
constexpr int kOob = 0x7FFFFFF0;            // buffer offset that reads zeros (launcher keeps N*K below it)
constexpr int kMaxLds = 160 * 1024;

struct MfvArgs {
    const int8_t *q;     // int8 activations [b, K] (or, fused, nothing)
    const float *s_a;    // their per-token scales [b]
    const uint16_t *x;   // fused: bf16 activations [b, K], quantized by every workgroup
    int8_t *q_out;       // fused, optional: workgroup 0 writes the quantized activations here
    float *s_out;        // fused, optional: and their scales here
    const int8_t *w;
    const float *s_w;
    int b, N, K;
    uint16_t *y;
    uint64_t *keys;  // KEYS: [b][gridDim.x], each workgroup's largest argmax key per token
    int keys_cap;    // KEYS (host side): the most workgroups the keys may cover
    int ntiles;  // ceil(N / 16)
    int nch;     // chunks per tile per wave
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

template <int U>
struct TChunk {
    v4i w[U][4];  // unit u, load i: rows 4 i + l / 16, bytes 16 (l % 16)
    float sw[4];  // weight scales of rows 4 (l / 16) .. + 3 (last chunk of a tile only)
};

__host__ __device__ constexpr int act_stride(int K) { return (K + kUnit - 1) / kUnit * kUnit + 16; }

// KEYS: the workgroup also leaves, per token, the largest argmax key of the
// outputs it wrote (the LM head's argmax reads no logits back).
template <int NW, int KS, int U, int D, int XB, bool WFIRST, bool FUSE, bool KEYS = false>
__global__ __launch_bounds__(NW * kWave) void k_w8a8_mfvec(MfvArgs a) {
    constexpr int NT = NW / KS;  // tile slots per workgroup
    static_assert(NW % KS == 0 && D >= 2, "tile slots and ring");
    static_assert(!(KEYS && FUSE), "argmax keys with the plain mat-vec only");
    __shared__ v4i red[KS > 1 ? 2 : 1][KS > 1 ? NW : 1][kWave];
    __shared__ uint64_t kb[KEYS ? 16 : 1];
    if constexpr (KEYS) {
        if (threadIdx.x < 16) kb[threadIdx.x] = 0;  // ordered before use by the barrier ahead of the main loop
    }
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];  // [NW][kTBytes], then x[b][KP]
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int slot = wave / KS, kp = wave - slot * KS;
    const int r = lane & 15, g = lane >> 4;
    const int K = a.K, N = a.N;
    const int nku = (K + kUnit - 1) / kUnit;
    const int KP = act_stride(K);
    const int u0 = kp * nku / KS, u1 = (kp + 1) * nku / KS;
    const int kend = min(kUnit * u1, K);
    const int gx = static_cast<int>(gridDim.x), bx = static_cast<int>(blockIdx.x);
    const int ngroups = (a.ntiles + NT - 1) / NT;
    const int nch = a.nch;
    const int total = ((ngroups - bx + gx - 1) / gx) * nch;  // uniform over the workgroup
    int8_t *tt = smem + wave * kTBytes;
    int8_t *xs = smem + NW * kTBytes;
    const __amdgpu_buffer_rsrc_t wr = rsrc(a.w, N * K);
    const __amdgpu_buffer_rsrc_t qr = rsrc(a.q, a.b * K);
    const __amdgpu_buffer_rsrc_t swr = rsrc(a.s_w, N * 4);
    const __amdgpu_buffer_rsrc_t sar = rsrc(a.s_a, a.b * 4);
    const int8_t *xrow = xs + min(r, a.b - 1) * KP + 16 * g;
    const int lrow = lane >> 4, lcol = 16 * (lane & 15);

    auto tile_of = [&](int c) __attribute__((always_inline)) { return (bx + (c / nch) * gx) * NT + slot; };
    // Chunk c of this wave.  In the main loop, dead chunks (c >= total) and
    // the scales of all but a tile's last chunk are skipped with uniform
    // branches: an out-of-range buffer load reads no memory but costs the
    // address unit as much as a real one.  The prologue chunks are all live
    // (the launcher keeps D - 1 <= chunks per tile) and load their scales
    // unconditionally (out of range unless the tile's last chunk), so that the
    // prologue's loads form a straight line whose wait counts are exact.
    auto load_chunk = [&](int c, bool prologue) __attribute__((always_inline)) {
        TChunk<U> ch;
        const int tile = tile_of(c);
        const int ub = u0 + (c % nch) * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kUnit * (ub + u) + lcol;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = tile * kTileRows + 4 * i + lrow;
                const unsigned lin = static_cast<unsigned>(row) * static_cast<unsigned>(K) + static_cast<unsigned>(k);
                const int off = (row < N && k < kend) ? static_cast<int>(lin) : kOob;  // a select, not a branch
                ch.w[u][i] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2);  // nt: read once
            }
        }
        const bool last = c % nch == nch - 1;  // the tile's scales ride with its last chunk
        if (prologue || last) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = last ? (tile * kTileRows + 4 * g + i) * 4 : kOob;
                ch.sw[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(swr, off, 0, 0));
            }
        }
        return ch;
    };

    // Vector memory loads return in issue order, so waiting for a staged
    // activation waits for every load issued before it.  The activations
    // therefore go out ahead of the prologue weight chunks (all of them, or
    // all but the first with WFIRST), XB 16-byte vectors per thread (the
    // launcher sizes XB to cover all b x K bytes when it can), and are
    // written to LDS while the later weight chunks are still in flight.
    constexpr int NTH = NW * kWave;
    const int tid = static_cast<int>(threadIdx.x);
    TChunk<U> ring[D];  // chunk c lives in ring[c % D]
    v4i xa[XB];
    float sa;
    if constexpr (!FUSE) {
        const int kv = K / 16;
        const int nv = a.b * kv;
        if constexpr (WFIRST) ring[0] = load_chunk(0, true);
#pragma unroll
        for (int j = 0; j < XB; ++j) {
            const int v = j * NTH + tid;
            xa[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, v < nv ? 16 * v : kOob, 0, 0);
        }
#pragma unroll
        for (int i = WFIRST ? 1 : 0; i < D - 1; ++i) ring[i] = load_chunk(i, true);
        // Lanes past the end store to their wave's transpose tile (rewritten
        // before it is read), so that the store, and the load feeding it,
        // stay unconditional and in issue order.
        auto put = [&](int base) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < XB; ++j) {
                const int v = base + j * NTH + tid;
                const int t = v < nv ? v / kv : 0;
                int8_t *dst = v < nv ? xs + t * KP + 16 * (v - t * kv) : tt + 16 * lane;
                *reinterpret_cast<v4i *>(dst) = xa[j];
            }
        };
        // The token scale is needed only by the epilogue: loaded behind the
        // prologue so that no prologue wait depends on it.
        sa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sar, r * 4, 0, 0));
        put(0);
        for (int base = XB * NTH; base < nv; base += XB * NTH) {  // only when b x K exceeds one batch
#pragma unroll
            for (int j = 0; j < XB; ++j) {
                const int v = base + j * NTH + tid;
                xa[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, v < nv ? 16 * v : kOob, 0, 0);
            }
            put(base);
        }
    } else {
        // Fused quantization: every workgroup reads the bf16 activations
        // (16-byte vectors of 8 values), forms the per-token absmax through
        // LDS, and writes the int8 codes of all b tokens into its staging
        // area; workgroup 0 also writes them (and the scales) out if asked.
        // The activations go out ahead of the weight prologue, so that the
        // quantization runs while the first weight chunks are in flight.
        __shared__ uint32_t amx[16];
        __shared__ float ssc[16], src[16];
        const int kvx = K / 8;  // vectors per token row
        const int nvx = a.b * kvx;
        const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, a.b * K * 2);
        // Vector base + j * NTH + tid lies in token row t at position p; both
        // advance by a constant per j, so one division per thread and batch
        // serves every vector.
        const int step_t = NTH / kvx, step_p = NTH - step_t * kvx;
        auto advance = [&](int &t, int &p) __attribute__((always_inline)) {
            p += step_p;
            t += step_t;
            const bool wrap = p >= kvx;
            p = wrap ? p - kvx : p;
            t = wrap ? t + 1 : t;
        };
        auto load_x = [&](int base) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < XB; ++j) {
                const int v = base + j * NTH + tid;
                xa[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, v < nvx ? 16 * v : kOob, 0, 0);
            }
        };
        load_x(0);
#pragma unroll
        for (int i = 0; i < D - 1; ++i) ring[i] = load_chunk(i, true);
        if (tid < 16) amx[tid] = 0u;
        __syncthreads();
        // When a token row is a whole number of 64-vector spans, the 64 vectors
        // of a wave instruction share one token: one maximum per vector over
        // the wave (lane exchanges, the XB reductions interleaved), one LDS
        // atomic per wave.  Other rows: one atomic per lane.  (|x| >= 0, so
        // float bits order as the values.)
        auto fold_max = [&](int base) __attribute__((always_inline)) {
            const int v0 = base + tid;
            int t = v0 / kvx, p = v0 - t * kvx;
            float m[XB];
            int tj[XB];
#pragma unroll
            for (int j = 0; j < XB; ++j) {
                m[j] = base + j * NTH + tid < nvx ? act_amax8(xa[j]) : 0.0f;
                tj[j] = t;
                advance(t, p);
            }
            if (kvx % kWave == 0) {
#pragma unroll
                for (int j = 0; j < XB; ++j) m[j] = fmaxf(m[j], xor_lane<1>(m[j]));
#pragma unroll
                for (int j = 0; j < XB; ++j) m[j] = fmaxf(m[j], xor_lane<2>(m[j]));
#pragma unroll
                for (int j = 0; j < XB; ++j) m[j] = fmaxf(m[j], xor_lane<4>(m[j]));
#pragma unroll
                for (int j = 0; j < XB; ++j) m[j] = fmaxf(m[j], xor_lane<8>(m[j]));
#pragma unroll
                for (int j = 0; j < XB; ++j) m[j] = fmaxf(m[j], xor_lane<16>(m[j]));
#pragma unroll
                for (int j = 0; j < XB; ++j) m[j] = fmaxf(m[j], xor_lane<32>(m[j]));
                if (lane == 0) {
#pragma unroll
                    for (int j = 0; j < XB; ++j)
                        if (base + j * NTH + tid < nvx) atomicMax(&amx[tj[j]], __float_as_uint(m[j]));
                }
            } else {
#pragma unroll
                for (int j = 0; j < XB; ++j)
                    if (base + j * NTH + tid < nvx) atomicMax(&amx[tj[j]], __float_as_uint(m[j]));
            }
        };
        fold_max(0);
        const bool multi = nvx > XB * NTH;  // rare: b x K exceeds one batch, x is read twice
        for (int base = XB * NTH; base < nvx; base += XB * NTH) {
            load_x(base);
            fold_max(base);
        }
        __syncthreads();
        if (tid < a.b) {
            const float sc = __uint_as_float(amx[tid]) / 127.0f;  // the quantizer's scale, IEEE division
            ssc[tid] = sc;
            src[tid] = 1.0f / sc;
        }
        __syncthreads();
        const bool out = bx == 0 && a.q_out != nullptr;
        auto put_q = [&](int base) __attribute__((always_inline)) {
            const int v0 = base + tid;
            int t = v0 / kvx, p = v0 - t * kvx;
#pragma unroll
            for (int j = 0; j < XB; ++j) {
                const int v = base + j * NTH + tid;
                if (v < nvx) {
                    const float rc = src[t];
                    const uint2 q8 = act_quant8(xa[j], ssc[t], rc, __builtin_isfinite(rc));
                    *reinterpret_cast<uint2 *>(xs + t * KP + 8 * p) = q8;
                    if (out) *reinterpret_cast<uint2 *>(a.q_out + 8 * static_cast<int64_t>(v)) = q8;
                }
                advance(t, p);
            }
        };
        if (multi) {
            for (int base = 0; base < nvx; base += XB * NTH) {
                load_x(base);
                put_q(base);
            }
        } else {
            put_q(0);
        }
        if (bx == 0 && a.s_out != nullptr && tid < a.b) a.s_out[tid] = ssc[tid];
        sa = ssc[min(r, a.b - 1)];
    }
    __syncthreads();
    const int kmax = KP - 16 - 64;  // last in-row start of a 64-byte step (past K the weights are 0)
    v4i acc = v4i{0, 0, 0, 0};
    uint64_t kbest = 0;  // KEYS: the largest key of the outputs this lane wrote
    for (int c0 = 0; c0 < total; c0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int c = c0 + i;
            if (c >= total) break;
            if (c + D - 1 < total) ring[(i + D - 1) % D] = load_chunk(c + D - 1, false);
            const int ub = u0 + (c % nch) * U;
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<v4i *>(tt + (4 * j + lrow) * kTRow + lcol) = ring[i].w[u][j];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const v4i wa = *reinterpret_cast<const v4i *>(tt + r * kTRow + 16 * (4 * s + g));
                    const v4i xb = *reinterpret_cast<const v4i *>(xrow + min(kUnit * (ub + u) + 64 * s, kmax));
                    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa, xb, acc, 0, 0, 0);
                }
                __builtin_amdgcn_wave_barrier();
            }
            if (c % nch == nch - 1) {  // tile done: add the KS partials, epilogue
                if constexpr (KS > 1) {
                    const int buf = (c / nch) & 1;
                    red[buf][wave][lane] = acc;
                    __syncthreads();
                    if (kp == 0) {
#pragma unroll
                        for (int j = 1; j < KS; ++j) acc += red[buf][wave + j][lane];
                    }
                }
                if (kp == 0 && r < a.b) {
                    const int row0 = tile_of(c) * kTileRows + 4 * g;
                    uint16_t *yo = a.y + static_cast<int64_t>(r) * N;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (row0 + e < N) {
                            const uint16_t h = w8a8_epilogue(acc[e], sa, ring[i].sw[e]);
                            yo[row0 + e] = h;
                            if constexpr (KEYS) kbest = umax64(kbest, argmax_key(h, static_cast<uint32_t>(row0 + e)));
                        }
                }
                acc = v4i{0, 0, 0, 0};
            }
        }
    }
    if constexpr (KEYS) {
        __syncthreads();
        if (kbest != 0) atomicMax(reinterpret_cast<unsigned long long *>(&kb[r]), static_cast<unsigned long long>(kbest));
        __syncthreads();
        if (tid < a.b) a.keys[static_cast<int64_t>(tid) * gx + bx] = kb[tid];
    }
}

template <int NW, int KS>
constexpr int lds_bytes_static() {
    return (KS > 1 ? 2 * NW : 1) * kWave * 16 + 256;  // + the fused path's per-token scale slots
}

template <int NW, int KS, int U, int D, int XB, bool WFIRST, bool FUSE, bool KEYS>
hipError_t launch_x(const MfvArgs &a, int grid, int smem, hipStream_t st, int *grid_out) {
    constexpr int NT = NW / KS;
    const int ngroups = (a.ntiles + NT - 1) / NT;
    const void *fn = reinterpret_cast<const void *>(&k_w8a8_mfvec<NW, KS, U, D, XB, WFIRST, FUSE, KEYS>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    if (grid <= 0) {  // one round of resident workgroups: past that, persistent ones (activations staged once each)
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NW * kWave, smem);
        if (e != hipSuccess) return e;
        // LDS is allocated in blocks; count it rounded up to 1 KiB so that a
        // workgroup the runtime would place in a later round is not counted.
        const int lds_blk = (smem + lds_bytes_static<NW, KS>() + 1023) / 1024 * 1024;
        if (per_cu > kMaxLds / lds_blk) per_cu = kMaxLds / lds_blk;
        grid = (per_cu < 1 ? 1 : per_cu) * device_info().cus;
    }
    if (grid > ngroups) grid = ngroups;
    if (KEYS && grid > a.keys_cap) grid = a.keys_cap;  // the kernel walks tiles with a grid stride
    if (grid_out) *grid_out = grid;
    hipLaunchKernelGGL((k_w8a8_mfvec<NW, KS, U, D, XB, WFIRST, FUSE, KEYS>), dim3(grid), dim3(NW * kWave), smem, st,
                       a);
    return hipGetLastError();
}

// Staged 16-byte vectors per thread (int8 codes, or bf16 values when fused):
// the smallest instantiated count that covers all of b x K in one batch (16
// and a loop beyond that).
template <int NW, int KS, int U, int D, bool WFIRST, bool FUSE, bool KEYS>
hipError_t launch_d(const MfvArgs &a, int grid, int smem, hipStream_t st, int *go) {
    const int vec_bytes = FUSE ? 8 : 16;  // K elements per 16-byte vector
    const int per_thread = (a.b * (a.K / vec_bytes) + NW * kWave - 1) / (NW * kWave);
    if constexpr (FUSE) {  // the weights-first order does not apply: the activations always go first
        if (per_thread <= 1) return launch_x<NW, KS, U, D, 1, false, FUSE, KEYS>(a, grid, smem, st, go);
        if (per_thread <= 2) return launch_x<NW, KS, U, D, 2, false, FUSE, KEYS>(a, grid, smem, st, go);
        if (per_thread <= 4) return launch_x<NW, KS, U, D, 4, false, FUSE, KEYS>(a, grid, smem, st, go);
        if (per_thread <= 8) return launch_x<NW, KS, U, D, 8, false, FUSE, KEYS>(a, grid, smem, st, go);
        return launch_x<NW, KS, U, D, 16, false, FUSE, KEYS>(a, grid, smem, st, go);  // past 16: x read twice
    }
    if (per_thread <= 1) return launch_x<NW, KS, U, D, 1, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    if (per_thread <= 2) return launch_x<NW, KS, U, D, 2, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    if (per_thread <= 3) return launch_x<NW, KS, U, D, 3, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    if (per_thread <= 4) return launch_x<NW, KS, U, D, 4, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    if (per_thread <= 6) return launch_x<NW, KS, U, D, 6, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    if (per_thread <= 8) return launch_x<NW, KS, U, D, 8, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    if (per_thread <= 12) return launch_x<NW, KS, U, D, 12, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    return launch_x<NW, KS, U, D, 16, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
}

// The prologue loads D - 1 chunks of the first tile, so D - 1 may not exceed
// the chunks of one tile; shorter K falls back to a ring of two.
template <int NW, int KS, int U, int D, bool WFIRST, bool FUSE, bool KEYS>
hipError_t launch_cfg(MfvArgs a, int grid, hipStream_t st, int *go) {
    a.ntiles = (a.N + kTileRows - 1) / kTileRows;
    const int nku = (a.K + kUnit - 1) / kUnit;
    a.nch = ((nku + KS - 1) / KS + U - 1) / U;
    const int smem = NW * kTBytes + a.b * act_stride(a.K);
    if (smem + lds_bytes_static<NW, KS>() > kMaxLds) return hipErrorInvalidValue;
    if constexpr (D > 2) {
        if (a.nch < D - 1) return launch_d<NW, KS, U, 2, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
    }
    return launch_d<NW, KS, U, D, WFIRST, FUSE, KEYS>(a, grid, smem, st, go);
}

// Launch shapes from a sweep on MI355X over the Qwen3-8B decode layers at
// b = 2..16 (the results are the same for every shape):
//  * up to 256 tiles of 16 rows (N <= 4096): one tile per 8-wave workgroup,
//    K split 8 ways, activations loaded ahead of the weights;
//  * up to 512 tiles: one tile per 4-wave workgroup, K split 4 ways, the
//    first weight chunk ahead of the activations; for b > 8 two tile slots
//    per 8-wave workgroup on a persistent grid;
//  * more tiles: two tile slots per 4-wave workgroup, K split 2 ways, the
//    first weight chunk first; for b > 12 two slots of 4 waves each.
struct Pick {
    int nw, ks;  // for the LDS estimate
    int id;
};

Pick pick(int b, int N, int K) {
    const int ntiles = (N + kTileRows - 1) / kTileRows;
    if (ntiles <= 256) return K > 8192 ? Pick{8, 8, 1} : Pick{8, 8, 0};
    // 257-512 tiles: the 4-wave, 4-way K split for few tokens (tuned at
    // 4096 -> 6144); from b = 4 with K > 4096 the persistent 8-wave grid
    // (measured at Qwen3-14B o, qkv and down, 5120 <= K <= 17408: b = 4
    // 9.10 / 9.67 / 24.8 -> 8.36 / 9.54 / 20.3 us).
    if (ntiles <= 512) return b > 8 || (b >= 4 && K > 4096) ? Pick{8, 4, 3} : Pick{4, 4, 2};
    return b > 12 ? Pick{8, 4, 5} : Pick{4, 2, 4};
}

template <bool FUSE, bool KEYS = false>
hipError_t launch_pick(const Pick &p, const MfvArgs &a, hipStream_t st, int *go = nullptr) {
    switch (p.id) {
        case 0: return launch_cfg<8, 8, 1, 2, false, FUSE, KEYS>(a, 0, st, go);
        case 1: return launch_cfg<8, 8, 2, 2, false, FUSE, KEYS>(a, 0, st, go);
        case 2: return launch_cfg<4, 4, 2, 2, true, FUSE, KEYS>(a, 0, st, go);
        case 3: return launch_cfg<8, 4, 2, 3, false, FUSE, KEYS>(a, device_info().cus, st, go);
        case 4: return launch_cfg<4, 2, 2, 2, true, FUSE, KEYS>(a, 0, st, go);
        case 5: return launch_cfg<8, 4, 2, 3, true, FUSE, KEYS>(a, 0, st, go);
    }
    return hipErrorInvalidValue;
}

int lds_need(const Pick &p, int b, int K) {
    return p.nw * kTBytes + b * act_stride(K) + (p.ks > 1 ? 2 * p.nw : 1) * kWave * 16 + 256;
}

}  // namespace

bool w8a8_mfvec_fits(int b, int N, int K) {
    if (b < 1 || b > 16) return false;
    // 32-bit buffer offsets: rows up to N + 47 (padding tiles of the last
    // workgroup) times K must stay below the out-of-range marker.
    if (static_cast<int64_t>(N + 48) * K >= kOob) return false;
    return lds_need(pick(b, N, K), b, K) <= kMaxLds;
}

hipError_t launch_w8a8_mfvec(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N,
                             int K, uint16_t *y, hipStream_t st) {
    if (!w8a8_mfvec_fits(b, N, K)) return hipErrorInvalidValue;
    MfvArgs a{};
    a.q = q;
    a.s_a = s_a;
    a.w = w;
    a.s_w = s_w;
    a.b = b;
    a.N = N;
    a.K = K;
    a.y = y;
    return launch_pick<false>(pick(b, N, K), a, st);
}

hipError_t launch_w8a8_mfvec_keys(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N,
                                  int K, uint16_t *y, uint64_t *keys, int keys_cap, int *grid, hipStream_t st) {
    if (!w8a8_mfvec_fits(b, N, K)) return hipErrorInvalidValue;
    MfvArgs a{};
    a.q = q;
    a.s_a = s_a;
    a.w = w;
    a.s_w = s_w;
    a.b = b;
    a.N = N;
    a.K = K;
    a.y = y;
    a.keys = keys;
    a.keys_cap = keys_cap;
    return launch_pick<false, true>(pick(b, N, K), a, st, grid);
}

// Every workgroup repeats the quantization of all b x K activations, while
// its first weight chunks are in flight; that pays while the work is small
// next to the workgroup's weights.  Measured on MI355X on the Qwen3-8B layers
// (fused call against the quantize kernel + mat-vec, b = 1..8): the fused
// kernel wins up to b = 4 with one tile per 8-wave workgroup (N <= 4096,
// K <= 8192) and with many tiles (N > 8192), up to b = 2 for K > 8192 and
// for 257..512 tiles, and loses beyond (at b = 8 by 1.2-13 us).  Past eight
// 16-byte vectors per thread the staging needs a second batch, which never
// paid.  Short rows (b x K <= 8192: at most two 8-value vectors per thread)
// fuse at every b (512 -> 256, b = 5: 5.6 -> 4.3 us).
bool w8a8_mfvec_fused_ok(int b, int N, int K) {
    if (!w8a8_mfvec_fits(b, N, K)) return false;
    const Pick p = pick(b, N, K);
    const int threads = p.nw * kWave;
    if (b * (K / 8) > 8 * threads) return false;
    if (b * K <= 8192) return true;  // a few vectors per thread: cheaper than a kernel boundary at any b
    switch (p.id) {
        case 0:
        case 4: return b <= 4;
        case 1:
        case 2: return b <= 2;
        default: return false;
    }
}

hipError_t launch_w8a8_mfvec_fused(const uint16_t *x, const int8_t *w, const float *s_w, int b, int N, int K,
                                   uint16_t *y, int8_t *q_out, float *s_out, hipStream_t st) {
    if (!w8a8_mfvec_fused_ok(b, N, K)) return hipErrorInvalidValue;
    MfvArgs a{};
    a.x = x;
    a.q_out = q_out;
    a.s_out = s_out;
    a.w = w;
    a.s_w = s_w;
    a.b = b;
    a.N = N;
    a.K = K;
    a.y = y;
    return launch_pick<true>(pick(b, N, K), a, st);
}

}  // namespace iqd
