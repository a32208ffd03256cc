// Decode / verify attention over a bf16 KV cache in fixed 256-cell chunks,
// batch-invariant by construction.
//
// Sources: "why speculative decoding changed my output", sections "attention"
// and "the bug that waited for position 384" (Fig. 5: the cache was summed in
// chunks spread over an occupancy-chosen number of blocks, so a batched
// query's last chunk could join another block's partial); "My speculative
// decoder got slower", sections "Fusion that lost" (two kernels: 256-token
// chunk partials, then a merge; a one-chunk fast path; chunks counted from
// the tokens present, not the allocation), "Why the decoders disagreed?"
// (slots past a query's position are never read) and "Shipping the 6.4x as
// its own backend" (a merge order is one valid rounding; it must be fixed).
//
// The float recipe (every step depends only on one query row, its position
// p and cells 0..p, never on the batch, the allocation or the grid):
//   qs[d]  = fl(q[d] * scale)
//   s_j    = tree over 16 slices of (fma chain over the slice's 8 dims from +0)
//   chunk c (cells [256c, 256c+256) cut at p):
//     m_c  = max_j s_j,  e_j = E(s_j - m_c),
//     per part k of 64 cells: l_k = sum_j e_j and o_k[d] = sum_j e_j v_j[d]
//     (fma), j increasing from +0 (+0 for an empty part);
//     l_c = (l_0 + l_1) + (l_2 + l_3), o_c likewise
//   merge, c increasing: M = max m_c, w_c = E(m_c - M),
//     L = w_0 l_0, O = w_0 o_0, then L = fma(w_c, l_c, L), O = fma(w_c, o_c, O)
//   out[d] = bf16(O[d] / L)
// E is e^x (x <= 0) from Cody and Waite's reduction and a degree-7 Taylor
// polynomial, all in binary32 operations.  With one chunk the merge returns
// o_0 / l_0 exactly, so the chunk kernel writes that directly.
//
// Layout: one workgroup per (chunk, kv head, group of up to 1, 2, 4 or 8
// query rows); a row is (query token, query head) with the query heads of one
// kv head adjacent.  Wave w of the workgroup owns part w of the chunk (64
// cells): it issues all of that part's key loads before computing its scores,
// and its value loads right after them; the K and V chunk rows are read once
// per workgroup.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kChunk = 256;
constexpr int kD = 128;
constexpr int kXcds = 8;
constexpr int kPart = 64;  // a chunk's sums are formed in four parts of 64 cells, one per wave
constexpr int kParts = 4;
constexpr int kThreads = kWave * kParts;
constexpr int kCB = 2;     // cells per lane that share one read of a query slice (scores)

// e^x for x <= 0, binary32 operations only (see the file header).
__device__ __forceinline__ float attn_exp(float x) {
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e4p-1f;
    const float ln2_lo = 0x1.7f7d1cp-20f;
    float n = __builtin_rintf(x * log2e);
    n = n > 127.0f ? 127.0f : n;
    const float r = (x - n * ln2_hi) - n * ln2_lo;
    float p = 0x1.a01a02p-13f;
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float two_n = __uint_as_float(static_cast<uint32_t>(static_cast<int32_t>(n) + 127) << 23);
    return n < -125.0f ? 0.0f : p * two_n;
}


// Buffer resource over [base, base + bytes): loads past the end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void *base, int64_t bytes) {
    const int nr = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nr, 0x00020000);
}

struct AttnArgs {
    const uint16_t *q;  // [b, Hq, 128]
    const uint16_t *k;  // cell * kc + head * kh + d
    const uint16_t *v;
    int64_t kc, kh, vc, vh;
    int b, Hq, Hkv, G, pos0;
    float scale;
    uint16_t *out;      // [b, Hq, 128]
    float *ml;          // [b * Hq][nc][2]: chunk max and sum (rows with >= 2 chunks)
    float *o;           // [b * Hq][nc][128]
    int nc;             // chunks of the longest row
};

// RM: the most query rows a workgroup holds.  The rows of one kv head are
// numbered t * G + g (token t, its query head hk * G + g); a workgroup takes
// RM consecutive ones, so a token's heads may span workgroups.
template <int RM>
__global__ __launch_bounds__(kThreads) void k_attn_chunk(AttnArgs a) {
    // Workgroups are dealt to the XCDs in turn; the row groups of one
    // (chunk, kv head) take consecutive slots of one XCD, so its K and V rows
    // come from that XCD's L2 after the first read.
    const int nrows = a.b * a.G;                // rows of one kv head
    const int nrg = (nrows + RM - 1) / RM;      // row groups
    const int id = blockIdx.x, xcd = id % kXcds, slot = id / kXcds;
    const int tile = (slot / nrg) * kXcds + xcd, rg = slot % nrg;
    if (tile >= a.nc * a.Hkv) return;           // padding slots of the last round
    const int c = tile / a.Hkv, hk = tile % a.Hkv;
    const int rb = rg * RM;                     // first row of this workgroup
    const int R = min(RM, nrows - rb);          // rows of this workgroup
    const int j0 = c * kChunk;
    const int pmax = a.pos0 + (rb + R - 1) / a.G;  // the last row's position
    if (pmax < j0) return;                      // no row reaches this chunk
    const int ncell = min(kChunk, pmax + 1 - j0);
    const int tid = static_cast<int>(threadIdx.x);
    const int wave = tid / kWave, lane = tid % kWave;

    __shared__ __attribute__((aligned(16))) float qs[RM][kD];
    __shared__ __attribute__((aligned(16))) float sc[kChunk][RM];  // scores, then e: [cell][row]
    __shared__ __attribute__((aligned(16))) float op[kParts][RM][kD];
    __shared__ float lp[kParts][RM];
    __shared__ float mrow[RM];

    // Wave w owns part w: cells 64 w .. 64 w + 63 of the chunk, for the scores
    // and for the value sums.  Its query and key loads go out first, all at
    // once, in the order they are used (they return in issue order): the
    // query rows, then the keys (four lanes per cell, lane `sub` holding dims
    // 32 sub .. 32 sub + 31).  The values (lane: dims 2 lane, 2 lane + 1 of
    // each cell) are loaded once the scores are done, so that their 64
    // registers are not held through the score loop: at about 150 VGPRs three
    // workgroups share a CU instead of two, which hides more of each one's
    // load latency (measured on MI355X at Qwen3-8B heads, 32768 cells: b = 1
    // 47 -> 41 us, b = 8 164 -> 120 us, with the score blocking below).
    // Cells past the last one read cell j0 instead (in range, never used).
    // Query element i = tid + kThreads u is row i / kD, dim i % kD.
    constexpr int QU = (RM * kD + kThreads - 1) / kThreads;
    uint16_t qv[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int i = tid + kThreads * u;
        const int r = i / kD < R ? i / kD : 0, d = i % kD;  // rows past R load row 0 (unused)
        const int t = (rb + r) / a.G, hq = hk * a.G + (rb + r) % a.G;
        qv[u] = a.q[(static_cast<int64_t>(t) * a.Hq + hq) * kD + d];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int pbase = kPart * wave;
    const int cs = lane >> 2, sub = lane & 3;
    v4i kw[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int jj = pbase + 16 * st + cs;
        const int j = j0 + (jj < ncell ? jj : 0);
        const v4i *kp = reinterpret_cast<const v4i *>(a.k + static_cast<int64_t>(j) * a.kc + hk * a.kh + 32 * sub);
#pragma unroll
        for (int i = 0; i < 4; ++i) kw[st][i] = kp[i];
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int i = tid + kThreads * u;
        if (i < R * kD) qs[i / kD][i % kD] = bf16_to_f32(qv[u]) * a.scale;
    }
    __syncthreads();

    // Scores: per cell, slice chains of 8 fused multiply-adds, then the tree:
    // two levels in the lane, two across the cell's four lanes.  A lane takes
    // kCB of its cells (16 apart) per pass, so that each query slice read
    // from LDS feeds kCB chains: with one cell per read the LDS, not the
    // vector ALUs, bounds this loop (kCB = 2: 32768 cells, b = 8, 164 -> 146
    // us; kCB = 4 needs 30 more VGPRs and costs a workgroup per CU).
#pragma unroll
    for (int sp = 0; sp < 4 / kCB; ++sp) {
        if (pbase + 16 * kCB * sp >= ncell) break;  // wave-uniform
        float kf[kCB][32];
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t wv = static_cast<uint32_t>(kw[kCB * sp + cb][i][h]);
                    kf[cb][8 * i + 2 * h] = bf16_to_f32(wv & 0xFFFFu);
                    kf[cb][8 * i + 2 * h + 1] = __uint_as_float(wv & 0xFFFF0000u);
                }
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            if (r >= R) break;  // wave-uniform
            const float4 *qr = reinterpret_cast<const float4 *>(&qs[r][32 * sub]);
            float part[kCB][4];
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                const float4 x0 = qr[2 * sl], x1 = qr[2 * sl + 1];
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb) {
                    float acc = __builtin_fmaf(x0.x, kf[cb][8 * sl + 0], 0.0f);
                    acc = __builtin_fmaf(x0.y, kf[cb][8 * sl + 1], acc);
                    acc = __builtin_fmaf(x0.z, kf[cb][8 * sl + 2], acc);
                    acc = __builtin_fmaf(x0.w, kf[cb][8 * sl + 3], acc);
                    acc = __builtin_fmaf(x1.x, kf[cb][8 * sl + 4], acc);
                    acc = __builtin_fmaf(x1.y, kf[cb][8 * sl + 5], acc);
                    acc = __builtin_fmaf(x1.z, kf[cb][8 * sl + 6], acc);
                    acc = __builtin_fmaf(x1.w, kf[cb][8 * sl + 7], acc);
                    part[cb][sl] = acc;
                }
            }
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) {
                const int jj = pbase + 16 * (kCB * sp + cb) + cs;
                float s = (part[cb][0] + part[cb][1]) + (part[cb][2] + part[cb][3]);
                s = s + xor_lane<1>(s);  // slices 0-7 with 8-15 of the pair of lanes
                s = s + xor_lane<2>(s);  // the root
                if (jj < ncell && sub == 0) sc[jj][r] = s;
            }
        }
    }
    // The values, while the other waves finish their scores.  32-bit offsets
    // into a buffer over the chunk's values (cell strides are below 2^22
    // elements, so a chunk spans less than 2^31 bytes).
    uint32_t vw[kPart];
    {
        const __amdgpu_buffer_rsrc_t vr =
            attn_rsrc(a.v + static_cast<int64_t>(j0) * a.vc + hk * a.vh, static_cast<int64_t>(kChunk) * a.vc * 2);
        const uint32_t vcb = static_cast<uint32_t>(a.vc) * 2;
#pragma unroll
        for (int i = 0; i < kPart; ++i) {
            const int jj = pbase + i;
            vw[i] = __builtin_amdgcn_raw_buffer_load_b32(vr, static_cast<uint32_t>(jj < ncell ? jj : 0) * vcb + 4 * lane,
                                                         0, 0);
        }
    }
    __syncthreads();

    // Per row: the chunk maximum over its own cells, then e_j (+0 past them,
    // to the end of the chunk; +0 for rows the workgroup does not hold).
    for (int r = wave; r < RM; r += kParts) {
        const int p = a.pos0 + (rb + r) / a.G;
        const int ncr = r < R ? min(ncell, p + 1 - j0) : 0;  // wave-uniform
        float m = -__builtin_inff();
        for (int i = lane; i < ncr; i += kWave) m = fmaxf(m, sc[i][r]);
        m = fmaxf(m, xor_lane<1>(m));
        m = fmaxf(m, xor_lane<2>(m));
        m = fmaxf(m, xor_lane<4>(m));
        m = fmaxf(m, xor_lane<8>(m));
        m = fmaxf(m, xor_lane<16>(m));
        m = fmaxf(m, xor_lane<32>(m));
        for (int i = lane; i < kChunk; i += kWave) sc[i][r] = i < ncr ? attn_exp(sc[i][r] - m) : 0.0f;
        if (lane == 0) mrow[r] = m;
    }
    __syncthreads();

    // This wave's part: l and o[d] = sums of e_j and e_j v_j[d] over the
    // part's cells in increasing j, from +0.  Cells outer (each value
    // unpacked once), rows inner.  When every row attends the whole part no
    // cell is skipped; otherwise a row's cells past its position leave its
    // sums untouched (a select, so not even the sign of a zero changes).
    {
        int n[RM];
#pragma unroll
        for (int r = 0; r < RM; ++r)
            n[r] = r < R ? min(kPart, min(ncell, a.pos0 + (rb + r) / a.G + 1 - j0) - pbase) : kPart;
        int nmin = kPart;
#pragma unroll
        for (int r = 0; r < RM; ++r) nmin = min(nmin, n[r]);
        float o[RM][2];
#pragma unroll
        for (int r = 0; r < RM; ++r) o[r][0] = o[r][1] = 0.0f;
        // e of cell i for all RM rows (16-byte reads when RM is a multiple of 4)
        auto erow = [&](int i, float (&ev)[RM]) __attribute__((always_inline)) {
            if constexpr (RM % 4 == 0) {
                const float4 *e4 = reinterpret_cast<const float4 *>(&sc[pbase + i][0]);
#pragma unroll
                for (int q4 = 0; q4 < RM / 4; ++q4) {
                    const float4 e = e4[q4];
                    ev[4 * q4 + 0] = e.x;
                    ev[4 * q4 + 1] = e.y;
                    ev[4 * q4 + 2] = e.z;
                    ev[4 * q4 + 3] = e.w;
                }
            } else {
#pragma unroll
                for (int r = 0; r < RM; ++r) ev[r] = sc[pbase + i][r];
            }
        };
        if (nmin == kPart) {
#pragma unroll
            for (int i = 0; i < kPart; ++i) {
                const uint32_t w = vw[i];
                const float v0 = bf16_to_f32(w & 0xFFFFu), v1 = __uint_as_float(w & 0xFFFF0000u);
                float ev[RM];
                erow(i, ev);
#pragma unroll
                for (int r = 0; r < RM; ++r) {
                    o[r][0] = __builtin_fmaf(ev[r], v0, o[r][0]);
                    o[r][1] = __builtin_fmaf(ev[r], v1, o[r][1]);
                }
            }
        } else if (nmin < kPart) {
#pragma unroll
            for (int i = 0; i < kPart; ++i) {
                const uint32_t w = vw[i];
                const float v0 = bf16_to_f32(w & 0xFFFFu), v1 = __uint_as_float(w & 0xFFFF0000u);
                float ev[RM];
                erow(i, ev);
#pragma unroll
                for (int r = 0; r < RM; ++r) {
                    const float x0 = __builtin_fmaf(ev[r], v0, o[r][0]);
                    const float x1 = __builtin_fmaf(ev[r], v1, o[r][1]);
                    o[r][0] = i < n[r] ? x0 : o[r][0];
                    o[r][1] = i < n[r] ? x1 : o[r][1];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r)
            if (r < R) reinterpret_cast<float2 *>(&op[wave][r][0])[lane] = make_float2(o[r][0], o[r][1]);
        if (lane < R) {
            // e is +0 past the row's cells, and l >= +0 throughout: adding those
            // +0 terms leaves l as it is
            float l = 0.0f;
#pragma unroll
            for (int i = 0; i < kPart; ++i) l = l + sc[pbase + i][lane];
            lp[wave][lane] = l;
        }
    }
    __syncthreads();

    // Join the parts, (0 + 1) + (2 + 3), and write: the output itself when the
    // row has one chunk (what the merge would give), else the chunk partial.
    for (int i = tid; i < R * (kD / 2); i += kThreads) {
        const int r = i / (kD / 2), dp = i % (kD / 2);
        const int t = (rb + r) / a.G, hq = hk * a.G + (rb + r) % a.G;
        const int p = a.pos0 + t;
        if (p < j0) continue;  // the row does not reach this chunk
        const float2 o0 = reinterpret_cast<const float2 *>(&op[0][r][0])[dp];
        const float2 o1 = reinterpret_cast<const float2 *>(&op[1][r][0])[dp];
        const float2 o2 = reinterpret_cast<const float2 *>(&op[2][r][0])[dp];
        const float2 o3 = reinterpret_cast<const float2 *>(&op[3][r][0])[dp];
        const float ox = (o0.x + o1.x) + (o2.x + o3.x);
        const float oy = (o0.y + o1.y) + (o2.y + o3.y);
        const float l = (lp[0][r] + lp[1][r]) + (lp[2][r] + lp[3][r]);
        const int64_t row = static_cast<int64_t>(t) * a.Hq + hq;
        if (p < kChunk) {
            const uint32_t packed =
                static_cast<uint32_t>(bf16_rne(ox / l)) | (static_cast<uint32_t>(bf16_rne(oy / l)) << 16);
            reinterpret_cast<uint32_t *>(a.out + row * kD)[dp] = packed;
        } else {
            reinterpret_cast<float2 *>(a.o + (row * a.nc + c) * kD)[dp] = make_float2(ox, oy);
            if (dp == 0) {
                a.ml[(row * a.nc + c) * 2] = mrow[r];
                a.ml[(row * a.nc + c) * 2 + 1] = l;
            }
        }
    }
}

// Merge the chunk partials of every row with two or more chunks, in
// increasing chunk order.  One workgroup of kMergeThreads per row.  The
// maximum is an exact reduction (any order).  The chunks go through LDS in
// windows of kMW: a window's partial values are kMW * kD consecutive floats
// (32 KB), which all the workgroup's threads load at once (4 x 16 bytes per
// thread) with the window's maxima and sums; then threads 0..kD-1 (thread d
// owns dim d) apply the window's chunks in order from LDS while the next
// window's loads are in flight.  Two LDS buffers alternate, one barrier per
// window.  Each row costs about one memory round trip per window, against
// one per kD-thread register window of 28 chunks before (Qwen3-8B heads,
// 32768 cells: 128 chunks, 7.2 us for the merge).
constexpr int kMergeThreads = 512;
constexpr int kMW = 64;
constexpr int kMF4 = kMW * kD / 4 / kMergeThreads;  // 16-byte loads per thread per window
static_assert(kMW * kD / 4 % kMergeThreads == 0, "a window is whole 16-byte loads per thread");
static_assert(kMW <= kMergeThreads && kD <= kMergeThreads, "");

__global__ __launch_bounds__(kMergeThreads) void k_attn_merge(AttnArgs a) {
    const int64_t row = blockIdx.x;
    const int t = static_cast<int>(row / a.Hq);
    const int p = a.pos0 + t;
    const int n = p / kChunk + 1;
    if (n < 2) return;  // uniform over the workgroup
    const int tid = static_cast<int>(threadIdx.x);
    // Row `row`'s partial values: chunk c, dim d at [c * kD + d]; its maxima
    // and sums: (m, l) of chunk c at [2 c], [2 c + 1].  Buffer loads over the
    // row's n chunks read zeros past them, so no load sits behind a branch.
    // The workspace is 16-byte aligned (checked at the boundary), the values
    // start a multiple of 256 bytes into it and a row is nc * 512 bytes, so
    // the 16-byte loads line up.
    const __amdgpu_buffer_rsrc_t orr = attn_rsrc(a.o + row * a.nc * kD, static_cast<int64_t>(n) * kD * 4);
    const __amdgpu_buffer_rsrc_t mlr = attn_rsrc(a.ml + row * a.nc * 2, static_cast<int64_t>(n) * 8);
    __shared__ v4i so[2][kMW * kD / 4];
    __shared__ float2 swl[2][kMW];  // (weight, sum) of each chunk of the window
    __shared__ float sred[kMergeThreads / kWave];

    v4i r[kMF4];
    float rm = 0.0f, rl = 0.0f;
    auto issue = [&](int w0) {
        // Threads past the window's chunks read from an offset past the
        // buffer (zeros, no memory access): a branch around this load would
        // make the compiler wait for every load in flight, the next window's
        // included, before the chain.  It goes out first, so that a wait for
        // it leaves the window's values in flight.
        const int off = tid < kMW ? 8 * (w0 + tid) : 0x7FFFFFF0;
        const uint64_t u = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(mlr, off, 0, 0));
#pragma unroll
        for (int j = 0; j < kMF4; ++j) {
            const int i = tid + j * kMergeThreads;  // 16-byte slot of the window
            r[j] = __builtin_amdgcn_raw_buffer_load_b128(orr, 16 * (w0 * (kD / 4) + i), 0, 0);
        }
        rm = __uint_as_float(static_cast<uint32_t>(u));
        rl = __uint_as_float(static_cast<uint32_t>(u >> 32));
    };

    // The first maxima load goes out before the first window's loads, so the
    // wait for it leaves those in flight.
    const float m0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mlr, 8 * tid, 0, 0));
    issue(0);
    float M = tid < n ? m0 : -__builtin_inff();  // zeros past n must not win
    for (int c0 = kMergeThreads; c0 < n; c0 += kMergeThreads) {
        const float mc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mlr, 8 * (c0 + tid), 0, 0));
        M = c0 + tid < n ? fmaxf(M, mc) : M;
    }
    M = fmaxf(M, xor_lane<1>(M));
    M = fmaxf(M, xor_lane<2>(M));
    M = fmaxf(M, xor_lane<4>(M));
    M = fmaxf(M, xor_lane<8>(M));
    M = fmaxf(M, xor_lane<16>(M));
    M = fmaxf(M, xor_lane<32>(M));
    if (tid % kWave == 0) sred[tid / kWave] = M;
    __syncthreads();
    M = sred[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / kWave; ++w) M = fmaxf(M, sred[w]);

    // From -0: fma(w, x, -0) is w * x bit for bit (signed zeros included),
    // so the first chunk needs no case of its own.
    float L = -0.0f, O = -0.0f;
    int buf = 0;
    for (int w0 = 0; w0 < n; w0 += kMW, buf ^= 1) {
#pragma unroll
        for (int j = 0; j < kMF4; ++j) so[buf][tid + j * kMergeThreads] = r[j];
        if (tid < kMW) swl[buf][tid] = make_float2(attn_exp(rm - M), rl);  // slots past n: unused
        __syncthreads();
        if (w0 + kMW < n) issue(w0 + kMW);
        if (tid < kD) {
            const float *sv = reinterpret_cast<const float *>(&so[buf][0]) + tid;
            const int cn = min(kMW, n - w0);
            int i = 0;
            // Groups of 16 chunks: every LDS read of the group is issued
            // before its chain of fused multiply-adds.
            for (; i + 16 <= cn; i += 16) {
                float2 wl[16];
                float ov[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    wl[u] = swl[buf][i + u];
                    ov[u] = sv[(i + u) * kD];
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    L = __builtin_fmaf(wl[u].x, wl[u].y, L);
                    O = __builtin_fmaf(wl[u].x, ov[u], O);
                }
            }
            for (; i < cn; ++i) {
                const float2 wl = swl[buf][i];
                L = __builtin_fmaf(wl.x, wl.y, L);
                O = __builtin_fmaf(wl.x, sv[i * kD], O);
            }
        }
    }
    if (tid < kD) a.out[row * kD + tid] = bf16_rne(O / L);
}

}  // namespace

int64_t attn_chunks(int64_t b, int64_t pos0) { return (pos0 + b - 1) / kChunk + 1; }

size_t attn_workspace_bytes(int64_t b, int64_t Hq, int64_t pos0) {
    if (pos0 + b - 1 < kChunk) return 0;  // every row has one chunk: no partials
    const int64_t nc = attn_chunks(b, pos0);
    const size_t ml = static_cast<size_t>(b * Hq * nc * 2) * sizeof(float);
    const size_t o = static_cast<size_t>(b * Hq * nc * kD) * sizeof(float);
    return (ml + 255) / 256 * 256 + o;
}

hipError_t launch_attn_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t kc, int64_t kh,
                              int64_t vc, int64_t vh, int b, int Hq, int Hkv, int pos0, float scale, uint16_t *out,
                              void *ws, hipStream_t st) {
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.kc = kc;
    a.kh = kh;
    a.vc = vc;
    a.vh = vh;
    a.b = b;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.pos0 = pos0;
    a.scale = scale;
    a.out = out;
    a.nc = static_cast<int>(attn_chunks(b, pos0));
    const bool merge = pos0 + b - 1 >= kChunk;
    const size_t mlb = static_cast<size_t>(b) * Hq * a.nc * 2 * sizeof(float);
    a.ml = merge ? static_cast<float *>(ws) : nullptr;
    a.o = merge ? reinterpret_cast<float *>(static_cast<char *>(ws) + (mlb + 255) / 256 * 256) : nullptr;
    // Rows per workgroup (every choice gives the same bits), from a sweep of
    // 1, 2, 4, 8 and 16 on MI355X at Qwen3-8B heads (32 query, 8 kv), 1024,
    // 4096 and 32768 cells, b = 1, 2, 4, 8.  Single-token decode (a kv head's
    // rows fit in 4): split them over 2 or 4 workgroups while that leaves no
    // more workgroups than CUs (1024 cells: 1 row, 9.9 us; 4096: 2 rows, 12.9
    // us; 32768: 4 rows, 40.6 us).  More rows: the most rows, at most 8, that
    // still give two workgroups per CU, else one row (1024 cells, b = 2, 4,
    // 8: 10.4 / 11.8 / 13.5 us against 14.7 / 14.8 / 15.1 with 4 rows; 32768
    // cells, b = 8: 8 rows 119 us, 4 rows 137, 16 rows 131; b = 16: 8 rows
    // 23 / 42 / 240 us at 1024 / 4096 / 32768 cells against 16 rows 37 / 45 /
    // 260).
    const int64_t tiles = static_cast<int64_t>(a.nc) * Hkv;
    const int64_t nr = static_cast<int64_t>(b) * a.G;  // rows of one kv head
    const int cus = device_info().cus;
    int rm;
    if (nr <= 4) {
        rm = 4;
        while (rm > 1 && tiles * ((nr + rm / 2 - 1) / (rm / 2)) <= cus) rm /= 2;
    } else {
        rm = 8;
        while (rm > 1 && tiles * ((nr + rm - 1) / rm) < 2 * cus) rm /= 2;
    }
    const int64_t nrg = (nr + rm - 1) / rm;
    const int64_t wgs = (tiles + kXcds - 1) / kXcds * kXcds * nrg;  // every XCD gets whole tiles
    const dim3 grid(static_cast<unsigned>(wgs));
    switch (rm) {
        case 1: hipLaunchKernelGGL(k_attn_chunk<1>, grid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_attn_chunk<2>, grid, dim3(kThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL(k_attn_chunk<4>, grid, dim3(kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL(k_attn_chunk<8>, grid, dim3(kThreads), 0, st, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !merge) return e;
    hipLaunchKernelGGL(k_attn_merge, dim3(static_cast<unsigned>(b) * Hq), dim3(kMergeThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace iqd
