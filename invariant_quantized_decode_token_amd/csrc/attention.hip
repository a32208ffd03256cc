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
//     l_c  = sum_j e_j and o_c[d] = sum_j e_j v_j[d] (fma), j increasing from +0
//   merge, c increasing: M = max m_c, w_c = E(m_c - M),
//     L = w_0 l_0, O = w_0 o_0, then L = fma(w_c, l_c, L), O = fma(w_c, o_c, O)
//   out[d] = bf16(O[d] / L)
// E is e^x (x <= 0) from Cody and Waite's reduction and a degree-7 Taylor
// polynomial, all in binary32 operations.  With one chunk the merge returns
// o_0 / l_0 exactly, so the chunk kernel writes that directly.
//
// Layout: one workgroup per (chunk, kv head, group of up to 16 query rows);
// a row is (query token, query head) with the query heads of one kv head
// adjacent.  The K and V chunk rows are read once per workgroup.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kChunk = 256;
constexpr int kD = 128;
constexpr int kRows = 16;  // query rows per workgroup
constexpr int kThreads = 256;

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

struct AttnArgs {
    const uint16_t *q;  // [b, Hq, 128]
    const uint16_t *k;  // cell * kc + head * kh + d
    const uint16_t *v;
    int64_t kc, kh, vc, vh;
    int b, Hq, G, pos0;
    float scale;
    uint16_t *out;      // [b, Hq, 128]
    float *ml;          // [b * Hq][nc][2]: chunk max and sum (rows with >= 2 chunks)
    float *o;           // [b * Hq][nc][128]
    int nc;             // chunks of the longest row
};

__global__ __launch_bounds__(kThreads) void k_attn_chunk(AttnArgs a) {
    const int c = blockIdx.x, hk = blockIdx.y;
    const int bq = kRows / a.G;                 // query tokens per workgroup
    const int t0 = blockIdx.z * bq;
    const int nq = min(bq, a.b - t0);
    const int R = nq * a.G;                     // rows of this workgroup
    const int j0 = c * kChunk;
    const int pmax = a.pos0 + t0 + nq - 1;      // the last row's position
    if (pmax < j0) return;                      // no row reaches this chunk
    const int ncell = min(kChunk, pmax + 1 - j0);
    const int tid = static_cast<int>(threadIdx.x);
    const int wave = tid / kWave, lane = tid % kWave;

    __shared__ __attribute__((aligned(16))) float qs[kRows][kD];
    __shared__ float sc[kRows][kChunk];
    __shared__ float mrow[kRows], lrow[kRows];

    // Row r: token t0 + r / G, query head hk * G + r % G.
    for (int i = tid; i < R * kD; i += kThreads) {
        const int r = i / kD, d = i % kD;
        const int t = t0 + r / a.G, hq = hk * a.G + r % a.G;
        qs[r][d] = bf16_to_f32(a.q[(static_cast<int64_t>(t) * a.Hq + hq) * kD + d]) * a.scale;
    }
    __syncthreads();

    // Scores: four lanes per cell, lane `sub` holding dims 32 sub .. 32 sub + 31
    // (slices 4 sub .. 4 sub + 3); 16 cells per wave and step.  Lanes past the
    // chunk's last cell read cell j0 (in range) and store nothing.
    {
        const int cs = lane >> 2, sub = lane & 3;
        for (int jb = wave * 16; jb < ncell; jb += 4 * 16) {
            const int jj = jb + cs;
            const bool valid = jj < ncell;
            const int j = j0 + (valid ? jj : 0);
            const v4i *kp = reinterpret_cast<const v4i *>(a.k + j * a.kc + hk * a.kh + 32 * sub);
            float kf[32];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4i w = kp[i];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    kf[8 * i + 2 * h] = bf16_to_f32(static_cast<uint32_t>(w[h]) & 0xFFFFu);
                    kf[8 * i + 2 * h + 1] = __uint_as_float(static_cast<uint32_t>(w[h]) & 0xFFFF0000u);
                }
            }
            for (int r = 0; r < R; ++r) {
                const float4 *qr = reinterpret_cast<const float4 *>(&qs[r][32 * sub]);
                float part[4];
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    const float4 x0 = qr[2 * sl], x1 = qr[2 * sl + 1];
                    float acc = __builtin_fmaf(x0.x, kf[8 * sl + 0], 0.0f);
                    acc = __builtin_fmaf(x0.y, kf[8 * sl + 1], acc);
                    acc = __builtin_fmaf(x0.z, kf[8 * sl + 2], acc);
                    acc = __builtin_fmaf(x0.w, kf[8 * sl + 3], acc);
                    acc = __builtin_fmaf(x1.x, kf[8 * sl + 4], acc);
                    acc = __builtin_fmaf(x1.y, kf[8 * sl + 5], acc);
                    acc = __builtin_fmaf(x1.z, kf[8 * sl + 6], acc);
                    acc = __builtin_fmaf(x1.w, kf[8 * sl + 7], acc);
                    part[sl] = acc;
                }
                float s = (part[0] + part[1]) + (part[2] + part[3]);
                s = s + xor_lane<1>(s);  // slices 0-7 with 8-15 of the pair of lanes
                s = s + xor_lane<2>(s);  // the root
                if (valid && sub == 0) sc[r][jj] = s;
            }
        }
    }
    __syncthreads();

    // Per row: the chunk maximum over its own cells, then e_j (0 past them).
    for (int r = wave; r < R; r += 4) {
        const int p = a.pos0 + t0 + r / a.G;
        const int ncr = min(ncell, p + 1 - j0);  // wave-uniform
        if (ncr <= 0) continue;
        float m = -__builtin_inff();
        for (int i = lane; i < ncr; i += kWave) m = fmaxf(m, sc[r][i]);
        m = fmaxf(m, xor_lane<1>(m));
        m = fmaxf(m, xor_lane<2>(m));
        m = fmaxf(m, xor_lane<4>(m));
        m = fmaxf(m, xor_lane<8>(m));
        m = fmaxf(m, xor_lane<16>(m));
        m = fmaxf(m, xor_lane<32>(m));
        for (int i = lane; i < ncell; i += kWave) sc[r][i] = i < ncr ? attn_exp(sc[r][i] - m) : 0.0f;
        if (lane == 0) mrow[r] = m;
    }
    __syncthreads();

    // l_r = sum of e_j in increasing j: one lane per row.
    if (tid < R) {
        const int p = a.pos0 + t0 + tid / a.G;
        const int ncr = min(ncell, p + 1 - j0);
        float l = 0.0f;
        for (int j = 0; j < ncr; ++j) l = l + sc[tid][j];
        lrow[tid] = l;
    }

    // o_r[d] = sum of e_j v_j[d] in increasing j.  Wave w owns rows w, w + 4,
    // w + 8, w + 12; lane owns dims 2 lane, 2 lane + 1.  Whether cell j counts
    // for a row is wave-uniform (a branch, not a select).
    float o[4][2];
    int ncr4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[i][0] = 0.0f;
        o[i][1] = 0.0f;
        const int r = wave + 4 * i;
        ncr4[i] = r < R ? min(ncell, a.pos0 + t0 + r / a.G + 1 - j0) : 0;
    }
    const uint32_t *vp = reinterpret_cast<const uint32_t *>(a.v + static_cast<int64_t>(j0) * a.vc + hk * a.vh) + lane;
    const int64_t vstep = a.vc / 2;  // in 32-bit words
    for (int j = 0; j < ncell; ++j) {
        const uint32_t w = vp[j * vstep];
        const float v0 = bf16_to_f32(w & 0xFFFFu), v1 = __uint_as_float(w & 0xFFFF0000u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (j < ncr4[i]) {
                const float e = sc[wave + 4 * i][j];
                o[i][0] = __builtin_fmaf(e, v0, o[i][0]);
                o[i][1] = __builtin_fmaf(e, v1, o[i][1]);
            }
        }
    }
    __syncthreads();  // lrow

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave + 4 * i;
        if (ncr4[i] <= 0) continue;
        const int t = t0 + r / a.G, hq = hk * a.G + r % a.G;
        const int p = a.pos0 + t;
        const int64_t row = static_cast<int64_t>(t) * a.Hq + hq;
        if (p < kChunk) {  // one chunk: out = o / l, what the merge would give
            const float l = lrow[r];
            const uint32_t packed = static_cast<uint32_t>(bf16_rne(o[i][0] / l)) |
                                    (static_cast<uint32_t>(bf16_rne(o[i][1] / l)) << 16);
            reinterpret_cast<uint32_t *>(a.out + row * kD)[lane] = packed;
        } else {
            float *op = a.o + (row * a.nc + c) * kD;
            reinterpret_cast<float2 *>(op)[lane] = make_float2(o[i][0], o[i][1]);
            if (lane == 0) {
                a.ml[(row * a.nc + c) * 2] = mrow[r];
                a.ml[(row * a.nc + c) * 2 + 1] = lrow[r];
            }
        }
    }
}

// Merge the chunk partials of every row with two or more chunks, in
// increasing chunk order.  One wave per row; lane owns dims 2 lane, +1.
__global__ __launch_bounds__(kWave) void k_attn_merge(AttnArgs a) {
    const int64_t row = blockIdx.x;
    const int t = static_cast<int>(row / a.Hq);
    const int p = a.pos0 + t;
    const int n = p / kChunk + 1;
    if (n < 2) return;
    const int lane = static_cast<int>(threadIdx.x);
    const float *ml = a.ml + row * a.nc * 2;
    const float2 *op = reinterpret_cast<const float2 *>(a.o + row * a.nc * kD) + lane;
    float M = -__builtin_inff();
    for (int c = 0; c < n; ++c) M = fmaxf(M, ml[2 * c]);
    float L, O0, O1;
    {
        const float w = attn_exp(ml[0] - M);
        const float2 oc = op[0];
        L = w * ml[1];
        O0 = w * oc.x;
        O1 = w * oc.y;
    }
    for (int c = 1; c < n; ++c) {
        const float w = attn_exp(ml[2 * c] - M);
        const float2 oc = op[static_cast<int64_t>(c) * (kD / 2)];
        L = __builtin_fmaf(w, ml[2 * c + 1], L);
        O0 = __builtin_fmaf(w, oc.x, O0);
        O1 = __builtin_fmaf(w, oc.y, O1);
    }
    const uint32_t packed =
        static_cast<uint32_t>(bf16_rne(O0 / L)) | (static_cast<uint32_t>(bf16_rne(O1 / L)) << 16);
    reinterpret_cast<uint32_t *>(a.out + row * kD)[lane] = packed;
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
    a.G = Hq / Hkv;
    a.pos0 = pos0;
    a.scale = scale;
    a.out = out;
    a.nc = static_cast<int>(attn_chunks(b, pos0));
    const bool merge = pos0 + b - 1 >= kChunk;
    const size_t mlb = static_cast<size_t>(b) * Hq * a.nc * 2 * sizeof(float);
    a.ml = merge ? static_cast<float *>(ws) : nullptr;
    a.o = merge ? reinterpret_cast<float *>(static_cast<char *>(ws) + (mlb + 255) / 256 * 256) : nullptr;
    const int bq = kRows / a.G;
    const dim3 grid(static_cast<unsigned>(a.nc), static_cast<unsigned>(Hkv), static_cast<unsigned>((b + bq - 1) / bq));
    hipLaunchKernelGGL(k_attn_chunk, grid, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !merge) return e;
    hipLaunchKernelGGL(k_attn_merge, dim3(static_cast<unsigned>(b) * Hq), dim3(kWave), 0, st, a);
    return hipGetLastError();
}

}  // namespace iqd
