// W8A8 mat-vec kernel template and its launcher (internal to libiqd).
// The kernel is described in w8a8_matvec.hip; this header holds the
// template so that every launch configuration shares one definition.
#pragma once

#include "device.hpp"

namespace iqd {

struct MvArgs {
    const int8_t *q;
    const float *s_a;
    const int8_t *w;
    const float *s_w;
    int N, K;
    uint16_t *y;
    int32_t *part;  // [split, B, N] when split > 1
    int split;
    int ks;      // waves sharing one row group along K (divides the wave count)
    int nsteps;  // row-group steps: ceil(N / rows per step)
    int nch;     // chunks per step per wave
};

struct AddI32 {
    __device__ int32_t operator()(int32_t x, int32_t y) const { return x + y; }
};

// One chunk of weights in registers: U vectors per lane for each of RS rows.
template <int U, int RS>
struct WChunk {
    v4i v[U][RS];
};

template <int U, int RS>
__device__ __forceinline__ WChunk<U, RS> mv_load_chunk(const int8_t *__restrict__ w, int K, int N, int row0, int vb,
                                                       int v1) {
    WChunk<U, RS> c;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int vu = vb + u * kWave;
        const bool ok = vu < v1;
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            const int row = min(row0 + r, N - 1);  // rows past N are computed and dropped
            c.v[u][r] = zero16();
            if (ok) c.v[u][r] = load_stream16(w + static_cast<int64_t>(row) * K + 16 * vu);
        }
    }
    return c;
}

// acc[r * B + t] += <weight chunk row r, token t>, tokens outermost so that
// one activation vector is live at a time.
template <int B, int U, int RS, int NP, bool LDS>
__device__ __forceinline__ void mv_compute_chunk(int32_t (&acc)[NP], const WChunk<U, RS> &c, const v4i *act,
                                                 int nvs, int sv0, const int8_t *__restrict__ q, int K, int vb,
                                                 int v1) {
#pragma unroll
    for (int t = 0; t < B; ++t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vu = min(vb + u * kWave, v1 - 1);  // weights are 0 past v1
            const v4i av = LDS ? act[t * nvs + (vu - sv0)] : load16(q + static_cast<int64_t>(t) * K + 16 * vu);
#pragma unroll
            for (int r = 0; r < RS; ++r) acc[r * B + t] = dot16(c.v[u][r], av, acc[r * B + t]);
        }
    }
}

template <int B, int RS, int U, int NW, int D, bool LDS>
__global__ __launch_bounds__(NW * kWave) void k_w8a8_matvec(MvArgs a) {
    extern __shared__ v4i smem[];
    const int K = a.K, N = a.N;
    const int lane = lane_id();
    const int wave = static_cast<int>(threadIdx.x) / kWave;
    const int s = blockIdx.y;
    const int kvec = K / 16;
    const int sv0 = s * kvec / a.split;
    const int sv1 = (s + 1) * kvec / a.split;
    const int nvs = sv1 - sv0;
    const int ks = a.ks;
    const int rg = wave / ks;
    const int kp = wave - rg * ks;
    const int rgs = NW / ks;
    const int v0 = sv0 + kp * nvs / ks;  // non-empty: the launcher keeps ks <= nvs
    const int v1 = sv0 + (kp + 1) * nvs / ks;
    const int nch = a.nch;
    const int gx = static_cast<int>(gridDim.x);
    const int bx = static_cast<int>(blockIdx.x);
    const int nst = (a.nsteps - bx + gx - 1) / gx;
    const int total = nst * nch;  // chunks this wave walks; the same for every wave of the workgroup

    constexpr int NV = RS * B;
    constexpr int NP = pow2_ceil(NV);
    static_assert(NP <= kWave, "one reduced value per lane at most");

    v4i *act = smem;                                                           // [B][nvs] when LDS
    int32_t *red = reinterpret_cast<int32_t *>(smem + (LDS ? B * nvs : 0));  // [NW][64]

    // chunk c: row group of step (c / nch), lane vector base of K chunk (c % nch)
#define IQD_MV_ROW0(c) ((((bx + ((c) / nch) * gx) * rgs + rg) * RS))
#define IQD_MV_VB(c) (v0 + ((c) % nch) * U * kWave + lane)

    int32_t acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = 0;

    static_assert(D >= 2, "ring of at least two chunks");
    WChunk<U, RS> ring[D];  // chunk c lives in ring[c % D]; D - 1 chunks stay in flight
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
        if (i < total) ring[i] = mv_load_chunk<U, RS>(a.w, K, N, IQD_MV_ROW0(i), IQD_MV_VB(i), v1);
    if (LDS) {  // after the first weight loads, so that their latency overlaps the staging
        for (int i = threadIdx.x; i < B * nvs; i += NW * kWave) {
            const int t = i / nvs;
            const int v = i - t * nvs;
            act[i] = load16(a.q + static_cast<int64_t>(t) * K + 16 * (sv0 + v));
        }
        __syncthreads();
    }

    // Finish a row group: reduce across lanes and waves, apply the epilogue.
    auto finish = [&](int c) __attribute__((always_inline)) {
        const int row0 = IQD_MV_ROW0(c);
        int32_t val = reduce_scatter<NP>(acc, lane, AddI32());
        const int idx = reduce_scatter_index<NP>(lane);
        if (ks > 1) {
            red[wave * kWave + lane] = val;
            __syncthreads();
            if (kp == 0)
                for (int j = 1; j < ks; ++j) val += red[(wave + j) * kWave + lane];
            __syncthreads();
        }
        if (kp == 0 && lane < NP && idx < NV) {
            const int r = idx / B;
            const int t = idx - r * B;
            const int row = row0 + r;
            if (row < N) {
                if (a.split == 1)
                    a.y[static_cast<int64_t>(t) * N + row] = w8a8_epilogue(val, a.s_a[t], a.s_w[row]);
                else
                    a.part[(static_cast<int64_t>(s) * B + t) * N + row] = val;
            }
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) acc[i] = 0;
    };

    for (int c0 = 0; c0 < total; c0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int c = c0 + i;
            if (c < total) {
                if (c + D - 1 < total)
                    ring[(i + D - 1) % D] =
                        mv_load_chunk<U, RS>(a.w, K, N, IQD_MV_ROW0(c + D - 1), IQD_MV_VB(c + D - 1), v1);
                mv_compute_chunk<B, U, RS, NP, LDS>(acc, ring[i], act, nvs, sv0, a.q, K, IQD_MV_VB(c), v1);
                if (c % nch == nch - 1) finish(c);
            }
        }
    }
#undef IQD_MV_ROW0
#undef IQD_MV_VB
}

// Exact int32 sum of the split partials, then the canonical epilogue.
__global__ __launch_bounds__(256) void k_w8a8_combine(const int32_t *__restrict__ part,
                                                             const float *__restrict__ s_a,
                                                             const float *__restrict__ s_w, int b, int N,
                                                             int split, uint16_t *__restrict__ y) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = static_cast<int64_t>(b) * N;
    if (i >= total) return;
    int32_t acc = 0;
    for (int s = 0; s < split; ++s) acc += part[static_cast<int64_t>(s) * total + i];
    const int t = static_cast<int>(i / N);
    const int n = static_cast<int>(i - static_cast<int64_t>(t) * N);
    y[i] = w8a8_epilogue(acc, s_a[t], s_w[n]);
}

// Launch k_w8a8_matvec<B, RS, U, NW, D, ...>.  ks = 0, lds = -1 and grid = 0
// select the automatic choice: enough (row group, K part) units for about 16
// waves per CU, activations in LDS when they fit, a persistent grid.
template <int B, int RS, int U, int NW, int D>
hipError_t mv_launch(MvArgs a, hipStream_t st, int cus, int lds_limit, int ks, int lds, int grid) {
    const int kvec = a.K / 16;
    const int nvs_min = kvec / a.split;
    const int nvs_max = (kvec + a.split - 1) / a.split;
    const int row_groups = (a.N + RS - 1) / RS;
    if (ks <= 0) {
        ks = 1;
        while (ks < NW && ks * 2 <= nvs_min && static_cast<int64_t>(row_groups) * ks * a.split < cus * 16) ks *= 2;
    }
    if (ks > NW || NW % ks != 0 || ks > nvs_min) return hipErrorInvalidValue;
    a.ks = ks;
    const int rows_per_step = (NW / ks) * RS;
    a.nsteps = (a.N + rows_per_step - 1) / rows_per_step;
    const int per_wave = (nvs_max + ks - 1) / ks;
    a.nch = (per_wave + kWave * U - 1) / (kWave * U);
    const size_t red_bytes = static_cast<size_t>(NW) * kWave * sizeof(int32_t);
    const size_t act_bytes = static_cast<size_t>(B) * nvs_max * 16;
    bool use_lds = lds < 0 ? (act_bytes + red_bytes <= static_cast<size_t>(lds_limit)) : lds != 0;
    if (use_lds && act_bytes + red_bytes > static_cast<size_t>(lds_limit)) return hipErrorInvalidValue;
    const size_t smem = use_lds ? act_bytes + red_bytes : red_bytes;
    if (grid <= 0) {
        int per_cu = use_lds ? static_cast<int>(static_cast<size_t>(160 * 1024) / smem) : 8;
        const int wave_cap = 32 / NW;  // at most 32 waves per CU
        per_cu = per_cu < 1 ? 1 : (per_cu > wave_cap ? wave_cap : per_cu);
        grid = cus * (per_cu > 0 ? per_cu : 1);
    }
    if (grid > a.nsteps) grid = a.nsteps;
    dim3 g(grid, a.split);
    if (use_lds)
        hipLaunchKernelGGL((k_w8a8_matvec<B, RS, U, NW, D, true>), g, dim3(NW * kWave), smem, st, a);
    else
        hipLaunchKernelGGL((k_w8a8_matvec<B, RS, U, NW, D, false>), g, dim3(NW * kWave), smem, st, a);
    return hipGetLastError();
}

}  // namespace iqd
