// W8A8 mat-vec kernel template and its launcher (internal to libiqd).
// The kernel is described in w8a8_matvec.hip; this header holds the
// template so that every launch configuration shares one definition.
#pragma once

#include "act_quant.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {

struct MvArgs {
    const int8_t *q;
    const float *s_a;
    const uint16_t *x;  // fused quantization: bf16 activations [B, K] (then q and s_a are unused)
    int8_t *q_out;      // fused, optional: workgroup 0 writes the quantized activations here
    float *s_out;       // fused, optional: and their scales here
    const int8_t *w;
    const float *s_w;
    int N, K;
    uint16_t *y;
    int32_t *part;  // [split, B, N] when split > 1
    uint64_t *keys; // KEYS: [B][gridDim.x], each workgroup's largest argmax key per token
    int keys_cap;   // KEYS (host side): the most workgroups the keys may cover
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
    float sw;  // weight scale of the output this lane writes for the chunk's row group
};

// Raw buffer resource over [base, base + bytes): a load whose offset
// (scalar offset + lane offset + immediate) is >= bytes returns 0 without
// touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

constexpr int kAuxStream = 2;  // non-temporal: weights are read exactly once

// XB > 0: the per-token quantization is fused in (split 1, activations in
// LDS): every workgroup loads the bf16 rows (XB 16-byte vectors of 8 values
// per thread, ahead of its first weight chunks), forms each token's absmax
// and quantizes the rows into its LDS activations.
// KEYS (split 1): the workgroup also leaves, per token, the largest argmax
// key of the outputs it wrote (the LM head's argmax reads no logits back).
template <int B, int RS, int U, int NW, int D, bool LDS, int XB = 0, bool KEYS = false>
__global__ __launch_bounds__(NW * kWave) void k_w8a8_matvec(MvArgs a) {
    static_assert(XB == 0 || LDS, "fused quantization stages the activations in LDS");
    static_assert(!KEYS || XB == 0, "argmax keys with the plain mat-vec only");
    __shared__ int32_t red[NW][kWave];
    __shared__ uint64_t kb[KEYS ? B : 1];
    if constexpr (KEYS) {
        if (threadIdx.x < B) kb[threadIdx.x] = 0;  // ordered before use by the barrier at the end
    }
    extern __shared__ v4i act[];  // [B][nvs] activations of this split when LDS
    const int K = a.K, N = a.N;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
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
    static_assert(U * kWave * 16 <= 4096, "chunk offsets must fit the 12-bit immediate");

    // Weight rows get one resource each, ending at this wave's K range, so
    // lanes past v1 read zeros.  The activation resource spans all B rows: a
    // lane past v1 may read another token's bytes (or zeros past the end),
    // which only ever meet zero weights.
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q, B * K);

    auto row0_of = [&](int c) __attribute__((always_inline)) {
        return ((bx + (c / nch) * gx) * rgs + rg) * RS;
    };
    auto voff_of = [&](int c) __attribute__((always_inline)) {
        return 16 * (v0 + (c % nch) * U * kWave + lane);
    };
    // The output this lane writes after the reduction (if any) is fixed by its
    // lane index: token t_out of row r_out of the row group.  Its scales are
    // fetched as soon as the row group is known, so that their latency hides
    // behind the weight stream instead of following it.
    const int idx = reduce_scatter_index<NP>(lane);
    const bool writer = kp == 0 && lane < NP && idx < NV;
    const int r_out = idx / B;
    const int t_out = idx - r_out * B;
    float sa_out = (XB == 0 && writer && a.split == 1) ? a.s_a[t_out] : 0.0f;
    uint64_t kbest = 0;  // KEYS: the largest key of the outputs this lane wrote
    auto scale_of = [&](int c) __attribute__((always_inline)) {
        const int row = min(row0_of(c) + r_out, N - 1);
        return (writer && a.split == 1) ? a.s_w[row] : 0.0f;
    };
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
        WChunk<U, RS> ch;
        ch.sw = scale_of(c);
        const int row0 = row0_of(c);
        const int vo = voff_of(c);
#pragma unroll
        for (int r = 0; r < RS; ++r) {
            const int row = min(row0 + r, N - 1);  // rows past N are computed and dropped
            const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w + static_cast<int64_t>(row) * K, 16 * v1);
#pragma unroll
            for (int u = 0; u < U; ++u)
                ch.v[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wr, vo + u * kWave * 16, 0, kAuxStream);
        }
        return ch;
    };

    int32_t acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = 0;

    auto compute_chunk = [&](const WChunk<U, RS> &ch, int c) __attribute__((always_inline)) {
        const int vo = voff_of(c);
#pragma unroll
        for (int t = 0; t < B; ++t) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                v4i av;
                if constexpr (LDS) {
                    const int v = min(vo / 16 + u * kWave, v1 - 1) - sv0;  // past v1 the weights are 0
                    av = act[t * nvs + v];
                } else {
                    av = __builtin_amdgcn_raw_buffer_load_b128(qr, vo + u * kWave * 16, t * K, 0);
                }
#pragma unroll
                for (int r = 0; r < RS; ++r) acc[r * B + t] = dot16(ch.v[u][r], av, acc[r * B + t]);
            }
        }
    };


    // Finish a row group: reduce across lanes and waves, apply the epilogue.
    auto finish = [&](int c, float sw_out) __attribute__((always_inline)) {
        const int row0 = row0_of(c);
        int32_t val = reduce_scatter<NP>(acc, lane, AddI32());
        if (ks > 1) {
            red[wave][lane] = val;
            __syncthreads();
            if (kp == 0)
                for (int j = 1; j < ks; ++j) val += red[wave + j][lane];
            __syncthreads();
        }
        if (writer) {
            const int row = row0 + r_out;
            if (row < N) {
                if (a.split == 1) {
                    const uint16_t h = w8a8_epilogue(val, sa_out, sw_out);
                    a.y[static_cast<int64_t>(t_out) * N + row] = h;
                    if constexpr (KEYS) kbest = umax64(kbest, argmax_key(h, static_cast<uint32_t>(row)));
                } else
                    a.part[(static_cast<int64_t>(s) * B + t_out) * N + row] = val;
            }
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) acc[i] = 0;
    };

    static_assert(D >= 2, "ring of at least two chunks");
    WChunk<U, RS> ring[D];  // chunk c lives in ring[c % D]; D - 1 chunks stay in flight
    if constexpr (XB > 0) {
        // Fused quantization.  The bf16 rows go out first (vector memory loads
        // return in issue order, so the quantization waits for them alone),
        // then the first weight chunks, which stay in flight meanwhile.
        constexpr int NTH = NW * kWave;
        const int tid = static_cast<int>(threadIdx.x);
        const int kv8 = K / 8;  // 16-byte vectors of 8 values per token row
        const int nv = B * kv8;
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, B * K * 2);
        v4i xa[XB];
#pragma unroll
        for (int j = 0; j < XB; ++j) {
            const int v = j * NTH + tid;
            xa[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, v < nv ? 16 * v : 0x7FFFFFF0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < D - 1; ++i)
            if (i < total) ring[i] = load_chunk(i);
        __shared__ uint32_t amx[B];
        __shared__ float ssc[B], src[B];
        if (tid < B) amx[tid] = 0u;
        __syncthreads();
        // Per-token maximum of |x| (|x| >= 0, so float bits order as the
        // values): per thread, then over the wave, one LDS atomic per wave
        // and token.
        float m[B];
#pragma unroll
        for (int t = 0; t < B; ++t) m[t] = 0.0f;
#pragma unroll
        for (int j = 0; j < XB; ++j) {
            const int v = j * NTH + tid;
            const float mj = v < nv ? act_amax8(xa[j]) : 0.0f;
#pragma unroll
            for (int t = 0; t < B; ++t) m[t] = (v >= t * kv8 && v < (t + 1) * kv8) ? fmaxf(m[t], mj) : m[t];
        }
#pragma unroll
        for (int t = 0; t < B; ++t) {
            m[t] = fmaxf(m[t], xor_lane<1>(m[t]));
            m[t] = fmaxf(m[t], xor_lane<2>(m[t]));
            m[t] = fmaxf(m[t], xor_lane<4>(m[t]));
            m[t] = fmaxf(m[t], xor_lane<8>(m[t]));
            m[t] = fmaxf(m[t], xor_lane<16>(m[t]));
            m[t] = fmaxf(m[t], xor_lane<32>(m[t]));
            if (lane == 0) atomicMax(&amx[t], __float_as_uint(m[t]));
        }
        __syncthreads();
        if (tid < B) {
            const float sc = __uint_as_float(amx[tid]) / 127.0f;  // the quantizer's scale, IEEE division
            ssc[tid] = sc;
            src[tid] = 1.0f / sc;
        }
        __syncthreads();
        int8_t *act8 = reinterpret_cast<int8_t *>(act);  // [B][K]
        const bool out = bx == 0 && a.q_out != nullptr;
#pragma unroll
        for (int j = 0; j < XB; ++j) {
            const int v = j * NTH + tid;
            if (v < nv) {
                const int t = B == 1 ? 0 : v / kv8;
                const float rc = src[t];
                const uint2 q8 = act_quant8(xa[j], ssc[t], rc, __builtin_isfinite(rc));
                *reinterpret_cast<uint2 *>(act8 + 8 * v) = q8;  // token t, bytes 8 (v - t kv8): t K + 8 (v - t kv8)
                if (out) *reinterpret_cast<uint2 *>(a.q_out + 8 * static_cast<int64_t>(v)) = q8;
            }
        }
        if (bx == 0 && a.s_out != nullptr && tid < B) a.s_out[tid] = ssc[tid];
        if (writer) sa_out = ssc[t_out];
        __syncthreads();
    } else {
#pragma unroll
        for (int i = 0; i < D - 1; ++i)
            if (i < total) ring[i] = load_chunk(i);
    }
    if constexpr (LDS && XB == 0) {  // staged after the first weight loads, whose latency it overlaps
        for (int i = threadIdx.x; i < B * nvs; i += NW * kWave) {
            const int t = i / nvs;
            act[i] = __builtin_amdgcn_raw_buffer_load_b128(qr, 16 * (sv0 + i - t * nvs), t * K, 0);
        }
        __syncthreads();
    }
    for (int c0 = 0; c0 < total; c0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int c = c0 + i;
            if (c < total) {
                if (c + D - 1 < total) ring[(i + D - 1) % D] = load_chunk(c + D - 1);
                compute_chunk(ring[i], c);
                if (c % nch == nch - 1) finish(c, ring[i].sw);
            }
        }
    }
    if constexpr (KEYS) {
        __syncthreads();
        if (kbest != 0) atomicMax(reinterpret_cast<unsigned long long *>(&kb[t_out]), static_cast<unsigned long long>(kbest));
        __syncthreads();
        if (threadIdx.x < B) a.keys[static_cast<int64_t>(threadIdx.x) * gx + bx] = kb[threadIdx.x];
    }
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

// Launch k_w8a8_matvec<B, RS, U, NW, D, LDS>.  ks = 0 picks enough
// (row group, K part) units for about 16 waves per CU; grid = 0 gives one
// workgroup per row-group step (with LDS: at most as many workgroups as fit,
// persistent over the steps, so that activations are staged once each).
// KEYS: the grid is capped at a.keys_cap (the kernel is persistent over row
// groups) and *grid_out receives it.
template <int B, int RS, int U, int NW, int D, int XB = 0, bool KEYS = false>
hipError_t mv_launch(MvArgs a, hipStream_t st, int cus, int ks, int grid, bool lds = false, int *grid_out = nullptr) {
    static_assert(XB == 0 || B <= 2, "fused quantization: one or two tokens (the kernel's token test)");
    if (KEYS && a.split != 1) return hipErrorInvalidValue;
    if (XB > 0 && (!lds || a.split != 1)) return hipErrorInvalidValue;
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
    if constexpr (XB == 0) {
        if (!lds) {
            if (grid <= 0 || grid > a.nsteps) grid = a.nsteps;
            if (KEYS && grid > a.keys_cap) grid = a.keys_cap;
            if (grid_out) *grid_out = grid;
            hipLaunchKernelGGL((k_w8a8_matvec<B, RS, U, NW, D, false, 0, KEYS>), dim3(grid, a.split), dim3(NW * kWave),
                               0, st, a);
            return hipGetLastError();
        }
    }
    const size_t smem = static_cast<size_t>(B) * nvs_max * 16;
    const size_t lds_total = smem + static_cast<size_t>(NW) * kWave * 4;
    if (lds_total > 160 * 1024) return hipErrorInvalidValue;
    if (smem > 48 * 1024) {
        hipError_t e =
            hipFuncSetAttribute(reinterpret_cast<const void *>(&k_w8a8_matvec<B, RS, U, NW, D, true, XB, KEYS>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
    }
    if (grid <= 0) {
        int per_cu = static_cast<int>(static_cast<size_t>(160 * 1024) / lds_total);
        const int wave_cap = 32 / NW;
        per_cu = per_cu < 1 ? 1 : (per_cu > wave_cap ? wave_cap : per_cu);
        grid = cus * per_cu;
    }
    if (grid > a.nsteps) grid = a.nsteps;
    if (KEYS && grid > a.keys_cap) grid = a.keys_cap;
    if (grid_out) *grid_out = grid;
    hipLaunchKernelGGL((k_w8a8_matvec<B, RS, U, NW, D, true, XB, KEYS>), dim3(grid, a.split), dim3(NW * kWave), smem,
                       st, a);
    return hipGetLastError();
}

}  // namespace iqd
