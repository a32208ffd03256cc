// FP8 (E4M3) W8A8 linear with a fixed summation tree, gfx950.
//
// Sources: "My speculative decoder got slower", sections "The FP8 kernel
// that was secretly FP16" and "A trained drafter and two matmul schedules"
// (projection weights in FP8) and "Two matmul schedules that survived"
// (split-K and the step size move the float rounding points); "Deterministic
// LLM Inference Across GPU Kernels ...", Abstract (FP8 differences between
// implementations grow with the reduction depth).
//
// The format is OCP E4M3 (bias 7, 3 mantissa bits, largest finite 448; the
// gfx950 conversion instructions decode it exactly).  A product of two E4M3
// values is exact in binary32, so only the order of the additions matters;
// it is fixed as: K in groups of 16; a group adds its products in increasing
// k from +0 (a fused multiply-add with an exact product rounds once, like the
// addition); the group sums are the leaves of the canonical tree (zero-padded
// to L = 2^ceil(log2(K/16)) leaves, adjacent pairs level by level); then
// y = bf16(fl(fl(root * s_a) * s_w)).
//
// Mapping (64-lane waves), as in the block-quantized mat-vec: a chunk is 64
// consecutive groups (1 KiB of a row); lane l owns group l of the chunk, one
// 16-byte load per row and per token.  Reduce-scatter steps over lane masks
// 1, 2, ..., 32 are the tree levels 1..6 inside the chunk; chunk roots go
// through a binary carry stack (the same tree built left to right); the waves
// of a workgroup own aligned sub-ranges of chunks, and API splits own aligned
// subtrees folded, with the epilogue, by k_fp8_combine.  Leaves of groups in
// [K/16, L) are +0; lanes beyond L (L < 64) hold -0, the exact identity.
#include "device.hpp"
#include "kernels.hpp"

namespace iqd {
namespace {

constexpr int kF8Waves = 4;
constexpr int kF8Threads = kF8Waves * kWave;
constexpr int kF8MaxLevels = 12;    // chunk-slot tree depth: K/16/64 slots <= 2^12 for K <= 2^22
constexpr int kF8Oob = 0x7FFFFFF0;  // a buffer offset past every range: the load returns zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t f8_rsrc(const void *base, int64_t bytes) {
    const int nr = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : static_cast<int>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nr, 0x00020000);
}

// 16 E4M3 codes (one 16-byte vector, byte i = element i) -> 16 floats.
__device__ __forceinline__ void decode16(const v4i &v, float (&f)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[i], false);  // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[i], true);   // bytes 2, 3
        f[4 * i + 0] = lo[0];
        f[4 * i + 1] = lo[1];
        f[4 * i + 2] = hi[0];
        f[4 * i + 3] = hi[1];
    }
}

struct F8Args {
    const uint8_t *q;
    const float *s_a;
    const uint8_t *w;
    const float *s_w;
    int N, K, G, LG;  // groups G = K / 16, tree leaves LG = 2^ceil(log2 G)
    uint16_t *y;
    float *part;      // [split, B, N] subtree roots when split > 1
    int split;
    int nslots;       // max(1, LG / 64) chunk slots in the whole tree
    int ks;           // waves sharing a row group
    int nsteps;
};

__device__ __forceinline__ float f8_carry_insert(float (&stk)[kF8MaxLevels], int i, float v) {
    bool open = true;
#pragma unroll
    for (int l = 0; l < kF8MaxLevels; ++l) {
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

struct F8Add {
    __device__ float operator()(float a, float b) const { return a + b; }
};

template <int B, int RS, int U>
__global__ __launch_bounds__(kF8Threads) void k_fp8_matvec(F8Args a) {
    __shared__ float red[kF8Waves][kWave];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int s = blockIdx.y;
    const int K = a.K, N = a.N, G = a.G, LG = a.LG;
    const int ks = a.ks;
    const int rg = wave / ks;
    const int kp = wave - rg * ks;
    const int rgs = kF8Waves / ks;
    const int nss = a.nslots / a.split;  // slots per split
    const int nsw = nss / ks;            // slots per wave
    const int slot0 = s * nss + kp * nsw;

    constexpr int NV = RS * B;
    constexpr int NP = pow2_ceil(NV);

    const __amdgpu_buffer_rsrc_t qr = f8_rsrc(a.q, static_cast<int64_t>(B) * K);

    for (int step = blockIdx.x; step < a.nsteps; step += gridDim.x) {
        const int row0 = (step * rgs + rg) * RS;
        // Weights of the RS rows from a buffer based at the first row; rows
        // past N re-read the last row and their results are dropped.
        const int rfirst = min(row0, N - 1);
        const int rlast = min(row0 + RS - 1, N - 1);
        const int nrows = rlast - rfirst + 1;
        const __amdgpu_buffer_rsrc_t wr =
            f8_rsrc(a.w + static_cast<int64_t>(rfirst) * K, static_cast<int64_t>(nrows) * K);
        int roff[RS];
#pragma unroll
        for (int r = 0; r < RS; ++r) roff[r] = min(row0 + r, N - 1) - rfirst;
        float stk[kF8MaxLevels];
#pragma unroll
        for (int l = 0; l < kF8MaxLevels; ++l) stk[l] = 0.0f;
        float root = 0.0f;
        for (int i0 = 0; i0 < nsw; i0 += U) {
            // All loads of U slots go out before any is used, with no branch
            // around them: groups past G (or slots past the wave's range) read
            // zeros from out-of-range offsets.
            v4i wv[U][RS], av[U][B];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = (slot0 + i0 + u) * 64 + lane;  // this lane's group
                const bool live = i0 + u < nsw && g < G;
                const int kb = 16 * g;
#pragma unroll
                for (int r = 0; r < RS; ++r)
                    wv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wr, live ? roff[r] * K + kb : kF8Oob, 0, 2);
#pragma unroll
                for (int t = 0; t < B; ++t)
                    av[u][t] = __builtin_amdgcn_raw_buffer_load_b128(qr, live ? t * K + kb : kF8Oob, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int slot = slot0 + i0 + u;
                if (i0 + u >= nsw) break;  // uniform: past the wave's slots
                const int g = slot * 64 + lane;
                float cr = 0.0f;  // a slot made only of padding leaves
                if (slot * 64 < G) {  // uniform
                    float v[NP];
#pragma unroll
                    for (int i = 0; i < NP; ++i) v[i] = 0.0f;
                    float wf[RS][16];  // each weight vector decoded once, used by every token
#pragma unroll
                    for (int r = 0; r < RS; ++r) decode16(wv[u][r], wf[r]);
#pragma unroll
                    for (int t = 0; t < B; ++t) {
                        float af[16];
                        decode16(av[u][t], af);
#pragma unroll
                        for (int r = 0; r < RS; ++r) {
                            float acc = __builtin_fmaf(af[0], wf[r][0], 0.0f);
#pragma unroll
                            for (int i = 1; i < 16; ++i) acc = __builtin_fmaf(af[i], wf[r][i], acc);
                            v[r * B + t] = acc;
                        }
                    }
                    const float pad = g < LG ? 0.0f : -0.0f;
#pragma unroll
                    for (int i = 0; i < NV; ++i) v[i] = g < G ? v[i] : pad;
                    // tree levels 1..6 inside the chunk: lane masks 1..32
                    cr = rs_chain<1, NP>(v, lane, F8Add());
                }
                root = f8_carry_insert(stk, i0 + u, cr);
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
            if (row < N) {
                if (a.split == 1) {
                    const float u = root * a.s_a[t];
                    a.y[static_cast<int64_t>(t) * N + row] = bf16_rne(u * a.s_w[row]);
                } else {
                    a.part[(static_cast<int64_t>(s) * B + t) * N + row] = root;
                }
            }
        }
        if (ks > 1) __syncthreads();
    }
}

// Top log2(split) tree levels over the split roots, then the epilogue.
__global__ __launch_bounds__(256) void k_fp8_combine(const float *__restrict__ part, const float *__restrict__ s_a,
                                                     const float *__restrict__ s_w, int b, int N, int split,
                                                     uint16_t *__restrict__ y) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = static_cast<int64_t>(b) * N;
    if (i >= total) return;
    float stk[kF8MaxLevels];
#pragma unroll
    for (int l = 0; l < kF8MaxLevels; ++l) stk[l] = 0.0f;
    float root = 0.0f;
    for (int s = 0; s < split; ++s) root = f8_carry_insert(stk, s, part[static_cast<int64_t>(s) * total + i]);
    const float u = root * s_a[i / N];
    y[i] = bf16_rne(u * s_w[i % N]);
}

template <int B, int RS, int U>
hipError_t f8_launch(const F8Args &a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((k_fp8_matvec<B, RS, U>), dim3(grid, a.split), dim3(kF8Threads), 0, st, a);
    return hipGetLastError();
}

template <int B>
hipError_t f8_launch_b(const F8Args &base, hipStream_t st) {
    constexpr int RS = B <= 8 ? 4 : 2;
    F8Args a = base;
    const int row_groups = (a.N + RS - 1) / RS;
    const int target = device_info().cus * 16;
    const int nss = a.nslots / a.split;
    int ks = 1;
    while (ks < kF8Waves && ks * 2 <= nss && static_cast<int64_t>(row_groups) * ks * a.split < target) ks *= 2;
    a.ks = ks;
    const int rows_per_step = (kF8Waves / ks) * RS;
    a.nsteps = (a.N + rows_per_step - 1) / rows_per_step;
    int grid = device_info().cus * 8;
    if (grid > a.nsteps) grid = a.nsteps;
    if constexpr (B == 1) {
        if (nss / ks >= 4) return f8_launch<B, RS, 2>(a, grid, st);
    }
    return f8_launch<B, RS, 1>(a, grid, st);
}

// E4M3 code of |f| (f >= 0, finite) rounded to nearest, ties to the even
// code, saturating at 448: normals by rounding the binary32 significand to 3
// bits (the carry may step the exponent), subnormals (below 2^-6) as
// rint(f * 2^9) steps of 2^-9 (8 steps being the smallest normal, code 8).
__device__ __forceinline__ uint32_t e4m3_mag(float f) {
    if (f >= 448.0f) return 0x7Eu;
    if (f < 0x1p-6f) return static_cast<uint32_t>(__builtin_rintf(f * 512.0f));
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;  // exponent and 3 mantissa bits
    return r - (120u << 3);
}

// One workgroup per token: amax, s = fl(amax / 448), q = e4m3(fl(x / s)).
__global__ __launch_bounds__(256) void k_quant_fp8(const uint16_t *__restrict__ x, int K, uint8_t *__restrict__ q,
                                                   float *__restrict__ s_out) {
    const int t = blockIdx.x;
    const uint16_t *xr = x + static_cast<int64_t>(t) * K;
    uint8_t *qr = q + static_cast<int64_t>(t) * K;
    float m = 0.0f;
    for (int k = threadIdx.x; k < K; k += 256) m = fmaxf(m, fabsf(bf16_to_f32(xr[k])));
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) m = fmaxf(m, shfl_xor(m, mask));
    __shared__ float wmax[4];
    if (lane_id() == 0) wmax[threadIdx.x / kWave] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax / 448.0f;
    if (threadIdx.x == 0) s_out[t] = s;
    for (int k = threadIdx.x; k < K; k += 256) {
        uint32_t c = 0;
        if (s != 0.0f) {
            const float v = bf16_to_f32(xr[k]) / s;
            c = e4m3_mag(fabsf(v)) | (__float_as_uint(v) >> 24 & 0x80u);
        }
        qr[k] = static_cast<uint8_t>(c);
    }
}

}  // namespace

int64_t fp8_tree_leaves(int K) {
    int64_t L = 1;
    while (L < K / 16) L *= 2;
    return L;
}

hipError_t launch_quantize_fp8(const uint16_t *x, int b, int K, uint8_t *q, float *s, hipStream_t st) {
    hipLaunchKernelGGL(k_quant_fp8, dim3(b), dim3(256), 0, st, x, K, q, s);
    return hipGetLastError();
}

hipError_t launch_fp8_matvec(const uint8_t *q, const float *s_a, const uint8_t *w, const float *s_w, int b, int N,
                             int K, uint16_t *y, int split, float *part, hipStream_t st) {
    const int G = K / 16;
    const int LG = static_cast<int>(fp8_tree_leaves(K));
    const int nslots = LG >= 64 ? LG / 64 : 1;
    F8Args a{q, s_a, w, s_w, N, K, G, LG, y, part, split, nslots, 1, 0};
    switch (b) {
        case 1: return f8_launch_b<1>(a, st);
        case 2: return f8_launch_b<2>(a, st);
        case 3: return f8_launch_b<3>(a, st);
        case 4: return f8_launch_b<4>(a, st);
        case 5: return f8_launch_b<5>(a, st);
        case 6: return f8_launch_b<6>(a, st);
        case 7: return f8_launch_b<7>(a, st);
        case 8: return f8_launch_b<8>(a, st);
        case 9: return f8_launch_b<9>(a, st);
        case 10: return f8_launch_b<10>(a, st);
        case 11: return f8_launch_b<11>(a, st);
        case 12: return f8_launch_b<12>(a, st);
        case 13: return f8_launch_b<13>(a, st);
        case 14: return f8_launch_b<14>(a, st);
        case 15: return f8_launch_b<15>(a, st);
        case 16: return f8_launch_b<16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fp8_combine(const float *part, const float *s_a, const float *s_w, int b, int N, int split,
                              uint16_t *y, hipStream_t st) {
    const int64_t total = static_cast<int64_t>(b) * N;
    hipLaunchKernelGGL(k_fp8_combine, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, part, s_a,
                       s_w, b, N, split, y);
    return hipGetLastError();
}

}  // namespace iqd
