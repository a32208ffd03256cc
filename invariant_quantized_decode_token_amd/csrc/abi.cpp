// C ABI of libiqd: argument validation and dispatch to the gfx950 kernels.
// Every check runs before any launch, so an error return leaves every
// buffer untouched.  The library allocates nothing and never synchronises.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/iqd.h"
#include "kernels.hpp"

namespace iqd {

const DeviceInfo &device_info() {
    static DeviceInfo infos[64];
    static bool filled[64] = {};
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!filled[dev]) {
        int cus = 0, lds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            infos[dev].cus = cus;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
            lds > 0)
            infos[dev].max_lds = lds;
        int ldsb = 0;
        if (hipDeviceGetAttribute(&ldsb, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && ldsb > 0)
            infos[dev].max_lds_block = ldsb;
        filled[dev] = true;
    }
    return infos[dev];
}

}  // namespace iqd

namespace {

constexpr int64_t kMatvecMaxB = 16;
constexpr int64_t kIntMax = 0x7FFFFFFF;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [p, p + n) and [r, r + m) share a byte.
bool overlap(const void *p, size_t n, const void *r, size_t m) {
    if (!p || !r || n == 0 || m == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + n;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(r), b1 = b0 + m;
    return a0 < b1 && b0 < a1;
}

struct Buf {
    const void *p;
    size_t n;
};

// Outputs must not overlap each other or any input.
bool any_overlap(std::initializer_list<Buf> outs, std::initializer_list<Buf> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (auto i = ins.begin(); i != ins.end(); ++i)
            if (overlap(o->p, o->n, i->p, i->n)) return true;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(o->p, o->n, o2->p, o2->n)) return true;
    }
    return false;
}

bool is_pow2(int64_t v) { return v >= 1 && (v & (v - 1)) == 0; }

int fp8_split_ok(int64_t b, int64_t K, int32_t split) {
    if (split == 1) return IQD_OK;
    int64_t L = 1;
    while (L < K / 16) L *= 2;
    if (b > 16 || !is_pow2(split) || split > IQD_SPLIT_K_MAX || 64 * static_cast<int64_t>(split) > L)
        return IQD_ERR_UNSUPPORTED;
    return IQD_OK;
}

int64_t pow2_ceil(int64_t v) {
    int64_t L = 1;
    while (L < v) L *= 2;
    return L;
}

size_t round16(size_t v) { return (v + 15) / 16 * 16; }

thread_local hipError_t g_last_hip = hipSuccess;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return IQD_OK;
    g_last_hip = e;
    return IQD_ERR_HIP;
}

// A launch is checked with hipGetLastError, which also reports errors that an
// earlier, unrelated runtime call of this thread left behind; clear those
// first so that only our own launches are judged.
void clear_stale_error() { (void)hipGetLastError(); }

int check_shape(int64_t b, int64_t N, int64_t K) {
    if (b < 1 || N < 1 || K < 16 || K % 16 != 0) return IQD_ERR_INVALID;
    if (b > kIntMax || N > kIntMax) return IQD_ERR_INVALID;
    if (K > IQD_K_MAX) return IQD_ERR_RANGE;
    return IQD_OK;
}

// Any b: the int32 partials are exact, so every split gives the same bits.
int w8a8_split_ok(int64_t, int64_t K, int32_t split) {
    if (split == 1) return IQD_OK;
    if (!is_pow2(split) || split > IQD_SPLIT_K_MAX || split > K / 16) return IQD_ERR_UNSUPPORTED;
    return IQD_OK;
}

int blockq8_split_ok(int64_t b, int64_t K, int32_t split) {
    if (split == 1) return IQD_OK;
    const int64_t L = pow2_ceil(K / 32);
    if (b > kMatvecMaxB || !is_pow2(split) || split > IQD_SPLIT_K_MAX || split > L)
        return IQD_ERR_UNSUPPORTED;
    return IQD_OK;
}

size_t ws_w8a8(int64_t b, int64_t N, int32_t split) {
    return split > 1 ? round16(static_cast<size_t>(split) * b * N * 4) : 0;
}
// [q int8 [b, K]][s_a fp32 [b]] for the separate quantize + linear path
size_t ws_w8a8_bf16(int64_t b, int64_t K) { return round16(static_cast<size_t>(b) * K) + round16(static_cast<size_t>(b) * 4); }

// [logits bf16 [b, N] when the caller passes none][argmax keys u64 of one pass
// of at most kMatvecMaxB tokens: one per (token, mat-vec workgroup), at most
// kArgKeysMaxGrid in all]
size_t ws_lm_head_logits(int64_t b, int64_t N, bool have_logits) {
    return have_logits ? 0 : round16(static_cast<size_t>(b) * N * 2);
}
size_t ws_lm_head(int64_t b, int64_t N, bool have_logits) {
    return ws_lm_head_logits(b, N, have_logits) + static_cast<size_t>(iqd::kArgKeysMaxGrid) * 8;
}

}  // namespace

namespace {

int attn_check(int64_t b, int64_t Hq, int64_t Hkv, int64_t D, int64_t pos0) {
    if (b < 1 || b > 65535 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || pos0 < 0 || pos0 + b > (int64_t{1} << 30) ||
        Hq > 65535 || Hkv > 65535)
        return IQD_ERR_INVALID;
    if (D != 128 || Hq / Hkv > 16) return IQD_ERR_UNSUPPORTED;
    // launch sizes: (chunks x kv heads, padded) x row groups and b x Hq workgroups
    const int64_t chunks = (pos0 + b - 1) / 256 + 1;
    if ((chunks * Hkv + 8) * b > kIntMax || b * Hq > kIntMax) return IQD_ERR_UNSUPPORTED;
    return IQD_OK;
}

// Bytes from a cache's base to the end of the last element read.
size_t attn_cache_extent(int64_t cells, int64_t Hkv, int64_t D, int64_t cs, int64_t hs) {
    return static_cast<size_t>((cells - 1) * cs + (Hkv - 1) * hs + D) * 2;
}

}  // namespace

extern "C" {

const char *iqd_status_str(int status) {
    switch (status) {
        case IQD_OK: return "IQD_OK";
        case IQD_ERR_INVALID: return "IQD_ERR_INVALID: bad shape, null pointer, aliasing or group";
        case IQD_ERR_ALIGN: return "IQD_ERR_ALIGN: pointer misaligned";
        case IQD_ERR_RANGE: return "IQD_ERR_RANGE: K above IQD_K_MAX (int32 accumulator bound)";
        case IQD_ERR_UNSUPPORTED: return "IQD_ERR_UNSUPPORTED: split_k or attention shape not supported";
        case IQD_ERR_WORKSPACE: return "IQD_ERR_WORKSPACE: workspace missing or too small";
        case IQD_ERR_HIP: return "IQD_ERR_HIP: HIP runtime call or launch failed";
        default: return "unknown iqd status";
    }
}

const char *iqd_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

size_t iqd_workspace_bytes(int op, int64_t b, int64_t N, int64_t K, int32_t split_k) {
    if (check_shape(b, N, K) != IQD_OK) return 0;
    switch (op) {
        case IQD_OP_W8A8:
            return w8a8_split_ok(b, K, split_k) == IQD_OK ? ws_w8a8(b, N, split_k) : 0;
        case IQD_OP_BLOCKQ8:
            if (K % 32 != 0 || blockq8_split_ok(b, K, split_k) != IQD_OK) return 0;
            return split_k > 1 ? round16(static_cast<size_t>(split_k) * b * N * 4) : 0;
        case IQD_OP_LM_HEAD:
            return ws_lm_head(b, N, false);
        case IQD_OP_W8A8_BF16:
            return ws_w8a8_bf16(b, K);
        case IQD_OP_KQ4:
        case IQD_OP_KQ6:
            if (K % 256 != 0 || blockq8_split_ok(b, K, split_k) != IQD_OK) return 0;
            return split_k > 1 ? round16(static_cast<size_t>(split_k) * b * N * 4) : 0;
        case IQD_OP_FP8:
            return fp8_split_ok(b, K, split_k) == IQD_OK && split_k > 1
                       ? round16(static_cast<size_t>(split_k) * b * N * 4)
                       : 0;
        default:
            return 0;
    }
}

int quantize_activations(const void *x_bf16, int64_t b, int64_t K, int32_t group, int8_t *q, float *scale,
                         void *stream) {
    if (!x_bf16 || !q || !scale) return IQD_ERR_INVALID;
    if (b < 1 || K < 16 || K % 16 != 0 || b > kIntMax || K > kIntMax) return IQD_ERR_INVALID;
    if (group != 0 && group != 32) return IQD_ERR_INVALID;
    if (group == 32 && K % 32 != 0) return IQD_ERR_INVALID;
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(scale, 4)) return IQD_ERR_ALIGN;
    const size_t ns = group == 0 ? static_cast<size_t>(b) : static_cast<size_t>(b) * (K / 32);
    if (any_overlap({{q, static_cast<size_t>(b * K)}, {scale, ns * 4}}, {{x_bf16, static_cast<size_t>(b * K * 2)}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    if (group == 0) return hip_status(iqd::launch_quantize_token(x, static_cast<int>(b), static_cast<int>(K), q, scale, st));
    return hip_status(iqd::launch_quantize_block32(x, static_cast<int>(b), static_cast<int>(K), q, scale, st));
}

int w8a8_linear(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b, int64_t N,
                int64_t K, void *y_bf16, int32_t split_k, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !s_a || !w || !s_w || !y_bf16) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    st = w8a8_split_ok(b, K, split_k);
    if (st != IQD_OK) return st;
    if (!aligned(q, 16) || !aligned(w, 16) || !aligned(s_a, 4) || !aligned(s_w, 4) || !aligned(y_bf16, 2))
        return IQD_ERR_ALIGN;
    const size_t ws = ws_w8a8(b, N, split_k);
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    const size_t ybytes = static_cast<size_t>(b) * N * 2;
    if (any_overlap({{y_bf16, ybytes}, {ws ? workspace : nullptr, ws}},
                    {{q, static_cast<size_t>(b * K)}, {s_a, static_cast<size_t>(b) * 4},
                     {w, static_cast<size_t>(N) * K}, {s_w, static_cast<size_t>(N) * 4}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    const int bi = static_cast<int>(b), Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    int32_t *part = static_cast<int32_t *>(workspace);
    if (b > kMatvecMaxB) return hip_status(iqd::launch_w8a8_mfma(q, s_a, w, s_w, bi, Ni, Ki, y, split_k, part, hs));
    if (split_k == 1)
        return hip_status(iqd::launch_w8a8_matvec(q, s_a, w, s_w, bi, Ni, Ki, y, 1, nullptr, hs));
    hipError_t e = iqd::launch_w8a8_matvec(q, s_a, w, s_w, bi, Ni, Ki, nullptr, split_k, part, hs);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(iqd::launch_w8a8_combine(part, s_a, s_w, bi, Ni, split_k, y, hs));
}

int w8a8_linear_bf16(const void *x_bf16, const int8_t *w, const float *s_w, int64_t b, int64_t N, int64_t K,
                     void *y_bf16, int8_t *q_out, float *s_a_out, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (!x_bf16 || !w || !s_w || !y_bf16) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    if (!aligned(x_bf16, 16) || !aligned(w, 16) || !aligned(s_w, 4) || !aligned(y_bf16, 2) ||
        (q_out && !aligned(q_out, 16)) || (s_a_out && !aligned(s_a_out, 4)))
        return IQD_ERR_ALIGN;
    const bool dot4_fused = b == 1 && K > 4096 && N <= K && iqd::w8a8_matvec_fused_ok(1, static_cast<int>(N),
                                                                                     static_cast<int>(K));
    const bool fused = (b <= kMatvecMaxB && iqd::w8a8_mfvec_fused_ok(static_cast<int>(b), static_cast<int>(N),
                                                                    static_cast<int>(K))) ||
                       dot4_fused;
    const size_t ws = (!fused && (!q_out || !s_a_out)) ? ws_w8a8_bf16(b, K) : 0;
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    const size_t qbytes = static_cast<size_t>(b) * K;
    if (any_overlap({{y_bf16, static_cast<size_t>(b) * N * 2}, {q_out, q_out ? qbytes : 0},
                     {s_a_out, s_a_out ? static_cast<size_t>(b) * 4 : 0}, {ws ? workspace : nullptr, ws}},
                    {{x_bf16, qbytes * 2}, {w, static_cast<size_t>(N) * K}, {s_w, static_cast<size_t>(N) * 4}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint16_t *x = static_cast<const uint16_t *>(x_bf16);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    const int bi = static_cast<int>(b), Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    // One token with rows longer than 4096 and no more rows than K: the dot4
    // kernel with the quantization fused in (Qwen3-8B down at b = 1: 12.8
    // against 13.4 us; Qwen3-14B o: 8.6 against 9.6 us; wider matrices, such
    // as the 14B qkv and gate_up, stay on the matrix-core kernel).
    if (dot4_fused) return hip_status(iqd::launch_w8a8_matvec_fused(x, w, s_w, bi, Ni, Ki, y, q_out, s_a_out, hs));
    if (fused) return hip_status(iqd::launch_w8a8_mfvec_fused(x, w, s_w, bi, Ni, Ki, y, q_out, s_a_out, hs));
    int8_t *q = q_out ? q_out : static_cast<int8_t *>(workspace);
    float *s_a = s_a_out ? s_a_out : reinterpret_cast<float *>(static_cast<char *>(workspace) + round16(qbytes));
    hipError_t e = iqd::launch_quantize_token(x, bi, Ki, q, s_a, hs);
    if (e != hipSuccess) return hip_status(e);
    if (b > kMatvecMaxB) return hip_status(iqd::launch_w8a8_mfma(q, s_a, w, s_w, bi, Ni, Ki, y, 1, nullptr, hs));
    return hip_status(iqd::launch_w8a8_matvec(q, s_a, w, s_w, bi, Ni, Ki, y, 1, nullptr, hs));
}

int blockq8_linear(const int8_t *q, const float *d_a, const int8_t *w, const void *d_w_fp16, int64_t b, int64_t N,
                   int64_t K, void *y_bf16, int32_t split_k, void *workspace, size_t workspace_bytes,
                   void *stream) {
    if (!q || !d_a || !w || !d_w_fp16 || !y_bf16) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    if (K % 32 != 0) return IQD_ERR_INVALID;
    st = blockq8_split_ok(b, K, split_k);
    if (st != IQD_OK) return st;
    if (!aligned(q, 16) || !aligned(w, 16) || !aligned(d_a, 4) || !aligned(d_w_fp16, 2) || !aligned(y_bf16, 2))
        return IQD_ERR_ALIGN;
    const size_t ws = split_k > 1 ? round16(static_cast<size_t>(split_k) * b * N * 4) : 0;
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    const size_t m = static_cast<size_t>(K / 32);
    if (any_overlap({{y_bf16, static_cast<size_t>(b) * N * 2}, {ws ? workspace : nullptr, ws}},
                    {{q, static_cast<size_t>(b * K)}, {d_a, static_cast<size_t>(b) * m * 4},
                     {w, static_cast<size_t>(N) * K}, {d_w_fp16, static_cast<size_t>(N) * m * 2}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    const uint16_t *dw = static_cast<const uint16_t *>(d_w_fp16);
    const int Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    if (split_k == 1) {
        // any b: chunks of at most 16 tokens (each token's row is independent of its chunk)
        for (int64_t t0 = 0; t0 < b; t0 += kMatvecMaxB) {
            const int bc = static_cast<int>(b - t0 < kMatvecMaxB ? b - t0 : kMatvecMaxB);
            hipError_t e = iqd::launch_blockq8_matvec(q + t0 * K, d_a + t0 * m, w, dw, bc, Ni, Ki, y + t0 * N, 1,
                                                      nullptr, hs);
            if (e != hipSuccess) return hip_status(e);
        }
        return IQD_OK;
    }
    float *part = static_cast<float *>(workspace);
    const int bi = static_cast<int>(b);
    hipError_t e = iqd::launch_blockq8_matvec(q, d_a, w, dw, bi, Ni, Ki, nullptr, split_k, part, hs);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(iqd::launch_blockq8_combine(part, bi, Ni, split_k, y, hs));
}

int kq6_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
               const void *d_fp16, int64_t b, int64_t N, int64_t K, void *y_bf16, int32_t split_k,
               void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !d_a || !ql || !qh || !sc || !d_fp16 || !y_bf16) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    if (K % 256 != 0) return IQD_ERR_INVALID;
    st = blockq8_split_ok(b, K, split_k);
    if (st != IQD_OK) return st;
    if (!aligned(q, 16) || !aligned(ql, 16) || !aligned(qh, 16) || !aligned(d_a, 4) || !aligned(d_fp16, 2) ||
        !aligned(y_bf16, 2))
        return IQD_ERR_ALIGN;
    const size_t ws = split_k > 1 ? round16(static_cast<size_t>(split_k) * b * N * 4) : 0;
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    const size_t m = static_cast<size_t>(K / 32), nk = static_cast<size_t>(N) * K;
    if (any_overlap({{y_bf16, static_cast<size_t>(b) * N * 2}, {ws ? workspace : nullptr, ws}},
                    {{q, static_cast<size_t>(b * K)}, {d_a, static_cast<size_t>(b) * m * 4}, {ql, nk / 2}, {qh, nk / 4},
                     {sc, nk / 16}, {d_fp16, nk / 256 * 2}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    const uint16_t *d = static_cast<const uint16_t *>(d_fp16);
    const int Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    if (split_k == 1) {
        // any b: chunks of at most 16 tokens (each token's row is independent of its chunk)
        for (int64_t t0 = 0; t0 < b; t0 += kMatvecMaxB) {
            const int bc = static_cast<int>(b - t0 < kMatvecMaxB ? b - t0 : kMatvecMaxB);
            hipError_t e = iqd::launch_kq6_matvec(q + t0 * K, d_a + t0 * m, ql, qh, sc, d, bc, Ni, Ki, y + t0 * N, 1,
                                                  nullptr, hs);
            if (e != hipSuccess) return hip_status(e);
        }
        return IQD_OK;
    }
    float *part = static_cast<float *>(workspace);
    const int bi = static_cast<int>(b);
    hipError_t e = iqd::launch_kq6_matvec(q, d_a, ql, qh, sc, d, bi, Ni, Ki, nullptr, split_k, part, hs);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(iqd::launch_blockq8_combine(part, bi, Ni, split_k, y, hs));
}

int kq4_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *scm, const void *dm_fp16,
               int64_t b, int64_t N, int64_t K, void *y_bf16, int32_t split_k, void *workspace,
               size_t workspace_bytes, void *stream) {
    if (!q || !d_a || !ql || !scm || !dm_fp16 || !y_bf16) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    if (K % 256 != 0) return IQD_ERR_INVALID;
    st = blockq8_split_ok(b, K, split_k);
    if (st != IQD_OK) return st;
    if (!aligned(q, 16) || !aligned(ql, 16) || !aligned(scm, 2) || !aligned(d_a, 4) || !aligned(dm_fp16, 4) ||
        !aligned(y_bf16, 2))
        return IQD_ERR_ALIGN;
    const size_t ws = split_k > 1 ? round16(static_cast<size_t>(split_k) * b * N * 4) : 0;
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    const size_t m = static_cast<size_t>(K / 32), nk = static_cast<size_t>(N) * K;
    if (any_overlap({{y_bf16, static_cast<size_t>(b) * N * 2}, {ws ? workspace : nullptr, ws}},
                    {{q, static_cast<size_t>(b * K)}, {d_a, static_cast<size_t>(b) * m * 4}, {ql, nk / 2},
                     {scm, nk / 16}, {dm_fp16, nk / 256 * 4}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    const uint16_t *dm = static_cast<const uint16_t *>(dm_fp16);
    const int Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    if (split_k == 1) {
        // any b: chunks of at most 16 tokens (each token's row is independent of its chunk)
        for (int64_t t0 = 0; t0 < b; t0 += kMatvecMaxB) {
            const int bc = static_cast<int>(b - t0 < kMatvecMaxB ? b - t0 : kMatvecMaxB);
            hipError_t e = iqd::launch_kq4_matvec(q + t0 * K, d_a + t0 * m, ql, scm, dm, bc, Ni, Ki, y + t0 * N, 1,
                                                  nullptr, hs);
            if (e != hipSuccess) return hip_status(e);
        }
        return IQD_OK;
    }
    float *part = static_cast<float *>(workspace);
    const int bi = static_cast<int>(b);
    hipError_t e = iqd::launch_kq4_matvec(q, d_a, ql, scm, dm, bi, Ni, Ki, nullptr, split_k, part, hs);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(iqd::launch_blockq8_combine(part, bi, Ni, split_k, y, hs));
}

namespace {

// The LM head after validation of everything but the workspace.
int lm_head_run(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b, int64_t N,
                int64_t K, void *logits_bf16, int32_t *argmax, void *workspace, hipStream_t hs) {
    clear_stale_error();
    uint16_t *logits = static_cast<uint16_t *>(logits_bf16 ? logits_bf16 : workspace);
    uint64_t *keys = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) +
                                                  ws_lm_head_logits(b, N, logits_bf16 != nullptr));
    const int Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    // Per pass of at most kMatvecMaxB tokens: the mat-vec writes the logits
    // and one argmax key per (token, workgroup), at most kArgKeysMaxGrid in
    // all; the fold picks each token's winner.  The next pass reuses the keys
    // after the fold (stream order).
    for (int64_t t0 = 0; t0 < b; t0 += kMatvecMaxB) {
        const int bc = static_cast<int>(b - t0 < kMatvecMaxB ? b - t0 : kMatvecMaxB);
        int nkeys = 0;
        hipError_t e = iqd::launch_w8a8_matvec_keys(q + t0 * K, s_a + t0, w, s_w, bc, Ni, Ki, logits + t0 * N, keys,
                                                    iqd::kArgKeysMaxGrid / bc, &nkeys, hs);
        if (e == hipSuccess) e = iqd::launch_argmax_fold(keys, bc, nkeys, argmax + t0, hs);
        if (e != hipSuccess) return hip_status(e);
    }
    return IQD_OK;
}

int lm_head_check(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b, int64_t N,
                  int64_t K, void *logits_bf16, int32_t *argmax) {
    if (!q || !s_a || !w || !s_w || !argmax) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    if (!aligned(q, 16) || !aligned(w, 16) || !aligned(s_a, 4) || !aligned(s_w, 4) || !aligned(argmax, 4) ||
        (logits_bf16 && !aligned(logits_bf16, 2)))
        return IQD_ERR_ALIGN;
    const size_t lbytes = static_cast<size_t>(b) * N * 2;
    if (any_overlap({{logits_bf16, logits_bf16 ? lbytes : 0}, {argmax, static_cast<size_t>(b) * 4}},
                    {{q, static_cast<size_t>(b * K)}, {s_a, static_cast<size_t>(b) * 4},
                     {w, static_cast<size_t>(N) * K}, {s_w, static_cast<size_t>(N) * 4}}))
        return IQD_ERR_INVALID;
    return IQD_OK;
}

}  // namespace

static_assert(IQD_STATIC_SCRATCH_BYTES == iqd::kStaticScratchBytes, "the header's scratch size is the library's");

int lm_head_argmax_static(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b,
                          int64_t N, int64_t K, void *logits_bf16, int32_t *argmax, void *stream) {
    int st = lm_head_check(q, s_a, w, s_w, b, N, K, logits_bf16, argmax);
    if (st != IQD_OK) return st;
    if (ws_lm_head(b, N, logits_bf16 != nullptr) > IQD_STATIC_SCRATCH_BYTES) return IQD_ERR_WORKSPACE;
    void *scratch = nullptr;
    hipError_t e = iqd::static_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e);
    return lm_head_run(q, s_a, w, s_w, b, N, K, logits_bf16, argmax, scratch, static_cast<hipStream_t>(stream));
}

int lm_head_argmax(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b, int64_t N,
                   int64_t K, void *logits_bf16, int32_t *argmax, void *workspace, size_t workspace_bytes,
                   void *stream) {
    if (!q || !s_a || !w || !s_w || !argmax) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    if (!aligned(q, 16) || !aligned(w, 16) || !aligned(s_a, 4) || !aligned(s_w, 4) || !aligned(argmax, 4) ||
        (logits_bf16 && !aligned(logits_bf16, 2)))
        return IQD_ERR_ALIGN;
    const size_t ws = ws_lm_head(b, N, logits_bf16 != nullptr);
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    const size_t lbytes = static_cast<size_t>(b) * N * 2;
    if (any_overlap({{logits_bf16, logits_bf16 ? lbytes : 0}, {ws ? workspace : nullptr, ws},
                     {argmax, static_cast<size_t>(b) * 4}},
                    {{q, static_cast<size_t>(b * K)}, {s_a, static_cast<size_t>(b) * 4},
                     {w, static_cast<size_t>(N) * K}, {s_w, static_cast<size_t>(N) * 4}}))
        return IQD_ERR_INVALID;
    return lm_head_run(q, s_a, w, s_w, b, N, K, logits_bf16, argmax, workspace, static_cast<hipStream_t>(stream));
}

size_t attn_workspace_bytes(int64_t b, int64_t Hq, int64_t Hkv, int64_t D, int64_t pos0) {
    if (attn_check(b, Hq, Hkv, D, pos0) != IQD_OK) return 0;
    return round16(iqd::attn_workspace_bytes(b, Hq, pos0));
}

int attn_decode(const void *q_bf16, const void *k_cache, const void *v_cache, int64_t k_cell_stride,
                int64_t k_head_stride, int64_t v_cell_stride, int64_t v_head_stride, int64_t b, int64_t Hq,
                int64_t Hkv, int64_t D, int64_t pos0, float scale, void *out_bf16, void *workspace,
                size_t workspace_bytes, void *stream) {
    if (!q_bf16 || !k_cache || !v_cache || !out_bf16) return IQD_ERR_INVALID;
    int st = attn_check(b, Hq, Hkv, D, pos0);
    if (st != IQD_OK) return st;
    if (!(scale == scale) || scale - scale != 0.0f) return IQD_ERR_INVALID;  // NaN or infinite
    if (k_cell_stride < 0 || k_head_stride < 0 || v_cell_stride < 0 || v_head_stride < 0 ||
        k_cell_stride > kIntMax || k_head_stride > kIntMax || v_cell_stride > kIntMax || v_head_stride > kIntMax)
        return IQD_ERR_INVALID;
    // cells hold D elements each and must not overlap
    if (k_cell_stride < D || v_cell_stride < D) return IQD_ERR_INVALID;
    // a chunk's 256 cells must span less than 2 GB (32-bit buffer offsets)
    if (k_cell_stride >= (int64_t{1} << 22) || v_cell_stride >= (int64_t{1} << 22)) return IQD_ERR_UNSUPPORTED;
    if (!aligned(q_bf16, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out_bf16, 16) ||
        k_cell_stride % 8 || k_head_stride % 8 || v_cell_stride % 8 || v_head_stride % 8)
        return IQD_ERR_ALIGN;
    const size_t ws = round16(iqd::attn_workspace_bytes(b, Hq, pos0));
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    const int64_t cells = pos0 + b;
    const size_t qbytes = static_cast<size_t>(b * Hq * D) * 2;
    if (any_overlap({{out_bf16, qbytes}, {ws ? workspace : nullptr, ws}},
                    {{q_bf16, qbytes}, {k_cache, attn_cache_extent(cells, Hkv, D, k_cell_stride, k_head_stride)},
                     {v_cache, attn_cache_extent(cells, Hkv, D, v_cell_stride, v_head_stride)}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    return hip_status(iqd::launch_attn_decode(
        static_cast<const uint16_t *>(q_bf16), static_cast<const uint16_t *>(k_cache),
        static_cast<const uint16_t *>(v_cache), k_cell_stride, k_head_stride, v_cell_stride, v_head_stride,
        static_cast<int>(b), static_cast<int>(Hq), static_cast<int>(Hkv), static_cast<int>(pos0), scale,
        static_cast<uint16_t *>(out_bf16), workspace, static_cast<hipStream_t>(stream)));
}

int quantize_fp8(const void *x_bf16, int64_t b, int64_t K, uint8_t *q, float *s_a, void *stream) {
    if (!x_bf16 || !q || !s_a) return IQD_ERR_INVALID;
    if (b < 1 || K < 16 || K % 16 != 0 || b > kIntMax || K > kIntMax) return IQD_ERR_INVALID;
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(s_a, 4)) return IQD_ERR_ALIGN;
    if (any_overlap({{q, static_cast<size_t>(b * K)}, {s_a, static_cast<size_t>(b) * 4}},
                    {{x_bf16, static_cast<size_t>(b * K * 2)}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    return hip_status(iqd::launch_quantize_fp8(static_cast<const uint16_t *>(x_bf16), static_cast<int>(b),
                                               static_cast<int>(K), q, s_a, static_cast<hipStream_t>(stream)));
}

int fp8_linear(const uint8_t *q, const float *s_a, const uint8_t *w, const float *s_w, int64_t b, int64_t N,
               int64_t K, void *y_bf16, int32_t split_k, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !s_a || !w || !s_w || !y_bf16) return IQD_ERR_INVALID;
    int st = check_shape(b, N, K);
    if (st != IQD_OK) return st;
    st = fp8_split_ok(b, K, split_k);
    if (st != IQD_OK) return st;
    if (!aligned(q, 16) || !aligned(w, 16) || !aligned(s_a, 4) || !aligned(s_w, 4) || !aligned(y_bf16, 2))
        return IQD_ERR_ALIGN;
    const size_t ws = split_k > 1 ? round16(static_cast<size_t>(split_k) * b * N * 4) : 0;
    if (ws > 0) {
        if (!workspace || workspace_bytes < ws) return IQD_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return IQD_ERR_ALIGN;
    }
    if (any_overlap({{y_bf16, static_cast<size_t>(b) * N * 2}, {ws ? workspace : nullptr, ws}},
                    {{q, static_cast<size_t>(b * K)}, {s_a, static_cast<size_t>(b) * 4},
                     {w, static_cast<size_t>(N) * K}, {s_w, static_cast<size_t>(N) * 4}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint16_t *y = static_cast<uint16_t *>(y_bf16);
    const int Ni = static_cast<int>(N), Ki = static_cast<int>(K);
    if (split_k == 1) {
        // any b: launches of at most 16 tokens (each token's row is independent of its launch)
        for (int64_t t0 = 0; t0 < b; t0 += 16) {
            const int bc = static_cast<int>(b - t0 < 16 ? b - t0 : 16);
            hipError_t e = iqd::launch_fp8_matvec(q + t0 * K, s_a + t0, w, s_w, bc, Ni, Ki, y + t0 * N, 1, nullptr,
                                                  hs);
            if (e != hipSuccess) return hip_status(e);
        }
        return IQD_OK;
    }
    float *part = static_cast<float *>(workspace);
    const int bi = static_cast<int>(b);
    hipError_t e = iqd::launch_fp8_matvec(q, s_a, w, s_w, bi, Ni, Ki, nullptr, split_k, part, hs);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(iqd::launch_fp8_combine(part, s_a, s_w, bi, Ni, split_k, y, hs));
}

int pow2_requantize(const int8_t *w, const float *s_w, int64_t N, int64_t K, int8_t *w_out, float *s_out,
                    void *stream) {
    if (!w || !s_w || !w_out || !s_out) return IQD_ERR_INVALID;
    if (N < 1 || K < 1 || N > kIntMax || K > kIntMax) return IQD_ERR_INVALID;
    if (!aligned(s_w, 4) || !aligned(s_out, 4)) return IQD_ERR_ALIGN;
    if (any_overlap({{w_out, static_cast<size_t>(N) * K}, {s_out, static_cast<size_t>(N) * 4}},
                    {{w, static_cast<size_t>(N) * K}, {s_w, static_cast<size_t>(N) * 4}}))
        return IQD_ERR_INVALID;
    clear_stale_error();
    return hip_status(iqd::launch_pow2_requant(w, s_w, static_cast<int>(N), static_cast<int>(K), w_out, s_out,
                                               static_cast<hipStream_t>(stream)));
}

int iqd_read_ceiling(const void *p, int64_t bytes, int32_t *sink, void *stream) {
    if (!p || !sink || bytes < 16 || bytes % 16 != 0) return IQD_ERR_INVALID;
    if (!aligned(p, 16) || !aligned(sink, 4)) return IQD_ERR_ALIGN;
    if (overlap(sink, 4, p, static_cast<size_t>(bytes))) return IQD_ERR_INVALID;
    clear_stale_error();
    return hip_status(iqd::launch_read_ceiling(p, bytes, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
