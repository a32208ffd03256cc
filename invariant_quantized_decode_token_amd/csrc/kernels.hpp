// Host-side launchers of the gfx950 kernels (internal to libiqd).  Each
// launcher assumes its arguments were validated by the C ABI layer and
// returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace iqd {

struct DeviceInfo {
    int cus = 256;
    int max_lds = 160 * 1024;       // LDS per CU
    int max_lds_block = 64 * 1024;  // LDS one workgroup may allocate
};
const DeviceInfo &device_info();

hipError_t launch_quantize_token(const uint16_t *x, int b, int K, int8_t *q, float *s, hipStream_t st);
hipError_t launch_quantize_block32(const uint16_t *x, int b, int K, int8_t *q, float *d, hipStream_t st);

// W8A8 mat-vec, 1 <= b <= 16.  With split > 1, writes int32 partial sums
// part[s, b, N] instead of y and needs launch_w8a8_combine afterwards.
hipError_t launch_w8a8_matvec(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w,
                              int b, int N, int K, uint16_t *y, int split, int32_t *part,
                              hipStream_t st);
// The same mat-vec on the int8 matrix cores (split 1 only).  fits() tells
// whether the shape is supported (activations must fit in LDS).
bool w8a8_mfvec_fits(int b, int N, int K);
hipError_t launch_w8a8_mfvec(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N,
                             int K, uint16_t *y, hipStream_t st);
// Quantization fused in: bf16 activations x [b, K] in; q_out [b, K] and
// s_out [b] (both optional) receive the quantized activations.  Supported
// where fused_ok() says so (a few tokens: up to 2 or 4 by shape).
bool w8a8_mfvec_fused_ok(int b, int N, int K);
hipError_t launch_w8a8_mfvec_fused(const uint16_t *x, const int8_t *w, const float *s_w, int b, int N, int K,
                                   uint16_t *y, int8_t *q_out, float *s_out, hipStream_t st);
hipError_t launch_w8a8_combine(const int32_t *part, const float *s_a, const float *s_w, int b, int N,
                               int split, uint16_t *y, hipStream_t st);
// The dot4 mat-vec with the quantization fused in (one token; fused_ok says
// which shapes): bf16 x [1, K] in, the bits of quantize + w8a8_linear out.
bool w8a8_matvec_fused_ok(int b, int N, int K);
hipError_t launch_w8a8_matvec_fused(const uint16_t *x, const int8_t *w, const float *s_w, int b, int N, int K,
                                    uint16_t *y, int8_t *q_out, float *s_out, hipStream_t st);

// W8A8 int8 matrix-core GEMM for b > 16 (prefill), same epilogue.  With
// split > 1 the K stages are divided among `split` workgroups per tile, which
// write int32 partial sums part[split, b, N]; the combine then runs too.
hipError_t launch_w8a8_mfma(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w,
                            int b, int N, int K, uint16_t *y, int split, int32_t *part, hipStream_t st);

// Block-quantized mat-vec, 1 <= b <= 16.  With split > 1, writes fp32 subtree
// roots part[s, b, N] and needs launch_blockq8_combine afterwards.
hipError_t launch_blockq8_matvec(const int8_t *q, const float *d_a, const int8_t *w,
                                 const uint16_t *d_w, int b, int N, int K, uint16_t *y, int split,
                                 float *part, hipStream_t st);
// The same block-quantized mat-vec on the int8 matrix cores (any split the
// ABI accepts); fits() tells whether the shape is supported (activations
// must fit in LDS).
bool blockq8_mfvec_fits(int b, int N, int K, int split);
hipError_t launch_blockq8_mfvec(const int8_t *q, const float *d_a, const int8_t *w, const uint16_t *d_w, int b,
                                int N, int K, uint16_t *y, int split, float *part, hipStream_t st);
hipError_t launch_blockq8_combine(const float *part, int b, int N, int split, uint16_t *y,
                                  hipStream_t st);
// The same block mat-vec over kq6 superblocks (1 <= b <= 16; split as above,
// finished by launch_blockq8_combine).
hipError_t launch_kq6_matvec(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
                             const uint16_t *d, int b, int N, int K, uint16_t *y, int split, float *part,
                             hipStream_t st);
// And over kq4 superblocks: scm holds (sub-scale, minimum) byte pairs per 32
// weights, dm (d, dmin) fp16 pairs per 256.
hipError_t launch_kq4_matvec(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *scm, const uint16_t *dm,
                             int b, int N, int K, uint16_t *y, int split, float *part, hipStream_t st);

// The LM head: the W8A8 mat-vec (1 <= b <= 16, split 1) that also leaves, per
// workgroup g and token t, the largest argmax key of the logits it wrote at
// keys[t * grid + g]; *grid receives the grid size (at most keys_cap).
// launch_argmax_fold then gives out[t], the smallest index of row t's
// maximum (at most kArgKeysMaxGrid keys per token).
constexpr int kArgKeysMaxGrid = 32768;
hipError_t launch_w8a8_matvec_keys(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N,
                                   int K, uint16_t *y, uint64_t *keys, int keys_cap, int *grid, hipStream_t st);
hipError_t launch_w8a8_mfvec_keys(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int b, int N,
                                  int K, uint16_t *y, uint64_t *keys, int keys_cap, int *grid, hipStream_t st);
hipError_t launch_argmax_fold(const uint64_t *keys, int b, int nkeys, int32_t *out, hipStream_t st);

// FP8 (E4M3) W8A8: per-token quantizer and the fixed-tree mat-vec (1 <= b <= 16;
// split > 1 writes fp32 subtree roots [split, b, N] for launch_fp8_combine).
int64_t fp8_tree_leaves(int K);
hipError_t launch_quantize_fp8(const uint16_t *x, int b, int K, uint8_t *q, float *s, hipStream_t st);
hipError_t launch_fp8_matvec(const uint8_t *q, const float *s_a, const uint8_t *w, const float *s_w, int b, int N,
                             int K, uint16_t *y, int split, float *part, hipStream_t st);
hipError_t launch_fp8_combine(const float *part, const float *s_a, const float *s_w, int b, int N, int split,
                              uint16_t *y, hipStream_t st);

// Decode attention in fixed 256-cell chunks (D = 128, Hq / Hkv <= 16).
// Workspace: attn_workspace_bytes(b, Hq, pos0) bytes of chunk partials.
int64_t attn_chunks(int64_t b, int64_t pos0);
size_t attn_workspace_bytes(int64_t b, int64_t Hq, int64_t pos0);
hipError_t launch_attn_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t kc, int64_t kh,
                              int64_t vc, int64_t vh, int b, int Hq, int Hkv, int pos0, float scale, uint16_t *out,
                              void *ws, hipStream_t st);

// The library-owned device scratch of the entry points that allocate
// nothing: kStaticScratchBytes per GPU, its device address for the current
// device (taken once per device; no allocation).
constexpr size_t kStaticScratchBytes = size_t{8} << 20;
hipError_t static_scratch(void **out);

// Read-ceiling measurement kernel: streams `bytes` (a multiple of 16) from p.
hipError_t launch_read_ceiling(const void *p, int64_t bytes, int32_t *sink, hipStream_t st);

hipError_t launch_pow2_requant(const int8_t *w, const float *s, int N, int K, int8_t *w_out,
                               float *s_out, hipStream_t st);

}  // namespace iqd
