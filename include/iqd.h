/*
 * iqd.h - batch-invariant int8 linear layer for decode and speculative-verify
 * passes on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libiqd.so.  Every entry point enqueues work on the caller's HIP
 * stream and returns at once; nothing is synchronised, nothing is allocated,
 * no pointer is kept after return.  The caller owns every buffer.
 *
 * Common conventions
 *  - Tensors are device-resident, row-major and contiguous: a [rows, cols]
 *    tensor has cols contiguous.  bf16 and fp16 are IEEE bfloat16 / binary16
 *    bit patterns in 16-bit words.
 *  - Alignment: int8 tensors and bf16 inputs 16 bytes; fp32 / int32 tensors
 *    4 bytes; bf16 / fp16 outputs and scales 2 bytes; workspace 16 bytes.
 *    Violations return IQD_ERR_ALIGN.
 *  - K (input features) must be a multiple of 16; 1 <= K <= IQD_K_MAX so that
 *    an int32 sum of K products of int8 values cannot overflow
 *    (128 * 128 * 131071 < 2^31).
 *  - Arguments are validated before any launch: on error nothing is written.
 *    Outputs must not overlap inputs (IQD_ERR_INVALID).  Inputs must be
 *    finite; NaN or Inf inputs give unspecified (but memory-safe) results.
 *  - A failed launch returns IQD_ERR_HIP.  Faults during execution surface
 *    at the caller's next synchronisation of the stream.
 *  - `stream` is a hipStream_t; NULL means the default stream.
 *  - Calls are stateless and re-entrant; concurrent calls on different
 *    streams are safe.
 *
 * The guarantee.  Every output element is a pure function of its token's
 * row of the inputs, the weights and the scales, computed in one canonical
 * order.  It does not depend on the number of tokens b in the call, on
 * split_k, on the grid, on the stream or on occupancy, and it equals the
 * plain CPU definition bit for bit.
 *
 * Sources (page title, then section / table / figure):
 *  [P1] "why speculative decoding changed my output": the guarantee
 *       speculative verification needs (a position's logits inside a batch
 *       equal its logits decoded alone); int8 activations in blocks of 32
 *       with float scales; per-block integer dot products scaled into fp32
 *       ("the mat-vec kernel"); fp32 order sensitivity ("floats care about
 *       order").
 *  [P2] "My speculative decoder got slower": split-K changes float rounding
 *       ("Two matmul schedules that survived"); a vocab head computing only
 *       the winning token ("We're nowhere near SOL").
 *  [P3] "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
 *       Quantization Scales and the Limits of Tolerance-Based Conformance":
 *       exact int32 accumulation (Abstract, Fig. 1); the epilogue faults of
 *       Table II; power-of-two scales with re-rounded weights (Abstract).
 */
#ifndef IQD_H
#define IQD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IQD_OK = 0,
    IQD_ERR_INVALID = -1,     /* bad shape, null pointer, aliasing, bad group */
    IQD_ERR_ALIGN = -2,       /* pointer misaligned */
    IQD_ERR_RANGE = -3,       /* K above IQD_K_MAX */
    IQD_ERR_UNSUPPORTED = -4, /* split_k (or an attention shape) not supported */
    IQD_ERR_WORKSPACE = -5,   /* workspace missing or too small */
    IQD_ERR_HIP = -6          /* a HIP runtime call or launch failed */
} iqd_status;

/* Operation codes for iqd_workspace_bytes. */
enum { IQD_OP_W8A8 = 1, IQD_OP_BLOCKQ8 = 2, IQD_OP_LM_HEAD = 3, IQD_OP_W8A8_BF16 = 4, IQD_OP_FP8 = 5, IQD_OP_KQ6 = 6,
       IQD_OP_KQ4 = 7 };

#define IQD_K_MAX 131071
#define IQD_SPLIT_K_MAX 64

/*
 * quantize_activations - int8 activations with fp32 scales.
 *
 * [P1 "the mat-vec kernel"]: activations are int8 with a float scale, in
 * blocks of 32 for block-quantized weights.  Per group of elements (a whole
 * token row when group == 0, each aligned 32-element block when group == 32):
 *     amax = max |x|                         (bf16 -> fp32 exact)
 *     s    = fl(amax / 127)                  (correctly rounded division)
 *     q    = clamp(rint_half_even(fl(x / s)), -127, 127)
 * A group whose amax is 0 gets s = 0 and q = 0.
 *
 *   x_bf16  in   bf16 [b, K]
 *   q       out  int8 [b, K]
 *   scale   out  fp32 [b] (group 0) or [b, K/32] (group 32)
 * Errors: IQD_ERR_INVALID for b < 1, K < 1, K % 16 (K % 32 for group 32),
 * a group other than 0 or 32, or overlapping buffers.
 */
int quantize_activations(const void *x_bf16, int64_t b, int64_t K, int32_t group, int8_t *q,
                         float *scale, void *stream);

/*
 * w8a8_linear - y = bf16( (fl32(sum_k q[t,k] * w[n,k]) * s_a[t]) * s_w[n] ).
 *
 * [P3 Abstract, Fig. 1]: the int32 sum is exact and order-free under the K
 * bound, so any decomposition of K is allowed.  [P3 Table II]: the epilogue
 * is the negation of faults F1-F5: fp32 scales, (acc * s_a) * s_w in that
 * order with no rounding between, no fused multiply-add, one round to
 * nearest even into bf16, applied once after the whole integer sum.
 *
 *   q      in  int8 [b, K]     s_a  in  fp32 [b]
 *   w      in  int8 [N, K]     s_w  in  fp32 [N]
 *   y_bf16 out bf16 [b, N]
 *   split_k    1, or a power of two <= min(IQD_SPLIT_K_MAX, K/16): the K
 *              range is cut into split_k int32 partial sums that a second
 *              kernel adds (exactly) before the epilogue.  Needs workspace.
 *   workspace  device scratch of iqd_workspace_bytes(IQD_OP_W8A8, ...) bytes
 *              (NULL allowed when that is 0).
 * b <= 16 streams the weights once (packed int8 dot products at b = 1 and
 * on small matrices at b = 2, the int8 matrix cores otherwise); larger b uses
 * the tiled matrix-core path, whose split_k divides each output tile's K
 * stages among split_k workgroups (more workgroups when tiles are few).  All
 * give identical bits.
 * Errors: IQD_ERR_INVALID, IQD_ERR_ALIGN, IQD_ERR_RANGE, IQD_ERR_UNSUPPORTED
 * (bad split_k), IQD_ERR_WORKSPACE, IQD_ERR_HIP.
 */
int w8a8_linear(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b,
                int64_t N, int64_t K, void *y_bf16, int32_t split_k, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * w8a8_linear_bf16 - quantize_activations (per token) and w8a8_linear in one
 * call, from bf16 activations.
 *
 * The results are those of quantize_activations(x, group 0) followed by
 * w8a8_linear(split_k 1), bit for bit.  For a few tokens (up to 2 or 4,
 * depending on N and K) one kernel does both: every workgroup quantizes the
 * activations it multiplies (the reciprocal of the scale first, the
 * correctly rounded division wherever the quotient lies within 2^-14 of a
 * rounding boundary) while its first weights are in flight, which removes
 * the separate quantization launch.  Wider passes run the two kernels.
 *
 *   x_bf16   in  bf16 [b, K]                (16-byte aligned)
 *   w, s_w   as w8a8_linear
 *   y_bf16   out bf16 [b, N]
 *   q_out    out int8 [b, K], or NULL       (16-byte aligned)
 *   s_a_out  out fp32 [b], or NULL
 *   workspace  iqd_workspace_bytes(IQD_OP_W8A8_BF16, b, N, K, 1) bytes,
 *              16-byte aligned; used (for q and s_a) only when a shape takes
 *              the separate quantize + linear path and q_out or s_a_out is
 *              NULL; NULL allowed when both outputs are given.
 * Errors: as w8a8_linear.
 */
int w8a8_linear_bf16(const void *x_bf16, const int8_t *w, const float *s_w, int64_t b, int64_t N, int64_t K,
                     void *y_bf16, int8_t *q_out, float *s_a_out, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * blockq8_linear - q8_0-style block-quantized linear.
 *
 * [P1 "the mat-vec kernel"]: per 32-element block j the integer dot product
 * isum_j is exact; it is scaled into fp32 as the leaf
 *     p_j = fl( fl( fl32(isum_j) * d_a[t,j] ) * fl32(d_w[n,j]) )
 * and the m = K/32 leaves are summed by the canonical tree: pad with +0.0f
 * leaves up to L = 2^ceil(log2 m), then add adjacent pairs in index order,
 * level by level.  y = bf16(root), rounded to nearest even.  The tree is
 * fixed, so the float order never depends on b, the grid or split_k
 * ([P1 "the mat-vec kernel"]: the stock kernel's block grouping changed
 * with the token count; [P2 "Two matmul schedules that survived"]: split-K
 * changed the rounding).
 *
 *   q      in  int8 [b, K]       d_a       in  fp32 [b, K/32]
 *   w      in  int8 [N, K]       d_w_fp16  in  fp16 [N, K/32]
 *   y_bf16 out bf16 [b, N]
 *   split_k    1, or a power of two <= min(IQD_SPLIT_K_MAX, L) (and b <= 16):
 *              split s owns the aligned subtree of leaves
 *              [s*L/split_k, (s+1)*L/split_k); a second kernel folds the top
 *              log2(split_k) tree levels.  Other values: IQD_ERR_UNSUPPORTED.
 * K must be a multiple of 32.
 */
int blockq8_linear(const int8_t *q, const float *d_a, const int8_t *w, const void *d_w_fp16,
                   int64_t b, int64_t N, int64_t K, void *y_bf16, int32_t split_k, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * kq6_linear - linear layer over k-quant-style superblocks of 256 weights
 * with 6-bit codes.
 *
 * [P1 "the mat-vec kernel"]: a q6_k row is read as weight blocks of 256
 * against int8 activations in blocks of 32; each block's exact integer
 * result is scaled into fp32.  The pages give no bit layout; this one is the
 * library's own (6.5625 bits per weight, the same as q6_k's): each group of
 * 16 weights is 8 + 4 contiguous bytes, arranged so that one shift and one
 * mask per plane give the codes of 4 consecutive weights:
 *   weight k = 16 g + i of a row has a code c in [-32, 31] kept as
 *   u = c + 32, a sub-scale sc[k / 16] and the scale d[k / 256] of its
 *   superblock;
 *   ql  in  uint8 [N, K/2]:  u & 15 of weight k in bits 4 (i/8) .. +3 of byte 8 g + i%8
 *   qh  in  uint8 [N, K/4]:  u >> 4 of weight k in bits 2 (i/4) .. +1 of byte 4 g + i%4
 *   sc  in  int8  [N, K/16]  sub-scales, one per 16 weights
 *   d_fp16 in fp16 [N, K/256] superblock scales
 * The result is the blockq8_linear tree with integer weights sc * c and the
 * superblock's scale as every block's weight scale:
 *     isum_j = sum over block j of (sc[k/16] * c[k]) * q[t,k]   (exact int32)
 *     p_j    = fl( fl( fl32(isum_j) * d_a[t,j] ) * fl32(d[n, j/8]) )
 *     y      = bf16(canonical tree over the K/32 leaves)
 * |isum_j| <= 2^24, so fl32(isum_j) is exact.
 *
 *   q      in  int8 [b, K]       d_a  in  fp32 [b, K/32]
 *   y_bf16 out bf16 [b, N]
 *   split_k    as blockq8_linear (aligned subtrees of the same tree).
 * K must be a multiple of 256.  q, ql and qh 16-byte aligned.
 * Errors: as blockq8_linear.
 */
int kq6_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
               const void *d_fp16, int64_t b, int64_t N, int64_t K, void *y_bf16, int32_t split_k,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * kq4_linear - linear layer over k-quant-style superblocks of 256 weights
 * with 4-bit codes and a minimum per 32 weights.
 *
 * [P1 opening]: the pages' decode workload is Qwen3-8B at q4_k_m; [P1 "the
 * mat-vec kernel"]: exact integer sums per activation block of 32, each
 * scaled into fp32.  Layout (the library's own; 4.625 bits per weight):
 *   ql  in  uint8 [N, K/2]     code q in [0, 15] of weight k = 16 g + i in
 *                              bits 4 (i/8) .. +3 of byte 8 g + i%8
 *   scm in  uint8 [N, K/32, 2] (sub-scale sc_j, minimum m_j) per 32 weights,
 *                              both in [0, 63] (not checked)
 *   dm  in  fp16  [N, K/256, 2] (d, dmin) per superblock
 * Weight k of block j stands for d sc_j q_k - dmin m_j.  Per block:
 *     isum_j = sc_j * sum q[t,k] * code_k,  msum_j = m_j * sum q[t,k]  (exact)
 *     p_j = fl( fl(fl(fl32(isum_j) * d_a[t,j]) * fl32(d)) - fl(fl(fl32(msum_j) * d_a[t,j]) * fl32(dmin)) )
 *     y   = bf16(canonical tree over the K/32 leaves)
 *
 *   q      in  int8 [b, K]       d_a  in  fp32 [b, K/32]
 *   y_bf16 out bf16 [b, N]
 *   split_k    as blockq8_linear.
 * K must be a multiple of 256.  q and ql 16-byte aligned, scm 2, dm 4.
 * Errors: as blockq8_linear.
 */
int kq4_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *scm, const void *dm_fp16,
               int64_t b, int64_t N, int64_t K, void *y_bf16, int32_t split_k, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * lm_head_argmax - W8A8 vocab projection and the winning token per row.
 *
 * [P2 "We're nowhere near SOL"]: a vocab head that returns only the winning
 * token.  logits are w8a8_linear's outputs; argmax[t] is the smallest n whose
 * bf16 logit equals the row maximum, compared as real numbers (+0 == -0).
 * The pages do not fix a tie rule ([P2 "Why the decoders disagreed?"] shows
 * a real bf16 tie); the lowest index wins.
 *
 *   logits_bf16  out bf16 [b, N], or NULL to keep the logits in the workspace
 *   argmax       out int32 [b]
 *   workspace    iqd_workspace_bytes(IQD_OP_LM_HEAD, b, N, K, 1) bytes, 16-byte
 *                aligned: the logits when logits_bf16 is NULL, then 256 KiB
 *                of argmax scratch (one 64-bit key per token and mat-vec
 *                workgroup; the logits are not read back)
 * Requires N <= 2^31 - 1.
 */
int lm_head_argmax(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b,
                   int64_t N, int64_t K, void *logits_bf16, int32_t *argmax, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * lm_head_argmax_static - lm_head_argmax without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace
 * lm_head_argmax would take from the caller comes from a library-owned
 * device array of IQD_STATIC_SCRATCH_BYTES per GPU, which each GPU the
 * library runs on holds until the process ends.  The call allocates nothing
 * (no hipMalloc, no hipFree, no allocating library routine).
 *
 * Same arguments, results and bits as lm_head_argmax.  Needs
 * iqd_workspace_bytes(IQD_OP_LM_HEAD, b, N, K, 1) <= IQD_STATIC_SCRATCH_BYTES
 * when logits_bf16 is NULL (b * N * 2 bytes of logits plus the argmax
 * scratch), and 256 KiB when the caller passes logits; larger sizes return
 * IQD_ERR_WORKSPACE with nothing written.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams or host threads) race on it and must be
 * serialised by the caller.  Nothing in the array needs to start at zero.
 */
#define IQD_STATIC_SCRATCH_BYTES (8u << 20)
int lm_head_argmax_static(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b,
                          int64_t N, int64_t K, void *logits_bf16, int32_t *argmax, void *stream);

/*
 * pow2_requantize - move each weight row to a power-of-two scale.
 *
 * [P3 Abstract]: once each row's scale is a power of two, multiplying by it
 * is exact, so the scale products no longer depend on their order; the
 * weights are re-rounded to the new scale as well (changing the scale alone
 * would change the layer's values).  Per row n, with |s| = m * 2^E, m in [1, 2):
 *     s'       = sign(s) * (m < 1.5 ? 2^E : 2^(E+1))
 *     w'[n,k]  = clamp(rint_half_even(w[n,k] * s / s'), -127, 127)
 * computed exactly (w * s has at most 32 significant bits; s' is a power of
 * two).  s == 0 gives s' = 0 and w' = 0.  Offline weight preparation, not a
 * per-token step.
 *
 *   w in int8 [N, K], s_w in fp32 [N]  ->  w_out int8 [N, K], s_out fp32 [N]
 */
int pow2_requantize(const int8_t *w, const float *s_w, int64_t N, int64_t K, int8_t *w_out,
                    float *s_out, void *stream);

/*
 * quantize_fp8 - per-token FP8 (OCP E4M3) quantization of bf16 activations.
 *
 * [P2 "A trained drafter and two matmul schedules"]: projection weights in FP8,
 * the activations with them.  Per token: s = fl(amax / 448) (448 is the
 * largest finite E4M3), q = e4m3(fl(x / s)) rounded to nearest with ties to
 * the even code, saturating at 448, the sign kept (-0 gives 0x80); an
 * all-zero token gives s = 0 and +0 codes.
 *
 *   x_bf16 in bf16 [b, K] (16-byte aligned)  ->  q out E4M3 [b, K], s_a out fp32 [b]
 * K a multiple of 16.
 */
int quantize_fp8(const void *x_bf16, int64_t b, int64_t K, uint8_t *q, float *s_a, void *stream);

/*
 * fp8_linear - FP8 (E4M3) W8A8 linear with a fixed summation tree.
 *
 * [P2 "Two matmul schedules that survived"]: split-K and the step size move
 * the rounding points of a float sum; [P3 Abstract]: FP8 differences between
 * implementations grow with the reduction depth.  The product of two E4M3
 * values is exact in binary32, so the order is all that can differ; it is
 * fixed: K in groups of 16, each group's products added in increasing k
 * from +0; the K/16 group sums are the leaves of the canonical tree (zero-
 * padded to L = 2^ceil(log2(K/16)) leaves, adjacent pairs); then
 * y = bf16(fl(fl(root * s_a) * s_w)), nearest even.
 *
 *   q      in  E4M3 [b, K]      s_a  in  fp32 [b]
 *   w      in  E4M3 [N, K]      s_w  in  fp32 [N]
 *   y_bf16 out bf16 [b, N]
 *   split_k    1, or (b <= 16) a power of two with 64 * split_k <= L: split s
 *              owns the aligned subtree of leaves [s L / split_k, (s+1) L /
 *              split_k); a second kernel folds the top levels and applies the
 *              epilogue.  Workspace: iqd_workspace_bytes(IQD_OP_FP8, ...).
 * K a multiple of 16, 16 <= K <= IQD_K_MAX; any b (tokens in launches of 16).
 * NaN codes (S.1111.111) give unspecified results.
 */
int fp8_linear(const uint8_t *q, const float *s_a, const uint8_t *w, const float *s_w, int64_t b, int64_t N,
               int64_t K, void *y_bf16, int32_t split_k, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode - decode / speculative-verify attention over a bf16 KV cache,
 * batch-invariant.
 *
 * [P1 "the bug that waited for position 384", Fig. 5]: the stock kernel summed
 * the cache in chunks spread over an occupancy-chosen number of blocks, so a
 * batched query could round differently from the same query alone.
 * [P2 "Fusion that lost"]: split-KV attention as fixed 256-token chunk
 * partials and a merge, with a one-chunk fast path, the chunk count taken
 * from the tokens present rather than the allocation; [P2 "Why the decoders
 * disagreed?"]: slots past a query's position are never read; [P2 "Shipping
 * the 6.4x as its own backend"]: a merge order is one valid rounding and must
 * stay fixed.
 *
 * Query t (0 <= t < b) sits at position pos0 + t and attends cells
 * 0 .. pos0 + t (its own key and value already written).  Query head hq reads
 * kv head hq / (Hq / Hkv).  Per query row, in binary32:
 *   qs = fl(q * scale); s_j = tree over 16 slices of 8 dims of fused
 *   multiply-add chains from +0 (adjacent pairs); per 256-cell chunk c:
 *   m_c = max s_j, e_j = E(s_j - m_c), l_c = sum e_j, o_c = sum e_j v_j
 *   (fused multiply-adds), j increasing; merge in increasing c with
 *   w_c = E(m_c - max m): L = w_0 l_0, O = w_0 o_0, then fused multiply-adds;
 *   out = bf16(O / L), nearest even.  E(x) = e^x for x <= 0 by Cody-Waite
 *   reduction and a degree-7 Taylor polynomial, 0 below 2^-125.
 * Each row's result depends on nothing but its q row, its position, scale
 * and cells 0..pos0 + t: not on b, the cache's allocated size, the strides
 * or the grid.
 *
 *   q_bf16   in  bf16 [b, Hq, D], contiguous, 16-byte aligned
 *   k_cache  in  bf16; the element (cell j, kv head h, dim d) is at
 *   v_cache      cache + j * cell_stride + h * head_stride + d (strides in
 *                elements, multiples of 8, so every 16-byte row piece is
 *                aligned; cell_stride >= D, or IQD_ERR_INVALID); both must
 *                hold cells 0 .. pos0 + b - 1, which are the only cells read;
 *                16-byte aligned
 *   out_bf16 out bf16 [b, Hq, D], contiguous, 16-byte aligned
 *   workspace    attn_workspace_bytes(b, Hq, Hkv, D, pos0) bytes, 16-byte
 *                aligned (none when pos0 + b <= 256): fp32 chunk partials
 * Supported: D = 128; Hq a multiple of Hkv with Hq / Hkv <= 16; cell
 * strides below 2^22 elements; b * Hq and
 * (chunks * Hkv + 8) * b below 2^31, chunks = (pos0 + b - 1) / 256 + 1 (else
 * IQD_ERR_UNSUPPORTED); 1 <= b <= 65535; 0 <= pos0 and pos0 + b <= 2^30;
 * scale finite.
 */
int attn_decode(const void *q_bf16, const void *k_cache, const void *v_cache, int64_t k_cell_stride,
                int64_t k_head_stride, int64_t v_cell_stride, int64_t v_head_stride, int64_t b, int64_t Hq,
                int64_t Hkv, int64_t D, int64_t pos0, float scale, void *out_bf16, void *workspace,
                size_t workspace_bytes, void *stream);

/* Workspace bytes attn_decode needs (0 if none, or for arguments it would
 * reject). */
size_t attn_workspace_bytes(int64_t b, int64_t Hq, int64_t Hkv, int64_t D, int64_t pos0);

/*
 * iqd_read_ceiling - measurement helper, not a step of the linear layer:
 * stream `bytes` of device memory with the 16-byte non-temporal loads of the
 * mat-vec kernels and keep nothing.  Timed over the byte count of one
 * layer's weights, it is the practical HBM ceiling of one launch of that
 * size (dispatch, first round trip and drain included, no arithmetic, no
 * output).  Every HBM-bound kernel is ultimately priced against the
 * device's peak; this gives the part of that peak a launch can reach.
 *
 *   p      in  device memory, 16-byte aligned, `bytes` readable
 *   bytes      a multiple of 16, >= 16
 *   sink   out 4 bytes of device memory, written only for one 32-bit value
 *              of the xor of all loaded words (the loads must look used)
 * Errors: IQD_ERR_INVALID (null, size, sink inside p), IQD_ERR_ALIGN,
 * IQD_ERR_HIP.
 */
int iqd_read_ceiling(const void *p, int64_t bytes, int32_t *sink, void *stream);

/* Workspace bytes the op needs for these sizes (0 if none); 0 also for
 * arguments the op would reject. */
size_t iqd_workspace_bytes(int op, int64_t b, int64_t N, int64_t K, int32_t split_k);

/* Static, human-readable name of a status code. */
const char *iqd_status_str(int status);

/* Name of the HIP error behind the calling thread's most recent IQD_ERR_HIP
 * (static string; "hipSuccess" if there was none).  Diagnostics only. */
const char *iqd_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IQD_H */
