/*
 * CPU oracle for the batch-invariant int8 linear layer of decode and
 * speculative-verify passes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * It is deliberately plain and slow: scalar loops, one IEEE-754 binary32
 * operation per C expression, no blocking, no vectorisation, no contraction:
 * the linear layers use no fused multiply-add, and the attention recipe at
 * the end uses only the explicit fmaf calls it names.  Build with `gcc -O2 -ffp-contract=off` (no -ffast-math, no
 * -march=native) on x86-64, where float arithmetic is SSE scalar with one
 * rounding per operation and FLT_EVAL_METHOD == 0.
 *
 * Sources (page title, then section / table):
 *  [P1] "why speculative decoding changed my output"
 *       - "floats care about order": fp32 addition is not associative; near
 *         1e8 neighbouring floats are 8 apart.
 *       - "the mat-vec kernel": int8 activations in blocks of 32, four int8
 *         products summed exactly into int32 per instruction, each block's
 *         integer result scaled into an fp32 accumulator.
 *  [P2] "My speculative decoder got slower"
 *       - "We're nowhere near SOL": a vocab head that returns only the
 *         winning token.
 *       - "Two matmul schedules that survived": split-K changes where a
 *         float running sum is rounded.
 *  [P3] "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
 *       Quantization Scales and the Limits of Tolerance-Based Conformance"
 *       - Abstract and Fig. 1: W8A8 integer accumulation is exact and
 *         order-independent under a no-overflow bound; weight scales moved to
 *         their nearest power of two with the weights re-rounded.
 *       - Table II: the epilogue faults F1-F5, whose negation fixes the
 *         canonical epilogue (acc * s_a) * s_w in fp32 with one
 *         round-to-nearest-even to bfloat16.
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function that implements it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS (-1)
#define ORACLE_ERR_OVERFLOW (-2)
#define ORACLE_ERR_THREAD (-3)

/* ------------------------------------------------------------------------ */
/* Scalar primitives.  Each is one binary32 operation with the default       */
/* round-to-nearest-even mode.  Exported so that tests can pin them.         */
/* ------------------------------------------------------------------------ */

float oracle_f32_add(float a, float b) { return a + b; }
float oracle_f32_sub(float a, float b) { return a - b; }
float oracle_f32_mul(float a, float b) { return a * b; }
float oracle_f32_div(float a, float b) { return a / b; }
/* int32 -> binary32, rounded to nearest even (cvtsi2ss under the default
 * MXCSR mode).  Inexact once |v| > 2^24. */
float oracle_i32_to_f32(int32_t v) { return (float)v; }

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even.  A NaN keeps its sign
 * and is made quiet; overflow carries into the exponent and gives +-Inf;
 * subnormals are rounded like any other value (no flush to zero). */
uint16_t oracle_bf16_rne(uint32_t u) {
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* bfloat16 -> binary32 is exact: the 16 bits become the high half. */
float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* IEEE binary16 -> binary32, exact, decoded from the field definitions. */
float oracle_fp16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    float mag;
    if (exp == 0)
        mag = ldexpf((float)man, -24); /* subnormal: man * 2^-24 */
    else if (exp == 31)
        mag = man ? NAN : INFINITY;
    else
        mag = ldexpf((float)(man | 0x400), exp - 25); /* 1.man * 2^(exp-15) */
    return sign ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* Activation quantization.                                                  */
/* ------------------------------------------------------------------------ */

/* Quantize n bf16 values with one shared scale.  [P1 "the mat-vec kernel"]
 * gives int8 activations with a float scale; the configuration text gives
 * the scale as absmax / 127.  Readings taken:
 *   s = fl(amax / 127) with a correctly rounded division;
 *   q = clamp(rint_half_even(fl(x / s)), -127, 127), division not a
 *       reciprocal multiply, so -128 never appears;
 *   an all-zero group gives s = 0 and q = 0.
 * |x| and the max are exact; bf16 -> fp32 is exact. */
static float quantize_group(const uint16_t *x, int64_t n, int8_t *q) {
    float amax = 0.0f;
    for (int64_t k = 0; k < n; ++k) {
        float v = fabsf(oracle_bf16_to_f32(x[k]));
        if (v > amax) amax = v;
    }
    float s = oracle_f32_div(amax, 127.0f);
    if (s == 0.0f) {
        for (int64_t k = 0; k < n; ++k) q[k] = 0;
        return 0.0f;
    }
    for (int64_t k = 0; k < n; ++k) {
        float r = rintf(oracle_f32_div(oracle_bf16_to_f32(x[k]), s));
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[k] = (int8_t)r;
    }
    return s;
}

/* Per-token quantization: x bf16 [b, K] -> q int8 [b, K], s fp32 [b]. */
int oracle_quantize_token(const uint16_t *x, int64_t b, int64_t K, int8_t *q, float *s) {
    if (!x || !q || !s || b < 0 || K < 1) return ORACLE_ERR_ARGS;
    for (int64_t t = 0; t < b; ++t) s[t] = quantize_group(x + t * K, K, q + t * K);
    return ORACLE_OK;
}

/* Per-32-block quantization: x bf16 [b, K] -> q int8 [b, K],
 * d fp32 [b, K/32]; each aligned 32-element block has its own scale
 * ([P1 "the mat-vec kernel"]: activations are int8 in blocks of 32). */
int oracle_quantize_block32(const uint16_t *x, int64_t b, int64_t K, int8_t *q, float *d) {
    if (!x || !q || !d || b < 0 || K < 32 || K % 32) return ORACLE_ERR_ARGS;
    int64_t m = K / 32;
    for (int64_t t = 0; t < b; ++t)
        for (int64_t j = 0; j < m; ++j)
            d[t * m + j] = quantize_group(x + t * K + 32 * j, 32, q + t * K + 32 * j);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Exact integer dot product.                                                */
/* ------------------------------------------------------------------------ */

/* sum_k a[k] * w[k] accumulated in int32 (wrapping arithmetic, so that an
 * overflow is defined behaviour here) with an int64 shadow.  [P3 Abstract,
 * Fig. 1]: under a no-overflow bound the int32 sum is exact, so its value is
 * independent of the order of the additions.  Returns 0 and stores the sum,
 * or returns ORACLE_ERR_OVERFLOW when the int32 and int64 sums differ. */
static int dot_i8(const int8_t *a, const int8_t *w, int64_t n, int32_t *out) {
    uint32_t acc32 = 0;
    int64_t acc64 = 0;
    for (int64_t k = 0; k < n; ++k) {
        int32_t p = (int32_t)a[k] * (int32_t)w[k];
        acc32 += (uint32_t)p;
        acc64 += p;
    }
    int32_t v = (int32_t)acc32;
    *out = v;
    return ((int64_t)v == acc64) ? ORACLE_OK : ORACLE_ERR_OVERFLOW;
}

/* Exported for tests: the int32 dot product of two int8 vectors. */
int oracle_dot_i8(const int8_t *a, const int8_t *w, int64_t n, int32_t *out) {
    if (!a || !w || !out || n < 0) return ORACLE_ERR_ARGS;
    return dot_i8(a, w, n, out);
}

/* ------------------------------------------------------------------------ */
/* Epilogue and block partial.                                               */
/* ------------------------------------------------------------------------ */

/* Canonical W8A8 epilogue, [P3 Table II] read as the negation of its five
 * faults: fp32 scales (not F1), no rounding between the two multiplies
 * (not F2), (acc * s_a) * s_w in that order (not F3), round to nearest even
 * on output (not F4), scales applied once after the integer sum (not F5).
 *   y = bf16( fl( fl( fl32(acc) * s_a ) * s_w ) ) */
uint16_t oracle_epilogue(int32_t acc, float s_a, float s_w) {
    float a = oracle_i32_to_f32(acc);
    float t = oracle_f32_mul(a, s_a);
    float y = oracle_f32_mul(t, s_w);
    return oracle_bf16_rne(f32_bits(y));
}

/* One 32-block partial of the block-quantized product.  [P1 "the mat-vec
 * kernel"] says only that each block's integer result is scaled into fp32;
 * the order is read to mirror the W8A8 epilogue: (fl32(isum) * d_a) * d_w,
 * with the fp16 weight scale widened exactly to fp32. */
float oracle_block_partial(int32_t isum, float d_a, uint16_t d_w) {
    float a = oracle_i32_to_f32(isum);
    float t = oracle_f32_mul(a, d_a);
    return oracle_f32_mul(t, oracle_fp16_to_f32(d_w));
}

/* ------------------------------------------------------------------------ */
/* The canonical pairwise tree.                                              */
/* ------------------------------------------------------------------------ */

/* Root of the tree over leaves [lo, lo + size) where size is a power of
 * two; leaves at index >= m are +0.0f.  Defined recursively: a single leaf
 * is itself; otherwise root(left half) + root(right half) in one fl-add.
 * This is the same as combining adjacent pairs in index order, level by
 * level. */
static float tree_rec(const float *leaf, int64_t m, int64_t lo, int64_t size) {
    if (size == 1) return lo < m ? leaf[lo] : 0.0f;
    int64_t h = size / 2;
    float left = tree_rec(leaf, m, lo, h);
    float right = tree_rec(leaf, m, lo + h, h);
    return oracle_f32_add(left, right);
}

static int64_t pow2_ceil(int64_t m) {
    int64_t L = 1;
    while (L < m) L *= 2;
    return L;
}

/* Canonical tree over m leaves, zero-padded to L = 2^ceil(log2 m).  The fixed
 * order answers [P1 "the mat-vec kernel"] (the stock block grouping changed
 * with the token count) and [P2 "Two matmul schedules that survived"]
 * (split-K moved the rounding points).  Reading: adjacent pairs in index
 * order, +0.0f leaves added literally. */
float oracle_tree_sum(const float *leaf, int64_t m) {
    if (m < 1) return 0.0f;
    return tree_rec(leaf, m, 0, pow2_ceil(m));
}

/* ------------------------------------------------------------------------ */
/* Thread pool over output rows.  Each output element is computed by exactly  */
/* one thread, start to finish, so the thread count cannot change a result.  */
/* ------------------------------------------------------------------------ */

typedef struct {
    int op; /* 0 = w8a8, 1 = blockq8 */
    const int8_t *q;
    const float *sa;   /* s_a [b] or d_a [b, K/32] */
    const int8_t *w;
    const float *sw;   /* s_w [N] (w8a8) */
    const uint16_t *dw; /* d_w fp16 [N, K/32] (blockq8) */
    int64_t b, N, K;
    uint16_t *y;
    int64_t n0, n1;
    int status;
} rows_job;

static void w8a8_rows(rows_job *j) {
    for (int64_t n = j->n0; n < j->n1; ++n) {
        const int8_t *wr = j->w + n * j->K;
        for (int64_t t = 0; t < j->b; ++t) {
            int32_t acc;
            if (dot_i8(j->q + t * j->K, wr, j->K, &acc) != ORACLE_OK) j->status = ORACLE_ERR_OVERFLOW;
            j->y[t * j->N + n] = oracle_epilogue(acc, j->sa[t], j->sw[n]);
        }
    }
}

static void blockq8_rows(rows_job *j) {
    int64_t m = j->K / 32;
    float *leaf = (float *)malloc(sizeof(float) * (size_t)m);
    if (!leaf) {
        j->status = ORACLE_ERR_ARGS;
        return;
    }
    for (int64_t n = j->n0; n < j->n1; ++n) {
        const int8_t *wr = j->w + n * j->K;
        for (int64_t t = 0; t < j->b; ++t) {
            for (int64_t i = 0; i < m; ++i) {
                int32_t isum;
                dot_i8(j->q + t * j->K + 32 * i, wr + 32 * i, 32, &isum); /* |isum| <= 32*128*128 */
                leaf[i] = oracle_block_partial(isum, j->sa[t * m + i], j->dw[n * m + i]);
            }
            float root = oracle_tree_sum(leaf, m);
            j->y[t * j->N + n] = oracle_bf16_rne(f32_bits(root));
        }
    }
    free(leaf);
}

static void *rows_worker(void *arg) {
    rows_job *j = (rows_job *)arg;
    if (j->op == 0)
        w8a8_rows(j);
    else
        blockq8_rows(j);
    return NULL;
}

static int run_rows(rows_job proto, int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > proto.N) nthreads = (int)proto.N;
    rows_job jobs[256];
    pthread_t th[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].n0 = proto.N * i / nthreads;
        jobs[i].n1 = proto.N * (i + 1) / nthreads;
        jobs[i].status = ORACLE_OK;
        started[i] = 0;
    }
    int status = ORACLE_OK;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, rows_worker, &jobs[i]) == 0)
            started[i] = 1;
        else
            rows_worker(&jobs[i]); /* fall back to running it here */
    }
    rows_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) status = jobs[i].status;
    return status;
}

/* ------------------------------------------------------------------------ */
/* The linear layers.                                                        */
/* ------------------------------------------------------------------------ */

/* W8A8 linear: q int8 [b, K], s_a fp32 [b], w int8 [N, K], s_w fp32 [N]
 * -> y bf16 [b, N].  acc = sum_k q[t,k] * w[n,k] exactly in int32
 * ([P3 Abstract, Fig. 1]), then the canonical epilogue ([P3 Table II]).
 * Returns ORACLE_ERR_OVERFLOW if any int32 sum left the int32 range. */
int oracle_w8a8(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b,
                int64_t N, int64_t K, uint16_t *y, int nthreads) {
    if (!q || !s_a || !w || !s_w || !y || b < 0 || N < 1 || K < 1) return ORACLE_ERR_ARGS;
    if (b == 0) return ORACLE_OK;
    rows_job j = {0, q, s_a, w, s_w, NULL, b, N, K, y, 0, N, ORACLE_OK};
    return run_rows(j, nthreads);
}

/* Block-quantized (q8_0-style) linear: q int8 [b, K], d_a fp32 [b, K/32],
 * w int8 [N, K], d_w fp16 [N, K/32] -> y bf16 [b, N].  Per 32-block an exact
 * int32 sum and the block partial, then the canonical tree over the K/32
 * partials and one rounding to bf16.  [P1 "the mat-vec kernel"]; the tree
 * reading is at oracle_tree_sum. */
int oracle_blockq8(const int8_t *q, const float *d_a, const int8_t *w, const uint16_t *d_w,
                   int64_t b, int64_t N, int64_t K, uint16_t *y, int nthreads) {
    if (!q || !d_a || !w || !d_w || !y || b < 0 || N < 1 || K < 32 || K % 32) return ORACLE_ERR_ARGS;
    if (b == 0) return ORACLE_OK;
    rows_job j = {1, q, d_a, w, NULL, d_w, b, N, K, y, 0, N, ORACLE_OK};
    return run_rows(j, nthreads);
}

/* Argmax over one row of bf16 logits: the smallest index whose value equals
 * the row maximum, comparing the fp32 values of the bf16 numbers (so +0 and
 * -0 are equal).  [P2 "We're nowhere near SOL"] describes a head returning
 * only the winning token; the pages do not say how ties break ([P2 "Why the
 * decoders disagreed?"] shows a real bf16 tie), so the lowest index wins. */
int32_t oracle_argmax_row(const uint16_t *y, int64_t N) {
    int32_t best = 0;
    float bv = oracle_bf16_to_f32(y[0]);
    for (int64_t n = 1; n < N; ++n) {
        float v = oracle_bf16_to_f32(y[n]);
        if (v > bv) {
            bv = v;
            best = (int32_t)n;
        }
    }
    return best;
}

/* LM head for a verify pass: W8A8 logits for every vocab row, then the
 * per-token argmax.  logits bf16 [b, N] must be provided (the oracle always
 * materialises them); argmax int32 [b]. */
int oracle_lm_head_argmax(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w,
                          int64_t b, int64_t N, int64_t K, uint16_t *logits, int32_t *argmax,
                          int nthreads) {
    if (!argmax || !logits) return ORACLE_ERR_ARGS;
    int st = oracle_w8a8(q, s_a, w, s_w, b, N, K, logits, nthreads);
    if (st != ORACLE_OK) return st;
    for (int64_t t = 0; t < b; ++t) argmax[t] = oracle_argmax_row(logits + t * N, N);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Power-of-two weight-scale requantization (offline weight preparation).    */
/* ------------------------------------------------------------------------ */

/* Nearest power of two to |s| with the sign of s.  [P3 Abstract] says only
 * "nearest"; reading: write |s| = m * 2^E with m in [1, 2), take 2^E when
 * m < 1.5 and 2^(E+1) otherwise (linear distance, a tie at m = 1.5 goes to
 * the larger power).  s = 0 maps to 0. */
float oracle_pow2_nearest(float s) {
    if (s == 0.0f) return 0.0f;
    int e;
    float f = frexpf(fabsf(s), &e); /* |s| = f * 2^e, f in [0.5, 1) */
    float p = (f < 0.75f) ? ldexpf(1.0f, e - 1) : ldexpf(1.0f, e);
    return s < 0.0f ? -p : p;
}

/* Requantize W8A8 weights to power-of-two scales, re-rounding the weights
 * ([P3 Abstract]: rewriting the scales without re-rounding the weights was
 * the artefact; the intervention that works requantizes).  Per row n:
 *   s'  = nearest power of two of s_w[n]
 *   w'  = clamp(rint_half_even(w * s / s'), -127, 127)
 * w * s has at most 8 + 24 significant bits and s' is a power of two, so the
 * quotient is exact in double and the only rounding is the final rint.
 * A zero scale gives s' = 0 and w' = 0. */
int oracle_pow2_requant(const int8_t *w, const float *s_w, int64_t N, int64_t K, int8_t *w_out,
                        float *s_out) {
    if (!w || !s_w || !w_out || !s_out || N < 1 || K < 1) return ORACLE_ERR_ARGS;
    for (int64_t n = 0; n < N; ++n) {
        float s = s_w[n];
        float sp = oracle_pow2_nearest(s);
        s_out[n] = sp;
        for (int64_t k = 0; k < K; ++k) {
            if (sp == 0.0f) {
                w_out[n * K + k] = 0;
                continue;
            }
            double r = rint((double)w[n * K + k] * (double)s / (double)sp);
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            w_out[n * K + k] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Decode attention over a KV cache in fixed chunks.                          */
/* ------------------------------------------------------------------------ */
/*
 * Sources:
 *  [P1] "the bug that waited for position 384" (Fig. 5): the stock kernel
 *       summed the cache in 128-cell chunks spread over P parallel blocks,
 *       P taken from an occupancy query, so a batched query's last chunk
 *       could join another block's partial and round differently.
 *  [P2] "Fusion that lost": split-KV attention as two kernels, 256-token
 *       chunks computed as independent partials and a merge kernel, and a
 *       fast path that writes the output directly when there is one chunk;
 *       the chunk count must come from the tokens present, not from the
 *       allocated cache.  "Why the decoders disagreed?": cache slots past a
 *       query's position are never read.  "Shipping the 6.4x as its own
 *       backend": a merge order is one valid rounding among many; what
 *       matters is that it is fixed.
 *
 * The pages fix the structure (fixed chunks, partials, a merge) but not the
 * float order inside it.  The recipe below is this library's fixed order,
 * chosen to match the GPU mapping (8-dim score slices = one 16-byte load of
 * keys per lane; 64-cell parts = one wave's cells); witnesses that tell it
 * from the other plausible orders pin it;
 * every step depends only on the query's own row, its position and the
 * cache cells 0..position, never on how many queries share a launch, the
 * cache's allocated size or the grid.  Unlike the linear layer, it uses
 * fused multiply-adds, each one explicit (fmaf, one rounding).
 */

#define ATTN_CHUNK 256
#define ATTN_PART 64 /* a chunk's sums are formed in four parts of 64 cells */
#define ATTN_PARTS 4

/* e^x for x <= 0 (the only arguments the recipe forms) in binary32 operations only (every implementation that
 * performs the same operations gets the same bits).  Cody and Waite's
 * additive reduction x = n ln2 + r, with ln 2 split into a head of 16
 * significant bits (n * head is exact for |n| < 256) and a tail; then the
 * degree-7 Taylor polynomial of e^r (|r| <= ln2/2 + rounding, truncation
 * below 6e-9 relative) in Horner form with fused multiply-adds; then the
 * exact scaling by 2^n built from its exponent field.  For n < -125 the
 * result is 0, so no step produces a subnormal. */
float oracle_attn_exp(float x) {
    const float log2e = 0x1.715476p+0f;  /* fl(1 / ln 2) */
    const float ln2_hi = 0x1.62e4p-1f;   /* 0.693145751953125 */
    const float ln2_lo = 0x1.7f7d1cp-20f; /* fl(ln 2 - ln2_hi) */
    float n = rintf(x * log2e);
    if (n < -125.0f) return 0.0f;
    if (n > 127.0f) n = 127.0f;
    float r = (x - n * ln2_hi) - n * ln2_lo;
    float p = 0x1.a01a02p-13f;          /* 1/7! */
    p = fmaf(p, r, 0x1.6c16c2p-10f);     /* 1/6! */
    p = fmaf(p, r, 0x1.111112p-7f);      /* 1/5! */
    p = fmaf(p, r, 0x1.555556p-5f);      /* 1/4! */
    p = fmaf(p, r, 0x1.555556p-3f);      /* 1/3! */
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return p * bits_f32((uint32_t)((int32_t)n + 127) << 23);
}

/* Score of one query row against one cached key.  qs = q * scale, rounded
 * per element.  D is cut into D/8 slices of 8 consecutive dimensions; each
 * slice is a chain of fused multiply-adds from +0 in increasing d (each step
 * rounds once); the slice sums are then added as an adjacent-pair tree
 * (D/8 a power of two). */
static float attn_score(const float *qs, const uint16_t *k, int64_t D) {
    float part[64];
    int64_t m = D / 8;
    for (int64_t l = 0; l < m; ++l) {
        float a = 0.0f;
        for (int64_t i = 0; i < 8; ++i) a = fmaf(qs[8 * l + i], oracle_bf16_to_f32(k[8 * l + i]), a);
        part[l] = a;
    }
    while (m > 1) {
        for (int64_t i = 0; i < m / 2; ++i) part[i] = part[2 * i] + part[2 * i + 1];
        m /= 2;
    }
    return part[0];
}

typedef struct {
    const uint16_t *q, *k, *v;
    int64_t kc, kh, vc, vh; /* cell and head strides of the caches, in elements */
    int64_t b, Hq, Hkv, D, pos0;
    float scale;
    int64_t h0, h1;         /* heads computed */
    uint16_t *out;
    int64_t r0, r1;         /* this thread's rows, r = t * (h1 - h0) + (hq - h0) */
    int status;
} attn_job;

/* One output row (token t, query head hq):
 *   position p = pos0 + t; the row attends cells 0..p; chunk c holds cells
 *   [256 c, 256 c + 256) cut at p; the row has n = p / 256 + 1 chunks.
 *   Per chunk: s_j = score(q * scale, k_j); m_c = max_j s_j;
 *     e_j = E(s_j - m_c); the chunk is cut into four parts of 64 cells;
 *     per part, l = sum_j e_j and o[d] = sum_j e_j v_j[d], both in increasing
 *     j from +0 (o with fused multiply-adds; an empty part gives +0); then
 *     l_c = (l_0 + l_1) + (l_2 + l_3) and o_c likewise.
 *   Merge in increasing c: M = max_c m_c, w_c = E(m_c - M);
 *     L = w_0 l_0, O[d] = w_0 o_0[d], then L = fma(w_c, l_c, L) and
 *     O[d] = fma(w_c, o_c[d], O[d]) for c = 1, 2, ...
 *   out[d] = bf16(O[d] / L).
 * With one chunk, w_0 = E(0) = 1 and the merge returns o_0 / l_0 exactly:
 * a fast path that skips it gives the same bits. */
static void attn_rows(attn_job *j) {
    const int64_t D = j->D, G = j->Hq / j->Hkv, nh = j->h1 - j->h0;
    float *qs = (float *)malloc(sizeof(float) * (size_t)D);
    float *op = (float *)malloc(sizeof(float) * (size_t)(ATTN_PARTS * D));
    float *O = (float *)malloc(sizeof(float) * (size_t)D);
    float *s = (float *)malloc(sizeof(float) * ATTN_CHUNK);
    if (!qs || !op || !O || !s) {
        j->status = ORACLE_ERR_ARGS;
        free(qs), free(op), free(O), free(s);
        return;
    }
    for (int64_t r = j->r0; r < j->r1; ++r) {
        const int64_t t = r / nh, hq = j->h0 + r % nh, hk = hq / G;
        const int64_t p = j->pos0 + t, nchunks = p / ATTN_CHUNK + 1;
        const uint16_t *qr = j->q + (t * j->Hq + hq) * D;
        for (int64_t d = 0; d < D; ++d) qs[d] = oracle_bf16_to_f32(qr[d]) * j->scale;
        float M = -INFINITY; /* the largest chunk maximum, needed by the merge weights */
        float *mc = (float *)malloc(sizeof(float) * (size_t)nchunks);
        float *lc = (float *)malloc(sizeof(float) * (size_t)nchunks);
        float *oc = (float *)malloc(sizeof(float) * (size_t)(nchunks * D));
        if (!mc || !lc || !oc) {
            j->status = ORACLE_ERR_ARGS;
            free(mc), free(lc), free(oc);
            break;
        }
        for (int64_t c = 0; c < nchunks; ++c) {
            const int64_t c0 = c * ATTN_CHUNK;
            const int64_t c1 = (c0 + ATTN_CHUNK < p + 1) ? c0 + ATTN_CHUNK : p + 1;
            float m = -INFINITY;
            for (int64_t cell = c0; cell < c1; ++cell) {
                s[cell - c0] = attn_score(qs, j->k + cell * j->kc + hk * j->kh, D);
                m = fmaxf(m, s[cell - c0]);
            }
            /* four parts of 64 cells, each summed in increasing j from +0 (an
             * empty part is +0), then joined as (part 0 + part 1) + (part 2 +
             * part 3) */
            float lp[ATTN_PARTS];
            for (int64_t k = 0; k < ATTN_PARTS; ++k) {
                const int64_t a0 = c0 + k * ATTN_PART;
                const int64_t a1 = (a0 + ATTN_PART < c1) ? a0 + ATTN_PART : c1;
                float l = 0.0f;
                float *ok = op + k * D;
                for (int64_t d = 0; d < D; ++d) ok[d] = 0.0f;
                for (int64_t cell = a0; cell < a1; ++cell) {
                    const float e = oracle_attn_exp(s[cell - c0] - m);
                    const uint16_t *vr = j->v + cell * j->vc + hk * j->vh;
                    l = l + e;
                    for (int64_t d = 0; d < D; ++d) ok[d] = fmaf(e, oracle_bf16_to_f32(vr[d]), ok[d]);
                }
                lp[k] = l;
            }
            mc[c] = m;
            lc[c] = (lp[0] + lp[1]) + (lp[2] + lp[3]);
            for (int64_t d = 0; d < D; ++d)
                oc[c * D + d] = (op[d] + op[D + d]) + (op[2 * D + d] + op[3 * D + d]);
            M = fmaxf(M, m);
        }
        float L = 0.0f;
        for (int64_t c = 0; c < nchunks; ++c) {
            const float w = oracle_attn_exp(mc[c] - M);
            if (c == 0) {
                L = w * lc[0];
                for (int64_t d = 0; d < D; ++d) O[d] = w * oc[d];
            } else {
                L = fmaf(w, lc[c], L);
                for (int64_t d = 0; d < D; ++d) O[d] = fmaf(w, oc[c * D + d], O[d]);
            }
        }
        uint16_t *orow = j->out + (t * j->Hq + hq) * D;
        for (int64_t d = 0; d < D; ++d) orow[d] = oracle_bf16_rne(f32_bits(O[d] / L));
        free(mc), free(lc), free(oc);
    }
    free(qs), free(op), free(O), free(s);
}

static void *attn_worker(void *arg) {
    attn_rows((attn_job *)arg);
    return NULL;
}

/* q bf16 [b, Hq, D]; k and v bf16 caches addressed as base + cell * cell_stride
 * + head * head_stride + d (strides in elements); query t sits at position
 * pos0 + t and attends cells 0..pos0 + t.  Query head hq reads kv head
 * hq / (Hq / Hkv).  Writes out bf16 [b, Hq, D] for heads h0 <= hq < h1. */
int oracle_attn_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t k_cell, int64_t k_head,
                       int64_t v_cell, int64_t v_head, int64_t b, int64_t Hq, int64_t Hkv, int64_t D, int64_t pos0,
                       float scale, int64_t h0, int64_t h1, uint16_t *out, int nthreads) {
    if (!q || !k || !v || !out || b < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 8 || D > 512 ||
        (D & (D - 1)) != 0 || pos0 < 0 || h0 < 0 || h1 > Hq || h0 >= h1)
        return ORACLE_ERR_ARGS;
    const int64_t rows = b * (h1 - h0);
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > rows) nthreads = (int)rows;
    attn_job jobs[256];
    pthread_t th[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        attn_job a = {q, k, v, k_cell, k_head, v_cell, v_head, b, Hq, Hkv, D, pos0, scale, h0, h1, out,
                      rows * i / nthreads, rows * (i + 1) / nthreads, ORACLE_OK};
        jobs[i] = a;
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, attn_worker, &jobs[i]) == 0)
            started[i] = 1;
        else
            attn_worker(&jobs[i]);
    }
    attn_worker(&jobs[0]);
    int status = ORACLE_OK;
    for (int i = 1; i < nthreads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) status = jobs[i].status;
    return status;
}

/* ------------------------------------------------------------------------ */
/* FP8 (E4M3) W8A8 linear with a fixed summation tree.                        */
/* ------------------------------------------------------------------------ */
/*
 * Sources:
 *  [P2] "My speculative decoder got slower", "The FP8 kernel that was secretly
 *       FP16" and "A trained drafter and two matmul schedules": projection
 *       weights in FP8; "Two matmul schedules that survived": with split-K the
 *       running float sum is rounded at points set by the block size, so
 *       schedules differ in the last bits.
 *  [P3] "Deterministic LLM Inference Across GPU Kernels ...", Abstract: across
 *       FP8 GEMM implementations the differences grow with the reduction depth
 *       (unlike int8, whose accumulation is exact).
 *
 * Readings: the format is OCP E4M3 (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448).
 * Activations are quantized per token like the int8 path with 448 in place
 * of 127; weights come with one fp32 scale per row.  The product of two E4M3
 * values is exact in binary32 (4 + 4 significant bits, exponents within
 * [-18, 18]), so only the summation order needs fixing: K is cut into groups
 * of 16; each group sum adds its products in increasing k from +0 (one
 * rounding per addition); the K/16 group sums are the leaves of the canonical
 * tree (zero-padded to a power of two, adjacent pairs); the epilogue is the
 * linear layer's, bf16(fl(fl(root * s_a) * s_w)).
 */

float oracle_e4m3_to_f32(uint8_t c) {
    const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexpf((float)m, -9); /* subnormal: m * 2^-9 */
    else
        v = ldexpf((float)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Nearest finite E4M3 value, ties to the even code (mantissa bit 0 clear);
 * magnitudes past 448 saturate to 448; the sign is kept (-0 gives 0x80); NaN
 * gives 0x7F with its sign.  By exhaustive search over the 127 non-negative
 * finite codes; differences are exact in double. */
uint8_t oracle_f32_to_e4m3(float x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return (uint8_t)(sign | 0x7F);
    const double a = fabs((double)x);
    int best = 0;
    double bd = a; /* distance to +0 */
    for (int c = 1; c < 0x7F; ++c) {
        const double d = fabs(a - (double)oracle_e4m3_to_f32((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

/* Per-token FP8 quantization: s = fl(amax / 448), q = e4m3(fl(x / s)); an
 * all-zero token gives s = 0 and q = +0 codes. */
int oracle_quantize_fp8(const uint16_t *x, int64_t b, int64_t K, uint8_t *q, float *s) {
    if (!x || !q || !s || b < 1 || K < 1) return ORACLE_ERR_ARGS;
    for (int64_t t = 0; t < b; ++t) {
        const uint16_t *xr = x + t * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = fabsf(oracle_bf16_to_f32(xr[k]));
            if (v > amax) amax = v;
        }
        const float sc = amax / 448.0f;
        s[t] = sc;
        for (int64_t k = 0; k < K; ++k)
            q[t * K + k] = sc == 0.0f ? 0x00 : oracle_f32_to_e4m3(oracle_bf16_to_f32(xr[k]) / sc);
    }
    return ORACLE_OK;
}

/* Sum of one 16-element group: products in increasing k added from +0. */
static float fp8_group_sum(const uint8_t *a, const uint8_t *w) {
    float s = 0.0f;
    for (int i = 0; i < 16; ++i) s = s + oracle_e4m3_to_f32(a[i]) * oracle_e4m3_to_f32(w[i]);
    return s;
}

typedef struct {
    const uint8_t *q, *w;
    const float *sa, *sw;
    int64_t b, N, K;
    uint16_t *y;
    int64_t n0, n1;
    int status;
} fp8_job;

static void *fp8_worker(void *arg) {
    fp8_job *j = (fp8_job *)arg;
    const int64_t G = j->K / 16;
    float *leaf = (float *)malloc(sizeof(float) * (size_t)G);
    if (!leaf) {
        j->status = ORACLE_ERR_ARGS;
        return NULL;
    }
    for (int64_t n = j->n0; n < j->n1; ++n)
        for (int64_t t = 0; t < j->b; ++t) {
            for (int64_t g = 0; g < G; ++g) leaf[g] = fp8_group_sum(j->q + t * j->K + 16 * g, j->w + n * j->K + 16 * g);
            const float root = oracle_tree_sum(leaf, G);
            const float u = root * j->sa[t];
            j->y[t * j->N + n] = oracle_bf16_rne(f32_bits(u * j->sw[n]));
        }
    free(leaf);
    return NULL;
}

/* q e4m3 [b, K], s_a fp32 [b], w e4m3 [N, K], s_w fp32 [N] -> y bf16 [b, N];
 * K a multiple of 16.  Threads split output rows only. */
int oracle_fp8_linear(const uint8_t *q, const float *s_a, const uint8_t *w, const float *s_w, int64_t b, int64_t N,
                      int64_t K, uint16_t *y, int nthreads) {
    if (!q || !s_a || !w || !s_w || !y || b < 1 || N < 1 || K < 16 || K % 16 != 0) return ORACLE_ERR_ARGS;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > N) nthreads = (int)N;
    fp8_job jobs[256];
    pthread_t th[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        fp8_job jb = {q, w, s_a, s_w, b, N, K, y, N * i / nthreads, N * (i + 1) / nthreads, ORACLE_OK};
        jobs[i] = jb;
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, fp8_worker, &jobs[i]) == 0)
            started[i] = 1;
        else
            fp8_worker(&jobs[i]);
    }
    fp8_worker(&jobs[0]);
    int status = ORACLE_OK;
    for (int i = 1; i < nthreads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) status = jobs[i].status;
    return status;
}


/* ------------------------------------------------------------------------ */
/* k-quant-style superblocks with 6-bit codes (kq6).                          */
/* ------------------------------------------------------------------------ */
/*
 * [P1 "the mat-vec kernel"]: decoding a q6_k matrix reads each 4096-wide row
 * as 16 weight blocks of 256 against int8 activations in blocks of 32; the
 * integer products are exact and each block's integer result is scaled into
 * an fp32 sum.  [P1 opening]: the pages' own decode workload is Qwen3-8B at
 * q4_k_m and q6_k.  The pages give no bit layout, so the layout here is this
 * library's own (not GGUF's), with the same 6.5625 bits per weight:
 *   - a superblock is 256 consecutive weights of a row, s = k / 256;
 *   - each weight is a code c in [-32, 31] stored as u = c + 32 in [0, 63];
 *   - weights go in groups of 16, g = k / 16, i = k % 16;
 *   - low plane  ql uint8 [N, K/2]: the low 4 bits of u for weight k are
 *     bits 4*(i/8) .. +3 of byte 8*g + i%8;
 *   - high plane qh uint8 [N, K/4]: the top 2 bits of u for weight k are
 *     bits 2*(i/4), +1 of byte 4*g + i%4;
 *   - sub-scales sc int8 [N, K/16], one per 16 weights;
 *   - superblock scale d fp16 [N, K/256].
 * Reading (the pages name only the block scaling): a weight's integer value is
 * sc[k/16] * c[k]; per 32-block j of activations, isum_j = sum of
 * (sc * c) * q over its 32 elements, exact in int32 (|isum_j| <= 2^24, so
 * fl32(isum_j) is exact too); the leaf is the blockq8 leaf with the
 * superblock scale, p_j = fl(fl(fl32(isum_j) * d_a[t,j]) * fl32(d[n, j/8]));
 * y = bf16 of the canonical tree over the K/32 leaves.
 */

/* Codes of an [N, K] kq6 matrix from its two planes, element by element. */
int oracle_kq6_decode(const uint8_t *ql, const uint8_t *qh, int64_t N, int64_t K, int8_t *codes) {
    if (!ql || !qh || !codes || N < 1 || K < 256 || K % 256 != 0) return ORACLE_ERR_ARGS;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = k / 16, i = k % 16;
            const int lo = (ql[n * (K / 2) + 8 * g + i % 8] >> (4 * (i / 8))) & 15;
            const int hi = (qh[n * (K / 4) + 4 * g + i % 4] >> (2 * (i / 4))) & 3;
            codes[n * K + k] = (int8_t)((lo | (hi << 4)) - 32);
        }
    return ORACLE_OK;
}

typedef struct {
    const int8_t *q;
    const float *da;
    const int8_t *codes;
    const int8_t *sc;
    const uint16_t *d;
    int64_t b, N, K;
    uint16_t *y;
    int64_t n0, n1;
    int status;
} kq6_job;

static void *kq6_worker(void *arg) {
    kq6_job *j = (kq6_job *)arg;
    const int64_t K = j->K, m = K / 32;
    float *leaf = (float *)malloc(sizeof(float) * (size_t)m);
    if (!leaf) {
        j->status = ORACLE_ERR_ARGS;
        return NULL;
    }
    for (int64_t n = j->n0; n < j->n1; ++n)
        for (int64_t t = 0; t < j->b; ++t) {
            for (int64_t i = 0; i < m; ++i) {
                int32_t isum = 0;
                int64_t shadow = 0;
                for (int64_t k = 32 * i; k < 32 * i + 32; ++k) {
                    const int32_t wv = (int32_t)j->sc[n * (K / 16) + k / 16] * (int32_t)j->codes[n * K + k];
                    isum += wv * (int32_t)j->q[t * K + k];
                    shadow += (int64_t)wv * (int64_t)j->q[t * K + k];
                }
                if ((int64_t)isum != shadow) j->status = ORACLE_ERR_OVERFLOW;
                leaf[i] = oracle_block_partial(isum, j->da[t * m + i], j->d[n * (K / 256) + i / 8]);
            }
            const float root = oracle_tree_sum(leaf, m);
            j->y[t * j->N + n] = oracle_bf16_rne(f32_bits(root));
        }
    free(leaf);
    return NULL;
}

/* q int8 [b, K], d_a fp32 [b, K/32], a kq6 matrix (ql, qh, sc, d as above)
 * -> y bf16 [b, N]; K a multiple of 256.  Threads split output rows only. */
int oracle_kq6_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
                      const uint16_t *d, int64_t b, int64_t N, int64_t K, uint16_t *y, int nthreads) {
    if (!q || !d_a || !ql || !qh || !sc || !d || !y || b < 1 || N < 1 || K < 256 || K % 256 != 0)
        return ORACLE_ERR_ARGS;
    int8_t *codes = (int8_t *)malloc((size_t)(N * K));
    if (!codes) return ORACLE_ERR_ARGS;
    int status = oracle_kq6_decode(ql, qh, N, K, codes);
    if (status != ORACLE_OK) {
        free(codes);
        return status;
    }
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > N) nthreads = (int)N;
    kq6_job jobs[256];
    pthread_t th[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        kq6_job jb = {q, d_a, codes, sc, d, b, N, K, y, N * i / nthreads, N * (i + 1) / nthreads, ORACLE_OK};
        jobs[i] = jb;
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, kq6_worker, &jobs[i]) == 0)
            started[i] = 1;
        else
            kq6_worker(&jobs[i]);
    }
    kq6_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) status = jobs[i].status;
    free(codes);
    return status;
}


/* ------------------------------------------------------------------------ */
/* k-quant-style superblocks with 4-bit codes and minimums (kq4).             */
/* ------------------------------------------------------------------------ */
/*
 * [P1 opening]: the pages' decode workload is Qwen3-8B at q4_k_m; [P1 "the
 * mat-vec kernel"] fixes the integer-then-scale structure per activation block
 * of 32.  The 4-bit form subtracts a per-sub-block minimum.  Layout (this
 * library's own):
 *   - weight k has a code q in [0, 15]; low plane ql uint8 [N, K/2] as kq6:
 *     q of weight k = 16 g + i in bits 4*(i/8) .. +3 of byte 8 g + i%8;
 *   - per 32 weights (one activation block) j: a sub-scale sc_j and a minimum
 *     m_j, both in [0, 63], as the byte pair scm[n, j] = (sc_j, m_j),
 *     uint8 [N, K/32, 2];
 *   - per superblock of 256: the fp16 pair dm[n, s] = (d, dmin), [N, K/256, 2].
 * Reading: weight k stands for d * sc_j * q_k - dmin * m_j.  Per block both
 * integer sums are exact,
 *   isum_j = sc_j * sum q*a  (|isum_j| <= 63 * 32 * 15 * 128 < 2^22),
 *   msum_j = m_j * sum a     (|msum_j| <= 63 * 32 * 128 < 2^18),
 * and each is scaled as the blockq8 leaf is, then subtracted:
 *   p_j = fl( fl(fl(fl32(isum_j) * d_a) * fl32(d)) - fl(fl(fl32(msum_j) * d_a) * fl32(dmin)) );
 * y = bf16 of the canonical tree over the K/32 leaves.
 */

typedef struct {
    const int8_t *q;
    const float *da;
    const uint8_t *ql, *scm;
    const uint16_t *dm;
    int64_t b, N, K;
    uint16_t *y;
    int64_t n0, n1;
    int status;
} kq4_job;

static void *kq4_worker(void *arg) {
    kq4_job *j = (kq4_job *)arg;
    const int64_t K = j->K, m = K / 32;
    float *leaf = (float *)malloc(sizeof(float) * (size_t)m);
    if (!leaf) {
        j->status = ORACLE_ERR_ARGS;
        return NULL;
    }
    for (int64_t n = j->n0; n < j->n1; ++n)
        for (int64_t t = 0; t < j->b; ++t) {
            for (int64_t i = 0; i < m; ++i) {
                const int32_t sc = j->scm[(n * m + i) * 2], mn = j->scm[(n * m + i) * 2 + 1];
                if (sc > 63 || mn > 63) j->status = ORACLE_ERR_ARGS;
                int32_t qa = 0, asum = 0;
                for (int64_t k = 32 * i; k < 32 * i + 32; ++k) {
                    const int32_t code = (j->ql[n * (K / 2) + 8 * (k / 16) + (k % 16) % 8] >> (4 * ((k % 16) / 8))) & 15;
                    qa += code * (int32_t)j->q[t * K + k];
                    asum += (int32_t)j->q[t * K + k];
                }
                const int32_t isum = sc * qa, msum = mn * asum;
                const float da = j->da[t * m + i];
                const uint16_t d = j->dm[(n * (K / 256) + i / 8) * 2], dmin = j->dm[(n * (K / 256) + i / 8) * 2 + 1];
                const float a = oracle_f32_mul(oracle_f32_mul(oracle_i32_to_f32(isum), da), oracle_fp16_to_f32(d));
                const float c = oracle_f32_mul(oracle_f32_mul(oracle_i32_to_f32(msum), da), oracle_fp16_to_f32(dmin));
                leaf[i] = oracle_f32_sub(a, c);
            }
            const float root = oracle_tree_sum(leaf, m);
            j->y[t * j->N + n] = oracle_bf16_rne(f32_bits(root));
        }
    free(leaf);
    return NULL;
}

/* q int8 [b, K], d_a fp32 [b, K/32], a kq4 matrix (ql, scm, dm as above)
 * -> y bf16 [b, N]; K a multiple of 256.  Threads split output rows only.
 * Sub-scales or minimums above 63 give ORACLE_ERR_ARGS. */
int oracle_kq4_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *scm, const uint16_t *dm,
                      int64_t b, int64_t N, int64_t K, uint16_t *y, int nthreads) {
    if (!q || !d_a || !ql || !scm || !dm || !y || b < 1 || N < 1 || K < 256 || K % 256 != 0) return ORACLE_ERR_ARGS;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > N) nthreads = (int)N;
    kq4_job jobs[256];
    pthread_t th[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        kq4_job jb = {q, d_a, ql, scm, dm, b, N, K, y, N * i / nthreads, N * (i + 1) / nthreads, ORACLE_OK};
        jobs[i] = jb;
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, kq4_worker, &jobs[i]) == 0)
            started[i] = 1;
        else
            kq4_worker(&jobs[i]);
    }
    kq4_worker(&jobs[0]);
    int status = ORACLE_OK;
    for (int i = 1; i < nthreads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) status = jobs[i].status;
    return status;
}
