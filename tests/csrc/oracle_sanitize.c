/* A host driver that runs every exported oracle function once on small,
 * deterministic inputs, for a build of oracle.c with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py).  It checks
 * return codes only; the values are pinned elsewhere.  Sizes are chosen to
 * reach the edges: ragged K, a padded tree (K = 96 -> 3 leaves of 4), two
 * attention chunks with a short last one, several threads. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quantize_token(const uint16_t *x, int64_t b, int64_t K, int8_t *q, float *s);
int oracle_quantize_block32(const uint16_t *x, int64_t b, int64_t K, int8_t *q, float *d);
int oracle_w8a8(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b, int64_t N, int64_t K,
                uint16_t *y, int nthreads);
int oracle_blockq8(const int8_t *q, const float *d_a, const int8_t *w, const uint16_t *d_w, int64_t b, int64_t N,
                   int64_t K, uint16_t *y, int nthreads);
int oracle_lm_head_argmax(const int8_t *q, const float *s_a, const int8_t *w, const float *s_w, int64_t b, int64_t N,
                          int64_t K, uint16_t *logits, int32_t *argmax, int nthreads);
int oracle_pow2_requant(const int8_t *w, const float *s_w, int64_t N, int64_t K, int8_t *w_out, float *s_out);
int oracle_attn_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t k_cell, int64_t k_head,
                       int64_t v_cell, int64_t v_head, int64_t b, int64_t Hq, int64_t Hkv, int64_t D, int64_t pos0,
                       float scale, int64_t h0, int64_t h1, uint16_t *out, int nthreads);
int oracle_quantize_fp8(const uint16_t *x, int64_t b, int64_t K, uint8_t *q, float *s);
int oracle_fp8_linear(const uint8_t *q, const float *s_a, const uint8_t *w, const float *s_w, int64_t b, int64_t N,
                      int64_t K, uint16_t *y, int nthreads);
int oracle_kq6_decode(const uint8_t *ql, const uint8_t *qh, int64_t N, int64_t K, int8_t *codes);
int oracle_kq6_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
                      const uint16_t *d, int64_t b, int64_t N, int64_t K, uint16_t *y, int nthreads);
int oracle_kq4_linear(const int8_t *q, const float *d_a, const uint8_t *ql, const uint8_t *scm, const uint16_t *dm,
                      int64_t b, int64_t N, int64_t K, uint16_t *y, int nthreads);
float oracle_tree_sum(const float *leaf, int64_t m);

static uint32_t state = 12345u;
static uint32_t next(void) {
    state = state * 1664525u + 1013904223u;
    return state >> 8;
}
/* bf16 bits of a value in about [-4, 4) (exponents 125..129, random mantissa and sign) */
static uint16_t bf16_rand(void) { return (uint16_t)(((next() & 1u) << 15) | ((125u + next() % 5u) << 7) | (next() & 0x7Fu)); }
static int8_t i8_rand(void) { return (int8_t)((int)(next() % 255u) - 127); }
static float scale_rand(void) { return 1e-3f + (float)(next() % 1000u) * 1e-4f; }

#define CHECK(call)                                             \
    do {                                                        \
        int rc_ = (call);                                       \
        if (rc_ != 0) {                                         \
            fprintf(stderr, "%s returned %d\n", #call, rc_);   \
            return 1;                                           \
        }                                                       \
    } while (0)

int main(void) {
    enum { B = 3, N = 19, K = 96, KQ = 512 };
    uint16_t x[B * KQ];
    for (int i = 0; i < B * KQ; ++i) x[i] = bf16_rand();
    memset(x + 2 * KQ, 0, KQ * 2); /* an all-zero token: s = 0 */
    int8_t q[B * KQ], w[N * KQ], w2[N * KQ];
    float s_a[B], d_a[B * KQ / 32], s_w[N], s2[N];
    uint16_t d_w[N * KQ / 32], y[B * N];
    for (int i = 0; i < N * KQ; ++i) w[i] = i8_rand();
    for (int i = 0; i < N; ++i) s_w[i] = scale_rand();
    for (int i = 0; i < N * KQ / 32; ++i) d_w[i] = (uint16_t)(0x1400u + next() % 0x1000u); /* small positive fp16 */
    CHECK(oracle_quantize_token(x, B, K, q, s_a));
    CHECK(oracle_w8a8(q, s_a, w, s_w, B, N, K, y, 4));
    CHECK(oracle_quantize_block32(x, B, K, q, d_a));
    CHECK(oracle_blockq8(q, d_a, w, d_w, B, N, K, y, 4));
    int32_t am[B];
    uint16_t logits[B * N];
    CHECK(oracle_quantize_token(x, B, K, q, s_a));
    CHECK(oracle_lm_head_argmax(q, s_a, w, s_w, B, N, K, logits, am, 3));
    CHECK(oracle_pow2_requant(w, s_w, N, K, w2, s2));
    float leaves[5] = {1.0f, -2.0f, 3.0f, 0.5f, 0.25f};
    (void)oracle_tree_sum(leaves, 5);

    /* decode attention: D = 16, 2 query heads on 1 kv head, 300 cells (two chunks) */
    enum { D = 16, CELLS = 300, AB = 2, HQ = 2 };
    uint16_t *kc = malloc(sizeof(uint16_t) * CELLS * D), *vc = malloc(sizeof(uint16_t) * CELLS * D);
    uint16_t aq[AB * HQ * D], ao[AB * HQ * D];
    if (!kc || !vc) return 1;
    for (int i = 0; i < CELLS * D; ++i) kc[i] = bf16_rand(), vc[i] = bf16_rand();
    for (int i = 0; i < AB * HQ * D; ++i) aq[i] = bf16_rand();
    CHECK(oracle_attn_decode(aq, kc, vc, D, D, D, D, AB, HQ, 1, D, CELLS - AB, 0.25f, 0, HQ, ao, 2));
    free(kc), free(vc);

    /* FP8 */
    uint8_t fq[B * K], fw[N * K];
    float fs[B];
    for (int i = 0; i < N * K; ++i) {
        uint8_t c = (uint8_t)(next() & 0xFFu);
        fw[i] = (c & 0x7Fu) == 0x7Fu ? 0x7Eu : c;
    }
    CHECK(oracle_quantize_fp8(x, B, K, fq, fs));
    CHECK(oracle_fp8_linear(fq, fs, fw, s_w, B, N, K, y, 4));

    /* kq6 / kq4 at K = 512 (two superblocks) */
    uint8_t ql[N * KQ / 2], qh[N * KQ / 4], scm[N * KQ / 16];
    int8_t sc[N * KQ / 16], codes[N * KQ];
    uint16_t d6[N * KQ / 256], dm[N * KQ / 256 * 2];
    for (int i = 0; i < N * KQ / 2; ++i) ql[i] = (uint8_t)next();
    for (int i = 0; i < N * KQ / 4; ++i) qh[i] = (uint8_t)next();
    for (int i = 0; i < N * KQ / 16; ++i) sc[i] = i8_rand(), scm[i] = (uint8_t)(next() % 64u);
    for (int i = 0; i < N * KQ / 256; ++i) d6[i] = (uint16_t)(0x0400u + next() % 0x0400u);
    for (int i = 0; i < N * KQ / 256 * 2; ++i) dm[i] = (uint16_t)(0x0400u + next() % 0x0400u);
    CHECK(oracle_quantize_block32(x, B, KQ, q, d_a));
    CHECK(oracle_kq6_decode(ql, qh, N, KQ, codes));
    CHECK(oracle_kq6_linear(q, d_a, ql, qh, sc, d6, B, N, KQ, y, 4));
    CHECK(oracle_kq4_linear(q, d_a, ql, scm, dm, B, N, KQ, y, 4));
    printf("oracle sanitize run: ok\n");
    return 0;
}
