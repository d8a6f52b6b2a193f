/*
 * sanitize_run.c -- drives every entry point of msa_oracle.c once on small
 * ragged inputs so that a build with gcc's AddressSanitizer and
 * UndefinedBehaviorSanitizer can check the oracle's memory accesses and
 * arithmetic.  TEST INFRASTRUCTURE ONLY: tests/test_oracle_sanitizers.py
 * builds and runs it.  It checks only what the oracle's contract states
 * (return codes, id invariants, finite outputs); values are pinned elsewhere.
 * Exits 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int msa_oracle_index_topk_forced(int num_seqs, const int32_t *cu_q, const int32_t *cu_k, int h, int d_idx, int B,
                                 int top_k, int sink, int local, const uint16_t *q_idx, const uint16_t *k_idx,
                                 int64_t n_rows, const int64_t *rows, int32_t *ids, float *kth, uint8_t *near_tie,
                                 int nthreads);
int64_t msa_oracle_block_scores(int num_seqs, const int32_t *cu_q, const int32_t *cu_k, int h, int d_idx, int B,
                                const uint16_t *q_idx, const uint16_t *k_idx, int64_t row, int g, float *S,
                                int64_t capacity);
int msa_oracle_sparse_attention(int num_seqs, const int32_t *cu_q, const int32_t *cu_k, int H, int h, int d, int B,
                                int top_k, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *ids, float scale, int64_t n_rows, const int64_t *rows, float *out,
                                float *lse, int nthreads);
int msa_oracle_sparse_attention_backward(int num_seqs, const int32_t *cu_q, const int32_t *cu_k, int H, int h,
                                         int d, int B, int top_k, const uint16_t *q, const uint16_t *k,
                                         const uint16_t *v, const int32_t *ids, float scale, const uint16_t *dout,
                                         const uint16_t *out, float *dq, float *dk, float *dv, int nthreads);

static uint32_t state = 12345u;
static uint16_t draw_bf16(void) {
    /* small integers and halves in [-4, 4): exact in bf16 */
    state = state * 1664525u + 1013904223u;
    float x = (float)((int)(state >> 24) % 16 - 8) * 0.5f;
    uint32_t bits;
    memcpy(&bits, &x, 4);
    return (uint16_t)(bits >> 16);
}

static uint16_t *bf16_array(size_t n) {
    uint16_t *a = (uint16_t *)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) a[i] = draw_bf16();
    return a;
}

#define CHECK(c, msg)                                   \
    do {                                                \
        if (!(c)) {                                     \
            fprintf(stderr, "sanitize_run: %s\n", msg); \
            return 1;                                   \
        }                                               \
    } while (0)

int main(void) {
    /* three sequences: a prefill with a partial last block, an empty one, a decode-like chunk */
    const int num_seqs = 3, H = 6, h = 2, d = 16, di = 8, B = 16, K = 3;
    const int32_t cu_q[4] = {0, 70, 70, 75};
    const int32_t cu_k[4] = {0, 70, 70, 120};
    const int64_t tq = 75, tk = 120;
    uint16_t *q = bf16_array((size_t)tq * H * d), *k = bf16_array((size_t)tk * h * d);
    uint16_t *v = bf16_array((size_t)tk * h * d), *qi = bf16_array((size_t)tq * h * di);
    uint16_t *ki = bf16_array((size_t)tk * di), *dout = bf16_array((size_t)tq * H * d);
    int64_t rows[75];
    for (int64_t r = 0; r < tq; ++r) rows[r] = r;
    int32_t *ids = (int32_t *)malloc((size_t)tq * h * K * sizeof(int32_t));
    float *kth = (float *)malloc((size_t)tq * h * 2 * sizeof(float));
    uint8_t *tie = (uint8_t *)malloc((size_t)tq * h);
    for (int forced = 0; forced < 2; ++forced) {
        CHECK(msa_oracle_index_topk_forced(num_seqs, cu_q, cu_k, h, di, B, K, forced, forced, qi, ki, tq, rows, ids,
                                           kth, tie, 2) == 0,
              "index_topk failed");
        for (int64_t r = 0; r < tq; ++r) {
            const int s = r < 70 ? 0 : 2;
            const int64_t p = (cu_k[s + 1] - cu_k[s]) - (cu_q[s + 1] - cu_q[s]) + (r - cu_q[s]);
            for (int g = 0; g < h; ++g)
                for (int a = 0; a < K; ++a) {
                    const int32_t j = ids[(r * h + g) * K + a];
                    CHECK(j >= -1 && j <= p / B, "ineligible id");
                }
        }
    }
    float S[16];
    /* row 74: the last of sequence 2 (5 queries over 50 keys), position 49, blocks 0..3 */
    CHECK(msa_oracle_block_scores(num_seqs, cu_q, cu_k, h, di, B, qi, ki, 74, 1, S, 16) == 49 / B + 1,
          "block_scores count");
    CHECK(msa_oracle_block_scores(num_seqs, cu_q, cu_k, h, di, B, qi, ki, 74, 1, S, 2) == -1,
          "block_scores must reject a short buffer");
    CHECK(msa_oracle_block_scores(num_seqs, cu_q, cu_k, h, di, B, qi, ki, 75, 0, S, 16) == -1,
          "block_scores must reject a row past the end");
    float *out = (float *)malloc((size_t)tq * H * d * sizeof(float)), *lse = (float *)malloc((size_t)tq * H * 4);
    CHECK(msa_oracle_sparse_attention(num_seqs, cu_q, cu_k, H, h, d, B, K, q, k, v, ids, 0.25f, tq, rows, out, lse,
                                      2) == 0,
          "sparse_attention failed");
    for (int64_t i = 0; i < tq * H * d; ++i) CHECK(isfinite(out[i]), "non-finite output");
    float *dq = (float *)malloc((size_t)tq * H * d * 4), *dk = (float *)malloc((size_t)tk * h * d * 4);
    float *dv = (float *)malloc((size_t)tk * h * d * 4);
    uint16_t *ob = bf16_array((size_t)tq * H * d);
    for (int given = 0; given < 2; ++given)
        CHECK(msa_oracle_sparse_attention_backward(num_seqs, cu_q, cu_k, H, h, d, B, K, q, k, v, ids, 0.25f, dout,
                                                   given ? ob : NULL, dq, dk, dv, 2) == 0,
              "backward failed");
    /* a duplicate id is rejected */
    ids[0 * K + 1] = ids[0 * K + 0];
    CHECK(msa_oracle_sparse_attention(num_seqs, cu_q, cu_k, H, h, d, B, K, q, k, v, ids, 0.25f, tq, rows, out, lse,
                                      1) != 0 || ids[0] == -1,
          "duplicate ids must be rejected");
    free(q); free(k); free(v); free(qi); free(ki); free(dout); free(ids); free(kth); free(tie);
    free(out); free(lse); free(dq); free(dk); free(dv); free(ob);
    puts("sanitize_run: ok");
    return 0;
}
