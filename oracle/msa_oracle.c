/*
 * msa_oracle.c -- plain, slow CPU reference of the MSA (MiniMax Sparse
 * Attention) hot path, in float32.
 *
 * TEST INFRASTRUCTURE ONLY.  It exists to check the HIP path.  Only the test
 * suite, the package smoke check and the benchmark's CPU-baseline leg may load
 * or call it; the product path never does.  It shares no code, header or
 * constant with the HIP library.
 *
 * What it computes follows two pages:
 *   [P4] "MiniMax M3 MSA vs Step 3.7 Flash MFA" (ai.air7.fun), section
 *        "MSA: a minimal sparse attention".
 *   [P5] "MiniMax Goes Sparse" (atlascloud.ai), section 1 "two-stage
 *        processing" (index branch, then sparse branch).
 *
 * Index branch [P4 MSA section; P5 section 1]: one index query per GQA group
 * is dotted with a single index-key head shared by all heads; the token-level
 * scores are max-pooled per key block (Block Max Pool) and the top-k blocks
 * are kept per (query, group).
 * Sparse branch [P4 MSA section; P5 section 1]: the selected blocks are taken
 * from the original, uncompressed K/V and ordinary softmax attention runs over
 * them only; every query head of a group uses that group's selection, heads
 * map to groups contiguously (the figure: Q1..Q3 use I1, Q4..Q6 use I2).
 *
 * Readings where the pages are silent (the Block Max Pool and sparse
 * attention formulas were images and are lost):
 *   - scores are raw dot products (no scale, no activation);
 *   - Block Max Pool = max of the visible token scores of the block; tokens
 *     after the query position are not visible (causal);
 *   - block j is eligible iff it holds at least one visible token, so a query
 *     at position p has E = floor(p/B) + 1 eligible blocks;
 *   - exactly min(k, E) blocks are kept, ordered by (score descending, block
 *     id ascending) -- ties go to the lower id, -0.0 equals +0.0 -- then
 *     emitted in ascending id order and padded with -1 up to k;
 *   - attention is one softmax over the union of the visible tokens of the
 *     kept blocks, logits scaled by the caller's scale (1/sqrt(d));
 *   - positions are bottom-right aligned: query row r of a sequence with
 *     len_q queries and len_k keys sits at p = len_k - len_q + r and sees
 *     keys 0..p (decode: len_q = 1, the query sees the whole cache).
 *
 * Arithmetic: every bf16 input is widened exactly to float32; a bf16 x bf16
 * product is exact in float32, sums run in ascending index order in float32,
 * exp/log are the C library's expf/logf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Sequence holding packed query row `row` (cu_q is non-decreasing). */
static int sequence_of_row(int num_seqs, const int32_t *cu_q, int64_t row)
{
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if ((int64_t)cu_q[mid] <= row) lo = mid; else hi = mid - 1;
    }
    return lo;
}

typedef struct {
    int s;          /* sequence */
    int64_t p;      /* position of the query inside its sequence's keys */
    int64_t k0;     /* packed index of the sequence's first key */
    int64_t len_k;  /* keys in the sequence */
} query_pos_t;

static int locate(int num_seqs, const int32_t *cu_q, const int32_t *cu_k, int64_t row, query_pos_t *qp)
{
    if (row < 0 || row >= cu_q[num_seqs]) return -1;
    int s = sequence_of_row(num_seqs, cu_q, row);
    int64_t len_q = cu_q[s + 1] - cu_q[s];
    int64_t len_k = cu_k[s + 1] - cu_k[s];
    int64_t r = row - cu_q[s];
    if (len_k < len_q) return -1;
    qp->s = s;
    qp->p = len_k - len_q + r;
    qp->k0 = cu_k[s];
    qp->len_k = len_k;
    return 0;
}

/* Index score of one (query, group) against one key token [P4 MSA section:
 * Q_idx . K_idx^T with the index key shared by all heads]. */
static float index_score(const uint16_t *qi, const uint16_t *ki, int d_idx)
{
    float s = 0.0f;
    for (int c = 0; c < d_idx; ++c) s += bf16_to_float(qi[c]) * bf16_to_float(ki[c]);
    return s;
}

/* Block Max Pool for one (query, group) [P5 section 1: token-level scores are
 * compressed to block-level scores]: S_j = max over the visible tokens of
 * block j.  Writes E values, returns E. */
static int64_t block_max_pool(const query_pos_t *qp, const uint16_t *qi, const uint16_t *k_idx,
                              int d_idx, int B, float *S)
{
    int64_t E = qp->p / B + 1;
    for (int64_t j = 0; j < E; ++j) {
        int64_t t_end = (j + 1) * B - 1;
        if (t_end > qp->p) t_end = qp->p;
        float m = -INFINITY;
        for (int64_t t = j * B; t <= t_end; ++t) {
            float s = index_score(qi, k_idx + (qp->k0 + t) * d_idx, d_idx);
            if (s > m) m = s;
        }
        /* one canonical zero: -0.0 and +0.0 are the same score */
        S[j] = (m == 0.0f) ? 0.0f : m;
    }
    return E;
}

typedef struct {
    float score;
    int32_t block;
} cand_t;

/* Selection order: higher score first; equal scores -> lower block id first. */
static int by_score_then_id(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->block > y->block) - (x->block < y->block);
}

static int by_id(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* TopK per (query, group) [P4 MSA section; P5 section 1: TopK decides which
 * KV blocks this layer and this GQA group keep].
 *
 * Optional forced inclusion (not part of the pages' method, which is pure
 * TopK; an option for the attention-sink and local-window blocks that [P5]
 * section 2 and [P4] section "waiting for the technical report" speculate
 * may stand in for the dropped sliding-window branch): blocks 0..sink-1 and
 * the `local` blocks ending at the diagonal block E-1 are always kept, and
 * the other min(k, E) - |forced| slots go to the remaining blocks in the
 * same (score descending, id ascending) order.  sink = local = 0 is plain
 * TopK.  Needs sink + local <= top_k.  Returns 0 or -1. */
static int topk_blocks(const float *S, int64_t E, int top_k, int sink, int local, int32_t *ids, float *kth,
                       uint8_t *near_tie)
{
    if (sink < 0 || local < 0 || sink + local > top_k) return -1;
    cand_t *c = (cand_t *)malloc((size_t)E * sizeof(cand_t));
    if (!c) return -1;
    int64_t m = E < top_k ? E : top_k;
    int64_t nf = 0, nr = 0;   /* forced blocks (straight into ids), ranked rest (into c) */
    for (int64_t j = 0; j < E; ++j) {
        if (j < sink || j >= E - local) {
            ids[nf++] = (int32_t)j;
        } else {
            c[nr].score = S[j];
            c[nr].block = (int32_t)j;
            ++nr;
        }
    }
    qsort(c, (size_t)nr, sizeof(cand_t), by_score_then_id);
    int64_t take = m - nf;   /* >= 0: nf <= min(sink + local, E) <= m */
    for (int64_t i = 0; i < take; ++i) ids[nf + i] = c[i].block;
    qsort(ids, (size_t)m, sizeof(int32_t), by_id);
    for (int64_t i = m; i < top_k; ++i) ids[i] = -1;
    /* near-tie: the last kept and the first dropped ranked scores differ by
     * <= 1e-3 relative (with nothing forced: the k-th and (k+1)-th scores) */
    if (take > 0 && nr > take) {
        float a = c[take - 1].score, b = c[take].score;
        kth[0] = a;
        kth[1] = b;
        float mag = fabsf(a) > fabsf(b) ? fabsf(a) : fabsf(b);
        *near_tie = (a - b) <= 1e-3f * mag;
    } else {
        kth[0] = NAN;
        kth[1] = NAN;
        *near_tie = 0;
    }
    free(c);
    return 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * Index branch for a list of packed query rows.
 *   q_idx [total_q, h, d_idx] bf16, k_idx [total_k, d_idx] bf16
 *   sink, local: forced blocks (see topk_blocks; 0, 0 = plain TopK)
 *   ids   [n_rows, h, top_k] int32 out, kth [n_rows, h, 2] float out
 *   (last kept and first dropped ranked score, NaN when nothing is
 *   dropped), near_tie [n_rows, h] uint8 out.
 * Returns 0, or -1 on a bad row / allocation failure.
 */
int msa_oracle_index_topk_forced(int num_seqs, const int32_t *cu_q, const int32_t *cu_k,
                                 int h, int d_idx, int B, int top_k, int sink, int local,
                                 const uint16_t *q_idx, const uint16_t *k_idx,
                                 int64_t n_rows, const int64_t *rows,
                                 int32_t *ids, float *kth, uint8_t *near_tie, int nthreads)
{
    if (num_seqs < 1 || h < 1 || d_idx < 1 || B < 1 || top_k < 1) return -1;
    if (sink < 0 || local < 0 || sink + local > top_k) return -1;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_rows * h; ++task) {
        int64_t i = task / h;
        int g = (int)(task % h);
        query_pos_t qp;
        if (locate(num_seqs, cu_q, cu_k, rows[i], &qp)) { err = 1; continue; }
        int64_t E = qp.p / B + 1;
        float *S = (float *)malloc((size_t)E * sizeof(float));
        if (!S) { err = 1; continue; }
        const uint16_t *qi = q_idx + (rows[i] * h + g) * (int64_t)d_idx;
        block_max_pool(&qp, qi, k_idx, d_idx, B, S);
        if (topk_blocks(S, E, top_k, sink, local, ids + task * top_k, kth + task * 2, near_tie + task)) err = 1;
        free(S);
    }
    return err ? -1 : 0;
}

/* Plain TopK (no forced blocks). */
int msa_oracle_index_topk(int num_seqs, const int32_t *cu_q, const int32_t *cu_k,
                          int h, int d_idx, int B, int top_k,
                          const uint16_t *q_idx, const uint16_t *k_idx,
                          int64_t n_rows, const int64_t *rows,
                          int32_t *ids, float *kth, uint8_t *near_tie, int nthreads)
{
    return msa_oracle_index_topk_forced(num_seqs, cu_q, cu_k, h, d_idx, B, top_k, 0, 0, q_idx, k_idx, n_rows, rows,
                                        ids, kth, near_tie, nthreads);
}

/*
 * Block-level scores S_j (j < E) of one (row, group); returns E, or -1.
 */
int64_t msa_oracle_block_scores(int num_seqs, const int32_t *cu_q, const int32_t *cu_k,
                                int h, int d_idx, int B, const uint16_t *q_idx, const uint16_t *k_idx,
                                int64_t row, int g, float *S, int64_t capacity)
{
    query_pos_t qp;
    if (g < 0 || g >= h || locate(num_seqs, cu_q, cu_k, row, &qp)) return -1;
    if (qp.p / B + 1 > capacity) return -1;
    return block_max_pool(&qp, q_idx + (row * h + g) * (int64_t)d_idx, k_idx, d_idx, B, S);
}

/*
 * Sparse branch for a list of packed query rows [P4 MSA section: standard
 * softmax attention over the selected blocks of the original K/V only;
 * P5 section 1: Q in R^{n x H x d}, K, V in R^{n x h x d}].
 *   q [total_q, H, d], k/v [total_k, h, d] bf16
 *   ids [n_rows, h, top_k]: block ids of each row's group (-1 = unused slot;
 *        any order; every id must be eligible and ids must be distinct)
 *   out [n_rows, H, d] float32, lse [n_rows, H] float32 (natural log).
 * Head q uses group q / (H / h).  Returns 0, or -1 on bad input.
 */
int msa_oracle_sparse_attention(int num_seqs, const int32_t *cu_q, const int32_t *cu_k,
                                int H, int h, int d, int B, int top_k,
                                const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *ids, float scale,
                                int64_t n_rows, const int64_t *rows,
                                float *out, float *lse, int nthreads)
{
    if (num_seqs < 1 || h < 1 || H < h || H % h || d < 1 || B < 1 || top_k < 1) return -1;
    const int G = H / h;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_rows * H; ++task) {
        int64_t i = task / H;
        int head = (int)(task % H);
        int g = head / G;
        query_pos_t qp;
        if (locate(num_seqs, cu_q, cu_k, rows[i], &qp)) { err = 1; continue; }
        int64_t E = qp.p / B + 1;
        const int32_t *sel = ids + (i * h + g) * (int64_t)top_k;
        int bad = 0;
        for (int a = 0; a < top_k; ++a) {
            if (sel[a] < -1 || sel[a] >= E) bad = 1;
            for (int b = 0; b < a; ++b)
                if (sel[a] >= 0 && sel[a] == sel[b]) bad = 1;
        }
        float *logit = (float *)malloc((size_t)top_k * B * sizeof(float));
        int64_t *tok = (int64_t *)malloc((size_t)top_k * B * sizeof(int64_t));
        float *acc = (float *)calloc((size_t)d, sizeof(float));
        if (bad || !logit || !tok || !acc) { err = 1; free(logit); free(tok); free(acc); continue; }
        const uint16_t *qr = q + (rows[i] * H + head) * (int64_t)d;
        /* T = visible tokens of the selected blocks, in the order the ids are given */
        int64_t n = 0;
        for (int a = 0; a < top_k; ++a) {
            if (sel[a] < 0) continue;
            for (int64_t t = (int64_t)sel[a] * B; t < (int64_t)(sel[a] + 1) * B && t <= qp.p; ++t) {
                const uint16_t *kt = k + ((qp.k0 + t) * h + g) * (int64_t)d;
                float s = 0.0f;
                for (int c = 0; c < d; ++c) s += bf16_to_float(qr[c]) * bf16_to_float(kt[c]);
                logit[n] = s * scale;
                tok[n] = qp.k0 + t;
                ++n;
            }
        }
        float M = -INFINITY;
        for (int64_t a = 0; a < n; ++a) if (logit[a] > M) M = logit[a];
        float Z = 0.0f;
        for (int64_t a = 0; a < n; ++a) {
            float w = expf(logit[a] - M);
            Z += w;
            const uint16_t *vt = v + (tok[a] * h + g) * (int64_t)d;
            for (int c = 0; c < d; ++c) acc[c] += w * bf16_to_float(vt[c]);
        }
        float *o = out + (i * H + head) * (int64_t)d;
        for (int c = 0; c < d; ++c) o[c] = (n > 0) ? acc[c] / Z : 0.0f;
        if (lse) lse[i * H + head] = (n > 0) ? M + logf(Z) : -INFINITY;
        free(logit); free(tok); free(acc);
    }
    return err ? -1 : 0;
}

/*
 * Backward of the sparse branch for a fixed selection (the ids are an input
 * and are not differentiated).  With P_t the softmax weights of one (row,
 * head) over its visible selected tokens T, O = sum_t P_t v_t and dO the
 * incoming gradient of O, the chain rule through softmax gives
 *     dP_t = dO . v_t,   D = sum_t P_t dP_t,   dS_t = P_t (dP_t - D),
 *     dq   = scale * sum_t dS_t k_t,
 *     dk_t += scale * dS_t q,   dv_t += P_t dO   (summed over every row and
 *     head of the group that sees token t).
 * The pages define only the forward pass; training through the sparse branch
 * is an open point there ([P4] section "waiting for the technical report":
 * hard or soft top-k in training is unknown).  This is the plain gradient of
 * the forward above with the selection held fixed.
 *   q [total_q, H, d], k/v [total_k, h, d], dout [total_q, H, d] bf16
 *   ids [total_q, h, top_k] (every row)
 *   dq [total_q, H, d], dk/dv [total_k, h, d] float32 out (fully written).
 * Parallel over groups (each thread owns its group's dk/dv).  Returns 0 or -1.
 */
int msa_oracle_sparse_attention_backward(int num_seqs, const int32_t *cu_q, const int32_t *cu_k,
                                         int H, int h, int d, int B, int top_k,
                                         const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                         const int32_t *ids, float scale, const uint16_t *dout,
                                         const uint16_t *out,
                                         float *dq, float *dk, float *dv, int nthreads)
{
    if (num_seqs < 1 || h < 1 || H < h || H % h || d < 1 || B < 1 || top_k < 1) return -1;
    const int G = H / h;
    const int64_t total_q = cu_q[num_seqs], total_k = cu_k[num_seqs];
    memset(dq, 0, (size_t)total_q * H * d * sizeof(float));
    memset(dk, 0, (size_t)total_k * h * d * sizeof(float));
    memset(dv, 0, (size_t)total_k * h * d * sizeof(float));
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int g = 0; g < h; ++g) {
        float *P = (float *)malloc((size_t)top_k * B * sizeof(float));
        float *dP = (float *)malloc((size_t)top_k * B * sizeof(float));
        int64_t *tok = (int64_t *)malloc((size_t)top_k * B * sizeof(int64_t));
        if (!P || !dP || !tok) { err = 1; free(P); free(dP); free(tok); continue; }
        for (int64_t row = 0; row < total_q; ++row) {
            query_pos_t qp;
            if (locate(num_seqs, cu_q, cu_k, row, &qp)) { err = 1; break; }
            const int64_t E = qp.p / B + 1;
            const int32_t *sel = ids + (row * h + g) * (int64_t)top_k;
            int bad = 0;
            for (int a = 0; a < top_k; ++a) {
                if (sel[a] < -1 || sel[a] >= E) bad = 1;
                for (int b = 0; b < a; ++b)
                    if (sel[a] >= 0 && sel[a] == sel[b]) bad = 1;
            }
            if (bad) { err = 1; break; }
            int64_t n = 0;
            for (int a = 0; a < top_k; ++a) {
                if (sel[a] < 0) continue;
                for (int64_t t = (int64_t)sel[a] * B; t < (int64_t)(sel[a] + 1) * B && t <= qp.p; ++t)
                    tok[n++] = qp.k0 + t;
            }
            for (int head = g * G; head < (g + 1) * G; ++head) {
                const uint16_t *qr = q + (row * H + head) * (int64_t)d;
                const uint16_t *dor = dout + (row * H + head) * (int64_t)d;
                /* forward weights */
                float M = -INFINITY;
                for (int64_t a = 0; a < n; ++a) {
                    const uint16_t *kt = k + (tok[a] * h + g) * (int64_t)d;
                    float s = 0.0f;
                    for (int c = 0; c < d; ++c) s += bf16_to_float(qr[c]) * bf16_to_float(kt[c]);
                    P[a] = s * scale;
                    if (P[a] > M) M = P[a];
                }
                float Z = 0.0f;
                for (int64_t a = 0; a < n; ++a) {
                    P[a] = expf(P[a] - M);
                    Z += P[a];
                }
                for (int64_t a = 0; a < n; ++a) P[a] /= Z;
                /* dP_t = dO . v_t and D = sum_t P_t dP_t (= dO . O for the exact
                 * output O); when the caller hands in the forward's output
                 * `out` (bf16, as a backward receives it), D = dO . out */
                float Dsum = 0.0f;
                for (int64_t a = 0; a < n; ++a) {
                    const uint16_t *vt = v + (tok[a] * h + g) * (int64_t)d;
                    float s = 0.0f;
                    for (int c = 0; c < d; ++c) s += bf16_to_float(dor[c]) * bf16_to_float(vt[c]);
                    dP[a] = s;
                    Dsum += P[a] * s;
                }
                if (out != NULL) {
                    const uint16_t *orow = out + (row * H + head) * (int64_t)d;
                    Dsum = 0.0f;
                    for (int c = 0; c < d; ++c) Dsum += bf16_to_float(dor[c]) * bf16_to_float(orow[c]);
                }
                float *dqr = dq + (row * H + head) * (int64_t)d;
                for (int64_t a = 0; a < n; ++a) {
                    const float dS = P[a] * (dP[a] - Dsum);
                    const uint16_t *kt = k + (tok[a] * h + g) * (int64_t)d;
                    float *dkt = dk + (tok[a] * h + g) * (int64_t)d;
                    float *dvt = dv + (tok[a] * h + g) * (int64_t)d;
                    for (int c = 0; c < d; ++c) {
                        dqr[c] += scale * dS * bf16_to_float(kt[c]);
                        dkt[c] += scale * dS * bf16_to_float(qr[c]);
                        dvt[c] += P[a] * bf16_to_float(dor[c]);
                    }
                }
            }
        }
        free(P); free(dP); free(tok);
    }
    return err ? -1 : 0;
}
