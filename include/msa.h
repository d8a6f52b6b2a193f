/*
 * msa.h -- C ABI of the MI355X (gfx950) MSA hot path: MiniMax Sparse
 * Attention, index branch (index scores -> Block Max Pool -> per-group TopK)
 * and sparse branch (exact softmax attention over the selected blocks of the
 * original K/V).
 *
 * Sources: "MiniMax Goes Sparse" (atlascloud.ai), section 1 "two-stage
 * processing"; "MiniMax M3 MSA vs Step 3.7 Flash MFA" (ai.air7.fun), section
 * "MSA: a minimal sparse attention".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are bfloat16 (raw bits, msa_bf16_t), token-major and packed over
 *    sequences like FlashAttention's varlen API:
 *        q      [total_q, H, d]        k, v   [total_k, h, d]
 *        q_idx  [total_q, h, d_idx]    k_idx  [total_k, d_idx]  (one shared head)
 *    H = num_heads, h = num_kv_heads (= GQA groups = index queries per token),
 *    d = head_dim, d_idx = index_dim.  Query head q belongs to group q / (H/h).
 *  - cu_seqlens_q / cu_seqlens_k are DEVICE int32 arrays of num_seqs+1
 *    non-decreasing offsets into the packed tensors, with
 *    len_k(s) >= len_q(s) >= 1 for every sequence.
 *  - Positions are bottom-right aligned: query row r of sequence s sits at
 *    p = len_k(s) - len_q(s) + r and sees keys 0..p of its own sequence.
 *    Prefill has len_q = len_k; decode has len_q = 1 (the query sees the
 *    whole cache, its own token included).
 *  - Key blocks of block_size B tokens restart at every sequence; a query at
 *    position p has E = floor(p/B) + 1 eligible blocks (the last one may be
 *    partial).
 *  - All pointers are device pointers unless stated otherwise; every buffer
 *    is owned by the caller.  The library allocates nothing, never frees,
 *    never synchronises; each call validates its arguments on the host,
 *    then enqueues kernels on `stream` and returns.  Calls are reentrant and
 *    keep no state between calls.
 *  - Errors: host-checkable argument problems return a non-zero status
 *    before anything is enqueued.  A failed launch returns
 *    MSA_ERROR_LAUNCH.  Device-side contents (cu_seqlens, topk_ids) are the
 *    caller's contract and are not checked.  No C++ exception crosses the ABI.
 *  - Supported shapes: d in {64, 128}; d_idx in {32, 64}; B in {64, 128};
 *    1 <= H/h <= 16; h <= 64; 1 <= top_k <= 4096.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t msa_bf16_t; /* raw bfloat16 bits */
typedef void *msa_stream_t;  /* a hipStream_t; NULL = the null stream */

typedef enum {
    MSA_SUCCESS = 0,
    MSA_ERROR_INVALID_VALUE = 1, /* null pointer, inconsistent sizes, H % h != 0, ... */
    MSA_ERROR_NOT_SUPPORTED = 2, /* a shape outside the supported set above */
    MSA_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than msa_workspace_size() */
    MSA_ERROR_LAUNCH = 4         /* a kernel launch failed */
} msa_status_t;

typedef enum {
    MSA_OP_INDEX_TOPK = 0,
    MSA_OP_SPARSE_ATTN_PREFILL = 1,
    MSA_OP_SPARSE_ATTN_DECODE = 2
} msa_op_t;

typedef struct {
    int32_t num_seqs;              /* >= 1 */
    int32_t total_q;               /* packed query tokens (>= 0; 0 = nothing to do) */
    int32_t total_k;               /* packed key tokens */
    const int32_t *cu_seqlens_q;   /* device, [num_seqs + 1] */
    const int32_t *cu_seqlens_k;   /* device, [num_seqs + 1] */
    int32_t max_seqlen_q;          /* host: max len_q over sequences (1 = decode) */
    int32_t max_seqlen_k;          /* host: max len_k over sequences */
    int32_t num_heads;             /* H */
    int32_t num_kv_heads;          /* h: GQA groups, one index query each */
    int32_t head_dim;              /* d */
    int32_t index_dim;             /* d_idx */
    int32_t block_size;            /* B: tokens per key block */
    int32_t top_k;                 /* k: blocks kept per (query, group) */
} msa_problem_t;

/*
 * Index branch: one index query per GQA group is scored against the single
 * shared index-key head; token scores are max-pooled to block scores; the top
 * k blocks are kept per (query, group).  ["MiniMax Goes Sparse", section 1,
 * step 1 (index branch); "MiniMax M3 MSA vs Step 3.7 Flash MFA", section
 * "MSA: a minimal sparse attention", first layer.]
 *
 *   s[t]  = sum_c q_idx[row, g, c] * k_idx[t, c]       (float32), t <= p
 *   S[j]  = max_{t in block j, t <= p} s[t]            (Block Max Pool)
 *   keep  = first min(k, E) blocks in (S descending, j ascending) order; ties
 *           go to the lower block id and -0.0 equals +0.0.
 *
 * q_idx    [total_q, h, d_idx] bf16 (device)
 * k_idx    [total_k, d_idx]    bf16 (device)
 * topk_ids [total_q, h, top_k] int32 (device, written): sequence-local block
 *          ids of each row and group in ascending order, -1 in unused slots.
 * workspace: device scratch of at least msa_workspace_size(MSA_OP_INDEX_TOPK)
 *          bytes (block-level scores); NULL allowed only when that size is 0.
 * max_seqlen_q == 1 takes the decode variant (one query per sequence).
 */
msa_status_t msa_index_topk(const msa_problem_t *problem, const msa_bf16_t *q_idx,
                            const msa_bf16_t *k_idx, int32_t *topk_ids, void *workspace,
                            size_t workspace_bytes, msa_stream_t stream);

/*
 * Sparse branch, prefill: every query head attends, with one softmax, to the
 * visible tokens (t <= p) of the blocks its group selected, taken from the
 * original, uncompressed K/V; the heads of a group share the group's
 * selection.  ["MiniMax Goes Sparse", section 1, step 2 (sparse branch);
 * "MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a minimal sparse
 * attention", second layer.]
 *
 * q        [total_q, H, d] bf16;  k, v [total_k, h, d] bf16
 * topk_ids [total_q, h, top_k] int32 as written by msa_index_topk (any id
 *          order is accepted; -1 slots are skipped; ids must be distinct and
 *          eligible)
 * softmax_scale  multiplies q.k (usually 1/sqrt(d))
 * out      [total_q, H, d] bf16 (written)
 * lse      [total_q, H] float32 natural-log sum-exp of the scaled logits
 *          (written), or NULL
 * workspace: at least msa_workspace_size(MSA_OP_SPARSE_ATTN_PREFILL) bytes,
 *          16-byte aligned: an fp16 copy of v (every value scaled by one
 *          power of two that puts max |v| in [2^14, 2^15), undone on the
 *          output) used for the P.V products, plus a few KB.
 */
msa_status_t msa_sparse_attn_prefill(const msa_problem_t *problem, const msa_bf16_t *q,
                                     const msa_bf16_t *k, const msa_bf16_t *v,
                                     const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     msa_stream_t stream);

/*
 * Sparse branch, decode (max_seqlen_q == 1, total_q == num_seqs): the same
 * operation for one query per sequence over its cache, split over the
 * selected blocks and merged by log-sum-exp.  The pages note that at decode
 * each query touches only its selected blocks, which is where the KV-cache
 * bandwidth saving comes from ("MiniMax Goes Sparse", section 3).
 *
 * q [num_seqs, H, d]; k_cache, v_cache [total_k, h, d]; topk_ids [num_seqs, h, top_k];
 * out [num_seqs, H, d] bf16; lse [num_seqs, H] float32 or NULL.
 * workspace: at least msa_workspace_size(MSA_OP_SPARSE_ATTN_DECODE) bytes
 * (split partial outputs).
 */
msa_status_t msa_sparse_attn_decode(const msa_problem_t *problem, const msa_bf16_t *q,
                                    const msa_bf16_t *k_cache, const msa_bf16_t *v_cache,
                                    const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out,
                                    float *lse, void *workspace, size_t workspace_bytes,
                                    msa_stream_t stream);

/* Workspace bytes an entry point needs for `problem` (0 if none).  Returns
 * (size_t)-1 when the problem is invalid or unsupported for that op. */
size_t msa_workspace_size(int op, const msa_problem_t *problem);

/* Static, human-readable text of a status code. */
const char *msa_status_string(msa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
