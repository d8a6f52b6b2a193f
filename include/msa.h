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
 *    non-decreasing offsets into the packed tensors, starting at 0 and
 *    ending at total_q / total_k, with len_k(s) >= len_q(s) >= 0 for every
 *    sequence: a sequence may have no queries (it is skipped), and
 *    max_seqlen_q / max_seqlen_k must be at least the largest lengths.
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
 *    caller's contract and are not checked, except in the debug mode: with
 *    the environment variable MSA_DEBUG_VALIDATE set (to anything but "" or
 *    "0"), every entry point that reads them first copies cu_seqlens_q,
 *    cu_seqlens_k and the ids it consumes to the host on `stream`, waits for
 *    the copies (the one case where a call synchronises) and checks them with
 *    msa_validate_host, returning MSA_ERROR_INVALID_VALUE before any launch
 *    if they break the contract.  No C++ exception crosses the ABI.
 *  - Supported shapes: d in {64, 128}; d_idx in {32, 64}; B in {64, 128};
 *    1 <= H/h <= 16; h <= 64; 1 <= top_k <= 4096.
 *  - Workspaces are bounded: where a workspace grows with the number of query
 *    rows (the index branch's block scores, the block-centric schedule's
 *    lists and partial outputs, the backward's lists and dq partials), the
 *    call splits the rows into chunks processed one after another, so that
 *    msa_workspace_size stays at or below MSA_WORKSPACE_CAP_BYTES.  Parts
 *    that do not grow with the rows stay whole: the block-centric lists'
 *    per-block counts, the backward's dO.O per row and, when it runs in
 *    several chunks, its float32 dk and dv accumulators (8 total_k h d
 *    bytes); the query-tile schedule's workspace is a copy of V.  A chunk has
 *    at least one row, so a problem whose single row needs more than the cap
 *    still runs, with a workspace of that size.  Results do not depend on the
 *    chunking, up to the order of float32 additions in dk and dv.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The workspace cap (see the conventions above): 8 GiB. */
#define MSA_WORKSPACE_CAP_BYTES ((size_t)8 << 30)

typedef uint16_t msa_bf16_t; /* raw bfloat16 bits */
typedef void *msa_stream_t;  /* a hipStream_t; NULL = the null stream */

typedef enum {
    MSA_SUCCESS = 0,
    MSA_ERROR_INVALID_VALUE = 1, /* null pointer, inconsistent sizes, H % h != 0, ... */
    MSA_ERROR_NOT_SUPPORTED = 2, /* a shape outside the supported set above */
    MSA_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than msa_workspace_size() */
    MSA_ERROR_LAUNCH = 4,        /* a kernel launch failed */
    /* not a status: makes every non-negative 32-bit value a valid
     * msa_status_t, so msa_status_string may be handed any code */
    MSA_STATUS_RANGE_ = 0x7fffffff
} msa_status_t;

typedef enum {
    MSA_OP_INDEX_TOPK = 0,
    MSA_OP_SPARSE_ATTN_PREFILL = 1,
    MSA_OP_SPARSE_ATTN_DECODE = 2,
    MSA_OP_SPARSE_ATTN_BACKWARD = 3,
    MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS = 4,
    MSA_OP_SPARSE_ATTN_PREFILL_TILES = 5
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
 * max_seqlen_q == 1 with total_q == num_seqs (one query per sequence) takes
 * the decode variant, a bandwidth-bound scan; any other batch, empty
 * sequences included, takes the prefill variant.
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
 *          16-byte aligned; its size depends on the schedule chosen below.
 *
 * Two schedules compute this, and the call picks the one expected to be
 * faster for the problem's shape (its choice depends only on the host-side
 * fields of the problem, so msa_workspace_size gives the matching size):
 *  - query tiles (msa_sparse_attn_prefill_tiles): a workgroup stages the
 *    union of its queries' blocks; best while a staged block serves many of
 *    the tile's queries (short contexts, large top_k);
 *  - block-centric (msa_sparse_attn_prefill_blocks): best at long contexts
 *    with a small top_k, where the tiles' unions cover nearly every block.
 * Both give the same result to rounding.
 */
msa_status_t msa_sparse_attn_prefill(const msa_problem_t *problem, const msa_bf16_t *q,
                                     const msa_bf16_t *k, const msa_bf16_t *v,
                                     const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     msa_stream_t stream);

/*
 * msa_sparse_attn_prefill on the query-tile schedule.  A workgroup owns up to
 * 64 consecutive queries of one group (all G heads), forms the union of the
 * blocks they selected and streams each union block through LDS once.
 * Arguments, layouts and errors as for msa_sparse_attn_prefill.
 * workspace: at least msa_workspace_size(MSA_OP_SPARSE_ATTN_PREFILL_TILES)
 * bytes, 16-byte aligned: an fp16 copy of v (the values of each (sequence,
 * KV head) scaled by one power of two that puts their max |v| in
 * [2^14, 2^15), undone on that group's output) used for the P.V products,
 * plus per-(sequence, head) chunk maxima and exponents (a few KB to MB),
 * among them the wait word (see
 * msa_workspace_wait_word): the waves of a workgroup hand staged K/V
 * sub-blocks to one another through LDS, and each hand-off wait is bounded;
 * a wait that reaches its bound is counted there and the output of that
 * call is then not valid.
 */
msa_status_t msa_sparse_attn_prefill_tiles(const msa_problem_t *problem, const msa_bf16_t *q,
                                           const msa_bf16_t *k, const msa_bf16_t *v, const int32_t *topk_ids,
                                           float softmax_scale, msa_bf16_t *out, float *lse, void *workspace,
                                           size_t workspace_bytes, msa_stream_t stream);

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

/*
 * msa_sparse_attn_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same problem, arguments, layouts,
 * result and errors as msa_sparse_attn_decode (the same kernels run), except
 * that the split partials live in a fixed device array inside the library:
 * MSA_DECODE_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load
 * until the process ends.  A problem whose
 * msa_workspace_size(MSA_OP_SPARSE_ATTN_DECODE) exceeds that returns
 * MSA_ERROR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing and frees nothing; its first call on a GPU looks the array's
 * address up on that GPU (the current device) once.  Every call on one GPU
 * shares that GPU's array, which keeps the last call's partials (nothing in
 * it needs clearing: each split writes its partial before the merge reads
 * it): calls that overlap in time on one GPU -- on different streams, or
 * from threads without an order between them -- race and give wrong
 * results; calls ordered on one stream do not.
 */
#define MSA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
msa_status_t msa_sparse_attn_decode_noalloc(const msa_problem_t *problem, const msa_bf16_t *q,
                                            const msa_bf16_t *k_cache, const msa_bf16_t *v_cache,
                                            const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out,
                                            float *lse, msa_stream_t stream);

/*
 * msa_sparse_attn_prefill on the block-centric ("KV-outer, gather-Q")
 * schedule: the same result, computed key block by key block.  The pages
 * name this operator flow ("深度解析M3多模态模型与Token Plan", section 二.2)
 * and their block-sparse prior art turns query-centric selections into
 * per-block lists of queries for it ("MoBA / FlashMoBA" page, section 3.1).
 * Each (group, block) of K/V is read once; each (row, selected slot, head)
 * leaves a normalised partial output that a last pass merges by
 * log-sum-exp.
 *
 * Arguments, layouts and errors as for msa_sparse_attn_prefill.
 * workspace: at least msa_workspace_size(MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS)
 * bytes, 16-byte aligned: the per-(group, block) lists and one fp16 partial
 * per (row, selected slot, head) -- total_q * top_k * H * (2 d + 8) bytes, the
 * bulk of it (8.7 GB for 32K tokens, 32 heads, k = 32).  Results are
 * reproducible bit for bit (each row's partials merge in slot order).  Needs
 * H/h <= 16 and total_q * top_k < 2^31 (MSA_ERROR_NOT_SUPPORTED otherwise).
 */
msa_status_t msa_sparse_attn_prefill_blocks(const msa_problem_t *problem, const msa_bf16_t *q,
                                            const msa_bf16_t *k, const msa_bf16_t *v, const int32_t *topk_ids,
                                            float softmax_scale, msa_bf16_t *out, float *lse, void *workspace,
                                            size_t workspace_bytes, msa_stream_t stream);

/*
 * Backward of the sparse branch, prefill, with the selection held fixed (the
 * ids are constants, not differentiated).  The pages define the forward pass
 * only and leave open whether training uses a hard or soft top-k ("MiniMax
 * M3 MSA vs Step 3.7 Flash MFA", section on waiting for the technical
 * report); this is the gradient of msa_sparse_attn_prefill's output for the
 * given ids:
 *     P_t = exp(scale q.k_t - lse),  dS_t = P_t (dO.v_t - dO.O),
 *     dq = scale sum_t dS_t k_t,  dk_t = scale sum dS_t q,  dv_t = sum P_t dO
 * (dk, dv summed over every row and head of the group that sees token t).
 *
 * q, out, dout [total_q, H, d] bf16; k, v [total_k, h, d] bf16;
 * topk_ids [total_q, h, top_k] as for msa_sparse_attn_prefill;
 * lse [total_q, H] float32 from the forward call (required);
 * dq [total_q, H, d], dk, dv [total_k, h, d] bf16, written (tokens that no row
 * sees get zero dk/dv).
 * workspace: at least msa_workspace_size(MSA_OP_SPARSE_ATTN_BACKWARD)
 * bytes, 16-byte aligned: dO.O per row, one bf16 partial of dq per (row,
 * selected slot, head) -- total_q * top_k * H * d * 2 bytes, the bulk of it
 * (8.6 GB for 32K tokens, 32 heads, k = 32) -- and the per-(group, block)
 * lists of selecting queries.  dk/dv sums run in list order; each list is
 * sorted first, so dq, dk and dv are bitwise reproducible from call to call
 * as long as no key block is selected by more than 16384 rows of one row
 * chunk (longer lists keep the order the count pass's atomics gave them,
 * and their dk/dv agree only to rounding).  Needs H/h <= 32 and
 * total_q * top_k < 2^31.
 */
msa_status_t msa_sparse_attn_prefill_backward(const msa_problem_t *problem, const msa_bf16_t *q,
                                              const msa_bf16_t *k, const msa_bf16_t *v, const int32_t *topk_ids,
                                              float softmax_scale, const msa_bf16_t *out, const float *lse,
                                              const msa_bf16_t *dout, msa_bf16_t *dq, msa_bf16_t *dk,
                                              msa_bf16_t *dv, void *workspace, size_t workspace_bytes,
                                              msa_stream_t stream);

/*
 * Paged KV cache (decode).  The pages keep the cache in the native GQA
 * layout, one physical block of B tokens per page with the K/V slices of
 * every group, and the index branch only picks which blocks to read
 * ("深度解析M3多模态模型与Token Plan", section 二.1 on storage/compute
 * decoupling: GQA physical blocks in a cache pool; "MiniMax M3 MSA vs Step
 * 3.7 Flash MFA", section on the three deliberate subtractions: with GQA the
 * serving engines' caches are reused unchanged).  Only the addressing
 * differs from the contiguous entry points; the arithmetic is the same, so
 * a paged call returns exactly what the contiguous call returns on the same
 * logical cache.
 *
 * Pools (device, caller-owned):
 *     k_pool, v_pool  [num_pages * B, h, d]     k_idx_pool  [num_pages * B, d_idx]
 * Page i holds pool rows i*B .. i*B + B - 1.  Token t of sequence s lives in
 * pool row block_table[s * max_blocks_per_seq + t / B] * B + t % B, where
 * len(s) = cu_seqlens_k[s+1] - cu_seqlens_k[s] (cu_seqlens_k then only gives
 * the lengths; total_k is their sum).  Page ids outside [0, num_pages) are
 * clamped into it, which keeps every access inside the pools (the result is
 * then meaningless, never a fault).  Several sequences may share a page
 * (e.g. a common prefix).
 */
typedef struct {
    const int32_t *block_table; /* device, [num_seqs, max_blocks_per_seq] page ids */
    int32_t max_blocks_per_seq; /* row stride of block_table, >= ceil(max_seqlen_k / B) */
    int32_t num_pages;          /* pages in each pool, >= 1 */
} msa_paged_kv_t;

/* msa_index_topk for decode (max_seqlen_q == 1, total_q == num_seqs) over a
 * paged index-key cache.  Same workspace as msa_index_topk
 * (msa_workspace_size(MSA_OP_INDEX_TOPK, problem)).  Other shapes return
 * MSA_ERROR_NOT_SUPPORTED. */
msa_status_t msa_index_topk_paged(const msa_problem_t *problem, const msa_paged_kv_t *paged,
                                  const msa_bf16_t *q_idx, const msa_bf16_t *k_idx_pool, int32_t *topk_ids,
                                  void *workspace, size_t workspace_bytes, msa_stream_t stream);

/* msa_sparse_attn_decode over paged K/V pools.  Same workspace as
 * msa_sparse_attn_decode (msa_workspace_size(MSA_OP_SPARSE_ATTN_DECODE,
 * problem)). */
msa_status_t msa_sparse_attn_decode_paged(const msa_problem_t *problem, const msa_paged_kv_t *paged,
                                          const msa_bf16_t *q, const msa_bf16_t *k_pool, const msa_bf16_t *v_pool,
                                          const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out, float *lse,
                                          void *workspace, size_t workspace_bytes, msa_stream_t stream);

/* Append: copy num_tokens new rows of k, v [num_tokens, h, d] and k_idx
 * [num_tokens, d_idx] (device, bf16) into the pools at pool row
 * slot_mapping[i] (device int32; the caller derives it from its block table
 * as page * B + offset).  Slots < 0 are skipped (padding); slots >= pool_rows
 * are skipped too, so a bad slot never writes outside the pools.  Rows with
 * equal slots race (the caller's contract).  d in {64, 128}; d_idx in
 * {32, 64}; 1 <= h <= 64.  No workspace. */
msa_status_t msa_kv_append_paged(int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t index_dim,
                                 int64_t pool_rows, const int32_t *slot_mapping, const msa_bf16_t *k,
                                 const msa_bf16_t *v, const msa_bf16_t *k_idx, msa_bf16_t *k_pool,
                                 msa_bf16_t *v_pool, msa_bf16_t *k_idx_pool, msa_stream_t stream);

/*
 * Selection options.  The pages' method is pure TopK (all fields 0).  Their
 * authors speculate that the dropped sliding-window branch may be replaced by
 * an attention sink or a local window ("MiniMax Goes Sparse", section 2, on
 * the three trade-offs; "MiniMax M3 MSA vs Step 3.7 Flash MFA", section on
 * waiting for the technical report).  These options force such blocks into
 * every selection:
 *   sink_blocks   blocks 0 .. sink_blocks-1 (those that are eligible);
 *   local_blocks  the local_blocks eligible blocks ending at the query's own
 *                 (diagonal) block E-1.
 * The other min(k, E) - |forced| slots go to the remaining blocks in the
 * usual (score descending, block id ascending) order; ids stay ascending.
 * Requires sink_blocks, local_blocks >= 0 and sink_blocks + local_blocks <=
 * top_k.  A dense-fallback layer needs no option: top_k >= ceil(max_len / B)
 * selects every eligible block, i.e. dense causal attention.
 */
typedef struct {
    int32_t sink_blocks;
    int32_t local_blocks;
} msa_select_options_t;

/* msa_index_topk with selection options (NULL = plain TopK) over a
 * contiguous cache (paged == NULL) or a paged one (decode only, see
 * msa_paged_kv_t).  Same workspace as msa_index_topk. */
msa_status_t msa_index_topk_ex(const msa_problem_t *problem, const msa_select_options_t *options,
                               const msa_paged_kv_t *paged, const msa_bf16_t *q_idx, const msa_bf16_t *k_idx,
                               int32_t *topk_ids, void *workspace, size_t workspace_bytes, msa_stream_t stream);

/*
 * Measurement helpers, not part of the method: the achievable ceilings that
 * the method's kernels are compared with, next to the published peaks.
 *
 * msa_ceiling_stream_read reads the first *bytes_read bytes of `buffer`
 * (device, 16-byte aligned) once with full-line non-temporal loads (which
 * stream past L2 and the MALL without settling there, as the decode's K/V
 * gathers do for large selections) and writes nothing but,
 * in the rarest case, one word of `sink` (device, 4 bytes).  *bytes_read
 * (host) is set before the launch to the largest multiple of the per-launch
 * stride (256 KB per compute unit) that fits in buffer_bytes; a buffer smaller
 * than one stride is rejected.
 *
 * msa_ceiling_mfma_bf16 runs `iterations` rounds of eight independent
 * v_mfma_f32_16x16x32_bf16 per wave, two waves per SIMD on every compute
 * unit, with no memory traffic; *flops (host) is set before the launch to the
 * multiply-add work of the launch (2 flop each).  `sink` (device, 4 bytes)
 * is written only in the rarest case.
 *
 * Both use the current device's compute-unit count and are asynchronous on
 * `stream`; time them with events on that stream.
 */
msa_status_t msa_ceiling_stream_read(const void *buffer, size_t buffer_bytes, uint32_t *sink, size_t *bytes_read,
                                     msa_stream_t stream);
msa_status_t msa_ceiling_mfma_bf16(int32_t iterations, float *sink, double *flops, msa_stream_t stream);

/* Workspace bytes an entry point needs for `problem` (0 if none).  Returns
 * (size_t)-1 when the problem is invalid or unsupported for that op. */
size_t msa_workspace_size(int op, const msa_problem_t *problem);

/* Byte offset, inside the workspace of `op` for `problem`, of a uint32 word
 * (4-byte aligned) that the call clears and then sets to the number of
 * bounded waits that gave up: 0 after a call means every wait ended
 * normally; anything else means that call's output is not valid.  The word
 * is written on the call's stream, so read it after the call has completed.
 * Ops whose kernels never wait on one another (and the prefill call when it
 * picks the block-centric schedule) have no such word: (size_t)-1, as for
 * an invalid or unsupported problem.  The environment variable
 * MSA_DEBUG_SPIN_LIMIT (a non-negative integer, read at each call) lowers
 * the bound, so that a test can make the waits give up while every kernel
 * still ends normally. */
size_t msa_workspace_wait_word(int op, const msa_problem_t *problem);

/* Host-side check of the contract on device-resident inputs, run on host
 * copies: cu_seqlens_q / cu_seqlens_k [num_seqs + 1] start at 0, end at
 * total_q / total_k, give 0 <= len_q <= len_k per sequence and lengths no
 * larger than max_seqlen_q / max_seqlen_k; and, when topk_ids [total_q, h,
 * top_k] is not NULL, every id is -1 or an eligible block (0 <= j <=
 * p / block_size for the row's position p) and no (row, group) holds an id
 * twice.  Only the problem's host fields are read (its device pointers are
 * ignored).  Returns MSA_SUCCESS or MSA_ERROR_INVALID_VALUE; touches no GPU
 * and needs none.  The debug mode (MSA_DEBUG_VALIDATE) runs it inside the
 * entry points. */
msa_status_t msa_validate_host(const msa_problem_t *problem, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, const int32_t *topk_ids);

/* Static, human-readable text of a status code. */
const char *msa_status_string(msa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
