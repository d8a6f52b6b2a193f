// Host-side launch helpers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

struct Shape {
    int num_seqs, total_q, total_k, max_q, max_k;
    int H, h, d, d_idx, B, top_k;
    const int32_t *cu_q, *cu_k;
    // Paged cache (decode only): page of logical block j of sequence s is
    // table[s * table_stride + j]; null table = contiguous packed cache.
    const int32_t *table = nullptr;
    int table_stride = 0, num_pages = 0;
    // Forced blocks in every selection: the first `sink` and the last `local`
    // eligible blocks (0, 0 = plain TopK).
    int sink = 0, local = 0;
    // The packed query rows [row0, row0 + rows) a launch covers: the entry
    // points split a problem whose workspace would exceed the cap into such
    // chunks (positions and key ranges still come from the whole problem's
    // cu_seqlens).  The whole problem by default.
    int row0 = 0, rows = 0;
    // Prefill rows split between the two attention schedules: a row whose
    // query tile (split_tq consecutive queries from its sequence's first)
    // starts at a position below tiles_below is the query-tile kernel's, one
    // whose tile starts at or after blocks_from the block-centric path's.
    // The defaults give every row to whichever schedule is called.
    int tiles_below = 0x7fffffff, blocks_from = -0x7fffffff - 1, split_tq = 1;
};

// Workspace cap per call: the size an entry point splits its query rows to
// stay under (MSA_WORKSPACE_CAP_BYTES, or the debugging override
// MSA_DEBUG_WORKSPACE_CAP when that is set to a positive byte count).
size_t workspace_cap();
// Query rows per chunk for a per-row workspace cost `per_row` on top of a
// fixed part `fixed` (at least 1, at most total_q).
int chunk_rows(const Shape &s, size_t fixed, size_t per_row);

// Block-level scores workspace: [rows, h, e_stride] float32 (the rows of one
// chunk).
inline int score_stride(const Shape &s) {
    int e = (s.max_k + s.B - 1) / s.B;
    return (e + 3) / 4 * 4;
}

// Bytes a decode call streams (the index keys it scans, or the K/V it
// selects) above which its loads are non-temporal: more than the 256 MB MALL
// could keep for the next call, where plain loads let consecutive calls find
// smaller inputs there.
constexpr double kDecodeStreamBytes = 192.0 * (1 << 20);

// Index branch, step 1+2: token scores (never stored) max-pooled per block.
hipError_t launch_index_prefill(const Shape &s, const uint16_t *q_idx, const uint16_t *k_idx,
                                float *scores, hipStream_t st);
hipError_t launch_index_decode(const Shape &s, const uint16_t *q_idx, const uint16_t *k_idx,
                               float *scores, hipStream_t st);
// Index branch, step 3: per (row, group) top-k of the block scores.
hipError_t launch_topk_select(const Shape &s, const float *scores, int32_t *ids, hipStream_t st);
int max_select_blocks();

// Sparse branch.
size_t prefill_workspace_bytes(const Shape &s);
// Byte offset in that workspace of the uint32 wait word (ring waits that
// reached their bound in the last call; 0 = none).
size_t prefill_wait_word_offset(const Shape &s);
hipError_t launch_attn_prefill(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *ids, float scale, uint16_t *out, float *lse, void *ws,
                               hipStream_t st);
// Queries per workgroup tile of the query-tile kernel (G = H/h <= 16).
int prefill_tile_queries(const Shape &s);
// The same attention on the block-centric schedule (lists, per-block
// partials, log-sum-exp merge), and whether it is the faster of the two for
// a shape.
size_t block_prefill_workspace_bytes(const Shape &s);
int block_prefill_chunk_rows(const Shape &s);
// Position from which the block-centric schedule beats the query tiles:
// rows whose query tile starts there or later go to it (<= 0: every row;
// >= max_seqlen_k: none).
int prefill_split_position(const Shape &s);
hipError_t launch_attn_prefill_blocks(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                      const int32_t *ids, float scale, uint16_t *out, float *lse, void *ws,
                                      hipStream_t st);
// Copy new K/V/K_idx rows into paged pools at the given pool rows.
hipError_t launch_kv_append(int n, int h, int d, int d_idx, long long pool_rows, const int32_t *slots,
                            const uint16_t *k, const uint16_t *v, const uint16_t *k_idx, uint16_t *k_pool,
                            uint16_t *v_pool, uint16_t *k_idx_pool, hipStream_t st);
// Ceilings: a streaming read of the whole buffer in iterations of
// stream_read_bytes_per_iter bytes, and a pure MFMA loop.
long long stream_read_bytes_per_iter(int num_cus);
hipError_t launch_stream_read(const void *buf, long long iters, int num_cus, uint32_t *sink, hipStream_t st);
double mfma_loop_flops(int num_cus, int iters);
hipError_t launch_mfma_loop(int iters, int num_cus, float *sink, hipStream_t st);
// Inverted index of a prefill selection (byte offsets into one workspace):
// per key g * nb_max + blk_off[s] + j, the entries row * top_k + slot of the
// selections holding block j of sequence s in group g, in
// entries[off[key] .. off[key + 1]).
struct BlockLists {
    size_t blk_off, cnt, off, entries, place, bytes;
    long nb_max;
};
BlockLists block_lists_layout(const Shape &s);
// sorted: each list in ascending entry order (lists of at most 16384
// entries; longer ones keep the count pass's order).
hipError_t launch_block_lists(const Shape &s, const int32_t *ids, const BlockLists &w, char *base, hipStream_t st,
                              bool sorted = false);
// Backward of the sparse branch (prefill, selection fixed).
size_t backward_workspace_bytes(const Shape &s);
hipError_t launch_attn_backward(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *ids, float scale, const uint16_t *out, const float *lse,
                                const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv, void *ws,
                                hipStream_t st);
int decode_splits(const Shape &s);
size_t decode_workspace_bytes(const Shape &s);
// The library's fixed decode scratch (allocation-free entry point): its size,
// and its device address on the current device.
size_t decode_scratch_bytes();
hipError_t decode_scratch(void **ptr);
hipError_t launch_attn_decode(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *ids, float scale, uint16_t *out, float *lse, void *ws,
                              hipStream_t st);

}  // namespace msa
