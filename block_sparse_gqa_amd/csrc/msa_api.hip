// C ABI of the MSA hot path (declared in include/msa.h): argument
// validation, workspace sizing and kernel dispatch.  Nothing here allocates,
// frees or synchronises; every check runs on the host before any launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <new>
#include <vector>

#include "msa.h"
#include "msa_internal.h"

using msa::Shape;

namespace {

bool supported_common(const msa_problem_t &p) {
    return (p.block_size == 64 || p.block_size == 128) && p.top_k >= 1 && p.top_k <= 4096;
}

// Structural validity shared by every op.  Returns MSA_SUCCESS or an error.
msa_status_t check_problem(const msa_problem_t *p) {
    if (p == nullptr) return MSA_ERROR_INVALID_VALUE;
    if (p->num_seqs < 1 || p->total_q < 0 || p->total_k < 0) return MSA_ERROR_INVALID_VALUE;
    if (p->cu_seqlens_q == nullptr || p->cu_seqlens_k == nullptr) return MSA_ERROR_INVALID_VALUE;
    if (p->num_heads < 1 || p->num_kv_heads < 1 || p->num_heads % p->num_kv_heads != 0)
        return MSA_ERROR_INVALID_VALUE;
    if (p->head_dim < 1 || p->index_dim < 1 || p->block_size < 1 || p->top_k < 1) return MSA_ERROR_INVALID_VALUE;
    if (p->total_q > 0 && (p->max_seqlen_q < 1 || p->max_seqlen_k < p->max_seqlen_q || p->total_k < 1))
        return MSA_ERROR_INVALID_VALUE;
    if (p->max_seqlen_q > p->total_q || p->max_seqlen_k > p->total_k) return MSA_ERROR_INVALID_VALUE;
    if (!supported_common(*p)) return MSA_ERROR_NOT_SUPPORTED;
    return MSA_SUCCESS;
}

}  // namespace

namespace msa {

size_t workspace_cap() {
    const char *e = getenv("MSA_DEBUG_WORKSPACE_CAP");
    if (e != nullptr && *e != 0) {
        char *end = nullptr;
        const unsigned long long v = strtoull(e, &end, 10);
        if (*end == 0 && v > 0) return (size_t)v;
    }
    return MSA_WORKSPACE_CAP_BYTES;
}

int chunk_rows(const Shape &s, size_t fixed, size_t per_row) {
    const size_t cap = workspace_cap();
    const size_t avail = cap > fixed ? cap - fixed : 0;
    size_t r = per_row > 0 ? avail / per_row : (size_t)s.total_q;
    // list entries are (row - row0) * top_k + slot in an int
    const size_t lim = (size_t)0x7fffffff / (size_t)(s.top_k > 0 ? s.top_k : 1);
    if (r > lim) r = lim;
    const size_t rows = s.rows > 0 ? (size_t)s.rows : (size_t)s.total_q;   // the rows the launch covers
    if (r > rows) r = rows;
    return r < 1 ? 1 : (int)r;
}

}  // namespace msa

namespace {

Shape to_shape(const msa_problem_t &p) {
    Shape s;
    s.num_seqs = p.num_seqs;
    s.total_q = p.total_q;
    s.total_k = p.total_k;
    s.max_q = p.max_seqlen_q;
    s.max_k = p.max_seqlen_k;
    s.H = p.num_heads;
    s.h = p.num_kv_heads;
    s.d = p.head_dim;
    s.d_idx = p.index_dim;
    s.B = p.block_size;
    s.top_k = p.top_k;
    s.cu_q = p.cu_seqlens_q;
    s.cu_k = p.cu_seqlens_k;
    s.row0 = 0;
    s.rows = p.total_q;
    return s;
}

msa_status_t index_support(const msa_problem_t &p) {
    if (p.index_dim != 32 && p.index_dim != 64) return MSA_ERROR_NOT_SUPPORTED;
    if (p.num_kv_heads > 64) return MSA_ERROR_NOT_SUPPORTED;
    if (p.max_seqlen_q == 1 && p.num_kv_heads > 16) return MSA_ERROR_NOT_SUPPORTED;
    const long e = ((long)p.max_seqlen_k + p.block_size - 1) / p.block_size;
    if (e > msa::max_select_blocks()) return MSA_ERROR_NOT_SUPPORTED;
    return MSA_SUCCESS;
}

msa_status_t attn_support(const msa_problem_t &p) {
    if (p.head_dim != 64 && p.head_dim != 128) return MSA_ERROR_NOT_SUPPORTED;
    if (p.num_heads / p.num_kv_heads > 16) return MSA_ERROR_NOT_SUPPORTED;
    return MSA_SUCCESS;
}

// One query per sequence: the bandwidth-bound decode scan (it takes the
// last query of every sequence, so it needs exactly one per sequence).
bool index_is_decode(const msa_problem_t &p) { return p.max_seqlen_q == 1 && p.total_q == p.num_seqs; }

// Rows per chunk of the index branch: the block scores of a chunk's rows sit
// in the workspace between the scoring and the select kernel.
int index_chunk_rows(const msa_problem_t &p) {
    const Shape s = to_shape(p);
    if (index_is_decode(p)) return p.total_q;
    return msa::chunk_rows(s, 0, (size_t)p.num_kv_heads * msa::score_stride(s) * sizeof(float));
}

size_t index_ws(const msa_problem_t &p) {
    Shape s = to_shape(p);
    if (p.total_q == 0) return 0;
    return (size_t)index_chunk_rows(p) * p.num_kv_heads * (size_t)msa::score_stride(s) * sizeof(float);
}

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// The automatic prefill: query tiles for the rows before the split position,
// the block-centric schedule for the rest (when any row can reach it); the
// query-tile part's workspace first, then the block-centric part's.
bool prefill_auto_split(const Shape &s, int *split) {
    *split = msa::prefill_split_position(s);
    return *split <= s.max_k - 1;
}

// The automatic prefill's two parts when it splits the rows at `split`: the
// query tiles take the rows whose tile starts below it, the block-centric
// schedule the rest.  With one sequence the latter are the rows from the
// first tile that starts at or past the split (positions are
// total_k - total_q + row), so its lists and partials cover only those.
void prefill_auto_shapes(const Shape &s, int split, Shape *st_tiles, Shape *st_blocks) {
    *st_tiles = s;
    *st_blocks = s;
    st_tiles->tiles_below = split;
    st_blocks->blocks_from = split;
    st_blocks->split_tq = msa::prefill_tile_queries(s);
    if (s.num_seqs == 1) {
        const long tq = st_blocks->split_tq;
        const long first = ((long)split - (s.total_k - s.total_q) + tq - 1) / tq * tq;
        const int r0 = (int)std::min<long>(std::max<long>(first, 0), s.total_q);
        st_blocks->row0 = r0;
        st_blocks->rows = s.total_q - r0;
    }
}

size_t prefill_auto_ws(const Shape &s) {
    int split = 0;
    const size_t tiles = msa::prefill_workspace_bytes(s);
    if (!prefill_auto_split(s, &split)) return tiles;
    Shape st_tiles, st_blocks;
    prefill_auto_shapes(s, split, &st_tiles, &st_blocks);
    return al256(tiles) + msa::block_prefill_workspace_bytes(st_blocks);
}

msa_status_t check_ws(void *ws, size_t have, size_t need) {
    if (need == 0) return MSA_SUCCESS;
    if (ws == nullptr || have < need) return MSA_ERROR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return MSA_ERROR_WORKSPACE;
    return MSA_SUCCESS;
}

msa_status_t launched(hipError_t e) { return e == hipSuccess ? MSA_SUCCESS : MSA_ERROR_LAUNCH; }

// The debug mode: with MSA_DEBUG_VALIDATE set to a non-empty value other than
// "0", the entry points copy cu_seqlens (and the ids they read) to the host,
// waiting for the copies, and check them with msa_validate_host before
// launching anything.
bool debug_validate_on() {
    const char *e = getenv("MSA_DEBUG_VALIDATE");
    return e != nullptr && *e != 0 && !(e[0] == '0' && e[1] == 0);
}

msa_status_t debug_validate(const msa_problem_t &p, const int32_t *ids, hipStream_t st);


}  // namespace

extern "C" {

const char *msa_status_string(msa_status_t status) {
    switch (status) {
        case MSA_SUCCESS: return "success";
        case MSA_ERROR_INVALID_VALUE: return "invalid value";
        case MSA_ERROR_NOT_SUPPORTED: return "shape not supported";
        case MSA_ERROR_WORKSPACE: return "workspace missing or too small";
        case MSA_ERROR_LAUNCH: return "kernel launch failed";
        default: break;
    }
    return "unknown status";
}

size_t msa_workspace_size(int op, const msa_problem_t *problem) {
    if (check_problem(problem) != MSA_SUCCESS) return (size_t)-1;
    const msa_problem_t &p = *problem;
    switch (op) {
        case MSA_OP_INDEX_TOPK:
            if (index_support(p) != MSA_SUCCESS) return (size_t)-1;
            return index_ws(p);
        case MSA_OP_SPARSE_ATTN_PREFILL:
            if (attn_support(p) != MSA_SUCCESS) return (size_t)-1;
            return prefill_auto_ws(to_shape(p));
        case MSA_OP_SPARSE_ATTN_PREFILL_TILES:
            if (attn_support(p) != MSA_SUCCESS) return (size_t)-1;
            return msa::prefill_workspace_bytes(to_shape(p));
        case MSA_OP_SPARSE_ATTN_DECODE:
            if (attn_support(p) != MSA_SUCCESS) return (size_t)-1;
            if (p.max_seqlen_q != 1 || p.total_q != p.num_seqs) return (size_t)-1;
            return msa::decode_workspace_bytes(to_shape(p));
        case MSA_OP_SPARSE_ATTN_BACKWARD:
            if (attn_support(p) != MSA_SUCCESS) return (size_t)-1;
            return msa::backward_workspace_bytes(to_shape(p));
        case MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS:
            if (attn_support(p) != MSA_SUCCESS || p.num_heads / p.num_kv_heads > 16) return (size_t)-1;
            return msa::block_prefill_workspace_bytes(to_shape(p));
    }
    return (size_t)-1;
}

msa_status_t msa_validate_host(const msa_problem_t *problem, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, const int32_t *topk_ids) {
    if (problem == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return MSA_ERROR_INVALID_VALUE;
    const msa_problem_t &p = *problem;
    if (p.num_seqs < 1 || p.total_q < 0 || p.total_k < 0 || p.num_kv_heads < 1 || p.block_size < 1 || p.top_k < 1)
        return MSA_ERROR_INVALID_VALUE;
    const int n = p.num_seqs;
    if (cu_seqlens_q[0] != 0 || cu_seqlens_k[0] != 0) return MSA_ERROR_INVALID_VALUE;
    if (cu_seqlens_q[n] != p.total_q || cu_seqlens_k[n] != p.total_k) return MSA_ERROR_INVALID_VALUE;
    for (int i = 0; i < n; ++i) {
        const long lq = (long)cu_seqlens_q[i + 1] - cu_seqlens_q[i];
        const long lk = (long)cu_seqlens_k[i + 1] - cu_seqlens_k[i];
        if (lq < 0 || lk < 0 || lk < lq) return MSA_ERROR_INVALID_VALUE;
        if (lq > p.max_seqlen_q || lk > p.max_seqlen_k) return MSA_ERROR_INVALID_VALUE;
    }
    if (topk_ids == nullptr) return MSA_SUCCESS;
    const int h = p.num_kv_heads, k = p.top_k;
    std::vector<unsigned char> seen;
    for (int i = 0; i < n; ++i) {
        const int lq = cu_seqlens_q[i + 1] - cu_seqlens_q[i];
        const int lk = cu_seqlens_k[i + 1] - cu_seqlens_k[i];
        for (int r = 0; r < lq; ++r) {
            const long E = (long)(lk - lq + r) / p.block_size + 1;
            seen.assign((size_t)E, 0);
            const int32_t *row = topk_ids + ((size_t)(cu_seqlens_q[i] + r) * h) * k;
            for (int g = 0; g < h; ++g) {
                for (int a = 0; a < k; ++a) {
                    const int32_t j = row[(size_t)g * k + a];
                    if (j == -1) continue;
                    if (j < 0 || j >= E) return MSA_ERROR_INVALID_VALUE;
                    if (seen[(size_t)j] == (unsigned char)(g + 1)) return MSA_ERROR_INVALID_VALUE;
                    seen[(size_t)j] = (unsigned char)(g + 1);
                }
            }
        }
    }
    return MSA_SUCCESS;
}

size_t msa_workspace_wait_word(int op, const msa_problem_t *problem) {
    if (check_problem(problem) != MSA_SUCCESS) return (size_t)-1;
    const msa_problem_t &p = *problem;
    if (attn_support(p) != MSA_SUCCESS) return (size_t)-1;
    const Shape s = to_shape(p);
    switch (op) {
        case MSA_OP_SPARSE_ATTN_PREFILL:   // the query-tile part's workspace comes first
            return msa::prefill_wait_word_offset(s);
        case MSA_OP_SPARSE_ATTN_PREFILL_TILES:
            return msa::prefill_wait_word_offset(s);
    }
    return (size_t)-1;
}

msa_status_t msa_index_topk(const msa_problem_t *problem, const msa_bf16_t *q_idx, const msa_bf16_t *k_idx,
                            int32_t *topk_ids, void *workspace, size_t workspace_bytes, msa_stream_t stream) {
    return msa_index_topk_ex(problem, nullptr, nullptr, q_idx, k_idx, topk_ids, workspace, workspace_bytes, stream);
}

namespace {
// Which prefill schedule a call runs.
enum class Schedule { kAuto, kTiles, kBlocks };


msa_status_t prefill_call(Schedule which, const msa_problem_t *problem, const msa_bf16_t *q, const msa_bf16_t *k,
                          const msa_bf16_t *v, const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out,
                          float *lse, void *workspace, size_t workspace_bytes, msa_stream_t stream) {
    msa_status_t st = check_problem(problem);
    if (st != MSA_SUCCESS) return st;
    const msa_problem_t &p = *problem;
    if (p.total_q == 0) return MSA_SUCCESS;
    if (q == nullptr || k == nullptr || v == nullptr || topk_ids == nullptr || out == nullptr)
        return MSA_ERROR_INVALID_VALUE;
    if (!(softmax_scale > 0.0f) || softmax_scale == __builtin_inff()) return MSA_ERROR_INVALID_VALUE;
    if ((st = attn_support(p)) != MSA_SUCCESS) return st;
    const Shape s = to_shape(p);
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (which == Schedule::kBlocks) {
        if ((st = check_ws(workspace, workspace_bytes, msa::block_prefill_workspace_bytes(s))) != MSA_SUCCESS)
            return st;
        if (debug_validate_on() && (st = debug_validate(p, topk_ids, hs)) != MSA_SUCCESS) return st;
        return launched(msa::launch_attn_prefill_blocks(s, q, k, v, topk_ids, softmax_scale, out, lse, workspace, hs));
    }
    int split = 0;
    const bool hybrid = which == Schedule::kAuto && prefill_auto_split(s, &split);
    const size_t need = hybrid ? prefill_auto_ws(s) : msa::prefill_workspace_bytes(s);
    if ((st = check_ws(workspace, workspace_bytes, need)) != MSA_SUCCESS) return st;
    if (debug_validate_on() && (st = debug_validate(p, topk_ids, hs)) != MSA_SUCCESS) return st;
    if (!hybrid) return launched(msa::launch_attn_prefill(s, q, k, v, topk_ids, softmax_scale, out, lse, workspace, hs));
    // rows split by position: the early ones (few eligible blocks) on the
    // query tiles, the late ones on the block-centric schedule
    Shape st_tiles, st_blocks;
    prefill_auto_shapes(s, split, &st_tiles, &st_blocks);
    char *wsb = static_cast<char *>(workspace);
    if (msa::launch_attn_prefill(st_tiles, q, k, v, topk_ids, softmax_scale, out, lse, workspace, hs) != hipSuccess)
        return MSA_ERROR_LAUNCH;
    return launched(msa::launch_attn_prefill_blocks(st_blocks, q, k, v, topk_ids, softmax_scale, out, lse,
                                                    wsb + al256(msa::prefill_workspace_bytes(s)), hs));
}
}  // namespace

msa_status_t msa_sparse_attn_prefill(const msa_problem_t *problem, const msa_bf16_t *q, const msa_bf16_t *k,
                                     const msa_bf16_t *v, const int32_t *topk_ids, float softmax_scale,
                                     msa_bf16_t *out, float *lse, void *workspace, size_t workspace_bytes,
                                     msa_stream_t stream) {
    return prefill_call(Schedule::kAuto, problem, q, k, v, topk_ids, softmax_scale, out, lse, workspace,
                        workspace_bytes, stream);
}

msa_status_t msa_sparse_attn_prefill_tiles(const msa_problem_t *problem, const msa_bf16_t *q, const msa_bf16_t *k,
                                           const msa_bf16_t *v, const int32_t *topk_ids, float softmax_scale,
                                           msa_bf16_t *out, float *lse, void *workspace, size_t workspace_bytes,
                                           msa_stream_t stream) {
    return prefill_call(Schedule::kTiles, problem, q, k, v, topk_ids, softmax_scale, out, lse, workspace,
                        workspace_bytes, stream);
}

msa_status_t msa_sparse_attn_prefill_blocks(const msa_problem_t *problem, const msa_bf16_t *q, const msa_bf16_t *k,
                                            const msa_bf16_t *v, const int32_t *topk_ids, float softmax_scale,
                                            msa_bf16_t *out, float *lse, void *workspace, size_t workspace_bytes,
                                            msa_stream_t stream) {
    return prefill_call(Schedule::kBlocks, problem, q, k, v, topk_ids, softmax_scale, out, lse, workspace,
                        workspace_bytes, stream);
}

msa_status_t msa_sparse_attn_prefill_backward(const msa_problem_t *problem, const msa_bf16_t *q, const msa_bf16_t *k,
                                              const msa_bf16_t *v, const int32_t *topk_ids, float softmax_scale,
                                              const msa_bf16_t *out, const float *lse, const msa_bf16_t *dout,
                                              msa_bf16_t *dq, msa_bf16_t *dk, msa_bf16_t *dv, void *workspace,
                                              size_t workspace_bytes, msa_stream_t stream) {
    msa_status_t st = check_problem(problem);
    if (st != MSA_SUCCESS) return st;
    const msa_problem_t &p = *problem;
    if (p.total_q == 0) return MSA_SUCCESS;
    if (q == nullptr || k == nullptr || v == nullptr || topk_ids == nullptr || out == nullptr || lse == nullptr ||
        dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
        return MSA_ERROR_INVALID_VALUE;
    if (!(softmax_scale > 0.0f) || softmax_scale == __builtin_inff()) return MSA_ERROR_INVALID_VALUE;
    if ((st = attn_support(p)) != MSA_SUCCESS) return st;
    Shape s = to_shape(p);
    if ((st = check_ws(workspace, workspace_bytes, msa::backward_workspace_bytes(s))) != MSA_SUCCESS) return st;
    if (debug_validate_on() &&
        (st = debug_validate(p, topk_ids, reinterpret_cast<hipStream_t>(stream))) != MSA_SUCCESS)
        return st;
    return launched(msa::launch_attn_backward(s, q, k, v, topk_ids, softmax_scale, out, lse, dout, dq, dk, dv,
                                              workspace, reinterpret_cast<hipStream_t>(stream)));
}

msa_status_t msa_sparse_attn_decode(const msa_problem_t *problem, const msa_bf16_t *q, const msa_bf16_t *k_cache,
                                    const msa_bf16_t *v_cache, const int32_t *topk_ids, float softmax_scale,
                                    msa_bf16_t *out, float *lse, void *workspace, size_t workspace_bytes,
                                    msa_stream_t stream) {
    msa_status_t st = check_problem(problem);
    if (st != MSA_SUCCESS) return st;
    const msa_problem_t &p = *problem;
    if (p.total_q == 0) return MSA_SUCCESS;
    if (p.max_seqlen_q != 1 || p.total_q != p.num_seqs) return MSA_ERROR_INVALID_VALUE;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || topk_ids == nullptr || out == nullptr)
        return MSA_ERROR_INVALID_VALUE;
    if (!(softmax_scale > 0.0f) || softmax_scale == __builtin_inff()) return MSA_ERROR_INVALID_VALUE;
    if ((st = attn_support(p)) != MSA_SUCCESS) return st;
    Shape s = to_shape(p);
    if ((st = check_ws(workspace, workspace_bytes, msa::decode_workspace_bytes(s))) != MSA_SUCCESS) return st;
    if (debug_validate_on() &&
        (st = debug_validate(p, topk_ids, reinterpret_cast<hipStream_t>(stream))) != MSA_SUCCESS)
        return st;
    return launched(msa::launch_attn_decode(s, q, k_cache, v_cache, topk_ids, softmax_scale, out, lse, workspace,
                                            reinterpret_cast<hipStream_t>(stream)));
}

msa_status_t msa_sparse_attn_decode_noalloc(const msa_problem_t *problem, const msa_bf16_t *q,
                                            const msa_bf16_t *k_cache, const msa_bf16_t *v_cache,
                                            const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out,
                                            float *lse, msa_stream_t stream) {
    msa_status_t st = check_problem(problem);
    if (st != MSA_SUCCESS) return st;
    const msa_problem_t &p = *problem;
    if (p.total_q == 0) return MSA_SUCCESS;
    if (p.max_seqlen_q != 1 || p.total_q != p.num_seqs) return MSA_ERROR_INVALID_VALUE;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || topk_ids == nullptr || out == nullptr)
        return MSA_ERROR_INVALID_VALUE;
    if (!(softmax_scale > 0.0f) || softmax_scale == __builtin_inff()) return MSA_ERROR_INVALID_VALUE;
    if ((st = attn_support(p)) != MSA_SUCCESS) return st;
    const Shape s = to_shape(p);
    if (msa::decode_workspace_bytes(s) > msa::decode_scratch_bytes()) return MSA_ERROR_WORKSPACE;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (debug_validate_on() && (st = debug_validate(p, topk_ids, hs)) != MSA_SUCCESS) return st;
    void *scratch = nullptr;
    if (msa::decode_scratch(&scratch) != hipSuccess) return MSA_ERROR_LAUNCH;
    return launched(msa::launch_attn_decode(s, q, k_cache, v_cache, topk_ids, softmax_scale, out, lse, scratch, hs));
}

namespace {

// The paged entry points: decode only, a table and a pool of at least one page.
msa_status_t check_paged(const msa_problem_t &p, const msa_paged_kv_t *pk) {
    if (pk == nullptr || pk->block_table == nullptr || pk->num_pages < 1) return MSA_ERROR_INVALID_VALUE;
    const long blocks = ((long)p.max_seqlen_k + p.block_size - 1) / p.block_size;
    if (pk->max_blocks_per_seq < blocks) return MSA_ERROR_INVALID_VALUE;
    if (p.max_seqlen_q != 1 || p.total_q != p.num_seqs) return MSA_ERROR_NOT_SUPPORTED;
    return MSA_SUCCESS;
}

void set_paged(Shape &s, const msa_paged_kv_t &pk) {
    s.table = pk.block_table;
    s.table_stride = pk.max_blocks_per_seq;
    s.num_pages = pk.num_pages;
}

}  // namespace

msa_status_t msa_index_topk_paged(const msa_problem_t *problem, const msa_paged_kv_t *paged, const msa_bf16_t *q_idx,
                                  const msa_bf16_t *k_idx_pool, int32_t *topk_ids, void *workspace,
                                  size_t workspace_bytes, msa_stream_t stream) {
    if (paged == nullptr) return MSA_ERROR_INVALID_VALUE;
    return msa_index_topk_ex(problem, nullptr, paged, q_idx, k_idx_pool, topk_ids, workspace, workspace_bytes, stream);
}

msa_status_t msa_index_topk_ex(const msa_problem_t *problem, const msa_select_options_t *options,
                               const msa_paged_kv_t *paged, const msa_bf16_t *q_idx, const msa_bf16_t *k_idx,
                               int32_t *topk_ids, void *workspace, size_t workspace_bytes, msa_stream_t stream) {
    msa_status_t st = check_problem(problem);
    if (st != MSA_SUCCESS) return st;
    const msa_problem_t &p = *problem;
    if (options != nullptr &&
        (options->sink_blocks < 0 || options->local_blocks < 0 ||
         (long)options->sink_blocks + options->local_blocks > p.top_k))
        return MSA_ERROR_INVALID_VALUE;
    if (p.total_q == 0) return MSA_SUCCESS;
    if (paged != nullptr && (st = check_paged(p, paged)) != MSA_SUCCESS) return st;
    if (q_idx == nullptr || k_idx == nullptr || topk_ids == nullptr) return MSA_ERROR_INVALID_VALUE;
    if ((st = index_support(p)) != MSA_SUCCESS) return st;
    if ((st = check_ws(workspace, workspace_bytes, index_ws(p))) != MSA_SUCCESS) return st;
    Shape s = to_shape(p);
    if (paged != nullptr) set_paged(s, *paged);
    if (options != nullptr) {
        s.sink = options->sink_blocks;
        s.local = options->local_blocks;
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (debug_validate_on() && (st = debug_validate(p, nullptr, hs)) != MSA_SUCCESS) return st;
    float *scores = reinterpret_cast<float *>(workspace);
    // A batch with empty sequences (fewer queries than sequences) goes
    // through the prefill kernel, which skips them.  (The paged path has
    // already required total_q == num_seqs.)
    if (index_is_decode(p)) {
        if (msa::launch_index_decode(s, q_idx, k_idx, scores, hs) != hipSuccess) return MSA_ERROR_LAUNCH;
        return launched(msa::launch_topk_select(s, scores, topk_ids, hs));
    }
    // Prefill: the rows in chunks whose block scores fit the workspace cap.
    const int per = index_chunk_rows(p);
    for (int r0 = 0; r0 < p.total_q; r0 += per) {
        Shape c = s;
        c.row0 = r0;
        c.rows = p.total_q - r0 < per ? p.total_q - r0 : per;
        if (msa::launch_index_prefill(c, q_idx, k_idx, scores, hs) != hipSuccess) return MSA_ERROR_LAUNCH;
        if (msa::launch_topk_select(c, scores, topk_ids, hs) != hipSuccess) return MSA_ERROR_LAUNCH;
    }
    return MSA_SUCCESS;
}

msa_status_t msa_sparse_attn_decode_paged(const msa_problem_t *problem, const msa_paged_kv_t *paged,
                                          const msa_bf16_t *q, const msa_bf16_t *k_pool, const msa_bf16_t *v_pool,
                                          const int32_t *topk_ids, float softmax_scale, msa_bf16_t *out, float *lse,
                                          void *workspace, size_t workspace_bytes, msa_stream_t stream) {
    msa_status_t st = check_problem(problem);
    if (st != MSA_SUCCESS) return st;
    const msa_problem_t &p = *problem;
    if (p.total_q == 0) return MSA_SUCCESS;
    if ((st = check_paged(p, paged)) != MSA_SUCCESS) return st;
    if (q == nullptr || k_pool == nullptr || v_pool == nullptr || topk_ids == nullptr || out == nullptr)
        return MSA_ERROR_INVALID_VALUE;
    if (!(softmax_scale > 0.0f) || softmax_scale == __builtin_inff()) return MSA_ERROR_INVALID_VALUE;
    if ((st = attn_support(p)) != MSA_SUCCESS) return st;
    Shape s = to_shape(p);
    if ((st = check_ws(workspace, workspace_bytes, msa::decode_workspace_bytes(s))) != MSA_SUCCESS) return st;
    set_paged(s, *paged);
    if (debug_validate_on() &&
        (st = debug_validate(p, topk_ids, reinterpret_cast<hipStream_t>(stream))) != MSA_SUCCESS)
        return st;
    return launched(msa::launch_attn_decode(s, q, k_pool, v_pool, topk_ids, softmax_scale, out, lse, workspace,
                                            reinterpret_cast<hipStream_t>(stream)));
}

msa_status_t msa_kv_append_paged(int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t index_dim,
                                 int64_t pool_rows, const int32_t *slot_mapping, const msa_bf16_t *k,
                                 const msa_bf16_t *v, const msa_bf16_t *k_idx, msa_bf16_t *k_pool,
                                 msa_bf16_t *v_pool, msa_bf16_t *k_idx_pool, msa_stream_t stream) {
    if (num_tokens < 0 || pool_rows < 1 || num_kv_heads < 1) return MSA_ERROR_INVALID_VALUE;
    if (head_dim != 64 && head_dim != 128) return MSA_ERROR_NOT_SUPPORTED;
    if (index_dim != 32 && index_dim != 64) return MSA_ERROR_NOT_SUPPORTED;
    if (num_kv_heads > 64) return MSA_ERROR_NOT_SUPPORTED;
    if (num_tokens == 0) return MSA_SUCCESS;
    if (slot_mapping == nullptr || k == nullptr || v == nullptr || k_idx == nullptr || k_pool == nullptr ||
        v_pool == nullptr || k_idx_pool == nullptr)
        return MSA_ERROR_INVALID_VALUE;
    const void *ptrs[] = {k, v, k_idx, k_pool, v_pool, k_idx_pool};
    for (const void *q : ptrs)
        if ((reinterpret_cast<uintptr_t>(q) & 15u) != 0) return MSA_ERROR_INVALID_VALUE;
    return launched(msa::launch_kv_append(num_tokens, num_kv_heads, head_dim, index_dim, (long long)pool_rows,
                                          slot_mapping, k, v, k_idx, k_pool, v_pool, k_idx_pool,
                                          reinterpret_cast<hipStream_t>(stream)));
}

namespace {
int current_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}
}  // namespace

msa_status_t msa_ceiling_stream_read(const void *buffer, size_t buffer_bytes, uint32_t *sink, size_t *bytes_read,
                                     msa_stream_t stream) {
    if (buffer == nullptr || sink == nullptr || bytes_read == nullptr) return MSA_ERROR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(buffer) & 15u) != 0) return MSA_ERROR_INVALID_VALUE;
    const int cus = current_cu_count();
    if (cus < 1) return MSA_ERROR_LAUNCH;
    const long long per = msa::stream_read_bytes_per_iter(cus);
    const long long iters = (long long)(buffer_bytes / (size_t)per);
    if (iters < 1) return MSA_ERROR_INVALID_VALUE;
    *bytes_read = (size_t)(iters * per);
    return launched(msa::launch_stream_read(buffer, iters, cus, sink, reinterpret_cast<hipStream_t>(stream)));
}

msa_status_t msa_ceiling_mfma_bf16(int32_t iterations, float *sink, double *flops, msa_stream_t stream) {
    if (iterations < 1 || sink == nullptr || flops == nullptr) return MSA_ERROR_INVALID_VALUE;
    const int cus = current_cu_count();
    if (cus < 1) return MSA_ERROR_LAUNCH;
    *flops = msa::mfma_loop_flops(cus, iterations);
    return launched(msa::launch_mfma_loop(iterations, cus, sink, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

msa_status_t debug_validate(const msa_problem_t &p, const int32_t *ids, hipStream_t st) {
    std::vector<int32_t> cq((size_t)p.num_seqs + 1), ck((size_t)p.num_seqs + 1), hid;
    const size_t cu_bytes = cq.size() * sizeof(int32_t);
    if (hipMemcpyAsync(cq.data(), p.cu_seqlens_q, cu_bytes, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipMemcpyAsync(ck.data(), p.cu_seqlens_k, cu_bytes, hipMemcpyDeviceToHost, st) != hipSuccess)
        return MSA_ERROR_LAUNCH;
    if (ids != nullptr) {
        hid.resize((size_t)p.total_q * p.num_kv_heads * p.top_k);
        if (hipMemcpyAsync(hid.data(), ids, hid.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
            return MSA_ERROR_LAUNCH;
    }
    if (hipStreamSynchronize(st) != hipSuccess) return MSA_ERROR_LAUNCH;
    return msa_validate_host(&p, cq.data(), ck.data(), ids != nullptr ? hid.data() : nullptr);
}

}  // namespace
