// C ABI of the MSA hot path (declared in include/msa.h): argument
// validation, workspace sizing and kernel dispatch.  Nothing here allocates,
// frees or synchronises; every check runs on the host before any launch.
#include <hip/hip_runtime.h>

#include <new>

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

size_t index_ws(const msa_problem_t &p) {
    Shape s = to_shape(p);
    return (size_t)p.total_q * p.num_kv_heads * (size_t)msa::score_stride(s) * sizeof(float);
}

msa_status_t check_ws(void *ws, size_t have, size_t need) {
    if (need == 0) return MSA_SUCCESS;
    if (ws == nullptr || have < need) return MSA_ERROR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return MSA_ERROR_WORKSPACE;
    return MSA_SUCCESS;
}

msa_status_t launched(hipError_t e) { return e == hipSuccess ? MSA_SUCCESS : MSA_ERROR_LAUNCH; }

}  // namespace

extern "C" {

const char *msa_status_string(msa_status_t status) {
    switch (status) {
        case MSA_SUCCESS: return "success";
        case MSA_ERROR_INVALID_VALUE: return "invalid value";
        case MSA_ERROR_NOT_SUPPORTED: return "shape not supported";
        case MSA_ERROR_WORKSPACE: return "workspace missing or too small";
        case MSA_ERROR_LAUNCH: return "kernel launch failed";
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
        case MSA_OP_SPARSE_ATTN_PREFILL: {
            if (attn_support(p) != MSA_SUCCESS) return (size_t)-1;
            const Shape s = to_shape(p);
            return msa::prefill_prefers_blocks(s) ? msa::block_prefill_workspace_bytes(s)
                                                  : msa::prefill_workspace_bytes(s);
        }
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
    if (which == Schedule::kBlocks && (long long)p.total_q * p.top_k > 0x7fffffffLL) return MSA_ERROR_NOT_SUPPORTED;
    const bool blocks = which == Schedule::kBlocks || (which == Schedule::kAuto && msa::prefill_prefers_blocks(s));
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (blocks) {
        if ((st = check_ws(workspace, workspace_bytes, msa::block_prefill_workspace_bytes(s))) != MSA_SUCCESS)
            return st;
        return launched(msa::launch_attn_prefill_blocks(s, q, k, v, topk_ids, softmax_scale, out, lse, workspace, hs));
    }
    if ((st = check_ws(workspace, workspace_bytes, msa::prefill_workspace_bytes(s))) != MSA_SUCCESS) return st;
    return launched(msa::launch_attn_prefill(s, q, k, v, topk_ids, softmax_scale, out, lse, workspace, hs));
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
    return launched(msa::launch_attn_decode(s, q, k_cache, v_cache, topk_ids, softmax_scale, out, lse, workspace,
                                            reinterpret_cast<hipStream_t>(stream)));
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
    float *scores = reinterpret_cast<float *>(workspace);
    hipError_t e = (p.max_seqlen_q == 1) ? msa::launch_index_decode(s, q_idx, k_idx, scores, hs)
                                         : msa::launch_index_prefill(s, q_idx, k_idx, scores, hs);
    if (e != hipSuccess) return MSA_ERROR_LAUNCH;
    return launched(msa::launch_topk_select(s, scores, topk_ids, hs));
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
