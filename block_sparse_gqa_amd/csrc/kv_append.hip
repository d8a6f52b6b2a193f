// Append to a paged KV cache: the K, V and K_idx rows of new tokens are
// copied into the pools at caller-chosen pool rows.  The pools keep the
// native GQA layout, one physical block of B tokens per page
// ("深度解析M3多模态模型与Token Plan", section 二.1 on storage/compute
// decoupling), so appending a token is a plain row copy.
//
// The rows are copied as 16-byte chunks.  Each thread moves UNROLL chunks of
// K and the same chunks of V, issuing all its loads before its stores, so many
// lines are in flight per thread; consecutive threads take consecutive chunks
// of a row, so every load and store instruction covers whole lines.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// Rows of chunks_per_row 16-byte chunks from src_a (and src_b, when given)
// to dst_a (dst_b) at the rows slots[i]; slots < 0 or >= pool_rows are skipped.
__global__ __launch_bounds__(kThreads) void scatter_rows(long long n_chunks, int chunks_per_row, long long pool_rows,
                                                         const int32_t *__restrict__ slots,
                                                         const uint4 *__restrict__ src_a,
                                                         const uint4 *__restrict__ src_b, uint4 *__restrict__ dst_a,
                                                         uint4 *__restrict__ dst_b) {
    const long long c0 = (long long)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    uint4 a[kUnroll], b[kUnroll];
    long long dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const long long c = c0 + (long long)u * kThreads;
        dst[u] = -1;
        if (c < n_chunks) {
            const long long i = c / chunks_per_row;
            const long long slot = slots[i];
            if (slot >= 0 && slot < pool_rows) {
                dst[u] = slot * chunks_per_row + (c - i * chunks_per_row);
                a[u] = src_a[c];
                if (src_b != nullptr) b[u] = src_b[c];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (dst[u] >= 0) {
            dst_a[dst[u]] = a[u];
            if (src_b != nullptr) dst_b[dst[u]] = b[u];
        }
    }
}

}  // namespace

hipError_t launch_kv_append(int n, int h, int d, int d_idx, long long pool_rows, const int32_t *slots,
                            const uint16_t *k, const uint16_t *v, const uint16_t *k_idx, uint16_t *k_pool,
                            uint16_t *v_pool, uint16_t *k_idx_pool, hipStream_t st) {
    // d and d_idx are multiples of 8, so every row is a whole number of
    // 16-byte chunks and every row start is 16-byte aligned (the tensors
    // themselves must be 16-byte aligned).
    const int row_chunks = h * d / 8, idx_chunks = d_idx / 8;
    const long long per_group = kThreads * kUnroll;
    const long long kv_chunks = (long long)n * row_chunks, idx_total = (long long)n * idx_chunks;
    if ((kv_chunks + per_group - 1) / per_group > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scatter_rows, dim3((unsigned)((kv_chunks + per_group - 1) / per_group)), dim3(kThreads), 0, st,
                       kv_chunks, row_chunks, pool_rows, slots, reinterpret_cast<const uint4 *>(k),
                       reinterpret_cast<const uint4 *>(v), reinterpret_cast<uint4 *>(k_pool),
                       reinterpret_cast<uint4 *>(v_pool));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scatter_rows, dim3((unsigned)((idx_total + per_group - 1) / per_group)), dim3(kThreads), 0, st,
                       idx_total, idx_chunks, pool_rows, slots, reinterpret_cast<const uint4 *>(k_idx), nullptr,
                       reinterpret_cast<uint4 *>(k_idx_pool), nullptr);
    return hipGetLastError();
}

}  // namespace msa
