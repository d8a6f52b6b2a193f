// Index branch, TopK: per (query, group), keep the k best of the E block
// scores ("MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a minimal
// sparse attention": TopK picks the KV blocks of this layer and GQA group;
// "MiniMax Goes Sparse", section 1, step 1).
//
// Exact selection: scores are mapped to order-preserving uint32 keys (-0.0
// folded onto +0.0) and the k-th largest key T is found bit by bit, most
// significant first; each step counts keys >= candidate with wave ballots.
// All keys > T are kept, then the lowest-indexed keys == T until k are kept
// (ties go to the lower block id).  Ids are written in ascending order, which
// falls out of giving every thread a contiguous run of block indices and
// prefix-summing per-thread counts.  A group of NT threads (one wave, or a
// 1024-thread workgroup for long contexts) handles one (row, group).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

// Sum of x over the NT threads of the group.
template <int NT>
__device__ __forceinline__ int group_sum(int x, int *red, int parity) {
    // wave-level: butterfly over 64 lanes with DPP-friendly shuffles
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    if constexpr (NT == 64) {
        return x;
    } else {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[parity * (NT / 64) + wave] = x;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) tot += red[parity * (NT / 64) + w];
        return tot;
    }
}

// Exclusive prefix sum of x (0 <= x < 2^bits) over the group's threads, in thread order.
template <int NT>
__device__ __forceinline__ int group_excl_scan(int x, int *red) {
    const int lane = threadIdx.x & 63;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    int excl = incl - x;
    if constexpr (NT == 64) {
        return excl;
    } else {
        const int wave = threadIdx.x >> 6;
        __syncthreads();
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wave; ++w) base += red[w];
        __syncthreads();
        return excl + base;
    }
}

template <int NT, int VPT>
__global__ __launch_bounds__(NT == 64 ? 256 : NT) void topk_select(
    const float *__restrict__ scores, int e_stride, const int32_t *__restrict__ cu_q,
    const int32_t *__restrict__ cu_k, int num_seqs, int total_q, int h, int B, int k,
    int32_t *__restrict__ ids) {
    constexpr int GROUPS = (NT == 64) ? 4 : 1;     // (row, group) pairs per workgroup
    __shared__ int red[2 * (NT / 64) + 1];

    const int sub = (NT == 64) ? (threadIdx.x >> 6) : 0;
    const long pair = (long)blockIdx.x * GROUPS + sub;
    if (pair >= (long)total_q * h) return;   // uniform per group (NT == 64) or per workgroup
    const int row = (int)(pair / h);
    const int t = (NT == 64) ? (threadIdx.x & 63) : threadIdx.x;

    // locate the row's sequence and position
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int len_q = cu_q[lo + 1] - cu_q[lo], len_k = cu_k[lo + 1] - cu_k[lo];
    const int p = len_k - len_q + (row - cu_q[lo]);
    const int E = p / B + 1;
    int32_t *out = ids + pair * k;

    if (E <= k) {
        for (int x = t; x < k; x += NT) out[x] = x < E ? x : -1;
        return;
    }

    const float *src = scores + pair * e_stride;
    uint32_t key[VPT];
#pragma unroll
    for (int v = 0; v < VPT; v += 4) {
        const int i = t * VPT + v;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < E) f = *reinterpret_cast<const float4 *>(src + i);
        key[v + 0] = (i + 0 < E) ? order_key(f.x) : 0u;
        key[v + 1] = (i + 1 < E) ? order_key(f.y) : 0u;
        key[v + 2] = (i + 2 < E) ? order_key(f.z) : 0u;
        key[v + 3] = (i + 3 < E) ? order_key(f.w) : 0u;
    }

    // T = largest value with count(key >= T) >= k, i.e. the k-th largest key.
    uint32_t T = 0;
    int parity = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int c = 0;
#pragma unroll
        for (int v = 0; v < VPT; ++v) c += key[v] >= cand;
        c = group_sum<NT>(c, red, parity);
        parity ^= 1;
        if (c >= k) T = cand;
    }
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        n_gt += key[v] > T;
        n_eq += key[v] == T;
    }
    const int total_gt = group_sum<NT>(n_gt, red, parity);
    const int need_eq = k - total_gt;
    const int eq_before = group_excl_scan<NT>(n_eq, red);

    int sel = 0;
    bool take[VPT];
    int eq_seen = eq_before;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        bool tk = key[v] > T;
        if (key[v] == T) {
            tk = eq_seen < need_eq;
            ++eq_seen;
        }
        take[v] = tk;
        sel += tk;
    }
    int pos = group_excl_scan<NT>(sel, red);
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        if (take[v] && pos < k) out[pos++] = t * VPT + v;
}

template <int NT, int VPT>
hipError_t launch(const Shape &s, const float *scores, int32_t *ids, hipStream_t st) {
    const long pairs = (long)s.total_q * s.h;
    const int per_wg = (NT == 64) ? 4 : 1;
    const long wgs = (pairs + per_wg - 1) / per_wg;
    hipLaunchKernelGGL((topk_select<NT, VPT>), dim3((unsigned)wgs), dim3(NT == 64 ? 256 : NT), 0, st, scores,
                       score_stride(s), s.cu_q, s.cu_k, s.num_seqs, s.total_q, s.h, s.B, s.top_k, ids);
    return hipGetLastError();
}

}  // namespace

int max_select_blocks() { return 1024 * 64; }

hipError_t launch_topk_select(const Shape &s, const float *scores, int32_t *ids, hipStream_t st) {
    const int e = score_stride(s);
    if (e <= 64 * 4) return launch<64, 4>(s, scores, ids, st);
    if (e <= 64 * 16) return launch<64, 16>(s, scores, ids, st);
    if (e <= 64 * 32) return launch<64, 32>(s, scores, ids, st);
    if (e <= 1024 * 16) return launch<1024, 16>(s, scores, ids, st);
    if (e <= 1024 * 32) return launch<1024, 32>(s, scores, ids, st);
    if (e <= 1024 * 64) return launch<1024, 64>(s, scores, ids, st);
    return hipErrorInvalidValue;
}

}  // namespace msa
