// Index branch, TopK: per (query, group), keep the k best of the E block
// scores ("MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a minimal
// sparse attention": TopK picks the KV blocks of this layer and GQA group;
// "MiniMax Goes Sparse", section 1, step 1).
//
// Exact selection.  Scores are mapped to order-preserving uint32 keys (-0.0
// folded onto +0.0) and the k-th largest key T is located; all keys > T are
// kept, then the lowest-indexed keys == T until k are kept (ties go to the
// lower block id).  Optionally the first `sink` and the last `local` eligible
// blocks are forced in (an option, not the pages' method: "MiniMax Goes
// Sparse", section 2, speculates that an attention sink may take the place of
// the dropped sliding-window branch); they get a key above every score.  Ids are written in ascending order, which falls out of
// giving every thread a contiguous run of block indices and prefix-summing
// per-thread counts.
//
// Short rows (E <= 2048, prefill) use one wave per (row, group): T is found
// bit by bit below the common prefix of the row's largest and smallest key,
// each step counting keys >= candidate with ballots.  Long rows (decode over
// long contexts) use a 1024-thread workgroup per (row, group) and a radix
// select: up to three 11-bit digits below the common prefix, each resolved
// with an LDS histogram and a suffix scan.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kDigit = 11;
constexpr int kBins = 1 << kDigit;

struct RowInfo {
    int E;
    long pair;
};

__device__ __forceinline__ RowInfo row_info(long pair, const int32_t *cu_q, const int32_t *cu_k, int num_seqs, int h,
                                            int B) {
    const int row = (int)(pair / h);
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int len_q = cu_q[lo + 1] - cu_q[lo], len_k = cu_k[lo + 1] - cu_k[lo];
    const int p = len_k - len_q + (row - cu_q[lo]);
    return RowInfo{p / B + 1, pair};
}

// Keys of blocks t*VPT .. t*VPT+VPT-1 (0 past E).  Forced blocks (the first
// `sink` and the last `local` eligible ones) get the largest key, above that
// of any score, so they are always kept; the caller guarantees
// sink + local <= k.
template <int VPT>
__device__ __forceinline__ void load_keys(uint32_t (&key)[VPT], const float *src, int t, int E, int sink, int local) {
#pragma unroll
    for (int v = 0; v < VPT; v += 4) {
        const int i = t * VPT + v;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < E) f = *reinterpret_cast<const float4 *>(src + i);
        const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = i + u;
            key[v + u] = (j < E) ? ((j < sink || j >= E - local) ? 0xffffffffu : order_key(fv[u])) : 0u;
        }
    }
}

// Wave-level exclusive prefix sum (lane order).
__device__ __forceinline__ int wave_excl_scan(int x) {
    const int lane = threadIdx.x & 63;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    return incl - x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ---------------------------------------------------------------- one wave
template <int VPT>
__global__ __launch_bounds__(256) void topk_select_wave(const float *__restrict__ scores, int e_stride,
                                                        const int32_t *__restrict__ cu_q,
                                                        const int32_t *__restrict__ cu_k, int num_seqs, int total_q,
                                                        int h, int B, int k, int sink, int local,
                                                        int32_t *__restrict__ ids) {
    const long pair = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= (long)total_q * h) return;   // uniform per wave
    const int t = threadIdx.x & 63;
    const RowInfo ri = row_info(pair, cu_q, cu_k, num_seqs, h, B);
    const int E = ri.E;
    int32_t *out = ids + pair * k;
    if (E <= k) {
        for (int x = t; x < k; x += 64) out[x] = x < E ? x : -1;
        return;
    }
    uint32_t key[VPT];
    load_keys<VPT>(key, scores + pair * e_stride, t, E, sink, local);

    // common prefix of the largest and smallest valid key
    uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        mx = max(mx, key[v]);
        mn = min(mn, key[v] ? key[v] : 0xffffffffu);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
    }
    // Equal in every lane after the butterfly; reading them into scalar
    // registers makes the search below scalar-controlled (no exec-mask
    // bookkeeping per step, the candidate is a scalar operand of the compares).
    mx = __builtin_amdgcn_readfirstlane(mx);
    mn = __builtin_amdgcn_readfirstlane(mn);
    // T = largest value with count(key >= T) >= k (the k-th largest key).  All
    // valid keys share the bits above `top`; start there with zeros below.
    const int top = (mx == mn) ? -1 : 31 - __builtin_clz(mx ^ mn);
    uint32_t T = (top < 0) ? mx : (mx & ~((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int c = 0;
#pragma unroll
        for (int v = 0; v < VPT; ++v) c += __builtin_popcountll(__ballot(key[v] >= cand));
        if (c >= k) T = cand;
        if (c == k) {
            // exactly k keys are >= cand: they are the selection (the k-th and
            // (k+1)-th largest keys are on opposite sides of cand, so no tie
            // crosses the boundary); lowering T to cand - 1 keeps every one of
            // them "> T" below
            T = cand - 1u;
            break;
        }
    }
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        n_gt += key[v] > T;
        n_eq += key[v] == T;
    }
    const int need_eq = k - wave_sum(n_gt);
    int eq_seen = wave_excl_scan(n_eq);
    int sel = 0;
    bool take[VPT];
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
    int pos = wave_excl_scan(sel);
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        if (take[v] && pos < k) out[pos++] = t * VPT + v;
}

// ---------------------------------------------------------------- workgroup
constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;

// Block-wide sum; `red` holds kNW ints and is reused after a barrier.
__device__ __forceinline__ int block_sum(int x, int *red) {
    x = wave_sum(x);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) tot += red[w];
    return tot;
}

// Block-wide exclusive prefix sum in thread order.
__device__ __forceinline__ int block_excl_scan(int x, int *red) {
    const int incl = wave_excl_scan(x) + x;
    __syncthreads();
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < (int)(threadIdx.x >> 6); ++w) base += red[w];
    return base + incl - x;
}

template <int VPT>
__global__ __launch_bounds__(kNT) void topk_select_block(const float *__restrict__ scores, int e_stride,
                                                         const int32_t *__restrict__ cu_q,
                                                         const int32_t *__restrict__ cu_k, int num_seqs, int total_q,
                                                         int h, int B, int k, int sink, int local,
                                                         int32_t *__restrict__ ids) {
    __shared__ int hist[kBins];
    __shared__ int red[kNW];
    __shared__ uint32_t bc[4];
    __shared__ int exact;

    const long pair = blockIdx.x;
    const int t = threadIdx.x;
    const RowInfo ri = row_info(pair, cu_q, cu_k, num_seqs, h, B);
    const int E = ri.E;
    int32_t *out = ids + pair * k;
    if (E <= k) {
        for (int x = t; x < k; x += kNT) out[x] = x < E ? x : -1;
        return;
    }
    uint32_t key[VPT];
    load_keys<VPT>(key, scores + pair * e_stride, t, E, sink, local);

    uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        mx = max(mx, key[v]);
        mn = min(mn, key[v] ? key[v] : 0xffffffffu);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
    }
    if (t == 0) {
        bc[0] = 0u;
        bc[1] = 0xffffffffu;
        exact = 0;
    }
    __syncthreads();
    if ((t & 63) == 0) {
        atomicMax(&bc[0], mx);
        atomicMin(&bc[1], mn);
    }
    __syncthreads();
    mx = bc[0];
    mn = bc[1];

    // Radix select of the k-th largest key below the common prefix.
    uint32_t T;
    if (mx == mn) {
        T = mx;
    } else {
        int lo_bit = 32 - __builtin_clz(mx ^ mn);   // bits [0, lo_bit) are undecided
        uint32_t P = mx & ~((lo_bit >= 32) ? 0xffffffffu : ((1u << lo_bit) - 1u));
        int rank = k;   // 1-based rank among keys that match P on the decided bits
        while (lo_bit > 0) {
            const int w = min(kDigit, lo_bit);
            const int sh = lo_bit - w;
            const uint32_t hi_mask = ~((lo_bit >= 32) ? 0xffffffffu : ((1u << lo_bit) - 1u));
            for (int b = t; b < (1 << w); b += kNT) hist[b] = 0;
            __syncthreads();
#pragma unroll
            for (int v = 0; v < VPT; ++v)
                if (key[v] != 0u && (key[v] & hi_mask) == P) atomicAdd(&hist[(key[v] >> sh) & ((1u << w) - 1u)], 1);
            __syncthreads();
            // suffix counts: thread t owns the bins (1<<w)-1-2t and (1<<w)-2-2t (high to low)
            const int nb = 1 << w;
            const int b0 = nb - 1 - 2 * t, b1 = b0 - 1;
            const int c0 = (b0 >= 0) ? hist[b0] : 0, c1 = (b1 >= 0) ? hist[b1] : 0;
            const int above = block_excl_scan(c0 + c1, red);   // keys in bins above b0
            if (b0 >= 0 && above < rank && above + c0 >= rank) {
                bc[2] = (uint32_t)b0;
                bc[3] = (uint32_t)above;
                exact = (above + c0 == rank) ? 1 : 0;
            } else if (b1 >= 0 && above + c0 < rank && above + c0 + c1 >= rank) {
                bc[2] = (uint32_t)b1;
                bc[3] = (uint32_t)(above + c0);
                exact = (above + c0 + c1 == rank) ? 1 : 0;
            }
            __syncthreads();
            P |= bc[2] << sh;
            rank -= (int)bc[3];
            lo_bit = sh;
            const bool done = exact != 0;
            __syncthreads();
            if (done && P > 0u) {
                // the k-th largest key is the smallest in its bin: the keys
                // from that bin up are exactly the selection, no tie crosses it
                P -= 1u;
                break;
            }
        }
        T = P;
    }

    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        n_gt += key[v] > T;
        n_eq += key[v] == T;
    }
    const int need_eq = k - block_sum(n_gt, red);
    int eq_seen = block_excl_scan(n_eq, red);
    int sel = 0;
    bool take[VPT];
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
    int pos = block_excl_scan(sel, red);
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        if (take[v] && pos < k) out[pos++] = t * VPT + v;
}

template <int VPT>
hipError_t launch_wave(const Shape &s, const float *scores, int32_t *ids, hipStream_t st) {
    const long pairs = (long)s.total_q * s.h;
    hipLaunchKernelGGL((topk_select_wave<VPT>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, st, scores,
                       score_stride(s), s.cu_q, s.cu_k, s.num_seqs, s.total_q, s.h, s.B, s.top_k, s.sink, s.local,
                       ids);
    return hipGetLastError();
}

template <int VPT>
hipError_t launch_block(const Shape &s, const float *scores, int32_t *ids, hipStream_t st) {
    const long pairs = (long)s.total_q * s.h;
    hipLaunchKernelGGL((topk_select_block<VPT>), dim3((unsigned)pairs), dim3(kNT), 0, st, scores, score_stride(s),
                       s.cu_q, s.cu_k, s.num_seqs, s.total_q, s.h, s.B, s.top_k, s.sink, s.local, ids);
    return hipGetLastError();
}

}  // namespace

int max_select_blocks() { return kNT * 64; }

hipError_t launch_topk_select(const Shape &s, const float *scores, int32_t *ids, hipStream_t st) {
    const int e = score_stride(s);
    if (e <= 64 * 4) return launch_wave<4>(s, scores, ids, st);
    if (e <= 64 * 8) return launch_wave<8>(s, scores, ids, st);
    if (e <= 64 * 16) return launch_wave<16>(s, scores, ids, st);
    if (e <= 64 * 32) return launch_wave<32>(s, scores, ids, st);
    if (e <= kNT * 16) return launch_block<16>(s, scores, ids, st);
    if (e <= kNT * 32) return launch_block<32>(s, scores, ids, st);
    if (e <= kNT * 64) return launch_block<64>(s, scores, ids, st);
    return hipErrorInvalidValue;
}

}  // namespace msa
