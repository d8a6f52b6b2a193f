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
#include "msa_select.h"

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

// ---------------------------------------------------------------- one wave
// Grid (rows / 4, h): each wave owns one (row, group) of the rows
// [row0, row0 + rows); its row and sequence are wave-uniform (scalar).
template <int VPT>
__global__ __launch_bounds__(256) void topk_select_wave(const float *__restrict__ scores, int e_stride,
                                                        const int32_t *__restrict__ cu_q,
                                                        const int32_t *__restrict__ cu_k, int num_seqs, int row0,
                                                        int rows, int b_shift, int k, int sink, int local,
                                                        int32_t *__restrict__ ids) {
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r = (int)blockIdx.x * 4 + w;   // row within the chunk (scores holds the chunk's rows)
    if (r >= rows) return;
    const int g = (int)blockIdx.y, h = (int)gridDim.y;
    const int row = row0 + r;
    int s = 0;
    if (num_seqs > 1) {
        int lo = 0, hi = num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
        }
        s = lo;
    }
    const int q0 = cu_q[s];
    const int p = (cu_k[s + 1] - cu_k[s]) - (cu_q[s + 1] - q0) + (row - q0);
    const int E = (p >> b_shift) + 1;
    int32_t *out = ids + ((long)row * h + g) * k;
    if (E <= k) {
        for (int x = threadIdx.x & 63; x < k; x += 64) out[x] = x < E ? x : -1;
        return;
    }
    wave_topk_row_fit<VPT>(scores + ((long)r * h + g) * e_stride, E, k, sink, local, out);
}

// ---------------------------------------------------------------- workgroup
constexpr int kNT = 1024;
constexpr int kNW = kNT / 64;

// Inclusive prefix sum over the 64 lanes of a wave, in lane order, without
// LDS: row_shr steps of 1, 2, 4 and 8 inside each row of 16 lanes (a lane
// whose source lies outside its row adds 0), then the totals of the lower
// rows, read from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47);
    const int row = (int)(threadIdx.x & 63) >> 4;
    return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Workgroup-wide exclusive prefix sum in thread order, and the total.  `red`
// holds kNW ints; callers alternate between two such arrays, so the barrier
// of one call also separates the reads of the call before it from the
// writes of the call after it.
__device__ __forceinline__ int block_excl_scan(int x, int *red, int &total) {
    const int incl = wave_incl_scan(x);
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = incl;
    __syncthreads();
    const int w = (int)(threadIdx.x >> 6);
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
        const int r = red[i];
        base += i < w ? r : 0;
        tot += r;
    }
    total = tot;
    return base + incl - x;
}

template <int VPT>
__global__ __launch_bounds__(kNT) void topk_select_block(const float *__restrict__ scores, int e_stride,
                                                         const int32_t *__restrict__ cu_q,
                                                         const int32_t *__restrict__ cu_k, int num_seqs, int row0,
                                                         int h, int B, int k, int sink, int local,
                                                         int32_t *__restrict__ ids) {
    __shared__ __attribute__((aligned(16))) int hist[2][kBins];
    __shared__ int red[2][kNW];
    int nscan = 0;   // scans so far: scan i uses red[i & 1]
    __shared__ uint32_t bc[4];
    __shared__ uint32_t wmx[kNW], wmn[kNW];
    __shared__ int exact;

    const long pr = blockIdx.x;                 // pair within the rows from row0 (scores holds those)
    const long pair = (long)row0 * h + pr;
    const int t = threadIdx.x;
    // The row's scores are loaded before its length is known (the sequence
    // search below is a chain of dependent loads): every float4 of the row's
    // e_stride-float slot is readable, and keys past E are zeroed after.
    float f[VPT];
    {
        const float *src = scores + pr * e_stride;
#pragma unroll
        for (int v = 0; v < VPT; v += 4) {
            const int i = min(t * VPT + v, e_stride - 4);
            const float4 x = *reinterpret_cast<const float4 *>(src + i);
            f[v] = x.x; f[v + 1] = x.y; f[v + 2] = x.z; f[v + 3] = x.w;
        }
    }
    const RowInfo ri = row_info(pair, cu_q, cu_k, num_seqs, h, B);
    const int E = ri.E;
    int32_t *out = ids + pair * k;
    if (E <= k) {
        for (int x = t; x < k; x += kNT) out[x] = x < E ? x : -1;
        return;
    }
    // the first pass's histogram starts at zero (the barrier below orders it)
    for (int i = t; i < kBins / 4; i += kNT) reinterpret_cast<int4 *>(hist[0])[i] = make_int4(0, 0, 0, 0);
    uint32_t key[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int j = t * VPT + v;
        key[v] = j < E ? ((j < sink || j >= E - local) ? 0xffffffffu : order_key(f[v])) : 0u;
    }
    uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        mx = max(mx, key[v]);
        mn = min(mn, key[v] ? key[v] : 0xffffffffu);
    }
    mx = wave_max_u32(mx);
    mn = wave_min_u32(mn);
    if ((t & 63) == 0) {
        wmx[t >> 6] = mx;
        wmn[t >> 6] = mn;
    }
    if (t == 0) exact = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
        mx = max(mx, wmx[i]);
        mn = min(mn, wmn[i]);
    }

    // Radix select of the k-th largest key below the common prefix.
    uint32_t T;
    if (mx == mn) {
        T = mx;
    } else {
        int lo_bit = 32 - __builtin_clz(mx ^ mn);   // bits [0, lo_bit) are undecided
        uint32_t P = mx & ~((lo_bit >= 32) ? 0xffffffffu : ((1u << lo_bit) - 1u));
        int rank = k;   // 1-based rank among keys that match P on the decided bits
        for (int pass = 0; lo_bit > 0; ++pass) {
            const int w = min(kDigit, lo_bit);
            const int sh = lo_bit - w;
            const uint32_t hi_mask = ~((lo_bit >= 32) ? 0xffffffffu : ((1u << lo_bit) - 1u));
            int *hc = hist[pass & 1];
            // Clear the other histogram for the next pass: its last reads (the
            // previous pass's scan) came before that pass's decision barrier.
            for (int i = t; i < kBins / 4; i += kNT)
                reinterpret_cast<int4 *>(hist[(pass + 1) & 1])[i] = make_int4(0, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < VPT; ++v)
                if (key[v] != 0u && (key[v] & hi_mask) == P) atomicAdd(&hc[(key[v] >> sh) & ((1u << w) - 1u)], 1);
            __syncthreads();
            // suffix counts: thread t owns the bins (1<<w)-1-2t and (1<<w)-2-2t (high to low)
            const int nb = 1 << w;
            const int b0 = nb - 1 - 2 * t, b1 = b0 - 1;
            const int c0 = (b0 >= 0) ? hc[b0] : 0, c1 = (b1 >= 0) ? hc[b1] : 0;
            int all;
            const int above = block_excl_scan(c0 + c1, red[nscan++ & 1], all);   // keys in bins above b0
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
            // (no barrier here: the next pass clears hist and rewrites bc and
            // exact only after barriers that every thread reaches after these
            // reads)
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
    // One scan of both counts: keys > T in the low 13 bits (at most k <=
    // 4096 of them in the whole row, so no carry), keys == T above them (at
    // most kNT * 64 = 2^16, so the sum stays below 2^29).
    int both;
    const int ex = block_excl_scan((n_eq << 13) | n_gt, red[nscan++ & 1], both);
    // Equal keys are kept lowest index first, so the keys kept in lower
    // threads are their keys > T plus min(their keys == T, need_eq): the
    // same scan gives every thread its first output place.
    const int need_eq = k - (both & 0x1fff);
    int eq_seen = ex >> 13;
    int pos = (ex & 0x1fff) + min(eq_seen, need_eq);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        bool tk = key[v] > T;
        if (key[v] == T) {
            tk = eq_seen < need_eq;
            ++eq_seen;
        }
        if (tk && pos < k) out[pos++] = t * VPT + v;
    }
}

template <int VPT>
hipError_t launch_wave(const Shape &s, const float *scores, int32_t *ids, hipStream_t st) {
    if (s.B < 1 || (s.B & (s.B - 1)) != 0 || s.h > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL((topk_select_wave<VPT>), dim3((unsigned)((s.rows + 3) / 4), (unsigned)s.h), dim3(256), 0, st,
                       scores, score_stride(s), s.cu_q, s.cu_k, s.num_seqs, s.row0, s.rows, __builtin_ctz(s.B),
                       s.top_k, s.sink, s.local, ids);
    return hipGetLastError();
}

template <int VPT>
hipError_t launch_block(const Shape &s, const float *scores, int32_t *ids, hipStream_t st) {
    const long pairs = (long)s.rows * s.h;
    hipLaunchKernelGGL((topk_select_block<VPT>), dim3((unsigned)pairs), dim3(kNT), 0, st, scores, score_stride(s),
                       s.cu_q, s.cu_k, s.num_seqs, s.row0, s.h, s.B, s.top_k, s.sink, s.local, ids);
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
