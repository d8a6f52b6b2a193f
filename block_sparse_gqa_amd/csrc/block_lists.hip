// Inverted index of a prefill selection: for every (group g, key block) the
// list of (query row, selected slot) pairs whose selection holds that block.
// The ids are query-centric (each (row, group) lists its k blocks); a
// key-centric kernel (the block-centric forward schedule and the backward's
// dk / dv) needs the other direction -- the conversion the block-sparse prior
// art on the pages performs before its key-outer kernel ("MoBA / FlashMoBA"
// page, section 3.1, its third kernel).
//
// Keys are g * nb_max + blk_off[s] + j (j = block of sequence s) and list
// entries are row * top_k + slot, built in four passes: block offsets of the
// sequences, a count whose atomics also give each selection its place in its
// list, an exclusive scan of the counts, and a scatter.  The place a
// selection gets depends on the order the atomics run in, so list order is
// fixed only per run.
#include <algorithm>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kScanThreads = 1024;

// blk_off[s] = number of key blocks of the sequences before s.
__global__ __launch_bounds__(kScanThreads) void lists_block_offsets(const int32_t *__restrict__ cu_k, int num_seqs, int B,
                                                                 int32_t *__restrict__ blk_off) {
    __shared__ int carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base <= num_seqs; base += kScanThreads) {
        const int s = base + (int)threadIdx.x;
        const int nb = (s < num_seqs) ? (cu_k[s + 1] - cu_k[s] + B - 1) / B : 0;
        // inclusive scan over the threads (wave scan, then across waves)
        int x = nb;
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        __shared__ int wsum[kScanThreads / 64];
        if (lane == 63) wsum[threadIdx.x >> 6] = x;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < (int)(threadIdx.x >> 6); ++w) before += wsum[w];
        const int c = carry;
        if (s <= num_seqs) blk_off[s] = c + before + x - nb;
        __syncthreads();
        if (threadIdx.x == kScanThreads - 1) carry = c + before + x;
        __syncthreads();
    }
}

// Count (pass 0: each selection takes the next place of its key, kept in
// `place`) or store (pass 1) every valid selection (row, g, block j) under key
// g * nb_max + blk_off[s] + j; an entry is row * top_k + slot.
template <int PASS>
__global__ __launch_bounds__(256) void lists_invert(const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q,
                                                  const int32_t *__restrict__ cu_k, const int32_t *__restrict__ blk_off,
                                                  int num_seqs, int total_q, int h, int B, int top_k, int nb_max,
                                                  int32_t *__restrict__ cnt, int32_t *__restrict__ place,
                                                  const int32_t *__restrict__ off, int32_t *__restrict__ entries) {
    const long pair = (long)blockIdx.x * 256 + threadIdx.x;
    if (pair >= (long)total_q * h) return;
    const int row = (int)(pair / h), g = (int)(pair % h);
    const int s = seq_of_row(cu_q, num_seqs, row);
    const int len_q = cu_q[s + 1] - cu_q[s], len_k = cu_k[s + 1] - cu_k[s];
    const int p = len_k - len_q + (row - cu_q[s]);
    const int32_t *sel = ids + pair * top_k;
    for (int a = 0; a < top_k; ++a) {
        const int j = sel[a];
        if (j < 0 || j > p / B) continue;
        const long key = (long)g * nb_max + blk_off[s] + j;
        if (PASS == 0)
            place[pair * top_k + a] = atomicAdd(&cnt[key], 1);
        else
            entries[off[key] + place[pair * top_k + a]] = row * top_k + a;
    }
}

// Pass 0 with the counting done in LDS first: the workgroup's selections take
// local places in an LDS histogram of all keys, then each key the workgroup
// touched takes one block of global places with a single atomic, so popular
// blocks see one global atomic per workgroup instead of one per selection.
constexpr int kHistKeys = 16384;  // largest key count this path handles (64 KB of LDS)
__global__ __launch_bounds__(256) void lists_count_lds(const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q,
                                                     const int32_t *__restrict__ cu_k,
                                                     const int32_t *__restrict__ blk_off, int num_seqs, int total_q,
                                                     int h, int B, int top_k, int nb_max, int keys,
                                                     int32_t *__restrict__ cnt, int32_t *__restrict__ place) {
    extern __shared__ int hist[];  // keys entries
    for (int x = threadIdx.x; x < keys; x += 256) hist[x] = 0;
    __syncthreads();
    const long pair = (long)blockIdx.x * 256 + threadIdx.x;
    const bool live = pair < (long)total_q * h;
    int row = 0, g = 0, s = 0, p = -1;
    if (live) {
        row = (int)(pair / h);
        g = (int)(pair % h);
        s = seq_of_row(cu_q, num_seqs, row);
        p = (cu_k[s + 1] - cu_k[s]) - (cu_q[s + 1] - cu_q[s]) + (row - cu_q[s]);
    }
    const int32_t *sel = ids + pair * top_k;
    if (live) {
        for (int a = 0; a < top_k; ++a) {
            const int j = sel[a];
            if (j < 0 || j > p / B) continue;
            const int key = g * nb_max + blk_off[s] + j;
            place[pair * top_k + a] = atomicAdd(&hist[key], 1);
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < keys; x += 256) {
        const int c = hist[x];
        if (c > 0) hist[x] = atomicAdd(&cnt[x], c);
    }
    __syncthreads();
    if (live) {
        for (int a = 0; a < top_k; ++a) {
            const int j = sel[a];
            if (j < 0 || j > p / B) continue;
            place[pair * top_k + a] += hist[g * nb_max + blk_off[s] + j];
        }
    }
}

// Exclusive scan of n counts into off[0..n] (one workgroup).
__global__ __launch_bounds__(kScanThreads) void lists_scan(const int32_t *__restrict__ cnt, long n,
                                                         int32_t *__restrict__ off) {
    __shared__ int wsum[kScanThreads / 64];
    __shared__ int carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    for (long base = 0; base < n; base += kScanThreads) {
        const long i = base + threadIdx.x;
        const int v = (i < n) ? cnt[i] : 0;
        int x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) wsum[threadIdx.x >> 6] = x;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < (int)(threadIdx.x >> 6); ++w) before += wsum[w];
        const int c = carry;
        if (i < n) off[i] = c + before + x - v;
        __syncthreads();
        if (threadIdx.x == kScanThreads - 1) carry = c + before + x;
        __syncthreads();
    }
    if (threadIdx.x == 0) off[n] = carry;
}

__global__ __launch_bounds__(256) void fill_zero_i32(int32_t *__restrict__ p, long n) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0;
}

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

BlockLists block_lists_layout(const Shape &s) {
    BlockLists w{};
    w.nb_max = (long)s.total_k / s.B + s.num_seqs;
    size_t at = 0;
    w.blk_off = at;
    at += al256((size_t)(s.num_seqs + 1) * sizeof(int32_t));
    w.cnt = at;
    at += al256((size_t)s.h * w.nb_max * sizeof(int32_t));
    w.off = at;
    at += al256(((size_t)s.h * w.nb_max + 1) * sizeof(int32_t));
    w.entries = at;
    at += al256((size_t)s.total_q * s.h * s.top_k * sizeof(int32_t));
    w.place = at;
    at += al256((size_t)s.total_q * s.h * s.top_k * sizeof(int32_t));
    w.bytes = at;
    return w;
}

hipError_t launch_block_lists(const Shape &s, const int32_t *ids, const BlockLists &w, char *base, hipStream_t st) {
    int32_t *blk_off = reinterpret_cast<int32_t *>(base + w.blk_off);
    int32_t *cnt = reinterpret_cast<int32_t *>(base + w.cnt);
    int32_t *off = reinterpret_cast<int32_t *>(base + w.off);
    int32_t *entries = reinterpret_cast<int32_t *>(base + w.entries);
    int32_t *place = reinterpret_cast<int32_t *>(base + w.place);
    const long keys = (long)s.h * w.nb_max;
    const long pairs = (long)s.total_q * s.h;
    auto grid_of = [](long n, long per) { return dim3((unsigned)((n + per - 1) / per)); };
    const dim3 zgrid = grid_of(std::min(keys, 1L << 22), 256);

    hipLaunchKernelGGL(lists_block_offsets, dim3(1), dim3(kScanThreads), 0, st, s.cu_k, s.num_seqs, s.B, blk_off);
    hipLaunchKernelGGL(fill_zero_i32, zgrid, dim3(256), 0, st, cnt, keys);
    if (keys <= kHistKeys)
        hipLaunchKernelGGL(lists_count_lds, grid_of(pairs, 256), dim3(256), (size_t)keys * sizeof(int), st, ids,
                           s.cu_q, s.cu_k, blk_off, s.num_seqs, s.total_q, s.h, s.B, s.top_k, (int)w.nb_max,
                           (int)keys, cnt, place);
    else
        hipLaunchKernelGGL((lists_invert<0>), grid_of(pairs, 256), dim3(256), 0, st, ids, s.cu_q, s.cu_k, blk_off,
                           s.num_seqs, s.total_q, s.h, s.B, s.top_k, (int)w.nb_max, cnt, place, nullptr, nullptr);
    hipLaunchKernelGGL(lists_scan, dim3(1), dim3(kScanThreads), 0, st, cnt, keys, off);
    hipLaunchKernelGGL((lists_invert<1>), grid_of(pairs, 256), dim3(256), 0, st, ids, s.cu_q, s.cu_k, blk_off,
                       s.num_seqs, s.total_q, s.h, s.B, s.top_k, (int)w.nb_max, cnt, place, off, entries);
    return hipGetLastError();
}

}  // namespace msa
