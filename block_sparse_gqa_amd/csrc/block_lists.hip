// Inverted index of a prefill selection: for every (group g, key block) the
// list of (query row, selected slot) pairs whose selection holds that block.
// The ids are query-centric (each (row, group) lists its k blocks); a
// key-centric kernel (the block-centric forward schedule and the backward's
// dk / dv) needs the other direction -- the conversion the block-sparse prior
// art on the pages performs before its key-outer kernel ("MoBA / FlashMoBA"
// page, section 3.1, its third kernel).
//
// Keys are g * nb_max + blk_off[s] + j (j = block of sequence s) and list
// entries are (row - row0) * top_k + slot for the rows [row0, row0 + rows) of
// one chunk (the whole problem unless the caller splits it), built in four
// passes: block offsets of the
// sequences, a count whose atomics also give each selection its place in its
// list, an exclusive scan of the counts, and a scatter.  The place a
// selection gets depends on the order the atomics run in, so list order is
// fixed only per run, unless the caller asks for a fifth pass that sorts
// every list ascending (the backward does: its dk and dv sums run in list
// order).
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

// Key of selection element e = (rr * h + g) * top_k + a of the chunk (rr =
// row - row0; `ids` points at the chunk's first row): g * nb_max +
// blk_off[s] + j for the block j in that slot, or -1 when the slot is empty or
// the block is not visible to the row.  *entry receives rr * top_k + a.
// Threads take consecutive elements, so the reads of the ids (and of `place`)
// are coalesced.
__device__ __forceinline__ int selection_key(const int32_t *__restrict__ ids, long e,
                                             const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
                                             const int32_t *__restrict__ blk_off, int num_seqs, int h, int B,
                                             int top_k, int nb_max, int row0, int blocks_from, int split_tq,
                                             int *entry) {
    const long pair = e / top_k;
    const int a = (int)(e - pair * top_k);
    const int rr = (int)(pair / h), g = (int)(pair - (long)rr * h);
    const int row = row0 + rr;
    *entry = rr * top_k + a;
    const int j = ids[e];
    if (j < 0) return -1;
    const int s = seq_of_row(cu_q, num_seqs, row);
    const int shift = (cu_k[s + 1] - cu_k[s]) - (cu_q[s + 1] - cu_q[s]);
    const int p = shift + (row - cu_q[s]);
    if (j > p / B) return -1;
    // rows of query tiles starting below blocks_from belong to the other schedule
    if (blocks_from > p - (row - cu_q[s]) % split_tq) return -1;
    return g * nb_max + blk_off[s] + j;
}

// Count (pass 0: each selection takes the next place of its key, kept in
// `place`) or store (pass 1) every valid selection element under its key; an
// entry is row * top_k + slot.  Grid-stride over the n elements.
template <int PASS>
__global__ __launch_bounds__(256) void lists_invert(const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q,
                                                  const int32_t *__restrict__ cu_k, const int32_t *__restrict__ blk_off,
                                                  int num_seqs, int h, int B, int top_k, int nb_max, int row0,
                                                  int blocks_from, int split_tq, long n,
                                                  int32_t *__restrict__ cnt, int32_t *__restrict__ place,
                                                  const int32_t *__restrict__ off, int32_t *__restrict__ entries) {
    for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) {
        int entry;
        const int key = selection_key(ids, e, cu_q, cu_k, blk_off, num_seqs, h, B, top_k, nb_max, row0, blocks_from, split_tq, &entry);
        if (key < 0) continue;
        if (PASS == 0)
            place[e] = atomicAdd(&cnt[key], 1);
        else
            entries[off[key] + place[e]] = entry;
    }
}

// Pass 0 with the counting done in LDS first: the elements of one contiguous
// chunk take local places in an LDS histogram of all keys, then each key the
// chunk touched takes one block of global places with a single atomic, so
// popular blocks see one global atomic per workgroup instead of one per
// selection.
constexpr int kHistKeys = 16384;  // largest key count this path handles (64 KB of LDS)
constexpr int kCountThreads = 1024;   // wide workgroups: the histogram's LDS caps how many fit on a CU
__global__ __launch_bounds__(kCountThreads) void lists_count_lds(const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q,
                                                     const int32_t *__restrict__ cu_k,
                                                     const int32_t *__restrict__ blk_off, int num_seqs, int h, int B,
                                                     int top_k, int nb_max, int row0, int blocks_from, int split_tq,
                                                     int keys, long n, long chunk,
                                                     int32_t *__restrict__ cnt, int32_t *__restrict__ place) {
    extern __shared__ int hist[];  // keys entries
    for (int x = threadIdx.x; x < keys; x += kCountThreads) hist[x] = 0;
    __syncthreads();
    const long e0 = (long)blockIdx.x * chunk, e1 = e0 + chunk < n ? e0 + chunk : n;
    for (long e = e0 + threadIdx.x; e < e1; e += kCountThreads) {
        int entry;
        const int key = selection_key(ids, e, cu_q, cu_k, blk_off, num_seqs, h, B, top_k, nb_max, row0, blocks_from, split_tq, &entry);
        if (key >= 0) place[e] = atomicAdd(&hist[key], 1);
    }
    __syncthreads();
    for (int x = threadIdx.x; x < keys; x += kCountThreads) {
        const int c = hist[x];
        if (c > 0) hist[x] = atomicAdd(&cnt[x], c);
    }
    __syncthreads();
    for (long e = e0 + threadIdx.x; e < e1; e += kCountThreads) {
        int entry;
        const int key = selection_key(ids, e, cu_q, cu_k, blk_off, num_seqs, h, B, top_k, nb_max, row0, blocks_from, split_tq, &entry);
        if (key >= 0) place[e] += hist[key];
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

// Sorts each key's entries ascending (bitonic, in LDS), so that a kernel
// walking a list sees its entries in one fixed order whatever order the
// atomics of the count pass handed out the places in.  One instance per list
// length class: lists of lo < n <= CAP entries; longer ones are the next
// instance's, and lists longer than the largest CAP keep their order.
template <int CAP, int NT>
__global__ __launch_bounds__(NT) void lists_sort(const int32_t *__restrict__ off, int32_t *__restrict__ entries,
                                                 int lo) {
    __shared__ int sbuf[CAP];
    const long key = blockIdx.x;
    const int e0 = off[key], n = off[key + 1] - e0;
    if (n <= lo || n > CAP || n < 2) return;
    int N = 2;
    while (N < n) N <<= 1;
    for (int i = threadIdx.x; i < N; i += NT) sbuf[i] = i < n ? entries[e0 + i] : 0x7fffffff;
    __syncthreads();
    for (int kk = 2; kk <= N; kk <<= 1) {
        for (int j = kk >> 1; j > 0; j >>= 1) {
            // pair p compares i (bit j clear) with i + j
            for (int p = threadIdx.x; p < N / 2; p += NT) {
                const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));
                const int l = i | j;
                const int a = sbuf[i], b = sbuf[l];
                if ((a > b) == ((i & kk) == 0)) {
                    sbuf[i] = b;
                    sbuf[l] = a;
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < n; i += NT) entries[e0 + i] = sbuf[i];
}

constexpr int kSortSmall = 2048;   // most lists: 8 KB of LDS, many workgroups per CU
constexpr int kSortCap = 16384;    // longest list sorted (64 KB of LDS)

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
    at += al256((size_t)s.rows * s.h * s.top_k * sizeof(int32_t));
    w.place = at;
    at += al256((size_t)s.rows * s.h * s.top_k * sizeof(int32_t));
    w.bytes = at;
    return w;
}

hipError_t launch_block_lists(const Shape &s, const int32_t *ids, const BlockLists &w, char *base, hipStream_t st,
                              bool sorted) {
    int32_t *blk_off = reinterpret_cast<int32_t *>(base + w.blk_off);
    int32_t *cnt = reinterpret_cast<int32_t *>(base + w.cnt);
    int32_t *off = reinterpret_cast<int32_t *>(base + w.off);
    int32_t *entries = reinterpret_cast<int32_t *>(base + w.entries);
    int32_t *place = reinterpret_cast<int32_t *>(base + w.place);
    const long keys = (long)s.h * w.nb_max;
    const long n = (long)s.rows * s.h * s.top_k;   // selection elements of the chunk
    ids += (size_t)s.row0 * s.h * s.top_k;
    auto grid_of = [](long m, long per) { return dim3((unsigned)((m + per - 1) / per)); };
    const dim3 zgrid = grid_of(std::min(keys, 1L << 22), 256);
    const dim3 egrid = grid_of(std::min(n, 16384L * 256), 256);   // grid-stride over the elements

    hipLaunchKernelGGL(lists_block_offsets, dim3(1), dim3(kScanThreads), 0, st, s.cu_k, s.num_seqs, s.B, blk_off);
    hipLaunchKernelGGL(fill_zero_i32, zgrid, dim3(256), 0, st, cnt, keys);
    if (n > 0 && keys <= kHistKeys) {
        // chunks of at least 4096 elements, at most 512 workgroups
        const long wgs = std::min(512L, (n + 4095) / 4096);
        const long chunk = ((n + wgs - 1) / wgs + kCountThreads - 1) / kCountThreads * kCountThreads;
        hipLaunchKernelGGL(lists_count_lds, grid_of(n, chunk), dim3(kCountThreads), (size_t)keys * sizeof(int), st, ids, s.cu_q,
                           s.cu_k, blk_off, s.num_seqs, s.h, s.B, s.top_k, (int)w.nb_max, s.row0, s.blocks_from,
                           s.split_tq, (int)keys, n, chunk, cnt, place);
    } else if (n > 0) {
        hipLaunchKernelGGL((lists_invert<0>), egrid, dim3(256), 0, st, ids, s.cu_q, s.cu_k, blk_off, s.num_seqs, s.h,
                           s.B, s.top_k, (int)w.nb_max, s.row0, s.blocks_from, s.split_tq, n, cnt, place, nullptr,
                           nullptr);
    }
    hipLaunchKernelGGL(lists_scan, dim3(1), dim3(kScanThreads), 0, st, cnt, keys, off);
    if (n > 0)
        hipLaunchKernelGGL((lists_invert<1>), egrid, dim3(256), 0, st, ids, s.cu_q, s.cu_k, blk_off, s.num_seqs, s.h,
                           s.B, s.top_k, (int)w.nb_max, s.row0, s.blocks_from, s.split_tq, n, cnt, place, off,
                           entries);
    if (sorted && n > 0) {
        hipLaunchKernelGGL((lists_sort<kSortSmall, 256>), dim3((unsigned)keys), dim3(256), 0, st, off, entries, 1);
        // a list holds at most one entry per row of the chunk
        if (s.rows > kSortSmall)
            hipLaunchKernelGGL((lists_sort<kSortCap, 1024>), dim3((unsigned)keys), dim3(1024), 0, st, off, entries,
                               kSortSmall);
    }
    return hipGetLastError();
}

}  // namespace msa
