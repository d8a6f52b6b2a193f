// Index branch for decode: one query per sequence scans the whole index-key
// cache.  Bandwidth-bound: every K_idx byte is read once and scored against
// all h index queries of the sequence at the same time (the index key has a
// single head: "MiniMax Goes Sparse", section 1, step 1; the decode scan
// touching the full length is discussed in section 3).
//
// Loads.  Each load instruction of a wave reads whole 128-byte lines (lane i
// takes the i-th 16-byte chunk of a contiguous 1 KB run): instructions that
// touch half lines stream markedly slower on this part.  The block is then
// re-laid out through a padded per-wave LDS tile into the MFMA operand
// layout.  The wave's next two blocks are already in flight in registers while
// the current one is scored; blocks are dealt round-robin over the waves.
// Scans larger than the MALL could keep between calls use non-temporal loads.
//
// Scores.  Tokens run along the M dimension of v_mfma_f32_16x16x32_bf16 and
// the h groups along N, so each lane holds 4 tokens of one group per 16-token
// tile; the Block Max Pool is an in-register max over the block's tiles plus
// two lane swaps (xor 16, xor 32).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kWaves = 4;

template <int DI, int B>
struct IdxTile {
    static constexpr int ROW = DI * 2 + 16;          // padded LDS row: conflict-free operand reads
    static constexpr int CPR = DI / 8;               // 16-byte chunks per key row
    static constexpr int LOADS = B * CPR / 64;       // 16-byte loads per lane per block
};

// PAGED: k_idx is a pool of pages of B rows and block j of sequence s sits in
// page table[s * table_stride + j] (clamped into [0, num_pages)).  NT: the
// index keys are loaded non-temporal.
template <int DI, int B, bool PAGED, bool NT>
__global__ __launch_bounds__(256) void index_decode_blockmax(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int h,
    float *__restrict__ scores, int e_stride, const int32_t *__restrict__ table, int table_stride,
    int num_pages) {
    using T = IdxTile<DI, B>;
    constexpr int KS = DI / 32;   // 32-dim k-steps
    constexpr int TT = B / 16;    // 16-token tiles per block
    __shared__ __attribute__((aligned(16))) char tile[kWaves][B * T::ROW];

    const int s = blockIdx.y;
    const int row = cu_q[s + 1] - 1;                  // the sequence's (last) query
    const int k_begin = cu_k[s], len_k = cu_k[s + 1] - k_begin;
    const int p = len_k - 1;
    const int E = p / B + 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar block loop
    // Blocks are dealt out round-robin over every wave of the sequence, so the
    // waves in flight at any moment read neighbouring blocks.
    const int nwaves = gridDim.x * kWaves;
    const int j_first = blockIdx.x * kWaves + wave;
    const int g = lane & 15, q4 = lane >> 4;
    char *my = tile[wave];

    bf16x8 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qop[ks] = as_bf16x8(load16_if(q_idx + ((size_t)row * h + g) * DI + 32 * ks + 8 * q4, g < h, q_idx));

    // Paged cache: lane i holds the page of the wave's i-th block, read once
    // up front so that no block's loads wait on a table read.
    int pages = 0;
    if constexpr (PAGED) {
        const long ji = (long)j_first + (long)lane * nwaves;
        if (ji < E) pages = min(max(table[(size_t)s * table_stride + ji], 0), num_pages - 1);
    }

    // Unconditional loads (no select on the loaded values, so nothing waits
    // for them until the block is used); rows past the sequence end repeat
    // its last key and are masked below.  A prefetch past the wave's last
    // block (`real` false) is never scored: plain loads repeat that block, a
    // cache hit, but a non-temporal load of it would go back to HBM, so those
    // read the sequence's index-query row instead, which the qop loads above
    // left in L2.
    const uint16_t *hot = q_idx + (size_t)row * h * DI;
    const int hot_elems = h * DI;
    auto load_block = [&](uint4(&r)[T::LOADS], int j, bool real) {
        j = __builtin_amdgcn_readfirstlane(j);
        const int t0 = j * B;
        // pool row of the block's first token
        size_t row0 = (size_t)(k_begin + t0);
        if constexpr (PAGED) {
            const int i = (j - j_first) / nwaves;   // the wave's i-th block
            const int pg = i < 64 ? __builtin_amdgcn_readlane(pages, i)
                                  : min(max(table[(size_t)s * table_stride + j], 0), num_pages - 1);
            row0 = (size_t)pg * B;
        }
#pragma unroll
        for (int x = 0; x < T::LOADS; ++x) {
            const int ci = x * 64 + lane;
            const int tok = ci / T::CPR, c16 = ci % T::CPR;
            const int t = min(tok, len_k - 1 - t0);
            const uint16_t *pk = k_idx + (row0 + t) * DI + c16 * 8;
            if constexpr (NT)
                r[x] = load16_nt(real ? pk : hot + (ci * 8) % hot_elems);
            else
                r[x] = load16(pk);
        }
    };

    // One block: registers -> padded LDS tile -> MFMA -> Block Max Pool.
    auto score_block = [&](const uint4(&r)[T::LOADS], int j) {
#pragma unroll
        for (int x = 0; x < T::LOADS; ++x) {
            const int ci = x * 64 + lane;
            const int tok = ci / T::CPR, c16 = ci % T::CPR;
            *reinterpret_cast<uint4 *>(my + tok * T::ROW + c16 * 16) = r[x];
        }
        wave_lds_sync();
        float m = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a =
                    *reinterpret_cast<const bf16x8 *>(my + (tt * 16 + g) * T::ROW + (32 * ks + 8 * q4) * 2);
                acc = mfma16x16x32(a, qop[ks], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = j * B + tt * 16 + 4 * q4 + i;
                m = fmaxf(m, t <= p ? acc[i] : -INFINITY);
            }
        }
        wave_lds_sync();   // operand reads done before the next block is written
        m = max_xor16(m);
        m = max_xor32(m);
        if (lane < h) scores[((size_t)row * h + lane) * e_stride + j] = m;
    };

    // Three register sets rotate so that two blocks are in flight while one
    // is scored; the loop is unrolled by three to keep the sets static.
    // Loads are issued unconditionally (past the wave's last block they
    // repeat it, a cache hit), so the wait before each block covers exactly
    // that block's loads and never the two younger ones.
    if (j_first >= E) return;
    const int j_last = j_first + (E - 1 - j_first) / nwaves * nwaves;
    uint4 ra[T::LOADS], rb[T::LOADS], rc[T::LOADS];
    int j = j_first;
    load_block(ra, j, true);
    load_block(rb, min(j + nwaves, j_last), j + nwaves <= j_last);
    for (;; j += 3 * nwaves) {
        load_block(rc, min(j + 2 * nwaves, j_last), j + 2 * nwaves <= j_last);
        score_block(ra, j);
        if (j + nwaves > j_last) break;
        load_block(ra, min(j + 3 * nwaves, j_last), j + 3 * nwaves <= j_last);
        score_block(rb, j + nwaves);
        if (j + 2 * nwaves > j_last) break;
        load_block(rb, min(j + 4 * nwaves, j_last), j + 4 * nwaves <= j_last);
        score_block(rc, j + 2 * nwaves);
        if (j + 3 * nwaves > j_last) break;
    }
}

template <int DI, int B>
hipError_t launch(const Shape &s, const uint16_t *q_idx, const uint16_t *k_idx, float *scores, hipStream_t st) {
    // 4 x 1M context (537 MB of index keys): 109 -> 105 us of index_topk with
    // non-temporal loads; 8 x 64K (67 MB) stays plain: 24 us back to back,
    // against 29 us non-temporal, since plain loads leave it in the MALL.
    const bool nt = (double)s.total_k * DI * 2.0 > kDecodeStreamBytes;
    // Each wave takes every nwaves-th block.  A streamed scan runs on about
    // 1536 workgroups: two rounds of the 768 that fit at once (three per CU,
    // by registers), so no round runs on part of the chip.  4 x 1M context,
    // index_topk: 103.5 us against 107-108.5 with 768, 3072 and 4096; the
    // paged form ties with 2048 and beats 4096 (its waves first read their
    // blocks' pages, a dependent load that longer-lived waves pay less often).
    // A scan the MALL holds takes one round of 768: 8 x 64K decode 52.8 us
    // against 53.7 us with 1536 back to back (57.8 against 60.0 behind a
    // flush).
    const int e_max = (s.max_k + s.B - 1) / s.B;
    int per_seq = ((nt ? 1536 : 768) + s.num_seqs - 1) / s.num_seqs;
    const int need = (e_max + kWaves - 1) / kWaves;
    if (per_seq > need) per_seq = need;
    dim3 grid(per_seq, s.num_seqs);
    auto go = [&](auto paged, auto ntag) {
        constexpr bool P = decltype(paged)::value, N = decltype(ntag)::value;
        hipLaunchKernelGGL((index_decode_blockmax<DI, B, P, N>), grid, dim3(256), 0, st, q_idx, k_idx, s.cu_q, s.cu_k,
                           s.h, scores, score_stride(s), P ? s.table : nullptr, P ? s.table_stride : 0,
                           P ? s.num_pages : 0);
    };
    if (s.table != nullptr) {
        if (nt) go(std::true_type{}, std::true_type{}); else go(std::true_type{}, std::false_type{});
    } else {
        if (nt) go(std::false_type{}, std::true_type{}); else go(std::false_type{}, std::false_type{});
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_decode(const Shape &s, const uint16_t *q_idx, const uint16_t *k_idx, float *scores,
                               hipStream_t st) {
    if (s.h > 16) return hipErrorInvalidValue;
    if (s.d_idx == 32 && s.B == 64) return launch<32, 64>(s, q_idx, k_idx, scores, st);
    if (s.d_idx == 32 && s.B == 128) return launch<32, 128>(s, q_idx, k_idx, scores, st);
    if (s.d_idx == 64 && s.B == 64) return launch<64, 64>(s, q_idx, k_idx, scores, st);
    if (s.d_idx == 64 && s.B == 128) return launch<64, 128>(s, q_idx, k_idx, scores, st);
    return hipErrorInvalidValue;
}

}  // namespace msa
