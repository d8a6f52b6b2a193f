// Sparse branch, prefill: exact softmax attention of every query head over
// the visible tokens of the blocks its GQA group selected, read from the
// original K/V ("MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a
// minimal sparse attention", second layer; "MiniMax Goes Sparse", section 1,
// step 2).
//
// Reuse.  The heads of a group share one selection, and neighbouring queries
// of a group pick overlapping block sets.  A workgroup therefore owns a tile
// of Tq consecutive queries of one group (all G heads), forms the union of
// their selected blocks and streams each union block through LDS once, as
// 64-token K and V sub-blocks.
//
// Staging.  A 4-stage LDS ring is filled with direct buffer->LDS loads
// (buffer_load_dwordx4 ... lds: lane i of a load writes base + 16*i), so
// several sub-blocks are in flight per workgroup without holding staging
// registers.  For d = 128 every load fills four whole token rows and groups of
// four rows sit 1056 bytes apart; for d = 64 rows are padded (K: 2d+16 bytes,
// V: 2d+64 bytes).  Either way the K operand reads and the transposing V reads
// are bank-conflict free.  Ring reads are issued in inline asm (each block
// waits for its own results) so the compiler does not serialise them behind
// the in-flight ring loads.  Stages are handed between waves with LDS stamps
// and counters instead of workgroup barriers (the protocol is described at
// the loop), so the waves sharing a SIMD drift apart and overlap one
// another's MFMA and VALU work.
//
// Rows.  A row is one (query, head) pair.  Each of the NW waves owns one
// fixed tile of 16 rows (16/G queries x G heads) whose O accumulators,
// reference max and running sum stay in registers for the whole tile; a wave
// visits only the sub-blocks whose block one of its queries selected, and
// masks the rows whose query did not (and future tokens).
//   S^T = K . Q^T     v_mfma_f32_16x16x32_bf16, A = K rows from LDS,
//                     B = Q^T resident in registers;
//   O^T += V^T . P^T  v_mfma_f32_16x16x32_f16, A = V^T read with the
//                     transposing ds_read_b64_tr_b16 from an fp16 copy of V
//                     scaled by one power of two per (sequence, KV head),
//                     B = P^T (fp16) straight from the S^T accumulators.
// Workgroups are numbered group-fastest, so with 8 groups all tiles of a
// group run on the same XCD and share its L2.
#include <algorithm>
#include <cstdlib>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;

constexpr int kWin = 256;    // key blocks per union window (one per thread)
constexpr int kStages = 4;   // ring depth (sub-blocks)
// Default bound on polls of one ready stamp (each poll sleeps ~64 cycles,
// so about 30 ms at 2.4 GHz: far above any wait of a working protocol).  A
// wait that reaches the bound counts itself in the workspace's wait word and
// goes on; the call's output is then not valid.
constexpr int kSpinLimit = 1 << 20;
// Fourth word of a raw buffer resource (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

// Layout of one ring stage (a 64-token sub-block of K, then of V).
//  * d = 128 ("grouped"): every 1 KB load instruction fills 4 whole token
//    rows; groups of 4 rows sit GROUP = 1056 bytes apart.  16-token MFMA
//    tile tt holds tokens 4m + tt (m = 0..15), i.e. row tt of every group, so
//    lane m of a K operand read and the lanes of a transposing V read step
//    through groups, 1056 = 32 (mod 256) bytes apart: bank-conflict free for
//    both ds_read_b128 and ds_read_b64_tr_b16.
//  * d = 64 ("padded"): rows padded to 2d+16 (K) and 2d+64 (V) bytes, tile
//    tt holds tokens 16 tt .. 16 tt + 15; loads fill 16-byte slots in order.
template <int D>
struct Ring {
    static constexpr bool GROUPED = (D == 128);
    static constexpr int GROUP = 1056;
    static constexpr int KROW = D * 2 + 16;
    static constexpr int VROW = D * 2 + 64;
    static constexpr int KSLOT_ROW = KROW / 16;   // 16-byte slots per row
    static constexpr int VSLOT_ROW = VROW / 16;
    static constexpr int KINSTR = KSLOT_ROW;      // 64 rows x slots / 64 lanes per load
    static constexpr int VINSTR = VSLOT_ROW;
    static constexpr int KBYTES = GROUPED ? 16 * GROUP : 64 * KROW;
    static constexpr int VBYTES = GROUPED ? 16 * GROUP : 64 * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    // K operand reads: lane stride (MFMA row) and offset between 16-token tiles
    static constexpr int K_LANE = GROUPED ? GROUP : KROW;
    static constexpr int K_TILE = GROUPED ? 256 : 16 * KROW;
    // transposing V reads: lane-group stride, tile 2 s2 + 1 offset, s2 offset
    static constexpr int V_LANE = GROUPED ? GROUP : VROW;
    static constexpr int V_ODD = GROUPED ? 256 : 16 * VROW;
    static constexpr int V_S2 = GROUPED ? 512 : 32 * VROW;
    // token (within the sub-block) of MFMA row 4 q4 + i of tile tt
    static __device__ __forceinline__ int token(int tt, int q4, int i) {
        return GROUPED ? 16 * q4 + 4 * i + tt : 16 * tt + 4 * q4 + i;
    }
};

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Multi-instruction asm blocks mark their outputs early-clobber ("=&v"): an
// output register must never alias the address input that later reads in the
// same block still use.

// K operands of two 16-token tiles (rows tok and tok + 16, all k-steps of
// 32 dims, 64 bytes apart), one wait.  ROW16 = 16 rows in bytes.
template <int KS, int ROW16>
__device__ __forceinline__ void lds_k_pair(uint4 (&a)[2 * KS], uint32_t addr) {
    if constexpr (KS == 4) {
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:64\n\t"
            "ds_read_b128 %2, %8 offset:128\n\t"
            "ds_read_b128 %3, %8 offset:192\n\t"
            "ds_read_b128 %4, %8 offset:%9\n\t"
            "ds_read_b128 %5, %8 offset:%9+64\n\t"
            "ds_read_b128 %6, %8 offset:%9+128\n\t"
            "ds_read_b128 %7, %8 offset:%9+192\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
            : "v"(addr), "i"(ROW16)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %4 offset:64\n\t"
            "ds_read_b128 %2, %4 offset:%5\n\t"
            "ds_read_b128 %3, %4 offset:%5+64\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
            : "v"(addr), "i"(ROW16)
            : "memory");
    }
}

// Transposing V reads of one 32-token half for every 16-column d-tile: rows
// tok and tok + 16 (ROW16 bytes apart), d-tiles 32 bytes apart, one wait.
template <int DT, int ROW16>
__device__ __forceinline__ void lds_v_half(i16x4 (&va)[DT], i16x4 (&vb)[DT], uint32_t addr) {
    if constexpr (DT == 8) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16\n\t"
            "ds_read_b64_tr_b16 %1, %16 offset:%17\n\t"
            "ds_read_b64_tr_b16 %2, %16 offset:32\n\t"
            "ds_read_b64_tr_b16 %3, %16 offset:%17+32\n\t"
            "ds_read_b64_tr_b16 %4, %16 offset:64\n\t"
            "ds_read_b64_tr_b16 %5, %16 offset:%17+64\n\t"
            "ds_read_b64_tr_b16 %6, %16 offset:96\n\t"
            "ds_read_b64_tr_b16 %7, %16 offset:%17+96\n\t"
            "ds_read_b64_tr_b16 %8, %16 offset:128\n\t"
            "ds_read_b64_tr_b16 %9, %16 offset:%17+128\n\t"
            "ds_read_b64_tr_b16 %10, %16 offset:160\n\t"
            "ds_read_b64_tr_b16 %11, %16 offset:%17+160\n\t"
            "ds_read_b64_tr_b16 %12, %16 offset:192\n\t"
            "ds_read_b64_tr_b16 %13, %16 offset:%17+192\n\t"
            "ds_read_b64_tr_b16 %14, %16 offset:224\n\t"
            "ds_read_b64_tr_b16 %15, %16 offset:%17+224\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(va[0]), "=&v"(vb[0]), "=&v"(va[1]), "=&v"(vb[1]), "=&v"(va[2]), "=&v"(vb[2]), "=&v"(va[3]),
              "=&v"(vb[3]), "=&v"(va[4]), "=&v"(vb[4]), "=&v"(va[5]), "=&v"(vb[5]), "=&v"(va[6]), "=&v"(vb[6]),
              "=&v"(va[7]), "=&v"(vb[7])
            : "v"(addr), "i"(ROW16)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:%9\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:32\n\t"
            "ds_read_b64_tr_b16 %3, %8 offset:%9+32\n\t"
            "ds_read_b64_tr_b16 %4, %8 offset:64\n\t"
            "ds_read_b64_tr_b16 %5, %8 offset:%9+64\n\t"
            "ds_read_b64_tr_b16 %6, %8 offset:96\n\t"
            "ds_read_b64_tr_b16 %7, %8 offset:%9+96\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(va[0]), "=&v"(vb[0]), "=&v"(va[1]), "=&v"(vb[1]), "=&v"(va[2]), "=&v"(vb[2]), "=&v"(va[3]),
              "=&v"(vb[3])
            : "v"(addr), "i"(ROW16)
            : "memory");
    }
}

__device__ __forceinline__ uint32_t lds_u32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ unsigned long long lds_u64(uint32_t addr) {
    unsigned long long v;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// (no wait: the wave's later LDS operations are ordered after it anyway, and
// the waves that poll the word need no more than that it lands)
__device__ __forceinline__ void lds_store_u32(uint32_t addr, int v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
// One wave-level increment of the counter at addr; returns its prior value
// (the same in every lane).
__device__ __forceinline__ int lds_add_rtn_u32(uint32_t addr) {
    int prior = 0;
    if ((threadIdx.x & 63) == 0) {
        asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=&v"(prior) : "v"(addr), "v"(1) : "memory");
    }
    return __builtin_amdgcn_readfirstlane(prior);
}

__device__ __forceinline__ uint4 pack_tr(i16x4 a, i16x4 b) {
    const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
    return uint4{x.x, x.y, y.x, y.y};
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_prefill_tile(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
    int num_seqs, int H, int h, int B, int top_k, int max_tiles, float c2, const int *__restrict__ v_exp,
    uint16_t *__restrict__ out, float *__restrict__ lse, int spin_limit, unsigned *__restrict__ wait_flag,
    int tiles_below) {
    using R = Ring<D>;
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    constexpr int CPR = D / 8;   // data slots per row
    constexpr float kLazy = 8.0f;   // log2 headroom before the reference max moves
    constexpr float kPScale = 7.0f; // weights are taken as 2^7 p (<= 2^15, fp16 normal down to 2^-21 p)
    __shared__ __attribute__((aligned(16))) char ring[kStages * R::STAGE];
    __shared__ unsigned long long masks[kWin];
    __shared__ unsigned long long list_m[kWin];
    __shared__ int list_u[kWin];
    __shared__ int list_n[kWin];
    __shared__ int wave_cnt[4];
    __shared__ int ready[kStages];
    __shared__ int done[kStages];

    const int G = H / h;
    const int Qt = 16 / G;                    // queries per row tile (one tile per wave)
    const int Tq = NW * Qt;                   // queries per workgroup (<= 64)
    const int bid = blockIdx.x;
    const int g = bid % h;
    const int rest = bid / h;
    const int s = rest % num_seqs;
    const int tile = max_tiles - 1 - rest / num_seqs;   // latest (heaviest) tiles first
    const int q_begin = cu_q[s], len_q = cu_q[s + 1] - q_begin;
    const size_t k_begin = (size_t)cu_k[s];
    const int len_k = cu_k[s + 1] - cu_k[s];
    const int r0 = tile * Tq;
    if (r0 >= len_q) return;
    const int shift = len_k - len_q;
    if (shift + r0 >= tiles_below) return;   // the block-centric schedule's rows
    const int tq_valid = min(Tq, len_q - r0);
    const int p_last = shift + r0 + tq_valid - 1;
    const int e_tile = p_last / B + 1;
    const int nsub = B / 64;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar control flow below
    const int l16 = lane & 15, q4 = lane >> 4;

    // This lane's row (query qi of the wave's tile, head `head` of the group).
    const int qi = l16 / G, head = l16 % G;
    const int qidx = wave * Qt + qi;
    const bool row_ok = (l16 < Qt * G) && (qidx < tq_valid);
    const int prow = row_ok ? shift + r0 + qidx : -1;
    const int p_first = shift + r0 + wave * Qt;   // smallest position of the wave's queries
    const int p_wave_last = shift + r0 + min(wave * Qt + Qt, tq_valid) - 1;
    bf16x8 qop[KS];
    {
        const uint16_t *src = q + ((size_t)(q_begin + r0 + qidx) * H + g * G + head) * D + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = as_bf16x8(load16_if(src + 32 * ks, row_ok, q));
    }
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;   // reference max (log2 units) the exponentials are taken against
    float l = 0.0f;
    const unsigned long long tile_bits = ((1ull << Qt) - 1ull) << (wave * Qt);

    const uint32_t ring0 = lds_addr(ring);
    const uint32_t list_u0 = lds_addr(list_u), list_m0 = lds_addr(list_m), list_n0 = lds_addr(list_n);
    const uint32_t ready0 = lds_addr(ready), done0 = lds_addr(done);
    // Per-lane read offsets inside a stage.
    const uint32_t k_rd = (uint32_t)(l16 * R::K_LANE + q4 * 16);
    const uint32_t v_rd = (uint32_t)(R::KBYTES + (4 * q4 + (l16 >> 2)) * R::V_LANE + 8 * (l16 & 3));

    // Direct loads of one 64-token sub-block into a ring stage, all issued by
    // one wave (lane i of a load instruction writes 16 bytes at M0 + 16 i).
    // The loads go through a buffer resource that ends at the group's row of
    // the sequence's last token; rows past the end repeat that token (finite
    // data, masked later), and pad slots of the padded layout, given an
    // out-of-range offset, move no data at all.
    auto issue_all = [&](int t0_in, int stage_in) {
        const int t0 = __builtin_amdgcn_readfirstlane(t0_in);
        const int stage = __builtin_amdgcn_readfirstlane(stage_in);
        const int hd2 = h * D * 2;
        const size_t row0 = ((k_begin + t0) * h + g) * D;
        const int nrec = (len_k - 1 - t0) * hd2 + 2 * D;   // through the last token's row of group g
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void *)(k + row0), 0, nrec, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void *)(v + row0), 0, nrec, kRsrcWord3);
        char *base = ring + stage * R::STAGE;
        // recomputed per call (kept out of registers across the loop)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if constexpr (R::GROUPED) {
            // instruction n: rows 4n .. 4n + 3, lane -> row 4n + ln/16, chunk ln%16
            if (t0 + 63 < len_k) {
                int off = (ln >> 4) * hd2 + (ln & 15) * 16;
#pragma unroll
                for (int n = 0; n < 16; ++n) {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(base + n * R::GROUP), 16, off, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(base + R::KBYTES + n * R::GROUP), 16, off,
                                                             0, 0, 0);
                    off += 4 * hd2;
                }
            } else {
                // the sequence ends inside the sub-block: later rows repeat its last token
                const int lim = len_k - 1 - t0;
#pragma unroll
                for (int n = 0; n < 16; ++n) {
                    const int off = min(4 * n + (ln >> 4), lim) * hd2 + (ln & 15) * 16;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(base + n * R::GROUP), 16, off, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(base + R::KBYTES + n * R::GROUP), 16, off,
                                                             0, 0, 0);
                }
            }
        } else {
            const int lim = min(63, len_k - 1 - t0);
            {
                int row = ln / R::KSLOT_ROW, c16 = ln % R::KSLOT_ROW;
#pragma unroll
                for (int i = 0; i < R::KINSTR; ++i) {
                    const int off = c16 < CPR ? min(row, lim) * hd2 + c16 * 16 : 0x7fffffff;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(base + i * 1024), 16, off, 0, 0, 0);
                    row += 64 / R::KSLOT_ROW;
                    c16 += 64 % R::KSLOT_ROW;
                    if (c16 >= R::KSLOT_ROW) {
                        c16 -= R::KSLOT_ROW;
                        ++row;
                    }
                }
            }
            {
                int row = ln / R::VSLOT_ROW, c16 = ln % R::VSLOT_ROW;
#pragma unroll
                for (int i = 0; i < R::VINSTR; ++i) {
                    const int off = c16 < CPR ? min(row, lim) * hd2 + c16 * 16 : 0x7fffffff;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(base + R::KBYTES + i * 1024), 16, off, 0, 0,
                                                             0);
                    row += 64 / R::VSLOT_ROW;
                    c16 += 64 % R::VSLOT_ROW;
                    if (c16 >= R::VSLOT_ROW) {
                        c16 -= R::VSLOT_ROW;
                        ++row;
                    }
                }
            }
        }
    };

    // One item for this wave's row tile: the sub-block at t0 staged at sbase;
    // mk = which queries of the workgroup tile selected its block.
    auto attend = [&](uint32_t sbase, int t0, unsigned long long mk) {
        // S^T = K . Q^T for the four 16-token tiles of the sub-block
        f32x4 sacc[4];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            uint4 a[2 * KS];
            lds_k_pair<KS, R::K_TILE>(a, sbase + k_rd + tp * 2 * R::K_TILE);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                sacc[2 * tp + u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    sacc[2 * tp + u] = mfma16x16x32(as_bf16x8(a[u * KS + ks]), qop[ks], sacc[2 * tp + u]);
            }
        }
        // Online softmax in log2 units.  A row whose query did not select the
        // block gets bias +inf (all its weights 0); future tokens are masked
        // only on diagonal sub-blocks.
        const bool selected = prow >= 0 && ((mk >> qidx) & 1ull);
        if (t0 + 63 > p_first) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (t0 + R::token(tt, q4, i) > prow) sacc[tt][i] = -INFINITY;
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sacc[tt][i]);
        mloc = max_xor32(max_xor16(mloc)) * c2;
        // The reference max moves only when the block max exceeds it by more
        // than kLazy, so weights stay <= 2^kLazy and O is rarely rescaled.
        const bool move = selected && mloc > m_ref + kLazy;
        if (__ballot(move) != 0ull) {
            const float alpha = move ? fast_exp2(m_ref - mloc) : 1.0f;   // 0 on a row's first block
            m_ref = move ? mloc : m_ref;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        }
        const float nbias = (selected && m_ref > -INFINITY) ? kPScale - m_ref : -INFINITY;
        float lsum = 0.0f;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = fast_exp2(fmaf(sacc[tt][i], c2, nbias));
                sacc[tt][i] = e;
                lsum += e;
            }
        l += lsum;
        // O^T += V^T . P^T in fp16 (V is the scaled fp16 copy)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            // slots 8*q4 + i <- tile 2*s2 value i, slots 8*q4 + 4 + i <- tile 2*s2+1 value i
            const f16x8 p16 = as_f16x8(uint4{pack_f16x2(sacc[2 * s2][0], sacc[2 * s2][1]),
                                             pack_f16x2(sacc[2 * s2][2], sacc[2 * s2][3]),
                                             pack_f16x2(sacc[2 * s2 + 1][0], sacc[2 * s2 + 1][1]),
                                             pack_f16x2(sacc[2 * s2 + 1][2], sacc[2 * s2 + 1][3])});
#pragma unroll
            for (int dq = 0; dq < DT / 4; ++dq) {
                i16x4 va[4], vb[4];
                lds_v_half<4, R::V_ODD>(va, vb, sbase + v_rd + s2 * R::V_S2 + dq * 128);
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    o[4 * dq + x] = mfma16x16x32_f16(as_f16x8(pack_tr(va[x], vb[x])), p16, o[4 * dq + x]);
            }
        }
    };

    for (int w0 = 0; w0 < e_tile; w0 += kWin) {
        if (tid < kWin) masks[tid] = 0ull;
        if (tid < kStages) {
            ready[tid] = 0;
            done[tid] = 0;
        }
        __syncthreads();
        // Which queries of the tile selected which block of this window.
        const int32_t *tile_ids = ids + ((size_t)(q_begin + r0) * h + g) * top_k;
        for (int e = tid; e < tq_valid * top_k; e += 64 * NW) {
            const int eq = e / top_k, a = e % top_k;
            const int j = tile_ids[(size_t)eq * h * top_k + a];
            const int pq = shift + r0 + eq;
            if (j >= w0 && j < w0 + kWin && j >= 0 && j <= pq / B) atomicOr(&masks[j - w0], 1ull << eq);
        }
        __syncthreads();
        // Compact the blocks somebody selected, ascending, with the number of
        // waves whose row tile holds a selecting query.
        const unsigned long long mv = tid < kWin ? masks[tid] : 0ull;
        const unsigned long long bal = __ballot(mv != 0ull);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (lane == 0 && wave < 4) wave_cnt[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int base = 0, count = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            base += (w < wave) ? wave_cnt[w] : 0;   // waves >= 4 hold no entries
            count += wave_cnt[w];
        }
        if (mv != 0ull) {
            int nact = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) nact += ((mv >> (w * Qt)) & ((1ull << Qt) - 1ull)) != 0ull;
            list_u[base + before] = w0 + tid;
            list_m[base + before] = mv;
            list_n[base + before] = nact;
        }
        __syncthreads();

        // Items are the 64-token sub-blocks of the listed blocks; a trailing
        // sub-block that starts after the tile's last query is dropped.
        count = __builtin_amdgcn_readfirstlane(count);   // the same in every lane
        int nitems = count * nsub;
        if (nsub > 1 && count > 0 && (int)lds_u32(list_u0 + 4 * (count - 1)) * B + 64 > p_last) --nitems;
        nitems = __builtin_amdgcn_readfirstlane(nitems);
        auto t0_of = [&](int it) {
            return (int)lds_u32(list_u0 + 4 * (it / nsub)) * B + (it % nsub) * 64;
        };
        // Ring protocol.  ready[s] holds the stamp (item + 1) of the sub-block
        // stage s holds once its loads have landed.  Only the waves whose row
        // tile is active read an item; done[s] counts them, and the last one
        // (the count reaching the item's active-wave count) clears the counter
        // and refills the stage with the item kStages ahead.  Its loads are
        // published after its next item, or before it would block, so no wave
        // ever waits while holding an unpublished stage.  Waves skip items
        // they have no work in and run ahead until the ring holds them back.
        // initial fill of every stage, spread over the waves
        if (wave < kStages && wave < nitems) {
            for (int x = wave; x < kStages && x < nitems; x += NW) issue_all(t0_of(x), x);
            wait_vm<0>();
            for (int x = wave; x < kStages && x < nitems; x += NW) lds_store_u32(ready0 + 4 * x, x + 1);
        }
        int pend_stage = -1, pend_stamp = 0;
        auto publish = [&]() {
            if (pend_stage >= 0) {
                wait_vm<0>();
                lds_store_u32(ready0 + 4 * pend_stage, pend_stamp);
                pend_stage = -1;
            }
        };

        for (int e0 = 0; e0 < count; e0 += 64) {
            // 64 list entries at a time, one per lane; an item's entry is then
            // read from its lane (no LDS round trip per item)
            const bool in_list = e0 + lane < count;
            const unsigned long long m_e = in_list ? lds_u64(list_m0 + 8 * (e0 + lane)) : 0ull;
            const int n_e = in_list ? (int)lds_u32(list_n0 + 4 * (e0 + lane)) : 0;
            const int u_e = in_list ? (int)lds_u32(list_u0 + 4 * (e0 + lane)) : 0;
            unsigned long long act = __ballot((m_e & tile_bits) != 0ull);
            while (act != 0ull) {
                const int li = __builtin_ctzll(act);
                const int ei = e0 + li;
                act &= act - 1ull;
                const unsigned long long mk =
                    ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(m_e >> 32), li) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m_e, li);
                const int nact = __builtin_amdgcn_readlane(n_e, li);
                const int blk = __builtin_amdgcn_readlane(u_e, li);
                for (int sub = 0; sub < nsub; ++sub) {
                    const int it = ei * nsub + sub;
                    if (it >= nitems) break;
                    const int stage = it % kStages;
                    const int t0 = blk * B + sub * 64;
                    if (__builtin_amdgcn_readfirstlane(lds_u32(ready0 + 4 * stage)) != it + 1) {
                        publish();
                        // bounded (spin_limit polls): a wait that never ends
                        // would hang the device, so one that reaches the bound
                        // is counted in the wait word and the item is attended
                        // as the stage holds it (the output is then invalid,
                        // and the caller can see it)
                        bool ready_now = false;
                        for (int spin = 0; spin < spin_limit; ++spin) {
                            if (__builtin_amdgcn_readfirstlane(lds_u32(ready0 + 4 * stage)) == it + 1) {
                                ready_now = true;
                                break;
                            }
                            __builtin_amdgcn_s_sleep(1);
                        }
                        if (!ready_now)
                            ready_now = __builtin_amdgcn_readfirstlane(lds_u32(ready0 + 4 * stage)) == it + 1;
                        if (!ready_now && lane == 0) atomicAdd(wait_flag, 1u);
                    }
                    const uint32_t sbase = ring0 + stage * R::STAGE;
                    if (t0 <= p_wave_last) {
                        attend(sbase, t0, mk);
                    }
                    publish();
                    const int prior = lds_add_rtn_u32(done0 + 4 * stage);
                    if (prior == nact - 1) {
                        lds_store_u32(done0 + 4 * stage, 0);
                        if (it + kStages < nitems) {
                            issue_all(t0_of(it + kStages), stage);
                            pend_stage = stage;
                            pend_stamp = it + kStages + 1;
                        }
                    }
                }
            }
        }
        publish();
        wait_vm<0>();
        __syncthreads();
    }

    // Epilogue: normalise and write this wave's rows.
    const float lt = sum_xor32(sum_xor16(l));
    if (prow < 0) return;
    const int row = q_begin + r0 + qidx;
    const float inv = lt > 0.f ? __builtin_ldexpf(1.0f / lt, v_exp[s * h + g]) : 0.0f;
    uint16_t *dst = out + ((size_t)row * H + g * G + head) * D + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        uint2 w;
        w.x = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
        w.y = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
        *reinterpret_cast<uint2 *>(dst + dt * 16) = w;
    }
    if (lse != nullptr && q4 == 0)
        lse[(size_t)row * H + g * G + head] =
            lt > 0.f ? (m_ref - kPScale + log2f(lt)) * 0.69314718055994531f : -INFINITY;
}

// fp16 copy of V for the P.V products.  The values of one (sequence, KV
// head) are scaled by one power of two 2^-e, chosen from that head's max |V|
// in that sequence so that its largest lands in [2^14, 2^15): bf16 values
// within 2^25 of the largest convert exactly, and smaller ones lose only bits
// below 2^-10 of the largest.  A tile's output is multiplied back by the 2^e
// of its own (sequence, group), so a head whose values sit far below those of
// another keeps its full relative precision.
//
// Three passes.  The max and conversion passes run on the grid (sequence,
// token chunk): chunk c of sequence s covers its tokens [c*T, c*T + T) with
// all their heads, a contiguous run of V of about 64 KB; chunks past a
// sequence's end exit at once.  Thread i of a workgroup takes the run's
// 16-byte pieces i, i + 256, ...; the head of a piece is tracked by adding
// 256 mod (h*D/8) to its offset within the token row, so no piece costs a
// division.  Between them one workgroup per (sequence, head) turns the chunk
// maxima into the exponent.
constexpr int kCvtChunks = 8192;   // at most this many chunks per sequence

struct CvtGrid {
    int chunks, tokens;   // chunks per sequence, tokens per chunk
};
CvtGrid cvt_grid(const Shape &s) {
    const int mk = std::max(s.max_k, 1);
    const int rw = std::max(s.h * (s.d / 8), 1);   // pieces per token row
    int tokens = std::max(1, 4096 / rw);
    tokens = std::max(tokens, (mk + kCvtChunks - 1) / kCvtChunks);
    return CvtGrid{(mk + tokens - 1) / tokens, tokens};
}

__device__ __forceinline__ uint32_t absmax_bf16x8(uint4 x) {
    // |bf16| bit patterns order like the values (NaN above infinity)
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
    return m;
}

// Max |v| per head over one token chunk of one sequence, as a bf16 bit
// pattern without the sign, into part[(s * chunks + c) * h + g] (h <= 1024).
template <int D>
__global__ __launch_bounds__(256) void v_absmax_bits(const uint4 *__restrict__ v, const int32_t *__restrict__ cu_k,
                                                     int h, int tokens, int chunks, int kcap,
                                                     uint32_t *__restrict__ part) {
    constexpr int CPR = D / 8, SH = D == 128 ? 4 : 3;   // pieces per (token, head), log2
    __shared__ uint32_t hm[1024];
    const int s = (int)blockIdx.x, c = (int)blockIdx.y;
    const int t0 = cu_k[s] + c * tokens;
    const int t1 = min(cu_k[s] + min(cu_k[s + 1] - cu_k[s], kcap), t0 + tokens);
    if (t0 >= t1) return;
    const int rw = h * CPR, step = 256 % rw;
    for (int g = threadIdx.x; g < h; g += 256) hm[g] = 0u;
    __syncthreads();
    const uint4 *run = v + (size_t)t0 * rw;
    const int n = (t1 - t0) * rw;
    int r = threadIdx.x % rw, cur = r >> SH;
    uint32_t m = 0;
    for (int e0 = threadIdx.x; e0 < n; e0 += 4 * 256) {   // four loads in flight per thread
        uint4 x[4];
        int gu[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            x[u] = run[min(e0 + 256 * u, n - 1)];
            gu[u] = r >> SH;
            r += step;
            if (r >= rw) r -= rw;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (e0 + 256 * u >= n) break;
            if (gu[u] != cur) {
                atomicMax(&hm[cur], m);
                cur = gu[u];
                m = 0;
            }
            m = max(m, absmax_bf16x8(x[u]));
        }
    }
    if (threadIdx.x < n) atomicMax(&hm[cur], m);
    __syncthreads();
    for (int g = threadIdx.x; g < h; g += 256) part[((size_t)s * chunks + c) * h + g] = hm[g];
}

// One workgroup per (sequence, head): e[s * h + g] from the maxima of the
// chunks that hold tokens.  max |v| < 2^(E - 126) for bf16 exponent field E:
// scaling by 2^-(E - 141) puts it in [2^14, 2^15) whatever its magnitude
// (2^-e stays a normal float).  Infinities and NaN keep e = 0 and pass
// through as such.  Workgroup 0 also clears the wait word.
__global__ __launch_bounds__(256) void v_scale_exp(const int32_t *__restrict__ cu_k, int h, int tokens, int chunks,
                                                   int kcap, const uint32_t *__restrict__ part,
                                                   int *__restrict__ v_exp, unsigned *__restrict__ wait_flag) {
    const int sg = (int)blockIdx.x, s = sg / h, g = sg % h;
    if (sg == 0 && threadIdx.x == 0) *wait_flag = 0u;   // the attention kernel that follows counts its given-up waits here
    const int nc = (min(cu_k[s + 1] - cu_k[s], kcap) + tokens - 1) / tokens;
    uint32_t m = 0;
#pragma unroll 4
    for (int c = threadIdx.x; c < nc; c += 256) m = max(m, part[((size_t)s * chunks + c) * h + g]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = max(max(red[0], red[1]), max(red[2], red[3]));
        v_exp[sg] = (m >= 0x7f80u) ? 0 : max(-126, (int)(m >> 7) - 141);
    }
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float mul) {
    return pack_f16x2(__uint_as_float(w << 16) * mul, __uint_as_float(w & 0xffff0000u) * mul);
}

// The fp16 copy of one token chunk of one sequence, each head times its 2^-e.
// Only the first kcap tokens of each sequence are converted (and measured by
// the max pass): when the call's rows are split between the schedules, the
// query tiles stage no key block past the one holding the split position plus
// one tile.
template <int D>
__global__ __launch_bounds__(256) void v_to_f16(const uint4 *__restrict__ v, const int32_t *__restrict__ cu_k, int h,
                                                int tokens, int kcap, const int *__restrict__ v_exp,
                                                uint4 *__restrict__ v16) {
    constexpr int CPR = D / 8, SH = D == 128 ? 4 : 3;
    const int s = (int)blockIdx.x, c = (int)blockIdx.y;
    const int t0 = cu_k[s] + c * tokens;
    const int t1 = min(cu_k[s] + min(cu_k[s + 1] - cu_k[s], kcap), t0 + tokens);
    if (t0 >= t1) return;
    __shared__ float muls[1024];
    const int rw = h * CPR, step = 256 % rw;
    for (int g = threadIdx.x; g < h; g += 256) muls[g] = __builtin_ldexpf(1.0f, -v_exp[(size_t)s * h + g]);
    __syncthreads();
    const size_t off = (size_t)t0 * rw;
    const int n = (t1 - t0) * rw;
    int r = threadIdx.x % rw;
    for (int e0 = threadIdx.x; e0 < n; e0 += 4 * 256) {   // four loads in flight per thread
        uint4 x[4];
        float mu[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            x[u] = v[off + min(e0 + 256 * u, n - 1)];
            mu[u] = muls[r >> SH];
            r += step;
            if (r >= rw) r -= rw;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (e0 + 256 * u < n)
                v16[off + e0 + 256 * u] = uint4{bf16x2_to_f16x2(x[u].x, mu[u]), bf16x2_to_f16x2(x[u].y, mu[u]),
                                                bf16x2_to_f16x2(x[u].z, mu[u]), bf16x2_to_f16x2(x[u].w, mu[u])};
    }
}

// Workspace: the fp16 copy of V, the max pass's chunk maxima, the exponents
// per (sequence, head), then one 256-byte slot whose word 0 is the wait word
// (the count of ring waits that reached their bound in the last call).
struct PrefillWs {
    size_t v16_off, part_off, exp_off, flag_off, bytes;
};
PrefillWs prefill_ws(const Shape &s) {
    PrefillWs w;
    const size_t vb = (size_t)s.total_k * s.h * s.d * 2;
    const size_t sh = (size_t)s.num_seqs * s.h;
    w.v16_off = 0;
    w.part_off = (vb + 255) / 256 * 256;
    w.exp_off = w.part_off + ((size_t)s.num_seqs * cvt_grid(s).chunks * s.h * sizeof(uint32_t) + 255) / 256 * 256;
    w.flag_off = w.exp_off + (sh * sizeof(int) + 255) / 256 * 256;
    w.bytes = w.flag_off + 256;
    return w;
}

// Polls per ring wait: kSpinLimit, or MSA_DEBUG_SPIN_LIMIT when that is set
// to a non-negative integer (a debugging aid: a tiny bound makes the waits
// give up, so the wait word can be seen to work; every kernel still ends).
int spin_limit_from_env() {
    const char *e = getenv("MSA_DEBUG_SPIN_LIMIT");
    if (e == nullptr || *e == 0) return kSpinLimit;
    char *end = nullptr;
    const long v = strtol(e, &end, 10);
    if (*end != 0 || v < 0) return kSpinLimit;
    return v > kSpinLimit ? kSpinLimit : (int)v;
}

template <int D, int NW>
hipError_t launch(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v16, const int *v_exp,
                  const int32_t *ids, float scale, uint16_t *out, float *lse, unsigned *wait_flag, hipStream_t st) {
    const int G = s.H / s.h;
    const int Tq = NW * (16 / G);
    // a tile starting at row r0 of a sequence sits at position >= r0, so with
    // rows split between the schedules no tile at or past tiles_below runs
    const int rows_max = s.tiles_below < s.max_q ? std::max(s.tiles_below, 0) : s.max_q;
    const int max_tiles = (rows_max + Tq - 1) / Tq;
    if (max_tiles == 0) return hipSuccess;
    const long grid = (long)max_tiles * s.num_seqs * s.h;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_prefill_tile<D, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, st, q, k, v16, ids, s.cu_q,
                       s.cu_k, s.num_seqs, s.H, s.h, s.B, s.top_k, max_tiles, scale * kLog2e, v_exp, out, lse,
                       spin_limit_from_env(), wait_flag, s.tiles_below);
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(const Shape &s) { return prefill_ws(s).bytes; }
size_t prefill_wait_word_offset(const Shape &s) { return prefill_ws(s).flag_off; }

int prefill_tile_queries(const Shape &s) {
    // One 16-row tile per wave, as many waves as keep the tile within 64
    // queries (one mask bit per query), at most 16 (four per SIMD).
    const int qt = 16 / (s.H / s.h);
    const int cap = 64 / qt;
    const int nw = cap >= 16 ? 16 : (cap >= 8 ? 8 : 4);
    return nw * qt;
}

hipError_t launch_attn_prefill(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *ids, float scale, uint16_t *out, float *lse, void *ws,
                               hipStream_t st) {
    const int G = s.H / s.h;
    if (G < 1 || G > 16) return hipErrorInvalidValue;
    if (s.d != 64 && s.d != 128) return hipErrorInvalidValue;
    if (s.total_k < 1) return hipErrorInvalidValue;
    // fp16 copy of V (two small passes over V)
    const PrefillWs w = prefill_ws(s);
    char *wsb = static_cast<char *>(ws);
    uint16_t *v16 = reinterpret_cast<uint16_t *>(wsb + w.v16_off);
    uint32_t *part = reinterpret_cast<uint32_t *>(wsb + w.part_off);
    int *v_exp = reinterpret_cast<int *>(wsb + w.exp_off);
    unsigned *wait_flag = reinterpret_cast<unsigned *>(wsb + w.flag_off);
    const CvtGrid cg = cvt_grid(s);
    if (s.h > 1024 || (long)s.num_seqs * s.h > 0x7fffffffL) return hipErrorInvalidValue;
    // keys the query tiles stage: whole key blocks up to the block holding the
    // last position they attend (below tiles_below plus one tile).  Masked
    // keys of a staged block still enter the P.V products with weight 0, so
    // they must hold converted (finite) values too.
    const long kc = ((long)s.tiles_below + prefill_tile_queries(s) + s.B - 1) / s.B * s.B;
    const int kcap = (int)std::min<long>(std::max<long>(kc, 0), 0x7fffffffL);
    const dim3 cvt((unsigned)s.num_seqs, (unsigned)cg.chunks);
    const uint4 *v4 = reinterpret_cast<const uint4 *>(v);
    if (s.d == 64)
        hipLaunchKernelGGL(v_absmax_bits<64>, cvt, dim3(256), 0, st, v4, s.cu_k, s.h, cg.tokens, cg.chunks, kcap,
                           part);
    else
        hipLaunchKernelGGL(v_absmax_bits<128>, cvt, dim3(256), 0, st, v4, s.cu_k, s.h, cg.tokens, cg.chunks, kcap,
                           part);
    hipLaunchKernelGGL(v_scale_exp, dim3((unsigned)(s.num_seqs * s.h)), dim3(256), 0, st, s.cu_k, s.h, cg.tokens,
                       cg.chunks, kcap, part, v_exp, wait_flag);
    if (s.d == 64)
        hipLaunchKernelGGL(v_to_f16<64>, cvt, dim3(256), 0, st, v4, s.cu_k, s.h, cg.tokens, kcap, v_exp,
                           reinterpret_cast<uint4 *>(v16));
    else
        hipLaunchKernelGGL(v_to_f16<128>, cvt, dim3(256), 0, st, v4, s.cu_k, s.h, cg.tokens, kcap, v_exp,
                           reinterpret_cast<uint4 *>(v16));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nw = prefill_tile_queries(s) / (16 / G);
    if (s.d == 64) {
        if (nw == 16) return launch<64, 16>(s, q, k, v16, v_exp, ids, scale, out, lse, wait_flag, st);
        if (nw == 8) return launch<64, 8>(s, q, k, v16, v_exp, ids, scale, out, lse, wait_flag, st);
        return launch<64, 4>(s, q, k, v16, v_exp, ids, scale, out, lse, wait_flag, st);
    }
    if (nw == 16) return launch<128, 16>(s, q, k, v16, v_exp, ids, scale, out, lse, wait_flag, st);
    if (nw == 8) return launch<128, 8>(s, q, k, v16, v_exp, ids, scale, out, lse, wait_flag, st);
    return launch<128, 4>(s, q, k, v16, v_exp, ids, scale, out, lse, wait_flag, st);
}

}  // namespace msa
