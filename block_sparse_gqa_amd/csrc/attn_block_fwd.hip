// Sparse branch, prefill, on the block-centric ("KV-outer, gather-Q")
// schedule: the same exact softmax attention over the selected blocks as the
// query-tile kernel ("MiniMax Goes Sparse", section 1, step 2; "MiniMax M3
// MSA vs Step 3.7 Flash MFA", section "MSA: a minimal sparse attention",
// second layer), computed key block by key block.  The pages name this
// operator flow ("深度解析M3多模态模型与Token Plan", section 二.2, on
// hardware-friendly operators) and their block-sparse prior art builds it on
// an inverted index ("MoBA / FlashMoBA" page, section 3.1).
//
// Pass 1 (block_lists.hip): the ids become, per (group, key block), the list
// of (query row, slot) pairs that selected it.
//
// Pass 2 (fwd_block): one workgroup per (group, block).  The block's K (bf16)
// and V (fp16, scaled by a power of two 2^-e chosen from the block's largest
// |v| so that every value and every partial output fits fp16) sit in LDS.
// Each wave takes 32-row tiles of the list (32/G selecting queries x G
// heads, two 16-row MFMA tiles sharing every K and V operand read), gathers
// their Q rows straight into the MFMA B operands (one tile ahead) and
// computes
//     S^T = K . Q^T         v_mfma_f32_16x16x32_bf16, A = K rows from LDS;
//     P   = 2^(S c2 - m)    m = the row's max over the block's visible tokens;
//     O^T = V^T . P^T       v_mfma_f32_16x16x32_f16, A = V^T (transposing LDS
//                           read), B = P^T straight from the S^T accumulators.
// Every (row, slot, head) gets a partial: O / l as fp16 (times 2^-e) and the
// pair (m + log2 l, e), the partial rows staged through a per-wave LDS tile
// so that stores cover whole rows.  No workgroup barrier after the staging:
// each wave walks its own tiles, with the list entries two tiles ahead and
// the Q rows one tile ahead in registers.
//
// Pass 3 (fwd_merge): per (row, head), the partials of the row's valid slots
// merge by log-sum-exp into O (bf16) and LSE (natural log) in one pass, in a
// fixed order; one wave takes the G heads of a (row, group).
#include <algorithm>
#include <cmath>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kStride = 288;   // LDS row stride of K and V in bytes (32 mod 256: conflict free)

// Waves per workgroup: B = 128 keeps two waves per SIMD with one workgroup
// per CU (its K/V tiles take 72 KB of LDS).
template <int B>
constexpr int fwd_waves() { return B == 128 ? 8 : 4; }

template <int D, int B>
__global__ __launch_bounds__(64 * fwd_waves<B>()) void fwd_block(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, const int32_t *__restrict__ blk_off,
    const int32_t *__restrict__ off, const int32_t *__restrict__ entries, int num_seqs, int H, int h, int nb_max,
    int top_k, FastDiv kdiv, int row0, float c2, uint16_t *__restrict__ part_o, float2 *__restrict__ part_w) {
    constexpr int KS = D / 32;            // 32-wide k steps over d
    constexpr int DT = D / 16;            // 16-wide d tiles
    constexpr int TT = B / 16;            // 16-token tiles of the block
    constexpr int NW = fwd_waves<B>();
    constexpr int NT = 64 * NW;
    constexpr int CH = B * (D / 8) / NT;  // 16-byte chunks per thread per tensor
    constexpr int OSTR = 2 * D + 16;      // LDS row stride of a wave's output tile
    __shared__ __attribute__((aligned(16))) char kt[B * kStride];
    __shared__ __attribute__((aligned(16))) char vt[B * kStride];
    __shared__ __attribute__((aligned(16))) char ot[NW][16 * OSTR];
    __shared__ uint32_t vmax_bits;

    const int gb = blockIdx.x, g = blockIdx.y;
    if (gb >= blk_off[num_seqs]) return;
    const int s = seq_of_row(blk_off, num_seqs, gb);
    const int j = gb - blk_off[s];
    const long key = (long)g * nb_max + gb;
    const int e0 = off[key], nq = off[key + 1] - e0;
    if (nq == 0) return;
    const int k_begin = cu_k[s], len_k = cu_k[s + 1] - k_begin;
    const int q_begin = cu_q[s], shift = len_k - (cu_q[s + 1] - q_begin);
    const int G = H / h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop over the tiles
    const int l16 = lane & 15, q4 = lane >> 4;
    const int t_valid = min(B, len_k - j * B);   // tokens of the block inside the sequence

    // Stage K (bf16) and V (fp16 x 2^-e); rows past the sequence end are zero.
    if (tid == 0) vmax_bits = 0u;
    uint4 kr[CH], vr[CH];
    uint32_t vmax = 0u;
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int c = x * NT + tid, t = c / (D / 8), c8 = c % (D / 8);
        const size_t src = ((size_t)(k_begin + j * B + min(t, t_valid - 1)) * h + g) * D + c8 * 8;
        kr[x] = load16(k + src);
        vr[x] = load16(v + src);
        const uint32_t m = t < t_valid ? 0xffffffffu : 0u;   // per-word mask
        kr[x] = uint4{kr[x].x & m, kr[x].y & m, kr[x].z & m, kr[x].w & m};
        vr[x] = uint4{vr[x].x & m, vr[x].y & m, vr[x].z & m, vr[x].w & m};
        const uint32_t w[4] = {vr[x].x, vr[x].y, vr[x].z, vr[x].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) vmax = max(vmax, max((w[i] & 0x7fffu) << 16, w[i] & 0x7fff0000u));   // |v| bits
    }
    __syncthreads();
    atomicMax(&vmax_bits, vmax);
    __syncthreads();
    // 2^-e brings the largest |v| into [2^14, 2^15): v and O / l fit fp16.
    const uint32_t amax = vmax_bits;
    const int e = amax == 0u ? 0 : min(max((int)(amax >> 23) - 127 - 14, -100), 113);
    const float vscale = __uint_as_float((uint32_t)(127 - e) << 23);
#pragma unroll
    for (int x = 0; x < CH; ++x) {
        const int c = x * NT + tid, t = c / (D / 8), c8 = c % (D / 8);
        *reinterpret_cast<uint4 *>(kt + t * kStride + 16 * c8) = kr[x];
        const uint32_t w[4] = {vr[x].x, vr[x].y, vr[x].z, vr[x].w};
        uint32_t f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f[i] = pack_f16x2(__uint_as_float(w[i] << 16) * vscale, __uint_as_float(w[i] & 0xffff0000u) * vscale);
        *reinterpret_cast<uint4 *>(vt + t * kStride + 16 * c8) = uint4{f[0], f[1], f[2], f[3]};
    }
    __syncthreads();

    // Tiles of 32 rows (32/G selecting queries x G heads) as two 16-row MFMA
    // tiles mt = 0, 1 that share every K and V operand read.  This lane's row
    // in tile mt is r = 16 mt + l16: query r / G of the tile, head g*G + r % G.
    constexpr int MT = 2;
    const int qpt = (16 * MT) / G, rows_used = qpt * G;
    int qi[MT], hd[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        qi[mt] = (16 * mt + l16) / G;
        hd[mt] = (16 * mt + l16) % G;
    }
    const int ntiles = (nq + qpt - 1) / qpt;
    auto entry = [&](int t, int mt) {   // (row - row0) * top_k + slot, or -1
        const int x = t * qpt + qi[mt];
        return (t < ntiles && 16 * mt + l16 < rows_used && x < nq) ? entries[e0 + x] : -1;
    };
    auto load_q = [&](uint4 (&qo)[KS], int ent, int hh) {   // row 0 stands in for unused lanes
        const size_t base = ((size_t)(ent >= 0 ? row0 + (int)fastdiv((uint32_t)ent, kdiv) : 0) * H + g * G + hh) * D + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qo[ks] = load16(q + base + 32 * ks);
    };

    int t = wave;
    int ent_cur[MT], ent_next[MT];
    uint4 qc[MT][KS], qn[MT][KS] = {};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        ent_cur[mt] = entry(t, mt);
        ent_next[mt] = entry(t + NW, mt);
        load_q(qc[mt], ent_cur[mt], hd[mt]);
    }
    for (; t < ntiles; t += NW) {
        int ent_after[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ent_after[mt] = entry(t + 2 * NW, mt);
        if (t + NW < ntiles) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) load_q(qn[mt], ent_next[mt], hd[mt]);
        }

        f32x4 sa[MT][TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sa[mt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = as_bf16x8(lds_row8<kStride>(kt, 16 * tt + l16, 4 * ks + q4));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) sa[mt][tt] = mfma16x16x32(a, as_bf16x8(qc[mt][ks]), sa[mt][tt]);
            }
        }
        // Visible tokens of this lane's rows: block token index <= lim.  The
        // causal compare is needed only where some row of the tile sees just
        // part of the block (its diagonal block); unused lanes count as
        // seeing all of it (their results are never stored).
        float mu[MT], lsum[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = ent_cur[mt] >= 0 ? row0 + (int)fastdiv((uint32_t)ent_cur[mt], kdiv) : -1;
            const int lim = row >= 0 ? shift + (row - q_begin) - j * B : B - 1;
            float mx = -INFINITY;
            if (__ballot(lim < B - 1) == 0) {
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = sa[mt][tt][i] * c2;
                        sa[mt][tt][i] = x;
                        mx = fmaxf(mx, x);
                    }
            } else {
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = 16 * tt + 4 * q4 + i <= lim ? sa[mt][tt][i] * c2 : -INFINITY;
                        sa[mt][tt][i] = x;
                        mx = fmaxf(mx, x);
                    }
            }
            mx = max_xor32(max_xor16(mx));
            mu[mt] = mx == -INFINITY ? 0.f : mx;
            float ls = 0.f;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = fast_exp2(sa[mt][tt][i] - mu[mt]);
                    sa[mt][tt][i] = pv;
                    ls += pv;
                }
            lsum[mt] = sum_xor32(sum_xor16(ls));
            // P / l, so that the product below is the normalised partial
            const float inv = lsum[mt] > 0.f ? 1.0f / lsum[mt] : 0.f;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sa[mt][tt][i] *= inv;
        }

        f32x4 oa[MT][DT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oa[mt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s32 = 0; s32 < B / 32; ++s32) {
            // B = P^T: k slot 8*q4 + i <- token 32*s32 + 4*q4 + i, slot 8*q4 + 4 + i <- token 32*s32 + 16 + 4*q4 + i
            f16x8 pb[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                pb[mt] = as_f16x8(uint4{pack_f16x2(sa[mt][2 * s32][0], sa[mt][2 * s32][1]),
                                        pack_f16x2(sa[mt][2 * s32][2], sa[mt][2 * s32][3]),
                                        pack_f16x2(sa[mt][2 * s32 + 1][0], sa[mt][2 * s32 + 1][1]),
                                        pack_f16x2(sa[mt][2 * s32 + 1][2], sa[mt][2 * s32 + 1][3])});
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f16x8 va = as_f16x8(lds_tr_rows<kStride>(vt, 32 * s32, dt));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) oa[mt][dt] = mfma16x16x32_f16(va, pb[mt], oa[mt][dt]);
            }
        }
        // O / l (fp16; P was already divided by l) goes through this wave's
        // LDS tile, 16 rows at a time, so that every store instruction writes
        // whole partial rows (16 lanes x 16 bytes per row for d = 128).
        char *my = ot[wave];
        constexpr int CPR = D / 8;      // 16-byte chunks per row
        constexpr int RPI = 64 / CPR;   // rows per store instruction
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<uint2 *>(my + l16 * OSTR + (16 * dt + 4 * q4) * 2) =
                    uint2{pack_f16x2(oa[mt][dt][0], oa[mt][dt][1]), pack_f16x2(oa[mt][dt][2], oa[mt][dt][3])};
            wave_lds_sync();
#pragma unroll
            for (int x = 0; x < 16 / RPI; ++x) {
                const int r = x * RPI + lane / CPR, c = lane % CPR;
                const int er = __shfl(ent_cur[mt], r, 64);   // the entry of tile row 16 mt + r (held by lane r)
                const uint4 val = *reinterpret_cast<const uint4 *>(my + r * OSTR + 16 * c);
                if (er >= 0)
                    store16_nt(part_o + ((size_t)er * H + g * G + (16 * mt + r) % G) * D + 8 * c, val);
            }
            wave_lds_sync();   // the tile's reads are done before the next rows are written
            if (ent_cur[mt] >= 0 && q4 == 0)
                part_w[(size_t)ent_cur[mt] * H + g * G + hd[mt]] = make_float2(mu[mt] + __log2f(lsum[mt]), (float)e);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            ent_cur[mt] = ent_next[mt];
            ent_next[mt] = ent_after[mt];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qc[mt][ks] = qn[mt][ks];
        }
    }
}

// O[row, head] and LSE from the partials of the row's valid slots, in one
// pass.  One wave per (row, group); lane = (head of the group, 16-byte chunk of
// a partial row), 64 / (D / 8) heads per pass, so every load instruction
// reads the contiguous partial rows of those heads for one slot.  Each lane
// walks all the row's slots in order, merging online (running max of the
// log2-sum-exp, the sums rescaled when it grows): every lane of a head holds
// the same max and denominator, so no cross-lane reduction is needed.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge(const uint16_t *__restrict__ part_o, const float2 *__restrict__ part_w,
                                                 const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q,
                                                 const int32_t *__restrict__ cu_k, int num_seqs, int row0,
                                                 long n_pairs, int H, int h, int B, int top_k, int blocks_from,
                                                 int split_tq, uint16_t *__restrict__ out, float *__restrict__ lse) {
    constexpr int CPR = D / 8;       // 16-byte chunks per partial row
    constexpr int HPP = 64 / CPR;    // heads per pass
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const long rg = (long)blockIdx.x * 4 + wave;
    if (rg >= n_pairs) return;
    const int lane = threadIdx.x & 63, c = lane % CPR, hs = lane / CPR;
    const int rr = (int)(rg / h), g = (int)(rg % h), G = H / h;   // rr: row within the chunk
    const int row = row0 + rr;
    const int s = seq_of_row(cu_q, num_seqs, row);
    const int p = (cu_k[s + 1] - cu_k[s]) - (cu_q[s + 1] - cu_q[s]) + (row - cu_q[s]);
    if (blocks_from > p - (row - cu_q[s]) % split_tq) return;   // a row of the query-tile schedule
    const int32_t *sel = ids + ((size_t)row * h + g) * top_k;
    const size_t base = (size_t)rr * top_k;   // the chunk's partials

    for (int h0 = 0; h0 < G; h0 += HPP) {
        const bool live = h0 + hs < G;
        const int head = g * G + (live ? h0 + hs : 0);
        float m = -INFINITY, acc[8], den = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 8
        for (int a = 0; a < top_k; ++a) {
            const int j = sel[a];
            const bool ok = j >= 0 && j <= p / B;   // the same in every lane
            // the loads are unconditional (slot 0's row stands in for a
            // skipped slot) so that the unrolled slots' loads overlap
            const size_t sh = (base + (ok ? a : 0)) * H + head;
            const float2 w = part_w[sh];
            const uint4 x = load16(part_o + sh * D + 8 * c);
            if (ok) {   // skipped slots hold no partial
                const float m_new = fmaxf(m, w.x);
                const float alpha = fast_exp2(m - m_new);   // 0 while m is -inf
                const float wd = fast_exp2(w.x - m_new);
                const float wn = wd * __builtin_ldexpf(1.0f, (int)w.y);   // the stored partial is scaled by 2^-e
                const f16x8 hv = as_f16x8(x);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(wn, (float)hv[i], acc[i] * alpha);
                den = fmaf(den, alpha, wd);
                m = m_new;
            }
        }
        const float inv = den > 0.f ? 1.0f / den : 0.f;
        const size_t rh = (size_t)row * H + head;
        if (live)
            *reinterpret_cast<uint4 *>(out + rh * D + 8 * c) =
                uint4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                      pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
        if (lse != nullptr && live && c == 0) lse[rh] = den > 0.f ? (m + __log2f(den)) * 0.69314718055994531f : -INFINITY;
    }
}

struct FwdWs {
    BlockLists lists;
    size_t part_o, part_w, bytes;
};

FwdWs fwd_ws(const Shape &s) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    FwdWs w;
    w.lists = block_lists_layout(s);
    size_t at = w.lists.bytes;
    w.part_o = at;
    at += al((size_t)s.rows * s.top_k * s.H * s.d * sizeof(uint16_t));
    w.part_w = at;
    at += al((size_t)s.rows * s.top_k * s.H * sizeof(float2));
    w.bytes = at;
    return w;
}

template <int D, int B>
hipError_t launch_fwd(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *ids,
                      float scale, uint16_t *out, float *lse, void *ws, hipStream_t st) {
    const FwdWs w = fwd_ws(s);
    char *base = static_cast<char *>(ws);
    const int32_t *blk_off = reinterpret_cast<const int32_t *>(base + w.lists.blk_off);
    const int32_t *off = reinterpret_cast<const int32_t *>(base + w.lists.off);
    const int32_t *entries = reinterpret_cast<const int32_t *>(base + w.lists.entries);
    uint16_t *part_o = reinterpret_cast<uint16_t *>(base + w.part_o);
    float2 *part_w = reinterpret_cast<float2 *>(base + w.part_w);
    const hipError_t e = launch_block_lists(s, ids, w.lists, base, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_block<D, B>), dim3((unsigned)w.lists.nb_max, s.h), dim3(64 * fwd_waves<B>()), 0, st, q, k, v, s.cu_q,
                       s.cu_k, blk_off, off, entries, s.num_seqs, s.H, s.h, (int)w.lists.nb_max, s.top_k,
                       make_fastdiv((uint32_t)s.top_k), s.row0, scale * kLog2e, part_o, part_w);
    const long pairs = (long)s.rows * s.h;
    hipLaunchKernelGGL((fwd_merge<D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, st, part_o, part_w, ids, s.cu_q,
                       s.cu_k, s.num_seqs, s.row0, pairs, s.H, s.h, s.B, s.top_k, s.blocks_from, s.split_tq, out,
                       lse);
    return hipGetLastError();
}

}  // namespace

// Rows per chunk of the block-centric schedule: the lists' per-key arrays are
// fixed, the entries, places and partials grow with the rows.
int block_prefill_chunk_rows(const Shape &s) {
    Shape one = s;
    one.rows = 1;
    const size_t fixed = fwd_ws(one).bytes;
    const size_t per_row = (size_t)s.h * s.top_k * 8 + (size_t)s.top_k * s.H * (2 * s.d + 8);
    return chunk_rows(s, fixed, per_row);
}

size_t block_prefill_workspace_bytes(const Shape &s) {
    Shape c = s;
    c.rows = block_prefill_chunk_rows(s);
    return fwd_ws(c).bytes;
}

// The query tiles stage the union of a tile's selections once per tile, so
// they pay off while a staged block serves many of the tile's queries: about
// R = Tq min(k, E) / E of them for a tile of Tq queries with E eligible
// blocks.  The block-centric schedule does no wasted work but writes and
// reads back one partial output per (row, slot, head).  Measured on
// 8K-64K-token prefills with clustered keys, each schedule called on its own
// (query-tile time / block-centric time, R taken at the average E): B = 64,
// G = 4 gave 0.48 at R = 32, 0.71-0.72 at 16, 0.92-0.96 at 8, 1.10 at 6,
// 1.31-1.32 at 4 and 1.68 at 2; B = 128, G = 6 gave 0.65 at R = 16, 0.89 at
// 12, 1.05 at 8, 1.22 at 6, 1.49 at 4, 2.13 at 2 and about 7 at about 1 (a
// 4-sequence 217K-token ragged prefill).  So the schedules break even near
// R = 7 (B = 64) and R = 10 (B = 128).  The rule is applied per query tile:
// E grows with the position, so the tiles take the early rows and the
// block-centric schedule the late ones.  Splitting a 32768-token prefill
// (B = 64, k = 32, G = 4) where R falls below R* = 6, 7, 8, 10 and 12
// (positions 21824, 18688, 16384, 13056 and 10880) took 4.47, 4.45, 4.40,
// 4.31 and 4.33 ms, against 4.88 ms on the tiles alone and 5.26 ms on the
// block-centric schedule alone; on the 217K-token ragged prefill (B = 128)
// R* = 10, 16 and 24 took 30.8, 30.8 and 31.2 ms.  R* = 10 for both.
int prefill_split_position(const Shape &s) {
    const int G = s.H / s.h;
    if (G < 1 || G > 16 || s.max_q < 1) return 0x7fffffff;
    const double thr = 10.0;
    // R = Tq k / E < thr  <=>  E > Tq k / thr (with E > k; for E <= k, R = Tq >= 16)
    const long e_star = (long)std::floor((double)prefill_tile_queries(s) * s.top_k / thr) + 1;
    const long p = (e_star - 1) * s.B;
    return p >= 0x7fffffffL ? 0x7fffffff : (int)p;
}

hipError_t launch_attn_prefill_blocks(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                      const int32_t *ids, float scale, uint16_t *out, float *lse, void *ws,
                                      hipStream_t st) {
    if (s.H / s.h > 16) return hipErrorInvalidValue;
    if (!((s.d == 64 || s.d == 128) && (s.B == 64 || s.B == 128))) return hipErrorInvalidValue;
    // The rows [s.row0, s.row0 + s.rows) in chunks that keep the workspace
    // under the cap; each chunk builds its own lists and merges its own rows.
    const int per = block_prefill_chunk_rows(s);
    const int r_end = s.row0 + s.rows;
    for (int r0 = s.row0; r0 < r_end; r0 += per) {
        Shape c = s;
        c.row0 = r0;
        c.rows = std::min(per, r_end - r0);
        hipError_t e = hipErrorInvalidValue;
        if (s.d == 64 && s.B == 64) e = launch_fwd<64, 64>(c, q, k, v, ids, scale, out, lse, ws, st);
        if (s.d == 64 && s.B == 128) e = launch_fwd<64, 128>(c, q, k, v, ids, scale, out, lse, ws, st);
        if (s.d == 128 && s.B == 64) e = launch_fwd<128, 64>(c, q, k, v, ids, scale, out, lse, ws, st);
        if (s.d == 128 && s.B == 128) e = launch_fwd<128, 128>(c, q, k, v, ids, scale, out, lse, ws, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace msa
