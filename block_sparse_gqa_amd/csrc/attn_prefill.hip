// Sparse branch, prefill: exact softmax attention of every query head over
// the visible tokens of the blocks its GQA group selected, read from the
// original K/V ("MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a
// minimal sparse attention", second layer; "MiniMax Goes Sparse", section 1,
// step 2).
//
// Reuse.  The heads of a group share one selection, and neighbouring queries
// of a group pick overlapping block sets.  A workgroup therefore owns a tile
// of Tq consecutive queries of one group (all G heads), forms the union of
// their selected blocks, and streams each union block through LDS once:
// 64-token K and V sub-blocks, double-buffered, staged by all 256 threads.
//
// Rows.  A row is one (query, head) pair.  Each wave owns RT fixed row tiles
// of 16 rows (16/G queries x G heads) whose O accumulators, running max and
// running sum stay in registers for the whole tile; for a staged block a wave
// runs MFMA only on its row tiles that contain a query which selected the
// block, and masks the rows whose query did not (and future tokens).
//   S^T = K . Q^T     v_mfma_f32_16x16x32_bf16, A = K rows from LDS,
//                     B = Q^T resident in registers;
//   O^T += V^T . P^T  A = V^T read from the token-major LDS copy with the
//                     transposing ds_read_b64_tr_b16, B = P^T straight from the
//                     S^T accumulators, split into bf16 head + tail.
// Workgroups are numbered group-fastest, so with 8 groups all tiles of a
// group run on the same XCD and share its L2.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kWin = 256;   // key blocks per union window (one per thread)

template <int D>
struct Stage {
    static constexpr int KROW = D * 2 + 16;   // padded LDS rows (bank-conflict free reads)
    static constexpr int VROW = D * 2 + 32;
    static constexpr int CH = 64 * D / 8 / 256;   // 16-byte chunks per thread per tensor
};

template <int D, int RT>
__global__ __launch_bounds__(256, 2) void attn_prefill_tile(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
    int num_seqs, int H, int h, int B, int top_k, int max_tiles, float c2, uint16_t *__restrict__ out,
    float *__restrict__ lse) {
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    constexpr int CH = Stage<D>::CH;
    constexpr int KROW = Stage<D>::KROW, VROW = Stage<D>::VROW;
    constexpr int CPR = D / 8;
    __shared__ __attribute__((aligned(16))) char kbuf[2][64 * KROW];
    __shared__ __attribute__((aligned(16))) char vbuf[2][64 * VROW];
    __shared__ unsigned long long masks[kWin];
    __shared__ unsigned long long list_m[kWin];
    __shared__ int list_u[kWin];
    __shared__ int wave_cnt[4];

    const int G = H / h;
    const int Qt = 16 / G;                    // queries per row tile
    const int Tq = 4 * RT * Qt;               // queries per workgroup (<= 64)
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
    const int tq_valid = min(Tq, len_q - r0);
    const int p_last = shift + r0 + tq_valid - 1;
    const int e_tile = p_last / B + 1;
    const int nsub = B / 64;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;

    // This lane's row in each of the wave's row tiles.
    bf16x8 qop[RT][KS];
    int prow[RT], qbit[RT];
    f32x4 o[RT][DT];
    float m[RT], l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int qi = l16 / G, head = l16 % G;
        const int qidx = (wave * RT + rt) * Qt + qi;
        const bool ok = (l16 < Qt * G) && (qidx < tq_valid);
        prow[rt] = ok ? shift + r0 + qidx : -1;
        qbit[rt] = qidx;
        const uint16_t *src = q + ((size_t)(q_begin + r0 + qidx) * H + g * G + head) * D + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[rt][ks] = as_bf16x8(load16_if(src + 32 * ks, ok, q));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[rt] = -INFINITY;
        l[rt] = 0.0f;
    }
    const unsigned long long tile_bits = (Qt >= 64) ? ~0ull : ((1ull << Qt) - 1ull);

    uint4 kst[CH], vst[CH];
    auto gload = [&](int t0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ci = c * 256 + tid;
            const int tok = ci / CPR, c16 = ci % CPR;
            const int t = t0 + tok;
            const bool ok = t < len_k;
            kst[c] = load16_if(k + ((k_begin + t) * h + g) * D + c16 * 8, ok, k);
            vst[c] = load16_if(v + ((k_begin + t) * h + g) * D + c16 * 8, ok, v);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ci = c * 256 + tid;
            const int tok = ci / CPR, c16 = ci % CPR;
            *reinterpret_cast<uint4 *>(&kbuf[buf][tok * KROW + c16 * 16]) = kst[c];
            *reinterpret_cast<uint4 *>(&vbuf[buf][tok * VROW + c16 * 16]) = vst[c];
        }
    };

    for (int w0 = 0; w0 < e_tile; w0 += kWin) {
        masks[tid] = 0ull;
        __syncthreads();
        // Which queries of the tile selected which block of this window.
        const int32_t *tile_ids = ids + ((size_t)(q_begin + r0) * h + g) * top_k;
        for (int e = tid; e < tq_valid * top_k; e += 256) {
            const int qi = e / top_k, a = e % top_k;
            const int j = tile_ids[(size_t)qi * h * top_k + a];
            const int pq = shift + r0 + qi;
            if (j >= w0 && j < w0 + kWin && j >= 0 && j <= pq / B) atomicOr(&masks[j - w0], 1ull << qi);
        }
        __syncthreads();
        // Compact the blocks somebody selected, ascending.
        const unsigned long long mv = masks[tid];
        const unsigned long long bal = __ballot(mv != 0ull);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (lane == 0) wave_cnt[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int base = 0, count = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            base += (w < wave) ? wave_cnt[w] : 0;
            count += wave_cnt[w];
        }
        if (mv != 0ull) {
            list_u[base + before] = w0 + tid;
            list_m[base + before] = mv;
        }
        __syncthreads();

        const int nitems = count * nsub;
        auto t0_of = [&](int it) { return list_u[it / nsub] * B + (it % nsub) * 64; };
        if (nitems > 0) {
            if (t0_of(0) <= p_last) gload(t0_of(0));
            lstore(0);
            __syncthreads();
        }
        for (int it = 0; it < nitems; ++it) {
            const int buf = it & 1;
            const int t0 = t0_of(it);
            const bool have_next = it + 1 < nitems;
            const int t0n = have_next ? t0_of(it + 1) : 0;
            if (have_next && t0n <= p_last) gload(t0n);
            const unsigned long long mk = list_m[it / nsub];
            const unsigned long long wbits = mk >> (wave * RT * Qt);
            bool act[RT];
            bool any = false;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                act[rt] = ((wbits >> (rt * Qt)) & tile_bits) != 0ull;
                any |= act[rt];
            }
            if (t0 <= p_last && any) {
                f32x4 sacc[RT][4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    bf16x8 a[KS];
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        a[ks] = *reinterpret_cast<const bf16x8 *>(
                            &kbuf[buf][(tt * 16 + l16) * KROW + (32 * ks + 8 * q4) * 2]);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        if (!act[rt]) continue;
                        sacc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) sacc[rt][tt] = mfma16x16x32(a[ks], qop[rt][ks], sacc[rt][tt]);
                    }
                }
                // online softmax per row (log2 domain)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    if (!act[rt]) continue;
                    const bool selected = prow[rt] >= 0 && ((mk >> qbit[rt]) & 1ull);
                    float mloc = -INFINITY;
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int t = t0 + tt * 16 + 4 * q4 + i;
                            const float x = (selected && t <= prow[rt]) ? sacc[rt][tt][i] * c2 : -INFINITY;
                            sacc[rt][tt][i] = x;
                            mloc = fmaxf(mloc, x);
                        }
                    mloc = max_xor32(max_xor16(mloc));
                    const float m_new = fmaxf(m[rt], mloc);
                    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
                    const float alpha = exp2f(m[rt] - m_use);
                    m[rt] = m_new;
                    float lsum = 0.0f;
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float e = exp2f(sacc[rt][tt][i] - m_use);
                            sacc[rt][tt][i] = e;
                            lsum += e;
                        }
                    l[rt] = l[rt] * alpha + lsum;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
                }
                // O^T += V^T . P^T, P split into bf16 head + tail
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    bf16x8 p_hi[RT], p_lo[RT];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        if (!act[rt]) continue;
                        // slots 8*q4 + i <- tile 2*s2 value i, slots 8*q4 + 4 + i <- tile 2*s2+1 value i
                        float pv[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pv[i] = sacc[rt][2 * s2][i];
                            pv[4 + i] = sacc[rt][2 * s2 + 1][i];
                        }
                        uint32_t hi[4], lo[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x0 = pv[2 * i], x1 = pv[2 * i + 1];
                            const uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
                            hi[i] = h0 | (h1 << 16);
                            lo[i] = pack_bf16x2(x0 - __uint_as_float(h0 << 16), x1 - __uint_as_float(h1 << 16));
                        }
                        p_hi[rt] = as_bf16x8(uint4{hi[0], hi[1], hi[2], hi[3]});
                        p_lo[rt] = as_bf16x8(uint4{lo[0], lo[1], lo[2], lo[3]});
                    }
                    const int tok_a = 32 * s2 + 4 * q4 + (l16 >> 2);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const int col = dt * 16 + 4 * (l16 & 3);
                        const i16x4 va = lds_read_tr16(&vbuf[buf][tok_a * VROW + col * 2]);
                        const i16x4 vb = lds_read_tr16(&vbuf[buf][(tok_a + 16) * VROW + col * 2]);
                        uint4 au;
                        au.x = (uint32_t)(uint16_t)va[0] | ((uint32_t)(uint16_t)va[1] << 16);
                        au.y = (uint32_t)(uint16_t)va[2] | ((uint32_t)(uint16_t)va[3] << 16);
                        au.z = (uint32_t)(uint16_t)vb[0] | ((uint32_t)(uint16_t)vb[1] << 16);
                        au.w = (uint32_t)(uint16_t)vb[2] | ((uint32_t)(uint16_t)vb[3] << 16);
                        const bf16x8 vop = as_bf16x8(au);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
                            if (!act[rt]) continue;
                            o[rt][dt] = mfma16x16x32(vop, p_hi[rt], o[rt][dt]);
                            o[rt][dt] = mfma16x16x32(vop, p_lo[rt], o[rt][dt]);
                        }
                    }
                }
            }
            if (have_next) lstore(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: normalise and write this wave's rows.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float lt = sum_xor32(sum_xor16(l[rt]));
        if (prow[rt] < 0) continue;
        const int qi = l16 / G, head = l16 % G;
        const int row = q_begin + r0 + (wave * RT + rt) * Qt + qi;
        const float inv = lt > 0.f ? 1.0f / lt : 0.0f;
        uint16_t *dst = out + ((size_t)row * H + g * G + head) * D + 4 * q4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            uint2 w;
            w.x = pack_bf16x2(o[rt][dt][0] * inv, o[rt][dt][1] * inv);
            w.y = pack_bf16x2(o[rt][dt][2] * inv, o[rt][dt][3] * inv);
            *reinterpret_cast<uint2 *>(dst + dt * 16) = w;
        }
        if (lse != nullptr && q4 == 0)
            lse[(size_t)row * H + g * G + head] = lt > 0.f ? (m[rt] + log2f(lt)) * 0.69314718055994531f : -INFINITY;
    }
}

template <int D, int RT>
hipError_t launch(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *ids,
                  float scale, uint16_t *out, float *lse, hipStream_t st) {
    const int G = s.H / s.h;
    const int Tq = 4 * RT * (16 / G);
    const int max_tiles = (s.max_q + Tq - 1) / Tq;
    const long grid = (long)max_tiles * s.num_seqs * s.h;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_prefill_tile<D, RT>), dim3((unsigned)grid), dim3(256), 0, st, q, k, v, ids, s.cu_q,
                       s.cu_k, s.num_seqs, s.H, s.h, s.B, s.top_k, max_tiles, scale * kLog2e, out, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *ids, float scale, uint16_t *out, float *lse, hipStream_t st) {
    const int G = s.H / s.h;
    if (G < 1 || G > 16) return hipErrorInvalidValue;
    const bool two = 4 * 2 * (16 / G) <= 64;   // at most 64 queries per tile (one mask bit each)
    if (s.d == 64) return two ? launch<64, 2>(s, q, k, v, ids, scale, out, lse, st)
                              : launch<64, 1>(s, q, k, v, ids, scale, out, lse, st);
    if (s.d == 128) return two ? launch<128, 2>(s, q, k, v, ids, scale, out, lse, st)
                               : launch<128, 1>(s, q, k, v, ids, scale, out, lse, st);
    return hipErrorInvalidValue;
}

}  // namespace msa
