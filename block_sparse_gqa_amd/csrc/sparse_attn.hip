// Sparse branch, decode: exact softmax attention of the G query heads of one GQA
// group over the blocks that group selected, read from the original,
// uncompressed K/V ("MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a
// minimal sparse attention", second layer: the heads of a group share one
// selection, so one load of a K/V block serves all G heads; "MiniMax Goes
// Sparse", section 1, step 2).
//
// One wave owns one (split, query, group).  The G heads sit on the N side of
// v_mfma_f32_16x16x32_bf16 (padded to 16).  Per 32-token sub-block, whose K
// and V rows are loaded as whole lines into registers (two sub-blocks ahead)
// and then copied to padded LDS tiles:
//   S^T = K . Q^T   A = K rows from LDS, B = Q^T held in registers;
//   online softmax in the exp2 domain, per head = per lane column;
//   O^T += V^T . P^T  B = P^T comes from the S^T accumulators without any data
//                   movement (the contraction index is permuted consistently on
//                   both sides), split into a bf16 head and tail; A = V^T is
//                   read from the token-major V tile with the transposing
//                   ds_read_b64_tr_b16.
// Decode splits a sequence's selected blocks over many waves and merges the
// partial results by log-sum-exp.
#include <mutex>
#include <type_traits>

#include "msa.h"
#include "msa_device.h"
#include "msa_internal.h"

// Fixed device memory for the allocation-free decode entry point: its split
// partials (the workspace msa_sparse_attn_decode takes from the caller).  Each
// GPU the library runs on holds its own copy from module load until the
// process ends.  Host code never uses this name as an address: the per-device
// address comes from hipGetSymbolAddress below.
constexpr size_t kDecodeScratchBytes = MSA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace msa {

namespace {

constexpr int kSub = 32;       // tokens per sub-block
constexpr int kTT = kSub / 16; // 16-token MFMA tiles per sub-block
constexpr int kChunk = 64;     // selected ids scanned per list refill

template <int D>
struct DecodeLds {
    static constexpr int KROW = D * 2 + 16;   // conflict-free K operand reads
    static constexpr int VROW = D * 2 + 32;   // conflict-free transposing V reads
    static constexpr int KBYTES = kSub * KROW;
    static constexpr int VBYTES = kSub * VROW;
    static constexpr int CH = kSub * D / 8 / 64;   // 16-byte chunks per lane per tensor
    static constexpr int KS = D / 32;
};

template <int D>
struct Acc {
    f32x4 o[D / 16];   // O^T: lane l -> head l%16, dims dt*16 + 4*(l/16) + i
    float m;           // running max (log2 domain), same in the 4 lanes of a head
    float l;           // this lane's partial sum of exp2
};

template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qop)[D / 32], const uint16_t *q, size_t row, int H, int head0, int G) {
    const int lane = lane_id();
    const int hq = lane & 15, q4 = lane >> 4;
    const bool ok = hq < G;
    const uint16_t *src = q + (row * H + head0 + hq) * D + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qop[ks] = as_bf16x8(load16_if(src + 32 * ks, ok, q));
}

// Sum the 4 per-lane partials of each head.
__device__ __forceinline__ float head_total(float l) {
    l = sum_xor16(l);
    return sum_xor32(l);
}

// K and V rows of one sub-block.  Every load instruction reads whole lines
// (lane i takes the i-th 16-byte chunk of 4 consecutive 256-byte rows), which
// streams markedly faster than operand-shaped loads; rows are re-laid out
// through LDS.  row0 (the cache row of the sub-block's first token) and nvalid
// (its tokens before the sequence end) are wave-uniform: the base address is
// scalar and lanes add 32-bit offsets.  Tokens past the end read as zeros.
template <int D, bool NT>
__device__ __forceinline__ void load_kv(uint4 (&kr)[DecodeLds<D>::CH], uint4 (&vr)[DecodeLds<D>::CH],
                                        const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int row0_in,
                                        int nvalid_in, int h, int g) {
    constexpr int CPR = D / 8;
    const int lane = lane_id();
    const int row0 = __builtin_amdgcn_readfirstlane(row0_in);
    const int nvalid = __builtin_amdgcn_readfirstlane(nvalid_in);
    const size_t base = ((size_t)row0 * h + g) * D;
    const bool inside = nvalid >= kSub;
#pragma unroll
    for (int x = 0; x < DecodeLds<D>::CH; ++x) {
        const int ci = x * 64 + lane;
        const int tok = ci / CPR, c16 = ci % CPR;
        const uint32_t off = (uint32_t)(tok * h * D + c16 * 8);
        if (inside) {
            kr[x] = NT ? load16_nt(k + base + off) : load16(k + base + off);
            vr[x] = NT ? load16_nt(v + base + off) : load16(v + base + off);
        } else {
            kr[x] = NT ? load16_nt_if(k + base + off, tok < nvalid, k) : load16_if(k + base + off, tok < nvalid, k);
            vr[x] = NT ? load16_nt_if(v + base + off, tok < nvalid, v) : load16_if(v + base + off, tok < nvalid, v);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_kv(const uint4 (&kr)[DecodeLds<D>::CH], const uint4 (&vr)[DecodeLds<D>::CH],
                                         char *klds, char *vlds) {
    constexpr int CPR = D / 8;
    const int lane = lane_id();
#pragma unroll
    for (int x = 0; x < DecodeLds<D>::CH; ++x) {
        const int ci = x * 64 + lane;
        const int tok = ci / CPR, c16 = ci % CPR;
        *reinterpret_cast<uint4 *>(klds + tok * DecodeLds<D>::KROW + c16 * 16) = kr[x];
        *reinterpret_cast<uint4 *>(vlds + tok * DecodeLds<D>::VROW + c16 * 16) = vr[x];
    }
}

// S^T = K . Q^T for the sub-block in LDS (A = K rows: token tt*16 + l%16,
// dims 32*ks + 8*(l/16)).
template <int D>
__device__ __forceinline__ void qk_sub(f32x4 (&s)[kTT], const char *klds, const bf16x8 (&qop)[D / 32]) {
    const int lane = lane_id();
    const int q4 = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(klds + (tt * 16 + l16) * DecodeLds<D>::KROW +
                                                               (32 * ks + 8 * q4) * 2);
            s[tt] = mfma16x16x32(a, qop[ks], s[tt]);
        }
    }
}

// Online-softmax update with the scores of one sub-block starting at token t0
// (scores become probabilities in place; O is rescaled).
template <int D>
__device__ __forceinline__ void softmax_sub(Acc<D> &acc, f32x4 (&s)[kTT], int len_k, int p, int t0, float c2) {
    const int lane = lane_id();
    const int q4 = lane >> 4;
    float mloc = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + tt * 16 + 4 * q4 + i;
            float x = s[tt][i] * c2;
            x = (t <= p && t < len_k) ? x : -INFINITY;
            s[tt][i] = x;
            mloc = fmaxf(mloc, x);
        }
    mloc = max_xor32(max_xor16(mloc));
    const float m_new = fmaxf(acc.m, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(acc.m - m_use);
    acc.m = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2(s[tt][i] - m_use);
            s[tt][i] = e;
            lsum += e;
        }
    acc.l = acc.l * alpha + lsum;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc.o[dt] *= alpha;
}

// O^T += V^T . P^T over the 32 tokens 32*s2 .. 32*s2+31 of the sub-block, V read
// from LDS with the transposing read.
template <int D>
__device__ __forceinline__ void pv_half(Acc<D> &acc, const f32x4 (&s)[kTT], const char *vlds, int s2) {
    constexpr int DT = D / 16;
    using L = DecodeLds<D>;
    const int lane = lane_id();
    const int q4 = lane >> 4, l16 = lane & 15;
    // B = P^T: slots 8*q4 + i <- token 32*s2 + 4*q4 + i, slots 8*q4 + 4 + i <- token 32*s2 + 16 + 4*q4 + i.
    // P is split into a bf16 head and a bf16 tail (p = hi + lo + O(2^-17 p)), so the
    // probabilities keep float32-like accuracy even when only a few tokens are visible.
    float pv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pv[i] = s[2 * s2][i];
        pv[4 + i] = s[2 * s2 + 1][i];
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hi[i] = split_bf16x2(pv[2 * i], pv[2 * i + 1], &lo[i]);
    const bf16x8 pop_hi = as_bf16x8(uint4{hi[0], hi[1], hi[2], hi[3]});
    const bf16x8 pop_lo = as_bf16x8(uint4{lo[0], lo[1], lo[2], lo[3]});
    const int tok_a = 32 * s2 + 4 * q4 + (l16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const int col = dt * 16 + 4 * (l16 & 3);
        const i16x4 va = lds_read_tr16(vlds + tok_a * L::VROW + col * 2);
        const i16x4 vb = lds_read_tr16(vlds + (tok_a + 16) * L::VROW + col * 2);
        const uint2 xa = __builtin_bit_cast(uint2, va), xb = __builtin_bit_cast(uint2, vb);
        const bf16x8 vop = as_bf16x8(uint4{xa.x, xa.y, xb.x, xb.y});
        acc.o[dt] = mfma16x16x32(vop, pop_hi, acc.o[dt]);
        acc.o[dt] = mfma16x16x32(vop, pop_lo, acc.o[dt]);
    }
}

// One wave per (split, group, sequence): attend its share of the selected
// blocks; write the partial output (normalised) and its log2-sum-exp.
// The current sub-block sits in LDS while the next one's loads are in flight.
// PAGED: k and v are pools of pages of B rows; block j of sequence s sits in
// page table[s * table_stride + j] (clamped into [0, num_pages)).
template <int D, int B, bool PAGED, bool NT>
__global__ __launch_bounds__(64, 2) void attn_decode_split(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
    int H, int h, int top_k, int per_split, float c2, float *__restrict__ part_o, float *__restrict__ part_lse,
    const int32_t *__restrict__ table, int table_stride, int num_pages) {
    using L = DecodeLds<D>;
    constexpr int NSUB = B / kSub;
    __shared__ __attribute__((aligned(16))) char klds[L::KBYTES];
    __shared__ __attribute__((aligned(16))) char vlds[L::VBYTES];
    __shared__ int list[kChunk * NSUB];   // first token of each sub-block (sequence position)
    __shared__ int rows[kChunk * NSUB];   // its cache row
    const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    const int nsplit = gridDim.x;
    const int G = H / h;
    const int row = cu_q[s + 1] - 1;
    const size_t k_begin = (size_t)cu_k[s];
    const int len_k = cu_k[s + 1] - cu_k[s];
    const int p = len_k - 1;
    const int lane = lane_id();

    bf16x8 qop[D / 32];
    load_q<D>(qop, q, (size_t)row, H, g * G, G);
    Acc<D> acc;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.m = -INFINITY;
    acc.l = 0.0f;

    const int32_t *sel = ids + ((size_t)row * h + g) * top_k;
    const int a0 = split * per_split, a1 = min(top_k, a0 + per_split);
    // Sub-block i sits in LDS (K and V) while the next two are in flight in
    // two register sets (A, B), 32 KB per wave; two waves share a SIMD.
    uint4 kA[L::CH], vA[L::CH], kB[L::CH], vB[L::CH];
    f32x4 sc[kTT];
    for (int c0 = a0; c0 < a1; c0 += kChunk) {
        // Sub-block starts of this chunk's valid, causal ids (any id order).
        const int a = c0 + lane;
        const int j = a < a1 ? sel[a] : -1;
        const bool jok = j >= 0 && j <= p / B;
        int row_j = (int)k_begin + j * B;
        if constexpr (PAGED) row_j = jok ? min(max(table[(size_t)s * table_stride + j], 0), num_pages - 1) * B : 0;
        int n = 0;
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            const bool ok = jok && j * B + sb * kSub <= p;
            const unsigned long long bal = __ballot(ok);
            const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
            if (ok) {
                list[n + pos] = j * B + sb * kSub;
                rows[n + pos] = row_j + sb * kSub;
            }
            n += __builtin_popcountll(bal);
        }
        wave_lds_sync();
        if (n == 0) continue;
        load_kv<D, NT>(kA, vA, k, v, rows[0], len_k - list[0], h, g);
        if (n > 1) load_kv<D, NT>(kB, vB, k, v, rows[1], len_k - list[1], h, g);
        store_kv<D>(kA, vA, klds, vlds);
        if (n > 2) load_kv<D, NT>(kA, vA, k, v, rows[2], len_k - list[2], h, g);
        for (int i = 0; i < n; i += 2) {
            // sub-block i in LDS; set B holds i+1, set A holds i+2
            wave_lds_sync();
            qk_sub<D>(sc, klds, qop);
            softmax_sub<D>(acc, sc, len_k, p, list[i], c2);
            pv_half<D>(acc, sc, vlds, 0);
            wave_lds_sync();
            if (i + 1 >= n) break;
            store_kv<D>(kB, vB, klds, vlds);
            if (i + 3 < n) load_kv<D, NT>(kB, vB, k, v, rows[i + 3], len_k - list[i + 3], h, g);
            // sub-block i+1 in LDS; set A holds i+2, set B holds i+3
            wave_lds_sync();
            qk_sub<D>(sc, klds, qop);
            softmax_sub<D>(acc, sc, len_k, p, list[i + 1], c2);
            pv_half<D>(acc, sc, vlds, 0);
            wave_lds_sync();
            if (i + 2 >= n) break;
            store_kv<D>(kA, vA, klds, vlds);
            if (i + 4 < n) load_kv<D, NT>(kA, vA, k, v, rows[i + 4], len_k - list[i + 4], h, g);
        }
    }
    const float l = head_total(acc.l);
    const int hq = lane & 15, q4 = lane >> 4;
    if (hq < G) {
        const size_t slot = (((size_t)s * H + g * G + hq) * nsplit + split);
        const float inv = l > 0.f ? 1.0f / l : 0.0f;
        float *o = part_o + slot * D + 4 * q4;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            *reinterpret_cast<float4 *>(o + dt * 16) =
                make_float4(acc.o[dt][0] * inv, acc.o[dt][1] * inv, acc.o[dt][2] * inv, acc.o[dt][3] * inv);
        if (q4 == 0) part_lse[slot] = l > 0.f ? acc.m + log2f(l) : -INFINITY;   // log2 domain
    }
}

// One wave per (sequence, head): O = sum_s w_s O_s / sum_s w_s with
// w_s = 2^(lse_s - max).  Split weights go through LDS; the d columns are
// spread over the lanes and every split's row is an independent load.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_merge(const float *__restrict__ part_o,
                                                        const float *__restrict__ part_lse, int H, int nsplit,
                                                        uint16_t *__restrict__ out, float *__restrict__ lse) {
    __shared__ float wsh[256];
    const int head = blockIdx.x, s = blockIdx.y;
    const int lane = lane_id();
    const size_t base = ((size_t)s * H + head) * nsplit;
    float m = -INFINITY;
    for (int x = lane; x < nsplit; x += 64) m = fmaxf(m, part_lse[base + x]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float wsum = 0.f;
    for (int x = lane; x < nsplit; x += 64) {
        const float ls = part_lse[base + x];
        const float w = (ls == -INFINITY) ? 0.f : exp2f(ls - m);
        wsh[x] = w;
        wsum += w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off, 64);
    wave_lds_sync();
    constexpr int PER = D / 64;
    float o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    const float *src = part_o + base * D + lane * PER;
    int x = 0;
    for (; x + 4 <= nsplit; x += 4) {
        float t[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < PER; ++i) t[u][i] = src[(size_t)(x + u) * D + i];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < PER; ++i) o[i] += wsh[x + u] * t[u][i];
    }
    for (; x < nsplit; ++x)
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += wsh[x] * src[(size_t)x * D + i];
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    uint16_t *dst = out + ((size_t)s * H + head) * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(o[0] * inv, o[1] * inv);
    } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) dst[i] = (uint16_t)(pack_bf16x2(o[i] * inv, 0.f) & 0xffffu);
    }
    if (lse != nullptr && lane == 0)
        lse[(size_t)s * H + head] = wsum > 0.f ? (m + log2f(wsum)) * 0.69314718055994531f : -INFINITY;
}


// K and V bytes a decode call gathers: top_k blocks of each per (sequence, group).
double decode_selected_bytes(const Shape &s) { return (double)s.num_seqs * s.h * s.top_k * s.B * s.d * 2.0 * 2.0; }

template <int D, int B>
hipError_t launch_decode(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *ids, float scale, uint16_t *out, float *lse, void *ws, hipStream_t st) {
    const int nsplit = decode_splits(s);
    const int per = (s.top_k + nsplit - 1) / nsplit;
    float *part_o = reinterpret_cast<float *>(ws);
    float *part_lse = part_o + (size_t)s.num_seqs * s.H * nsplit * s.d;
    const dim3 grid(nsplit, s.h, s.num_seqs);
    // Selections larger than the MALL could keep between calls are streamed
    // with non-temporal loads (the 4 x 1M decode's 1.07 GB: 196 -> 176 us);
    // smaller ones keep plain loads, which let consecutive steps find them in
    // the MALL (the 8 x 64K decode's 134 MB: 31 against 33 us with nt).
    const bool nt = decode_selected_bytes(s) > kDecodeStreamBytes;
    auto go = [&](auto paged, auto ntag) {
        constexpr bool P = decltype(paged)::value, N = decltype(ntag)::value;
        hipLaunchKernelGGL((attn_decode_split<D, B, P, N>), grid, dim3(64), 0, st, q, k, v, ids, s.cu_q, s.cu_k, s.H,
                           s.h, s.top_k, per, scale * kLog2e, part_o, part_lse, P ? s.table : nullptr,
                           P ? s.table_stride : 0, P ? s.num_pages : 0);
    };
    if (s.table != nullptr) {
        if (nt) go(std::true_type{}, std::true_type{}); else go(std::true_type{}, std::false_type{});
    } else {
        if (nt) go(std::false_type{}, std::true_type{}); else go(std::false_type{}, std::false_type{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_decode_merge<D>), dim3(s.H, s.num_seqs), dim3(64), 0, st, part_o, part_lse, s.H, nsplit,
                       out, lse);
    return hipGetLastError();
}

}  // namespace

int decode_splits(const Shape &s) {
    // Aim for ~768 waves (three per CU) when the selection streams from HBM,
    // ~1024 when it is small enough to stay in the MALL; each split keeps at
    // least one block.  Swept with the current kernels (512, 768, 1024, 1536
    // waves): the 4 x 1M decode's attention took 200, 175, 188 and 178 us, the
    // 8 x 64K decode's 32.1, 31.4, 29.9 and 32.2 us.
    long pairs = (long)s.num_seqs * s.h;
    const long waves = decode_selected_bytes(s) > kDecodeStreamBytes ? 768 : 1024;
    long want = (waves + pairs - 1) / pairs;
    if (want > s.top_k) want = s.top_k;
    if (want < 1) want = 1;
    if (want > 256) want = 256;
    return (int)want;
}

size_t decode_workspace_bytes(const Shape &s) {
    const size_t n = (size_t)s.num_seqs * s.H * decode_splits(s);
    return n * (size_t)s.d * sizeof(float) + n * sizeof(float);
}

hipError_t launch_attn_decode(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *ids, float scale, uint16_t *out, float *lse, void *ws,
                              hipStream_t st) {
    if (s.d == 64 && s.B == 64) return launch_decode<64, 64>(s, q, k, v, ids, scale, out, lse, ws, st);
    if (s.d == 64 && s.B == 128) return launch_decode<64, 128>(s, q, k, v, ids, scale, out, lse, ws, st);
    if (s.d == 128 && s.B == 64) return launch_decode<128, 64>(s, q, k, v, ids, scale, out, lse, ws, st);
    if (s.d == 128 && s.B == 128) return launch_decode<128, 128>(s, q, k, v, ids, scale, out, lse, ws, st);
    return hipErrorInvalidValue;
}

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

hipError_t decode_scratch(void **ptr) {
    // Device address of `scratch` on the current device, looked up once per
    // device (with that device current) and kept.
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace msa
