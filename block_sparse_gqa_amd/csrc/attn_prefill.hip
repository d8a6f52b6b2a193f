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
// Staging.  A 4-stage LDS ring is filled with direct global->LDS loads
// (global_load_lds_dwordx4: lane i of a load writes base + 16*i), so three
// sub-blocks are in flight per workgroup without holding staging registers.
// Row strides are padded (K: 2d+16 bytes, V: 2d+64 bytes) so that the K
// operand reads and the transposing V reads are bank-conflict free; pad
// slots are filled by the same loads and never read.  Ring reads are issued
// in inline asm (each block waits for its own results) so the compiler does
// not serialise them behind the in-flight ring loads; completion of a stage
// is tracked with explicit vmcnt waits plus a barrier.
//
// Rows.  A row is one (query, head) pair.  Each of the NW waves owns RT fixed row tiles
// of 16 rows (16/G queries x G heads) whose O accumulators, running max and
// running sum stay in registers for the whole tile; for a staged sub-block a
// wave runs MFMA only on its row tiles that contain a query which selected
// the block, and masks the rows whose query did not (and future tokens).
//   S^T = K . Q^T     v_mfma_f32_16x16x32_bf16, A = K rows from LDS,
//                     B = Q^T resident in registers;
//   O^T += V^T . P^T  A = V^T read with the transposing ds_read_b64_tr_b16,
//                     B = P^T straight from the S^T accumulators, split into
//                     a bf16 head and tail.
// Workgroups are numbered group-fastest, so with 8 groups all tiles of a
// group run on the same XCD and share its L2.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;

constexpr int kWin = 256;    // key blocks per union window (one per thread)
constexpr int kStages = 4;   // ring depth (sub-blocks)

template <int D>
struct Ring {
    static constexpr int KROW = D * 2 + 16;
    static constexpr int VROW = D * 2 + 64;
    static constexpr int KSLOT_ROW = KROW / 16;   // 16-byte slots per row
    static constexpr int VSLOT_ROW = VROW / 16;
    static constexpr int KINSTR = KSLOT_ROW;      // 64 rows x slots / 64 lanes per load
    static constexpr int VINSTR = VSLOT_ROW;
    static constexpr int KBYTES = 64 * KROW;
    static constexpr int VBYTES = 64 * VROW;
    static constexpr int STAGE = KBYTES + VBYTES;
    // loads issued per sub-block by wave w of NW (instructions i = w, w+NW, ...)
    template <int NW>
    static constexpr int per_wave(int w) { return (KINSTR - w + NW - 1) / NW + (VINSTR - w + NW - 1) / NW; }
    // waves fall into at most three classes of equal per-wave counts
    template <int NW>
    static constexpr int wave_class(int w) {
        return per_wave<NW>(w) == per_wave<NW>(0) ? 0 : (per_wave<NW>(w) == per_wave<NW>(NW - 1) ? 2 : 1);
    }
    template <int NW>
    static constexpr int class_rep(int c) {
        for (int w = 0; w < NW; ++w)
            if (wave_class<NW>(w) == c) return w;
        return NW - 1;
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

// Four 16-byte K operand reads (k-steps 0..3, 64 bytes apart), one wait.
__device__ __forceinline__ void lds_k4(uint4 &a0, uint4 &a1, uint4 &a2, uint4 &a3, uint32_t addr) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:64\n\t"
        "ds_read_b128 %2, %4 offset:128\n\t"
        "ds_read_b128 %3, %4 offset:192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
        : "v"(addr)
        : "memory");
}
__device__ __forceinline__ void lds_k2(uint4 &a0, uint4 &a1, uint32_t addr) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1)
        : "v"(addr)
        : "memory");
}

// Transposing V reads for 4 consecutive 16-column d-tiles: for each, rows
// tok and tok + 16 (offset ROW16 bytes), columns 32 bytes apart.
template <int OFF, int ROW16>
__device__ __forceinline__ void lds_v4(i16x4 (&va)[4], i16x4 (&vb)[4], uint32_t addr) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(va[0]), "=&v"(vb[0]), "=&v"(va[1]), "=&v"(vb[1]), "=&v"(va[2]), "=&v"(vb[2]), "=&v"(va[3]), "=&v"(vb[3])
        : "v"(addr), "i"(OFF), "i"(OFF + ROW16), "i"(OFF + 32), "i"(OFF + 32 + ROW16), "i"(OFF + 64),
          "i"(OFF + 64 + ROW16), "i"(OFF + 96), "i"(OFF + 96 + ROW16)
        : "memory");
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

__device__ __forceinline__ uint4 pack_tr(i16x4 a, i16x4 b) {
    const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
    return uint4{x.x, x.y, y.x, y.y};
}

template <int D, int RT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_prefill_tile(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ ids, const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
    int num_seqs, int H, int h, int B, int top_k, int max_tiles, float c2, uint16_t *__restrict__ out,
    float *__restrict__ lse) {
    using R = Ring<D>;
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    constexpr int CPR = D / 8;   // data slots per row
    __shared__ __attribute__((aligned(16))) char ring[kStages * R::STAGE];
    __shared__ unsigned long long masks[kWin];
    __shared__ unsigned long long list_m[kWin];
    __shared__ int list_u[kWin];
    __shared__ int wave_cnt[4];

    const int G = H / h;
    const int Qt = 16 / G;                    // queries per row tile
    const int Tq = NW * RT * Qt;              // queries per workgroup (<= 64)
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
    const unsigned long long tile_bits = (1ull << Qt) - 1ull;

    const uint32_t ring0 = lds_addr(ring);
    const uint32_t list_u0 = lds_addr(list_u), list_m0 = lds_addr(list_m);
    // Per-lane read offsets inside a stage.
    const uint32_t k_rd = (uint32_t)(l16 * R::KROW + q4 * 16);
    const uint32_t v_rd = (uint32_t)(R::KBYTES + (4 * q4 + (l16 >> 2)) * R::VROW + 8 * (l16 & 3));

    // Direct global->LDS loads of one 64-token sub-block into a ring stage.
    // Each lane's element offset inside a sub-block is fixed per load slot and
    // computed once.  Pad slots read chunk 0 of their own row; for a sub-block
    // that runs past the sequence end, rows are clamped to the last valid
    // token (finite data, masked later), so no lane leaves the sequence.
    constexpr int KI = (R::KINSTR + NW - 1) / NW, VI = (R::VINSTR + NW - 1) / NW;
    uint32_t koff[KI], voff[VI];
#pragma unroll
    for (int ii = 0; ii < KI; ++ii) {
        const int slot = (ii * NW + wave) * 64 + lane;
        const int row = slot / R::KSLOT_ROW, c16 = slot % R::KSLOT_ROW;
        koff[ii] = (uint32_t)(row * h * D + (c16 < CPR ? c16 : 0) * 8);
    }
#pragma unroll
    for (int ii = 0; ii < VI; ++ii) {
        const int slot = (ii * NW + wave) * 64 + lane;
        const int row = slot / R::VSLOT_ROW, c16 = slot % R::VSLOT_ROW;
        voff[ii] = (uint32_t)(row * h * D + (c16 < CPR ? c16 : 0) * 8);
    }
    auto issue = [&](int t0, int stage) {
        char *base = ring + stage * R::STAGE;
        const bool inside = t0 + 63 < len_k;
        const size_t tok0 = (k_begin + t0) * h + g;
        const uint16_t *kb = k + tok0 * D, *vb = v + tok0 * D;
#pragma unroll
        for (int ii = 0; ii < KI; ++ii) {
            const int i = ii * NW + wave;
            if (i < R::KINSTR) {
                const uint16_t *src = kb + koff[ii];
                if (!inside) {
                    const int slot = i * 64 + lane;
                    const int row = slot / R::KSLOT_ROW, c16 = slot % R::KSLOT_ROW;
                    const int t = min(t0 + row, len_k - 1);
                    src = k + ((k_begin + t) * h + g) * D + (c16 < CPR ? c16 : 0) * 8;
                }
                __builtin_amdgcn_global_load_lds((const gbl_void *)src, (lds_void *)(base + i * 1024), 16, 0, 0);
            }
        }
#pragma unroll
        for (int ii = 0; ii < VI; ++ii) {
            const int i = ii * NW + wave;
            if (i < R::VINSTR) {
                const uint16_t *src = vb + voff[ii];
                if (!inside) {
                    const int slot = i * 64 + lane;
                    const int row = slot / R::VSLOT_ROW, c16 = slot % R::VSLOT_ROW;
                    const int t = min(t0 + row, len_k - 1);
                    src = v + ((k_begin + t) * h + g) * D + (c16 < CPR ? c16 : 0) * 8;
                }
                __builtin_amdgcn_global_load_lds((const gbl_void *)src, (lds_void *)(base + R::KBYTES + i * 1024), 16,
                                                 0, 0);
            }
        }
    };
    // Wait until only the `ahead` sub-blocks issued after this one are still in
    // flight (per-wave load counts differ: waves issue loads i = w, w+NW, ...).
    auto wait_stage = [&](int ahead) {
        const int a = ahead >= 2 ? 2 : ahead;
        switch (R::template wave_class<NW>(wave) * 3 + a) {
            case 0: wait_vm<0>(); break;
            case 1: wait_vm<R::template per_wave<NW>(0)>(); break;
            case 2: wait_vm<2 * R::template per_wave<NW>(0)>(); break;
            case 3: wait_vm<0>(); break;
            case 4: wait_vm<R::template per_wave<NW>(R::template class_rep<NW>(1))>(); break;
            case 5: wait_vm<2 * R::template per_wave<NW>(R::template class_rep<NW>(1))>(); break;
            case 6: wait_vm<0>(); break;
            case 7: wait_vm<R::template per_wave<NW>(R::template class_rep<NW>(2))>(); break;
            default: wait_vm<2 * R::template per_wave<NW>(R::template class_rep<NW>(2))>(); break;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    };

    for (int w0 = 0; w0 < e_tile; w0 += kWin) {
        if (tid < kWin) masks[tid] = 0ull;
        __syncthreads();
        // Which queries of the tile selected which block of this window.
        const int32_t *tile_ids = ids + ((size_t)(q_begin + r0) * h + g) * top_k;
        for (int e = tid; e < tq_valid * top_k; e += 64 * NW) {
            const int qi = e / top_k, a = e % top_k;
            const int j = tile_ids[(size_t)qi * h * top_k + a];
            const int pq = shift + r0 + qi;
            if (j >= w0 && j < w0 + kWin && j >= 0 && j <= pq / B) atomicOr(&masks[j - w0], 1ull << qi);
        }
        __syncthreads();
        // Compact the blocks somebody selected, ascending.
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
            list_u[base + before] = w0 + tid;
            list_m[base + before] = mv;
        }
        __syncthreads();

        const int nitems = count * nsub;
        auto t0_of = [&](int it) {
            return (int)lds_u32(list_u0 + 4 * (it / nsub)) * B + (it % nsub) * 64;
        };
#pragma unroll
        for (int x = 0; x < kStages - 1; ++x)
            if (x < nitems) issue(t0_of(x), x);

        for (int it = 0; it < nitems; ++it) {
            const int stage = it % kStages;
            wait_stage(min(kStages - 2, nitems - 1 - it));
            const int t0 = t0_of(it);
            const unsigned long long mk = lds_u64(list_m0 + 8 * (it / nsub));
            const unsigned long long wbits = mk >> (wave * RT * Qt);
            bool act[RT];
            bool any = false;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                act[rt] = ((wbits >> (rt * Qt)) & tile_bits) != 0ull;
                any |= act[rt];
            }
            const uint32_t sbase = ring0 + stage * R::STAGE;
            if (t0 <= p_last && any) {
                f32x4 sacc[RT][4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    uint4 a[KS];
                    if constexpr (KS == 4) lds_k4(a[0], a[1], a[2], a[3], sbase + k_rd + tt * 16 * R::KROW);
                    else lds_k2(a[0], a[1], sbase + k_rd + tt * 16 * R::KROW);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        if (!act[rt]) continue;
                        sacc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks)
                            sacc[rt][tt] = mfma16x16x32(as_bf16x8(a[ks]), qop[rt][ks], sacc[rt][tt]);
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
                        for (int i = 0; i < 4; ++i) hi[i] = split_bf16x2(pv[2 * i], pv[2 * i + 1], &lo[i]);
                        p_hi[rt] = as_bf16x8(uint4{hi[0], hi[1], hi[2], hi[3]});
                        p_lo[rt] = as_bf16x8(uint4{lo[0], lo[1], lo[2], lo[3]});
                    }
#pragma unroll
                    for (int dq = 0; dq < DT / 4; ++dq) {
                        i16x4 va[4], vb[4];
                        const uint32_t addr = sbase + v_rd + s2 * 32 * R::VROW;
                        if (dq == 0) lds_v4<0, 16 * R::VROW>(va, vb, addr);
                        else lds_v4<128, 16 * R::VROW>(va, vb, addr);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const int dt = dq * 4 + x;
                            const bf16x8 vop = as_bf16x8(pack_tr(va[x], vb[x]));
#pragma unroll
                            for (int rt = 0; rt < RT; ++rt) {
                                if (!act[rt]) continue;
                                o[rt][dt] = mfma16x16x32(vop, p_hi[rt], o[rt][dt]);
                                o[rt][dt] = mfma16x16x32(vop, p_lo[rt], o[rt][dt]);
                            }
                        }
                    }
                }
            }
            // refill the stage read in the previous iteration (every wave is past it)
            if (it + kStages - 1 < nitems) issue(t0_of(it + kStages - 1), (it + kStages - 1) % kStages);
        }
        wait_vm<0>();
        __syncthreads();
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

template <int D, int RT, int NW>
hipError_t launch(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *ids,
                  float scale, uint16_t *out, float *lse, hipStream_t st) {
    const int G = s.H / s.h;
    const int Tq = NW * RT * (16 / G);
    const int max_tiles = (s.max_q + Tq - 1) / Tq;
    const long grid = (long)max_tiles * s.num_seqs * s.h;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_prefill_tile<D, RT, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, st, q, k, v, ids,
                       s.cu_q, s.cu_k, s.num_seqs, s.H, s.h, s.B, s.top_k, max_tiles, scale * kLog2e, out, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const int32_t *ids, float scale, uint16_t *out, float *lse, hipStream_t st) {
    const int G = s.H / s.h;
    if (G < 1 || G > 16) return hipErrorInvalidValue;
    // 8 waves; two row tiles per wave when the tile stays within 64 queries
    // (one mask bit per query), else one; 4 waves of one tile for G = 1.
    const int qt = 16 / G;
    if (s.d == 64) {
        if (8 * 2 * qt <= 64) return launch<64, 2, 8>(s, q, k, v, ids, scale, out, lse, st);
        if (8 * qt <= 64) return launch<64, 1, 8>(s, q, k, v, ids, scale, out, lse, st);
        return launch<64, 1, 4>(s, q, k, v, ids, scale, out, lse, st);
    }
    if (s.d == 128) {
        if (8 * 2 * qt <= 64) return launch<128, 2, 8>(s, q, k, v, ids, scale, out, lse, st);
        if (8 * qt <= 64) return launch<128, 1, 8>(s, q, k, v, ids, scale, out, lse, st);
        return launch<128, 1, 4>(s, q, k, v, ids, scale, out, lse, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace msa
