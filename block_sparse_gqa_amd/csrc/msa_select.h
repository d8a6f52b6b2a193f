// Wave-level exact TopK of one row of block scores (device code shared by the
// select kernel and the scoring kernel's fused tail).  The selection is the
// pages' per-group TopK over Block-Max-Pooled scores ("MiniMax M3 MSA vs Step
// 3.7 Flash MFA", section "MSA: a minimal sparse attention"; "MiniMax Goes
// Sparse", section 1, step 1): the k best blocks in (score descending, block
// id ascending) order, emitted ascending.
//
// Scores map to order-preserving uint32 keys (-0.0 folded onto +0.0); the
// k-th largest key T is found bit by bit below the common prefix of the row's
// largest and smallest key, each step counting keys >= candidate with ballots;
// keys > T are kept, then the lowest-indexed keys == T.  Forced blocks (the
// first `sink` and the last `local` eligible ones) get a key above every score.
#pragma once

#include "msa_device.h"

namespace msa {

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

// One wave (64 lanes, all active) selects the top k of the E > k block scores
// at src (16-byte aligned) and writes the ids ascending to out[0 .. k).
// VPT keys per lane: E <= 64 * VPT.
template <int VPT>
__device__ __forceinline__ void wave_topk_row(const float *src, int E, int k, int sink, int local, int32_t *out) {
    const int t = threadIdx.x & 63;
    uint32_t key[VPT];
    load_keys<VPT>(key, src, t, E, sink, local);

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

}  // namespace msa
