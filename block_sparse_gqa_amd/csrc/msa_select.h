// Exact TopK of one row of block scores: the key helpers shared by the wave-
// and workgroup-level select kernels, and the wave-level row select.  The
// selection is the pages' per-group TopK over Block-Max-Pooled scores
// ("MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a minimal sparse
// attention"; "MiniMax Goes Sparse", section 1, step 1): the k best blocks in
// (score descending, block id ascending) order, emitted ascending.
//
// Scores map to order-preserving uint32 keys (-0.0 folded onto +0.0); the
// k-th largest key T is found bit by bit below the common prefix of the row's
// largest and smallest key, each step counting keys >= candidate with ballots;
// keys > T are kept, then the lowest-indexed keys == T.  Ids come out
// ascending: a kept key's place is counted from ballots (mbcnt).  Forced
// blocks (the first `sink` and the last `local` eligible ones) get a key above
// every score.
#pragma once

#include "msa_device.h"

namespace msa {

// Wave-wide max / min of a uint32: DPP permutations inside each row of 16
// lanes (pair swap, quad swap, half-row mirror, row mirror), then the
// permlane swaps with the lanes 16 and 32 positions away.  Every lane ends
// with the result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, dpp_u32<0xB1>(x));    // quad_perm [1,0,3,2]
    x = max(x, dpp_u32<0x4E>(x));    // quad_perm [2,3,0,1]
    x = max(x, dpp_u32<0x141>(x));   // row_half_mirror
    x = max(x, dpp_u32<0x140>(x));   // row_mirror
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)a[0], (uint32_t)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)b[0], (uint32_t)b[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    x = min(x, dpp_u32<0xB1>(x));
    x = min(x, dpp_u32<0x4E>(x));
    x = min(x, dpp_u32<0x141>(x));
    x = min(x, dpp_u32<0x140>(x));
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = min((uint32_t)a[0], (uint32_t)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return min((uint32_t)b[0], (uint32_t)b[1]);
}

// Set lanes of `mask` below this lane, plus acc.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask, uint32_t acc) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, acc));
}

// Keys of blocks t*VPT .. t*VPT+VPT-1 of a row of E scores at src: 0 past E,
// the largest key for forced blocks (the caller guarantees sink + local <=
// k).  The loads are unconditional: chunk starts past the row's
// last chunk are clamped onto it (a cache hit), so no load leaves the row's
// round_up(E, 4) floats and none waits behind a branch.
template <int VPT>
__device__ __forceinline__ void row_keys(uint32_t (&key)[VPT], const float *src, int t, int E, int sink, int local) {
    constexpr int W = VPT < 4 ? VPT : 4;       // floats per load
    const int last = (E - 1) & ~(W - 1);
    const int base = t * VPT;
    float f[VPT];
#pragma unroll
    for (int c = 0; c < VPT; c += W) {
        const int i = min(base + c, last);
        if constexpr (W == 4) {
            const float4 x = *reinterpret_cast<const float4 *>(src + i);
            f[c] = x.x; f[c + 1] = x.y; f[c + 2] = x.z; f[c + 3] = x.w;
        } else if constexpr (W == 2) {
            const float2 x = *reinterpret_cast<const float2 *>(src + i);
            f[c] = x.x; f[c + 1] = x.y;
        } else {
            f[c] = src[i];
        }
    }
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t u = __float_as_uint(f[v]);
        uint32_t kv = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
        kv = (f[v] == 0.0f) ? 0x80000000u : kv;     // -0.0 ties with +0.0
        key[v] = (base < E - v) ? kv : 0u;
    }
    if (sink | local) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int j = base + v;
            if (j < E && (j < sink || j >= E - local)) key[v] = 0xffffffffu;
        }
    }
}

// One wave (64 lanes, all active) selects the top k of the E > k block scores
// at src (16-byte aligned, round_up(E, 4) floats readable) and writes the ids
// ascending to out[0 .. k).  VPT keys per lane: E <= 64 * VPT.  E, k, sink
// and local are the same in every lane.
template <int VPT>
__device__ __forceinline__ void wave_topk_row(const float *src, int E, int k, int sink, int local, int32_t *out) {
    const int t = threadIdx.x & 63;
    uint32_t key[VPT];
    row_keys<VPT>(key, src, t, E, sink, local);

    // common prefix of the largest and smallest valid key (invalid keys are 0
    // and drop out of the min as 0 - 1)
    uint32_t mx = key[0], mnm1 = key[0] - 1u;
#pragma unroll
    for (int v = 1; v < VPT; ++v) {
        mx = max(mx, key[v]);
        mnm1 = min(mnm1, key[v] - 1u);
    }
    // Equal in every lane after the reduction; in scalar registers the search
    // below is scalar-controlled and the candidate a scalar operand.
    mx = __builtin_amdgcn_readfirstlane(wave_max_u32(mx));
    const uint32_t mn = __builtin_amdgcn_readfirstlane(wave_min_u32(mnm1)) + 1u;
    // T = largest value with count(key >= T) >= k (the k-th largest key).  All
    // valid keys share the bits above `top`; start there with zeros below.
    const int top = (mx == mn) ? -1 : 31 - __builtin_clz(mx ^ mn);
    uint32_t T = (top < 0) ? mx : (mx & ~((2u << top) - 1u));
    uint32_t m = (top < 0) ? 0u : (1u << top);   // the bit under test
    for (; m != 0u; m >>= 1) {
        // (readfirstlane keeps the search in scalar registers: the compiler
        // otherwise carries T and the bit in vector registers)
        m = __builtin_amdgcn_readfirstlane(m);
        const uint32_t cand = __builtin_amdgcn_readfirstlane(T | m);
        int c = 0;
#pragma unroll
        for (int v = 0; v < VPT; ++v) c += __builtin_popcountll(__ballot(key[v] >= cand));
        if (c >= k) {
            T = cand;
            // exactly k keys are >= T: they are the selection (the k-th and
            // (k+1)-th largest keys lie on opposite sides of T, so no tie
            // crosses it)
            if (c == k) break;
        }
    }
    bool take[VPT];
    if (m != 0u) {   // stopped early: exactly the keys >= T
#pragma unroll
        for (int v = 0; v < VPT; ++v) take[v] = key[v] >= T;
    } else {
        // T is the k-th largest key: keys > T, then the lowest-indexed == T
        int n_gt = 0;
        uint32_t eq_rank = 0;   // equal keys in lower lanes
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            n_gt += __builtin_popcountll(__ballot(key[v] > T));
            eq_rank = lanes_below(__ballot(key[v] == T), eq_rank);
        }
        const uint32_t need_eq = (uint32_t)(k - n_gt);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const bool eq = key[v] == T;
            take[v] = key[v] > T || (eq && eq_rank < need_eq);
            eq_rank += eq;
        }
    }
    // Ascending ids: a taken key's place is the number of taken keys in lower
    // lanes plus those before it in its own lane; exactly k are taken.
    uint32_t pos = 0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) pos = lanes_below(__ballot(take[v]), pos);
    const int base = t * VPT;
    char *out_b = reinterpret_cast<char *>(out);   // scalar base + 32-bit byte offset per store
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        if (take[v]) *reinterpret_cast<int32_t *>(out_b + 4u * pos++) = base + v;
}

// The narrowest instance of wave_topk_row that holds E keys (E <= 64 * VPT).
template <int VPT>
__device__ __forceinline__ void wave_topk_row_fit(const float *src, int E, int k, int sink, int local, int32_t *out) {
    if constexpr (VPT > 1) {
        if (E <= 32 * VPT) {
            wave_topk_row_fit<VPT / 2>(src, E, k, sink, local, out);
            return;
        }
    }
    wave_topk_row<VPT>(src, E, k, sink, local, out);
}

}  // namespace msa
