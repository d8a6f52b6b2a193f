// Index branch for decode: one query per sequence scans the whole index-key
// cache.  Bandwidth-bound: every K_idx byte is read once and scored against
// all h index queries of the sequence at the same time (the index key has a
// single head: "MiniMax Goes Sparse", section 1, step 1; the decode scan
// touching the full length is discussed in section 3).
//
// Tokens run along the MFMA M dimension of v_mfma_f32_16x16x32_bf16 and the
// h groups along N, so each lane holds 4 tokens of one group per 16-token
// tile; the Block Max Pool is an in-register max over the block's tiles plus
// two lane swaps (xor 16, xor 32).  K_idx operands are loaded straight from
// HBM with 16-byte loads, 16 tokens x 128 bytes per tile: fully coalesced.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

template <int DI, int B>
__global__ __launch_bounds__(256) void index_decode_blockmax(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int h,
    float *__restrict__ scores, int e_stride, int blocks_per_wg) {
    constexpr int KS = DI / 32;   // 32-dim k-steps
    constexpr int TT = B / 16;    // 16-token tiles per block

    const int s = blockIdx.y;
    const int row = cu_q[s + 1] - 1;                  // the sequence's (last) query
    const int k_begin = cu_k[s], len_k = cu_k[s + 1] - k_begin;
    const int p = len_k - 1;
    const int E = p / B + 1;
    const int j_begin = blockIdx.x * blocks_per_wg;
    if (j_begin >= E) return;
    const int j_end = min(E, j_begin + blocks_per_wg);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 15, q4 = lane >> 4;

    bf16x8 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qop[ks] = as_bf16x8(load16_if(q_idx + ((size_t)row * h + g) * DI + 32 * ks + 8 * q4, g < h, q_idx));

    for (int j = j_begin + wave; j < j_end; j += 4) {
        uint4 a[TT][KS];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int t = j * B + tt * 16 + g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a[tt][ks] = load16_if(k_idx + (size_t)(k_begin + t) * DI + 32 * ks + 8 * q4, t < len_k, k_idx);
        }
        float m = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(as_bf16x8(a[tt][ks]), qop[ks], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = j * B + tt * 16 + 4 * q4 + i;
                m = fmaxf(m, t <= p ? acc[i] : -INFINITY);
            }
        }
        m = max_xor16(m);
        m = max_xor32(m);
        if (lane < h) scores[((size_t)row * h + lane) * e_stride + j] = m;
    }
}

template <int DI, int B>
hipError_t launch(const Shape &s, const uint16_t *q_idx, const uint16_t *k_idx, float *scores, hipStream_t st) {
    const int e_max = (s.max_k + s.B - 1) / s.B;
    long total_blocks = (long)e_max * s.num_seqs;
    int bpw = (int)((total_blocks + 2047) / 2048);
    bpw = (bpw + 3) / 4 * 4;
    bpw = bpw < 4 ? 4 : (bpw > 64 ? 64 : bpw);
    dim3 grid((e_max + bpw - 1) / bpw, s.num_seqs);
    hipLaunchKernelGGL((index_decode_blockmax<DI, B>), grid, dim3(256), 0, st, q_idx, k_idx, s.cu_q, s.cu_k, s.h,
                       scores, score_stride(s), bpw);
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
