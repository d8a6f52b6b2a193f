// Index branch for prefill: Q_idx . K_idx^T on MFMA with the Block Max Pool
// fused into the epilogue, so token-level scores never leave registers.
//
// Method: "MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a minimal
// sparse attention" (index queries shared per GQA group, one index-key head
// shared by all heads, Block Max Pool of token scores); "MiniMax Goes Sparse",
// section 1, step 1.
//
// Work decomposition.  A workgroup (4 waves) owns 4*64 "columns"; a column is
// one (query, group) pair, so one staged K_idx tile serves every group of
// every query of the tile (the index key has a single head).  Keys run along
// the MFMA M dimension (v_mfma_f32_32x32x16_bf16): each lane then holds one
// column and 16 keys of a 32-key tile, the block max is an in-register max
// plus one permlane32 swap.  K_idx tiles are double-buffered in LDS; the
// block scores of 32 consecutive blocks are staged in LDS and written to the
// [row, group, block] workspace as whole 128-byte lines, eight lanes per line.
#include <type_traits>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kWaves = 4;
constexpr int kCols = 64;     // columns per wave
constexpr int kStage = 32;    // blocks per staged flush: one 128-byte line of scores per column

// Three workgroups per CU for B = 64 (168 VGPRs, 52 KB of LDS each): with a
// bound of two the compiler spends 212 VGPRs and only two waves share a SIMD
// (32K prefill index_topk 0.72 against 0.755 ms).  B = 128 keeps two: its
// 71 KB of LDS admit no third workgroup.
template <int DI, int B>
__global__ __launch_bounds__(256, B == 64 ? 3 : 2) void index_prefill_blockmax(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int h,
    float *__restrict__ scores, int e_stride, int row0, int row1) {
    // Only the packed rows [row0, row1) are scored; scores holds their rows
    // from row0 on.
    constexpr int ROWB = DI * 2 + 16;          // padded LDS row (bytes)
    constexpr int KS = DI / 16;                // 16-dim k-steps
    constexpr int MT = B / 32;                 // 32-key tiles per block
    constexpr int CPR = DI / 8;                // 16-byte chunks per key row
    constexpr int CHUNKS = B * CPR;
    constexpr int PASSES = (CHUNKS + 255) / 256;

    __shared__ __attribute__((aligned(16))) char ktile[2][B * ROWB];
    __shared__ float stage[kWaves][kCols][kStage + 1];

    const int s = blockIdx.y;
    const int q_begin = cu_q[s], len_q = cu_q[s + 1] - q_begin;
    const int k_begin = cu_k[s], len_k = cu_k[s + 1] - k_begin;
    const int qw = kCols / h;                  // queries per wave
    const int tq = qw * kWaves;                // queries per workgroup
    const int tile = gridDim.x - 1 - blockIdx.x;   // heaviest (latest) tiles first
    const int r0 = tile * tq;
    if (r0 >= len_q) return;
    if (q_begin + r0 >= row1 || q_begin + min(r0 + tq, len_q) <= row0) return;   // no row of the chunk

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int shift = len_k - len_q;           // position of row r is shift + r
    const int r_last = min(r0 + tq, len_q) - 1;
    const int p_first = shift + r0;
    const int nblk = (shift + r_last) / B + 1;

    // This lane's two columns (one per 32-wide N tile) and their Q_idx operands.
    bf16x8 qop[2][KS];
    int col_p[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int c = nt * 32 + (lane & 31);
        const int r = r0 + wave * qw + c / h;
        const int g = c % h;
        const bool ok = (c < qw * h) && (r < len_q);
        col_p[nt] = ok ? shift + r : -1;   // rows outside the chunk are scored but not written
        const uint16_t *src = q_idx + ((size_t)(q_begin + r) * h + g) * DI + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[nt][ks] = as_bf16x8(load16_if(src + 16 * ks, ok, q_idx));
    }

    // Tile prefetch: plain loads (no select on the loaded value, which would
    // make the wave wait for them right away); rows past the sequence end
    // repeat its last key and are masked with the diagonal blocks.
    // CHUNKS is a multiple of 256 for every supported (d_idx, B).
    static_assert(CHUNKS % 256 == 0, "tile chunks must fill whole passes");
    uint4 pre[PASSES];
    // The sequence's keys from a scalar base; each load's offset is a 32-bit
    // byte offset (a sequence's K_idx stays far below 4 GB).
    const char *kseq = reinterpret_cast<const char *>(k_idx + (size_t)k_begin * DI);
    auto gload = [&](int j) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int ci = ps * 256 + tid;
            const int row = ci / CPR, c8 = ci % CPR;
            const int t = min(j * B + row, len_k - 1);
            pre[ps] = load16(kseq + (unsigned)(t * (2 * DI) + c8 * 16));
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int ci = ps * 256 + tid;
            const int row = ci / CPR, c8 = ci % CPR;
            *reinterpret_cast<uint4 *>(&ktile[buf][row * ROWB + c8 * 16]) = pre[ps];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    // One key block: scores on MFMA, Block Max Pool, staged flush.  MASK is
    // needed only on the diagonal blocks, where some key follows some column.
    auto step = [&](int j, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int buf = j & 1;
        if (j + 1 < nblk) gload(j + 1);

        f32x16 acc[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                a[mt] = *reinterpret_cast<const bf16x8 *>(
                    &ktile[buf][(mt * 32 + (lane & 31)) * ROWB + (16 * ks + 8 * (lane >> 5)) * 2]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32x32x16(a[mt], qop[nt][ks], acc[mt][nt]);
        }

        // Block Max Pool: keys after a column's position are not visible.
        const int slot = j % kStage;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float m = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float v = acc[mt][nt][i];
                    if constexpr (MASK) {
                        const int t = j * B + mt * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                        if (t > col_p[nt]) v = -INFINITY;
                    }
                    m = fmaxf(m, v);
                }
            m = max_xor32(m);
            if (lane < 32) stage[wave][nt * 32 + lane][slot] = m;
        }

        if (slot == kStage - 1 || j == nblk - 1) {
            wave_lds_sync();
            const int j0 = j - slot;
            // The wave's earliest row has the fewest blocks: if even it holds
            // all kStage of them, every column's run is one whole 128-byte
            // line, and each store instruction writes eight such lines (eight
            // lanes per column), so memory sees whole lines rather than
            // 16-byte pieces.
            if ((shift + r0 + wave * qw) / B + 1 >= j0 + kStage) {
#pragma unroll
                for (int it = 0; it < kCols / 8; ++it) {
                    const int c = it * 8 + (lane >> 3), ch = lane & 7;
                    const int r = r0 + wave * qw + c / h;
                    const int g = c % h;
                    if (c < qw * h && r < len_q && q_begin + r >= row0 && q_begin + r < row1) {
                        const float *src = &stage[wave][c][4 * ch];
                        *reinterpret_cast<float4 *>(scores + ((size_t)(q_begin + r - row0) * h + g) * e_stride + j0 +
                                                    4 * ch) = make_float4(src[0], src[1], src[2], src[3]);
                    }
                }
            } else {
                const int c = lane;
                const int r = r0 + wave * qw + c / h;
                const int g = c % h;
                if (c < qw * h && r < len_q && q_begin + r >= row0 && q_begin + r < row1) {
                    const int E = (shift + r) / B + 1;
                    const int n = min(kStage, E - j0);
                    float *dst = scores + ((size_t)(q_begin + r - row0) * h + g) * e_stride + j0;
                    const float *src = stage[wave][c];
                    for (int x = 0; x < n; ++x) dst[x] = src[x];
                }
            }
            wave_lds_sync();
        }

        if (j + 1 < nblk) lstore(buf ^ 1);
        __syncthreads();
    };
    // blocks [0, j_full) are entirely visible to every column of the tile
    const int j_full = min(nblk, (p_first + 1) / B);
    int j = 0;
    for (; j < j_full; ++j) step(j, std::false_type{});
    for (; j < nblk; ++j) step(j, std::true_type{});
}

template <int DI, int B>
hipError_t launch(const Shape &s, const uint16_t *q_idx, const uint16_t *k_idx, float *scores, hipStream_t st) {
    const int tq = (kCols / s.h) * kWaves;
    dim3 grid((s.max_q + tq - 1) / tq, s.num_seqs);
    hipLaunchKernelGGL((index_prefill_blockmax<DI, B>), grid, dim3(256), 0, st, q_idx, k_idx, s.cu_q, s.cu_k,
                       s.h, scores, score_stride(s), s.row0, s.row0 + s.rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_prefill(const Shape &s, const uint16_t *q_idx, const uint16_t *k_idx, float *scores,
                                hipStream_t st) {
    if (s.d_idx == 32 && s.B == 64) return launch<32, 64>(s, q_idx, k_idx, scores, st);
    if (s.d_idx == 32 && s.B == 128) return launch<32, 128>(s, q_idx, k_idx, scores, st);
    if (s.d_idx == 64 && s.B == 64) return launch<64, 64>(s, q_idx, k_idx, scores, st);
    if (s.d_idx == 64 && s.B == 128) return launch<64, 128>(s, q_idx, k_idx, scores, st);
    return hipErrorInvalidValue;
}

}  // namespace msa
