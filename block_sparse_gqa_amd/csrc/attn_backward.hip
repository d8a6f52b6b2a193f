// Backward of the sparse branch, prefill, with the selection held fixed.
// The pages define the forward pass only (sparse attention over the
// selected blocks of the original K/V: "MiniMax Goes Sparse", section 1,
// step 2; "MiniMax M3 MSA vs Step 3.7 Flash MFA", section "MSA: a minimal
// sparse attention"); whether training uses a hard or a soft top-k is an
// open point there (same page, section on waiting for the technical
// report).  This is the plain gradient with the ids as constants:
//     P_t = exp(scale q.k_t - lse),  dP_t = dO.v_t,  D = dO.O,
//     dS_t = P_t (dP_t - D),
//     dq = scale sum_t dS_t k_t,  dk_t += scale dS_t q,  dv_t += P_t dO.
//
// Key-centric schedule.  dk and dv of a key block need every (query, head)
// that selected it, so the query-centric ids are first turned into one list
// of selecting queries per (group, block) (block_lists.hip; each list is
// sorted, so the dk/dv sums run in a fixed order).  One workgroup then
// owns one (group, block): K and V of the block sit in LDS, dk and dv in
// registers, and the selecting queries stream through in chunks of up to 32
// (query, head) rows.  For each chunk and 16-token tile:
//     S  = Q . K^T,  dP = dO . V^T        A = Q / dO rows, B = K / V rows (LDS)
//     dV += P^T . dO,  dK += dS^T . Q     A = P^T / dS^T straight from the
//                                         S / dP accumulators, B = dO / Q read
//                                         with the transposing LDS read
//     dQ^T = K^T . dS^T                   A = K^T (transposing read), B = dS
//                                         staged in LDS; written as a bf16
//                                         partial per (row, selected slot).
// A last pass sums each row's partials into dq (no atomics: float32 atomic
// adds of every partial element ran at a small fraction of HBM speed).
#include <algorithm>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kRows = 32;                 // (query, head) rows per chunk
constexpr int kRowStride = 288;           // LDS row stride of K, V, Q, dO (bytes; 32 mod 256: conflict free)

// delta[row, head] = dO . O (float32).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep(const uint16_t *__restrict__ out, const uint16_t *__restrict__ dout,
                                                long n_rows, float *__restrict__ delta) {
    constexpr int PER = D / 64;   // elements per lane
    const long rh = (long)blockIdx.x * 4 + (threadIdx.x >> 6);   // (row, head) pair
    if (rh >= n_rows) return;
    const int lane = threadIdx.x & 63;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const size_t idx = (size_t)rh * D + lane * PER + i;
        s += bf16_to_f32(out[idx]) * bf16_to_f32(dout[idx]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) delta[rh] = s;
}

// Transposing reads of rows r0 + 4*q4 .. +3 and r0 + 16 + 4*q4 .. +3 of a
// row-major bf16 tile (row stride kRowStride), column 16*ct + (lane % 16):
// the 8 values of an MFMA operand whose k slots 8*q4 + i are those rows.
__device__ __forceinline__ bf16x8 tr_rows(const char *tile, int r0, int ct) {
    const int lane = lane_id(), l16 = lane & 15, q4 = lane >> 4;
    const char *p = tile + (r0 + 4 * q4 + (l16 >> 2)) * kRowStride + 8 * (l16 & 3) + 32 * ct;
    const i16x4 a = lds_read_tr16(p);
    const i16x4 b = lds_read_tr16(p + 16 * kRowStride);
    const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
    return as_bf16x8(uint4{x.x, x.y, y.x, y.y});
}

// Row `r` of a row-major bf16 tile, 8 values at column 8 * c8.
__device__ __forceinline__ bf16x8 row8(const char *tile, int r, int c8) {
    return *reinterpret_cast<const bf16x8 *>(tile + r * kRowStride + 16 * c8);
}

template <int D, int B>
__global__ __launch_bounds__(256, B == 64 ? 2 : 1) void bwd_block(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, const int32_t *__restrict__ blk_off,
    const int32_t *__restrict__ off, const int32_t *__restrict__ entries, int num_seqs, int H, int h, int nb_max,
    int top_k, int row0, float scale, float c2, uint16_t *__restrict__ dq_part, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv, float *__restrict__ dk_acc, float *__restrict__ dv_acc) {
    // The list entries are (row - row0) * top_k + slot for the rows of one
    // chunk, and dq_part holds that chunk's rows.  dk_acc / dv_acc (float32,
    // [total_k, h, d]) are null for a problem run in one chunk, where dk and
    // dv are written as bf16 directly; otherwise each chunk adds its share
    // there (a workgroup owns its block's rows within a launch).
    constexpr int KS = D / 32;           // 32-wide k steps over d
    constexpr int DT = D / 16;           // 16-wide d tiles
    constexpr int TPW = B / 64;          // 16-token tiles per wave
    constexpr int DS_STRIDE = B * 2 + 16;
    __shared__ __attribute__((aligned(16))) char kt[B * kRowStride];
    __shared__ __attribute__((aligned(16))) char vt[B * kRowStride];
    __shared__ __attribute__((aligned(16))) char qc[kRows * kRowStride];
    __shared__ __attribute__((aligned(16))) char doc[kRows * kRowStride];
    __shared__ __attribute__((aligned(16))) char dst[kRows * DS_STRIDE];      // dS, bf16 head
    __shared__ __attribute__((aligned(16))) char dst_lo[kRows * DS_STRIDE];   // dS, bf16 tail
    // per-row data of the current and the next chunk
    __shared__ int r_row[2][kRows], r_slot[2][kRows], r_pos[2][kRows];
    __shared__ float r_lse2[2][kRows], r_delta[2][kRows];

    const int gb = blockIdx.x, g = blockIdx.y;
    if (gb >= blk_off[num_seqs]) return;
    // sequence and block of this workgroup
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (blk_off[mid] <= gb) lo = mid; else hi = mid - 1;
    }
    const int s = lo, j = gb - blk_off[s];
    const int k_begin = cu_k[s], len_k = cu_k[s + 1] - k_begin;
    const int q_begin = cu_q[s], shift = len_k - (cu_q[s + 1] - q_begin);
    const int G = H / h;
    const int qpc = kRows / G;                   // queries per chunk
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loops over tiles
    const int l16 = lane & 15, q4 = lane >> 4;
    const int t_valid = min(B, len_k - j * B);   // tokens of the block inside the sequence

    // K and V rows of the block (zeros past the sequence end).
    for (int c = tid; c < B * (D / 8); c += 256) {
        const int t = c / (D / 8), c8 = c % (D / 8);
        uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (t < t_valid) {
            const size_t src = ((size_t)(k_begin + j * B + t) * h + g) * D + c8 * 8;
            kv = load16(k + src);
            vv = load16(v + src);
        }
        *reinterpret_cast<uint4 *>(kt + t * kRowStride + 16 * c8) = kv;
        *reinterpret_cast<uint4 *>(vt + t * kRowStride + 16 * c8) = vv;
    }

    f32x4 dka[TPW][DT], dva[TPW][DT];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            dka[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dva[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const long key = (long)g * nb_max + gb;
    const int e0 = off[key], e1 = off[key + 1];
    const int nchunks = (e1 - e0 + qpc - 1) / qpc;

    // Chunk c covers entries e0 + c*qpc ..; row r of a chunk is its query
    // r / G, head g*G + r % G.  Row data of chunk c+2 and the Q / dO rows of
    // chunk c+1 are loaded into registers while chunk c is computed.
    int i_row = -1, i_slot = 0, i_pos = -1;
    float i_lse2 = INFINITY, i_dlt = 0.f;
    auto load_info = [&](int c) {   // threads < kRows
        const int c0 = e0 + c * qpc;
        const int qi = tid / G, hd = tid % G;
        const bool ok = qi < min(qpc, e1 - c0) && tid < qpc * G;
        const int e = ok ? entries[c0 + qi] : 0;
        i_row = ok ? row0 + e / top_k : -1;
        i_slot = e % top_k;
        i_pos = ok ? shift + (i_row - q_begin) : -1;
        const size_t ix = (size_t)max(i_row, 0) * H + g * G + hd;
        const float l = lse[ix], dl = delta[ix];   // row 0 stands in for unused rows
        i_lse2 = ok ? l * kLog2e : INFINITY;
        i_dlt = ok ? dl : 0.f;
    };
    auto store_info = [&](int buf) {
        r_row[buf][tid] = i_row;
        r_slot[buf][tid] = i_slot;
        r_pos[buf][tid] = i_pos;
        r_lse2[buf][tid] = i_lse2;
        r_delta[buf][tid] = i_dlt;
    };
    constexpr int QCH = kRows * (D / 8) / 256;   // 16-byte chunks per thread per tile
    uint4 pq[QCH], pd[QCH];
    auto load_tiles = [&](int buf) {
#pragma unroll
        for (int x = 0; x < QCH; ++x) {
            const int c = x * 256 + tid, r = c / (D / 8), c8 = c % (D / 8);
            const int row = r_row[buf][r];
            const size_t src = row >= 0 ? ((size_t)row * H + g * G + r % G) * D + c8 * 8 : 0;
            pq[x] = load16(q + src);
            pd[x] = load16(dout + src);
        }
    };
    auto store_tiles = [&](int buf) {   // unused rows are stored as zeros
#pragma unroll
        for (int x = 0; x < QCH; ++x) {
            const int c = x * 256 + tid, r = c / (D / 8), c8 = c % (D / 8);
            const uint32_t m = r_row[buf][r] >= 0 ? 0xffffffffu : 0u;   // per-word mask (no select of whole vectors)
            *reinterpret_cast<uint4 *>(qc + r * kRowStride + 16 * c8) =
                uint4{pq[x].x & m, pq[x].y & m, pq[x].z & m, pq[x].w & m};
            *reinterpret_cast<uint4 *>(doc + r * kRowStride + 16 * c8) =
                uint4{pd[x].x & m, pd[x].y & m, pd[x].z & m, pd[x].w & m};
        }
    };

    if (nchunks > 0) {
        if (tid < kRows) {
            load_info(0);
            store_info(0);
            if (nchunks > 1) {
                load_info(1);
                store_info(1);
            }
        }
        __syncthreads();
        load_tiles(0);
        store_tiles(0);
        __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
        const int cur = c & 1;
        // the row-data loads go first: their dependent loads then wait only
        // for them, not for the Q / dO prefetch issued after
        if (tid < kRows && c + 2 < nchunks) load_info(c + 2);
        if (c + 1 < nchunks) load_tiles(cur ^ 1);

        // this lane's rows 16*mt + 4*q4 + i
        float lse2[2][4], dlt[2][4];
        int pos[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * q4 + i;
                lse2[mt][i] = r_lse2[cur][r];
                dlt[mt][i] = r_delta[cur][r];
                pos[mt][i] = r_pos[cur][r];
            }

#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tt = wave + 4 * u;          // 16-token tile of the block
            f32x4 sa[2], pa[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                sa[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                pa[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 kb = row8(kt, 16 * tt + l16, 4 * ks + q4);
                    const bf16x8 vb = row8(vt, 16 * tt + l16, 4 * ks + q4);
                    sa[mt] = mfma16x16x32(row8(qc, 16 * mt + l16, 4 * ks + q4), kb, sa[mt]);
                    pa[mt] = mfma16x16x32(row8(doc, 16 * mt + l16, 4 * ks + q4), vb, pa[mt]);
                }
            }
            // P and dS for token 16*tt + l16 and the lane's 8 rows
            const int t_abs = j * B + 16 * tt + l16;
            float pv[2][4], dsv[2][4];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool vis = t_abs <= pos[mt][i];
                    const float p = vis ? fast_exp2(fmaf(sa[mt][i], c2, -lse2[mt][i])) : 0.f;
                    pv[mt][i] = p;
                    dsv[mt][i] = p * (pa[mt][i] - dlt[mt][i]);
                }
            // A operands: k slot 8*q4 + i <- row 4*q4 + i (i < 4), row 16 + 4*q4 + i - 4.
            // P and dS enter the products as a bf16 head plus a bf16 tail
            // (x = head + tail to 2^-17 |x|), so their rounding stays far
            // below that of the bf16 outputs; dO, Q and K are bf16 inputs and
            // exact as they are.
            uint32_t pl[4], dl[4];
            const uint32_t ph[4] = {split_bf16x2(pv[0][0], pv[0][1], &pl[0]), split_bf16x2(pv[0][2], pv[0][3], &pl[1]),
                                    split_bf16x2(pv[1][0], pv[1][1], &pl[2]), split_bf16x2(pv[1][2], pv[1][3], &pl[3])};
            const uint32_t dh[4] = {split_bf16x2(dsv[0][0], dsv[0][1], &dl[0]),
                                    split_bf16x2(dsv[0][2], dsv[0][3], &dl[1]),
                                    split_bf16x2(dsv[1][0], dsv[1][1], &dl[2]),
                                    split_bf16x2(dsv[1][2], dsv[1][3], &dl[3])};
            const bf16x8 pA = as_bf16x8(uint4{ph[0], ph[1], ph[2], ph[3]});
            const bf16x8 pAl = as_bf16x8(uint4{pl[0], pl[1], pl[2], pl[3]});
            const bf16x8 dsA = as_bf16x8(uint4{dh[0], dh[1], dh[2], dh[3]});
            const bf16x8 dsAl = as_bf16x8(uint4{dl[0], dl[1], dl[2], dl[3]});
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 dob = tr_rows(doc, 0, dt), qb = tr_rows(qc, 0, dt);
                dva[u][dt] = mfma16x16x32(pA, dob, dva[u][dt]);
                dka[u][dt] = mfma16x16x32(dsA, qb, dka[u][dt]);
                dva[u][dt] = mfma16x16x32(pAl, dob, dva[u][dt]);
                dka[u][dt] = mfma16x16x32(dsAl, qb, dka[u][dt]);
            }
            // dS (head and tail) to LDS, [row][token], for the dq products
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int at = (16 * mt + 4 * q4 + i) * DS_STRIDE + 2 * (16 * tt + l16);
                    const uint32_t w = dh[2 * mt + (i >> 1)], wl = dl[2 * mt + (i >> 1)];
                    *reinterpret_cast<uint16_t *>(dst + at) = (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu));
                    *reinterpret_cast<uint16_t *>(dst_lo + at) = (uint16_t)((i & 1) ? (wl >> 16) : (wl & 0xffffu));
                }
        }
        __syncthreads();

        // dQ^T = K^T . dS^T: output tile (d tile dt, row tile mt), k = the B tokens
        for (int ti = wave; ti < DT * 2; ti += 4) {
            const int dt = ti >> 1, mt = ti & 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s32 = 0; s32 < B / 32; ++s32) {
                const bf16x8 a = tr_rows(kt, 32 * s32, dt);
                const int at = (16 * mt + l16) * DS_STRIDE + 2 * (32 * s32 + 4 * q4);
                const uint2 lo2 = *reinterpret_cast<const uint2 *>(dst + at);
                const uint2 hi2 = *reinterpret_cast<const uint2 *>(dst + at + 32);
                const uint2 lo2t = *reinterpret_cast<const uint2 *>(dst_lo + at);
                const uint2 hi2t = *reinterpret_cast<const uint2 *>(dst_lo + at + 32);
                acc = mfma16x16x32(a, as_bf16x8(uint4{lo2.x, lo2.y, hi2.x, hi2.y}), acc);
                acc = mfma16x16x32(a, as_bf16x8(uint4{lo2t.x, lo2t.y, hi2t.x, hi2t.y}), acc);
            }
            const int r = 16 * mt + l16;
            const int row = r_row[cur][r];
            if (row >= 0) {
                uint16_t *dstq = dq_part + (((size_t)(row - row0) * top_k + r_slot[cur][r]) * H + g * G + r % G) * D +
                                 16 * dt + 4 * q4;
                *reinterpret_cast<uint2 *>(dstq) =
                    uint2{pack_bf16x2(acc[0] * scale, acc[1] * scale), pack_bf16x2(acc[2] * scale, acc[3] * scale)};
            }
        }
        __syncthreads();   // every read of this chunk's tiles and row data is done
        if (c + 1 < nchunks) store_tiles(cur ^ 1);
        if (tid < kRows && c + 2 < nchunks) store_info(cur);
        __syncthreads();
    }

    // dk, dv of the block's tokens of group g (bf16)
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tt = wave + 4 * u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * tt + 4 * q4 + i;
            if (t >= t_valid) continue;
            const size_t rowbase = ((size_t)(k_begin + j * B + t) * h + g) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const size_t idx = rowbase + 16 * dt + l16;
                if (dk_acc != nullptr) {
                    dk_acc[idx] += dka[u][dt][i] * scale;
                    dv_acc[idx] += dva[u][dt][i];
                } else {
                    dk[idx] = (uint16_t)(pack_bf16x2(dka[u][dt][i] * scale, 0.f) & 0xffffu);
                    dv[idx] = (uint16_t)(pack_bf16x2(dva[u][dt][i], 0.f) & 0xffffu);
                }
            }
        }
    }
}

// dq[row, head] = sum of the row's partials over its valid selected slots.
// One wave per (row, head): lane = (slot lane group, 16-byte chunk of the
// row), so every load instruction reads whole partial rows; the slot groups
// are then summed with lane swaps.
template <int D>
__global__ __launch_bounds__(256) void bwd_finish(const uint16_t *__restrict__ dq_part, const int32_t *__restrict__ ids,
                                                  const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
                                                  int num_seqs, int row0, long n_rows, int H, int h, int B,
                                                  int top_k, uint16_t *__restrict__ dq) {
    // rows [row0, row0 + n_rows / H) of one chunk; dq_part holds those rows
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int NSO = 64 / CPR;     // slot lane groups
    const long rh0 = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rh0 >= n_rows) return;
    const int lane = threadIdx.x & 63, c = lane % CPR, so = lane / CPR;
    const int rr = (int)(rh0 / H), head = (int)(rh0 % H), g = head / (H / h);
    const int row = row0 + rr;
    const long rh = (long)row * H + head;
    const int s = seq_of_row(cu_q, num_seqs, row);
    const int p = (cu_k[s + 1] - cu_k[s]) - (cu_q[s + 1] - cu_q[s]) + (row - cu_q[s]);
    const int32_t *sel = ids + ((size_t)row * h + g) * top_k;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 4
    for (int a = so; a < top_k; a += NSO) {
        const int j = sel[a];
        const bool ok = j >= 0 && j <= p / B;
        const uint4 x = load16(dq_part + (((size_t)rr * top_k + (ok ? a : 0)) * H + head) * D + 8 * c);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += ok ? __uint_as_float(w[i] << 16) : 0.f;
            acc[2 * i + 1] += ok ? __uint_as_float(w[i] & 0xffff0000u) : 0.f;
        }
    }
#pragma unroll
    for (int m = CPR; m < 64; m <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], m, 64);
    if (so == 0)
        *reinterpret_cast<uint4 *>(dq + (size_t)rh * D + 8 * c) =
            uint4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                  pack_bf16x2(acc[6], acc[7])};
}

// float32 dk, dv -> bf16 (a problem run in several chunks).
__global__ __launch_bounds__(256) void bwd_kv_out(const float *__restrict__ dk_acc, const float *__restrict__ dv_acc,
                                                  long n, uint16_t *__restrict__ dk, uint16_t *__restrict__ dv) {
    for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 2; i < n; i += (long)gridDim.x * 512) {
        const float2 a = *reinterpret_cast<const float2 *>(dk_acc + i);
        const float2 b = *reinterpret_cast<const float2 *>(dv_acc + i);
        *reinterpret_cast<uint32_t *>(dk + i) = pack_bf16x2(a.x, a.y);
        *reinterpret_cast<uint32_t *>(dv + i) = pack_bf16x2(b.x, b.y);
    }
}

__global__ __launch_bounds__(256) void fill_zero_f32(float *__restrict__ p, long n) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) p[i] = 0.f;
}

// Workspace: the block lists of one chunk, delta of every row, the chunk's dq
// partials, and (several chunks only) float32 dk and dv.
struct BwdWs {
    BlockLists lists;
    size_t delta, dq_part, dk_acc, dv_acc, bytes;
};

BwdWs bwd_ws(const Shape &s, bool acc) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    BwdWs w;
    w.lists = block_lists_layout(s);
    size_t at = w.lists.bytes;
    w.delta = at;
    at += al((size_t)s.total_q * s.H * sizeof(float));
    w.dq_part = at;
    at += al((size_t)s.rows * s.top_k * s.H * s.d * sizeof(uint16_t));
    w.dk_acc = w.dv_acc = 0;
    if (acc) {
        const size_t kv = al((size_t)s.total_k * s.h * s.d * sizeof(float));
        w.dk_acc = at;
        at += kv;
        w.dv_acc = at;
        at += kv;
    }
    w.bytes = at;
    return w;
}

// Rows per chunk: the whole problem if its workspace fits the cap, else as
// many as fit next to the float32 dk / dv accumulators.
int bwd_chunk_rows(const Shape &s) {
    Shape one = s;
    one.rows = 1;
    const size_t per_row = (size_t)s.h * s.top_k * 8 + (size_t)s.top_k * s.H * s.d * 2;
    Shape all = s;
    all.rows = s.total_q;
    if (bwd_ws(all, false).bytes <= workspace_cap()) return s.total_q;
    return chunk_rows(s, bwd_ws(one, true).bytes - per_row, per_row);
}

template <int D, int B>
hipError_t launch_bwd(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *ids,
                      float scale, const uint16_t *out, const float *lse, const uint16_t *dout, uint16_t *dq,
                      uint16_t *dk, uint16_t *dv, void *ws, hipStream_t st) {
    const int per = bwd_chunk_rows(s);
    const bool chunked = per < s.total_q;
    Shape c0 = s;
    c0.rows = per;
    const BwdWs wl = bwd_ws(c0, chunked);   // the largest chunk: delta and the accumulators sit where it puts them
    char *base = static_cast<char *>(ws);
    float *delta = reinterpret_cast<float *>(base + wl.delta);
    uint16_t *dq_part = reinterpret_cast<uint16_t *>(base + wl.dq_part);
    float *dk_acc = chunked ? reinterpret_cast<float *>(base + wl.dk_acc) : nullptr;
    float *dv_acc = chunked ? reinterpret_cast<float *>(base + wl.dv_acc) : nullptr;
    auto grid_of = [](long n, long per_wg) { return dim3((unsigned)((n + per_wg - 1) / per_wg)); };
    const long rows_all = (long)s.total_q * s.H;
    hipLaunchKernelGGL((bwd_prep<D>), grid_of(rows_all, 4), dim3(256), 0, st, out, dout, rows_all, delta);
    const long kv = (long)s.total_k * s.h * s.d;
    if (chunked) {
        hipLaunchKernelGGL(fill_zero_f32, grid_of(std::min(kv, 1L << 22), 256), dim3(256), 0, st, dk_acc, kv);
        hipLaunchKernelGGL(fill_zero_f32, grid_of(std::min(kv, 1L << 22), 256), dim3(256), 0, st, dv_acc, kv);
    }
    for (int r0 = 0; r0 < s.total_q; r0 += per) {
        Shape c = s;
        c.row0 = r0;
        c.rows = std::min(per, s.total_q - r0);
        // the chunk's lists sit at the start of the workspace (their size
        // grows with the rows, so a short last chunk fits where the first did)
        const BlockLists lists = block_lists_layout(c);
        const int32_t *blk_off = reinterpret_cast<const int32_t *>(base + lists.blk_off);
        const int32_t *off = reinterpret_cast<const int32_t *>(base + lists.off);
        const int32_t *entries = reinterpret_cast<const int32_t *>(base + lists.entries);
        // sorted lists: dk and dv then sum in a fixed order, bitwise reproducible
        const hipError_t e = launch_block_lists(c, ids, lists, base, st, true);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_block<D, B>), dim3((unsigned)lists.nb_max, s.h), dim3(256), 0, st, q, k, v, dout, lse,
                           delta, s.cu_q, s.cu_k, blk_off, off, entries, s.num_seqs, s.H, s.h, (int)lists.nb_max,
                           s.top_k, c.row0, scale, scale * kLog2e, dq_part, dk, dv, dk_acc, dv_acc);
        const long rows = (long)c.rows * s.H;
        hipLaunchKernelGGL((bwd_finish<D>), grid_of(rows, 4), dim3(256), 0, st, dq_part, ids, s.cu_q, s.cu_k,
                           s.num_seqs, c.row0, rows, s.H, s.h, s.B, s.top_k, dq);
    }
    if (chunked)
        hipLaunchKernelGGL(bwd_kv_out, grid_of(std::min(kv / 2, 1L << 22), 256), dim3(256), 0, st, dk_acc, dv_acc, kv,
                           dk, dv);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(const Shape &s) {
    const int per = bwd_chunk_rows(s);
    Shape c = s;
    c.rows = per;
    return bwd_ws(c, per < s.total_q).bytes;
}

hipError_t launch_attn_backward(const Shape &s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *ids, float scale, const uint16_t *out, const float *lse,
                                const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv, void *ws,
                                hipStream_t st) {
    if (s.H / s.h > kRows) return hipErrorInvalidValue;
    if (s.d == 64 && s.B == 64) return launch_bwd<64, 64>(s, q, k, v, ids, scale, out, lse, dout, dq, dk, dv, ws, st);
    if (s.d == 64 && s.B == 128) return launch_bwd<64, 128>(s, q, k, v, ids, scale, out, lse, dout, dq, dk, dv, ws, st);
    if (s.d == 128 && s.B == 64) return launch_bwd<128, 64>(s, q, k, v, ids, scale, out, lse, dout, dq, dk, dv, ws, st);
    if (s.d == 128 && s.B == 128)
        return launch_bwd<128, 128>(s, q, k, v, ids, scale, out, lse, dout, dq, dk, dv, ws, st);
    return hipErrorInvalidValue;
}

}  // namespace msa
