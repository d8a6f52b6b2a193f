// Device-side helpers for the gfx950 MSA kernels: bf16 packing, MFMA wrappers,
// cross-lane reductions and the monotone float key used for selection.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split two floats into bf16 heads (returned) and bf16 tails (*lo_out) with
// x = head + tail + O(2^-17 |x|).
__device__ __forceinline__ uint32_t split_bf16x2(float x0, float x1, uint32_t *lo_out) {
    const uint32_t hi = pack_bf16x2(x0, x1);
    const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
    *lo_out = pack_bf16x2(x0 - h0, x1 - h1);
    return hi;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }
// Two floats -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ uint4 load16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte global store marked non-temporal (the nt bit): for write-once data
// that a later kernel reads, so that it streams to memory instead of taking
// cache lines that the running kernel's own re-read operands hold.
__device__ __forceinline__ void store16_nt(void *p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}

// 16-byte global load marked non-temporal (the nt bit), for data read once:
// a streaming read of HBM with it measured about 9% faster than with plain
// loads on this part (6.8 against 6.2 TB/s).
__device__ __forceinline__ uint4 load16_nt(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return uint4{v[0], v[1], v[2], v[3]};
}

// 16-byte global load that yields zeros when `ok` is false.  The load itself
// is unconditional (one global_load_dwordx4): when `ok` is false it reads the
// always-valid address `safe` instead of `p`, and the value is then dropped.
__device__ __forceinline__ uint4 load16_if(const void *p, bool ok, const void *safe) {
    const uint4 v = *reinterpret_cast<const uint4 *>(ok ? p : safe);
    const uint4 z = {0u, 0u, 0u, 0u};
    return ok ? v : z;
}
__device__ __forceinline__ uint4 load16_nt_if(const void *p, bool ok, const void *safe) {
    const uint4 v = load16_nt(ok ? p : safe);
    const uint4 z = {0u, 0u, 0u, 0u};
    return ok ? v : z;
}

// D(16x16, f32) += A(16x32) * B(32x16).  Operand layout (lane l, q = l / 16):
//   A: row l % 16, k = 8q .. 8q+7;  B: column l % 16, k = 8q .. 8q+7;
//   D: column l % 16, rows 4q .. 4q+3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same shape with fp16 operands.
__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D(32x32, f32) += A(32x16) * B(16x32).  Operand layout (lane l, q = l / 32):
//   A: row l % 32, k = 8q .. 8q+7;  B: column l % 32, k = 8q .. 8q+7;
//   D[i] (i < 16): column l % 32, row 8*(i/4) + 4q + (i%4).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x with the hardware v_exp_f32: results below 2^-126 come out as zero
// (softmax weights that small relative to the row maximum are negligible),
// without the denormal range fix-up exp2f adds around it.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions with the lane 16 (resp. 32) positions away: the swap returns the
// own value in one slot and the partner's in the other.
__device__ __forceinline__ float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunks addressed by the group's
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4, in that order.
__device__ __forceinline__ i16x4 lds_read_tr16(const void *lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)((__attribute__((address_space(3))) char *)lds_ptr));
}

// 16-byte read of row r of a row-major 16-bit LDS tile (row stride STRIDE
// bytes), 8 values from column 8 * c8: the A/B operand of lane (r, c8).
template <int STRIDE>
__device__ __forceinline__ uint4 lds_row8(const char *tile, int r, int c8) {
    return *reinterpret_cast<const uint4 *>(tile + r * STRIDE + 16 * c8);
}

// Transposing reads of rows r0 + 4*q4 .. +3 and r0 + 16 + 4*q4 .. +3 of a
// row-major 16-bit LDS tile (row stride STRIDE bytes), column
// 16*ct + (lane % 16): the 8 values of an MFMA operand whose k slots
// 8*q4 + i are those rows.
template <int STRIDE>
__device__ __forceinline__ uint4 lds_tr_rows(const char *tile, int r0, int ct) {
    const int lane = (int)__lane_id(), l16 = lane & 15, q4 = lane >> 4;
    const char *p = tile + (r0 + 4 * q4 + (l16 >> 2)) * STRIDE + 8 * (l16 & 3) + 32 * ct;
    const uint2 x = __builtin_bit_cast(uint2, lds_read_tr16(p));
    const uint2 y = __builtin_bit_cast(uint2, lds_read_tr16(p + 16 * STRIDE));
    return uint4{x.x, x.y, y.x, y.y};
}

// Order-preserving map of a float32 onto uint32 (larger float -> larger key).
// -0.0 is folded onto +0.0 so both zeros tie.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Completes this wave's outstanding LDS operations; also a compiler barrier.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Sequence of a packed row: the last s with cu[s] <= row (binary search over
// the num_seqs + 1 prefix offsets).
// floor(n / d) for 0 <= n < 2^31 and 1 <= d < 2^31 without a division:
// with l = ceil(log2 d) and m = ceil(2^(31 + l) / d) (< 2^32),
// floor(n m / 2^(31 + l)) = floor(n / d), because n m / 2^(31 + l) exceeds
// n / d by less than n / 2^(31 + l) < 2^-l <= 1/d.  s = l - 1 is the shift
// after the high half of the 64-bit product (s = -1 marks d = 1).
struct FastDiv {
    uint32_t m;
    int s;
};
inline FastDiv make_fastdiv(uint32_t d) {
    if (d <= 1) return FastDiv{1u, -1};
    int l = 0;
    while ((1ull << l) < d) ++l;
    const unsigned long long num = 1ull << (31 + l);
    return FastDiv{(uint32_t)((num + d - 1) / d), l - 1};
}
__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv f) {
    return f.s < 0 ? n : (__umulhi(n, f.m) >> f.s);
}

__device__ __forceinline__ int seq_of_row(const int32_t *cu, int num_seqs, int row) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= row) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace msa
