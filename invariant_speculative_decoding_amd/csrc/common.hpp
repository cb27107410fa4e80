// Device helpers shared by the isd kernels (gfx950, wave64).
//
// Nothing here depends on how many query rows a call carries: every helper
// performs the same instruction sequence for a row wherever that row sits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace isd {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned long long u64;

constexpr int kWave = 64;

// --------------------------------------------------------------- bit casts

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float f16_bits(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Whole-vector reinterpretation only.  __builtin_bit_cast of a single
// ext_vector_type element (e.g. bit_cast<float>(v.y)) compiles to a read of
// element 0 with hipcc 7.2; extract elements into scalars first.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// v_perm_b32: bytes of the result picked from {hi_src : lo_src} by `sel`
// (selector byte values 0-3 name lo_src bytes, 4-7 hi_src bytes).
__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// ---------------------------------------------------------------- loads

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) { return *(const u32x2*)p; }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *(const uint32_t*)p; }

// ------------------------------------------------------ cross-lane moves

// xor-shuffle within the wave through ds_bpermute (lane ^ m).
__device__ __forceinline__ float shfl_xor(float v, int m) {
  int lane = __lane_id();
  int src = (lane ^ m) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

// 4x4 transpose of 32-bit registers across the four 16-lane groups of a
// wave: on entry register j of lane group G holds M[G][j]; on exit register
// j of lane group G holds M[j][G].  Two v_permlane32_swap (exchange the
// upper 32 lanes of one register with the lower 32 of another) followed by
// two v_permlane16_swap (exchange odd 16-lane groups of one register with
// even groups of another).
__device__ __forceinline__ void transpose4x4_lanegroups(u32x4& v) {
  auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  uint32_t v0 = a[0], v2 = a[1], v1 = b[0], v3 = b[1];
  auto c = __builtin_amdgcn_permlane16_swap(v0, v1, false, false);
  auto d = __builtin_amdgcn_permlane16_swap(v2, v3, false, false);
  v.x = c[0];
  v.y = c[1];
  v.z = d[0];
  v.w = d[1];
}

// ------------------------------------------------------- bf16 operands

// Exact split of an fp32 value (given as its bits) into three bf16 parts by
// truncation: v = hi + mid + lo, each part holding at most 8 significant
// bits of v's 24.  Returns the three bf16 bit patterns in the low halves.
__device__ __forceinline__ void split3(uint32_t u, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t hb = u & 0xFFFF0000u;
  const float r1 = __builtin_bit_cast(float, u) - __builtin_bit_cast(float, hb);
  const uint32_t u1 = __builtin_bit_cast(uint32_t, r1);
  const uint32_t mb = u1 & 0xFFFF0000u;
  const float r2 = r1 - __builtin_bit_cast(float, mb);
  h = hb >> 16;
  m = mb >> 16;
  l = __builtin_bit_cast(uint32_t, r2) >> 16;
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- row ranges

// Rows of sequence s of a ragged batch: row_start[s] .. row_start[s+1] - 1,
// at most `cap` of them.  The last entry, row_start[B], is the row count
// the caller's row arrays are sized by, so a range that does not lie within
// [0, row_start[B]) -- a negative start or an end past that entry, which
// well-formed offsets never have -- gives no rows: no kernel then indexes a
// row outside those arrays.  Returns the row count; *r0 receives the first
// row.  seq_range_of takes the three offsets already loaded:
// a = row_start[s], b = row_start[s + 1], R = row_start[B].
__device__ __forceinline__ int seq_range_of(int a, int b, int R, int cap, int* r0) {
  long n = (long)b - a;
  if (n > cap) n = cap;
  if (a < 0 || n < 0 || a + n > (long)R) n = 0;
  *r0 = a;
  return (int)n;
}

__device__ __forceinline__ int seq_range(const int32_t* row_start, int s, int B, int cap,
                                         int* r0) {
  return seq_range_of(row_start[s], row_start[s + 1], row_start[B], cap, r0);
}

// Waits once for wave-uniform values just loaded, so that their loads are
// issued together: without it the compiler may sink each load to its first
// use, past branches, and wait for each in turn.
#define ISD_MATERIALIZE4(x0, x1, x2, x3) \
  asm volatile("" ::"s"(x0), "s"(x1), "s"(x2), "s"(x3))

// ------------------------------------------------------------ argmax keys
//
// The greedy target token is the lowest id among the maxima of a logit row.
// Every logit becomes a 64-bit key: order-preserving float bits above the
// complemented index, so the largest key is the largest value at the lowest
// index, and the maximum of any set of keys is the same whichever way the
// keys are combined.  NaN never wins (key 0 above the index bits) and -0
// counts as +0.

__device__ __forceinline__ u64 max_u64(u64 a, u64 b) { return a > b ? a : b; }

__device__ __forceinline__ u64 argmax_key(float v, uint32_t idx) {
  uint32_t o;
  if (v != v) {
    o = 0u;  // NaN never wins
  } else {
    uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);  // -0 -> +0
    o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  return ((u64)o << 32) | (u64)(0xFFFFFFFFu - idx);
}

// xor-shuffle of a 64-bit value within the wave (two 32-bit permutes)
__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int m) {
  const int src = (__lane_id() ^ m) << 2;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(v >> 32));
  return ((u64)hi << 32) | lo;
}

// A 64-bit DPP move: both halves take the same lane pattern CTRL.
template <int CTRL>
__device__ __forceinline__ u64 dpp_u64(u64 v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((u64)hi << 32) | lo;
}

// Maximum of v over each DPP row (lanes 16r .. 16r+15), in every lane of the
// row: swap neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1),
// mirror each half row, mirror the row.  Every lane must be active.
__device__ __forceinline__ u64 row16_max_u64(u64 v) {
  v = max_u64(v, dpp_u64<0xB1>(v));
  v = max_u64(v, dpp_u64<0x4E>(v));
  v = max_u64(v, dpp_u64<0x141>(v));
  v = max_u64(v, dpp_u64<0x140>(v));
  return v;
}

}  // namespace isd
