// spec_verify: accept a prefix of each sequence's drafts and emit the
// correction or bonus token.
//
// Greedy (temperature 0): the target's choice is the lowest id among the
// maxima of its logit row (ramgpt.org, "When Lossless Speculation Stops
// Being Lossless on Blackwell", section "The Hidden Contract Behind
// Lossless Speculation").  The argmax is an order-free reduction: every
// logit becomes a 64-bit key (order-preserving float bits above the
// complemented index), and the maximum key is the same whichever way the
// keys are combined, so slicing the vocabulary over work-groups cannot
// change the result.
//
// Sampling (temperature > 0): the accept-or-reject rule of Leviathan et al.
// and Chen et al. (proofoftech.org, "'Lossless' speculative decoding is a
// property of the math, not your deployment.", section "Lossless is a
// theorem, and theorems have hypotheses").  Softmax statistics (max and sum
// of exponentials) are reduced per row in a fixed order; uniforms come from
// Philox4x32-10 keyed by (seed, sequence id, position, stream), so nothing
// depends on how sequences are batched; the residual max(0, p - q) is
// sampled by an inverse CDF walked in ascending id order with a fixed
// segmentation of the vocabulary.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

constexpr int kVThreads = 256;
constexpr int kCh = 4096;              // vocabulary entries per work-group (slice or chunk)
constexpr int kPer = kCh / kVThreads;  // entries per thread
constexpr int kMaxChunks = kVThreads;  // chunk sums are located with one block scan
constexpr int kMaxDevices = 64;        // GPUs per process with a spec_verify_noalloc scratch

// ------------------------------------------------------------------ Philox

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// u in [0, 1) from the first output word: (w0 >> 8) * 2^-24.
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint32_t seq, uint32_t pos,
                                                uint32_t stream) {
  uint32_t c[4] = {pos, seq, stream, 0u};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (float)(c[0] >> 8) * 5.9604644775390625e-8f;
}

// ------------------------------------------------------- wave reductions

__device__ __forceinline__ u64 wave_max_u64(u64 v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max_u64(v, shfl_xor_u64(v, m));
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// Butterfly sum: every lane ends with the same bits (each step adds the
// same two values, a + b == b + a).
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = v + shfl_xor(v, m);
  return v;
}

// ------------------------------------------------------------------ argmax


// grid = (slices, max_rows), block = 256.  ws[row][slice] = the largest key
// of the slice's 4096 entries.  Each thread loads its 16 entries with
// independent loads (clamped addresses), then keys past V are dropped.
__global__ __launch_bounds__(256) void argmax_slices_kernel(const float* __restrict__ z,
                                                            const int32_t* __restrict__ row_start,
                                                            int B, int V, int nslice,
                                                            u64* __restrict__ ws) {
  __shared__ u64 part[4];
  const int row = blockIdx.y;
  if (row >= row_start[B]) return;  // row < gridDim.y = max_rows as well
  const int tid = threadIdx.x;
  const int v0 = blockIdx.x * kCh;
  const float* zr = z + (size_t)row * V;
  float val[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) val[e] = zr[min(v0 + tid + e * kVThreads, V - 1)];
  u64 best = 0ull;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = v0 + tid + e * kVThreads;
    if (v < V) best = max_u64(best, argmax_key(val[e], (uint32_t)v));
  }
  best = wave_max_u64(best);
  if ((tid & 63) == 0) part[tid >> 6] = best;
  __syncthreads();
  if (tid == 0)
    ws[(size_t)row * nslice + blockIdx.x] =
        max_u64(max_u64(part[0], part[1]), max_u64(part[2], part[3]));
}

// First target row and draft count of sequence s; k = -1 marks a sequence
// that cannot be verified: no rows, rows outside [0, row_start[B]) or
// beyond the sized workspace (max_rows), or draft entries -- row_start[s] -
// s onwards, one per row after the first -- outside the R - B the drafts
// hold.  Well-formed offsets (non-decreasing from 0, every sequence at
// least one row) always pass.
__device__ __forceinline__ void seq_layout(const int32_t* row_start, int s, int B, int max_rows,
                                           int* r0, int* k) {
  int a;
  int n = seq_range(row_start, s, B, ISD_MAX_OUT, &a);
  const int R = row_start[B];
  if (n > 0 && (a < s || (long)a + n > max_rows || (long)a - s + n - 1 > (long)R - B)) n = 0;
  *r0 = a;
  *k = n - 1;
}

// kv_commit's COMMIT for sequence s after accepting a drafts:
// seq_len[s] += a + 1 and pos_id[s] = seq_len[s].
__device__ __forceinline__ void commit_one(int32_t* seq_len, int32_t* pos_id, int s, int a) {
  const int c = seq_len[s] + a + 1;
  seq_len[s] = c;
  pos_id[s] = c;
}

// Wave 0 of a sequence's work-group: the first draft that differs from the
// target's choice (drafts one per lane, a ballot) ends the accepted prefix;
// the emitted tokens are the accepted drafts and the target's token after
// them.  With seq_len given it also commits, exactly as kv_commit's COMMIT
// does after it: seq_len[s] += accept_len[s] + 1 and pos_id[s] = seq_len[s].
__device__ __forceinline__ void greedy_decide(const int* tgt, int k, int d, int s, int lane,
                                              int32_t* __restrict__ acc,
                                              int32_t* __restrict__ out,
                                              int32_t* __restrict__ seq_len,
                                              int32_t* __restrict__ pos_id) {
  int32_t* o = out + (size_t)s * ISD_MAX_OUT;
  int a = 0;
  if (k < 0) {
    if (lane < ISD_MAX_OUT) o[lane] = -1;
  } else {
    const bool miss = lane < k && d != tgt[min(lane, ISD_MAX_OUT - 1)];
    const u64 mb = __ballot(miss);
    a = mb ? (int)__builtin_ctzll(mb) : k;
    if (lane < ISD_MAX_OUT) o[lane] = lane < a ? d : (lane == a ? tgt[a] : -1);
  }
  if (lane == 0) {
    acc[s] = a;
    if (seq_len) commit_one(seq_len, pos_id, s, a);
  }
}

// grid = B, block = 256.  Greedy accept-prefix of one sequence.  Wave w
// reduces the slice keys of target rows w, w + 4, w + 8 (every key of a row
// loaded at once); wave 0 holds the drafts (one per lane) and decides
// (greedy_decide), committing when seq_len is given.
__global__ __launch_bounds__(256) void greedy_accept_kernel(const u64* __restrict__ ws,
                                                           const int32_t* __restrict__ drafts,
                                                           const int32_t* __restrict__ row_start,
                                                           int B, int nslice, int max_rows,
                                                           int32_t* __restrict__ acc,
                                                           int32_t* __restrict__ out,
                                                           int32_t* __restrict__ seq_len,
                                                           int32_t* __restrict__ pos_id) {
  __shared__ int tgt[ISD_MAX_OUT];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int r0, k;
  seq_layout(row_start, s, B, max_rows, &r0, &k);
  int d = -1;
  if (w == 0 && lane < k) d = drafts[(r0 - s) + lane];
  u64 best[3] = {0ull, 0ull, 0ull};
  for (int sl0 = 0; sl0 < nslice; sl0 += kWave) {
    const int sl = sl0 + lane;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int j = w + 4 * q;
      if (j <= k && sl < nslice) best[q] = max_u64(best[q], ws[(size_t)(r0 + j) * nslice + sl]);
    }
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int j = w + 4 * q;
    if (j <= k) {  // uniform
      const u64 b = wave_max_u64(best[q]);
      if (lane == 0) tgt[j] = (int)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
    }
  }
  __syncthreads();
  if (w != 0) return;
  greedy_decide(tgt, k, d, s, lane, acc, out, seq_len, pos_id);
}

// grid = B, block = 64 * ISD_MAX_OUT.  The same accept-prefix from
// per-block argmax keys (keys[row][nkeys], e.g. one per work-group of
// qgemm_w4_argmax): wave j reduces target row j of its sequence, lane l
// taking keys l, l+64, ...  kKeyBatch of them per lane are loaded at once
// (indexes clamped to the last key, which cannot change a maximum), so a
// row of up to 64 * kKeyBatch keys costs one round of loads, and all rows'
// rounds overlap.  The maximum of keys is order-free, so the targets equal
// those of the logits.
constexpr int kKeyBatch = 32;  // 2048 keys per round: the 152064-row lm_head has 1902

__global__ __launch_bounds__(kWave * ISD_MAX_OUT) void greedy_keys_kernel(
    const u64* __restrict__ keys, int nkeys, const int32_t* __restrict__ drafts,
    const int32_t* __restrict__ row_start, int B, int max_rows, int32_t* __restrict__ acc,
    int32_t* __restrict__ out, int32_t* __restrict__ seq_len, int32_t* __restrict__ pos_id) {
  __shared__ int tgt[ISD_MAX_OUT];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int r0, k;
  seq_layout(row_start, s, B, max_rows, &r0, &k);
  // wave 0's drafts are requested before the keys, so they arrive with them
  const int d = w == 0 && lane < k ? drafts[(r0 - s) + lane] : -1;
  if (w <= k) {  // uniform
    const u64* kr = keys + (size_t)(r0 + w) * nkeys;
    u64 best = 0ull;
    for (int e0 = lane; e0 < nkeys; e0 += kWave * kKeyBatch) {
      u64 v[kKeyBatch];
#pragma unroll
      for (int u = 0; u < kKeyBatch; ++u) v[u] = kr[min(e0 + kWave * u, nkeys - 1)];
#pragma unroll
      for (int u = 0; u < kKeyBatch; ++u) best = max_u64(best, v[u]);
    }
    best = wave_max_u64(best);
    if (lane == 0) tgt[w] = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
  }
  __syncthreads();
  if (w != 0) return;
  greedy_decide(tgt, k, d, s, lane, acc, out, seq_len, pos_id);
}

// ---------------------------------------------------- margin re-check
//
// The greedy verify plus, for every target row, the margin between its two
// best logits, and per sequence the first deciding row whose margin is
// below a threshold: the near-tie steps where the last rounding digit picks
// the token (tokenstrom.com, "'Lossless,' but not quite", sections "Why the
// math checks out and the text still flips" and "What the big servers offer
// and what it costs": re-check only the uncertain steps).  The two best keys
// of a set are order-free like the best one (keys are distinct), so slices
// merge in any order.

// Insert key k into the pair a1 > a2 of distinct keys, branch-free: the new
// second is the larger of the old second and the smaller of (a1, k).
__device__ __forceinline__ void top2_insert(u64& a1, u64& a2, u64 k) {
  a2 = max_u64(a2, k < a1 ? k : a1);
  a1 = max_u64(a1, k);
}

// merge of two top-2 lists of distinct keys (commutative)
__device__ __forceinline__ void top2_merge(u64& a1, u64& a2, u64 b1, u64 b2) {
  const u64 hi = max_u64(a1, b1), lo = a1 > b1 ? b1 : a1;
  a2 = max_u64(lo, max_u64(a2, b2));
  a1 = hi;
}

__device__ __forceinline__ void wave_top2(u64& a1, u64& a2) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int src = (__lane_id() ^ m) << 2;
    const uint32_t l1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)a1);
    const uint32_t h1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(a1 >> 32));
    const uint32_t l2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)a2);
    const uint32_t h2 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(a2 >> 32));
    top2_merge(a1, a2, ((u64)h1 << 32) | l1, ((u64)h2 << 32) | l2);
  }
}

// the logit a key was made from (NaN for NaN entries)
__device__ __forceinline__ float key_value(u64 key) {
  const uint32_t o = (uint32_t)(key >> 32);
  const uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, b);
}

// grid = (slices, max_rows), block = 256.  ws[row][slice] = the two largest
// keys of the slice (0 when the slice has a single entry).
__global__ __launch_bounds__(256) void argmax_top2_kernel(const float* __restrict__ z,
                                                          const int32_t* __restrict__ row_start,
                                                          int B, int V, int nslice,
                                                          u64* __restrict__ ws) {
  __shared__ u64 part[4][2];
  const int row = blockIdx.y;
  if (row >= row_start[B]) return;
  const int tid = threadIdx.x;
  const int v0 = blockIdx.x * kCh;
  const float* zr = z + (size_t)row * V;
  float val[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) val[e] = zr[min(v0 + tid + e * kVThreads, V - 1)];
  u64 a1 = 0ull, a2 = 0ull;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = v0 + tid + e * kVThreads;
    if (v < V) top2_insert(a1, a2, argmax_key(val[e], (uint32_t)v));
  }
  wave_top2(a1, a2);
  if ((tid & 63) == 0) {
    part[tid >> 6][0] = a1;
    part[tid >> 6][1] = a2;
  }
  __syncthreads();
  if (tid == 0) {
    u64 b1 = part[0][0], b2 = part[0][1];
    for (int w = 1; w < 4; ++w) top2_merge(b1, b2, part[w][0], part[w][1]);
    u64* o = ws + ((size_t)row * nslice + blockIdx.x) * 2;
    o[0] = b1;
    o[1] = b2;
  }
}

// grid = B, block = 256.  As greedy_accept_kernel, plus margins of the
// sequence's target rows and the re-check row.
__global__ __launch_bounds__(256) void greedy_margin_kernel(const u64* __restrict__ ws,
                                                           const int32_t* __restrict__ drafts,
                                                           const int32_t* __restrict__ row_start,
                                                           int B, int nslice, int max_rows,
                                                           float threshold,
                                                           int32_t* __restrict__ acc,
                                                           int32_t* __restrict__ out,
                                                           float* __restrict__ margins,
                                                           int32_t* __restrict__ recheck) {
  __shared__ int tgt[ISD_MAX_OUT];
  __shared__ float mg[ISD_MAX_OUT];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int r0, k;
  seq_layout(row_start, s, B, max_rows, &r0, &k);
  int d = -1;
  if (w == 0 && lane < k) d = drafts[(r0 - s) + lane];
  u64 b1[3] = {0ull, 0ull, 0ull}, b2[3] = {0ull, 0ull, 0ull};
  for (int sl0 = 0; sl0 < nslice; sl0 += kWave) {
    const int sl = sl0 + lane;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int j = w + 4 * q;
      if (j <= k && sl < nslice) {
        const u64* p = ws + ((size_t)(r0 + j) * nslice + sl) * 2;
        top2_merge(b1[q], b2[q], p[0], p[1]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int j = w + 4 * q;
    if (j <= k) {  // uniform
      u64 t1 = b1[q], t2 = b2[q];
      wave_top2(t1, t2);
      if (lane == 0) {
        tgt[j] = (int)(0xFFFFFFFFu - (uint32_t)(t1 & 0xFFFFFFFFull));
        const float m = t2 ? key_value(t1) - key_value(t2) : INFINITY;
        mg[j] = m;
        margins[r0 + j] = m;
      }
    }
  }
  __syncthreads();
  if (w != 0) return;
  int32_t* o = out + (size_t)s * ISD_MAX_OUT;
  if (k < 0) {
    if (lane < ISD_MAX_OUT) o[lane] = -1;
    if (lane == 0) {
      acc[s] = 0;
      recheck[s] = -1;
    }
    return;
  }
  const bool miss = lane < k && d != tgt[min(lane, ISD_MAX_OUT - 1)];
  const u64 mb = __ballot(miss);
  const int a = mb ? (int)__builtin_ctzll(mb) : k;
  if (lane < ISD_MAX_OUT) o[lane] = lane < a ? d : (lane == a ? tgt[a] : -1);
  const u64 low = __ballot(lane <= a && mg[min(lane, ISD_MAX_OUT - 1)] < threshold);
  if (lane == 0) {
    acc[s] = a;
    recheck[s] = low ? (int)__builtin_ctzll(low) : -1;
  }
}

// ------------------------------------------------------------------ sampling
//
// Two launches, every reduction in a fixed order:
//  1. chunk_stats: per (row, 4096-entry chunk) the max of z/T and the sum of
//     exp(z/T - max) (16 entries per thread, a fixed butterfly per wave,
//     the four waves in order).  It also clears the per-sequence arrival
//     counters of launch 2.
//  2. decide_draw: per (sequence, chunk) work-group: the accept decisions
//     (row statistics merged from the chunk statistics by one fixed tree;
//     all draft tests evaluated at once, the first failure taken), then the
//     chunk's sum of the distribution a draw would use -- the residual
//     max(0, p_{a+1} - q_{a+1}) after a rejection at draft a+1, p_{k+1}
//     when all k drafts pass -- and of p_{a+1} itself (the fallback for an
//     all-zero residual).  The last work-group of the sequence to finish
//     (counted by an atomic once its sums are published) locates the chunk that
//     holds u' * S from the chunk sums in ascending order and walks it in
//     ascending id order.
// A chunk's sum and its walk use one summation order: thread t adds its 16
// consecutive entries in order, then the 256 thread sums are combined by
// one fixed inclusive scan (a shuffle scan inside each wave, then the wave
// totals in wave order), whose last element is the chunk sum.  Logits are
// scaled as z * fp32(1/T).

__device__ __forceinline__ float shfl_up_f32(float v, int off) {
  const int lane = __lane_id();
  const int src = (lane >= off ? lane - off : lane) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

// Inclusive prefix sums of two values over the 256 threads of a block in a
// fixed order; `excl` receives the previous thread's inclusive values
// exactly (0 for thread 0) and `total` the last thread's.  `lds` holds 4
// entries.
__device__ __forceinline__ float2 block_scan2(float2 v, float2* lds, float2& excl,
                                              float2& total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float tx = shfl_up_f32(v.x, off), ty = shfl_up_f32(v.y, off);
    if (lane >= off) {
      v.x = tx + v.x;
      v.y = ty + v.y;
    }
  }
  if (lane == kWave - 1) lds[w] = v;
  __syncthreads();
  // the wave's base: totals of the earlier waves folded left to right, so
  // that base + (last lane of the previous wave) is exactly that lane's
  // final value
  float2 base = make_float2(0.f, 0.f);
  for (int j = 0; j < w; ++j) base = make_float2(base.x + lds[j].x, base.y + lds[j].y);
  const float2 r = make_float2(base.x + v.x, base.y + v.y);
  float2 prev = make_float2(shfl_up_f32(r.x, 1), shfl_up_f32(r.y, 1));
  if (lane == 0) prev = base;
  excl = prev;
  float2 t = make_float2(0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kVThreads / kWave; ++j) t = make_float2(t.x + lds[j].x, t.y + lds[j].y);
  total = t;
  __syncthreads();
  return r;
}

// Log-sum-exp merge of two (max, sum of exp(x - max)) pairs; commutative
// bit for bit, (-inf, 0) is its identity.  Branch-free (a select instead
// of an early return), so independent merges can be interleaved.
__device__ __forceinline__ float2 lse_merge(float2 a, float2 b) {
  const float M = fmaxf(a.x, b.x);
  const float sum = a.y * __expf(a.x - M) + b.y * __expf(b.x - M);
  return make_float2(M, M == -INFINITY ? 0.f : sum);
}

__device__ __forceinline__ float prob_of(float z, float invT, float2 st) {
  return __expf(z * invT - st.x) / st.y;
}

// The probability of an entry inside a chunk walk: the row's 1/S is formed
// once (rinv) and each entry takes a product instead of a division.
__device__ __forceinline__ float prob_r(float z, float invT, float m, float rinv) {
  return __expf(z * invT - m) * rinv;
}

// Value of one entry in the distribution a draw uses: the residual
// max(0, p - q) when the drafter row is given, else p.
__device__ __forceinline__ float entry_value(float p, float zq, bool use_q, float invT, float mq,
                                             float rq) {
  return use_q ? fmaxf(0.f, p - prob_r(zq, invT, mq, rq)) : p;
}

// grid = (nch, 2 * max_rows), block = 256.  cs[row][chunk] = (max, sum).
__global__ __launch_bounds__(256) void chunk_stats_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd,
    const int32_t* __restrict__ row_start, int B, int V, int max_rows, int nch, float invT,
    float2* __restrict__ cs, uint32_t* __restrict__ cnt) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e < B; e += kVThreads) cnt[e] = 0u;
  const int R = row_start[B];
  const int row = blockIdx.y;
  const float* z;
  if (row < max_rows) {
    if (row >= R) return;
    z = zt + (size_t)row * V;
  } else {
    const int dr = row - max_rows;
    if (dr >= R - B) return;
    z = zd + (size_t)dr * V;
  }
  const int lane = tid & 63, w = tid >> 6;
  const int v0 = blockIdx.x * kCh;
  float val[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) val[e] = z[min(v0 + tid + e * kVThreads, V - 1)] * invT;
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (v0 + tid + e * kVThreads < V) m = fmaxf(m, val[e]);
  m = wave_max_f32(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (v0 + tid + e * kVThreads < V) sum += __expf(val[e] - M);
  }
  sum = wave_sum_f32(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  if (tid == 0) cs[(size_t)row * nch + blockIdx.x] = make_float2(M, ((red[0] + red[1]) + red[2]) + red[3]);
}

// The 16 consecutive entries of thread t in chunk c of rows zp (and zq):
// p (and the residual max(0, p - q) when zq is given, else p again).
// Entries past V are 0.  With `vec` (rows 16-byte aligned) a thread whose
// entries all lie below V loads them as four 16-byte vectors; otherwise
// loads are clamped and unconditional.
__device__ __forceinline__ void chunk_values(const float* zp, const float* zq, int V, int c,
                                            float invT, float2 sp, float2 sq, bool vec,
                                            float* pv, float* cv) {
  const int base = c * kCh + threadIdx.x * kPer;
  float a[kPer], b[kPer];
  if (vec && base + kPer <= V) {
#pragma unroll
    for (int e = 0; e < kPer; e += 4) {
      const float4 t = *(const float4*)(zp + base + e);
      a[e] = t.x;
      a[e + 1] = t.y;
      a[e + 2] = t.z;
      a[e + 3] = t.w;
    }
    if (zq) {
#pragma unroll
      for (int e = 0; e < kPer; e += 4) {
        const float4 t = *(const float4*)(zq + base + e);
        b[e] = t.x;
        b[e + 1] = t.y;
        b[e + 2] = t.z;
        b[e + 3] = t.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) a[e] = zp[min(base + e, V - 1)];
    if (zq) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) b[e] = zq[min(base + e, V - 1)];
    }
  }
  const float rp = 1.0f / sp.y, rq = 1.0f / sq.y;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const bool in = base + e < V;
    const float p = in ? prob_r(a[e], invT, sp.x, rp) : 0.f;
    pv[e] = p;
    cv[e] = zq ? (in ? entry_value(p, b[e], true, invT, sq.x, rq) : 0.f) : p;
  }
}

struct Decision {
  int a, rej;
  float2 st[2 * ISD_MAX_OUT];  // target rows 0..k, then draft rows at ISD_MAX_OUT + j
};

// grid = (nch, B), block = 256.  See the overview above.
__global__ __launch_bounds__(256) void decide_draw_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ seq_id, const int32_t* pos0,
    int B, int V, int max_rows, int nch, float invT, uint64_t seed, int vec,
    const float2* __restrict__ cs, float* __restrict__ rsum, float* __restrict__ psum,
    uint32_t* __restrict__ cnt, int32_t* __restrict__ acc, int32_t* __restrict__ out,
    int32_t* seq_len, int32_t* pos_id) {
  __shared__ float2 scan[kVThreads / kWave];
  __shared__ Decision dec;
  __shared__ int sh_last, sh_chunk, sh_tok;
  __shared__ float sh_t;
  const int c = blockIdx.x;
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  int r0, k;
  seq_layout(row_start, s, B, max_rows, &r0, &k);
  int32_t* o = out + (size_t)s * ISD_MAX_OUT;
  if (k < 0) {
    if (c == 0 && tid == 0) {
      acc[s] = 0;
      for (int e = 0; e < ISD_MAX_OUT; ++e) o[e] = -1;
      if (seq_len) commit_one(seq_len, pos_id, s, 0);
    }
    return;
  }
  const int dbase = r0 - s;
  const uint32_t sid = (uint32_t)seq_id[s];
  // In the commit form pos0 is pos_id, which the last work-group advances:
  // every work-group of the sequence reads it here, before it counts in,
  // and the last one writes it only after every arrival.
  const uint32_t p0 = (uint32_t)pos0[s];

  // ---- draft j's token and its target / drafter logits (thread j < k),
  // fetched while the chunk statistics are staged
  int x = -1;
  float zpx = 0.f, zqx = 0.f;
  if (tid < k) {
    x = drafts[dbase + tid];
    const int xc = min(max(x, 0), V - 1);
    zpx = zt[(size_t)(r0 + tid) * V + xc];
    zqx = zd[(size_t)(dbase + tid) * V + xc];
  }
  // Row statistics of the 2k+1 rows (targets 0..k, then drafts): 8
  // threads per row (thread t takes row t / 8; rows past 2k+1 repeat the
  // last one and are not stored), thread j of a row folds chunks j, j+8,
  // j+16, ... in that order, then a butterfly merges the 8 threads.  Every
  // work-group of the sequence computes the same bits.  All loads are
  // issued first.
  const int nrow = 2 * k + 1;
  {
    constexpr int TPR = 8;                 // threads per row
    constexpr int CPT = kMaxChunks / TPR;  // most chunks per thread
    static_assert(2 * ISD_MAX_OUT - 1 <= kVThreads / TPR, "one thread group per row");
    const int rr = tid / TPR, j0 = tid % TPR;
    const int r = min(rr, nrow - 1);
    const size_t row = r <= k ? (size_t)(r0 + r) : (size_t)(max_rows + dbase + (r - k - 1));
    float2 cv_[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      if (TPR * j < nch)  // uniform
        cv_[j] = cs[row * nch + min(j0 + TPR * j, nch - 1)];
    float2 racc = make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      if (TPR * j < nch)  // uniform
        racc = lse_merge(racc, j0 + TPR * j < nch ? cv_[j] : make_float2(-INFINITY, 0.f));
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1)
      racc = lse_merge(racc, make_float2(shfl_xor(racc.x, m), shfl_xor(racc.y, m)));
    if (j0 == 0 && rr < nrow) dec.st[rr <= k ? rr : ISD_MAX_OUT + (rr - k - 1)] = racc;
  }
  __syncthreads();

  // ---- every draft test at once; the first failure ends the prefix
  if (tid < kWave) {
    bool fail = false;
    if (tid < k) {
      bool ok = false;
      if (x >= 0 && x < V) {
        const float p = prob_of(zpx, invT, dec.st[tid]);
        const float q = prob_of(zqx, invT, dec.st[ISD_MAX_OUT + tid]);
        const float u = philox_uniform(seed, sid, p0 + (uint32_t)tid, 0u);
        ok = u < fminf(1.f, q > 0.f ? p / q : INFINITY);
      }
      fail = !ok;
    }
    const u64 mb = __ballot(fail);
    if (tid == 0) {
      dec.a = mb ? (int)__builtin_ctzll(mb) : k;
      dec.rej = mb != 0ull;
    }
  }
  __syncthreads();
  const int a = dec.a;
  const int rej = dec.rej;
  const float* zp = zt + (size_t)(r0 + a) * V;
  const float2 sp = dec.st[a];
  const float* zq = rej ? zd + (size_t)(dbase + a) * V : nullptr;
  const float2 sq = rej ? dec.st[ISD_MAX_OUT + a] : sp;

  // ---- this chunk's sums of the candidate distribution and of p
  float pv[kPer], cv[kPer];
  chunk_values(zp, zq, V, c, invT, sp, sq, vec != 0, pv, cv);
  float2 mine = make_float2(0.f, 0.f);
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    mine.x += cv[e];
    mine.y += pv[e];
  }
  float2 before, tot;
  const float2 after = block_scan2(mine, scan, before, tot);
  // Publishing the sums.  Writer side: the two sums are agent-scope atomic
  // stores, which are performed at the level every XCD reads (not held
  // dirty in this XCD's L2), and the wait for the vector-memory counter
  // makes both complete before the arrival is counted.  These are the only
  // values handed over, so the L2 write-back of a release fence (which
  // would flush every ordinary store of the XCD) has nothing to publish.
  // Reader side: the last work-group takes an agent-scope acquire fence
  // after its arrival, which invalidates its L2's stale lines, and then
  // reads the sums with agent-scope atomic loads.
  if (tid == 0) {
    __hip_atomic_store(&rsum[(size_t)s * nch + c], tot.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&psum[(size_t)s * nch + c], tot.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // both stores complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    sh_last = __hip_atomic_fetch_add(&cnt[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (uint32_t)(nch - 1);
  }
  __syncthreads();
  if (!sh_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- the last work-group draws: the chunk from the chunk sums in
  // ascending order, then the entry inside it in ascending id order; an
  // all-zero residual falls back to p_{a+1}
  const float u2 = philox_uniform(seed, sid, p0 + (uint32_t)a, 1u);
  const float* rs = rsum + (size_t)s * nch;
  const float* ps = psum + (size_t)s * nch;
  float2 cexcl, S;
  const float2 cincl = block_scan2(
      tid < nch ? make_float2(__hip_atomic_load(rs + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                              __hip_atomic_load(ps + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                : make_float2(0.f, 0.f),
      scan, cexcl, S);
  const bool use_q = rej && S.x > 0.f;
  const float St = use_q ? S.x : S.y;
  const float incl = use_q ? cincl.x : cincl.y;
  const float excl = use_q ? cexcl.x : cexcl.y;
  const float* sums = use_q ? rs : ps;
  const float t = u2 * St;
  if (tid == 0) {
    sh_chunk = -1;
    sh_tok = -1;
  }
  __syncthreads();
  // the first chunk whose inclusive sum passes t (prefixes never decrease
  // and `excl` is exactly the previous inclusive value: one thread)
  if (tid < nch && incl > t && !(excl > t)) {
    sh_chunk = tid;
    sh_t = t - excl;
  }
  __syncthreads();
  if (tid == 0 && sh_chunk < 0) {  // t at or past the rounded total
    for (int cc = nch - 1; cc >= 0; --cc)
      if (__hip_atomic_load(sums + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > 0.f) {
        sh_chunk = cc;
        sh_t = INFINITY;
        break;
      }
  }
  __syncthreads();
  const int cstar = sh_chunk;
  if (cstar >= 0) {
    const float tc = sh_t;
    if (cstar != c) chunk_values(zp, zq, V, cstar, invT, sp, sq, vec != 0, pv, cv);
    float vals[kPer];
    float th = 0.f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      vals[e] = use_q ? cv[e] : pv[e];
      th += vals[e];
    }
    float2 b2, t2;
    const float2 a2 = block_scan2(make_float2(th, 0.f), scan, b2, t2);
    // The prefix never decreases, so exactly one thread is the first whose
    // range passes tc; it walks its entries in ascending id order.
    const int base = cstar * kCh + tid * kPer;
    if (a2.x > tc && (tid == 0 || !(b2.x > tc))) {
      float run = b2.x;
      for (int e = 0; e < kPer; ++e) {
        run += vals[e];
        if (run > tc) {
          sh_tok = base + e;
          break;
        }
      }
    }
    __syncthreads();
    if (tid == 0 && sh_tok < 0) {
      // nothing positive at or after t in this chunk: last positive entry
      for (int v = min(V, (cstar + 1) * kCh) - 1; v >= cstar * kCh; --v) {
        const float p = prob_r(zp[v], invT, sp.x, 1.0f / sp.y);
        const float val = use_q ? entry_value(p, zq[v], true, invT, sq.x, 1.0f / sq.y) : p;
        if (val > 0.f) {
          sh_tok = v;
          break;
        }
      }
    }
    __syncthreads();
  }
  if (tid < ISD_MAX_OUT) {
    // thread j < k already holds draft j (x, loaded at the start)
    o[tid] = tid < a ? x : (tid == a ? sh_tok : -1);
  }
  if (tid == 0) {
    acc[s] = a;
    if (seq_len) commit_one(seq_len, pos_id, s, a);
  }
}

}  // namespace isd

namespace isd {

// Workspace of spec_verify: greedy, the slice keys u64 [max_rows][nch];
// sampling, chunk statistics float2 [2 max_rows][nch], then per-chunk
// residual and p sums float [B][nch] each, then arrival counters u32 [B]
// (each part 256-byte aligned).  Returns 0 for arguments no call accepts.
static size_t verify_ws_bytes(int B, int V, int max_rows, float temperature) {
  if (B < 1 || V < 1 || max_rows < B || max_rows > ISD_MAX_VERIFY_ROWS ||
      !(temperature >= 0.f) || temperature == INFINITY)
    return 0;
  const bool greedy = temperature == 0.f;
  const int nch = (V + kCh - 1) / kCh;
  if (!greedy && nch > kMaxChunks) return 0;  // V > 1,048,576
  if (greedy) return (size_t)max_rows * nch * sizeof(unsigned long long);
  const size_t cs_bytes = round_up(2 * (size_t)max_rows * nch * sizeof(float2), 256);
  const size_t rs_bytes = round_up((size_t)B * nch * sizeof(float), 256);
  const size_t cnt_bytes = round_up((size_t)B * sizeof(uint32_t), 256);
  return cs_bytes + 2 * rs_bytes + cnt_bytes;
}

// Pointer checks of spec_verify (sizes are checked by verify_ws_bytes).
static int verify_check(const float* target_logits, const float* draft_logits,
                        const int32_t* drafts, const int32_t* row_start, const int32_t* seq_id,
                        const int32_t* pos0, float temperature, int32_t* accept_len,
                        int32_t* out_tokens) {
  const bool greedy = temperature == 0.f;
  if (!target_logits || !drafts || !row_start || !accept_len || !out_tokens) return ISD_EINVAL;
  if (!aligned(target_logits, 4) || !aligned(drafts, 4) || !aligned(row_start, 4) ||
      !aligned(accept_len, 4) || !aligned(out_tokens, 4))
    return ISD_EINVAL;
  if (greedy) return ISD_OK;
  if (!draft_logits || !seq_id || !pos0) return ISD_EINVAL;
  if (!aligned(draft_logits, 4) || !aligned(seq_id, 4) || !aligned(pos0, 4)) return ISD_EINVAL;
  return ISD_OK;
}

// Launches of spec_verify on a workspace of at least verify_ws_bytes()
// bytes, after verify_check.  The arrival counters are cleared by the
// first launch, so the workspace needs no initial contents.
static int verify_run(const float* target_logits, const float* draft_logits,
                      const int32_t* drafts, const int32_t* row_start, const int32_t* seq_id,
                      const int32_t* pos0, int B, int V, int max_rows, float temperature,
                      uint64_t seed, int32_t* accept_len, int32_t* out_tokens, void* ws,
                      hipStream_t st, int32_t* seq_len = nullptr, int32_t* pos_id = nullptr) {
  const bool greedy = temperature == 0.f;
  if (!aligned(ws, 16)) return ISD_EINVAL;
  const int nch = (V + kCh - 1) / kCh;
  if (greedy) {
    hipLaunchKernelGGL(argmax_slices_kernel, dim3(nch, max_rows), dim3(kVThreads), 0, st,
                       target_logits, row_start, B, V, nch, (unsigned long long*)ws);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(greedy_accept_kernel, dim3(B), dim3(kVThreads), 0, st,
                       (const unsigned long long*)ws, drafts, row_start, B, nch, max_rows,
                       accept_len, out_tokens, seq_len, pos_id);
  } else {
    const size_t cs_bytes = round_up((size_t)(2 * max_rows) * nch * sizeof(float2), 256);
    const size_t rs_bytes = round_up((size_t)B * nch * sizeof(float), 256);
    float2* cs = (float2*)ws;
    float* rsum = (float*)((char*)ws + cs_bytes);
    float* psum = (float*)((char*)ws + cs_bytes + rs_bytes);
    uint32_t* cnt = (uint32_t*)((char*)ws + cs_bytes + 2 * rs_bytes);
    const float invT = 1.0f / temperature;
    const int vec = (V % 4) == 0 && aligned(target_logits, 16) && aligned(draft_logits, 16);
    hipLaunchKernelGGL(chunk_stats_kernel, dim3(nch, 2 * max_rows), dim3(kVThreads), 0, st,
                       target_logits, draft_logits, row_start, B, V, max_rows, nch, invT, cs, cnt);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(decide_draw_kernel, dim3(nch, B), dim3(kVThreads), 0, st, target_logits,
                       draft_logits, drafts, row_start, seq_id, pos0, B, V, max_rows, nch, invT, seed,
                       vec, (const float2*)cs, rsum, psum, cnt, accept_len, out_tokens, seq_len,
                       pos_id);
  }
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

}  // namespace isd

extern "C" int spec_verify(const float* target_logits, const float* draft_logits,
                           const int32_t* drafts, const int32_t* row_start, const int32_t* seq_id,
                           const int32_t* pos0, int B, int V, int max_rows, float temperature,
                           uint64_t seed, int32_t* accept_len, int32_t* out_tokens, void* ws,
                           size_t* ws_bytes, void* stream) {
  using namespace isd;
  if (!ws_bytes) return ISD_EINVAL;
  const size_t need = verify_ws_bytes(B, V, max_rows, temperature);
  if (need == 0) return ISD_EINVAL;
  if (!ws) {
    *ws_bytes = need;
    return ISD_OK;
  }
  if (*ws_bytes < need) {
    *ws_bytes = need;
    return ISD_ENOSPC;
  }
  const int err = verify_check(target_logits, draft_logits, drafts, row_start, seq_id, pos0,
                               temperature, accept_len, out_tokens);
  if (err != ISD_OK) return err;
  return verify_run(target_logits, draft_logits, drafts, row_start, seq_id, pos0, B, V, max_rows,
                    temperature, seed, accept_len, out_tokens, ws, (hipStream_t)stream);
}

// ------------------------------------------------ spec_verify_noalloc
//
// spec_verify for callers that cannot allocate (code under graph capture,
// tight serving loops): the workspace is this file-scope device array, one
// copy per GPU that loads the library, held until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol): its device address is looked up once per
// device with hipGetSymbolAddress and kept.  Every call on a GPU shares
// that GPU's copy, so calls that overlap on one GPU race.
static __device__ __align__(256) unsigned char scratch[ISD_VERIFY_SCRATCH_BYTES];

namespace isd {

static std::mutex scratch_mu;
static std::atomic<void*> scratch_dev[kMaxDevices];

// Device address of `scratch` on the current device, or NULL on failure.
static void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_dev[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(scratch_mu);
  p = scratch_dev[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_dev[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace isd

extern "C" int spec_verify_noalloc(const float* target_logits, const float* draft_logits,
                                   const int32_t* drafts, const int32_t* row_start,
                                   const int32_t* seq_id, const int32_t* pos0, int B, int V,
                                   int max_rows, float temperature, uint64_t seed,
                                   int32_t* accept_len, int32_t* out_tokens, void* stream) {
  using namespace isd;
  const size_t need = verify_ws_bytes(B, V, max_rows, temperature);
  if (need == 0) return ISD_EINVAL;
  if (need > (size_t)ISD_VERIFY_SCRATCH_BYTES) return ISD_ENOSPC;
  const int err = verify_check(target_logits, draft_logits, drafts, row_start, seq_id, pos0,
                               temperature, accept_len, out_tokens);
  if (err != ISD_OK) return err;
  void* ws = scratch_ptr();
  if (!ws) return ISD_EHIP;
  return verify_run(target_logits, draft_logits, drafts, row_start, seq_id, pos0, B, V, max_rows,
                    temperature, seed, accept_len, out_tokens, ws, (hipStream_t)stream);
}

extern "C" int spec_verify_keys(const uint64_t* keys, int nkeys, const int32_t* drafts,
                                const int32_t* row_start, int B, int max_rows,
                                int32_t* accept_len, int32_t* out_tokens, int32_t* seq_len,
                                int32_t* pos_id, void* stream) {
  using namespace isd;
  if (!keys || !drafts || !row_start || !accept_len || !out_tokens) return ISD_EINVAL;
  if (B < 1 || nkeys < 1 || max_rows < B || max_rows > ISD_MAX_VERIFY_ROWS) return ISD_EINVAL;
  if ((seq_len == nullptr) != (pos_id == nullptr)) return ISD_EINVAL;
  if (!aligned(keys, 8) || !aligned(drafts, 4) || !aligned(row_start, 4) ||
      !aligned(accept_len, 4) || !aligned(out_tokens, 4) || !aligned(seq_len, 4) ||
      !aligned(pos_id, 4))
    return ISD_EINVAL;
  hipLaunchKernelGGL(greedy_keys_kernel, dim3(B), dim3(kWave * ISD_MAX_OUT), 0, (hipStream_t)stream,
                     (const u64*)keys, nkeys, drafts, row_start, B, max_rows, accept_len, out_tokens,
                     seq_len, pos_id);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int spec_verify_margin(const float* target_logits, const int32_t* drafts,
                                  const int32_t* row_start, int B, int V, int max_rows,
                                  float threshold, int32_t* accept_len, int32_t* out_tokens,
                                  float* margins, int32_t* recheck, void* ws, size_t* ws_bytes,
                                  void* stream) {
  using namespace isd;
  if (!ws_bytes) return ISD_EINVAL;
  if (B < 1 || V < 1 || max_rows < B || max_rows > ISD_MAX_VERIFY_ROWS || threshold != threshold)
    return ISD_EINVAL;
  const int nslice = (V + kCh - 1) / kCh;
  const size_t need = (size_t)max_rows * nslice * 2 * sizeof(unsigned long long);
  if (!ws) {
    *ws_bytes = need;
    return ISD_OK;
  }
  if (*ws_bytes < need) {
    *ws_bytes = need;
    return ISD_ENOSPC;
  }
  if (!target_logits || !drafts || !row_start || !accept_len || !out_tokens || !margins ||
      !recheck)
    return ISD_EINVAL;
  if (!aligned(ws, 16) || !aligned(target_logits, 4) || !aligned(drafts, 4) ||
      !aligned(row_start, 4) || !aligned(accept_len, 4) || !aligned(out_tokens, 4) ||
      !aligned(margins, 4) || !aligned(recheck, 4))
    return ISD_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(argmax_top2_kernel, dim3(nslice, max_rows), dim3(kVThreads), 0, st,
                     target_logits, row_start, B, V, nslice, (unsigned long long*)ws);
  if (hipGetLastError() != hipSuccess) return ISD_EHIP;
  hipLaunchKernelGGL(greedy_margin_kernel, dim3(B), dim3(kVThreads), 0, st,
                     (const unsigned long long*)ws, drafts, row_start, B, nslice, max_rows, threshold,
                     accept_len, out_tokens, margins, recheck);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int spec_verify_commit(const float* target_logits, const int32_t* drafts,
                                  const int32_t* row_start, int B, int V, int max_rows,
                                  int32_t* accept_len, int32_t* out_tokens, int32_t* seq_len,
                                  int32_t* pos_id, void* ws, size_t* ws_bytes, void* stream) {
  using namespace isd;
  if (!ws_bytes) return ISD_EINVAL;
  if (B < 1 || V < 1 || max_rows < B || max_rows > ISD_MAX_VERIFY_ROWS) return ISD_EINVAL;
  const int nch = (V + kCh - 1) / kCh;
  const size_t need = (size_t)max_rows * nch * sizeof(unsigned long long);
  if (!ws) {
    *ws_bytes = need;
    return ISD_OK;
  }
  if (*ws_bytes < need) {
    *ws_bytes = need;
    return ISD_ENOSPC;
  }
  if (!target_logits || !drafts || !row_start || !accept_len || !out_tokens || !seq_len ||
      !pos_id)
    return ISD_EINVAL;
  if (!aligned(ws, 16) || !aligned(target_logits, 4) || !aligned(drafts, 4) ||
      !aligned(row_start, 4) || !aligned(accept_len, 4) || !aligned(out_tokens, 4) ||
      !aligned(seq_len, 4) || !aligned(pos_id, 4))
    return ISD_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(argmax_slices_kernel, dim3(nch, max_rows), dim3(kVThreads), 0, st,
                     target_logits, row_start, B, V, nch, (unsigned long long*)ws);
  if (hipGetLastError() != hipSuccess) return ISD_EHIP;
  hipLaunchKernelGGL(greedy_accept_kernel, dim3(B), dim3(kVThreads), 0, st,
                     (const unsigned long long*)ws, drafts, row_start, B, nch, max_rows, accept_len,
                     out_tokens, seq_len, pos_id);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

// ---------------------------------------------- spec_verify_sampled_commit
//
// The rejection-sampling verify with kv_commit's COMMIT done by the
// work-group that draws each sequence's token, so a sampled verify pass
// needs no commit launch.  pos0 is pos_id, read by every work-group before
// the sequence's last work-group advances it.

extern "C" int spec_verify_sampled_commit(const float* target_logits, const float* draft_logits,
                                          const int32_t* drafts, const int32_t* row_start,
                                          const int32_t* seq_id, int B, int V, int max_rows,
                                          float temperature, uint64_t seed, int32_t* accept_len,
                                          int32_t* out_tokens, int32_t* seq_len, int32_t* pos_id,
                                          void* ws, size_t* ws_bytes, void* stream) {
  using namespace isd;
  if (!ws_bytes || !(temperature > 0.f)) return ISD_EINVAL;
  const size_t need = verify_ws_bytes(B, V, max_rows, temperature);
  if (need == 0) return ISD_EINVAL;
  if (!ws) {
    *ws_bytes = need;
    return ISD_OK;
  }
  if (*ws_bytes < need) {
    *ws_bytes = need;
    return ISD_ENOSPC;
  }
  if (!seq_len || !aligned(seq_len, 4)) return ISD_EINVAL;
  const int err = verify_check(target_logits, draft_logits, drafts, row_start, seq_id, pos_id,
                               temperature, accept_len, out_tokens);
  if (err != ISD_OK) return err;
  return verify_run(target_logits, draft_logits, drafts, row_start, seq_id, pos_id, B, V, max_rows,
                    temperature, seed, accept_len, out_tokens, ws, (hipStream_t)stream, seq_len,
                    pos_id);
}
