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

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

constexpr int kSlice = 4096;   // vocabulary entries per argmax work-group
constexpr int kVThreads = 256;

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

// ------------------------------------------------------------------ argmax

__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  uint32_t o;
  if (v != v) {
    o = 0u;  // NaN never wins
  } else {
    uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);  // -0 -> +0
    o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const int src = (__lane_id() ^ m) << 2;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(v >> 32));
    v = max_u64(v, ((unsigned long long)hi << 32) | lo);
  }
  return v;
}

// grid = (slices, max_rows), block = 256.  ws[row][slice] = max key.
__global__ __launch_bounds__(256) void argmax_slices_kernel(const float* __restrict__ z,
                                                            const int32_t* __restrict__ row_start,
                                                            int B, int V, int nslice,
                                                            unsigned long long* __restrict__ ws) {
  __shared__ unsigned long long part[4];
  const int row = blockIdx.y;
  const int R = row_start[B];
  if (row >= R) return;  // row < gridDim.y = max_rows as well
  const int v0 = blockIdx.x * kSlice;
  const float* zr = z + (size_t)row * V;
  unsigned long long best = 0ull;
  for (int v = v0 + threadIdx.x; v < min(V, v0 + kSlice); v += kVThreads)
    best = max_u64(best, argmax_key(zr[v], (uint32_t)v));
  best = wave_max_u64(best);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long m = max_u64(max_u64(part[0], part[1]), max_u64(part[2], part[3]));
    ws[(size_t)row * nslice + blockIdx.x] = m;
  }
}

// First target row and draft count of sequence s; k = -1 marks a sequence
// that cannot be verified (no rows, or rows beyond the sized workspace).
__device__ __forceinline__ void seq_layout(const int32_t* row_start, int s, int max_rows, int* r0,
                                           int* k) {
  const int a = row_start[s], b = row_start[s + 1];
  int n = b - a;
  if (n > ISD_MAX_OUT) n = ISD_MAX_OUT;
  if (a < 0 || a + n > max_rows) n = 0;
  *r0 = a;
  *k = n - 1;
}

// grid = B, block = 64.  Greedy accept-prefix per sequence.  The slice maxima
// of the sequence's rows are gathered by all lanes and reduced with an
// order-free 64-bit LDS max.
__global__ __launch_bounds__(64) void greedy_accept_kernel(const unsigned long long* __restrict__ ws,
                                                           const int32_t* __restrict__ drafts,
                                                           const int32_t* __restrict__ row_start,
                                                           int nslice, int max_rows,
                                                           int32_t* __restrict__ acc,
                                                           int32_t* __restrict__ out) {
  __shared__ unsigned long long best[ISD_MAX_OUT];
  const int s = blockIdx.x;
  int r0, k;
  seq_layout(row_start, s, max_rows, &r0, &k);
  const int t = threadIdx.x;
  if (t < ISD_MAX_OUT) best[t] = 0ull;
  __syncthreads();
  const int total = (k + 1) * nslice;
  for (int e = t; e < total; e += 64) {
    const int j = e / nslice, sl = e % nslice;
    atomicMax(&best[j], ws[(size_t)(r0 + j) * nslice + sl]);
  }
  __syncthreads();
  if (t != 0) return;
  int32_t* o = out + (size_t)s * ISD_MAX_OUT;
  if (k < 0) {
    acc[s] = 0;
    for (int e = 0; e < ISD_MAX_OUT; ++e) o[e] = -1;
    return;
  }
  int tgt[ISD_MAX_OUT];
  for (int j = 0; j <= k; ++j) tgt[j] = (int)(0xFFFFFFFFu - (uint32_t)(best[j] & 0xFFFFFFFFull));
  const int32_t* d = drafts + (r0 - s);
  int a = 0;
  while (a < k && d[a] == tgt[a]) ++a;
  for (int e = 0; e < a; ++e) o[e] = d[e];
  o[a] = tgt[a];
  for (int e = a + 1; e < ISD_MAX_OUT; ++e) o[e] = -1;
  acc[s] = a;
}

// ------------------------------------------------------------------ sampling
//
// Three launches, every reduction in a fixed order:
//  1. chunk_stats: per (row, 4096-entry chunk) the max of z/T and the sum of
//     exp(z/T - max) (strided per-thread sums, then a fixed tree).
//  2. decide_sum: per (sequence, chunk) the accept decisions (row
//     statistics folded from the chunk statistics in ascending order, tests
//     in draft order) and that chunk's sum of the distribution a draw would
//     use -- the residual max(0, p_{a+1} - q_{a+1}) after a rejection at
//     draft a+1, p_{k+1} when all k drafts pass -- plus, after a rejection,
//     of p_{a+1} itself (the fallback when a residual is all zero).
//  3. sample_finalize: per sequence, the same decisions, then one inverse-
//     CDF draw: the chunk is located from the chunk sums in ascending order
//     and walked entry by entry in ascending id order.
// A chunk's sum and its walk use one summation order: thread t adds its 16
// consecutive entries in order, then the 256 thread sums are combined by
// one fixed inclusive scan (Kogge-Stone over 8 doubling steps), whose last
// element is the chunk sum.  Logits are scaled as z * fp32(1/T).

constexpr int kCh = 4096;       // vocabulary entries per chunk
constexpr int kPerThread = kCh / kVThreads;
constexpr int kMaxChunks = kVThreads;  // chunk sums are located with one block scan

// Inclusive prefix sum over the 256 threads of a block in a fixed order;
// `excl` receives the previous thread's inclusive value exactly (0 for
// thread 0) and `total` the last one (the sum of all 256 inputs).
__device__ __forceinline__ float block_incl_scan(float v, float* lds, float& excl, float& total) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < kVThreads; off <<= 1) {
    const float t = tid >= off ? lds[tid - off] : 0.f;
    __syncthreads();
    lds[tid] += t;
    __syncthreads();
  }
  const float r = lds[tid];
  excl = tid > 0 ? lds[tid - 1] : 0.f;
  total = lds[kVThreads - 1];
  __syncthreads();
  return r;
}

// Row statistics (max of z/T, sum of exp(z/T - max)) from the chunk
// statistics, folded in ascending chunk order.  `cs` may be global or LDS.
__device__ __forceinline__ float2 fold_stats(const float2* cs, int nch) {
  float M = -INFINITY, S = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float2 v = cs[c];
    const float Mn = fmaxf(M, v.x);
    S = S * __expf(M - Mn) + v.y * __expf(v.x - Mn);
    M = Mn;
  }
  return make_float2(M, S);
}

__device__ __forceinline__ float prob(const float* z, int v, float invT, float2 st) {
  return __expf(z[v] * invT - st.x) / st.y;
}

// Entry v of candidate distribution: residual (zq != nullptr) or p.
__device__ __forceinline__ float cand_value(const float* zp, const float* zq, int v, float invT,
                                            float2 sp, float2 sq) {
  const float p = prob(zp, v, invT, sp);
  return zq ? fmaxf(0.f, p - prob(zq, v, invT, sq)) : p;
}

// grid = (nch, 2 * max_rows), block = 256.  cs[row][chunk] = (max, sum).
__global__ __launch_bounds__(256) void chunk_stats_kernel(const float* __restrict__ zt,
                                                          const float* __restrict__ zd,
                                                          const int32_t* __restrict__ row_start,
                                                          int B, int V, int max_rows, int nch,
                                                          float invT, float2* __restrict__ cs) {
  __shared__ float red[kVThreads];
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
  const int tid = threadIdx.x;
  const int v0 = blockIdx.x * kCh, v1 = min(V, v0 + kCh);
  float m = -INFINITY;
  for (int v = v0 + tid; v < v1; v += kVThreads) m = fmaxf(m, z[v] * invT);
  red[tid] = m;
  __syncthreads();
  for (int w = kVThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int v = v0 + tid; v < v1; v += kVThreads) sum += __expf(z[v] * invT - M);
  red[tid] = sum;
  __syncthreads();
  for (int w = kVThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = red[tid] + red[tid + w];
    __syncthreads();
  }
  if (tid == 0) cs[(size_t)row * nch + blockIdx.x] = make_float2(M, red[0]);
}

// Sum of one chunk of a candidate distribution in the walk's order (every
// thread returns it).
__device__ __forceinline__ float chunk_sum(const float* zp, const float* zq, int V, int c,
                                           float invT, float2 sp, float2 sq, float* red) {
  const int base = c * kCh + threadIdx.x * kPerThread;
  float t = 0.f;
  for (int e = 0; e < kPerThread; ++e) {
    const int v = base + e;
    if (v < V) t += cand_value(zp, zq, v, invT, sp, sq);
  }
  float excl, total;
  block_incl_scan(t, red, excl, total);
  return total;
}

// Accept decisions of one sequence (identical in every work-group that
// makes them: same inputs, same instructions).  Folds the chunk statistics
// of the sequence's k+1 target and k draft rows (staged in LDS, one row per
// thread), then runs the tests in draft order on thread 0.  Leaves a,
// rejected and the row statistics in LDS.
struct Decision {
  int a, rej;
  float2 st[2 * ISD_MAX_OUT];  // target rows 0..k, then draft rows at ISD_MAX_OUT + j
};

__device__ void decide(const float* __restrict__ zt, const float* __restrict__ zd,
                       const int32_t* __restrict__ drafts, const float2* __restrict__ cs,
                       int r0, int k, int dbase, int V, int max_rows, int nch, float invT,
                       uint64_t seed, uint32_t sid, uint32_t p0, float2* stage, Decision* dec) {
  const int tid = threadIdx.x;
  const int nrow = 2 * k + 1;  // targets 0..k, drafts k+1..2k
  for (int e = tid; e < nrow * nch; e += kVThreads) {
    const int r = e / nch, c = e % nch;
    const size_t row = r <= k ? (size_t)(r0 + r) : (size_t)(max_rows + dbase + (r - k - 1));
    stage[e] = cs[row * nch + c];
  }
  __syncthreads();
  if (tid < nrow) {
    const float2 st = fold_stats(stage + tid * nch, nch);
    dec->st[tid <= k ? tid : ISD_MAX_OUT + (tid - k - 1)] = st;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0, rej = 0;
    while (a < k) {
      const int x = drafts[dbase + a];
      bool ok = false;
      if (x >= 0 && x < V) {
        const float p = prob(zt + (size_t)(r0 + a) * V, x, invT, dec->st[a]);
        const float q = prob(zd + (size_t)(dbase + a) * V, x, invT, dec->st[ISD_MAX_OUT + a]);
        const float u = philox_uniform(seed, sid, p0 + (uint32_t)a, 0u);
        ok = u < fminf(1.f, q > 0.f ? p / q : INFINITY);
      }
      if (!ok) {
        rej = 1;
        break;
      }
      ++a;
    }
    dec->a = a;
    dec->rej = rej;
  }
  __syncthreads();
}

// grid = (nch, B), block = 256.  Every chunk's work-group of a sequence
// takes the same accept decisions, then sums its chunk of the distribution
// to draw from (residual of decision a+1, or p_{k+1} when all drafts pass)
// and of p_{a+1} (the fallback for an all-zero residual).
__global__ __launch_bounds__(256) void decide_sum_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ seq_id,
    const int32_t* __restrict__ pos0, int V, int max_rows, int nch, float invT, uint64_t seed,
    const float2* __restrict__ cs, float* __restrict__ rsum, float* __restrict__ psum) {
  __shared__ float red[kVThreads];
  __shared__ float2 stage[(2 * ISD_MAX_OUT - 1) * kMaxChunks];
  __shared__ Decision dec;
  const int c = blockIdx.x;
  const int s = blockIdx.y;
  int r0, k;
  seq_layout(row_start, s, max_rows, &r0, &k);
  if (k < 0) return;
  const int dbase = r0 - s;
  decide(zt, zd, drafts, cs, r0, k, dbase, V, max_rows, nch, invT, seed, (uint32_t)seq_id[s],
         (uint32_t)pos0[s], stage, &dec);
  const int a = dec.a;
  const float* zp = zt + (size_t)(r0 + a) * V;
  const float2 sp = dec.st[a];
  const size_t o = (size_t)s * nch + c;
  if (dec.rej) {  // uniform
    const float* zq = zd + (size_t)(dbase + a) * V;
    const float rs = chunk_sum(zp, zq, V, c, invT, sp, dec.st[ISD_MAX_OUT + a], red);
    const float ps = chunk_sum(zp, nullptr, V, c, invT, sp, sp, red);
    if (threadIdx.x == 0) {
      rsum[o] = rs;
      psum[o] = ps;
    }
  } else {
    const float rs = chunk_sum(zp, nullptr, V, c, invT, sp, sp, red);
    if (threadIdx.x == 0) rsum[o] = rs;
  }
}

// grid = B, block = 256.  Same decisions again, then one inverse-CDF draw:
// the chunk is located from the chunk sums in ascending order and walked
// entry by entry in ascending id order.
__global__ __launch_bounds__(256) void sample_finalize_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ seq_id,
    const int32_t* __restrict__ pos0, int V, int max_rows, int nch, float invT, uint64_t seed,
    const float2* __restrict__ cs, const float* __restrict__ rsum,
    const float* __restrict__ psum, int32_t* __restrict__ acc, int32_t* __restrict__ out) {
  __shared__ float red[kVThreads];
  __shared__ float2 stage[(2 * ISD_MAX_OUT - 1) * kMaxChunks];
  __shared__ Decision dec;
  __shared__ int sh_chunk, sh_tok;
  __shared__ float sh_t;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  int r0, k;
  seq_layout(row_start, s, max_rows, &r0, &k);
  int32_t* o = out + (size_t)s * ISD_MAX_OUT;
  if (k < 0) {
    if (tid == 0) {
      acc[s] = 0;
      for (int e = 0; e < ISD_MAX_OUT; ++e) o[e] = -1;
    }
    return;
  }
  const int dbase = r0 - s;
  const uint32_t sid = (uint32_t)seq_id[s];
  const uint32_t p0 = (uint32_t)pos0[s];
  decide(zt, zd, drafts, cs, r0, k, dbase, V, max_rows, nch, invT, seed, sid, p0, stage, &dec);
  const int a = dec.a;
  const int rej = dec.rej;
  if (tid == 0) sh_tok = -1;
  // ---- chunk sums of the distribution to draw from; an all-zero residual
  // falls back to p_{a+1}
  const float u2 = philox_uniform(seed, sid, p0 + (uint32_t)a, 1u);
  const float* sums = rsum + (size_t)s * nch;
  float S, cexcl;
  float cincl = block_incl_scan(tid < nch ? sums[tid] : 0.f, red, cexcl, S);
  int use_q = rej;
  if (rej && !(S > 0.f)) {
    use_q = 0;
    sums = psum + (size_t)s * nch;
    cincl = block_incl_scan(tid < nch ? sums[tid] : 0.f, red, cexcl, S);
  }
  const float t = u2 * S;
  {
    const float before = cexcl;
    if (tid == 0) sh_chunk = -1;
    __syncthreads();
    // the first chunk whose inclusive sum passes t (prefixes never decrease
    // and `before` is exactly the previous inclusive value: one thread)
    if (tid < nch && cincl > t && !(before > t)) {
      sh_chunk = tid;
      sh_t = t - before;
    }
    __syncthreads();
    if (tid == 0 && sh_chunk < 0) {  // t at or past the rounded total
      for (int c = nch - 1; c >= 0; --c)
        if (sums[c] > 0.f) {
          sh_chunk = c;
          sh_t = INFINITY;
          break;
        }
    }
    __syncthreads();
  }
  const int cstar = sh_chunk;
  if (cstar >= 0) {
    const float* zp = zt + (size_t)(r0 + a) * V;
    const float2 sp = dec.st[a];
    const float* zq = use_q ? zd + (size_t)(dbase + a) * V : nullptr;
    const float2 sq = use_q ? dec.st[ISD_MAX_OUT + a] : sp;
    const float tc = sh_t;
    const int base = cstar * kCh + tid * kPerThread;
    float vals[kPerThread];
    float mine = 0.f;
    for (int e = 0; e < kPerThread; ++e) {
      const int v = base + e;
      vals[e] = v < V ? cand_value(zp, zq, v, invT, sp, sq) : 0.f;
      mine += vals[e];
    }
    float before, total;
    const float after = block_incl_scan(mine, red, before, total);
    (void)total;
    // The prefix never decreases, so exactly one thread is the first whose
    // range passes t; it walks its entries in ascending id order.
    if (after > tc && (tid == 0 || !(before > tc))) {
      float run = before;
      for (int e = 0; e < kPerThread; ++e) {
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
      for (int v = min(V, (cstar + 1) * kCh) - 1; v >= cstar * kCh; --v)
        if (cand_value(zp, zq, v, invT, sp, sq) > 0.f) {
          sh_tok = v;
          break;
        }
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int32_t* d = drafts + dbase;
    for (int e = 0; e < a; ++e) o[e] = d[e];
    o[a] = sh_tok;
    for (int e = a + 1; e < ISD_MAX_OUT; ++e) o[e] = -1;
    acc[s] = a;
  }
}

}  // namespace isd

extern "C" int spec_verify(const float* target_logits, const float* draft_logits,
                           const int32_t* drafts, const int32_t* row_start, const int32_t* seq_id,
                           const int32_t* pos0, int B, int V, int max_rows, float temperature,
                           uint64_t seed, int32_t* accept_len, int32_t* out_tokens, void* ws,
                           size_t* ws_bytes, void* stream) {
  using namespace isd;
  if (!ws_bytes) return ISD_EINVAL;
  if (B < 1 || V < 1 || max_rows < B || !(temperature >= 0.f) || temperature == INFINITY)
    return ISD_EINVAL;
  const bool greedy = temperature == 0.f;
  const int nslice = (V + kSlice - 1) / kSlice;
  const int nch = (V + kCh - 1) / kCh;
  if (!greedy && nch > kMaxChunks) return ISD_EINVAL;  // V > 1,048,576
  const size_t cs_bytes = round_up((size_t)(2 * max_rows) * nch * sizeof(float2), 256);
  const size_t rs_bytes = round_up((size_t)B * nch * sizeof(float), 256);
  const size_t need = greedy ? (size_t)max_rows * nslice * sizeof(unsigned long long)
                             : cs_bytes + 2 * rs_bytes;
  if (!ws) {
    *ws_bytes = need;
    return ISD_OK;
  }
  if (*ws_bytes < need) {
    *ws_bytes = need;
    return ISD_ENOSPC;
  }
  if (!target_logits || !drafts || !row_start || !accept_len || !out_tokens) return ISD_EINVAL;
  if (!greedy && (!draft_logits || !seq_id || !pos0)) return ISD_EINVAL;
  if (!aligned(ws, 16) || !aligned(target_logits, 4) || !aligned(row_start, 4)) return ISD_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (greedy) {
    hipLaunchKernelGGL(argmax_slices_kernel, dim3(nslice, max_rows), dim3(256), 0, st,
                       target_logits, row_start, B, V, nslice, (unsigned long long*)ws);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(greedy_accept_kernel, dim3(B), dim3(64), 0, st,
                       (const unsigned long long*)ws, drafts, row_start, nslice, max_rows,
                       accept_len, out_tokens);
  } else {
    float2* cs = (float2*)ws;
    float* rsum = (float*)((char*)ws + cs_bytes);
    float* psum = (float*)((char*)ws + cs_bytes + rs_bytes);
    const float invT = 1.0f / temperature;
    hipLaunchKernelGGL(chunk_stats_kernel, dim3(nch, 2 * max_rows), dim3(256), 0, st,
                       target_logits, draft_logits, row_start, B, V, max_rows, nch, invT, cs);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(decide_sum_kernel, dim3(nch, B), dim3(256), 0, st, target_logits,
                       draft_logits, drafts, row_start, seq_id, pos0, V, max_rows, nch, invT, seed,
                       (const float2*)cs, rsum, psum);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(sample_finalize_kernel, dim3(B), dim3(256), 0, st, target_logits,
                       draft_logits, drafts, row_start, seq_id, pos0, V, max_rows, nch, invT,
                       seed, (const float2*)cs, (const float*)rsum, (const float*)psum,
                       accept_len, out_tokens);
  }
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}
