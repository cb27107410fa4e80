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

// grid = B, block = 64.  Greedy accept-prefix per sequence.
__global__ __launch_bounds__(64) void greedy_accept_kernel(const unsigned long long* __restrict__ ws,
                                                           const int32_t* __restrict__ drafts,
                                                           const int32_t* __restrict__ row_start,
                                                           int nslice, int max_rows,
                                                           int32_t* __restrict__ acc,
                                                           int32_t* __restrict__ out) {
  __shared__ int tgt[ISD_MAX_OUT];
  const int s = blockIdx.x;
  int r0, k;
  seq_layout(row_start, s, max_rows, &r0, &k);
  const int j = threadIdx.x;
  if (j <= k) {
    unsigned long long m = 0ull;
    for (int sl = 0; sl < nslice; ++sl) m = max_u64(m, ws[(size_t)(r0 + j) * nslice + sl]);
    tgt[j] = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int32_t* o = out + (size_t)s * ISD_MAX_OUT;
  if (k < 0) {
    acc[s] = 0;
    for (int e = 0; e < ISD_MAX_OUT; ++e) o[e] = -1;
    return;
  }
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
//  2. resid_chunks: per (sequence, candidate j, chunk) the chunk sum of the
//     distribution a draw at decision j+1 would use -- the residual
//     max(0, p_{j+1} - q_{j+1}) for j < k, p_{k+1} for j = k -- and of
//     p_{j+1} itself (the fallback when a residual is all zero).  Row
//     statistics are folded from the chunk statistics in ascending order.
//  3. sample_finalize: per sequence, the accept tests in order, then one
//     inverse-CDF draw: the chunk is located from the chunk sums in
//     ascending order and walked entry by entry in ascending id order.
// A chunk's sum and its walk use one summation order: thread t adds its 16
// consecutive entries in order, then the 256 thread sums are added in
// thread order.

constexpr int kCh = 4096;       // vocabulary entries per chunk
constexpr int kPerThread = kCh / kVThreads;
constexpr int kCand = ISD_MAX_OUT;  // candidate distributions per sequence

__device__ __forceinline__ float2 fold_stats(const float2* __restrict__ cs, int nch) {
  float M = -INFINITY, S = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float2 v = cs[c];
    const float Mn = fmaxf(M, v.x);
    S = S * __expf(M - Mn) + v.y * __expf(v.x - Mn);
    M = Mn;
  }
  return make_float2(M, S);
}

__device__ __forceinline__ float prob(const float* z, int v, float T, float2 st) {
  return __expf(z[v] / T - st.x) / st.y;
}

// Entry v of candidate distribution: residual (zq != nullptr) or p.
__device__ __forceinline__ float cand_value(const float* zp, const float* zq, int v, float T,
                                            float2 sp, float2 sq) {
  const float p = prob(zp, v, T, sp);
  return zq ? fmaxf(0.f, p - prob(zq, v, T, sq)) : p;
}

// grid = (nch, 2 * max_rows), block = 256.  cs[row][chunk] = (max, sum).
__global__ __launch_bounds__(256) void chunk_stats_kernel(const float* __restrict__ zt,
                                                          const float* __restrict__ zd,
                                                          const int32_t* __restrict__ row_start,
                                                          int B, int V, int max_rows, int nch,
                                                          float T, float2* __restrict__ cs) {
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
  for (int v = v0 + tid; v < v1; v += kVThreads) m = fmaxf(m, z[v] / T);
  red[tid] = m;
  __syncthreads();
  for (int w = kVThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int v = v0 + tid; v < v1; v += kVThreads) sum += __expf(z[v] / T - M);
  red[tid] = sum;
  __syncthreads();
  for (int w = kVThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = red[tid] + red[tid + w];
    __syncthreads();
  }
  if (tid == 0) cs[(size_t)row * nch + blockIdx.x] = make_float2(M, red[0]);
}

// Sum of one chunk of a candidate distribution in the walk's order.
__device__ __forceinline__ float chunk_sum(const float* zp, const float* zq, int V, int c, float T,
                                           float2 sp, float2 sq, float* red) {
  const int tid = threadIdx.x;
  const int base = c * kCh + tid * kPerThread;
  float t = 0.f;
  for (int e = 0; e < kPerThread; ++e) {
    const int v = base + e;
    if (v < V) t += cand_value(zp, zq, v, T, sp, sq);
  }
  red[tid] = t;
  __syncthreads();
  float total = 0.f;
  if (tid == 0)
    for (int e = 0; e < kVThreads; ++e) total += red[e];
  __syncthreads();
  return total;  // valid in thread 0
}

// grid = (nch, B * kCand), block = 256.
// rsum[s][j][c] = chunk sum of candidate j; psum[s][j][c] = chunk sum of p_{j+1}.
__global__ __launch_bounds__(256) void resid_chunks_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd,
    const int32_t* __restrict__ row_start, int V, int max_rows, int nch, float T,
    const float2* __restrict__ cs, float* __restrict__ rsum, float* __restrict__ psum) {
  __shared__ float red[kVThreads];
  const int s = blockIdx.y / kCand;
  const int j = blockIdx.y % kCand;
  const int c = blockIdx.x;
  int r0, k;
  seq_layout(row_start, s, max_rows, &r0, &k);
  if (j > k) return;
  const int tr = r0 + j;
  const float* zp = zt + (size_t)tr * V;
  const float2 sp = fold_stats(cs + (size_t)tr * nch, nch);
  const float* zq = nullptr;
  float2 sq = make_float2(0.f, 1.f);
  if (j < k) {
    const int dr = r0 - s + j;
    zq = zd + (size_t)dr * V;
    sq = fold_stats(cs + (size_t)(max_rows + dr) * nch, nch);
  }
  const size_t o = ((size_t)s * kCand + j) * nch + c;
  const float rs = chunk_sum(zp, zq, V, c, T, sp, sq, red);
  if (threadIdx.x == 0) rsum[o] = rs;
  if (zq) {
    const float ps = chunk_sum(zp, nullptr, V, c, T, sp, sq, red);
    if (threadIdx.x == 0) psum[o] = ps;
  }
}

// grid = B, block = 256.
__global__ __launch_bounds__(256) void sample_finalize_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ seq_id,
    const int32_t* __restrict__ pos0, int V, int max_rows, int nch, float T, uint64_t seed,
    const float2* __restrict__ cs, const float* __restrict__ rsum, const float* __restrict__ psum,
    int32_t* __restrict__ acc, int32_t* __restrict__ out) {
  __shared__ float red[kVThreads];
  __shared__ int sh_a, sh_rej, sh_use_p, sh_chunk, sh_tok;
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
  if (tid == 0) {
    int a = 0, rej = 0;
    while (a < k) {
      const int x = drafts[dbase + a];
      bool ok = false;
      if (x >= 0 && x < V) {
        const float2 sp = fold_stats(cs + (size_t)(r0 + a) * nch, nch);
        const float2 sq = fold_stats(cs + (size_t)(max_rows + dbase + a) * nch, nch);
        const float p = prob(zt + (size_t)(r0 + a) * V, x, T, sp);
        const float q = prob(zd + (size_t)(dbase + a) * V, x, T, sq);
        const float u = philox_uniform(seed, sid, p0 + (uint32_t)a, 0u);
        ok = u < fminf(1.f, q > 0.f ? p / q : INFINITY);
      }
      if (!ok) {
        rej = 1;
        break;
      }
      ++a;
    }
    // chunk sums of the distribution to draw from, located in ascending order
    const float* sums = rsum + ((size_t)s * kCand + a) * nch;
    float S = 0.f;
    for (int c = 0; c < nch; ++c) S += sums[c];
    int use_p = 0;
    if (rej && !(S > 0.f)) {  // residual all zero: draw from p instead
      use_p = 1;
      sums = psum + ((size_t)s * kCand + a) * nch;
      S = 0.f;
      for (int c = 0; c < nch; ++c) S += sums[c];
    }
    const float t = philox_uniform(seed, sid, p0 + (uint32_t)a, 1u) * S;
    float run = 0.f;
    int cstar = -1, lastpos = -1;
    for (int c = 0; c < nch; ++c) {
      if (sums[c] > 0.f) {
        lastpos = c;
        if (run + sums[c] > t) {
          cstar = c;
          break;
        }
      }
      run += sums[c];
    }
    if (cstar >= 0) {
      sh_t = t - run;
    } else {  // t at or past the rounded total: the last positive entry
      cstar = lastpos;
      sh_t = INFINITY;
    }
    sh_a = a;
    sh_rej = rej;
    sh_use_p = use_p;
    sh_chunk = cstar;
    sh_tok = -1;
  }
  __syncthreads();
  const int a = sh_a;
  const int cstar = sh_chunk;
  if (cstar >= 0) {
    const float* zp = zt + (size_t)(r0 + a) * V;
    const float2 sp = fold_stats(cs + (size_t)(r0 + a) * nch, nch);
    const float* zq = nullptr;
    float2 sq = make_float2(0.f, 1.f);
    if (sh_rej && !sh_use_p) {
      zq = zd + (size_t)(dbase + a) * V;
      sq = fold_stats(cs + (size_t)(max_rows + dbase + a) * nch, nch);
    }
    const float t = sh_t;
    const int base = cstar * kCh + tid * kPerThread;
    float vals[kPerThread];
    float mine = 0.f;
    for (int e = 0; e < kPerThread; ++e) {
      const int v = base + e;
      vals[e] = v < V ? cand_value(zp, zq, v, T, sp, sq) : 0.f;
      mine += vals[e];
    }
    red[tid] = mine;
    __syncthreads();
    if (tid == 0) {
      float run = 0.f;
      for (int e = 0; e < kVThreads; ++e) {
        const float nx = run + red[e];
        red[e] = run;  // exclusive prefix
        run = nx;
      }
    }
    __syncthreads();
    const float before = red[tid];
    const float after = before + mine;
    // The prefix never decreases, so exactly one thread is the first whose
    // range passes t; it walks its entries in ascending id order.
    if (after > t && (tid == 0 || !(before > t))) {
      float run = before;
      for (int e = 0; e < kPerThread; ++e) {
        run += vals[e];
        if (run > t) {
          sh_tok = base + e;
          break;
        }
      }
    }
    __syncthreads();
    if (tid == 0 && sh_tok < 0) {
      // nothing positive at or after t in this chunk: last positive entry
      for (int v = min(V, (cstar + 1) * kCh) - 1; v >= cstar * kCh; --v)
        if (cand_value(zp, zq, v, T, sp, sq) > 0.f) {
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
  const size_t cs_bytes = round_up((size_t)(2 * max_rows) * nch * sizeof(float2), 256);
  const size_t rs_bytes = round_up((size_t)B * kCand * nch * sizeof(float), 256);
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
    hipLaunchKernelGGL(chunk_stats_kernel, dim3(nch, 2 * max_rows), dim3(256), 0, st,
                       target_logits, draft_logits, row_start, B, V, max_rows, nch, temperature,
                       cs);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(resid_chunks_kernel, dim3(nch, B * kCand), dim3(256), 0, st,
                       target_logits, draft_logits, row_start, V, max_rows, nch, temperature,
                       (const float2*)cs, rsum, psum);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(sample_finalize_kernel, dim3(B), dim3(256), 0, st, target_logits,
                       draft_logits, drafts, row_start, seq_id, pos0, V, max_rows, nch,
                       temperature, seed, (const float2*)cs, (const float*)rsum,
                       (const float*)psum, accept_len, out_tokens);
  }
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}
