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

// Per-row softmax statistics of y = z / T: (max y, sum exp(y - max)).
// grid = rows (target rows then draft rows), block = 256.
__global__ __launch_bounds__(256) void row_stats_kernel(const float* __restrict__ zt,
                                                        const float* __restrict__ zd,
                                                        const int32_t* __restrict__ row_start,
                                                        int B, int V, int max_rows, float T,
                                                        float2* __restrict__ stats) {
  __shared__ float red[kVThreads];
  const int R = row_start[B];
  int row = blockIdx.x;
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
  float m = -INFINITY;
  for (int v = tid; v < V; v += kVThreads) m = fmaxf(m, z[v] / T);
  red[tid] = m;
  __syncthreads();
  for (int w = kVThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int v = tid; v < V; v += kVThreads) sum += __expf(z[v] / T - M);
  red[tid] = sum;
  __syncthreads();
  for (int w = kVThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = red[tid] + red[tid + w];
    __syncthreads();
  }
  if (tid == 0) stats[blockIdx.x] = make_float2(M, red[0]);
}

__device__ __forceinline__ float prob(const float* z, int v, float T, float2 st) {
  return __expf(z[v] / T - st.x) / st.y;
}

// grid = B, block = 256.  Sequential accept tests, then one inverse-CDF draw.
__global__ __launch_bounds__(256) void sample_accept_kernel(
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ drafts,
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ seq_id,
    const int32_t* __restrict__ pos0, int V, int max_rows, float T, uint64_t seed,
    const float2* __restrict__ stats, int32_t* __restrict__ acc, int32_t* __restrict__ out) {
  __shared__ float seg[kVThreads];
  __shared__ float pre[kVThreads + 1];
  __shared__ int sh_a, sh_rej, sh_tok;
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
  const int dbase = r0 - s;  // first draft entry of this sequence
  const uint32_t sid = (uint32_t)seq_id[s];
  const uint32_t p0 = (uint32_t)pos0[s];
  if (tid == 0) {
    int a = 0, rej = 0;
    while (a < k) {
      const int x = drafts[dbase + a];
      bool ok = false;
      if (x >= 0 && x < V) {
        const float p = prob(zt + (size_t)(r0 + a) * V, x, T, stats[r0 + a]);
        const float q = prob(zd + (size_t)(dbase + a) * V, x, T, stats[max_rows + dbase + a]);
        const float u = philox_uniform(seed, sid, p0 + (uint32_t)a, 0u);
        const float ratio = q > 0.f ? p / q : INFINITY;
        ok = u < fminf(1.f, ratio);
      }
      if (!ok) {
        rej = 1;
        break;
      }
      ++a;
    }
    sh_a = a;
    sh_rej = rej;
  }
  __syncthreads();
  const int a = sh_a;
  const int rej = sh_rej;
  // Distribution to draw from: residual of decision a+1, or bonus p_{k+1}.
  const float* zp = zt + (size_t)(r0 + a) * V;
  const float2 sp = stats[r0 + a];
  const float* zq = rej ? zd + (size_t)(dbase + a) * V : nullptr;
  const float2 sq = rej ? stats[max_rows + dbase + a] : make_float2(0.f, 1.f);
  const float u2 = philox_uniform(seed, sid, p0 + (uint32_t)a, 1u);
  const int L = (V + kVThreads - 1) / kVThreads;
  const int v_lo = min(V, tid * L), v_hi = min(V, v_lo + L);

  for (int pass = 0; pass < 2; ++pass) {
    // pass 0: residual (or p for the bonus); pass 1: p, used when the
    // residual sums to zero.
    const bool use_q = rej && pass == 0;
    float ssum = 0.f;
    for (int v = v_lo; v < v_hi; ++v) {
      const float p = prob(zp, v, T, sp);
      const float r = use_q ? fmaxf(0.f, p - prob(zq, v, T, sq)) : p;
      ssum += r;
    }
    seg[tid] = ssum;
    __syncthreads();
    if (tid == 0) {
      float run = 0.f;
      for (int e = 0; e < kVThreads; ++e) {
        pre[e] = run;
        run += seg[e];
      }
      pre[kVThreads] = run;
      sh_tok = -1;
    }
    __syncthreads();
    const float S = pre[kVThreads];
    if (S > 0.f) {
      const float t = u2 * S;
      // the first segment whose end exceeds t walks its entries
      const bool mine = (pre[tid + 1] > t) && (tid == 0 || pre[tid] <= t) && v_lo < v_hi;
      if (mine) {
        float run = pre[tid];
        int pick = -1, last_pos = -1;
        for (int v = v_lo; v < v_hi; ++v) {
          const float p = prob(zp, v, T, sp);
          const float r = use_q ? fmaxf(0.f, p - prob(zq, v, T, sq)) : p;
          if (r > 0.f) last_pos = v;
          run += r;
          if (run > t) {
            pick = v;
            break;
          }
        }
        sh_tok = pick >= 0 ? pick : last_pos;
      }
      __syncthreads();
      if (sh_tok < 0 && tid == 0) {
        // t reached the end of the walk through rounding: last positive entry
        for (int e = kVThreads - 1; e >= 0 && sh_tok < 0; --e) {
          const int lo = min(V, e * L), hi = min(V, lo + L);
          for (int v = hi - 1; v >= lo; --v) {
            const float p = prob(zp, v, T, sp);
            const float r = use_q ? fmaxf(0.f, p - prob(zq, v, T, sq)) : p;
            if (r > 0.f) {
              sh_tok = v;
              break;
            }
          }
        }
      }
      __syncthreads();
      break;
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
  const size_t need = greedy ? (size_t)max_rows * nslice * sizeof(unsigned long long)
                             : (size_t)(2 * max_rows) * sizeof(float2);
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
    hipLaunchKernelGGL(row_stats_kernel, dim3(2 * max_rows), dim3(256), 0, st, target_logits,
                       draft_logits, row_start, B, V, max_rows, temperature, (float2*)ws);
    if (hipGetLastError() != hipSuccess) return ISD_EHIP;
    hipLaunchKernelGGL(sample_accept_kernel, dim3(B), dim3(256), 0, st, target_logits,
                       draft_logits, drafts, row_start, seq_id, pos0, V, max_rows, temperature,
                       seed, (const float2*)ws, accept_len, out_tokens);
  }
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}
