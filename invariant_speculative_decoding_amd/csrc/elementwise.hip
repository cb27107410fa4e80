// Row-wise operations of a synthetic decoder layer: embedding gather,
// residual add + RMS normalisation, rotary embedding with the q/k/v split,
// and the SiLU-gated product.  They let a whole target model run through
// the library so that the end-to-end property can be checked: speculative
// output equal to serial greedy decoding (ramgpt.org, "When Lossless
// Speculation Stops Being Lossless on Blackwell", sections "Why Tiny
// Numerical Differences Can Change Entire Answers" and "A Better Backend
// Test Matrix").
//
// Every output row is computed by one work-group from that row's inputs
// only, with one fixed reduction order (RMS normalisation), so none of
// these can tell a width-n block from n width-one calls.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

constexpr int kEwThreads = 256;
constexpr int kMaxPerThread = 32;  // H <= 8192

constexpr int kBatch = 8;  // elements per thread whose loads are issued together

// grid = rows, block = 256.  h[r] = table[tokens[r]] (bf16 -> fp32, exact).
// With `vec` (table rows and h rows 16-byte aligned: H % 8 == 0 and both
// bases 16-byte aligned) a thread moves 8 elements per 16-byte load and two
// 16-byte stores, issuing up to four loads before any store; otherwise 8
// single-element loads at a time.  Ids outside [0, V) give zero rows.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const uint16_t* __restrict__ table,
                                                    float* __restrict__ h, int V, int H,
                                                    int vec) {
  const int r = blockIdx.x;
  const int t = tokens[r];
  const bool ok = t >= 0 && t < V;
  const uint16_t* src = table + (size_t)(ok ? t : 0) * H;
  float* dst = h + (size_t)r * H;
  if (vec) {
    constexpr int kLoads = 4;
    const int n8 = H / 8;
    for (int c0 = threadIdx.x; c0 < n8; c0 += kEwThreads * kLoads) {
      u32x4 b[kLoads];
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int c = min(c0 + kEwThreads * u, n8 - 1);
        b[u] = ld16(src + 8 * c);
      }
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int c = c0 + kEwThreads * u;
        if (c < n8) {
          const uint32_t w[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
          f32x4 lo, hi;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            lo[2 * j] = ok ? __builtin_bit_cast(float, w[j] << 16) : 0.f;
            lo[2 * j + 1] = ok ? __builtin_bit_cast(float, w[j] & 0xFFFF0000u) : 0.f;
            hi[2 * j] = ok ? __builtin_bit_cast(float, w[j + 2] << 16) : 0.f;
            hi[2 * j + 1] = ok ? __builtin_bit_cast(float, w[j + 2] & 0xFFFF0000u) : 0.f;
          }
          *(f32x4*)(dst + 8 * c) = lo;
          *(f32x4*)(dst + 8 * c + 4) = hi;
        }
      }
    }
    return;
  }
  for (int c0 = threadIdx.x; c0 < H; c0 += kEwThreads * kBatch) {
    uint16_t b[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + kEwThreads * u;
      b[u] = c < H ? src[c] : (uint16_t)0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + kEwThreads * u;
      if (c < H) dst[c] = ok ? bf16_to_f32(b[u]) : 0.f;
    }
  }
}

// grid = rows, block = 256.  h[r] += d[r] (if d), then y[r] = bf16(h[r] /
// sqrt(mean(h[r]^2) + eps) * w).  The sum of squares: thread t adds
// elements t, t+256, ... in order, a butterfly per wave, the four waves in
// order.  Every load of the row (h, d and w) is issued before the
// arithmetic, and the stores come last.
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(float* __restrict__ h,
                                                          const float* __restrict__ d,
                                                          const float* __restrict__ w,
                                                          uint16_t* __restrict__ y, int H,
                                                          float eps) {
  __shared__ float part[4];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  float* hr = h + (size_t)r * H;
  const float* dr = d ? d + (size_t)r * H : nullptr;
  float v[kMaxPerThread], dv[kMaxPerThread], wv[kMaxPerThread];
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) {
    const int c = tid + kEwThreads * j;
    v[j] = dv[j] = wv[j] = 0.f;
    if (c < H) {
      v[j] = hr[c];
      wv[j] = w[c];
      if (dr) dv[j] = dr[c];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) {
    const int c = tid + kEwThreads * j;
    if (c < H) {
      float x = v[j];
      if (dr) x = x + dv[j];
      v[j] = x;
      ss = __builtin_fmaf(x, x, ss);
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) ss = ss + shfl_xor(ss, m);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float inv = 1.0f / __fsqrt_rn(tot / (float)H + eps);
  uint16_t* yr = y + (size_t)r * H;
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) {
    const int c = tid + kEwThreads * j;
    if (c < H) {
      if (dr) hr[c] = v[j];
      yr[c] = f32_to_bf16(v[j] * inv * wv[j]);
    }
  }
}

// fp64 -> fp16 with a single rounding to nearest even.  The value is first
// rounded to fp32 by rounding to odd (truncated toward zero, lowest bit set
// when inexact), which keeps every bit the fp16 rounding depends on: with
// 24 >= 11 + 2 bits, rounding to odd and then to nearest equals one rounding
// to nearest (Boldo and Melquiond, "When double rounding is odd").  The
// fp32 -> fp16 step is the hardware conversion.
__device__ __forceinline__ _Float16 f64_to_f16(double d) {
  const float f = (float)d;  // nearest
  const double back = (double)f;
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (back != d) {
    if (fabs(back) > fabs(d)) u -= 1u;  // the truncation
    u |= 1u;                            // made odd
  }
  return (_Float16)__builtin_bit_cast(float, u);
}

// grid = rows, block = 256.  Row r of sequence s (row_start[s] <= r <
// row_start[s+1]) sits at position pos_id[s] + (r - row_start[s]).  The
// row [q heads | k heads | v heads] (fp32) is split; the (i, i + D/2) pairs
// of every q and k head are rotated by pos * theta^(-2i/D) (angles and
// rotation in fp64), and all three are rounded to fp16.
__global__ __launch_bounds__(256) void rope_qkv_kernel(const float* __restrict__ qkv,
                                                       const int32_t* __restrict__ row_start,
                                                       const int32_t* __restrict__ pos_id, int B,
                                                       int Hq, int Hkv, int D, double theta,
                                                       uint16_t* __restrict__ q,
                                                       uint16_t* __restrict__ k,
                                                       uint16_t* __restrict__ v) {
  __shared__ double cs[2][64];  // D <= 128
  __shared__ int sh_s;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int half = D / 2;
  if (tid == 0) sh_s = B;
  __syncthreads();
  // the sequence whose rows hold r (the lowest such one if malformed
  // offsets give several)
  for (int s0 = 0; s0 < B; s0 += kEwThreads) {
    const int s = s0 + tid;
    if (s < B && row_start[s] <= r && r < row_start[s + 1]) atomicMin(&sh_s, s);
  }
  __syncthreads();
  const int s = sh_s;
  if (s >= B) return;
  const long pos = (long)pos_id[s] + (r - row_start[s]);
  if (tid < half) {
    const double a = (double)pos * pow(theta, -2.0 * tid / (double)D);
    double sn, c;
    sincos(a, &sn, &c);  // one argument reduction for both
    cs[0][tid] = c;
    cs[1][tid] = sn;
  }
  __syncthreads();
  const int W = (Hq + 2 * Hkv) * D;
  const float* x = qkv + (size_t)r * W;
  const int np = (Hq + 2 * Hkv) * half;  // rotation pairs of the row
  // one rotation pair: (x1, x2) at dims i and i + D/2 of head hd
  auto pair = [&](int e, float x1, float x2) {
    const int hd = e / half, i = e % half;
    _Float16 o1, o2;
    if (hd < Hq + Hkv) {
      const double c = cs[0][i], sn = cs[1][i];
      o1 = f64_to_f16((double)x1 * c - (double)x2 * sn);
      o2 = f64_to_f16((double)x2 * c + (double)x1 * sn);
    } else {
      o1 = (_Float16)x1;
      o2 = (_Float16)x2;
    }
    uint16_t* dst;
    if (hd < Hq)
      dst = q + ((size_t)r * Hq + hd) * D;
    else if (hd < Hq + Hkv)
      dst = k + ((size_t)r * Hkv + (hd - Hq)) * D;
    else
      dst = v + ((size_t)r * Hkv + (hd - Hq - Hkv)) * D;
    dst[i] = __builtin_bit_cast(uint16_t, o1);
    dst[i + half] = __builtin_bit_cast(uint16_t, o2);
  };
  // the loads of 8 pairs per thread are issued before their arithmetic
  for (int e0 = tid; e0 < np; e0 += kEwThreads * kBatch) {
    float y1[kBatch], y2[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = min(e0 + kEwThreads * u, np - 1);
      const int hd = e / half, i = e % half;
      y1[u] = x[hd * D + i];
      y2[u] = x[hd * D + i + half];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = e0 + kEwThreads * u;
      if (e < np) pair(e, y1[u], y2[u]);
    }
  }
}

// grid = (ceil(F / 256), rows), block = 256.  y[r][i] = bf16(silu(g) * u)
// for g = gu[r][i], u = gu[r][F + i], silu(g) = g / (1 + e^-g).
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ gu,
                                                       uint16_t* __restrict__ y, int F) {
  const int r = blockIdx.y;
  const int i = blockIdx.x * kEwThreads + threadIdx.x;
  if (i >= F) return;
  const float g = gu[(size_t)r * 2 * F + i];
  const float u = gu[(size_t)r * 2 * F + F + i];
  y[(size_t)r * F + i] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
}

}  // namespace isd

extern "C" int embed_rows(const int32_t* tokens, const uint16_t* table, float* h, int rows,
                          int V, int H, void* stream) {
  using namespace isd;
  if (!tokens || !table || !h || rows < 1 || V < 1 || H < 1) return ISD_EINVAL;
  if (!aligned(tokens, 4) || !aligned(table, 2) || !aligned(h, 4)) return ISD_EINVAL;
  const int vec = (H % 8) == 0 && aligned(table, 16) && aligned(h, 16);
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(kEwThreads), 0, (hipStream_t)stream, tokens,
                     table, h, V, H, vec);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int add_rmsnorm(float* h, const float* d, const float* w, uint16_t* y, int rows, int H,
                           float eps, void* stream) {
  using namespace isd;
  if (!h || !w || !y || rows < 1 || H < 1 || H > kEwThreads * kMaxPerThread) return ISD_EINVAL;
  if (!(eps >= 0.f)) return ISD_EINVAL;
  if (!aligned(h, 4) || !aligned(w, 4) || !aligned(y, 2) || (d && !aligned(d, 4)))
    return ISD_EINVAL;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(rows), dim3(kEwThreads), 0, (hipStream_t)stream, h,
                     d, w, y, H, eps);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int rope_qkv(const float* qkv, const int32_t* row_start, const int32_t* pos_id, int B,
                        int rows, int Hq, int Hkv, int D, float theta, uint16_t* q, uint16_t* k,
                        uint16_t* v, void* stream) {
  using namespace isd;
  if (!qkv || !row_start || !pos_id || !q || !k || !v) return ISD_EINVAL;
  if (B < 1 || rows < 1 || Hq < 1 || Hkv < 1 || D < 2 || D > 128 || (D % 2) != 0)
    return ISD_EINVAL;
  if (!(theta > 1.f)) return ISD_EINVAL;
  if (((long)Hq + 2L * Hkv) * D > 0x7FFFFFFFL) return ISD_EINVAL;  // a row indexes in 32 bits
  if (!aligned(qkv, 4) || !aligned(row_start, 4) || !aligned(pos_id, 4) || !aligned(q, 2) ||
      !aligned(k, 2) || !aligned(v, 2))
    return ISD_EINVAL;
  hipLaunchKernelGGL(rope_qkv_kernel, dim3(rows), dim3(kEwThreads), 0, (hipStream_t)stream, qkv,
                     row_start, pos_id, B, Hq, Hkv, D, (double)theta, q, k, v);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int silu_mul(const float* gu, uint16_t* y, int rows, int F, void* stream) {
  using namespace isd;
  if (!gu || !y || rows < 1 || F < 1) return ISD_EINVAL;
  if (!aligned(gu, 4) || !aligned(y, 2)) return ISD_EINVAL;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)(((long)F + kEwThreads - 1) / kEwThreads), rows),
                     dim3(kEwThreads), 0, (hipStream_t)stream, gu, y, F);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}
