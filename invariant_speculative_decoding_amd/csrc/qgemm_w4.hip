// qgemm_w4: y[c][r] = sum_k W[r][k] x[c][k] with W in the 4-bit block format
// (32-value blocks, fp16 scale d and minimum m, w = d*q + m).
//
// Batch invariance (ramgpt.org, "When Lossless Speculation Stops Being
// Lossless on Blackwell", section "Quantized Matrix Multiplication Shows
// the Same Class of Failure"; tokenstrom.com, "'Lossless,' but not quite",
// section "Why the math checks out and the text still flips": the mat-vec
// for one token and for eight used different warp counts and so summed
// partials in a different order).  Here one geometry serves every width:
//
//  * A 16x16x32 bf16 MFMA tile always has 16 activation slots (M) against
//    16 weight rows (N); a call with n < 16 rows fills the other slots with
//    zeros.  Each output element of an MFMA depends only on its own A row
//    and B column, so what the other slots hold cannot touch a row's bits.
//  * One MFMA covers exactly one 32-value block (K = 32), so the per-block
//    scale and minimum are applied to the block's exact partial sum.  The
//    codes enter as bf16 values 128 + q (bit pattern 0x4300 | q, one AND-OR
//    per pair); the block result is d * sum((128+q) x) + (m - 128 d) *
//    sum(x), where sum(x) comes from an MFMA against a tile of ones.
//  * Blocks are accumulated in ascending order inside a wave; a wave owns a
//    fixed, contiguous range of blocks; the `ks` waves of a work-group that
//    split K are summed in wave order through LDS.  (rt, ks) are functions
//    of (N, K, x dtype) only.
//  * fp32 activations are split exactly into three bf16 parts (hi, mid, lo
//    by truncation) and the three MFMAs are chained.
//
// Weights stream from HBM with 16-byte loads: lane (row i, group g) loads
// block b+g of row i, and a register transpose across the four lane groups
// hands every lane its own 8-code slice of four consecutive blocks.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

constexpr uint32_t kMagicPair = 0x43004300u;  // bf16 128.0 in both halves
constexpr uint32_t kOnesPair = 0x3F803F80u;   // bf16 1.0 in both halves

// Codes of one lane's k-group (8 nibbles, element u at bits 4u) as bf16
// values 128+q in k-slot order [e0, e4, e1, e5, e2, e6, e3, e7].
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t cw) {
  u32x4 r;
  r.x = (cw & 0x000F000Fu) | kMagicPair;
  r.y = ((cw >> 4) & 0x000F000Fu) | kMagicPair;
  r.z = ((cw >> 8) & 0x000F000Fu) | kMagicPair;
  r.w = ((cw >> 12) & 0x000F000Fu) | kMagicPair;
  return as_bf16x8(r);
}

// Eight consecutive bf16 activations (x0..x7 in four dwords) reordered to
// the k-slot order [x0, x4, x1, x5, x2, x6, x3, x7] of codes_to_bf16.
__device__ __forceinline__ bf16x8 x_to_slots(u32x4 v) {
  u32x4 r;
  r.x = perm(v.z, v.x, 0x05040100u);
  r.y = perm(v.z, v.x, 0x07060302u);
  r.z = perm(v.w, v.y, 0x05040100u);
  r.w = perm(v.w, v.y, 0x07060302u);
  return as_bf16x8(r);
}

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

template <int XT>
struct XOperand;

// bf16 activations: one A tile per block.
template <>
struct XOperand<ISD_BF16> {
  bf16x8 a[4];
  __device__ __forceinline__ void load(const void* xv, int K, int n, int nb, int b, int c, int g) {
    const uint16_t* x = (const uint16_t*)xv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < n && b + j < nb) v = ld16(x + (size_t)c * K + 32 * (b + j) + 8 * g);
      a[j] = x_to_slots(v);
    }
  }
  __device__ __forceinline__ f32x4 dot(int j, bf16x8 w) const {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return mfma_bf16(a[j], w, z);
  }
};

// fp32 activations: three exact bf16 parts per block, chained MFMAs.
template <>
struct XOperand<ISD_F32> {
  bf16x8 a[4][3];
  __device__ __forceinline__ void load(const void* xv, int K, int n, int nb, int b, int c, int g) {
    const float* x = (const float*)xv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (c < n && b + j < nb) {
        const float* p = x + (size_t)c * K + 32 * (b + j) + 8 * g;
        lo = ld16(p);
        hi = ld16(p + 4);
      }
      const uint32_t v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split3(v[e], h[e], m[e], l[e]);
      // k-slot order [x0, x4, x1, x5, x2, x6, x3, x7]
      u32x4 ph = {h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16)};
      u32x4 pm = {m[0] | (m[4] << 16), m[1] | (m[5] << 16), m[2] | (m[6] << 16), m[3] | (m[7] << 16)};
      u32x4 pl = {l[0] | (l[4] << 16), l[1] | (l[5] << 16), l[2] | (l[6] << 16), l[3] | (l[7] << 16)};
      a[j][0] = as_bf16x8(ph);
      a[j][1] = as_bf16x8(pm);
      a[j][2] = as_bf16x8(pl);
    }
  }
  __device__ __forceinline__ f32x4 dot(int j, bf16x8 w) const {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    z = mfma_bf16(a[j][0], w, z);
    z = mfma_bf16(a[j][1], w, z);
    return mfma_bf16(a[j][2], w, z);
  }
};

// One work-group: ks waves x 64 lanes; it owns rows [row0, row0 + 16 rt).
// Wave w accumulates 4-block steps [w*nsteps/ks, (w+1)*nsteps/ks).
template <int XT, int RT>
__global__ __launch_bounds__(64 * (16 / RT)) void qgemm_w4_kernel(const uint8_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ sm,
                                                        const void* __restrict__ xv,
                                                        float* __restrict__ y, int N, int K,
                                                        int n, int ks) {
  extern __shared__ float red[];  // [ks][RT][32][4] when ks > 1
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;  // A: activation slot; B: weight row in the tile
  const int g = lane >> 4;  // k-group of 8 within a block
  const int nb = K >> 5;
  const int nsteps = (nb + 3) >> 2;
  const int s0 = (int)(((long)wave * nsteps) / ks);
  const int s1 = (int)(((long)(wave + 1) * nsteps) / ks);
  const int row0 = blockIdx.x * (16 * RT);
  const size_t rowbytes = (size_t)K >> 1;
  const bool sm16 = (nb & 3) == 0;

  const bf16x8 ones = as_bf16x8(u32x4{kOnesPair, kOnesPair, kOnesPair, kOnesPair});

  float acc[RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = 0.f;

  for (int s = s0; s < s1; ++s) {
    const int b = 4 * s;
    const int nblk = min(4, nb - b);  // uniform

    XOperand<XT> xo;
    xo.load(xv, K, n, nb, b, c, g);
    f32x4 sx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sx[j] = xo.dot(j, ones);

    u32x4 cw[RT], sc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int r = row0 + 16 * t + c;
      const bool rv = r < N;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rv && g < nblk) v = ld16_stream(codes + (size_t)r * rowbytes + 16 * (b + g));
      cw[t] = v;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (rv) {
        const uint16_t* p = sm + ((size_t)r * nb + b) * 2;
        if (sm16) {
          w = ld16(p);
        } else {
          w.x = ld4(p);
          if (nblk > 1) w.y = ld4(p + 2);
          if (nblk > 2) w.z = ld4(p + 4);
          if (nblk > 3) w.w = ld4(p + 6);
        }
      }
      sc[t] = w;
    }

#pragma unroll
    for (int t = 0; t < RT; ++t) {
      transpose4x4_lanegroups(cw[t]);
      const uint32_t cws[4] = {cw[t].x, cw[t].y, cw[t].z, cw[t].w};
      const uint32_t scs[4] = {sc[t].x, sc[t].y, sc[t].z, sc[t].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < nblk) {
          f32x4 S = xo.dot(j, codes_to_bf16(cws[j]));
          const float d = f16_lo(scs[j]);
          const float mprime = f16_hi(scs[j]) - 128.0f * d;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[t][i] = __builtin_fmaf(d, S[i], acc[t][i]);
            acc[t][i] = __builtin_fmaf(mprime, sx[j][i], acc[t][i]);
          }
        }
      }
    }
  }

  // Lanes 0..31 hold activation slots 4g+i < 8; slots 8..15 are padding.
  if (ks > 1) {
    if (lane < 32) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wave * RT + t) * 32 + lane) * 4 + i] = acc[t][i];
    }
    __syncthreads();
    if (wave != 0) return;
    if (lane < 32) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = red[((0 * RT + t) * 32 + lane) * 4 + i];
          for (int w = 1; w < ks; ++w) v += red[((w * RT + t) * 32 + lane) * 4 + i];
          acc[t][i] = v;
        }
    }
  }
  if (lane < 32) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int r = row0 + 16 * t + c;
      if (r < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = 4 * g + i;
          if (cc < n) y[(size_t)cc * N + r] = acc[t][i];
        }
      }
    }
  }
}

// Work split: rows per work-group (16 rt) and waves splitting K (ks), from
// (N, K, dtype) only.
void qgemm_geometry(int N, int K, int x_dtype, int* rt, int* ks) {
  (void)x_dtype;
  const int nsteps = (K / 32 + 3) / 4;
  int r = 4;
  if (N < 16384) r = 2;
  if (N < 2048) r = 1;
  const int tiles = (N + 16 * r - 1) / (16 * r);
  int k = (3072 + tiles - 1) / tiles;
  if (k > 16 / r) k = 16 / r;  // work-group of at most 64 * 16 / rt lanes
  if (k > nsteps) k = nsteps;
  if (k < 1) k = 1;
  *rt = r;
  *ks = k;
}

template <int XT, int RT>
static hipError_t launch_qgemm(const uint8_t* codes, const uint16_t* sm, const void* x, float* y,
                               int N, int K, int n, int ks, hipStream_t st) {
  const int rows = 16 * RT;
  dim3 grid((N + rows - 1) / rows);
  dim3 block(64 * ks);
  size_t lds = ks > 1 ? (size_t)ks * RT * 32 * 4 * sizeof(float) : 0;
  hipLaunchKernelGGL((qgemm_w4_kernel<XT, RT>), grid, block, lds, st, codes, sm, x, y, N, K, n, ks);
  return hipGetLastError();
}

}  // namespace isd

extern "C" int qgemm_w4(const uint8_t* codes, const uint16_t* scale_min, const void* x,
                        int x_dtype, float* y, int N, int K, int n, void* stream) {
  using namespace isd;
  if (!codes || !scale_min || !x || !y) return ISD_EINVAL;
  if (N < 1 || K < 32 || (K % 32) != 0 || n < 1 || n > ISD_MAX_ROWS) return ISD_EINVAL;
  if (x_dtype != ISD_F32 && x_dtype != ISD_BF16) return ISD_EINVAL;
  if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4)) return ISD_EINVAL;
  if (!aligned(scale_min, ((K / 32) % 4 == 0) ? 16 : 4)) return ISD_EINVAL;
  if ((size_t)N * (size_t)K / 2 > (size_t)1 << 40) return ISD_EINVAL;
  int rt, ks;
  qgemm_geometry(N, K, x_dtype, &rt, &ks);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (x_dtype == ISD_BF16) {
    e = rt == 4 ? launch_qgemm<ISD_BF16, 4>(codes, scale_min, x, y, N, K, n, ks, st)
      : rt == 2 ? launch_qgemm<ISD_BF16, 2>(codes, scale_min, x, y, N, K, n, ks, st)
                : launch_qgemm<ISD_BF16, 1>(codes, scale_min, x, y, N, K, n, ks, st);
  } else {
    e = rt == 4 ? launch_qgemm<ISD_F32, 4>(codes, scale_min, x, y, N, K, n, ks, st)
      : rt == 2 ? launch_qgemm<ISD_F32, 2>(codes, scale_min, x, y, N, K, n, ks, st)
                : launch_qgemm<ISD_F32, 1>(codes, scale_min, x, y, N, K, n, ks, st);
  }
  return e == hipSuccess ? ISD_OK : ISD_EHIP;
}
