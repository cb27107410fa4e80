// qgemm_q6: y[c][r] = sum_k W[r][k] x[c][k] with W in the 6-bit super-block
// format: 256-value super-blocks with an fp16 scale d, 16-value sub-blocks
// with a signed 8-bit scale s, w = d * s * (q - 32) for codes q in 0..63.
// The pages name this K-quant format beside the 4-bit one as the formats
// whose mat-vec sums its partials in a different order at width one and at
// width eight (tokenstrom.com, "'Lossless,' but not quite", section "Why
// the math checks out and the text still flips").
//
// Same width-independent idea as the 4-bit kernel (qgemm_w4_kernel.hpp): one
// geometry per (N, K, x dtype), a fixed per-row summation order, and an
// MFMA tile whose slot count does not depend on the number of activation
// rows.  What changes with the format:
//
//  * One 16x16x32 bf16 MFMA covers two 16-value sub-blocks for 8 activation
//    slots: MFMA rows 0-7 hold the 8 slots' activations of the even
//    sub-block in K positions 0-15 (zeros in 16-31), rows 8-15 the same
//    slots' activations of the odd sub-block in positions 16-31.  Output
//    rows 0-7 are then the even sub-block's exact partial sums and rows 8-15
//    the odd one's, so every sub-block's scale multiplies that sub-block's
//    own sum and each lane applies a single scale.  Activation rows fill the
//    8 slots 8 at a time (one slot group per grid row; a group with fewer
//    rows repeats its last one), and an MFMA output element depends only on
//    its own A row and B column, so a row's bits cannot depend on the width.
//  * Codes enter as bf16 values 128 + q (bit pattern 0x4300 | q, q < 64).
//    The offset is a constant of the format and is folded into the
//    accumulator the code MFMA starts from: N = sum over the sub-block of
//    -160 x (one MFMA of the activations against a constant -160 operand,
//    shared by every row tile of the wave), and C = N + sum (128 + q) x =
//    sum (q - 32) x.
//  * The sub-block result is scaled by c = d * s (four fp32 FMAs per lane
//    and sub-block pair, in ascending pair order); c is exact in fp32 (an
//    fp16 times an 8-bit integer), computed as fma(d, s + 128, -128 d) from
//    the stored biased byte.
//  * At the end the even and odd halves of each slot are added (even +
//    odd), the waves that split K are summed in wave order through LDS, and
//    128-input steps are accumulated in ascending order inside a wave.
//
// Weights stream in the packed layout written by qgemm_q6_pack: for every
// 16-row tile and 128-input step, one contiguous 1536-byte run of codes in
// MFMA lane order (1 KB of 16-byte lane slices, then 512 bytes of 8-byte
// slices), a 128-byte run of sub-block scales and, per super-block, a
// 32-byte run of d values.  Lane i + 16g holds, for each of the step's four
// sub-block pairs p, the eight codes of inputs 8(g & 1) .. 8(g & 1) + 7 of
// sub-block 2p + (g >> 1) of row i: three 32-bit words per two pairs, words
// k = 0..2 carrying four codes in the low six bits of each byte and two
// bits of the fourth code word in the top two, so a byte mask yields three
// code words and three shifts and masks the fourth.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

constexpr uint32_t kMinus160Pair = 0xC320C320u;  // bf16 -160.0 in both halves

// Four code words from the three packed words (see above).
__device__ __forceinline__ void q6_unpack(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t (&cd)[4]) {
  cd[0] = p0 & 0x3F3F3F3Fu;
  cd[1] = p1 & 0x3F3F3F3Fu;
  cd[2] = p2 & 0x3F3F3F3Fu;
  cd[3] = ((p0 >> 6) & 0x03030303u) | ((p1 >> 4) & 0x0C0C0C0Cu) | ((p2 >> 2) & 0x30303030u);
}

template <int XT>
struct Q6X;

// Whether lane (c, g) carries activations: MFMA row c < 8 (even sub-block)
// uses K groups 0 and 1, row c >= 8 (odd sub-block) groups 2 and 3.
__device__ __forceinline__ bool q6_active(int c, int g) { return (c >> 3) == (g >> 1); }

// bf16 activations: one A operand per sub-block pair.  Lane (c, g) loads
// inputs 8(g & 1)..+7 of sub-block 2p + (c >> 3) for slot c & 7 (its row
// of the slot group) and keeps them only where active.
template <>
struct Q6X<ISD_BF16> {
  bf16x8 a[4];
  __device__ __forceinline__ void load(const void* xv, int K, int xr, int s, int c, int g) {
    const uint16_t* x = (const uint16_t*)xv + (size_t)xr * K + 128 * s + 16 * (c >> 3) + 8 * (g & 1);
    const bool on = q6_active(c, g);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4 v = ld16(x + 32 * p);
      a[p] = as_bf16x8(on ? v : u32x4{0u, 0u, 0u, 0u});
    }
  }
  __device__ __forceinline__ void prepare() {}
  __device__ __forceinline__ f32x4 offset(int p) const {
    const u32x4 m = {kMinus160Pair, kMinus160Pair, kMinus160Pair, kMinus160Pair};
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return mfma_bf16(a[p], as_bf16x8(m), z);
  }
  __device__ __forceinline__ f32x4 dot(int p, bf16x8 w, f32x4 c) const {
    return mfma_bf16(a[p], w, c);
  }
};

// fp32 activations: three exact bf16 parts per pair, chained MFMAs.
template <>
struct Q6X<ISD_F32> {
  bf16x8 a[4][3];
  u32x4 raw[4][2];
  bool on;
  __device__ __forceinline__ void load(const void* xv, int K, int xr, int s, int c, int g) {
    const float* x = (const float*)xv + (size_t)xr * K + 128 * s + 16 * (c >> 3) + 8 * (g & 1);
    on = q6_active(c, g);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      raw[p][0] = ld16(x + 32 * p);
      raw[p][1] = ld16(x + 32 * p + 4);
    }
  }
  __device__ __forceinline__ void prepare() {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4 lo = raw[p][0], hi = raw[p][1];
      const uint32_t v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        split3(on ? v[e] : 0u, h[e], m[e], l[e]);
      }
      a[p][0] = as_bf16x8(u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
      a[p][1] = as_bf16x8(u32x4{m[0] | (m[1] << 16), m[2] | (m[3] << 16), m[4] | (m[5] << 16), m[6] | (m[7] << 16)});
      a[p][2] = as_bf16x8(u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)});
    }
  }
  __device__ __forceinline__ f32x4 offset(int p) const {
    const u32x4 m = {kMinus160Pair, kMinus160Pair, kMinus160Pair, kMinus160Pair};
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    z = mfma_bf16(a[p][0], as_bf16x8(m), z);
    z = mfma_bf16(a[p][1], as_bf16x8(m), z);
    return mfma_bf16(a[p][2], as_bf16x8(m), z);
  }
  __device__ __forceinline__ f32x4 dot(int p, bf16x8 w, f32x4 c) const {
    c = mfma_bf16(a[p][0], w, c);
    c = mfma_bf16(a[p][1], w, c);
    return mfma_bf16(a[p][2], w, c);
  }
};

// Registers of one 128-input step.
template <int XT, int RT>
struct Q6Step {
  Q6X<XT> xo;
  u32x4 ca[RT];   // P00 P01 P02 P10 of the lane
  u32x2 cb[RT];   // P11 P12
  uint32_t su[RT];  // the lane's four biased sub-block scales (pairs 0..3)
  uint32_t dd[RT];
};

struct Q6Ptrs {
  const uint8_t* codes;  // [ntiles][nsteps][1536]
  const uint8_t* subs;   // [ntiles][nsteps][16][2][4]
  const uint16_t* sups;  // [ntiles][nsteps / 2][16]
};

template <int XT, int RT>
__device__ __forceinline__ void q6_load_step(Q6Step<XT, RT>& r, const Q6Ptrs& p, const void* xv,
                                             int K, int xr, int ntiles, int nsteps, int s,
                                             int tile0, int lane, int c, int g) {
  r.xo.load(xv, K, xr, s, c, g);
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const size_t tile = (size_t)min(tile0 + t, ntiles - 1);
    const size_t ts = tile * nsteps + s;
    const uint8_t* rec = p.codes + ts * 1536;
    r.ca[t] = ld16_stream(rec + lane * 16);
    r.cb[t] = __builtin_nontemporal_load((const u32x2*)(rec + 1024 + lane * 8));
    r.su[t] = ld4(p.subs + ts * 128 + c * 8 + 4 * (g >> 1));
    r.dd[t] = p.sups[(tile * (nsteps >> 1) + (s >> 1)) * 16 + c];
  }
}

// Codes of one pair as bf16 values 128 + q: code word lo holds elements
// 0..3, hi elements 4..7 of the lane's k-group.
__device__ __forceinline__ bf16x8 q6_pair_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = perm(0x43434343u, lo, 0x04010400u);
  r.y = perm(0x43434343u, lo, 0x04030402u);
  r.z = perm(0x43434343u, hi, 0x04010400u);
  r.w = perm(0x43434343u, hi, 0x04030402u);
  return as_bf16x8(r);
}

template <int XT, int RT>
__device__ __forceinline__ void q6_compute_step(Q6Step<XT, RT>& r, f32x4 (&acc)[RT]) {
  r.xo.prepare();
  f32x4 off[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) off[p] = r.xo.offset(p);
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    uint32_t cd[8];
    uint32_t lo[4], hi[4];
    q6_unpack(r.ca[t].x, r.ca[t].y, r.ca[t].z, lo);
    q6_unpack(r.ca[t].w, r.cb[t].x, r.cb[t].y, hi);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cd[j] = lo[j];
      cd[4 + j] = hi[j];
    }
    f32x4 C[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) C[p] = r.xo.dot(p, q6_pair_to_bf16(cd[2 * p], cd[2 * p + 1]), off[p]);
    const float d = f16_lo(r.dd[t]);
    const float nd = -128.0f * d;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float u = (float)((r.su[t] >> (8 * p)) & 0xFFu);
      const float cp = __builtin_fmaf(d, u, nd);  // d * s, exact
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(cp, C[p][i], acc[t][i]);
    }
  }
}

// Work split as in qgemm_w4_kernel: wave (wn_i, ks_i) owns row tiles
// [(blockIdx.x * wn + wn_i) * RT, + RT) and steps [ks_i * nsteps / ks,
// (ks_i + 1) * nsteps / ks) in ascending order, DEPTH register sets in
// rotation, every load unconditional (clamped to the wave's last step).
template <int XT, int RT, int DEPTH>
__global__ __launch_bounds__((XT == ISD_F32 ? 32 : 64) * (16 / RT)) void qgemm_q6_kernel(
    Q6Ptrs p, const void* __restrict__ xv, float* __restrict__ y, int N, int K, int n, int ks,
    int wn) {
  extern __shared__ __attribute__((aligned(16))) float red[];  // [wn][ks][RT][32][4] when ks > 1
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wk = wave % ks;
  const int wi = wave / ks;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int nsteps = K >> 7;
  const int ntiles = (N + 15) >> 4;
  const int s0 = (int)(((long)wk * nsteps) / ks);
  const int s1 = (int)(((long)(wk + 1) * nsteps) / ks);
  const int tile0 = (blockIdx.x * wn + wi) * RT;
  const int row0 = tile0 * 16;
  // activation rows 8 * blockIdx.y .. +7 fill the 8 slots; slots past n
  // repeat row n-1 (never stored)
  const int slot0 = blockIdx.y * 8;
  const int xr = min(slot0 + (c & 7), n - 1);

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (s0 < s1) {
    const int last = s1 - 1;
    Q6Step<XT, RT> buf[DEPTH];
#pragma unroll
    for (int i = 0; i + 1 < DEPTH; ++i)
      q6_load_step(buf[i], p, xv, K, xr, ntiles, nsteps, min(s0 + i, last), tile0, lane, c, g);
    bool done = false;
    for (int s = s0; !done; s += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        if (!done) {
          q6_load_step(buf[(i + DEPTH - 1) % DEPTH], p, xv, K, xr, ntiles, nsteps,
                       min(s + i + DEPTH - 1, last), tile0, lane, c, g);
          q6_compute_step(buf[i], acc);
          done = s + i >= last;
        }
      }
    }
  }

  // Lane (c, g < 2) holds the even sub-blocks' sums of slots 4g..4g+3 for
  // weight row c, lane (c, g + 2) the odd ones': even + odd.
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] += shfl_xor(acc[t][i], 32);
  const int act = n - slot0 > 4 ? 32 : 16;  // lanes holding slots that can be real
  if (ks > 1) {
    if (lane < act) {
#pragma unroll
      for (int t = 0; t < RT; ++t) *(f32x4*)&red[((wave * RT + t) * 32 + lane) * 4] = acc[t];
    }
    __syncthreads();
    if (wk != 0) return;
    // each lane reads its four values of every wave as one 16-byte vector
    // (consecutive lanes, consecutive 16-byte slots: no bank conflicts) and
    // adds them element by element in wave order
    if (lane < act) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        f32x4 v = *(const f32x4*)&red[((wave * RT + t) * 32 + lane) * 4];
        for (int w = 1; w < ks; ++w) {
          const f32x4 p = *(const f32x4*)&red[(((wave + w) * RT + t) * 32 + lane) * 4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = v[i] + p[i];
        }
        acc[t] = v;
      }
    }
  }
  if (lane < act) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int r = row0 + 16 * t + c;
      if (r < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = slot0 + 4 * g + i;
          if (cc < n) y[(size_t)cc * N + r] = acc[t][i];
        }
      }
    }
  }
}

template <int XT, int RT, int DEPTH>
inline hipError_t launch_qgemm_q6(const Q6Ptrs& p, const void* x, float* y, int N, int K, int n,
                                  int ks, int wn, hipStream_t st) {
  const int ntiles = (N + 15) / 16;
  dim3 grid((ntiles + RT * wn - 1) / (RT * wn), (n + 7) / 8);
  dim3 block(64 * ks * wn);
  size_t lds = ks > 1 ? (size_t)wn * ks * RT * 32 * 4 * sizeof(float) : 0;
  hipLaunchKernelGGL((qgemm_q6_kernel<XT, RT, DEPTH>), grid, block, lds, st, p, x, y, N, K, n, ks,
                     wn);
  return hipGetLastError();
}

// ---------------------------------------------------------------- packing
//
// Packed layout for N rows and K inputs (nsteps = K/128 steps of eight
// sub-blocks, nsup = K/256 super-blocks, ntiles = ceil(N/16) tiles):
//   codes  uint8 [ntiles][nsteps][1536]: lane l = i + 16g of tile T, step S
//          holds code words w[0..7], w[2p + h] = bytes e = 0..3 the codes of
//          inputs 128S + 16(2p + (g >> 1)) + 8(g & 1) + 4h + e of row 16T+i;
//          packed words P[j][k] (j = 0, 1; k = 0..2) have byte e =
//          w[4j+k] byte e | (bits 2k, 2k+1 of w[4j+3] byte e) << 6; bytes
//          16l..16l+15 hold P00 P01 P02 P10, bytes 1024+8l..+7 hold P11 P12;
//   subs   uint8 [ntiles][nsteps][16][2][4]: (T, S, i, h, p) = s of sub-block
//          8S + 2p + h of row 16T+i, plus 128;
//   sups   uint16 [ntiles][nsup][16]: d of super-block U of row 16T+i.
// Rows past N: codes 0, scale bytes 128 (s = 0), d = 0.
//
// grid = ntiles * nsteps; block = 64 code lanes, 16 sub-scale rows, 16 d
// rows (written by even steps only).
__global__ __launch_bounds__(128) void qgemm_q6_pack_kernel(
    const uint8_t* __restrict__ ql, const uint8_t* __restrict__ qh, const int8_t* __restrict__ sc,
    const uint16_t* __restrict__ d, uint8_t* __restrict__ codes_p, uint8_t* __restrict__ subs_p,
    uint16_t* __restrict__ sups_p, int N, int K) {
  const int nsteps = K >> 7;
  const int ts = blockIdx.x;
  const int T = ts / nsteps, S = ts % nsteps;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int i = tid & 15, g = tid >> 4;
    const int row = 16 * T + i;
    uint32_t w[8];
    for (int wi = 0; wi < 8; ++wi) {
      const int pr = wi >> 1, h = wi & 1;
      uint32_t v = 0u;
      for (int e = 0; e < 4; ++e) {
        uint32_t q = 0u;
        if (row < N) {
          const size_t k = (size_t)128 * S + 16 * (2 * pr + (g >> 1)) + 8 * (g & 1) + 4 * h + e;
          const uint32_t lo = (ql[(size_t)row * (K >> 1) + (k >> 1)] >> (4 * (k & 1))) & 0xFu;
          const uint32_t hi = (qh[(size_t)row * (K >> 2) + (k >> 2)] >> (2 * (k & 3))) & 0x3u;
          q = lo | (hi << 4);
        }
        v |= q << (8 * e);
      }
      w[wi] = v;
    }
    uint32_t P[6];
    for (int j = 0; j < 2; ++j)
      for (int k = 0; k < 3; ++k) {
        uint32_t v = 0u;
        for (int e = 0; e < 4; ++e) {
          const uint32_t b = ((w[4 * j + k] >> (8 * e)) & 0x3Fu) |
                             ((((w[4 * j + 3] >> (8 * e)) >> (2 * k)) & 3u) << 6);
          v |= b << (8 * e);
        }
        P[3 * j + k] = v;
      }
    uint8_t* rec = codes_p + (size_t)ts * 1536;
    *(u32x4*)(rec + tid * 16) = u32x4{P[0], P[1], P[2], P[3]};
    *(u32x2*)(rec + 1024 + tid * 8) = u32x2{P[4], P[5]};
  } else if (tid < 80) {
    const int i = tid - 64;
    const int row = 16 * T + i;
    uint32_t v[2] = {0u, 0u};
    for (int h = 0; h < 2; ++h)
      for (int pr = 0; pr < 4; ++pr) {
        const int s = row < N ? (int)sc[(size_t)row * (K >> 4) + 8 * S + 2 * pr + h] : 0;
        v[h] |= (uint32_t)(s + 128) << (8 * pr);
      }
    *(u32x2*)(subs_p + (size_t)ts * 128 + i * 8) = u32x2{v[0], v[1]};
  } else if (tid < 96 && (S & 1) == 0) {
    const int i = tid - 80;
    const int row = 16 * T + i;
    const int nsup = K >> 8;
    sups_p[((size_t)T * nsup + (S >> 1)) * 16 + i] =
        row < N ? d[(size_t)row * nsup + (S >> 1)] : (uint16_t)0;
  }
}

}  // namespace isd
