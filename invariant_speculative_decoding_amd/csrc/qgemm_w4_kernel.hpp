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
//    16 weight rows (N); activation rows fill the slots 16 at a time (slot
//    groups; a grid row serves one or two of them, which changes how often
//    a weight is read, not any row's arithmetic) and a group with fewer
//    real rows repeats its last one.  Each output element of an MFMA depends only on its own A
//    row and B column, so neither the other slots nor the slot a row lands
//    in can touch its bits: a row of a 512-row prefill block equals the
//    same row evaluated alone.
//  * One MFMA covers exactly one 32-value block (K = 32), so the per-block
//    scale is applied to the block's exact partial sum.  The codes enter as
//    bf16 values 128 + q (bit pattern 0x4300 | q, built with byte
//    permutes); the block result is d * sum((128+q) x) + (m - 128 d) *
//    sum(x).  The first term is four fp32 FMAs per lane and block; the
//    second is summed over the four blocks of a step by one fp32 16x16x4
//    MFMA (slots x blocks of sum(x) against blocks x rows of m - 128 d),
//    where lane (row r, group g) supplies sum(x) of slot r over block g --
//    produced by four "indicator" MFMAs whose A operand is 1 exactly on
//    output rows 4g..4g+3 -- and m - 128 d of its row for block g.  Both
//    terms of a slot depend on that slot's activations only.
//  * Within a step the blocks' d-terms are accumulated in ascending block
//    order, then the step's minimum term; steps are accumulated in
//    ascending order inside a wave; a wave owns a fixed, contiguous range
//    of steps; the `ks` waves of a work-group that split K are summed in
//    wave order through LDS.  ks is a function of (N, K, x dtype) only; how
//    many row tiles a wave takes (rt) and how many waves sit side by side
//    (wn) decide which wave computes a tile, never its arithmetic.  The `wn`
//    waves of a work-group that share a K range take neighbouring row
//    tiles, so their activation loads meet in the L1 cache.
//  * fp32 activations are split exactly into three bf16 parts (hi, mid, lo
//    by truncation) and the three MFMAs are chained.
//
// Weights stream from HBM in the packed layout (see qgemm_w4_pack): for
// every 16-row tile and every step of four blocks, one contiguous 1 KB run
// of codes already in MFMA lane order (lane i + 16g holds the k-group g
// slices of the four blocks of row i, nibbles arranged so that they decode
// in element order and meet the activations as loaded) and one 256-byte
// run of scales.  A
// wave's load of a tile-step is therefore a single fully coalesced 1 KB
// read; the row-major layout would scatter it over 16 DRAM rows.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

constexpr uint32_t kOnesPair = 0x3F803F80u;   // bf16 1.0 in both halves

// Codes of one lane's k-group as bf16 values 128+q (bit pattern 0x4300 | q)
// in element order e0..e7.  The packed word holds element u in the low
// nibble of byte u and element u+4 in the high nibble of byte u (see
// qgemm_w4_pack), so masking the low and high nibbles yields the bytes
// e0..e3 and e4..e7, and each output dword takes two code bytes and two
// 0x43 bytes with one v_perm_b32.
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t cw) {
  const uint32_t lo = cw & 0x0F0F0F0Fu;         // e0 e1 e2 e3
  const uint32_t hi = (cw >> 4) & 0x0F0F0F0Fu;  // e4 e5 e6 e7
  u32x4 r;
  r.x = perm(0x43434343u, lo, 0x04010400u);
  r.y = perm(0x43434343u, lo, 0x04030402u);
  r.z = perm(0x43434343u, hi, 0x04010400u);
  r.w = perm(0x43434343u, hi, 0x04030402u);
  return as_bf16x8(r);
}

template <int XT>
struct XOperand;

// bf16 activations: one A tile per block.
template <>
struct XOperand<ISD_BF16> {
  bf16x8 a[4];
  // Unconditional loads (so the compiler can count them across the
  // software pipeline): the caller clamps the activation row (padding
  // slots read the last real row and feed MFMA rows whose results are
  // never stored), and blocks past K read the last block, whose weights
  // are zero in the packed layout.
  __device__ __forceinline__ void load(const void* xv, int K, int xr, int nb, int b, int g) {
    const uint16_t* x = (const uint16_t*)xv;
    const size_t row = (size_t)xr * K;
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = as_bf16x8(ld16(x + row + 32 * min(b + j, nb - 1) + 8 * g));
  }
  __device__ __forceinline__ void prepare() {}
  __device__ __forceinline__ f32x4 dot(int j, bf16x8 w) const {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return mfma_bf16(a[j], w, z);
  }
  // sum(x) of slot (lane & 15) over block (lane >> 4) of the step, in every
  // element: block j's activations as the B operand against indicator j.
  __device__ __forceinline__ f32x4 sx_lanes(const bf16x8 (&ind)[4]) const {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) z = mfma_bf16(ind[j], a[j], z);
    return z;
  }
};

// fp32 activations: three exact bf16 parts per block, chained MFMAs.
template <>
struct XOperand<ISD_F32> {
  bf16x8 a[4][3];
  u32x4 raw[4][2];
  __device__ __forceinline__ void load(const void* xv, int K, int xr, int nb, int b, int g) {
    const float* x = (const float*)xv;
    const size_t row = (size_t)xr * K;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* p = x + row + 32 * min(b + j, nb - 1) + 8 * g;
      raw[j][0] = ld16(p);
      raw[j][1] = ld16(p + 4);
    }
  }
  __device__ __forceinline__ void prepare() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 lo = raw[j][0], hi = raw[j][1];
      const uint32_t v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split3(v[e], h[e], m[e], l[e]);
      u32x4 ph = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      u32x4 pm = {m[0] | (m[1] << 16), m[2] | (m[3] << 16), m[4] | (m[5] << 16), m[6] | (m[7] << 16)};
      u32x4 pl = {l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
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
  __device__ __forceinline__ f32x4 sx_lanes(const bf16x8 (&ind)[4]) const {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z = mfma_bf16(ind[j], a[j][0], z);
      z = mfma_bf16(ind[j], a[j][1], z);
      z = mfma_bf16(ind[j], a[j][2], z);
    }
    return z;
  }
};

// Registers of one 4-block step: the activation tiles of SG slot groups,
// the codes of every row tile (lane i + 16g: k-group g of blocks
// 4s..4s+3 of row i) and the tile's (d, m) pairs for the lane's row.
template <int XT, int RT, int SG>
struct Step {
  XOperand<XT> xo[SG];
  u32x4 cw[RT];
  u32x4 sc[RT];
};

// Every load of a step is unconditional (the compiler can then count the
// loads in flight): tiles past the last read the last tile (never stored);
// the packed layout zero-fills rows past N and blocks past K.
template <int XT, int RT, int SG>
__device__ __forceinline__ void load_step(Step<XT, RT, SG>& r, const uint8_t* __restrict__ codes,
                                          const uint16_t* __restrict__ sc, const void* xv, int K,
                                          const int (&xr)[SG], int nb, int ntiles, int nsteps,
                                          int s, int tile0, int lane, int c, int g) {
#pragma unroll
  for (int q = 0; q < SG; ++q) r.xo[q].load(xv, K, xr[q], nb, 4 * s, g);
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const size_t ts = (size_t)min(tile0 + t, ntiles - 1) * nsteps + s;
    r.cw[t] = ld16_stream(codes + (ts * 64 + lane) * 16);
    r.sc[t] = ld16(sc + (ts * 16 + c) * 8);
  }
}

// Accumulates the four blocks of a step for every slot group: the d-terms
// in block order, then the step's minimum term through the fp32 MFMA.  The
// codes of a tile are unpacked once and serve every slot group; each
// group's arithmetic is the same as with one group per work-group.  Blocks
// past K have d = m = 0 in the packed layout (and finite activations: the
// last real block's), so they add exact zeros.
template <int XT, int RT, int SG>
__device__ __forceinline__ void compute_step(Step<XT, RT, SG>& r, f32x4 (&acc)[SG][RT],
                                             const bf16x8 (&ind)[4], int g) {
  float sxa[SG];
#pragma unroll
  for (int q = 0; q < SG; ++q) {
    r.xo[q].prepare();
    sxa[q] = r.xo[q].sx_lanes(ind)[0];
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const uint32_t cws[4] = {r.cw[t].x, r.cw[t].y, r.cw[t].z, r.cw[t].w};
    const uint32_t scs[4] = {r.sc[t].x, r.sc[t].y, r.sc[t].z, r.sc[t].w};
    bf16x8 wq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wq[j] = codes_to_bf16(cws[j]);
    // (d, m) of this lane's row for block g
    const uint32_t sg = g == 0 ? scs[0] : g == 1 ? scs[1] : g == 2 ? scs[2] : scs[3];
    const float mp = __builtin_fmaf(-128.0f, f16_lo(sg), f16_hi(sg));
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      f32x4 S[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) S[j] = r.xo[q].dot(j, wq[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d = f16_lo(scs[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[q][t][i] = __builtin_fmaf(d, S[j][i], acc[q][t][i]);
      }
      acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sxa[q], mp, acc[q][t], 0, 0, 0);
    }
  }
}

// One work-group: wn x ks waves of 64 lanes.  Wave (wn_i, ks_i) owns row
// tiles [(blockIdx.x * wn + wn_i) * RT, + RT) and accumulates 4-block steps
// [ks_i * nsteps / ks, (ks_i + 1) * nsteps / ks) in ascending order with
// DEPTH register sets in rotation: while step s computes, steps s+1 ..
// s+DEPTH-1 are in flight.  Loads past a wave's last step are clamped to it
// (a cached reload), so every load is unconditional and the compiler can
// wait for exactly the oldest set.  A work-group serves SG consecutive slot
// groups of 16 activation rows (grid row blockIdx.y), so a block of many
// rows reads each weight once per SG groups; SG changes which work-group
// computes a row, never its arithmetic.
//
// CNT selects the loop form (counted rounds and a load-free tail, or a
// loop that checks for the last step inside each round); it changes when
// loads are waited for, never a result bit.  Measured on MI355X (rotated
// weight copies): the counted form is 0.6 us faster for the 8-wave K-split
// class (5120 x 5120 7.9 -> 7.4 us, 5120 x 17408 17.1 -> 16.4 us) and for
// the 34816-row shape at 3 tiles per wave, 1-5 % slower for the lm_head,
// which keeps the other form.
//
// With AM (argmax epilogue, one slot group per work-group) the kernel also
// writes, for every activation row cc and wave column v = blockIdx.x * wn +
// wn_i, the largest argmax key (common.hpp) of y[cc][r] over the column's
// rows r into keys[cc * gridDim.x * wn + v]: the keys of a row hold its
// greedy token, so a verify can skip the separate pass over the logits, and
// y may be null (logits not written).  The keys come from the registers y
// is stored from.
template <int XT, int RT, int DEPTH, int SG, bool AM, bool CNT>
__global__ __launch_bounds__((XT == ISD_F32 ? 32 : 64) * (16 / RT)) void qgemm_w4_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ sc,
    const void* __restrict__ xv, float* __restrict__ y, int N, int K, int n, int ks, int wn,
    u64* __restrict__ keys) {
  // [wn][ks][SG][RT][64][4] when ks > 1
  extern __shared__ __attribute__((aligned(16))) float red[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wk = wave % ks;   // position along K
  const int wi = wave / ks;   // position along N
  const int c = lane & 15;  // A: activation slot; B: weight row in the tile
  const int g = lane >> 4;  // k-group of 8 within a block
  const int nb = K >> 5;
  const int nsteps = (nb + 3) >> 2;
  const int ntiles = (N + 15) >> 4;
  const int s0 = (int)(((long)wk * nsteps) / ks);
  const int s1 = (int)(((long)(wk + 1) * nsteps) / ks);
  const int tile0 = (blockIdx.x * wn + wi) * RT;
  const int row0 = tile0 * 16;
  // slot group q holds activation rows slot0 + 16q .. +15 in the tile's 16
  // slots; slots past n repeat row n-1 (never stored)
  const int slot0 = blockIdx.y * 16 * SG;
  int xr[SG];
#pragma unroll
  for (int q = 0; q < SG; ++q) xr[q] = min(slot0 + 16 * q + c, n - 1);

  // indicator operands: 1 on output rows 4j..4j+3 (A rows (lane & 15))
  bf16x8 ind[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = (c >> 2) == j ? kOnesPair : 0u;
    ind[j] = as_bf16x8(u32x4{v, v, v, v});
  }

  f32x4 acc[SG][RT];
#pragma unroll
  for (int q = 0; q < SG; ++q)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (s0 < s1) {
    const int last = s1 - 1;
    Step<XT, RT, SG> buf[DEPTH];
#pragma unroll
    for (int i = 0; i + 1 < DEPTH; ++i)
      load_step(buf[i], codes, sc, xv, K, xr, nb, ntiles, nsteps, min(s0 + i, last), tile0, lane, c,
                g);
    if constexpr (CNT) {
      // Counted form: whole rounds of DEPTH steps with every load
      // unconditional, then the last (steps mod DEPTH) steps, whose loads
      // are already in flight, with no loads at all.  The loop body is
      // straight-line, so the compiler waits only for the oldest register
      // set at the loop head, not for every load in flight.
      const int nst = s1 - s0;
      const int nfull = nst / DEPTH;
      int s = s0;
      for (int it = 0; it < nfull; ++it, s += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
          load_step(buf[(i + DEPTH - 1) % DEPTH], codes, sc, xv, K, xr, nb, ntiles, nsteps,
                    min(s + i + DEPTH - 1, last), tile0, lane, c, g);
          compute_step(buf[i], acc, ind, g);
        }
      }
      const int rem = nst - nfull * DEPTH;
#pragma unroll
      for (int i = 0; i + 1 < DEPTH; ++i)
        if (i < rem) compute_step(buf[i], acc, ind, g);
    } else {
      bool done = false;
      for (int s = s0; !done; s += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
          if (!done) {
            load_step(buf[(i + DEPTH - 1) % DEPTH], codes, sc, xv, K, xr, nb, ntiles, nsteps,
                      min(s + i + DEPTH - 1, last), tile0, lane, c, g);
            compute_step(buf[i], acc, ind, g);
            done = s + i >= last;
          }
        }
      }
    }
  }

  // Lane (c, g) holds slots 4g+i of each group; only lanes below a group's
  // `act` can hold real ones (4g + i < n - its first slot).  With a K split
  // only the first wave of each column holds final sums after the reduction.
  if (ks > 1) {
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      const int act = n - (slot0 + 16 * q) > 8 ? 64 : 32;
      if (lane < act) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
          *(f32x4*)&red[(((wave * SG + q) * RT + t) * 64 + lane) * 4] = acc[q][t];
      }
    }
    __syncthreads();
    if (wk != 0) return;
    // each lane reads its four values of every wave as one 16-byte vector
    // (consecutive lanes, consecutive 16-byte slots: no bank conflicts) and
    // adds them element by element in wave order
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      const int act = n - (slot0 + 16 * q) > 8 ? 64 : 32;
      if (lane < act) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          f32x4 v = *(const f32x4*)&red[(((wave * SG + q) * RT + t) * 64 + lane) * 4];
          for (int w = 1; w < ks; ++w) {
            const f32x4 p = *(const f32x4*)&red[((((wave + w) * SG + q) * RT + t) * 64 + lane) * 4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = v[i] + p[i];
          }
          acc[q][t] = v;
        }
      }
    }
  }
  if (!AM || y) {
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      const int sq = slot0 + 16 * q;
      const int act = n - sq > 8 ? 64 : 32;
      if (lane < act) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int r = row0 + 16 * t + c;
          if (r < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int cc = sq + 4 * g + i;
              if (cc < n) y[(size_t)cc * N + r] = acc[q][t][i];
            }
          }
        }
      }
    }
  }
  if constexpr (AM) {
    static_assert(SG == 1, "the argmax epilogue serves one slot group");
    // the lane's best key for each of its slots over its rows (rows past N
    // give key 0), then over the 16 lanes of each slot, which form one DPP
    // row; one key per wave and activation row
    u64 kb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb[i] = 0ull;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int r = row0 + 16 * t + c;
        const u64 kv = argmax_key(acc[0][t][i], (uint32_t)r);
        kb[i] = max_u64(kb[i], r < N ? kv : 0ull);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) kb[i] = row16_max_u64(kb[i]);
    if (c == 0) {
      const size_t nw = (size_t)gridDim.x * wn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = slot0 + 4 * g + i;
        if (cc < n) keys[(size_t)cc * nw + blockIdx.x * wn + wi] = kb[i];
      }
    }
  }
}

template <int XT, int RT, int DEPTH, int SG, bool AM = false, bool CNT = false>
inline hipError_t launch_qgemm(const uint8_t* codes, const uint16_t* sc, const void* x, float* y,
                               int N, int K, int n, int ks, int wn, hipStream_t st,
                               u64* keys = nullptr) {
  const int ntiles = (N + 15) / 16;
  const int groups = (n + 15) / 16;
  dim3 grid((ntiles + RT * wn - 1) / (RT * wn), (groups + SG - 1) / SG);
  dim3 block(64 * ks * wn);
  size_t lds = ks > 1 ? (size_t)wn * ks * SG * RT * 64 * 4 * sizeof(float) : 0;
  hipLaunchKernelGGL((qgemm_w4_kernel<XT, RT, DEPTH, SG, AM, CNT>), grid, block, lds, st, codes, sc, x,
                     y, N, K, n, ks, wn, keys);
  return hipGetLastError();
}

// ---------------------------------------------------------------- packing
//
// Packed layout for N rows and K inputs (nb = K/32 blocks, nsteps =
// ceil(nb/4) steps of four blocks, ntiles = ceil(N/16) tiles of 16 rows):
//   codes  uint8 [ntiles][nsteps][64][16]: entry (T, S, i + 16g) holds, for
//          j = 0..3, 4 bytes with the codes of elements 8g..8g+7 of block
//          4S+j of row 16T+i -- byte u: element 8g+u in the low nibble,
//          element 8g+u+4 in the high nibble;
//   scales uint16 [ntiles][nsteps][16][4][2]: (d, m) of block 4S+j of row
//          16T+i.
// Rows past N and blocks past K are zero.

// grid = ntiles * nsteps, block = 64 + 16 (codes lanes, then scale rows).
__global__ __launch_bounds__(128) void qgemm_w4_pack_kernel(const uint8_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ sm,
                                                            uint8_t* __restrict__ codes_p,
                                                            uint16_t* __restrict__ sc_p, int N,
                                                            int K) {
  const int nb = K >> 5;
  const int nsteps = (nb + 3) >> 2;
  const int ts = blockIdx.x;
  const int T = ts / nsteps, S = ts % nsteps;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int i = tid & 15, g = tid >> 4;
    const int row = 16 * T + i;
    uint32_t w[4];
    for (int j = 0; j < 4; ++j) {
      const int blk = 4 * S + j;
      // row-major: byte t holds element 2t (low nibble) and 2t+1 (high)
      const uint32_t r = (row < N && blk < nb)
                             ? ld4(codes + (size_t)row * (K >> 1) + 16 * blk + 4 * g)
                             : 0u;
      uint32_t o = 0u;
      for (int u = 0; u < 8; ++u) {
        const uint32_t q = (r >> (4 * u)) & 0xFu;  // element u of the k-group
        o |= q << (u < 4 ? 8 * u : 8 * (u - 4) + 4);
      }
      w[j] = o;
    }
    u32x4 v = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(codes_p + ((size_t)ts * 64 + tid) * 16) = v;
  } else if (tid < 80) {
    const int i = tid - 64;
    const int row = 16 * T + i;
    uint32_t w[4];
    for (int j = 0; j < 4; ++j) {
      const int blk = 4 * S + j;
      w[j] = (row < N && blk < nb) ? ld4(sm + ((size_t)row * nb + blk) * 2) : 0u;
    }
    u32x4 v = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(sc_p + ((size_t)ts * 16 + i) * 8) = v;
  }
}

}  // namespace isd
