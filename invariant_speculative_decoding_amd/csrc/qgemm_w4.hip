// qgemm_w4 entry point: argument checks, the fixed work split, dispatch.
// The kernel (and the reasoning behind its width-invariant geometry) is in
// qgemm_w4_kernel.hpp.
#include <hip/hip_runtime.h>

#include "qgemm_w4_kernel.hpp"

namespace isd {

// Class geometry: row tiles per wave (rt), waves splitting K (ks) and waves
// side by side along N (wn), from (N, K, dtype) only -- never from the
// number of activation rows.  ks fixes every output's arithmetic; the 4-bit
// kernel deals out its tiles as w4_schedule says below, the 6-bit one as
// here.  Chosen from interleaved timing sweeps on MI355X at the four dense
// shapes (152064, 34816 and 5120 rows):
//   very tall (>= 64K rows): 4 tiles per wave, no K split, two waves per
//     work-group sharing the activations through L1;
//   tall (>= 16K rows): 2 tiles per wave, K split over 2 waves;
//   mid (>= 2K rows): 2 tiles per wave, K split over 8 waves (a single
//     round of work-groups over the chip);
//   small: 1 tile per wave, about 4096 waves in all.
void qgemm_geometry(int N, int K, int x_dtype, int* rt, int* ks, int* wn) {
  const int nsteps = (K / 32 + 3) / 4;
  const int lanes16 = x_dtype == ISD_F32 ? 8 : 16;  // rt * ks * wn bound (kernel launch bounds)
  int r, k, w = 1;
  if (N >= 65536) {
    r = 4;
    k = 1;
    w = 2;
  } else if (N >= 16384) {
    r = 2;
    k = 2;
  } else if (N >= 2048) {
    r = 2;
    k = 8;
  } else {
    r = 1;
    const int tiles = (N + 15) / 16;
    k = (4096 + tiles - 1) / tiles;
  }
  if (r * k * w > lanes16) k = lanes16 / (r * w);
  if (k > nsteps) k = nsteps;
  if (k < 1) k = 1;
  *rt = r;
  *ks = k;
  *wn = w;
}

// The 4-bit kernel's schedule for one launch.  The K split `ks` is the class
// geometry's and fixes every output's arithmetic; the rest only deals the
// row tiles out to waves and work-groups and never changes a bit:
//   rt, wn  row tiles per wave and waves side by side along N;
//   sg      activation slot groups (16 rows each) per work-group;
//   cnt     the counted loop form (qgemm_w4_kernel).
// With bf16 activations and one slot group per work-group (every decode
// width, and the argmax form, whose key count must not depend on n) the two
// tall classes deal out more tiles per wave than the class geometry: 5 in
// the very tall class (180 VGPRs, two waves per SIMD: 1901 waves for the
// 152064-row lm_head fit on the chip at once, and no SIMD holds more than
// 10 tiles where three waves of 4 could hold 12) and 3 in the tall class,
// counted.  Measured on MI355X with 1-1.5 GB of rotated weight copies,
// outputs bit-identical: lm_head 85.7 -> 79.4 us at width 1 and 91.5 ->
// 86.6 us at width 8; 34816 x 5120 24.9 -> 22.7 us and 29.0 -> 23.5 us.
// 6 tiles per wave (very tall) or 4 (tall) are slower again.  Blocks of
// more than 16 rows (prefill) keep the class tiles and take two slot groups
// per work-group, which the wider tiles cannot hold in registers.
struct W4Sched {
  int rt, ks, wn, sg;
  bool cnt;
};

static W4Sched w4_schedule(int N, int K, int x_dtype, int groups, bool argmax) {
  W4Sched s;
  qgemm_geometry(N, K, x_dtype, &s.rt, &s.ks, &s.wn);
  s.sg = 1;
  s.cnt = s.ks >= 4;  // the counted form where K is split over 4 or more waves
  if (x_dtype != ISD_BF16) return s;
  if (!argmax && groups >= 2 && (s.rt == 4 || (s.rt == 2 && s.ks <= 2))) {
    s.sg = 2;
  } else if (N >= 65536) {
    s.rt = 5;
  } else if (N >= 16384) {
    s.rt = 3;
    s.cnt = true;
  }
  return s;
}

}  // namespace isd

extern "C" size_t qgemm_w4_packed_bytes(int N, int K) {
  if (N < 1 || N > (1 << 30) || K < 32 || (K % 32) != 0) return 0;
  return (size_t)((N + 15) / 16) * (size_t)((K / 32 + 3) / 4) * 1024;
}

extern "C" int qgemm_w4_pack(const uint8_t* codes, const uint16_t* scale_min, uint8_t* codes_p,
                             uint16_t* scales_p, int N, int K, void* stream) {
  using namespace isd;
  if (!codes || !scale_min || !codes_p || !scales_p) return ISD_EINVAL;
  if (N < 1 || N > (1 << 30) || K < 32 || (K % 32) != 0) return ISD_EINVAL;
  if (!aligned(codes, 4) || !aligned(scale_min, 4) || !aligned(codes_p, 16) ||
      !aligned(scales_p, 16))
    return ISD_EINVAL;
  const int nsteps = (K / 32 + 3) / 4;
  const long ts = (long)((N + 15) / 16) * nsteps;
  if (ts > 0x7FFFFFFFL) return ISD_EINVAL;
  hipLaunchKernelGGL(qgemm_w4_pack_kernel, dim3((unsigned)ts), dim3(128), 0, (hipStream_t)stream,
                     codes, scale_min, codes_p, scales_p, N, K);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int qgemm_w4(const uint8_t* codes_p, const uint16_t* scales_p, const void* x,
                        int x_dtype, float* y, int N, int K, int n, void* stream) {
  using namespace isd;
  if (!codes_p || !scales_p || !x || !y) return ISD_EINVAL;
  if (N < 1 || N > (1 << 30) || K < 32 || (K % 32) != 0 || n < 1 || n > ISD_QGEMM_MAX_N)
    return ISD_EINVAL;
  if (x_dtype != ISD_F32 && x_dtype != ISD_BF16) return ISD_EINVAL;
  if (!aligned(codes_p, 16) || !aligned(scales_p, 16) || !aligned(x, 16) || !aligned(y, 4))
    return ISD_EINVAL;
  if ((size_t)N * (size_t)K / 2 > (size_t)1 << 40) return ISD_EINVAL;
  // Slot groups of 16 rows per work-group: a block of more than 16 rows
  // (prefill) reads each weight once per two groups in the tall and very
  // tall classes with bf16 activations (measured on MI355X at 512 rows:
  // lm_head 1.46x, 34816x5120 1.18x faster).  Not in the mid class, whose
  // eight-wave K split loses occupancy to the second group's registers, nor
  // with one tile per wave or fp32 activations (the registers would spill).
  // The choice moves rows between work-groups and never changes a row's
  // arithmetic.
  const W4Sched q = w4_schedule(N, K, x_dtype, (n + 15) / 16, false);
  const int ks = q.ks, wn = q.wn;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  const uint8_t* c = codes_p;
  const uint16_t* s = scales_p;
  if (x_dtype == ISD_BF16) {
    if (q.sg == 2)
      e = q.rt == 4 ? launch_qgemm<ISD_BF16, 4, 2, 2>(c, s, x, y, N, K, n, ks, wn, st)
                    : launch_qgemm<ISD_BF16, 2, 2, 2>(c, s, x, y, N, K, n, ks, wn, st);
    else if (q.rt == 5)
      e = launch_qgemm<ISD_BF16, 5, 2, 1>(c, s, x, y, N, K, n, ks, wn, st);
    else if (q.rt == 3)
      e = launch_qgemm<ISD_BF16, 3, 2, 1, false, true>(c, s, x, y, N, K, n, ks, wn, st);
    else if (q.rt == 2)
      e = q.cnt ? launch_qgemm<ISD_BF16, 2, 2, 1, false, true>(c, s, x, y, N, K, n, ks, wn, st)
                : launch_qgemm<ISD_BF16, 2, 2, 1>(c, s, x, y, N, K, n, ks, wn, st);
    else
      e = q.cnt ? launch_qgemm<ISD_BF16, 1, 2, 1, false, true>(c, s, x, y, N, K, n, ks, wn, st)
                : launch_qgemm<ISD_BF16, 1, 2, 1>(c, s, x, y, N, K, n, ks, wn, st);
  } else {
    const bool cnt = q.cnt;
    const int rt = q.rt;
    e = rt == 4 ? launch_qgemm<ISD_F32, 4, 2, 1>(c, s, x, y, N, K, n, ks, wn, st)
      : rt == 2 ? (cnt ? launch_qgemm<ISD_F32, 2, 2, 1, false, true>(c, s, x, y, N, K, n, ks, wn, st)
                       : launch_qgemm<ISD_F32, 2, 2, 1>(c, s, x, y, N, K, n, ks, wn, st))
      : cnt ? launch_qgemm<ISD_F32, 1, 2, 1, false, true>(c, s, x, y, N, K, n, ks, wn, st)
            : launch_qgemm<ISD_F32, 1, 2, 1>(c, s, x, y, N, K, n, ks, wn, st);
  }
  return e == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int qgemm_w4_argmax(const uint8_t* codes_p, const uint16_t* scales_p, const void* x,
                               int x_dtype, float* y, int N, int K, int n, uint64_t* keys,
                               int* nkeys, void* stream) {
  using namespace isd;
  if (!nkeys) return ISD_EINVAL;
  if (N < 1 || N > (1 << 30) || K < 32 || (K % 32) != 0) return ISD_EINVAL;
  if (x_dtype != ISD_F32 && x_dtype != ISD_BF16) return ISD_EINVAL;
  const W4Sched q = w4_schedule(N, K, x_dtype, 1, true);
  const int rt = q.rt, ks = q.ks, wn = q.wn;
  const int nk = ((N + 15) / 16 + rt * wn - 1) / (rt * wn) * wn;  // wave columns along N
  if (!keys) {
    *nkeys = nk;
    return ISD_OK;
  }
  if (*nkeys != nk) return ISD_EINVAL;
  if (!codes_p || !scales_p || !x) return ISD_EINVAL;
  if (n < 1 || n > ISD_QGEMM_MAX_N) return ISD_EINVAL;
  if (!aligned(codes_p, 16) || !aligned(scales_p, 16) || !aligned(x, 16) || !aligned(keys, 8) ||
      (y && !aligned(y, 4)))
    return ISD_EINVAL;
  if ((size_t)N * (size_t)K / 2 > (size_t)1 << 40) return ISD_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* c = codes_p;
  const uint16_t* s = scales_p;
  u64* kk = (u64*)keys;
  hipError_t e;
  const bool cnt = q.cnt;  // the loop form, as in qgemm_w4
  if (x_dtype == ISD_BF16) {
    e = rt == 5 ? launch_qgemm<ISD_BF16, 5, 2, 1, true>(c, s, x, y, N, K, n, ks, wn, st, kk)
      : rt == 3 ? launch_qgemm<ISD_BF16, 3, 2, 1, true, true>(c, s, x, y, N, K, n, ks, wn, st, kk)
      : rt == 2 ? (cnt ? launch_qgemm<ISD_BF16, 2, 2, 1, true, true>(c, s, x, y, N, K, n, ks, wn, st, kk)
                       : launch_qgemm<ISD_BF16, 2, 2, 1, true>(c, s, x, y, N, K, n, ks, wn, st, kk))
      : cnt ? launch_qgemm<ISD_BF16, 1, 2, 1, true, true>(c, s, x, y, N, K, n, ks, wn, st, kk)
            : launch_qgemm<ISD_BF16, 1, 2, 1, true>(c, s, x, y, N, K, n, ks, wn, st, kk);
  } else {
    e = rt == 4 ? launch_qgemm<ISD_F32, 4, 2, 1, true>(c, s, x, y, N, K, n, ks, wn, st, kk)
      : rt == 2 ? (cnt ? launch_qgemm<ISD_F32, 2, 2, 1, true, true>(c, s, x, y, N, K, n, ks, wn, st, kk)
                       : launch_qgemm<ISD_F32, 2, 2, 1, true>(c, s, x, y, N, K, n, ks, wn, st, kk))
      : cnt ? launch_qgemm<ISD_F32, 1, 2, 1, true, true>(c, s, x, y, N, K, n, ks, wn, st, kk)
            : launch_qgemm<ISD_F32, 1, 2, 1, true>(c, s, x, y, N, K, n, ks, wn, st, kk);
  }
  return e == hipSuccess ? ISD_OK : ISD_EHIP;
}
