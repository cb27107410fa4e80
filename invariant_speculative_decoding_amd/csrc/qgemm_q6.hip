// qgemm_q6 entry points: argument checks, packed-section offsets, dispatch.
// The kernel and its width-invariant geometry are in qgemm_q6_kernel.hpp.
#include <hip/hip_runtime.h>

#include "qgemm_q6_kernel.hpp"

namespace isd {

struct Q6Sections {
  size_t codes, subs, sups, total;
};

// Offsets of the three sections of a packed 6-bit matrix: per (tile, step)
// 1536 code bytes and 128 sub-scale bytes, per (tile, super-block) 32 d bytes.
static bool q6_sections(int N, int K, Q6Sections* s) {
  if (N < 1 || N > (1 << 30) || K < 256 || (K % 256) != 0) return false;
  const size_t ntiles = (size_t)(N + 15) / 16;
  const size_t nsteps = (size_t)K / 128, nsup = (size_t)K / 256;
  s->codes = 0;
  s->subs = ntiles * nsteps * 1536;
  s->sups = s->subs + ntiles * nsteps * 128;
  s->total = s->sups + ntiles * nsup * 32;
  return true;
}

// Work split for the 6-bit kernel, from (N, K, dtype) only.  The 4-bit
// shape classes, except that very tall matrices with bf16 activations take
// 5 row tiles per wave (176 VGPRs, two waves per SIMD; 1901 waves for the
// 152064-row lm_head fit on the chip at once) with 2 waves along N and no
// K split.  Measured on MI355X (two rotated copies, widths 1 / 8): 108.2 /
// 117.0 us against 108.5 / 126.7 us for 4 tiles with K split over two
// waves, and 109-123 / 125-156 us for 3-6 tiles with or without the split;
// the other classes' best configurations matched the 4-bit ones at 34816,
// 5120 and 5120 x 17408.
static void q6_geometry(int N, int K, int x_dtype, int* rt, int* ks, int* wn) {
  qgemm_geometry(N, K, x_dtype, rt, ks, wn);
  if (N >= 65536 && x_dtype == ISD_BF16) {
    *rt = 5;
    *ks = 1;
    *wn = 2;
  }
}

}  // namespace isd

extern "C" size_t qgemm_q6_packed_bytes(int N, int K) {
  isd::Q6Sections s;
  return isd::q6_sections(N, K, &s) ? s.total : 0;
}

extern "C" int qgemm_q6_pack(const uint8_t* ql, const uint8_t* qh, const int8_t* sc,
                             const uint16_t* d, uint8_t* packed, int N, int K, void* stream) {
  using namespace isd;
  Q6Sections s;
  if (!ql || !qh || !sc || !d || !packed) return ISD_EINVAL;
  if (!q6_sections(N, K, &s)) return ISD_EINVAL;
  if (!aligned(d, 2) || !aligned(packed, 16)) return ISD_EINVAL;
  const long ts = (long)((N + 15) / 16) * (K / 128);
  if (ts > 0x7FFFFFFFL) return ISD_EINVAL;
  hipLaunchKernelGGL(qgemm_q6_pack_kernel, dim3((unsigned)ts), dim3(128), 0, (hipStream_t)stream,
                     ql, qh, sc, d, packed, packed + s.subs, (uint16_t*)(packed + s.sups), N, K);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" int qgemm_q6(const uint8_t* packed, const void* x, int x_dtype, float* y, int N, int K,
                        int n, void* stream) {
  using namespace isd;
  Q6Sections s;
  if (!packed || !x || !y) return ISD_EINVAL;
  if (!q6_sections(N, K, &s) || n < 1 || n > ISD_QGEMM_MAX_N) return ISD_EINVAL;
  if (x_dtype != ISD_F32 && x_dtype != ISD_BF16) return ISD_EINVAL;
  if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 4)) return ISD_EINVAL;
  if ((size_t)N * (size_t)K > (size_t)1 << 41) return ISD_EINVAL;
  const Q6Ptrs p = {packed + s.codes, packed + s.subs, (const uint16_t*)(packed + s.sups)};
  int rt, ks, wn;
  q6_geometry(N, K, x_dtype, &rt, &ks, &wn);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (x_dtype == ISD_BF16) {
    e = rt == 5 ? launch_qgemm_q6<ISD_BF16, 5, 2>(p, x, y, N, K, n, ks, wn, st)
      : rt == 4 ? launch_qgemm_q6<ISD_BF16, 4, 2>(p, x, y, N, K, n, ks, wn, st)
      : rt == 2 ? launch_qgemm_q6<ISD_BF16, 2, 2>(p, x, y, N, K, n, ks, wn, st)
                : launch_qgemm_q6<ISD_BF16, 1, 2>(p, x, y, N, K, n, ks, wn, st);
  } else {
    e = rt == 4 ? launch_qgemm_q6<ISD_F32, 4, 2>(p, x, y, N, K, n, ks, wn, st)
      : rt == 2 ? launch_qgemm_q6<ISD_F32, 2, 2>(p, x, y, N, K, n, ks, wn, st)
                : launch_qgemm_q6<ISD_F32, 1, 2>(p, x, y, N, K, n, ks, wn, st);
  }
  return e == hipSuccess ? ISD_OK : ISD_EHIP;
}
