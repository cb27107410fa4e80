// kv_commit: ragged paged-KV bookkeeping around a verify pass.
//
// proofoftech.org, "'Lossless' speculative decoding is a property of the
// math, not your deployment.", section "Batching breaks the
// implementation": after sequences accept different numbers of drafts their
// lengths, position ids, masks and KV state fall out of alignment, and a
// batched step reproduces each sequence decoded alone only if that
// realignment is exact.  Here every sequence carries its own committed
// length and position id; APPEND writes a block's rows at that sequence's
// own slots, COMMIT keeps the accepted prefix and rolls the rest back by
// truncation.  No operation reads or writes another sequence's state.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

// grid = (Hkv, 8, B), block = D.  Row j of sequence s goes to position
// seq_len[s] + j: keys [page][Hkv][16][D], values [page][Hkv][D][16].
__global__ __launch_bounds__(128) void kv_append_kernel(
    uint16_t* __restrict__ kp, uint16_t* __restrict__ vp, const int32_t* __restrict__ table,
    int max_pages, int num_pages, const uint16_t* __restrict__ kn,
    const uint16_t* __restrict__ vn, const int32_t* __restrict__ row_start,
    const int32_t* __restrict__ seq_len, int B, int Hkv, int D) {
  const int h = blockIdx.x;
  const int j = blockIdx.y;
  const int s = blockIdx.z;
  const int d = threadIdx.x;
  int r0;
  const int n = seq_range(row_start, s, B, ISD_MAX_ROWS, &r0);
  if (j >= n) return;
  const long pos = (long)seq_len[s] + j;
  if (pos < 0 || pos >= (long)max_pages * ISD_PAGE) return;
  const int page = table[(size_t)s * max_pages + pos / ISD_PAGE];
  if (page < 0 || page >= num_pages) return;
  const int off = (int)(pos % ISD_PAGE);
  const size_t src = ((size_t)(r0 + j) * Hkv + h) * D + d;
  const size_t base = ((size_t)page * Hkv + h) * ISD_PAGE * D;
  kp[base + (size_t)off * D + d] = kn[src];
  vp[base + (size_t)d * ISD_PAGE + off] = vn[src];
}

// grid = ceil(B / 256), block = 256.
__global__ __launch_bounds__(256) void kv_commit_kernel(int32_t* __restrict__ seq_len,
                                                        int32_t* __restrict__ pos_id,
                                                        const int32_t* __restrict__ acc, int B) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= B) return;
  const int c = seq_len[s] + acc[s] + 1;
  seq_len[s] = c;
  pos_id[s] = c;
}

}  // namespace isd

extern "C" int kv_commit(uint16_t* k_pages, uint16_t* v_pages, const int32_t* page_table,
                         int max_pages, int num_pages, const uint16_t* k_new,
                         const uint16_t* v_new, const int32_t* row_start, int32_t* seq_len,
                         int32_t* pos_id, const int32_t* accept_len, int B, int Hkv, int D,
                         void* stream) {
  using namespace isd;
  if (B < 1 || Hkv < 1 || (D != 64 && D != 128) || max_pages < 1 || num_pages < 1)
    return ISD_EINVAL;
  if (!seq_len || !pos_id) return ISD_EINVAL;
  if (!aligned(seq_len, 4) || !aligned(pos_id, 4) || !aligned(accept_len, 4)) return ISD_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (accept_len) {
    hipLaunchKernelGGL(kv_commit_kernel, dim3((B + 255) / 256), dim3(256), 0, st, seq_len,
                       pos_id, accept_len, B);
  } else {
    if (!k_pages || !v_pages || !page_table || !k_new || !v_new || !row_start) return ISD_EINVAL;
    if (!aligned(k_pages, 2) || !aligned(v_pages, 2) || !aligned(k_new, 2) ||
        !aligned(v_new, 2) || !aligned(page_table, 4) || !aligned(row_start, 4))
      return ISD_EINVAL;
    hipLaunchKernelGGL(kv_append_kernel, dim3(Hkv, ISD_MAX_ROWS, B), dim3(D), 0, st, k_pages,
                       v_pages, page_table, max_pages, num_pages, k_new, v_new, row_start,
                       seq_len, B, Hkv, D);
  }
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}

extern "C" const char* isd_version(void) { return "isd 0.1 gfx950"; }
