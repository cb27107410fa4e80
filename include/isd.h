/*
 * isd.h -- batch-invariant speculative-verify kernels for AMD MI355X (gfx950).
 *
 * Four calls make up one verify pass of a target model over a block of
 * n = k + 1 query rows (the last committed token plus k drafted tokens):
 *
 *   kv_commit (APPEND)  write the block's keys/values into the paged cache
 *   decode_attn         causal attention of every row over its visible prefix
 *   qgemm_w4            4-bit block-quantised projections / lm_head
 *                       (weights packed once by qgemm_w4_pack; qgemm_q6 is
 *                       the same product for 6-bit super-block weights)
 *   spec_verify         argmax or rejection-sampling accept of the drafts
 *   kv_commit (COMMIT)  keep the accepted prefix, roll back the rest
 *
 * The contract of every call: each output row is a function of that row's
 * own inputs only.  How many rows are evaluated together (widths 1..8) and
 * what neighbouring rows hold never change a single bit of it.  This is the
 * property that makes a width-k verify pass reproduce serial width-one
 * decoding: checking several drafted tokens in one pass has to give exactly
 * the result the model would give decoding them one by one (ramgpt.org,
 * "When Lossless Speculation Stops Being Lossless on Blackwell",
 * introduction and section "The Hidden Contract Behind Lossless
 * Speculation").  The order in which
 * any one row's results are accumulated is a function of the matrix and
 * head shapes only; the number of rows and the sequence lengths decide only
 * how many work-groups run and which of them have work, never how a row is
 * computed.  There are no floating-point atomics.
 *
 * Conventions for all calls
 *   - Every array argument is a device pointer owned by the caller.  The
 *     library allocates nothing, keeps no mutable global state, never
 *     synchronises, and enqueues its kernels on `stream` (a hipStream_t;
 *     NULL is the default stream).  Calls are re-entrant and thread-safe.
 *     The one exception is spec_verify_noalloc, whose workspace is a fixed
 *     device array inside the library (see there).
 *   - Half-precision values travel as raw uint16_t bits (fp16 or bf16 as
 *     stated per argument).
 *   - Arrays of 32-bit values (int32, float) are 4-byte aligned and arrays
 *     of 16-bit values 2-byte aligned, unless a stricter alignment is
 *     stated per argument; a misaligned pointer is ISD_EINVAL.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is launched and nothing is written.
 *   - Device-side index data (page ids, positions, row offsets, draft ids)
 *     is range-checked inside the kernels: out-of-range entries are treated
 *     as described per call and never cause an out-of-bounds access.
 */
#ifndef ISD_H
#define ISD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ISD_OK 0
#define ISD_EINVAL (-1) /* bad size / null or misaligned pointer / bad dtype   */
#define ISD_ENOSPC (-2) /* workspace too small; *ws_bytes holds the need      */
#define ISD_EHIP (-3)   /* a HIP launch reported an error                     */

enum isd_dtype { ISD_F32 = 0, ISD_BF16 = 1 };

#define ISD_MAX_ROWS 8      /* query rows per sequence (k <= 7 drafts ... n <= 8) */
#define ISD_MAX_OUT 9       /* emitted tokens per sequence: up to 8 drafts + 1    */
#define ISD_PAGE 16         /* positions per KV page                             */
#define ISD_CHUNK 256       /* fixed attention split, in absolute positions      */
#define ISD_QGEMM_MAX_N 512 /* activation rows per qgemm_w4 call (prefill blocks) */
#define ISD_VERIFY_SCRATCH_BYTES (1 << 20) /* spec_verify_noalloc's device scratch  */
#define ISD_MAX_VERIFY_ROWS (1 << 24) /* bound on max_rows of the spec_verify calls */

/*
 * qgemm_w4 -- y[c][r] = sum_k W[r][k] * x[c][k] for c < n, r < N.
 *
 * W is 4-bit block quantised: the K inputs of a row form K/32 blocks; block
 * b of row r has fp16 scale d and fp16 minimum m and w = d*q + m for codes
 * q in 0..15.  This is the quantised matrix product whose batched result
 * must equal repeated single-column products (ramgpt.org, "When Lossless
 * Speculation Stops Being Lossless on Blackwell", section "Quantized Matrix
 * Multiplication Shows the Same Class of Failure"; tokenstrom.com,
 * "'Lossless,' but not quite", section "Why the math checks out and the
 * text still flips": the Q4_K/Q6_K mat-vec adds partial sums in a different
 * order for one token and for eight).
 *
 * The weights are passed in the packed layout produced by qgemm_w4_pack.
 *
 *   codes_p    packed codes, qgemm_w4_packed_bytes(N, K) bytes, 16-byte
 *              aligned.
 *   scales_p   packed scales, qgemm_w4_packed_bytes(N, K) / 4 bytes,
 *              16-byte aligned.
 *   x          [n][K] row-major activations, fp32 (x_dtype = ISD_F32) or
 *              bf16 bits (ISD_BF16).  16-byte aligned.
 *   y          float [n][N] row-major output.  4-byte aligned.
 *   1 <= N <= 2^30, K >= 32 with K % 32 == 0, N * K / 2 <= 2^40,
 *   1 <= n <= ISD_QGEMM_MAX_N (512).
 *
 * Every (r, c) result is accumulated in fp32 in an order fixed by (N, K,
 * x_dtype) alone: any width n -- a verify block of up to 8 rows or a
 * prefill block of up to 512 -- gives bit-identical rows, whatever the
 * rows of x beyond n hold.
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int qgemm_w4(const uint8_t* codes_p, const uint16_t* scales_p, const void* x,
             int x_dtype, float* y, int N, int K, int n, void* stream);

/*
 * qgemm_w4_argmax -- qgemm_w4 that also hands over each row's greedy token
 * in pieces: the lm_head of a greedy verify, whose target token is the
 * lowest id among the maxima of the row's logits (ramgpt.org, "When
 * Lossless Speculation Stops Being Lossless on Blackwell", section "The
 * Hidden Contract Behind Lossless Speculation").  The product runs on the
 * kernel of qgemm_w4 with the same per-row order, so y is bit-identical to
 * qgemm_w4's; before it is stored, every wave column of the launch (a
 * wave and the row tiles it owns) reduces its share of each row to one
 * 64-bit key (the order-preserving bits of the
 * value above the complemented index: the largest key is the largest value
 * at the lowest index, NaN never wins, -0 counts as +0).  spec_verify_keys
 * turns the keys into accept lengths and tokens without a pass over the
 * logits.
 *
 *   codes_p, scales_p, x, x_dtype, N, K, n  as for qgemm_w4.
 *   y          float [n][N], or NULL when the logits are not needed (only
 *              the keys are written).  4-byte aligned.
 *   keys       uint64 [n][*nkeys] row-major, 8-byte aligned; NULL to query.
 *   nkeys      in: the row stride of keys, which must equal the value the
 *              query returned for (N, K, x_dtype); out (query): that value
 *              (the number of wave columns along N).
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int qgemm_w4_argmax(const uint8_t* codes_p, const uint16_t* scales_p, const void* x,
                    int x_dtype, float* y, int N, int K, int n, uint64_t* keys,
                    int* nkeys, void* stream);

/*
 * qgemm_w4_pack -- one-time conversion of row-major 4-bit weights into the
 * packed layout qgemm_w4 streams (each wave-wide load is one contiguous
 * 1 KB run in MFMA lane order instead of 16 scattered row fragments).
 *
 * Input (row-major):
 *   codes      uint8 [N][K/2]; element 2t of a row in the low nibble of
 *              byte t, element 2t+1 in the high nibble.  4-byte aligned.
 *   scale_min  uint16 [N][K/32][2] fp16 bits (d, m) per block.  4-byte
 *              aligned.
 * Output (packed; nb = K/32, nsteps = ceil(nb/4), ntiles = ceil(N/16)):
 *   codes_p    uint8 [ntiles][nsteps][64][16]: entry (T, S, i + 16g) holds,
 *              for j = 0..3, four bytes with the codes of elements
 *              8g..8g+7 of block 4S+j of row 16T+i: byte u carries element
 *              8g+u in its low nibble and element 8g+u+4 in its high nibble.
 *   scales_p   uint16 [ntiles][nsteps][16][4][2]: (d, m) of block 4S+j of
 *              row 16T+i.
 *   Rows past N and blocks past K are written as zero.  Both outputs are
 *   16-byte aligned and sized by qgemm_w4_packed_bytes (codes) and a
 *   quarter of that (scales).
 *   1 <= N <= 2^30, K >= 32 with K % 32 == 0, ntiles * nsteps < 2^31.
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int qgemm_w4_pack(const uint8_t* codes, const uint16_t* scale_min,
                  uint8_t* codes_p, uint16_t* scales_p, int N, int K,
                  void* stream);

/* Bytes of the packed codes for an N x K matrix (0 for sizes qgemm_w4_pack
 * rejects by N or K alone). */
size_t qgemm_w4_packed_bytes(int N, int K);

/*
 * qgemm_q6 -- the same product, y[c][r] = sum_k W[r][k] * x[c][k], for
 * weights in the 6-bit super-block format: every row is split into
 * super-blocks of 256 inputs with an fp16 scale d, each super-block into 16
 * sub-blocks of 16 inputs with a signed 8-bit scale s, and
 * w = d * s * (q - 32) for a code q in 0..63.  The pages name this K-quant
 * format beside the 4-bit one among those whose mat-vec changes its
 * summation order with the number of tokens (tokenstrom.com, "'Lossless,'
 * but not quite", section "Why the math checks out and the text still
 * flips"); the layout is this library's reading of that name.
 *
 *   packed     the buffer written by qgemm_q6_pack, qgemm_q6_packed_bytes
 *              (N, K) bytes, 16-byte aligned.
 *   x          [n][K] row-major activations, fp32 (ISD_F32) or bf16 bits
 *              (ISD_BF16), 16-byte aligned.
 *   y          float [n][N] row-major output, 4-byte aligned.
 *   1 <= N <= 2^30, K >= 256 with K % 256 == 0, N * K <= 2^41,
 *   1 <= n <= ISD_QGEMM_MAX_N.
 *
 * Same contract as qgemm_w4: each (r, c) result is accumulated in fp32 in
 * an order fixed by (N, K, x_dtype) alone -- sub-blocks in ascending order,
 * each scaled by d * s after its own exact-product MFMA -- so every width n
 * gives bit-identical rows, whatever the rows of x beyond n hold.
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int qgemm_q6(const uint8_t* packed, const void* x, int x_dtype, float* y,
             int N, int K, int n, void* stream);

/*
 * qgemm_q6_pack -- one-time conversion of row-major 6-bit weights into the
 * packed layout qgemm_q6 streams (per 16-row tile and 128-input step one
 * contiguous 1536-byte run of codes in MFMA lane order, then the sub-block
 * scales and super-block scales as separate sections).
 *
 * Input (row-major, device memory, no alignment needed beyond d's 2 bytes):
 *   ql   uint8 [N][K/2]: low four bits of each code, element 2t in the low
 *        nibble of byte t, element 2t+1 in the high nibble.
 *   qh   uint8 [N][K/4]: high two bits, element 4t+i in bits 2i, 2i+1 of
 *        byte t.
 *   sc   int8 [N][K/16]: sub-block scales.
 *   d    uint16 [N][K/256]: fp16 bits of the super-block scales.
 * Output: packed, qgemm_q6_packed_bytes(N, K) bytes, 16-byte aligned;
 * every byte is written (rows past N are zero weights).
 * 1 <= N <= 2^30, K >= 256 with K % 256 == 0, ceil(N/16) * K/128 < 2^31.
 * qgemm_q6_packed_bytes returns 0 for an invalid N or K.
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int qgemm_q6_pack(const uint8_t* ql, const uint8_t* qh, const int8_t* sc,
                  const uint16_t* d, uint8_t* packed, int N, int K, void* stream);
size_t qgemm_q6_packed_bytes(int N, int K);

/*
 * decode_attn -- causal decode attention over a paged fp16 cache for a
 * ragged batch of verify blocks.
 *
 * Sequence s (s < B) owns query rows row_start[s] .. row_start[s+1]-1
 * (n_s = row_start[s+1] - row_start[s], 1 <= n_s <= 8).  Its row i sits at
 * position q_pos[s] + i and attends to cache positions 0 .. q_pos[s] + i
 * (the block's own keys/values must already be in the cache).  Query head
 * h reads key/value head h / (Hq / Hkv).  Position p of sequence s is in
 * page page_table[s * max_pages + p / 16] at offset p % 16.
 *
 *   score_j = scale * <Q[row][h], K_j[g]>;  out[row][h] = softmax(score) V
 *
 * Positions are split into fixed chunks [256c, 256c + 256) counted from
 * position 0; each chunk's partial (max, sum of exponentials, weighted
 * value sum) is folded into the running result in ascending chunk order
 * with the log-sum-exp rule.  The split never depends on the number of
 * rows or on the lengths, so row i of a width-n block is bit-identical to
 * a width-one call at q_pos + i (ramgpt.org, same page, section "Flash
 * Attention Changes Geometry With Batch Width": tile geometry chosen by
 * query width changes KV traversal and the reduction/combine order).
 * Positions beyond a row's prefix contribute nothing to any max or sum and
 * positions beyond a block's last row never enter any product (they may
 * be fetched and discarded).
 *
 *   q          fp16 [R][Hq][D], R = row_start[B].          16-byte aligned.
 *   k_pages    fp16 [num_pages][Hkv][16][D].                16-byte aligned.
 *   v_pages    fp16 [num_pages][Hkv][D][16].                16-byte aligned.
 *   page_table int32 [B][max_pages]; an id outside [0, num_pages) makes
 *              that page read as absent (zeros, masked scores).
 *   q_pos      int32 [B]; positions at or beyond max_pages * 16 are absent.
 *   row_start  int32 [B + 1], non-decreasing, row_start[0] = 0; a sequence
 *              with more than 8 rows contributes only its first 8 rows, and
 *              one whose rows do not lie within [0, row_start[B]) has none
 *              (nothing of it is read or written).
 *   out        float [R][Hq][D].
 *   ws         device workspace of at least *ws_bytes bytes, 16-byte
 *              aligned.  Call with ws == NULL to query the size: *ws_bytes
 *              is set and ISD_OK returned without launching anything.
 *   Hq % Hkv == 0, Hq / Hkv <= 16, D in {64, 128}, B >= 1, num_pages >= 1,
 *   1 <= max_pages <= 2^26 (2^30 positions); the launch's work count, u
 *   rounded up to a multiple of 8 times ceil(Hq / Hkv / 2), is below 2^31,
 *   where u = B * Hkv * ceil(max_pages / 16) (sequence, kv-head, chunk
 *   units).
 * Returns ISD_OK, ISD_EINVAL, ISD_ENOSPC or ISD_EHIP.
 */
int decode_attn(const uint16_t* q, const uint16_t* k_pages,
                const uint16_t* v_pages, const int32_t* page_table,
                int max_pages, int num_pages, const int32_t* q_pos,
                const int32_t* row_start, float* out, int B, int Hq, int Hkv,
                int D, float scale, void* ws, size_t* ws_bytes, void* stream);

/*
 * decode_attn_append -- kv_commit's APPEND followed by decode_attn, in the
 * launches of decode_attn alone: row j of sequence s (k_new / v_new, fp16
 * bits [R][Hkv][D], 16-byte aligned) is written at position
 * q_pos[s] + j of the cache -- positions past the table or on pages
 * outside [0, num_pages) are skipped, as APPEND skips them -- and the
 * attention outputs are those decode_attn gives after that append (the
 * block's own positions are read from k_new / v_new).  Outputs and cache
 * contents equal the two separate calls bit for bit.  Every other argument
 * is as for decode_attn (k_pages / v_pages are written).  Each kernel
 * boundary of a verify pass costs a few microseconds on its own, so the
 * append is done by the attention kernel.
 * Returns ISD_OK, ISD_EINVAL, ISD_ENOSPC or ISD_EHIP.
 */
int decode_attn_append(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                       uint16_t* k_pages, uint16_t* v_pages, const int32_t* page_table,
                       int max_pages, int num_pages, const int32_t* q_pos,
                       const int32_t* row_start, float* out, int B, int Hq, int Hkv, int D,
                       float scale, void* ws, size_t* ws_bytes, void* stream);

/*
 * spec_verify -- accept a prefix of each sequence's drafts and emit the
 * correction or bonus token (proofoftech.org, "'Lossless' speculative
 * decoding is a property of the math, not your deployment.", opening
 * section and section "Lossless is a theorem, and theorems have
 * hypotheses").
 *
 * Sequence s owns target rows row_start[s] .. row_start[s+1]-1
 * (k_s + 1 rows, 1 <= k_s + 1 <= 9; row j: the target's logits for the
 * token after input j) and draft entries row_start[s] - s .. row_start[s+1]
 * - s - 2 of `drafts` (d_1..d_k) and of `draft_logits`.
 *
 * temperature == 0 (greedy): t_j = the lowest id among the maxima of target
 *   row j (NaN never wins, -0 == +0).  a_s = the number of leading drafts
 *   with d_j == t_{j-1}; emitted: d_1..d_a, t_a.
 * temperature > 0 (sampling): p_j = softmax(target row j-1 / T),
 *   q_j = softmax(draft row j / T).  d_j is accepted if u < min(1,
 *   p_j(d_j)/q_j(d_j)) with u = U(seed, seq_id[s], pos0[s] + j - 1, 0);
 *   at the first rejection a token is drawn from max(0, p_j - q_j) by
 *   inverse CDF over ascending ids with u' = U(seed, seq_id[s], pos0[s] +
 *   j - 1, 1) (from p_j if that residual is all zero); if all k drafts are
 *   accepted a bonus token is drawn from p_{k+1} with U(..., pos0[s] + k, 1).
 *   U(seed, seq, pos, stream) = (w0 >> 8) * 2^-24 where w0 is the first
 *   word of Philox4x32-10 with key (seed low, seed high) and counter
 *   (pos, seq, stream, 0).
 *
 *   target_logits  float [R][V], R = row_start[B].
 *   draft_logits   float [R - B][V]; ignored (may be NULL) when greedy.
 *   drafts         int32 [R - B]; ids outside [0, V) are never accepted.
 *                  Neither may be NULL where it is used, even when R - B
 *                  is 0 (one row per sequence): any valid address then
 *                  serves, as nothing is read from it.
 *   row_start      int32 [B + 1], non-decreasing, row_start[0] = 0, every
 *                  sequence at least one row; a sequence with more than 9
 *                  rows uses only its first 9.  A sequence whose rows do
 *                  not lie within [0, row_start[B]) or [0, max_rows), or
 *                  whose draft entries do not lie within [0, R - B), is not
 *                  verified: accept_len 0, out_tokens all -1 (the forms
 *                  that commit still add accept_len + 1 to its seq_len).
 *   seq_id, pos0   int32 [B]; Philox key material (sampling only; may be
 *                  NULL when greedy).
 *   accept_len     int32 [B] output.
 *   out_tokens     int32 [B][9] output, unused slots set to -1.
 *   ws             workspace (query with ws == NULL as for decode_attn).
 *   B >= 1, V >= 1, max_rows = an upper bound on row_start[B] (used only to
 *   size the workspace and the grid), B <= max_rows <= ISD_MAX_VERIFY_ROWS;
 *   sampling also needs V <= 1048576.
 * Returns ISD_OK, ISD_EINVAL, ISD_ENOSPC or ISD_EHIP.
 */
int spec_verify(const float* target_logits, const float* draft_logits,
                const int32_t* drafts, const int32_t* row_start,
                const int32_t* seq_id, const int32_t* pos0, int B, int V,
                int max_rows, float temperature, uint64_t seed,
                int32_t* accept_len, int32_t* out_tokens, void* ws,
                size_t* ws_bytes, void* stream);

/*
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * spec_verify (the results are bit-identical), minus the workspace: it
 * uses a file-scope device array of ISD_VERIFY_SCRATCH_BYTES (1 MiB) in the
 * library instead, one copy per GPU, held until the process ends.  Its
 * device address is looked up on the first call on each device (the
 * current device; `stream` must belong to it).  The call allocates
 * nothing and needs no cleared memory (its counters are reset by its own
 * first launch).
 *
 *   Limit: the workspace spec_verify would ask for (greedy: 8 max_rows
 *   ceil(V/4096) bytes; sampling: about 16 max_rows ceil(V/4096) + 8 B
 *   ceil(V/4096) bytes) must fit in ISD_VERIFY_SCRATCH_BYTES, else
 *   ISD_ENOSPC and nothing is launched.
 *   Every call on one GPU shares that GPU's scratch: calls that may
 *   overlap on one GPU (different streams without ordering between them)
 *   race and must not be issued.
 * Returns ISD_OK, ISD_EINVAL, ISD_ENOSPC or ISD_EHIP (also when the
 * scratch address cannot be obtained).
 */
int spec_verify_noalloc(const float* target_logits, const float* draft_logits,
                        const int32_t* drafts, const int32_t* row_start,
                        const int32_t* seq_id, const int32_t* pos0, int B, int V,
                        int max_rows, float temperature, uint64_t seed,
                        int32_t* accept_len, int32_t* out_tokens, void* stream);

/*
 * kv_commit -- ragged paged-KV bookkeeping of a verify step
 * (proofoftech.org, same page, section "Batching breaks the
 * implementation": after unequal accepts, position ids, masks and per-
 * sequence KV state must be realigned exactly).
 *
 * APPEND (accept_len == NULL): the n_s = row_start[s+1] - row_start[s]
 *   rows of k_new / v_new (at most the first 8; row_start as for
 *   decode_attn, so a sequence whose rows do not lie within [0,
 *   row_start[B]) writes nothing) are written at positions seq_len[s] ..
 *   seq_len[s] + n_s - 1 of sequence s.  seq_len and pos_id are not
 *   changed.  Rows whose position falls outside the page table, or whose
 *   page id is outside [0, num_pages), are skipped.
 * COMMIT (accept_len != NULL): seq_len[s] += accept_len[s] + 1 and
 *   pos_id[s] = seq_len[s] (the last committed token plus the accepted
 *   drafts stay; rejected rows remain beyond seq_len and are overwritten
 *   by the next APPEND -- rollback by truncation).  k_new, v_new and the
 *   caches are not touched.
 *
 *   k_pages    fp16 [num_pages][Hkv][16][D], v_pages fp16 [num_pages][Hkv]
 *              [D][16] (the layouts decode_attn reads).
 *   k_new, v_new  fp16 [R][Hkv][D], R = row_start[B] (APPEND only).
 *   page_table int32 [B][max_pages].
 *   seq_len, pos_id  int32 [B], in/out.
 *   Hkv >= 1, D in {64, 128}, B >= 1, max_pages >= 1, num_pages >= 1.
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int kv_commit(uint16_t* k_pages, uint16_t* v_pages, const int32_t* page_table,
              int max_pages, int num_pages, const uint16_t* k_new,
              const uint16_t* v_new, const int32_t* row_start,
              int32_t* seq_len, int32_t* pos_id, const int32_t* accept_len,
              int B, int Hkv, int D, void* stream);

/*
 * spec_verify_margin -- greedy spec_verify (temperature 0) that also
 * reports how close each decision was: the margin between the two best
 * logits of every target row, and per sequence the first deciding row whose
 * margin is below `threshold`.  A near tie is the step where the last
 * rounding digit picks the token (tokenstrom.com, "'Lossless,' but not
 * quite", section "Why the math checks out and the text still flips"); a
 * caller can re-check just those steps instead of paying for deterministic
 * kernels everywhere (same page, section "What the big servers offer and
 * what it costs").
 *
 *   target_logits, drafts, row_start, B, V, max_rows, accept_len,
 *   out_tokens  as for spec_verify with temperature 0 (same results).
 *   threshold   margins strictly below it are flagged; not NaN.
 *   margins     float [R] output: top1 - top2 of each target row (exact fp32
 *               difference of the two largest values; +inf when V = 1; 0 for
 *               an exact tie; undefined for rows holding NaN).  Rows of
 *               sequences that cannot be verified are not written.
 *   recheck     int32 [B] output: the smallest j in 0..accept_len[s] (the
 *               rows that decided the emitted tokens) with margins[row_start
 *               [s] + j] < threshold, or -1.
 *   ws          workspace (query with ws == NULL as for decode_attn).
 * Returns ISD_OK, ISD_EINVAL, ISD_ENOSPC or ISD_EHIP.
 */
int spec_verify_margin(const float* target_logits, const int32_t* drafts,
                       const int32_t* row_start, int B, int V, int max_rows,
                       float threshold, int32_t* accept_len, int32_t* out_tokens,
                       float* margins, int32_t* recheck, void* ws,
                       size_t* ws_bytes, void* stream);

/*
 * spec_verify_commit -- greedy spec_verify (temperature 0) followed by
 * kv_commit's COMMIT, in one pair of launches instead of three: the same
 * accept_len and out_tokens as spec_verify, then seq_len[s] +=
 * accept_len[s] + 1 and pos_id[s] = seq_len[s] for every s < B.  Every
 * kernel boundary of a verify pass costs a few microseconds on its own, so
 * the commit is done by the kernel that decides the accept length.
 *
 *   target_logits, drafts, row_start, B, V, max_rows, accept_len,
 *   out_tokens, ws, ws_bytes  as for spec_verify with temperature 0.
 *   seq_len, pos_id  int32 [B] in/out, as for kv_commit.
 * Returns ISD_OK, ISD_EINVAL, ISD_ENOSPC or ISD_EHIP.
 */
int spec_verify_commit(const float* target_logits, const int32_t* drafts,
                       const int32_t* row_start, int B, int V, int max_rows,
                       int32_t* accept_len, int32_t* out_tokens, int32_t* seq_len,
                       int32_t* pos_id, void* ws, size_t* ws_bytes, void* stream);

/*
 * spec_verify_sampled_commit -- spec_verify with temperature > 0 followed
 * by kv_commit's COMMIT, in the launches of spec_verify alone: the same
 * accept_len and out_tokens as spec_verify with pos0 = pos_id, then
 * seq_len[s] += accept_len[s] + 1 and pos_id[s] = seq_len[s] for every
 * s < B, done by the work-group that draws sequence s's token (every
 * work-group of the sequence reads pos_id[s] before that one writes it).
 * The greedy verify's commit forms are spec_verify_commit and
 * spec_verify_keys; this is the same for the rejection-sampling rule (the
 * rule: proofoftech.org, as for spec_verify; the commit: same page,
 * section "Batching breaks the implementation", as for kv_commit).
 *
 *   target_logits, draft_logits, drafts, row_start, seq_id, B, V,
 *   max_rows, temperature, seed, accept_len, out_tokens, ws, ws_bytes
 *              as for spec_verify; temperature > 0.
 *   seq_len, pos_id  int32 [B] in/out, as for kv_commit; pos_id is also
 *              spec_verify's pos0 (the position of each block's first row).
 * Returns ISD_OK, ISD_EINVAL, ISD_ENOSPC or ISD_EHIP.
 */
int spec_verify_sampled_commit(const float* target_logits, const float* draft_logits,
                               const int32_t* drafts, const int32_t* row_start,
                               const int32_t* seq_id, int B, int V, int max_rows,
                               float temperature, uint64_t seed, int32_t* accept_len,
                               int32_t* out_tokens, int32_t* seq_len, int32_t* pos_id,
                               void* ws, size_t* ws_bytes, void* stream);

/*
 * spec_verify_keys -- the greedy verify (and, with seq_len, the commit) of
 * spec_verify_commit from the keys of qgemm_w4_argmax instead of the
 * logits: a target row's token is the index in the largest of its keys.
 * The maximum of keys is order-free, so accept_len and out_tokens equal
 * those of spec_verify on the logits the keys were made from.
 *
 *   keys       uint64 [max_rows][nkeys] (rows as in spec_verify), 8-byte
 *              aligned.
 *   nkeys      keys per row, >= 1.
 *   B <= max_rows <= ISD_MAX_VERIFY_ROWS.
 *   drafts, row_start, B, max_rows, accept_len, out_tokens  as for
 *              spec_verify with temperature 0.
 *   seq_len, pos_id  both NULL (no commit) or both int32 [B] in/out, as
 *              for spec_verify_commit.
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int spec_verify_keys(const uint64_t* keys, int nkeys, const int32_t* drafts,
                     const int32_t* row_start, int B, int max_rows, int32_t* accept_len,
                     int32_t* out_tokens, int32_t* seq_len, int32_t* pos_id, void* stream);

/*
 * Row-wise layer operations.  Together with qgemm_w4, decode_attn and
 * kv_commit they run a whole decoder layer, so that the end-to-end property
 * -- speculative output equal to serial greedy decoding -- can be checked
 * through a multi-layer target (ramgpt.org, "When Lossless Speculation Stops
 * Being Lossless on Blackwell", sections "Why Tiny Numerical Differences Can
 * Change Entire Answers" and "A Better Backend Test Matrix").  Each output
 * row is a function of that row's inputs only, in one fixed order.
 *
 * embed_rows  h[r][:] = table[tokens[r]][:] as fp32.
 *   tokens int32 [rows] (ids outside [0, V) give zero rows); table bf16 bits
 *   [V][H]; h float [rows][H].
 *
 * add_rmsnorm  if d != NULL: h[r] += d[r] (in place); then
 *   y[r] = bf16(h[r] / sqrt(mean(h[r]^2) + eps) * w), the sum of squares
 *   in one fixed order per row.
 *   h float [rows][H] (in/out); d float [rows][H] or NULL; w float [H];
 *   y bf16 bits [rows][H].  1 <= H <= 8192, eps >= 0.
 *
 * rope_qkv  split rows of [Hq q heads | Hkv k heads | Hkv v heads] (fp32,
 *   head size D) and rotate q and k: pair (i, i + D/2) of a head turns by
 *   pos * theta^(-2i/D), where row r of sequence s (row_start[s] <= r <
 *   row_start[s+1]) sits at pos = pos_id[s] + r - row_start[s]; angles and
 *   rotation in fp64, results rounded to fp16.
 *   qkv float [rows][(Hq + 2 Hkv) D]; row_start int32 [B + 1]; pos_id
 *   int32 [B]; q fp16 bits [rows][Hq][D]; k, v fp16 bits [rows][Hkv][D].
 *   Rows in no sequence's range (past row_start[B]) are not written; a
 *   row in several (malformed offsets) takes the lowest such sequence.
 *   2 <= D <= 128 even, theta > 1,
 *   (Hq + 2 Hkv) D < 2^31.
 *
 * silu_mul  y[r][i] = bf16(silu(g) * u), g = gu[r][i], u = gu[r][F + i],
 *   silu(g) = g / (1 + e^-g).  gu float [rows][2F]; y bf16 bits [rows][F].
 *
 * All return ISD_OK, ISD_EINVAL or ISD_EHIP; pointers are device pointers,
 * float arrays 4-byte aligned, 16-bit arrays 2-byte aligned.
 */
int embed_rows(const int32_t* tokens, const uint16_t* table, float* h, int rows,
               int V, int H, void* stream);
int add_rmsnorm(float* h, const float* d, const float* w, uint16_t* y, int rows,
                int H, float eps, void* stream);
int rope_qkv(const float* qkv, const int32_t* row_start, const int32_t* pos_id,
             int B, int rows, int Hq, int Hkv, int D, float theta, uint16_t* q,
             uint16_t* k, uint16_t* v, void* stream);
int silu_mul(const float* gu, uint16_t* y, int rows, int F, void* stream);

/*
 * stream_read -- measurement only, not a step of the verify pass: one read
 * of `bytes` bytes of `buf` with 16-byte non-temporal loads, 32 KB per
 * work-group, nothing computed but an XOR fold.  Its rate is the practical
 * HBM read ceiling the other kernels are compared with.
 *   buf   device buffer, 16-byte aligned; bytes >= 16, a multiple of 16.
 *   sink  uint32 [sink_words] device buffer, sink_words >=
 *         stream_read_sink_words(bytes); almost never written.
 * Returns ISD_OK, ISD_EINVAL or ISD_EHIP.
 */
int stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                void* stream);
size_t stream_read_sink_words(size_t bytes);

/* Library version string, e.g. "isd 0.1 gfx950". */
const char* isd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ISD_H */
