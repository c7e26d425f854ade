/*
 * kvc.h - C ABI of the MI355X (gfx950) KV compressor.
 *
 * The compressor turns each block of `compress_ratio` tokens of a request
 * into one compressed kv row.  Ratio 4 pools a window of 8 tokens (the block
 * being closed plus the block before it); ratio 128 pools the 128 tokens of
 * the block.  Every output channel d is
 *
 *     out[d] = sum_i exp(t_i[d]) kv_i[d] / sum_i exp(t_i[d]),
 *     t_i[d] = score_i[d] + ape[i][d]
 *
 * over the window entries i (c4.cuh page, c4_forward; compressor_v2.py page,
 * _c128_compress_prefill_compress_kernel and _compress_forward_c128_fallback).
 *
 * Pages cited below: "c_plan.cuh" is
 * sgl-project--sglang/python/sglang/jit_kernel/csrc/deepseek_v4/c_plan.cuh,
 * "c4.cuh" is .../jit_kernel/csrc/deepseek_v4/c4.cuh and "compressor_v2.py"
 * is .../srt/layers/attention/dsv4/compressor_v2.py.
 *
 * Conventions for every call
 * --------------------------
 *  - Pointers to tensors, plans, counts and status words are DEVICE pointers
 *    (HBM of the current HIP device).  Tensors and C / D record buffers are
 *    16-byte aligned, W record buffers 8-byte, int32 arrays (lengths,
 *    indices, counts, status words) 4-byte; a misaligned or null pointer is
 *    KVC_EINVAL.  Sizes are host ints.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on `stream`: it never synchronises, never
 *    allocates and keeps no pointer after it returns.  The caller owns every
 *    buffer and must keep it alive until the stream has run the work.
 *  - Return value: KVC_OK, or KVC_EINVAL when a host-visible argument is bad
 *    (nothing is enqueued), or KVC_EHIP when the launch failed.
 *  - Errors in DEVICE data (lengths, indices, records) cannot be seen on the
 *    host without a sync.  They are reported as bits in a device error word
 *    (KVC_DERR_*), and the offending work is skipped, never performed out of
 *    bounds.
 *
 * Data layout
 * -----------
 *  - dtype KVC_BF16 (bf16 bit patterns) or KVC_F32; `ape`, input and state
 *    share the dtype.  head_dim (hd) is 128, 256 or 512.
 *  - A ratio-4 row holds 4*hd elements laid out |kv overlap|kv|score
 *    overlap|score| (c4.cuh, Compress4PrefillParams).  Window entries 0..3
 *    (the previous block) use the two overlap quarters, entries 4..7 the
 *    others.  A ratio-128 row holds 2*hd elements laid out |kv|score|.
 *  - The input is the ragged batch [num_q, row] (requests back to back, each
 *    request's new tokens in position order); decode input is [B, row].
 *  - The state buffer is [num_state_rows, row].  Ratio 4: request slot `idx`
 *    owns rows idx*8 .. idx*8+7, two pages of 4 rows, position p at page
 *    idx*2 + ((p/4) & 1), row page*4 + p%4.  Ratio 128: slot `idx` owns the
 *    page of rows idx*128 .. idx*128+127, position p at row idx*128 + p%128
 *    (c_plan.cuh, plan_compress_prefill_legacy_kernel).
 *  - `ape` is [8, hd] (ratio 4) or [128, hd] (ratio 128).
 *  - Compressed output is float32 [rows, hd].
 *
 * Arithmetic and accuracy of the pool
 * -----------------------------------
 *  - bf16 inputs are pooled in fp32 (bf16 widens exactly).  score + ape and
 *    the differences to the window maximum are then exact for scores of any
 *    usual size, and a weight carries the exponential's few-ulp error: a
 *    pooled value is within 2e-2 of the exact one for |kv| up to about 10^4.
 *  - fp32 inputs are pooled in fp64 (score + ape, the window maximum, the
 *    exponential, both sums and the quotient), then rounded once to fp32.
 *    For any finite input with |kv| <= 2^30 a pooled value is within
 *    1e-5 + 1e-5 * |exact| of the exact one, whatever the scores' size.
 *  - The online ratio-128 slot (kvc_*_c128_online) keeps its running sums
 *    in fp32 between calls: each call that stores a slot moves the value it
 *    stands for by at most 2^-23 * max |kv| of the block, so rows built
 *    over many calls carry that much more.
 *
 * Call order
 * ----------
 *  prefill chunk: kvc_plan_prefill -> kvc_compress_c4 | kvc_compress_c128 ->
 *                 kvc_write (compress must read the state as it was before
 *                 this chunk's writes: c4.cuh, flash_c4_prefill launches the
 *                 compress kernel before the write kernel);
 *  decode step:   kvc_plan_decode -> kvc_decode_c4 | kvc_decode_c128 (for
 *                 ratio 128 the planner can also write a boundary list that
 *                 the decode then takes: the same results, fewer loads).
 *  The compressed rows then go through norm + rotary embedding into a bf16
 *  cache: kvc_norm_rope_store_prefill / kvc_norm_rope_store_decode after the
 *  pool, or kvc_compress_c4_norm_rope_store / kvc_compress_c128_norm_rope_store
 *  in place of the prefill pool (still before kvc_write), and
 *  kvc_decode_c4_norm_rope_store in place of kvc_decode_c4.
 *  Plans depend only on lengths and indices, so one plan serves every layer.
 *  The state slots of one call must be distinct: the prefill planners check
 *  it (KVC_DERR_DUPLICATE, a plan error); for a decode batch it is the
 *  caller's precondition (two requests on one slot make the decode's writes
 *  and pools race).
 */
#ifndef KVC_H_
#define KVC_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* host return codes */
#define KVC_OK 0
#define KVC_EINVAL (-1)
#define KVC_EHIP (-2)

/* device error bits (counts[2], counts[3] or *status) */
#define KVC_DERR_EXTEND 1   /* prefill: extend_len <= 0 or > seq_len; decode: seq_len <= 0 */
#define KVC_DERR_NUMQ 2     /* prefill: sum of extend_len != num_q */
#define KVC_DERR_INDEX 4    /* state_index outside [0, num_state_rows / window) */
#define KVC_DERR_CAPACITY 8 /* prefill: more C or W records than cap_c or cap_w */
#define KVC_DERR_RECORD 16  /* a consumer met a record that points outside its buffers */
#define KVC_DERR_DUPLICATE 32 /* prefill: two requests name the same state slot */

/* limits */
#define KVC_MAX_PREFILL_BATCH 1024
#define KVC_MAX_DECODE_BATCH 65536
#define KVC_MAX_TOKENS (1 << 24)

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* Compress record, 16 bytes: one per compressed row of a prefill chunk
 * (c_plan.cuh, CompressPlan as filled by plan_compress_prefill_legacy and
 * its translation kernel).  The row closes the window ending at token
 * seq_len - 1; ragged_id is that token's row in the ragged input;
 * buffer_len (0..127) counts the window entries that precede the chunk and
 * are read from the state; the others are input rows ragged_id - (W-1) + i.
 * read_page_1 is the page of position seq_len - 1, read_page_0 the page of
 * position max(seq_len - 1 - ratio, 0).  The page's ragged id is 16 bits
 * wide; here it takes bits 0..23 and buffer_len bits 24..31. */
typedef struct kvc_plan_c {
  uint32_t seq_len;
  uint32_t ragged_blen; /* ragged_id | buffer_len << 24 */
  int32_t read_page_0;
  int32_t read_page_1;
} kvc_plan_c;

/* Write record, 8 bytes: copy input row ragged_id to state row write_loc
 * (c_plan.cuh, WritePlan). */
typedef struct kvc_plan_w {
  uint32_t ragged_id;
  int32_t write_loc;
} kvc_plan_w;

/* Decode record, 16 bytes (c_plan.cuh, DecodePlan via
 * plan_compress_decode_legacy_kernel): the new token is position
 * seq_len - 1 and goes to state row write_loc; read pages as for kvc_plan_c. */
typedef struct kvc_plan_d {
  uint32_t seq_len;
  int32_t write_loc;
  int32_t read_page_0;
  int32_t read_page_1;
} kvc_plan_d;

/* An invalid (padding) record has every byte 0xFF: seq_len == 0xFFFFFFFF
 * for C and D records, ragged_id == 0xFFFFFFFF for W records. */

/*
 * kvc_plan_prefill - plan one ragged prefill chunk (c_plan.cuh,
 * plan_compress_prefill_legacy and plan_compress_prefill_legacy_kernel;
 * the device-built variant is plan_compress_prefill_kernel0).
 *
 * For request b (seq_len s, extend_len e, prefix p0 = s - e, new tokens at
 * positions p0 .. s-1, ragged rows starting at the sum of earlier extends):
 *  - position p emits a C record iff (p + 1) % ratio == 0;
 *  - position p emits a W record iff p >= floor(s/ratio)*ratio - (ratio==4 ? 4 : 0),
 *    i.e. the chunk's tokens that the next window still needs.
 * Records are ordered request by request, positions ascending (the order of
 * the pages' host loop); the build is deterministic.  Records [num_c, cap_c)
 * and [num_w, cap_w) are filled with invalid records.
 *
 *  compress_ratio  4 or 128
 *  batch           1 .. KVC_MAX_PREFILL_BATCH requests
 *  num_q           batch .. KVC_MAX_TOKENS-1 rows in the ragged input
 *  seq_lens, extend_lens, state_index   device int32 [batch]
 *  num_state_rows  rows of the state buffer (0 .. INT32_MAX); a state index
 *                  must lie in [0, num_state_rows / W), W = 8 or 128, and no
 *                  two requests may share one (KVC_DERR_DUPLICATE)
 *  plan_c, cap_c   device output, cap_c >= 0 records (never more than
 *                  min(num_q, num_q/ratio + batch) are needed)
 *  plan_w, cap_w   device output, cap_w >= 0 records (never more than
 *                  min(num_q, batch*(W-1)) are needed)
 *  counts          device int32 [4], written: num_c, num_w, device error
 *                  bits of the plan, 0 (consumers OR their errors into
 *                  counts[3]).  On any plan error num_c = num_w = 0 and every
 *                  record is invalid, so the consumers do nothing.
 *  runs            NULL, or (ratio 128 only) device int32 [batch, 4], 16-byte
 *                  aligned, written: for request b its run of W records as
 *                  (ragged_id of the first, write_loc of the first, n, 0); the
 *                  run's records are positions write_loc % 128 .. + n - 1 of
 *                  one page with consecutive ragged rows.  A request without
 *                  W records, and every request of a plan with an error, gets
 *                  (0, 0, 0, 0).
 *                  kvc_write_c128_online takes it in place of a scan of the W
 *                  records.  NULL for ratio 4 (else KVC_EINVAL).
 */
int kvc_plan_prefill(int compress_ratio, int batch, int num_q, const int32_t* seq_lens,
                     const int32_t* extend_lens, const int32_t* state_index, int64_t num_state_rows,
                     kvc_plan_c* plan_c, int cap_c, kvc_plan_w* plan_w, int cap_w, int32_t* counts,
                     int32_t* runs, void* stream);

/*
 * kvc_plan_decode - plan one decode step, one record per request
 * (c_plan.cuh, plan_compress_decode_legacy_kernel).  seq_lens are the
 * lengths AFTER the new token.  A request with seq_len <= 0 or a state index
 * out of range gets an invalid record; `status` (device int32 [1], may be
 * NULL) receives the OR of the error bits.
 *  batch 1 .. KVC_MAX_DECODE_BATCH.
 *
 * boundaries (ratio 128 only, else NULL; may be NULL): device int32
 * [2 * batch + 2], 8-byte aligned, owned by the caller.  The planner fills
 * it with the boundary list, an index of the records for kvc_decode_c128:
 * each of the n requests whose record is valid and whose seq_len % 128 == 0
 * (the new token closes a block) has one entry, the pair (request b,
 * read_page_0 of its record) at [2k], [2k + 1] for some k < n; the order of
 * the entries is not fixed and may differ between calls.  n is at
 * [2 * batch] and [2 * batch + 1] is 0; entries past n are left as they
 * were.  The list is not part of the method: it lets the decode find its
 * pooling requests without scanning the records.
 */
int kvc_plan_decode(int compress_ratio, int batch, const int32_t* seq_lens, const int32_t* state_index,
                    int64_t num_state_rows, kvc_plan_d* plan_d, int32_t* boundaries, int32_t* status,
                    void* stream);

/*
 * SWA-paged state mapping (c_plan.cuh page: plan_compress_prefill_kernel0,
 * plan_compress_prefill_kernel_1, plan_compress_decode_kernel).
 *
 * A serving system that keeps the ratio-4 state in its sliding-window (SWA)
 * page pool plans with these two calls instead of the per-request ones; the
 * records have the same layout and feed the same compress / write / decode
 * calls.  Tables (device int32):
 *   req_to_token [num_reqs, r2t_stride]: full-cache slot of token pos of
 *                 request slot rid (row rid = req_pool_indices[b]);
 *   full_to_swa  [num_full]: SWA slot of a full-cache slot (< 0: none).
 * Ratio 4: the token lives at state row (swa / swa_page_size) * ring_size +
 * swa % ring_size, swa = full_to_swa[req_to_token[rid][pos]]: every SWA page
 * owns a ring of ring_size rows.  Ratio 128 keeps its request-scoped ring:
 * row rid * ring_size + pos % ring_size.
 * Write rule: as kvc_plan_prefill, but the first unconditionally written
 * position is capped at seq_len - min(ring_size - ratio, 4), and ratio 4 also
 * writes the last 4 positions of every SWA page (a request that resumes at a
 * page boundary reads them as its first window's overlap block).
 * A C record with buffer_len 0 reads nothing from the state and keeps
 * read_page_0 = -1, read_page_1 = its batch index (untranslated).
 * Requirements (else KVC_EINVAL): swa_page_size % ring_size == 0; ratio 4:
 * ring_size a multiple of 8; ratio 128: ring_size == 128.
 * Errors: seq_len > r2t_stride or a request slot outside [0, num_reqs) is a
 * plan error (KVC_DERR_INDEX in counts[2], no records), and so are two
 * requests with one request slot (KVC_DERR_DUPLICATE).  A lookup that leaves
 * its table, a missing SWA slot or a row outside the state buffer makes just
 * that record invalid and ORs KVC_DERR_INDEX into *status (device int32,
 * may be NULL; the caller clears it).
 */
int kvc_plan_prefill_swa(int compress_ratio, int batch, int num_q, const int32_t* seq_lens,
                         const int32_t* extend_lens, const int32_t* req_pool_indices, const int32_t* req_to_token,
                         int64_t r2t_stride, int64_t num_reqs, const int32_t* full_to_swa, int64_t num_full,
                         int swa_page_size, int ring_size, int64_t num_state_rows, kvc_plan_c* plan_c, int cap_c,
                         kvc_plan_w* plan_w, int cap_w, int32_t* counts, int32_t* status, void* stream);

/*
 * kvc_plan_decode_swa - one decode record per request under the SWA-paged
 * mapping: write_loc = row of position seq_len - 1, read pages = rows of
 * positions max(seq_len - 1 - ratio, 0) and seq_len - 1 divided by the ratio.
 * A request with seq_len <= 0, a bad slot or a failed lookup gets an invalid
 * record; *status (may be NULL) receives the OR of the error bits.
 * boundaries: as for kvc_plan_decode (ratio 128 only, may be NULL).
 */
int kvc_plan_decode_swa(int compress_ratio, int batch, const int32_t* seq_lens, const int32_t* req_pool_indices,
                        const int32_t* req_to_token, int64_t r2t_stride, int64_t num_reqs, const int32_t* full_to_swa,
                        int64_t num_full, int swa_page_size, int ring_size, int64_t num_state_rows,
                        kvc_plan_d* plan_d, int32_t* boundaries, int32_t* status, void* stream);

/*
 * Ratio 4 over caller-allocated 4-row pages (c4.cuh page, PageMode::Page4Align
 * with C4IndexBundle in flash_c4_prefill, and the previous page of
 * flash_c4_decode).  Instead of the per-request ring of two pages, the caller
 * hands over the pages (4 state rows each; page P is rows 4P .. 4P+3); the
 * records are ordinary C / W / D records for kvc_compress_c4, kvc_write and
 * kvc_decode_c4.
 *
 * kvc_plan_prefill_page4 - as kvc_plan_prefill (ratio 4) with, per request
 * b, page_index[b] (the page of the positions from last_position on) and
 * bundle[b] (device int32 [batch, 4], 16-byte aligned) = {load_first_page,
 * load_second_page, write_first_page, last_position}:
 *  - a C record whose window reaches before the chunk (buffer_len > 0)
 *    reads those entries from load_second_page when buffer_len <= 4, else
 *    entries 0..3 from load_first_page and 4.. from load_second_page
 *    (read_page_0 / read_page_1); other C records carry pages -1;
 *  - the written positions are those of kvc_plan_prefill; position p goes to
 *    row (p < last_position ? write_first_page : page_index[b]) * 4 + p % 4.
 * A page_index outside [0, num_state_rows / 4) is a plan error
 * (KVC_DERR_INDEX in counts[2], no records), and so is a page_index that two
 * requests share (KVC_DERR_DUPLICATE).  A bundle page outside that
 * range which a record reads or writes makes that record invalid and ORs
 * KVC_DERR_INDEX into *status (may be NULL; the caller clears it); pages that
 * are not read (the first block's masked entries) are not checked.
 */
int kvc_plan_prefill_page4(int batch, int num_q, const int32_t* seq_lens, const int32_t* extend_lens,
                           const int32_t* page_index, const int32_t* bundle, int64_t num_state_rows,
                           kvc_plan_c* plan_c, int cap_c, kvc_plan_w* plan_w, int cap_w, int32_t* counts,
                           int32_t* status, void* stream);

/*
 * kvc_plan_decode_page4 - one decode record per request: the new token
 * (position seq_len - 1) goes to page_index[b] at slot (seq_len - 1) % 4
 * (write_loc), read_page_1 = page_index[b], read_page_0 = prev_page[b] (the
 * page of the block before; read only when seq_len % 4 == 0 and
 * seq_len > 4).  A request with seq_len <= 0 or a needed page out of range
 * gets an invalid record; *status (may be NULL) receives the error bits.
 *  batch 1 .. KVC_MAX_DECODE_BATCH.
 */
int kvc_plan_decode_page4(int batch, const int32_t* seq_lens, const int32_t* page_index, const int32_t* prev_page,
                          int64_t num_state_rows, kvc_plan_d* plan_d, int32_t* status, void* stream);

/*
 * kvc_write - for each valid W record k < counts[1], copy input row
 * ragged_id (all 4*hd or 2*hd elements, bit for bit) into state row
 * write_loc (c4.cuh, c4_write; compressor_v2.py,
 * _c128_compress_prefill_write_kernel).  Must run after the chunk's
 * compress.  A record outside [0, num_q) x [0, num_state_rows) is skipped
 * and sets KVC_DERR_RECORD in counts[3].
 */
int kvc_write(int compress_ratio, kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows,
              const void* input, int num_q, const kvc_plan_w* plan_w, int cap_w, int32_t* counts, void* stream);

/*
 * kvc_compress_c4 - pool every valid C record k < counts[0] of a ratio-4
 * plan into out[k] (float32 [cap_c, hd]; rows >= counts[0] are untouched).
 * Window entry i (0..7) is state row (i < 4 ? read_page_0*4 + i :
 * read_page_1*4 + i - 4) when i < buffer_len, else input row
 * ragged_id - 7 + i.  When seq_len == 4 (the first block) entries 0..3 lie
 * before the sequence and take no part (c4.cuh, c4_forward: kv 0,
 * score -1e9, whose weight is exactly zero); their rows are not read.
 * Reads the state as it was before this chunk's kvc_write.
 * ape: [8, hd], same dtype as input and state.
 */
int kvc_compress_c4(kvc_dtype dtype, int head_dim, const void* state, int64_t num_state_rows, const void* input,
                    int num_q, const void* ape, const kvc_plan_c* plan_c, int cap_c, int32_t* counts, float* out,
                    void* stream);

/*
 * kvc_compress_c128 - as kvc_compress_c4 for ratio 128: entry i (0..127)
 * is state row read_page_0*128 + i when i < buffer_len, else input row
 * ragged_id - 127 + i (compressor_v2.py, _c128_compress_prefill_compress_kernel
 * and _compress_forward_c128_fallback).  ape: [128, hd].
 */
int kvc_compress_c128(kvc_dtype dtype, int head_dim, const void* state, int64_t num_state_rows,
                      const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c, int cap_c,
                      int32_t* counts, float* out, void* stream);

/*
 * kvc_decode_c4 - fused decode step for ratio 4 (c4.cuh, flash_c4_decode):
 * for each request b, write input row b to state row write_loc; if
 * seq_len % 4 == 0, pool the 8-entry window ending at the new token (read
 * from the state after the write; first-block masking as in
 * kvc_compress_c4) into out[b], else set out[b] to zeros.  An invalid
 * record gives a zero row and no write.  A record pointing outside the state
 * gives a zero row, no write, and KVC_DERR_RECORD in *status (status may be
 * NULL; it is OR-ed, not cleared).  out: float32 [batch, hd].
 */
int kvc_decode_c4(kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows, const void* input,
                  const void* ape, const kvc_plan_d* plan_d, int batch, int32_t* status, float* out, void* stream);

/*
 * kvc_decode_c128 - fused decode step for ratio 128 (compressor_v2.py,
 * _c128_compress_decode_kernel): as kvc_decode_c4 with the 128-entry window
 * of page read_page_0, pooled when seq_len % 128 == 0.
 * boundaries (may be NULL; 8-byte aligned): the boundary list that
 * kvc_plan_decode or kvc_plan_decode_swa wrote in the same call as plan_d.
 * With it, the pooled rows are those of its entries; without it, the decode
 * finds the pooling requests in plan_d itself.  The results are the same,
 * bit for bit.  A list that does not match plan_d is the caller's error:
 * the count is clamped to [0, batch], an entry outside the batch or the
 * state is skipped with KVC_DERR_RECORD in *status, and other mismatches
 * leave the pooled rows undefined (never an access outside the buffers).
 */
int kvc_decode_c128(kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows, const void* input,
                    const void* ape, const kvc_plan_d* plan_d, const int32_t* boundaries, int batch,
                    int32_t* status, float* out, void* stream);

/*
 * Norm, rotary embedding and store of the compressed rows (compressor_v2.py
 * page: compress_norm_rope_store, and the steps of _forward_unified_hip that
 * follow the pool).  Each stored row x (head_dim fp32 channels) becomes
 *
 *     y_d = x_d / sqrt(mean_e x_e^2 + eps) * norm_weight[d]      (RMSNorm)
 *
 * then its last rope_dim channels, taken as rope_dim/2 complex numbers
 * (y[2k] + i y[2k+1] of that slice), are multiplied by
 * freqs_cis[pos][k] = cos + i sin, pos = seq_len - compress_ratio of the
 * record (_extract_positions_from_plan; never negative for a stored row), and
 * y is rounded to bf16 (nearest even) into cache row out_loc[key].  Prefill:
 * one stored row per valid C record, key = its ragged_id.  Decode: one per
 * valid D record whose seq_len is a multiple of the ratio, key = b; the rows
 * of the other requests are not stored (the pages store a zero row at
 * location 0 for them).  The fp8 / fp4 cache packs and the indexer's
 * Hadamard rotation are not part of this step.  Arithmetic is fp32.
 * A record whose key, location or position falls outside num_loc,
 * num_cache_rows or max_position (position checked only when rope_dim > 0)
 * is not stored and sets KVC_DERR_RECORD (prefill: counts[3]; decode:
 * *status, may be NULL).  Two stored rows of one call must not share a
 * location.
 */
typedef struct kvc_store_args {
  const float* norm_weight; /* device fp32 [head_dim] */
  const float* freqs_cis;   /* device fp32 [max_position, rope_dim / 2, 2] (cos, sin); unused if rope_dim == 0 */
  const int32_t* out_loc;   /* device int32 [num_loc]: cache row per ragged token (prefill) or request (decode) */
  uint16_t* cache;          /* device bf16 bit patterns [num_cache_rows, head_dim] */
  int64_t num_loc;          /* 0 .. INT32_MAX */
  int64_t max_position;     /* rows of freqs_cis, >= 0 */
  int64_t num_cache_rows;   /* 0 .. INT32_MAX */
  float eps;                /* >= 0, finite */
  int32_t rope_dim;         /* 0 .. head_dim, a multiple of 8 */
} kvc_store_args;

/*
 * kvc_norm_rope_store_prefill - store the compressed rows of a prefill
 * chunk: row k of `rows` (float32 [cap_c, head_dim], as kvc_compress_c4 /
 * kvc_compress_c128 leave it) for every valid C record k < counts[0].
 * `args` is a HOST pointer, read during the call.
 */
int kvc_norm_rope_store_prefill(int compress_ratio, int head_dim, const float* rows, const kvc_plan_c* plan_c,
                                int cap_c, int32_t* counts, const kvc_store_args* args, void* stream);

/*
 * kvc_norm_rope_store_decode - store the rows of a decode step that close a
 * block: row b of `rows` (float32 [batch, head_dim], as kvc_decode_c4 /
 * kvc_decode_c128 leave it) for every valid D record b with
 * seq_len % compress_ratio == 0.  `args` is a HOST pointer.
 */
int kvc_norm_rope_store_decode(int compress_ratio, int head_dim, const float* rows, const kvc_plan_d* plan_d,
                               int batch, int32_t* status, const kvc_store_args* args, void* stream);

/*
 * kvc_compress_c4_norm_rope_store / kvc_compress_c128_norm_rope_store -
 * kvc_compress_c4 / kvc_compress_c128 followed by
 * kvc_norm_rope_store_prefill in one kernel: the pooled row stays in
 * registers and only its bf16 form reaches HBM (no float32 rows).  Same
 * arguments as the pool, with `args` (HOST pointer) in place of `out`; the
 * stored values are those of the two calls in sequence, up to fp32 rounding.
 */
int kvc_compress_c4_norm_rope_store(kvc_dtype dtype, int head_dim, const void* state, int64_t num_state_rows,
                                    const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c,
                                    int cap_c, int32_t* counts, const kvc_store_args* args, void* stream);
int kvc_compress_c128_norm_rope_store(kvc_dtype dtype, int head_dim, const void* state, int64_t num_state_rows,
                                      const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c,
                                      int cap_c, int32_t* counts, const kvc_store_args* args, void* stream);

/*
 * kvc_decode_c4_norm_rope_store - kvc_decode_c4 followed by
 * kvc_norm_rope_store_decode in one kernel: the new token goes to the state
 * as in kvc_decode_c4, and a request whose seq_len closes a block has its
 * pooled row normalised, rotated and stored as bf16 at out_loc[b]; nothing
 * is written for the other requests (no float32 rows).  Same arguments as
 * kvc_decode_c4 with `args` (HOST pointer) in place of `out`.  A record or
 * store target out of range sets KVC_DERR_RECORD in *status (may be NULL).
 */
int kvc_decode_c4_norm_rope_store(kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows,
                                  const void* input, const void* ape, const kvc_plan_d* plan_d, int batch,
                                  int32_t* status, const kvc_store_args* args, void* stream);

/*
 * Online ratio-128 state (compressor_v2.py page, _use_online_compress and
 * _forward_unified: the state of a request is one slot of 3 * head_dim
 * values instead of a 128-row page).  A slot is fp32 [3, hd]: per channel
 * the running maximum m, the running sum l = sum exp(t - m) and the running
 * weighted sum acc = sum exp(t - m) kv over the positions of the request's
 * unfinished block, t = score + ape[pos % 128].  `state` is a device fp32
 * array of num_slots such slots (6 KiB each at hd 512).  The ordinary
 * ratio-128 plans drive it, built with num_state_rows = 128 * num_slots
 * (request slot idx owns virtual rows idx*128 .. idx*128+127); record fields
 * keep their meaning, and a slot holds nothing until its first token.
 * Call order per prefill chunk: kvc_plan_prefill (or _swa) ->
 * kvc_compress_c128_online -> kvc_write_c128_online; per decode step:
 * kvc_plan_decode (or _swa) -> kvc_decode_c128_online.
 *
 * kvc_compress_c128_online - for each valid C record k < counts[0]: pool
 * window entries [buffer_len, 128) (input rows ragged_id - 127 + i, ape row
 * i) and, when buffer_len > 0, the partial in slot read_page_0; out[k] =
 * acc / l (float32 [cap_c, hd]).  A record whose rows or slot are out of
 * range is skipped and sets KVC_DERR_RECORD in counts[3].
 */
int kvc_compress_c128_online(kvc_dtype dtype, int head_dim, const float* state, int64_t num_slots,
                             const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c, int cap_c,
                             int32_t* counts, float* out, void* stream);

/*
 * kvc_write_c128_online - fold each request's run of W records (consecutive
 * records of one slot, write_loc / 128, with consecutive rows and positions)
 * into its slot: positions write_loc % 128 .. on of the block, input rows
 * from ragged_id, ape rows by position.  The run starts a fresh block when
 * its first position is a multiple of 128, else it continues the slot.  Must
 * run after the chunk's kvc_compress_c128_online.  A run whose rows or slot
 * are out of range is skipped and sets KVC_DERR_RECORD in counts[3].
 *  runs, batch     NULL (batch unused): the runs are found by scanning
 *                  plan_w.  Else the run list that kvc_plan_prefill wrote
 *                  for the same chunk (int32 [batch, 4], 16-byte aligned,
 *                  1 <= batch <= KVC_MAX_PREFILL_BATCH): one run per entry
 *                  with n > 0, nothing when counts[1] == 0.  The slots end
 *                  bit for bit as with the scan.
 */
int kvc_write_c128_online(kvc_dtype dtype, int head_dim, float* state, int64_t num_slots, const void* input,
                          int num_q, const void* ape, const kvc_plan_w* plan_w, int cap_w, int32_t* counts,
                          const int32_t* runs, int batch, void* stream);

/*
 * kvc_decode_c128_online - for each request b: fold input row b at position
 * seq_len - 1 into slot read_page_0 (a fresh block when that position is a
 * multiple of 128); out[b] = acc / l when seq_len % 128 == 0, else zeros
 * (float32 [batch, hd]).  An invalid record gives a zero row; a slot out of
 * range gives a zero row and KVC_DERR_RECORD in *status (may be NULL).
 */
int kvc_decode_c128_online(kvc_dtype dtype, int head_dim, float* state, int64_t num_slots, const void* input,
                           const void* ape, const kvc_plan_d* plan_d, int batch, int32_t* status, float* out,
                           void* stream);

/* kvc_strerror - static text for a host return code or a device error bit. */
const char* kvc_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
