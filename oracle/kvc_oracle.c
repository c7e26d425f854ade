/*
 * kvc_oracle.c - plain, slow CPU oracle for the KV-compressor hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the graft
 * entry point and the cpu_baseline leg of bench.py may load this library.
 * The product path (the HIP library and its Python binding) never calls it.
 * It shares no source, header, table or helper with the HIP path.
 *
 * What it computes, and where the pages state it ("c_plan.cuh" = the page
 * sglang/jit_kernel/csrc/deepseek_v4/c_plan.cuh, "c4.cuh" = the page
 * .../deepseek_v4/c4.cuh, "compressor_v2.py" = the page
 * sglang/srt/layers/attention/dsv4/compressor_v2.py):
 *
 *   plan prefill  - c_plan.cuh, plan_compress_prefill_legacy (host loop over
 *                   requests and positions) followed by
 *                   plan_compress_prefill_legacy_kernel (per-request ring /
 *                   page translation).  Records are emitted in loop order:
 *                   request-major, position ascending.
 *   plan decode   - c_plan.cuh, plan_compress_decode_legacy_kernel.
 *   compress      - c4.cuh, c4_forward (8-entry window, overlap halves,
 *                   first-block mask) and compressor_v2.py,
 *                   _compress_forward_c128_fallback (softmax over the 128
 *                   window entries of score + ape, weighted sum of kv).
 *                   Entries that precede the chunk come from the state buffer
 *                   as it was BEFORE this chunk's write; the rest come from
 *                   the ragged input (c4.cuh, flash_c4_prefill launches the
 *                   compress kernel before the write kernel).
 *   write         - c4.cuh, c4_write / flash_c4_prefill<kWrite=true>, and
 *                   compressor_v2.py, _c128_compress_prefill_write_kernel:
 *                   a whole input row copied into one state row.
 *   decode        - c4.cuh, flash_c4_decode and compressor_v2.py,
 *                   _c128_compress_decode_kernel: write the new token, then
 *                   pool the window if the new length is a multiple of the
 *                   ratio, else emit a zero row.
 *   store         - compressor_v2.py, compress_norm_rope_store and the steps
 *                   of _forward_unified_hip after the pool: RMSNorm, rotary
 *                   embedding at seq_len - ratio, store at out_loc (the
 *                   readings are listed beside oracle_store_prefill).
 *
 * All pooling arithmetic is float64: a two-pass softmax (max, then the sums
 * of exp(t - max) and exp(t - max) * kv).  bf16 and fp32 inputs are widened
 * exactly to double.  Record layouts (little endian, written byte by byte):
 *   C record 16 B: u32 seq_len | u32 ragged_id (bits 0..23) + buffer_len
 *                  (bits 24..31) | i32 read_page_0 | i32 read_page_1
 *   W record  8 B: u32 ragged_id | i32 write_loc
 *   D record 16 B: u32 seq_len | i32 write_loc | i32 read_page_0 | i32 read_page_1
 *   invalid record: every byte 0xFF.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* device-data error bits, as the library documents them */
#define ERR_EXTEND 1   /* some extend_len <= 0 or > seq_len (decode: seq_len <= 0) */
#define ERR_NUMQ 2     /* sum of extend_len != num_q */
#define ERR_INDEX 4    /* some state_index outside [0, num_state_rows / window) */
#define ERR_CAPACITY 8 /* more C or W records than cap_c / cap_w */
#define ERR_RECORD 16  /* a consumer met a record pointing outside its buffers */
#define ERR_DUPLICATE 32 /* two requests of a prefill chunk name the same state slot */

static void put_u32(uint8_t* p, uint32_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)((v >> 8) & 0xFF);
  p[2] = (uint8_t)((v >> 16) & 0xFF);
  p[3] = (uint8_t)((v >> 24) & 0xFF);
}

static uint32_t get_u32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static int32_t get_i32(const uint8_t* p) {
  uint32_t u = get_u32(p);
  int32_t s;
  memcpy(&s, &u, 4);
  return s;
}

static uint32_t as_u32(int32_t v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  return u;
}

/* window length: 8 for ratio 4 (two overlapping blocks), 128 for ratio 128 */
static int window_of(int cr) { return cr == 4 ? 8 : 128; }

/* Per-request state page of a position (c_plan.cuh, legacy_compute_page):
 * ratio 4 owns two pages of 4 slots per request and alternates between them
 * block by block; ratio 128 owns one page of 128 slots. */
static int64_t page_of(int cr, int64_t idx, int64_t pos) {
  if (cr == 4) return idx * 2 + ((pos / 4) & 1);
  return idx;
}

/* state row of a position (c_plan.cuh, legacy_compute_loc) */
static int64_t loc_of(int cr, int64_t idx, int64_t pos) { return page_of(cr, idx, pos) * cr + pos % cr; }

static double widen(const void* base, int is_bf16, int64_t row, int64_t row_len, int64_t col) {
  if (is_bf16) {
    uint16_t h = ((const uint16_t*)base)[row * row_len + col];
    uint32_t bits = (uint32_t)h << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
  }
  return (double)((const float*)base)[row * row_len + col];
}

/* Whether two requests of a chunk name the same in-range slot (request ring
 * or page, request-pool row, or caller page): both would write the same
 * state rows.  The pages leave distinct slots unstated; a chunk that breaks
 * it is refused as a whole.  Out-of-range slots are ERR_INDEX already and
 * are not compared. */
static int has_duplicate(const int32_t* idx, int B, int64_t limit) {
  for (int b = 0; b < B; ++b) {
    if (idx[b] < 0 || idx[b] >= limit) continue;
    for (int c = b + 1; c < B; ++c)
      if (idx[c] == idx[b]) return 1;
  }
  return 0;
}

static int bad_host_args(int cr, int B) {
  if (cr != 4 && cr != 128) return 1;
  if (B < 1 || B > 1024) return 1;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* plan prefill                                                              */
/* ------------------------------------------------------------------------ */

int oracle_plan_prefill(int cr, int B, int num_q, const int32_t* seq_lens, const int32_t* extend_lens,
                        const int32_t* state_index, int64_t num_state_rows, uint8_t* plan_c, int cap_c,
                        uint8_t* plan_w, int cap_w, int32_t* counts) {
  if (bad_host_args(cr, B)) return -1;
  if (num_q < B || num_q >= (1 << 24)) return -1;
  if (cap_c < 0 || cap_w < 0 || num_state_rows < 0 || num_state_rows > INT32_MAX) return -1;
  if (!seq_lens || !extend_lens || !state_index || !counts) return -1;
  if ((cap_c > 0 && !plan_c) || (cap_w > 0 && !plan_w)) return -1;

  const int W = window_of(cr);
  int err = 0;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t s = seq_lens[b], e = extend_lens[b], idx = state_index[b];
    if (e <= 0 || e > s) err |= ERR_EXTEND;
    total += e;
    if (idx < 0 || idx >= num_state_rows / W) err |= ERR_INDEX;
  }
  if (total != num_q) err |= ERR_NUMQ;
  if (has_duplicate(state_index, B, num_state_rows / W)) err |= ERR_DUPLICATE;

  int num_c = 0, num_w = 0;
  uint8_t* tmp_c = NULL;
  uint8_t* tmp_w = NULL;
  if (!(err & (ERR_EXTEND | ERR_NUMQ))) {
    tmp_c = (uint8_t*)malloc((size_t)num_q * 16);
    tmp_w = (uint8_t*)malloc((size_t)num_q * 8);
    int64_t ragged_base = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t s = seq_lens[b], e = extend_lens[b], idx = state_index[b];
      const int64_t p0 = s - e;
      /* last block boundary at or before s; ratio 4 also keeps the block
       * before it, which the next window overlaps */
      const int64_t last_c = (s / cr) * cr;
      const int64_t first_w = last_c - (cr == 4 ? 4 : 0);
      for (int64_t j = 0; j < e; ++j) {
        const int64_t pos = p0 + j;
        const int64_t ragged = ragged_base + j;
        if ((pos + 1) % cr == 0) {
          const int64_t in_chunk = (j + 1 < W) ? j + 1 : W;
          const int64_t blen = W - in_chunk; /* window entries taken from the state */
          const int64_t pos0 = (pos - cr > 0) ? pos - cr : 0;
          uint8_t* r = tmp_c + (size_t)num_c * 16;
          put_u32(r + 0, (uint32_t)(pos + 1));
          put_u32(r + 4, (uint32_t)ragged | ((uint32_t)blen << 24));
          put_u32(r + 8, as_u32((int32_t)page_of(cr, idx, pos0)));
          put_u32(r + 12, as_u32((int32_t)page_of(cr, idx, pos)));
          ++num_c;
        }
        if (pos >= first_w) {
          uint8_t* r = tmp_w + (size_t)num_w * 8;
          put_u32(r + 0, (uint32_t)ragged);
          put_u32(r + 4, as_u32((int32_t)loc_of(cr, idx, pos)));
          ++num_w;
        }
      }
      ragged_base += e;
    }
    if (num_c > cap_c || num_w > cap_w) err |= ERR_CAPACITY;
  }

  if (err) {
    num_c = 0;
    num_w = 0;
  } else {
    memcpy(plan_c, tmp_c, (size_t)num_c * 16);
    memcpy(plan_w, tmp_w, (size_t)num_w * 8);
  }
  if (cap_c > num_c) memset(plan_c + (size_t)num_c * 16, 0xFF, (size_t)(cap_c - num_c) * 16);
  if (cap_w > num_w) memset(plan_w + (size_t)num_w * 8, 0xFF, (size_t)(cap_w - num_w) * 8);
  counts[0] = num_c;
  counts[1] = num_w;
  counts[2] = err;
  counts[3] = 0;
  free(tmp_c);
  free(tmp_w);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* plan decode                                                               */
/* ------------------------------------------------------------------------ */

/* Requests are independent in decode: a request with a bad length or index
 * gets an invalid record, the others are planned as usual.  The error bits of
 * the whole batch are OR-ed into status[0]. */
int oracle_plan_decode(int cr, int B, const int32_t* seq_lens, const int32_t* state_index, int64_t num_state_rows,
                       uint8_t* plan_d, int32_t* status) {
  if (cr != 4 && cr != 128) return -1;
  if (B < 1 || B > 65536) return -1;
  if (num_state_rows < 0 || num_state_rows > INT32_MAX) return -1;
  if (!seq_lens || !state_index || !plan_d) return -1;
  const int W = window_of(cr);
  int err = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t s = seq_lens[b], idx = state_index[b];
    uint8_t* r = plan_d + (size_t)b * 16;
    int bad = 0;
    if (s <= 0) bad |= ERR_EXTEND;
    if (idx < 0 || idx >= num_state_rows / W) bad |= ERR_INDEX;
    err |= bad;
    if (bad) {
      memset(r, 0xFF, 16);
      continue;
    }
    const int64_t pos1 = s - 1; /* the new token */
    const int64_t pos0 = (pos1 - cr > 0) ? pos1 - cr : 0;
    put_u32(r + 0, (uint32_t)s);
    put_u32(r + 4, as_u32((int32_t)loc_of(cr, idx, pos1)));
    put_u32(r + 8, as_u32((int32_t)page_of(cr, idx, pos0)));
    put_u32(r + 12, as_u32((int32_t)page_of(cr, idx, pos1)));
  }
  if (status) status[0] = err;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* pooling                                                                   */
/* ------------------------------------------------------------------------ */

/* Softmax over the n kept entries of t[], applied to v[] (two passes).
 * Returns sum_i exp(t_i - m) v_i / sum_i exp(t_i - m), m = max_i t_i. */
static double softmax_pool(const double* t, const double* v, int n) {
  double m = t[0];
  for (int i = 1; i < n; ++i)
    if (t[i] > m) m = t[i];
  double num = 0.0, den = 0.0;
  for (int i = 0; i < n; ++i) {
    const double w = exp(t[i] - m);
    num += w * v[i];
    den += w;
  }
  return num / den;
}

/* Where window entry i of a compressed row comes from, and which columns of
 * that row hold its kv and score.  For ratio 4 the row is laid out as
 * |kv overlap|kv|score overlap|score| (c4.cuh, Compress4PrefillParams);
 * entries 0..3 (the previous block) read the overlap halves, entries 4..7
 * (the block being closed) the others.  For ratio 128 the row is |kv|score|. */
typedef struct {
  int from_state; /* 1: state buffer row; 0: ragged input row */
  int64_t row;
  int64_t kv_col;
  int64_t sc_col;
} entry_src;

static entry_src c4_entry(int i, int64_t blen, int64_t ragged, int64_t rp0, int64_t rp1, int64_t hd) {
  entry_src e;
  if (i < blen) {
    e.from_state = 1;
    e.row = (i < 4) ? rp0 * 4 + i : rp1 * 4 + (i - 4);
  } else {
    e.from_state = 0;
    e.row = ragged - 7 + i;
  }
  e.kv_col = (i < 4) ? 0 : hd;
  e.sc_col = (i < 4) ? 2 * hd : 3 * hd;
  return e;
}

static entry_src c128_entry(int i, int64_t blen, int64_t ragged, int64_t rp0, int64_t hd) {
  entry_src e;
  if (i < blen) {
    e.from_state = 1;
    e.row = rp0 * 128 + i;
  } else {
    e.from_state = 0;
    e.row = ragged - 127 + i;
  }
  e.kv_col = 0;
  e.sc_col = hd;
  return e;
}

/* Pool one compressed row (all hd channels) from entries described by src[].
 * For ratio 4, seq_len == 4 is block 0: entries 0..3 lie before the sequence
 * and are dropped (c4.cuh, c4_forward sets their kv to 0 and score to -1e9,
 * whose weight underflows to exactly zero). */
static void pool_row(int cr, int is_bf16, int64_t hd, const entry_src* src, int64_t seq_len, const void* state,
                     const void* input, const void* ape, double* out) {
  const int W = window_of(cr);
  const int64_t R = (cr == 4 ? 4 : 2) * hd;
  double* t = (double*)malloc(sizeof(double) * (size_t)W);
  double* v = (double*)malloc(sizeof(double) * (size_t)W);
  const int first = (cr == 4 && seq_len == 4) ? 4 : 0;
  for (int64_t d = 0; d < hd; ++d) {
    int n = 0;
    for (int i = first; i < W; ++i) {
      const void* base = src[i].from_state ? state : input;
      const double kv = widen(base, is_bf16, src[i].row, R, src[i].kv_col + d);
      const double sc = widen(base, is_bf16, src[i].row, R, src[i].sc_col + d);
      t[n] = sc + widen(ape, is_bf16, i, hd, d);
      v[n] = kv;
      ++n;
    }
    out[d] = softmax_pool(t, v, n);
  }
  free(t);
  free(v);
}

/* Compress every C record in [0, num_c).  Invalid records are skipped (their
 * output rows untouched).  A record that points outside the input or the
 * state is skipped too and reported with ERR_RECORD.  Returns the error bits. */
int oracle_compress(int cr, int is_bf16, int hd, const void* state, int64_t num_state_rows, const void* input,
                    int num_q, const void* ape, const uint8_t* plan_c, int num_c, double* out) {
  const int W = window_of(cr);
  int err = 0;
  entry_src* src = (entry_src*)malloc(sizeof(entry_src) * (size_t)W);
  for (int k = 0; k < num_c; ++k) {
    const uint8_t* r = plan_c + (size_t)k * 16;
    const uint32_t seq_len = get_u32(r);
    if (seq_len == 0xFFFFFFFFu) continue;
    const uint32_t rb = get_u32(r + 4);
    const int64_t ragged = rb & 0xFFFFFF;
    const int64_t blen = rb >> 24;
    const int64_t rp0 = get_i32(r + 8), rp1 = get_i32(r + 12);
    const int first = (cr == 4 && seq_len == 4) ? 4 : 0;
    int ok = 1;
    for (int i = 0; i < W; ++i) {
      src[i] = (cr == 4) ? c4_entry(i, blen, ragged, rp0, rp1, hd) : c128_entry(i, blen, ragged, rp0, hd);
      if (i < first) continue;
      const int64_t lim = src[i].from_state ? num_state_rows : num_q;
      if (src[i].row < 0 || src[i].row >= lim) ok = 0;
    }
    if (!ok) {
      err |= ERR_RECORD;
      continue;
    }
    pool_row(cr, is_bf16, hd, src, seq_len, state, input, ape, out + (size_t)k * hd);
  }
  free(src);
  return err;
}

/* Copy input row ragged_id into state row write_loc for every W record in
 * [0, num_w).  Returns the error bits. */
int oracle_write(int cr, int is_bf16, int hd, void* state, int64_t num_state_rows, const void* input, int num_q,
                 const uint8_t* plan_w, int num_w) {
  const int64_t R = (cr == 4 ? 4 : 2) * (int64_t)hd;
  const int64_t esz = is_bf16 ? 2 : 4;
  int err = 0;
  for (int k = 0; k < num_w; ++k) {
    const uint8_t* r = plan_w + (size_t)k * 8;
    const uint32_t ragged = get_u32(r);
    if (ragged == 0xFFFFFFFFu) continue;
    const int64_t loc = get_i32(r + 4);
    if ((int64_t)ragged >= num_q || loc < 0 || loc >= num_state_rows) {
      err |= ERR_RECORD;
      continue;
    }
    memcpy((uint8_t*)state + (size_t)(loc * R * esz), (const uint8_t*)input + (size_t)((int64_t)ragged * R * esz),
           (size_t)(R * esz));
  }
  return err;
}

/* Decode: for every request b, write input row b into the state, then pool
 * the window if seq_len is a multiple of the ratio (reading the state after
 * the write), else emit a zero row.  Invalid records emit a zero row and
 * leave the state alone.  Returns the error bits. */
int oracle_decode(int cr, int is_bf16, int hd, void* state, int64_t num_state_rows, const void* input,
                  const void* ape, const uint8_t* plan_d, int B, double* out) {
  const int W = window_of(cr);
  const int64_t R = (cr == 4 ? 4 : 2) * (int64_t)hd;
  const int64_t esz = is_bf16 ? 2 : 4;
  int err = 0;
  entry_src* src = (entry_src*)malloc(sizeof(entry_src) * (size_t)W);
  for (int b = 0; b < B; ++b) {
    const uint8_t* r = plan_d + (size_t)b * 16;
    double* o = out + (size_t)b * hd;
    const uint32_t seq_len = get_u32(r);
    for (int d = 0; d < hd; ++d) o[d] = 0.0;
    if (seq_len == 0xFFFFFFFFu) continue;
    const int64_t wl = get_i32(r + 4), rp0 = get_i32(r + 8), rp1 = get_i32(r + 12);
    const int boundary = (seq_len % (uint32_t)cr) == 0;
    int ok = (wl >= 0 && wl < num_state_rows);
    if (boundary) {
      for (int i = 0; i < W; ++i) {
        /* every window entry is in the state once the token is written */
        src[i] = (cr == 4) ? c4_entry(i, W, 0, rp0, rp1, hd) : c128_entry(i, W, 0, rp0, hd);
        if (cr == 4 && seq_len == 4 && i < 4) continue;
        if (src[i].row < 0 || src[i].row >= num_state_rows) ok = 0;
      }
    }
    if (!ok) {
      err |= ERR_RECORD;
      continue;
    }
    memcpy((uint8_t*)state + (size_t)(wl * R * esz), (const uint8_t*)input + (size_t)((int64_t)b * R * esz),
           (size_t)(R * esz));
    if (boundary) pool_row(cr, is_bf16, hd, src, seq_len, state, input, ape, o);
  }
  free(src);
  return err;
}

/* ------------------------------------------------------------------------ */
/* SWA-paged state mapping                                                   */
/* ------------------------------------------------------------------------ */
/*
 * c_plan.cuh: plan_compress_prefill_kernel0 (records on the device),
 * plan_compress_prefill_kernel_1 (translation) and plan_compress_decode_kernel.
 * The state of ratio 4 is paged with the sliding-window (SWA) pool: a token's
 * full-cache slot req_to_token[rid][pos] maps to an SWA slot full_to_swa[...];
 * SWA page swa / swa_page_size owns a ring of ring_size state rows and the
 * token lives at row (swa / swa_page_size) * ring_size + swa % ring_size.
 * Ratio 128 keeps its request-scoped ring: row rid * ring_size + pos % ring_size
 * (ring_size must be 128: the consumer pools page read_page_0).  A ratio-4 ring
 * is a multiple of 8 rows, so the two 4-row pages of a window never coincide.
 * The write rule adds, for ratio 4, the last `ratio` slots of every SWA page
 * (the next page's first window overlaps them), and caps the first written
 * position at seq_len - mtp_pad, mtp_pad = min(ring_size - ratio, 4).
 * A C record whose window takes nothing from the state (buffer_len == 0) keeps
 * read_page_0 = -1 and read_page_1 = its request's batch index, untranslated.
 * A lookup that leaves its table makes that one record invalid and sets
 * ERR_INDEX in *status (OR-ed; the caller clears it).
 */

static int64_t swa_row(int cr, int64_t rid, int64_t pos, const int32_t* r2t, int64_t stride, const int32_t* f2s,
                       int64_t num_full, int sps, int ring, int64_t num_state_rows) {
  int64_t row;
  if (cr == 128) {
    row = rid * ring + pos % ring;
  } else {
    const int64_t full = r2t[rid * stride + pos];
    if (full < 0 || full >= num_full) return -1;
    const int64_t swa = f2s[full];
    if (swa < 0) return -1;
    row = (swa / sps) * ring + swa % ring;
  }
  if (row < 0 || row >= num_state_rows) return -1;
  return row;
}

/* The ratio-4 window spans two 4-row pages, which must be distinct rows of the
 * ring: a ring of ratio-4 rows is a multiple of 8.  The ratio-128 ring is one
 * page of 128 rows. */
static int swa_host_args(int cr, int sps, int ring) {
  if (sps <= 0 || ring <= 0 || sps % ring != 0 || ring % cr != 0) return 1;
  if (cr == 4 && ring % 8 != 0) return 1;
  if (cr == 128 && ring != 128) return 1;
  return 0;
}

int oracle_plan_prefill_swa(int cr, int B, int num_q, const int32_t* seq_lens, const int32_t* extend_lens,
                            const int32_t* req_pool_indices, const int32_t* req_to_token, int64_t r2t_stride,
                            int64_t num_reqs, const int32_t* full_to_swa, int64_t num_full, int swa_page_size,
                            int ring_size, int64_t num_state_rows, uint8_t* plan_c, int cap_c, uint8_t* plan_w,
                            int cap_w, int32_t* counts, int32_t* status) {
  if (bad_host_args(cr, B) || swa_host_args(cr, swa_page_size, ring_size)) return -1;
  if (num_q < B || num_q >= (1 << 24)) return -1;
  if (cap_c < 0 || cap_w < 0 || num_state_rows < 0 || num_state_rows > INT32_MAX) return -1;
  if (r2t_stride <= 0 || num_reqs <= 0 || num_full < 0) return -1;
  if (!seq_lens || !extend_lens || !req_pool_indices || !req_to_token || !full_to_swa || !counts) return -1;
  if ((cap_c > 0 && !plan_c) || (cap_w > 0 && !plan_w)) return -1;

  const int W = window_of(cr);
  const int mtp_pad = (ring_size - cr < 4) ? ring_size - cr : 4;
  int err = 0, rec_err = 0;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t s = seq_lens[b], e = extend_lens[b], rid = req_pool_indices[b];
    if (e <= 0 || e > s) err |= ERR_EXTEND;
    total += e;
    if (rid < 0 || rid >= num_reqs || s > r2t_stride) err |= ERR_INDEX;
  }
  if (total != num_q) err |= ERR_NUMQ;
  if (has_duplicate(req_pool_indices, B, num_reqs)) err |= ERR_DUPLICATE;

  int num_c = 0, num_w = 0;
  uint8_t* tmp_c = NULL;
  uint8_t* tmp_w = NULL;
  if (!(err & (ERR_EXTEND | ERR_NUMQ))) {
    tmp_c = (uint8_t*)malloc((size_t)num_q * 16);
    tmp_w = (uint8_t*)malloc((size_t)num_q * 8);
    int64_t ragged_base = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t s = seq_lens[b], e = extend_lens[b], rid = req_pool_indices[b];
      const int64_t p0 = s - e;
      const int64_t last_c = (s / cr) * cr;
      int64_t first_w = last_c - (cr == 4 ? 4 : 0);
      if (s - mtp_pad < first_w) first_w = s - mtp_pad;
      for (int64_t j = 0; j < e; ++j) {
        const int64_t pos = p0 + j;
        const int64_t ragged = ragged_base + j;
        if ((pos + 1) % cr == 0) {
          const int64_t in_chunk = (j + 1 < W) ? j + 1 : W;
          const int64_t blen = W - in_chunk;
          uint8_t* r = tmp_c + (size_t)num_c * 16;
          int64_t rp0 = -1, rp1 = b;
          int ok = 1;
          if (blen > 0 && !(err & ERR_INDEX)) {
            const int64_t pos0 = (pos - cr > 0) ? pos - cr : 0;
            const int64_t row0 = swa_row(cr, rid, pos0, req_to_token, r2t_stride, full_to_swa, num_full,
                                         swa_page_size, ring_size, num_state_rows);
            const int64_t row1 = swa_row(cr, rid, pos, req_to_token, r2t_stride, full_to_swa, num_full,
                                         swa_page_size, ring_size, num_state_rows);
            ok = row0 >= 0 && row1 >= 0;
            rp0 = row0 / cr;
            rp1 = row1 / cr;
          }
          if (ok) {
            put_u32(r + 0, (uint32_t)(pos + 1));
            put_u32(r + 4, (uint32_t)ragged | ((uint32_t)blen << 24));
            put_u32(r + 8, as_u32((int32_t)rp0));
            put_u32(r + 12, as_u32((int32_t)rp1));
          } else {
            memset(r, 0xFF, 16);
            rec_err |= ERR_INDEX;
          }
          ++num_c;
        }
        const int page_tail = (cr == 4) && (pos % swa_page_size >= swa_page_size - cr);
        if (pos >= first_w || page_tail) {
          uint8_t* r = tmp_w + (size_t)num_w * 8;
          const int64_t row = (err & ERR_INDEX) ? -1
                                                : swa_row(cr, rid, pos, req_to_token, r2t_stride, full_to_swa,
                                                          num_full, swa_page_size, ring_size, num_state_rows);
          if (row >= 0) {
            put_u32(r + 0, (uint32_t)ragged);
            put_u32(r + 4, as_u32((int32_t)row));
          } else {
            memset(r, 0xFF, 8);
            rec_err |= ERR_INDEX;
          }
          ++num_w;
        }
      }
      ragged_base += e;
    }
    if (num_c > cap_c || num_w > cap_w) err |= ERR_CAPACITY;
  }
  if (err) {
    num_c = 0;
    num_w = 0;
  } else {
    memcpy(plan_c, tmp_c, (size_t)num_c * 16);
    memcpy(plan_w, tmp_w, (size_t)num_w * 8);
    if (status) status[0] |= rec_err;
  }
  if (cap_c > num_c) memset(plan_c + (size_t)num_c * 16, 0xFF, (size_t)(cap_c - num_c) * 16);
  if (cap_w > num_w) memset(plan_w + (size_t)num_w * 8, 0xFF, (size_t)(cap_w - num_w) * 8);
  counts[0] = num_c;
  counts[1] = num_w;
  counts[2] = err;
  counts[3] = 0;
  free(tmp_c);
  free(tmp_w);
  return 0;
}

int oracle_plan_decode_swa(int cr, int B, const int32_t* seq_lens, const int32_t* req_pool_indices,
                           const int32_t* req_to_token, int64_t r2t_stride, int64_t num_reqs,
                           const int32_t* full_to_swa, int64_t num_full, int swa_page_size, int ring_size,
                           int64_t num_state_rows, uint8_t* plan_d, int32_t* status) {
  if (cr != 4 && cr != 128) return -1;
  if (B < 1 || B > 65536 || swa_host_args(cr, swa_page_size, ring_size)) return -1;
  if (num_state_rows < 0 || num_state_rows > INT32_MAX || r2t_stride <= 0 || num_reqs <= 0 || num_full < 0) return -1;
  if (!seq_lens || !req_pool_indices || !req_to_token || !full_to_swa || !plan_d) return -1;
  int err = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t s = seq_lens[b], rid = req_pool_indices[b];
    uint8_t* r = plan_d + (size_t)b * 16;
    int bad = 0;
    if (s <= 0) bad |= ERR_EXTEND;
    if (rid < 0 || rid >= num_reqs || s > r2t_stride) bad |= ERR_INDEX;
    int64_t row0 = -1, row1 = -1;
    if (!bad) {
      const int64_t pos1 = s - 1;
      const int64_t pos0 = (pos1 - cr > 0) ? pos1 - cr : 0;
      row0 = swa_row(cr, rid, pos0, req_to_token, r2t_stride, full_to_swa, num_full, swa_page_size, ring_size,
                     num_state_rows);
      row1 = swa_row(cr, rid, pos1, req_to_token, r2t_stride, full_to_swa, num_full, swa_page_size, ring_size,
                     num_state_rows);
      if (row0 < 0 || row1 < 0) bad |= ERR_INDEX;
    }
    err |= bad;
    if (bad) {
      memset(r, 0xFF, 16);
      continue;
    }
    put_u32(r + 0, (uint32_t)s);
    put_u32(r + 4, as_u32((int32_t)row1));
    put_u32(r + 8, as_u32((int32_t)(row0 / cr)));
    put_u32(r + 12, as_u32((int32_t)(row1 / cr)));
  }
  if (status) status[0] = err;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* norm + rotary embedding + store of the compressed rows                    */
/* ------------------------------------------------------------------------ */
/*
 * compressor_v2.py, _forward_unified_hip (steps 2 and 4) and
 * compress_norm_rope_store: every compressed row goes through an RMSNorm over
 * its head_dim channels, then a rotary embedding at the position of the
 * compressed token, seq_len - ratio (_extract_positions_from_plan, clamped at
 * 0), and is stored into the compressed cache row out_loc[...].  Readings
 * taken here:
 *   - RMSNorm: y_d = x_d / sqrt(mean_e x_e^2 + eps) * w_d.
 *   - the rotated channels are the last rope_dim of the row (the stored pack
 *     puts the un-rotated part first and the rotated part after it); channel
 *     pairs (2k, 2k+1) of that slice are one complex number, multiplied by
 *     freqs_cis[pos][k] = (cos, sin).
 *   - the cache holds bf16 rows; this oracle returns the exact value (double),
 *     the caller compares against the rounded bf16 store.
 *   - prefill: one stored row per valid C record, at out_loc[ragged_id];
 *     decode: one per valid D record whose seq_len closes a block, at
 *     out_loc[b]; rows of other requests are not stored.
 */
static void norm_rope_row(int64_t hd, int64_t rope_dim, const float* x, const float* w, double eps,
                          const float* cis, double* y) {
  double ss = 0.0;
  for (int64_t d = 0; d < hd; ++d) ss += (double)x[d] * (double)x[d];
  const double inv = 1.0 / sqrt(ss / (double)hd + eps);
  for (int64_t d = 0; d < hd; ++d) y[d] = (double)x[d] * inv * (double)w[d];
  const int64_t base = hd - rope_dim;
  for (int64_t k = 0; k < rope_dim / 2; ++k) {
    const double re = y[base + 2 * k], im = y[base + 2 * k + 1];
    const double c = cis[2 * k], s = cis[2 * k + 1];
    y[base + 2 * k] = re * c - im * s;
    y[base + 2 * k + 1] = re * s + im * c;
  }
}

/* One record's store: row k of x at the position of seq_len into cache row
 * out_loc[key].  Returns the error bits (nothing stored on error). */
static int store_one(int cr, int64_t hd, int64_t rope_dim, const float* x, uint32_t seq_len, int64_t key,
                     const float* w, double eps, const float* freqs, int64_t max_pos, const int32_t* out_loc,
                     int64_t num_loc, double* cache, int64_t num_cache_rows) {
  int64_t pos = (int64_t)seq_len - cr;
  if (pos < 0) pos = 0;
  if (key < 0 || key >= num_loc) return ERR_RECORD;
  const int64_t loc = out_loc[key];
  if (loc < 0 || loc >= num_cache_rows) return ERR_RECORD;
  if (rope_dim > 0 && pos >= max_pos) return ERR_RECORD;
  norm_rope_row(hd, rope_dim, x, w, eps, rope_dim > 0 ? freqs + pos * rope_dim : NULL, cache + loc * hd);
  return 0;
}

int oracle_store_prefill(int cr, int hd, int rope_dim, const float* x, const uint8_t* plan_c, int num_c,
                         const float* w, double eps, const float* freqs, int64_t max_pos, const int32_t* out_loc,
                         int64_t num_loc, double* cache, int64_t num_cache_rows) {
  int err = 0;
  for (int k = 0; k < num_c; ++k) {
    const uint8_t* r = plan_c + (size_t)k * 16;
    const uint32_t seq_len = get_u32(r);
    if (seq_len == 0xFFFFFFFFu) continue;
    const int64_t ragged = get_u32(r + 4) & 0xFFFFFF;
    err |= store_one(cr, hd, rope_dim, x + (size_t)k * hd, seq_len, ragged, w, eps, freqs, max_pos, out_loc, num_loc,
                     cache, num_cache_rows);
  }
  return err;
}

int oracle_store_decode(int cr, int hd, int rope_dim, const float* x, const uint8_t* plan_d, int B, const float* w,
                        double eps, const float* freqs, int64_t max_pos, const int32_t* out_loc, int64_t num_loc,
                        double* cache, int64_t num_cache_rows) {
  int err = 0;
  for (int b = 0; b < B; ++b) {
    const uint32_t seq_len = get_u32(plan_d + (size_t)b * 16);
    if (seq_len == 0xFFFFFFFFu || seq_len % (uint32_t)cr != 0) continue;
    err |= store_one(cr, hd, rope_dim, x + (size_t)b * hd, seq_len, b, w, eps, freqs, max_pos, out_loc, num_loc,
                     cache, num_cache_rows);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* online ratio-128 state                                                    */
/* ------------------------------------------------------------------------ */
/*
 * compressor_v2.py, _use_online_compress and _forward_unified: with the
 * online path the ratio-128 state of a request is one slot of 3 * head_dim
 * values (the kv_score_buffer viewed as [slots, 1, 3 * head_dim]) instead of
 * a 128-row page.  Reading taken here: the slot holds, per channel, the
 * running maximum m, the running sum l = sum exp(t - m) and the running
 * weighted sum acc = sum exp(t - m) kv over the positions of the current
 * (unfinished) block, t = score + ape[pos % 128]; a block's compressed row is
 * acc / l once its 128th position is folded in.  Slots here are float64
 * [slots][3][hd] (m, l, acc).  The usual ratio-128 plans drive it: a C record
 * with buffer_len > 0 starts from the slot's partial (the entries before the
 * chunk); the W records of a request (its tail positions) are folded into the
 * slot; a decode record folds one token.
 */
static void fold(double* m, double* l, double* acc, int fresh, double t, double kv) {
  if (fresh) {
    *m = t;
    *l = 1.0;
    *acc = kv;
    return;
  }
  const double nm = t > *m ? t : *m;
  const double a = exp(*m - nm), b = exp(t - nm);
  *l = *l * a + b;
  *acc = *acc * a + kv * b;
  *m = nm;
}

/* Pool every valid C record of a ratio-128 plan with the online state.
 * Entries [0, blen) are the slot's partial (slot = read_page_0); entries
 * [blen, 128) are input rows ragged - 127 + i.  out[k] = acc / l.
 * A planner never emits buffer_len above 127 (the row's own token is always
 * in the chunk), so a larger one marks a malformed record: skipped, with
 * ERR_RECORD. */
int oracle_compress_online(int is_bf16, int hd, const double* state, int64_t num_slots, const void* input, int num_q,
                           const void* ape, const uint8_t* plan_c, int num_c, double* out) {
  const int64_t R = 2 * (int64_t)hd;
  int err = 0;
  for (int k = 0; k < num_c; ++k) {
    const uint8_t* r = plan_c + (size_t)k * 16;
    if (get_u32(r) == 0xFFFFFFFFu) continue;
    const uint32_t rb = get_u32(r + 4);
    const int64_t ragged = rb & 0xFFFFFF, blen = rb >> 24, slot = get_i32(r + 8);
    if (blen > 127 || (blen > 0 && (slot < 0 || slot >= num_slots)) || ragged - 127 + blen < 0 ||
        ragged >= num_q) {
      err |= ERR_RECORD;
      continue;
    }
    for (int64_t d = 0; d < hd; ++d) {
      double m = 0, l = 0, acc = 0;
      int fresh = 1;
      if (blen > 0) {
        const double* s = state + slot * 3 * hd;
        m = s[d];
        l = s[hd + d];
        acc = s[2 * hd + d];
        fresh = 0;
      }
      for (int64_t i = blen; i < 128; ++i) {
        const int64_t row = ragged - 127 + i;
        const double t = widen(input, is_bf16, row, R, hd + d) + widen(ape, is_bf16, i, hd, d);
        fold(&m, &l, &acc, fresh, t, widen(input, is_bf16, row, R, d));
        fresh = 0;
      }
      out[(size_t)k * hd + d] = acc / l;
    }
  }
  return err;
}

/* Fold each request's W records (its positions after the chunk's last
 * completed block, consecutive records with the same slot = write_loc / 128)
 * into its slot.  The run starts a fresh block when its first position is a
 * multiple of 128 (write_loc % 128 == 0), else it continues the slot. */
int oracle_write_online(int is_bf16, int hd, double* state, int64_t num_slots, const void* input, int num_q,
                        const void* ape, const uint8_t* plan_w, int num_w) {
  const int64_t R = 2 * (int64_t)hd;
  int err = 0;
  int k = 0;
  while (k < num_w) {
    const uint8_t* r = plan_w + (size_t)k * 8;
    const uint32_t ragged = get_u32(r);
    const int64_t loc = get_i32(r + 4);
    if (ragged == 0xFFFFFFFFu) {
      ++k;
      continue;
    }
    const int64_t slot = loc / 128, p0 = loc % 128;
    int n = 1;
    while (k + n < num_w && get_u32(plan_w + (size_t)(k + n) * 8) != 0xFFFFFFFFu &&
           get_i32(plan_w + (size_t)(k + n) * 8 + 4) / 128 == slot)
      ++n;
    if (loc < 0 || slot >= num_slots || (int64_t)ragged + n > num_q || p0 + n > 128) {
      err |= ERR_RECORD;
      k += n;
      continue;
    }
    double* s = state + slot * 3 * hd;
    for (int64_t d = 0; d < hd; ++d) {
      double m = s[d], l = s[hd + d], acc = s[2 * hd + d];
      int fresh = p0 == 0;
      for (int i = 0; i < n; ++i) {
        const int64_t row = (int64_t)ragged + i;
        const double t = widen(input, is_bf16, row, R, hd + d) + widen(ape, is_bf16, p0 + i, hd, d);
        fold(&m, &l, &acc, fresh, t, widen(input, is_bf16, row, R, d));
        fresh = 0;
      }
      s[d] = m;
      s[hd + d] = l;
      s[2 * hd + d] = acc;
    }
    k += n;
  }
  return err;
}

/* Decode with the online state: fold input row b at position seq_len - 1
 * into slot read_page_0 (fresh when that position is a multiple of 128); if
 * seq_len closes a block, out[b] = acc / l, else a zero row. */
int oracle_decode_online(int is_bf16, int hd, double* state, int64_t num_slots, const void* input, const void* ape,
                         const uint8_t* plan_d, int B, double* out) {
  const int64_t R = 2 * (int64_t)hd;
  int err = 0;
  for (int b = 0; b < B; ++b) {
    const uint8_t* r = plan_d + (size_t)b * 16;
    double* o = out + (size_t)b * hd;
    for (int64_t d = 0; d < hd; ++d) o[d] = 0.0;
    const uint32_t seq_len = get_u32(r);
    if (seq_len == 0xFFFFFFFFu) continue;
    const int64_t slot = get_i32(r + 8), pos = (int64_t)seq_len - 1;
    if (slot < 0 || slot >= num_slots) {
      err |= ERR_RECORD;
      continue;
    }
    double* s = state + slot * 3 * hd;
    for (int64_t d = 0; d < hd; ++d) {
      double m = s[d], l = s[hd + d], acc = s[2 * hd + d];
      const double t = widen(input, is_bf16, b, R, hd + d) + widen(ape, is_bf16, pos % 128, hd, d);
      fold(&m, &l, &acc, pos % 128 == 0, t, widen(input, is_bf16, b, R, d));
      s[d] = m;
      s[hd + d] = l;
      s[2 * hd + d] = acc;
      if (seq_len % 128 == 0) o[d] = acc / l;
    }
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* ratio 4 with caller-allocated 4-row pages (Page4Align)                    */
/* ------------------------------------------------------------------------ */
/*
 * c4.cuh, PageMode::Page4Align with C4IndexBundle (flash_c4_prefill) and the
 * previous page of flash_c4_decode: instead of a ring of two 4-row pages per
 * request, the caller hands over the pages.  Prefill, per request b: its
 * page index[b] (the page of positions >= last_position) and a bundle
 * {load_first_page, load_second_page, write_first_page, last_position}.
 *   - the window entries before the chunk (buffer_len of them) come from
 *     load_second_page alone when buffer_len <= 4 (they all lie in the block
 *     before the closing one), else entries 0..3 from load_first_page and
 *     4.. from load_second_page: read_page_0 / read_page_1 of the record;
 *     a record that reads nothing from the state keeps pages -1, and only
 *     pages that are read are checked (the first block's entries 0..3 are
 *     masked, so a request starting at position 0 needs no earlier page);
 *   - the written positions are those of the ratio-4 rule (the next window's
 *     overlap block and the current block); position p goes to row
 *     (p < last_position ? write_first_page : index[b]) * 4 + p % 4.
 * Decode, per request: page index[b] takes the new token at slot
 * (seq_len - 1) % 4; the window's overlap block is page prev[b].
 * A page outside [0, num_state_rows / 4) that a record needs makes that
 * record invalid and sets ERR_INDEX in *status.
 */
static int page4_ok(int64_t page, int64_t num_state_rows) { return page >= 0 && page < num_state_rows / 4; }

int oracle_plan_prefill_page4(int B, int num_q, const int32_t* seq_lens, const int32_t* extend_lens,
                              const int32_t* page_index, const int32_t* bundle, int64_t num_state_rows,
                              uint8_t* plan_c, int cap_c, uint8_t* plan_w, int cap_w, int32_t* counts,
                              int32_t* status) {
  if (bad_host_args(4, B)) return -1;
  int err = 0, st = 0;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    if (extend_lens[b] < 1 || extend_lens[b] > seq_lens[b]) err |= ERR_EXTEND;
    if (!page4_ok(page_index[b], num_state_rows)) err |= ERR_INDEX;
    total += extend_lens[b];
  }
  if (!(err & ERR_EXTEND) && total != num_q) err |= ERR_NUMQ;
  if (has_duplicate(page_index, B, num_state_rows / 4)) err |= ERR_DUPLICATE;
  int nc = 0, nw = 0;
  if (!err) {
    int64_t ragged_base = 0;
    for (int b = 0; b < B && !err; ++b) {
      const int64_t s = seq_lens[b], e = extend_lens[b], p0 = s - e;
      const int64_t lfp = bundle[4 * b], lsp = bundle[4 * b + 1], wfp = bundle[4 * b + 2], last = bundle[4 * b + 3];
      const int64_t first_w = (s / 4) * 4 - 4;
      for (int64_t j = 0; j < e; ++j) {
        const int64_t pos = p0 + j, ragged = ragged_base + j;
        if ((pos + 1) % 4 == 0) {
          if (nc >= cap_c) {
            err |= ERR_CAPACITY;
            break;
          }
          uint8_t* r = plan_c + (size_t)nc * 16;
          const int64_t in_chunk = (j + 1 < 8) ? j + 1 : 8;
          const int64_t blen = 8 - in_chunk;
          int64_t rp0 = -1, rp1 = -1;
          if (blen > 0) {
            rp0 = blen <= 4 ? lsp : lfp;
            rp1 = lsp;
          }
          /* pages the consumer reads: entries 0..3 unless masked (seq_len 4), entries 4.. when blen > 4 */
          const int needs0 = blen > 0 && pos + 1 != 4, needs1 = blen > 4;
          if ((needs0 && !page4_ok(rp0, num_state_rows)) || (needs1 && !page4_ok(rp1, num_state_rows))) {
            memset(r, 0xFF, 16);
            st |= ERR_INDEX;
          } else {
            put_u32(r, (uint32_t)(pos + 1));
            put_u32(r + 4, (uint32_t)ragged | ((uint32_t)blen << 24));
            put_u32(r + 8, as_u32((int32_t)rp0));
            put_u32(r + 12, as_u32((int32_t)rp1));
          }
          ++nc;
        }
        if (pos >= first_w) {
          if (nw >= cap_w) {
            err |= ERR_CAPACITY;
            break;
          }
          uint8_t* r = plan_w + (size_t)nw * 8;
          const int64_t page = pos < last ? wfp : page_index[b];
          if (!page4_ok(page, num_state_rows)) {
            memset(r, 0xFF, 8);
            st |= ERR_INDEX;
          } else {
            put_u32(r, (uint32_t)ragged);
            put_u32(r + 4, as_u32((int32_t)(page * 4 + pos % 4)));
          }
          ++nw;
        }
      }
      ragged_base += e;
    }
  }
  if (err) {
    nc = nw = 0;
    st = 0;
  }
  memset(plan_c + (size_t)nc * 16, 0xFF, (size_t)(cap_c - nc) * 16);
  memset(plan_w + (size_t)nw * 8, 0xFF, (size_t)(cap_w - nw) * 8);
  counts[0] = nc;
  counts[1] = nw;
  counts[2] = err;
  counts[3] = 0;
  if (status) *status |= st;
  return err;
}

int oracle_plan_decode_page4(int B, const int32_t* seq_lens, const int32_t* page_index, const int32_t* prev_page,
                             int64_t num_state_rows, uint8_t* plan_d, int32_t* status) {
  if (B < 1 || B > 65536) return -1;
  int err = 0;
  for (int b = 0; b < B; ++b) {
    uint8_t* r = plan_d + (size_t)b * 16;
    const int64_t s = seq_lens[b];
    memset(r, 0xFF, 16);
    if (s <= 0) {
      err |= ERR_EXTEND;
      continue;
    }
    const int64_t page = page_index[b], prev = prev_page[b];
    const int needs_prev = (s % 4 == 0) && s > 4; /* the overlap block exists and is read */
    if (!page4_ok(page, num_state_rows) || (needs_prev && !page4_ok(prev, num_state_rows))) {
      err |= ERR_INDEX;
      continue;
    }
    put_u32(r, (uint32_t)s);
    put_u32(r + 4, as_u32((int32_t)(page * 4 + (s - 1) % 4)));
    put_u32(r + 8, as_u32((int32_t)prev));
    put_u32(r + 12, as_u32((int32_t)page));
  }
  if (status) *status = err;
  return err;
}
