// kvc_plan.hip - prefill and decode planners (c_plan.cuh page:
// plan_compress_prefill_kernel0 / plan_compress_prefill_legacy with the
// per-request translation of plan_compress_prefill_legacy_kernel, the
// SWA-paged translation of plan_compress_prefill_kernel_1, and
// plan_compress_decode_legacy_kernel / plan_compress_decode_kernel; and the
// ratio-4 mapping onto caller-allocated 4-row pages of the c4.cuh page,
// PageMode::Page4Align with C4IndexBundle).  The mapping is a template
// parameter: per-request ring or page, SWA pages, or 4-row pages.
//
// Prefill plan, one launch, no host sync, no scratch memory:
//   stage A  every workgroup loads the <= 1024 requests (4 per thread), checks
//            them (two requests on one slot are found with an LDS hash set),
//            and forms per request e, num_c = s/r - p0/r and num_w (the
//            chunk's positions the next window needs; in SWA mode also the
//            last 4 slots of every SWA page, counted in closed form);
//   stage B  64-lane wavefront scans (shuffles) + a 4-wave combine in LDS
//            give exclusive offsets of the ragged rows, C records and W
//            records, plus the sum / OR / min / max reductions;
//   stage C  records are written in host-loop order (request-major,
//            positions ascending), so the result is deterministic:
//              general path  - one thread per output record; the owning
//                              request comes from a binary search of the
//                              offsets in LDS and the position from a
//                              closed form;
//              uniform path  - when every extend is the same E <= 32 (the
//                              multi-token-prediction shape), one thread per
//                              token: request k / E, offset k % E, no search;
//            in SWA mode each record's rows are looked up through
//            req_to_token and full_to_swa as it is written; in page-4 mode
//            they come from the request's page index and bundle;
//   stage D  [num_c, cap_c) and [num_w, cap_w) are filled with 0xFF records.
// Every workgroup repeats stages A/B (12 KiB of L2-resident loads), which is
// cheaper than a second launch and needs no workspace; workgroup 0 writes
// the counts.
#include <algorithm>

#include "kvc_device.hpp"
#include "kvc_launch.hpp"

namespace kvc {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPerThread = KVC_MAX_PREFILL_BATCH / kPlanThreads;  // 4 requests per thread
constexpr int kUniformMaxExtend = 32;

template <int CR>
__device__ __forceinline__ int32_t page_of(int32_t idx, int32_t pos) {
  if constexpr (CR == 4) {
    return idx * 2 + ((pos >> 2) & 1);  // two 4-slot pages per request, alternating per block
  } else {
    return idx;  // one 128-slot page per request
  }
}

template <int CR>
__device__ __forceinline__ int32_t loc_of(int32_t idx, int32_t pos) {
  return page_of<CR>(idx, pos) * CR + (pos & (CR - 1));
}

// State row of position pos of request rid under the SWA-paged mapping, or -1
// when a lookup leaves its table or the row leaves the state buffer.
template <int CR>
__device__ __forceinline__ int64_t swa_row(const SwaTables& t, int64_t rid, int32_t pos, int64_t num_state_rows) {
  int64_t row;
  if constexpr (CR == 128) {
    row = rid * t.ring_size + pos % t.ring_size;  // request-scoped ring
  } else {
    const int64_t full = t.req_to_token[rid * t.stride + pos];
    if (full < 0 || full >= t.num_full) return -1;
    const int64_t swa = t.full_to_swa[full];
    if (swa < 0) return -1;
    row = (swa / t.swa_page_size) * t.ring_size + swa % t.ring_size;  // the SWA page's ring
  }
  return (row >= 0 && row < num_state_rows) ? row : -1;
}

// Ratio-4 SWA page tails: positions p with p % sps >= sps - 4.  Count in [0, x):
__device__ __forceinline__ int64_t tails_before(int64_t x, int sps) {
  const int64_t r = x % sps - (sps - 4);
  return (x / sps) * 4 + (r > 0 ? r : 0);
}
__device__ __forceinline__ int64_t tails_in(int64_t lo, int64_t hi, int sps) {
  return hi > lo ? tails_before(hi, sps) - tails_before(lo, sps) : 0;
}
// the t-th page-tail position at or after lo
__device__ __forceinline__ int32_t tail_pos(int64_t lo, int64_t t, int sps) {
  const int64_t n = tails_before(lo, sps) + t;
  return (int32_t)((n / 4) * sps + sps - 4 + n % 4);
}

// a 4-row page of the state buffer (page-4 mode)
__device__ __forceinline__ bool page4_ok(int32_t page, int64_t num_state_rows) {
  return page >= 0 && (int64_t)page < num_state_rows / 4;
}

// Open-addressing set of the slots of a chunk's requests, in LDS: at most
// KVC_MAX_PREFILL_BATCH keys in twice as many entries, so a probe sequence
// always meets an empty entry.  Two requests with the same slot follow the
// same probe sequence, and entries only go from empty to taken, so exactly
// one of them inserts the key and the other finds it.
constexpr int kDupBits = 11;
constexpr int kDupSlots = 1 << kDupBits;
static_assert(kDupSlots >= 2 * KVC_MAX_PREFILL_BATCH, "load factor of the slot set");

// Insert slot v (>= 0); true when another request had inserted it already.
__device__ __forceinline__ bool slot_seen(int32_t* set, int32_t v) {
  uint32_t h = ((uint32_t)v * 2654435761u) >> (32 - kDupBits);  // multiplicative hash
  for (int probe = 0; probe < kDupSlots; ++probe) {
    const int32_t old = atomicCAS(&set[h], -1, v);
    if (old == -1) return false;
    if (old == v) return true;
    h = (h + 1) & (kDupSlots - 1);
  }
  return false;  // not reached (an empty entry always exists)
}

struct RequestTable {
  int32_t s[KVC_MAX_PREFILL_BATCH];
  int32_t p0[KVC_MAX_PREFILL_BATCH];
  int32_t idx[KVC_MAX_PREFILL_BATCH];
  int32_t roff[KVC_MAX_PREFILL_BATCH];  // first ragged row of the request
  int32_t coff[KVC_MAX_PREFILL_BATCH];  // first C record of the request
  int32_t woff[KVC_MAX_PREFILL_BATCH];  // first W record of the request
};

__device__ __forceinline__ void store_invalid_c(kvc_plan_c* dst) {
  const u32x4 ones = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  store16(dst, ones);
}
__device__ __forceinline__ void store_invalid_w(kvc_plan_w* dst) {
  const uint2 ones = {0xFFFFFFFFu, 0xFFFFFFFFu};
  *reinterpret_cast<uint2*>(dst) = ones;
}

// C record for the compressed row closing at position pos of batch entry b
template <int CR, int MAP>
__device__ __forceinline__ void emit_c(const PlanPrefillArgs& a, kvc_plan_c* dst, int b, int32_t pos, int32_t p0,
                                       int32_t idx, int32_t roff) {
  constexpr int32_t W = CR == 4 ? 8 : 128;
  const int32_t j = pos - p0;                                      // offset inside the chunk
  const uint32_t blen = (j + 1 < W) ? (uint32_t)(W - 1 - j) : 0u;  // window entries before the chunk
  const int32_t pos0 = pos - CR > 0 ? pos - CR : 0;
  u32x4 v;
  v.x = (uint32_t)(pos + 1);
  v.y = (uint32_t)(roff + j) | (blen << 24);
  if constexpr (MAP == kPlanSwa) {
    int64_t rp0 = -1, rp1 = b;  // nothing is read from the state: left untranslated
    if (blen > 0) {
      const int64_t r0 = swa_row<CR>(a.swa, idx, pos0, a.num_state_rows);
      const int64_t r1 = swa_row<CR>(a.swa, idx, pos, a.num_state_rows);
      if (r0 < 0 || r1 < 0) {
        if (a.status) atomicOr(a.status, KVC_DERR_INDEX);
        store_invalid_c(dst);
        return;
      }
      rp0 = r0 / CR;
      rp1 = r1 / CR;
    }
    v.z = (uint32_t)(int32_t)rp0;
    v.w = (uint32_t)(int32_t)rp1;
  } else if constexpr (MAP == kPlanPage4) {
    // the entries before the chunk lie on load_second_page alone when there are at most 4 of
    // them, else entries 0..3 on load_first_page; only pages that are read are checked (the
    // first block's entries 0..3 are masked)
    int32_t rp0 = -1, rp1 = -1;
    if (blen > 0) {
      rp0 = blen <= 4 ? a.bundle[4 * b + 1] : a.bundle[4 * b];
      rp1 = a.bundle[4 * b + 1];
      const bool bad0 = pos + 1 != 4 && !page4_ok(rp0, a.num_state_rows);
      const bool bad1 = blen > 4 && !page4_ok(rp1, a.num_state_rows);
      if (bad0 || bad1) {
        if (a.status) atomicOr(a.status, KVC_DERR_INDEX);
        store_invalid_c(dst);
        return;
      }
    }
    v.z = (uint32_t)rp0;
    v.w = (uint32_t)rp1;
  } else {
    v.z = (uint32_t)page_of<CR>(idx, pos0);
    v.w = (uint32_t)page_of<CR>(idx, pos);
  }
  store16(dst, v);
}

template <int CR, int MAP>
__device__ __forceinline__ void emit_w(const PlanPrefillArgs& a, kvc_plan_w* dst, int b, int32_t pos, int32_t p0,
                                       int32_t idx, int32_t roff) {
  uint2 v;
  v.x = (uint32_t)(roff + (pos - p0));
  if constexpr (MAP == kPlanSwa) {
    const int64_t row = swa_row<CR>(a.swa, idx, pos, a.num_state_rows);
    if (row < 0) {
      if (a.status) atomicOr(a.status, KVC_DERR_INDEX);
      store_invalid_w(dst);
      return;
    }
    v.y = (uint32_t)row;
  } else if constexpr (MAP == kPlanPage4) {
    // positions before last_position go to write_first_page, the rest to the request's page
    const int32_t page = pos < a.bundle[4 * b + 3] ? a.bundle[4 * b + 2] : idx;
    if (!page4_ok(page, a.num_state_rows)) {
      if (a.status) atomicOr(a.status, KVC_DERR_INDEX);
      store_invalid_w(dst);
      return;
    }
    v.y = (uint32_t)(page * 4 + (pos & 3));
  } else {
    v.y = (uint32_t)loc_of<CR>(idx, pos);
  }
  *reinterpret_cast<uint2*>(dst) = v;
}

// largest b in [0, n) with off[b] <= k; off[0] == 0 <= k
__device__ __forceinline__ int find_owner(const int32_t* off, int n, int k) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= k) {
      lo = mid;
    } else {
      hi = mid - 1;
    }
  }
  return lo;
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t n = __shfl_up(v, d, kWave);
    if (lane >= d) v += n;
  }
  return v;
}

// First position written unconditionally: the block the next window overlaps
// (ratio 4) or the current block (ratio 128); in SWA mode also capped at
// s - mtp_pad, mtp_pad = min(ring_size - ratio, 4).
template <int CR, int MAP>
__device__ __forceinline__ int32_t first_write(int32_t s, const SwaTables& t) {
  int32_t fw = (s / CR) * CR - (CR == 4 ? 4 : 0);
  if constexpr (MAP == kPlanSwa) {
    const int32_t pad = min(t.ring_size - CR, 4);
    fw = min(fw, s - pad);
  }
  return fw;
}

template <int CR, int MAP>
__global__ __launch_bounds__(kPlanThreads) void plan_prefill_kernel(PlanPrefillArgs a) {
  constexpr int32_t W = CR == 4 ? 8 : 128;
  constexpr bool kTails = MAP == kPlanSwa && CR == 4;  // ratio-4 SWA pages also keep their last 4 slots
  __shared__ RequestTable T;
  __shared__ uint32_t w_incl[kPlanWaves][3];
  __shared__ long long w_esum[kPlanWaves];
  __shared__ int w_err[kPlanWaves];
  __shared__ uint32_t w_min[kPlanWaves];
  __shared__ uint32_t w_max[kPlanWaves];
  __shared__ int32_t slot_set[kDupSlots];

  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int64_t max_idx = MAP == kPlanSwa ? a.swa.num_reqs : a.num_state_rows / (MAP == kPlanPage4 ? 4 : W);
  const int sps = a.swa.swa_page_size;
  for (int i = t; i < kDupSlots; i += kPlanThreads) slot_set[i] = -1;
  __syncthreads();

  // ---- stage A: this thread's requests t*4 .. t*4+3 ----
  uint32_t ve[kPerThread], vc[kPerThread], vw[kPerThread];
  long long esum = 0;
  int err = 0;
  uint32_t emin = 0xFFFFFFFFu, emax = 0u;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int b = t * kPerThread + k;
    ve[k] = vc[k] = vw[k] = 0u;
    if (b < a.batch) {
      const int32_t s = a.seq_lens[b], e = a.extend_lens[b], idx = a.state_index[b];
      const bool ok = e >= 1 && e <= s;
      if (!ok) err |= KVC_DERR_EXTEND;
      if (idx < 0 || (int64_t)idx >= max_idx) {
        err |= KVC_DERR_INDEX;
      } else if (slot_seen(slot_set, idx)) {
        err |= KVC_DERR_DUPLICATE;  // two requests would write the same state rows
      }
      if (MAP == kPlanSwa && (int64_t)s > a.swa.stride) err |= KVC_DERR_INDEX;
      esum += e;
      const int32_t p0 = ok ? s - e : 0;
      if (ok) {
        const int32_t fw = first_write<CR, MAP>(s, a.swa);
        ve[k] = (uint32_t)e;
        vc[k] = (uint32_t)(s / CR - p0 / CR);
        uint32_t nw = (uint32_t)(s - (p0 > fw ? p0 : fw));
        if constexpr (kTails) nw += (uint32_t)tails_in(p0, min(fw, s), sps);
        vw[k] = nw;
      }
      emin = min(emin, (uint32_t)e);
      emax = max(emax, (uint32_t)e);
      T.s[b] = s;
      T.p0[b] = p0;
      T.idx[b] = idx;
    }
  }

  // ---- stage B: scans and reductions ----
  uint32_t te = 0, tc = 0, tw = 0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    te += ve[k];
    tc += vc[k];
    tw += vw[k];
  }
  const uint32_t ie = wave_inclusive_sum(te, lane);
  const uint32_t ic = wave_inclusive_sum(tc, lane);
  const uint32_t iw = wave_inclusive_sum(tw, lane);
#pragma unroll
  for (int m = kWave / 2; m > 0; m >>= 1) {
    esum += __shfl_xor(esum, m, kWave);
    err |= __shfl_xor(err, m, kWave);
    emin = min(emin, (uint32_t)__shfl_xor(emin, m, kWave));
    emax = max(emax, (uint32_t)__shfl_xor(emax, m, kWave));
  }
  if (lane == kWave - 1) {
    w_incl[wave][0] = ie;
    w_incl[wave][1] = ic;
    w_incl[wave][2] = iw;
  }
  if (lane == 0) {
    w_esum[wave] = esum;
    w_err[wave] = err;
    w_min[wave] = emin;
    w_max[wave] = emax;
  }
  __syncthreads();

  uint32_t oe = 0, oc = 0, ow = 0, tot_c = 0, tot_w = 0;
  long long tot_e = 0;
  int tot_err = 0;
  uint32_t tmin = 0xFFFFFFFFu, tmax = 0u;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    if (w < wave) {
      oe += w_incl[w][0];
      oc += w_incl[w][1];
      ow += w_incl[w][2];
    }
    tot_c += w_incl[w][1];
    tot_w += w_incl[w][2];
    tot_e += w_esum[w];
    tot_err |= w_err[w];
    tmin = min(tmin, w_min[w]);
    tmax = max(tmax, w_max[w]);
  }
  uint32_t xe = oe + ie - te, xc = oc + ic - tc, xw = ow + iw - tw;  // exclusive offsets
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int b = t * kPerThread + k;
    if (b < a.batch) {
      T.roff[b] = (int32_t)xe;
      T.coff[b] = (int32_t)xc;
      T.woff[b] = (int32_t)xw;
    }
    xe += ve[k];
    xc += vc[k];
    xw += vw[k];
  }
  if (tot_e != (long long)a.num_q) tot_err |= KVC_DERR_NUMQ;
  if (!(tot_err & (KVC_DERR_EXTEND | KVC_DERR_NUMQ)) &&
      ((int64_t)tot_c > (int64_t)a.cap_c || (int64_t)tot_w > (int64_t)a.cap_w))
    tot_err |= KVC_DERR_CAPACITY;
  const int n_c = tot_err ? 0 : (int)tot_c;
  const int n_w = tot_err ? 0 : (int)tot_w;
  __syncthreads();

  if (blockIdx.x == 0 && t == 0) {
    a.counts[0] = n_c;
    a.counts[1] = n_w;
    a.counts[2] = tot_err;
    a.counts[3] = 0;
  }

  // ---- stage C: records ----
  const int gtid = blockIdx.x * kPlanThreads + t;
  const int gstride = gridDim.x * kPlanThreads;
  if constexpr (CR == 128 && MAP == kPlanRing) {
    // the run list: request b's W records are positions first .. s - 1 of its page, consecutive
    // input rows from roff + (first - p0); a request without W records, and every request of a
    // plan with an error, gets an all-zero entry
    if (a.runs != nullptr) {
      for (int b = gtid; b < a.batch; b += gstride) {
        const int32_t s = T.s[b], p0 = T.p0[b];
        const int32_t fw = first_write<CR, MAP>(s, a.swa);
        const int32_t first = p0 > fw ? p0 : fw;
        const int32_t n = tot_err ? 0 : s - first;
        int4 v = {0, 0, 0, 0};
        if (n > 0) {
          v.x = T.roff[b] + (first - p0);
          v.y = loc_of<CR>(T.idx[b], first);
          v.z = n;
        }
        *reinterpret_cast<int4*>(a.runs + 4 * (int64_t)b) = v;
      }
    }
  }
  const bool uniform = !tot_err && tmin == tmax && tmax <= (uint32_t)kUniformMaxExtend;
  if (uniform) {
    const int E = (int)tmax;  // num_q == batch * E
    for (int k = gtid; k < a.num_q; k += gstride) {
      const int b = k / E;
      const int32_t j = k - b * E;
      const int32_t s = T.s[b], p0 = T.p0[b], idx = T.idx[b], roff = T.roff[b];
      const int32_t pos = p0 + j;
      if (((pos + 1) & (CR - 1)) == 0)
        emit_c<CR, MAP>(a, a.plan_c + (T.coff[b] + pos / CR - p0 / CR), b, pos, p0, idx, roff);
      const int32_t fw = first_write<CR, MAP>(s, a.swa);
      bool write = pos >= fw;
      if constexpr (kTails) write = write || (pos % sps >= sps - 4);
      if (write) {
        // W records of this request before pos: page tails below fw, then the block from max(p0, fw)
        int64_t before = pos >= fw ? (int64_t)pos - (p0 > fw ? p0 : fw) : 0;
        if constexpr (kTails) before += tails_in(p0, min(pos, fw), sps);
        emit_w<CR, MAP>(a, a.plan_w + (T.woff[b] + before), b, pos, p0, idx, roff);
      }
    }
  } else {
    for (int k = gtid; k < n_c; k += gstride) {
      const int b = find_owner(T.coff, a.batch, k);
      const int32_t p0 = T.p0[b];
      const int32_t pos = (p0 / CR + 1 + (k - T.coff[b])) * CR - 1;  // (k - coff)-th boundary at or after p0
      emit_c<CR, MAP>(a, a.plan_c + k, b, pos, p0, T.idx[b], T.roff[b]);
    }
    for (int k = gtid; k < n_w; k += gstride) {
      const int b = find_owner(T.woff, a.batch, k);
      const int32_t s = T.s[b], p0 = T.p0[b];
      const int32_t fw = first_write<CR, MAP>(s, a.swa);
      const int32_t first = p0 > fw ? p0 : fw;
      int64_t r = k - T.woff[b];
      int32_t pos;
      if constexpr (kTails) {
        const int64_t nt = tails_in(p0, min(fw, s), sps);  // page tails precede the block
        pos = r < nt ? tail_pos(p0, r, sps) : (int32_t)(first + (r - nt));
      } else {
        pos = (int32_t)(first + r);
      }
      emit_w<CR, MAP>(a, a.plan_w + k, b, pos, p0, T.idx[b], T.roff[b]);
    }
  }

  // ---- stage D: invalid padding ----
  for (int k = n_c + gtid; k < a.cap_c; k += gstride) store_invalid_c(a.plan_c + k);
  for (int k = n_w + gtid; k < a.cap_w; k += gstride) store_invalid_w(a.plan_w + k);
}

// Ratio 128's boundary list: the requests whose valid record closes a block,
// as (request, read_page_0) pairs, then their count at [2 * batch].  In the
// record loop a wave with closing requests in a pass takes that many entries
// from a workgroup counter in LDS (one atomic add by its first lane) and its
// closing lanes write theirs in lane order, so the list needs no pass of its
// own; the entries of different waves and passes land in the order the waves
// reach the counter.
constexpr int kDecodePlanThreads = 1024;

// One workgroup; requests are independent, the error word needs the whole batch.
template <int CR, int MAP>
__global__ __launch_bounds__(kDecodePlanThreads) void plan_decode_kernel(PlanDecodeArgs a) {
  constexpr int32_t W = CR == 4 ? 8 : 128;
  __shared__ int s_err;
  __shared__ int s_listed;  // ratio 128 with a boundary list: entries taken so far
  const bool listed = CR == 128 && a.boundaries != nullptr;
  if (threadIdx.x == 0) {
    s_err = 0;
    s_listed = 0;
  }
  __syncthreads();
  const int64_t max_idx = MAP == kPlanSwa ? a.swa.num_reqs : a.num_state_rows / (MAP == kPlanPage4 ? 4 : W);
  int err = 0;
  // one request: its record, its error bits, and whether it joins the boundary list
  auto one = [&](int b, int32_t s, int32_t idx, int32_t prev) {
    int bad = 0;
    if (s <= 0) bad |= KVC_DERR_EXTEND;
    if (idx < 0 || (int64_t)idx >= max_idx) bad |= KVC_DERR_INDEX;
    if (MAP == kPlanSwa && (int64_t)s > a.swa.stride) bad |= KVC_DERR_INDEX;
    u32x4 v = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    if (!bad) {
      const int32_t pos1 = s - 1;  // the new token
      const int32_t pos0 = pos1 - CR > 0 ? pos1 - CR : 0;
      if constexpr (MAP == kPlanSwa) {
        const int64_t r0 = swa_row<CR>(a.swa, idx, pos0, a.num_state_rows);
        const int64_t r1 = swa_row<CR>(a.swa, idx, pos1, a.num_state_rows);
        if (r0 < 0 || r1 < 0) {
          bad |= KVC_DERR_INDEX;
        } else {
          v.x = (uint32_t)s;
          v.y = (uint32_t)r1;
          v.z = (uint32_t)(r0 / CR);
          v.w = (uint32_t)(r1 / CR);
        }
      } else if constexpr (MAP == kPlanPage4) {
        // the new token goes to its block's page; the window's overlap block is the previous page,
        // needed only when the token closes a block past the first
        if ((s & 3) == 0 && s > 4 && !page4_ok(prev, a.num_state_rows)) {
          bad |= KVC_DERR_INDEX;
        } else {
          v.x = (uint32_t)s;
          v.y = (uint32_t)(idx * 4 + (pos1 & 3));
          v.z = (uint32_t)prev;
          v.w = (uint32_t)idx;
        }
      } else {
        v.x = (uint32_t)s;
        v.y = (uint32_t)loc_of<CR>(idx, pos1);
        v.z = (uint32_t)page_of<CR>(idx, pos0);
        v.w = (uint32_t)page_of<CR>(idx, pos1);
      }
    }
    store16(a.plan_d + b, v);
    err |= bad;
    if constexpr (CR == 128) {
      if (listed) {  // uniform; the wave's active lanes ballot (lane 0 is active whenever any is)
        const bool f = !bad && (s & 127) == 0;
        const uint64_t m = __ballot(f);
        if (m != 0) {  // uniform over the wave
          const int lane = threadIdx.x % kWave;
          int base = 0;
          if (lane == 0) base = atomicAdd(&s_listed, __popcll(m));
          base = __builtin_amdgcn_readfirstlane(base);  // lane 0's
          if (f) {
            // the lanes below this one, written out (__lanemask_lt() also masks by the active lanes)
            const int k = base + __popcll(m & ((1ull << lane) - 1ull));
            *reinterpret_cast<int2*>(a.boundaries + 2 * (int64_t)k) = make_int2(b, (int32_t)v.z);
          }
        }
      }
    }
  };
  for (int b = threadIdx.x; b < a.batch; b += kDecodePlanThreads)
    one(b, a.seq_lens[b], a.state_index[b], MAP == kPlanPage4 ? a.prev_page[b] : 0);
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.status) a.status[0] = s_err;
    if (listed) *reinterpret_cast<int2*>(a.boundaries + 2 * (int64_t)a.batch) = make_int2(s_listed, 0);
  }
}

template <int CR, int MAP>
hipError_t prefill_go(const PlanPrefillArgs& a, hipStream_t stream) {
  // enough workgroups that every record (or, on the uniform path, every
  // token) has a thread; the loops are grid-strided, so any count is correct
  const int64_t work = std::max<int64_t>((int64_t)a.cap_c + a.cap_w, std::min(a.num_q, a.batch * kUniformMaxExtend));
  const int grid = (int)std::min<int64_t>(1024, std::max<int64_t>(1, (work + kPlanThreads - 1) / kPlanThreads));
  plan_prefill_kernel<CR, MAP><<<grid, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <int CR, int MAP>
hipError_t decode_go(const PlanDecodeArgs& a, hipStream_t stream) {
  plan_decode_kernel<CR, MAP><<<1, kDecodePlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan_prefill(int compress_ratio, int map, const PlanPrefillArgs& a, hipStream_t stream) {
  if (compress_ratio == 4) {
    if (map == kPlanPage4) return prefill_go<4, kPlanPage4>(a, stream);
    return map == kPlanSwa ? prefill_go<4, kPlanSwa>(a, stream) : prefill_go<4, kPlanRing>(a, stream);
  }
  return map == kPlanSwa ? prefill_go<128, kPlanSwa>(a, stream) : prefill_go<128, kPlanRing>(a, stream);
}

hipError_t launch_plan_decode(int compress_ratio, int map, const PlanDecodeArgs& a, hipStream_t stream) {
  if (compress_ratio == 4) {
    if (map == kPlanPage4) return decode_go<4, kPlanPage4>(a, stream);
    return map == kPlanSwa ? decode_go<4, kPlanSwa>(a, stream) : decode_go<4, kPlanRing>(a, stream);
  }
  return map == kPlanSwa ? decode_go<128, kPlanSwa>(a, stream) : decode_go<128, kPlanRing>(a, stream);
}

}  // namespace kvc
