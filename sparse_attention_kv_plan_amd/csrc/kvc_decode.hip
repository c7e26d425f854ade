// kvc_decode.hip - fused decode step: store the new token, pool on a block
// boundary (c4.cuh page, flash_c4_decode; compressor_v2.py page,
// _c128_compress_decode_kernel).
//
// The window's last entry is the new token itself.  Instead of reading it
// back through the state (a read-after-write across lanes), the pool takes it
// from the input row, which holds the same bits; the other entries are state
// rows that this step does not write (indices are distinct per call).
//  - ratio 4: one lane group (64 lanes for hd 512 bf16) per request; each lane
//    loads its 16-byte slice of the 4 quarters with the record, then on a
//    boundary the 7 state entries, stores the row and pools 8 entries.
//  - ratio 128: copy workgroups move 8 requests' rows each; pool workgroups
//    pool the boundary requests, each over a 64-channel slice of the
//    128-entry page.
//  - ratio 4 with the store step (compressor_v2.py, compress_norm_rope_store):
//    the pooled row is normalised, rotated and stored as bf16 into the
//    compressed cache straight from registers; nothing else is written for it.
#include <algorithm>

#include "kvc_device.hpp"
#include "kvc_launch.hpp"
#include "kvc_pool.hpp"
#include "kvc_store.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;

// Ratio 4: a lane group of HD / V lanes per request (64 at hd 512 bf16).  Two
// dependent rounds of loads: the record and the lane's slice of the new row
// (its four quarters; they depend on nothing) go out together; on a boundary
// the window's state entries 0..6 follow as soon as the record is in, before
// the row is stored (they are other rows of the ring: 0..3 on the block
// before's page, 4..6 on the new token's page below its slot).  Entry 7 is the
// new token, taken from the row already in registers.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void decode_c4_kernel(DecodeArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int V = Elem<T>::kVec;
  constexpr int kLanes = HD / V;
  constexpr int kReq = kThreads / kLanes;
  constexpr int64_t R = 4 * HD;
  const int64_t b = (int64_t)blockIdx.x * kReq + threadIdx.x / kLanes;
  const int c = (threadIdx.x % kLanes) * V;
  if (b >= a.batch) return;
  float* out = a.out + b * HD + c;
  const E* input = static_cast<const E*>(a.input);
  const kvc_plan_d rec = load_plan_d(a.plan_d + b);
  u32x4 q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = load16(input + b * R + i * HD + c);
  // keep the row's loads here, in flight with the record's, rather than moved
  // into the branches below that use them
  asm volatile("" ::: "memory");
  if (plan_d_invalid(rec)) {
    store_zeros<V>(out);
    return;
  }
  const bool boundary = (rec.seq_len & 3u) == 0u;
  const bool first_block = rec.seq_len == 4u;
  const int64_t wl = rec.write_loc, rp0 = rec.read_page_0, rp1 = rec.read_page_1;
  bool ok = wl >= 0 && wl < a.num_state_rows;
  // the pool reads entries 0..6 from the state (7 = the new token)
  if (boundary) ok = ok && c4_record_ok(b, 7, rp0, rp1, first_block ? 4 : 0, a.batch, a.num_state_rows);
  if (!ok) {
    if (c == 0 && a.status) atomicOr(a.status, KVC_DERR_RECORD);
    store_zeros<V>(out);
    return;
  }
  E* state = static_cast<E*>(a.state);
  const E* ape = static_cast<const E*>(a.ape);
  u32x4 kv_raw[8], sc_raw[8], ap_raw[8];
  if (boundary) {
    if (first_block) {
      c4_decode_window<T, HD, 4>(state, ape, rp0, rp1, c, q, kv_raw, sc_raw, ap_raw);
    } else {
      c4_decode_window<T, HD, 0>(state, ape, rp0, rp1, c, q, kv_raw, sc_raw, ap_raw);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) store16_stream(state + wl * R + i * HD + c, q[i]);
  if (!boundary) {
    store_zeros<V>(out);
    return;
  }
  float res[V];
  if (first_block) {
    c4_pool_math<T, 4>(kv_raw, sc_raw, [&](int i) { return ap_raw[i]; }, res);
  } else {
    c4_pool_math<T, 0>(kv_raw, sc_raw, [&](int i) { return ap_raw[i]; }, res);
  }
  store_floats<V, true>(out, res);
}

// Ratio 4 with the store step, with the loads of decode_c4.  No early return:
// a row of more than 64 lanes (fp32, hd 512) reduces its sum of squares
// across two waves with a barrier.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void decode_c4_store_kernel(DecodeArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int V = Elem<T>::kVec;
  constexpr int kLanes = HD / V;
  constexpr int kReq = kThreads / kLanes;
  constexpr int64_t R = 4 * HD;
  __shared__ float red[kThreads / kWave];
  const int64_t b = (int64_t)blockIdx.x * kReq + threadIdx.x / kLanes;
  const int c = (threadIdx.x % kLanes) * V;
  float res[V];
#pragma unroll
  for (int v = 0; v < V; ++v) res[v] = 0.f;
  bool pooled = false;
  int32_t loc = -1, pos = 0;
  StoreOperands<V> ops;
  if (b < a.batch) {
    const E* input = static_cast<const E*>(a.input);
    const kvc_plan_d rec = load_plan_d(a.plan_d + b);
    u32x4 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = load16(input + b * R + i * HD + c);
    asm volatile("" ::: "memory");  // the row's loads stay in flight with the record's
    if (!plan_d_invalid(rec)) {
      const bool boundary = (rec.seq_len & 3u) == 0u;
      const bool first_block = rec.seq_len == 4u;
      const int64_t wl = rec.write_loc, rp0 = rec.read_page_0, rp1 = rec.read_page_1;
      bool ok = wl >= 0 && wl < a.num_state_rows;
      if (boundary) ok = ok && c4_record_ok(b, 7, rp0, rp1, first_block ? 4 : 0, a.batch, a.num_state_rows);
      if (!ok) {
        if (c == 0 && a.status) atomicOr(a.status, KVC_DERR_RECORD);
      } else {
        E* state = static_cast<E*>(a.state);
        const E* ape = static_cast<const E*>(a.ape);
        u32x4 kv_raw[8], sc_raw[8], ap_raw[8];
        if (boundary) {
          pos = (int32_t)rec.seq_len - 4;
          if (first_block) {
            c4_decode_window<T, HD, 4>(state, ape, rp0, rp1, c, q, kv_raw, sc_raw, ap_raw);
          } else {
            c4_decode_window<T, HD, 0>(state, ape, rp0, rp1, c, q, kv_raw, sc_raw, ap_raw);
          }
          loc = fetch_loc(a.st, b);  // in flight with the window
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) store16_stream(state + wl * R + i * HD + c, q[i]);
        if (boundary) {
          if (first_block) {
            c4_pool_math<T, 4>(kv_raw, sc_raw, [&](int i) { return ap_raw[i]; }, res);
          } else {
            c4_pool_math<T, 0>(kv_raw, sc_raw, [&](int i) { return ap_raw[i]; }, res);
          }
          pooled = store_ok(a.st, loc, pos);
          if (pooled) {
            fetch_operands<V, HD>(a.st, c, pos, ops);
          } else {
            if (c == 0 && a.status) atomicOr(a.status, KVC_DERR_RECORD);
#pragma unroll
            for (int v = 0; v < V; ++v) res[v] = 0.f;
          }
        }
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) ss = fmaf(res[v], res[v], ss);
  ss = row_sum<kLanes>(ss, red);  // reached by every thread
  if (pooled) norm_rope_store<V, HD>(res, ss, c, loc, ops, a.st);
}

// Ratio 128: one launch, two roles chosen by workgroup index.
//  - Pool workgroups (the first n_pool) pool the boundary requests (those
//    whose new token closes a block), each over one channel slice of SL
//    channels: the workgroup's 256 threads are streams of SL/V lanes, each
//    stream holding every S-th entry of the 128-entry window, and the stream
//    partials merge in LDS.  The slices of a row need no merge (the softmax
//    is per channel), so a boundary request is spread over HD/SL workgroups
//    on different CUs with no exchange.  Which boundary requests a pool
//    workgroup takes:
//    - with the planner's boundary list (the boundary requests, each once
//      with its page, and their count): slot p of P takes list entries p,
//      p + P, p + 2P, ...; it loads the count and its first entry in one
//      round, so it goes straight to the window, and the requests are spread
//      evenly over the slots wherever they sit in the batch (a request's row
//      is the same whichever slot pools it);
//    - without it: the batch is cut into ranges of 1024 requests with R rank
//      slots each.  Workgroup (q, r, cs) loads the range's records (4 per
//      thread, one round of loads), ranks the range's boundary requests in
//      request order (a ballot per wave and pass, prefix counts in LDS), and
//      pools those whose rank is r modulo R.  Every slot scans the whole
//      range, so more slots cost more scanning.
//  - Copy workgroups: 8 requests each.  The 8 input rows are loaded at once
//    (16-byte vectors, 2*HD/V per row, the vectors of a row on consecutive
//    lanes; 4 per thread at hd 512 bf16: copies with 8 or more vectors per
//    thread run slower) while 8 threads load the records and leave each request's
//    verdict in LDS; then the rows go to their state rows, and requests that
//    close no block (or whose record is invalid or out of range) get a zero
//    output row.  A boundary request's output row is the pool workgroups'.
// The pool reads entries 0..126 of the page and takes entry 127, the new
// token, from the input row; the copy writes only row 127 of the page
// (write_loc of a boundary request), so the two roles touch disjoint rows.
// SL (the slice width) is chosen by the host: a slice reads a 2*SL*sizeof(T)
// byte piece of each of the window's rows (kv and score halves), and wider
// pieces stream better from HBM, while narrower slices finish a single
// boundary request sooner.
constexpr int kDec128Threads = 256;
constexpr int kDec128CopyGroup = 8;
constexpr int kDec128Range = 1024;  // requests ranked together
constexpr int kDec128Passes = kDec128Range / kDec128Threads;

template <typename T, int HD, int SL>
struct Dec128Shape {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int CS = HD / SL;                    // channel slices per request
  static constexpr int S = kDec128Threads / (SL / V);  // streams of a pool workgroup
  // entries per stream and round of loads: the whole window in one round at
  // 64 channels, rounds of 4 entries in wider slices (register budget)
  static constexpr int U = SL == 64 || 128 / S < 4 ? 128 / S : 4;
  typedef C128Pool<T, HD, kDec128Threads, CS, U> Pool;
};

// Whether decode record rec (request b) can run, and whether it pools.
__device__ __forceinline__ bool dec128_ok(const kvc_plan_d& rec, int64_t b, const DecodeArgs& a) {
  const bool boundary = (rec.seq_len & 127u) == 0u;
  bool ok = rec.write_loc >= 0 && rec.write_loc < a.num_state_rows;
  if (boundary) ok = ok && c128_record_ok(b, 127, rec.read_page_0, a.batch, a.num_state_rows);
  return ok;
}

template <typename T, int HD, int SL>
__device__ __forceinline__ void dec128_pool_role(const DecodeArgs& a, int64_t q, int r, int n_slots, int cs,
                                                 typename Dec128Shape<T, HD, SL>::Pool::A* lds) {
  typedef typename Elem<T>::storage E;
  typedef typename Dec128Shape<T, HD, SL>::Pool Pool;
  constexpr int kWaves = kDec128Threads / kWave;
  __shared__ int32_t req[kDec128Range], page[kDec128Range];
  __shared__ int cnt[kDec128Passes][kWaves];  // boundary requests per pass and wave
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int64_t base = q * kDec128Range;
  // the range's records, clamped into the batch (a record past the batch is
  // loaded from the last request and not counted), all in one round of loads
  kvc_plan_d rec[kDec128Passes];
#pragma unroll
  for (int i = 0; i < kDec128Passes; ++i)
    rec[i] = load_plan_d(a.plan_d + min(base + i * kDec128Threads + t, (int64_t)a.batch - 1));
  bool pools[kDec128Passes];
  unsigned long long mask[kDec128Passes];
#pragma unroll
  for (int i = 0; i < kDec128Passes; ++i) {
    const int64_t b = base + i * kDec128Threads + t;
    pools[i] = b < a.batch && !plan_d_invalid(rec[i]) && (rec[i].seq_len & 127u) == 0u && dec128_ok(rec[i], b, a);
    mask[i] = __ballot(pools[i]);
    if (lane == 0) cnt[i][wave] = __popcll(mask[i]);
  }
  __syncthreads();
  // rank = the boundary requests before this one in the range (request order)
  int total = 0;
#pragma unroll
  for (int i = 0; i < kDec128Passes; ++i) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += cnt[i][w];
  }
#pragma unroll
  for (int i = 0; i < kDec128Passes; ++i) {
    int pre = 0;  // boundary requests of the earlier passes and of the earlier waves of this pass
#pragma unroll
    for (int i2 = 0; i2 < kDec128Passes; ++i2) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) pre += (i2 < i || (i2 == i && w < wave)) ? cnt[i2][w] : 0;
    }
    const int rank = pre + __popcll(mask[i] & __lanemask_lt());
    if (pools[i] && rank % n_slots == r) {
      req[rank / n_slots] = (int32_t)(base + i * kDec128Threads + t);
      page[rank / n_slots] = rec[i].read_page_0;
    }
  }
  __syncthreads();
  const int cnt_mine = total > r ? (total - 1 - r) / n_slots + 1 : 0;
  const E* state = static_cast<const E*>(a.state);
  const E* input = static_cast<const E*>(a.input);
  const E* ape = static_cast<const E*>(a.ape);
  for (int j = 0; j < cnt_mine; ++j) {  // uniform over the workgroup
    Pool::accumulate(state, input, ape, req[j], 127, page[j], cs, lds);
    Pool::store_merged_par(lds, cs, a.out + (int64_t)req[j] * HD);
    __syncthreads();  // the next pool reuses lds
  }
}

// Slot p of n_slots with the planner's boundary list: entries p, p + n_slots,
// ... below the count (clamped to [0, batch]).  An entry outside the batch
// or the state is skipped and reported.
template <typename T, int HD, int SL>
__device__ __forceinline__ void dec128_list_role(const DecodeArgs& a, int p, int n_slots, int cs,
                                                 typename Dec128Shape<T, HD, SL>::Pool::A* lds) {
  typedef typename Elem<T>::storage E;
  typedef typename Dec128Shape<T, HD, SL>::Pool Pool;
  const int32_t* list = a.boundaries;
  // the count and the first entry in one round of loads (p < n_slots <= batch:
  // the entry lies inside the list whatever the count)
  const int32_t raw = list[2 * (int64_t)a.batch];
  int2 e = *reinterpret_cast<const int2*>(list + 2 * p);
  const int n = raw < 0 ? 0 : (raw > a.batch ? a.batch : raw);
  const E* state = static_cast<const E*>(a.state);
  const E* input = static_cast<const E*>(a.input);
  const E* ape = static_cast<const E*>(a.ape);
  for (int j = p; j < n; j += n_slots) {  // uniform over the workgroup
    if (j != p) e = *reinterpret_cast<const int2*>(list + 2 * (int64_t)j);
    const int64_t b = e.x;
    if (b >= 0 && b < a.batch && c128_record_ok(b, 127, e.y, a.batch, a.num_state_rows)) {
      Pool::accumulate(state, input, ape, b, 127, e.y, cs, lds);
      Pool::store_merged_par(lds, cs, a.out + b * HD);
      __syncthreads();  // the next pool reuses lds
    } else if (threadIdx.x == 0 && a.status) {
      atomicOr(a.status, KVC_DERR_RECORD);
    }
  }
}

template <typename T, int HD>
__device__ __forceinline__ void dec128_copy_role(const DecodeArgs& a, int64_t b0) {
  typedef typename Elem<T>::storage E;
  constexpr int V = Elem<T>::kVec;
  constexpr int64_t R = 2 * HD;
  constexpr int RV = 2 * HD / V;                   // vectors of an input / state row
  constexpr int RPP = kDec128Threads / RV;         // rows per pass of the workgroup
  constexpr int PER = kDec128CopyGroup / RPP;      // vectors per thread
  constexpr int OV = HD / 4;                       // vectors of an fp32 output row
  constexpr int ORPP = kDec128Threads / OV;
  constexpr int OPER = kDec128CopyGroup / ORPP;
  static_assert(kDec128Threads % RV == 0 && kDec128CopyGroup % RPP == 0, "copy shape");
  static_assert(kDec128Threads % OV == 0 && kDec128CopyGroup % ORPP == 0, "zero-row shape");
  __shared__ int64_t dst[kDec128CopyGroup];  // state row of the request's new token, or -1
  __shared__ int zero[kDec128CopyGroup];     // whether this workgroup writes its output row
  const int t = threadIdx.x;
  const int col = t % RV, r0 = t / RV;
  const E* input = static_cast<const E*>(a.input);
  // the input rows depend on nothing: in flight with the records.  A row past
  // the batch loads the last row instead (unconditional loads stay in one
  // straight run; that row is never stored).  Cached loads: a decode step's
  // new rows were just written by the layer that produced them.
  u32x4 buf[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t b = min(b0 + r0 + i * RPP, (int64_t)a.batch - 1);
    buf[i] = load16(input + b * R + col * V);
  }
  if (t < kDec128CopyGroup) {
    const int64_t b = b0 + t;
    int64_t d = -1;
    int z = 0;
    if (b < a.batch) {
      const kvc_plan_d rec = load_plan_d(a.plan_d + b);
      z = 1;
      if (!plan_d_invalid(rec)) {
        if (dec128_ok(rec, b, a)) {
          d = rec.write_loc;
          z = (rec.seq_len & 127u) != 0u;
        } else if (a.status) {
          atomicOr(a.status, KVC_DERR_RECORD);
        }
      }
    }
    dst[t] = d;
    zero[t] = z;
  }
  __syncthreads();
  E* state = static_cast<E*>(a.state);
  int64_t d[PER];  // all verdicts read before the first store
#pragma unroll
  for (int i = 0; i < PER; ++i) d[i] = dst[r0 + i * RPP];
  const int ocol = t % OV, or0 = t / OV;
  int z[OPER];
#pragma unroll
  for (int i = 0; i < OPER; ++i) z[i] = zero[or0 + i * ORPP];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (d[i] >= 0) store16_stream(state + d[i] * R + col * V, buf[i]);
  }
  const u32x4 zv = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < OPER; ++i) {
    if (z[i]) store16_stream(a.out + (b0 + or0 + i * ORPP) * HD + ocol * 4, zv);
  }
}

template <typename T, int HD, int SL>
__global__ __launch_bounds__(kDec128Threads) void decode_c128_kernel(DecodeArgs a, int n_slots, int n_pool) {
  typedef typename Dec128Shape<T, HD, SL>::Pool Pool;
  constexpr int CS = Dec128Shape<T, HD, SL>::CS;
  if ((int)blockIdx.x < n_pool) {
    __shared__ typename Pool::A lds[Pool::kLdsElems];  // the stream partials, either way of choosing requests
    const int slot = blockIdx.x / CS;
    if (a.boundaries != nullptr) {
      dec128_list_role<T, HD, SL>(a, slot, n_slots, blockIdx.x % CS, lds);
    } else {  // slot = (range, rank slot)
      dec128_pool_role<T, HD, SL>(a, slot / n_slots, slot % n_slots, n_slots, blockIdx.x % CS, lds);
    }
  } else {
    dec128_copy_role<T, HD>(a, (int64_t)(blockIdx.x - n_pool) * kDec128CopyGroup);
  }
}

// Rank slots per range of 1024 requests (no boundary list): 8 up to 32 768
// requests, then 4.  Measured on MI355X at hd 512 bf16 (HIP events, 1/128 of
// the requests closing a block) against the previous design, which pooled the
// boundary requests of each group of 16-256 neighbours in one workgroup:
//  - boundaries at random places: 24.9 against 29.6 us at 16 384 requests,
//    49.3 against 47.6 at 32 768, 88.2 against 84.8 at 65 536 (4 slots;
//    8 slots take 91.2 there);
//  - all boundaries in the first requests of the batch: 60 against 198 us,
//    116 against 208, 399 against 754;
//  - 1024 requests (5 closing): 5.8 against 6.0 us by kernel trace.
// More slots spread a cluster wider but make more workgroups scan each range.
inline int dec128_rank_slots(int batch) {
  return batch <= 32768 ? 8 : 4;
}

// List slots: one per 64 requests, about twice the boundary requests of a
// batch with random lengths, so that a slot rarely pools two.
inline int dec128_list_slots(int batch) {
  return std::max(1, std::min(batch, (batch + 63) / 64));
}

// Slice width: 64 channels, and 256-byte pieces (128 bf16 channels) above
// 16 384 requests.  Measured on MI355X at hd 512 bf16 (kernel trace, rank
// slots): 47.7 against 50.7 us at 32 768 requests and 83.0 against 91.7 at
// 65 536, but 26.0 against 23.9 at 16 384 and 7.3 against 6.2 at 1024.
constexpr int kDec128WideBatch = 16384;
template <typename T>
constexpr int dec128_wide_slice() {
  return 256 / (int)sizeof(typename Elem<T>::storage) > 64 ? 256 / (int)sizeof(typename Elem<T>::storage) : 64;
}

template <typename T, int HD, int SL>
hipError_t dec128_go(const DecodeArgs& a, hipStream_t s) {
  constexpr int CS = Dec128Shape<T, HD, SL>::CS;
  int n_slots, n_pool;
  if (a.boundaries != nullptr) {
    n_slots = dec128_list_slots(a.batch);
    n_pool = n_slots * CS;
  } else {
    n_slots = dec128_rank_slots(a.batch);
    n_pool = (a.batch + kDec128Range - 1) / kDec128Range * n_slots * CS;
  }
  const int n_copy = (a.batch + kDec128CopyGroup - 1) / kDec128CopyGroup;
  decode_c128_kernel<T, HD, SL><<<(unsigned)(n_pool + n_copy), kDec128Threads, 0, s>>>(a, n_slots, n_pool);
  return hipGetLastError();
}

template <typename T, int HD>
struct C4Go {
  static hipError_t go(const DecodeArgs& a, hipStream_t s) {
    constexpr int kReq = kThreads / (HD / Elem<T>::kVec);
    decode_c4_kernel<T, HD><<<(a.batch + kReq - 1) / kReq, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
};

template <typename T, int HD>
struct C128Go {
  static hipError_t go(const DecodeArgs& a, hipStream_t s) {
    constexpr int kNarrow = HD < 64 ? HD : 64;
    constexpr int kWide = HD < dec128_wide_slice<T>() ? HD : dec128_wide_slice<T>();
    if (kWide != kNarrow && a.batch > kDec128WideBatch) return dec128_go<T, HD, kWide>(a, s);
    return dec128_go<T, HD, kNarrow>(a, s);
  }
};

template <template <typename, int> class F>
hipError_t dispatch(kvc_dtype dtype, int hd, const DecodeArgs& a, hipStream_t stream) {
  if (dtype == KVC_BF16) {
    if (hd == 128) return F<Bf16, 128>::go(a, stream);
    if (hd == 256) return F<Bf16, 256>::go(a, stream);
    return F<Bf16, 512>::go(a, stream);
  }
  if (hd == 128) return F<float, 128>::go(a, stream);
  if (hd == 256) return F<float, 256>::go(a, stream);
  return F<float, 512>::go(a, stream);
}

}  // namespace

template <typename T, int HD>
struct C4StoreGo {
  static hipError_t go(const DecodeArgs& a, hipStream_t s) {
    constexpr int kReq = kThreads / (HD / Elem<T>::kVec);
    decode_c4_store_kernel<T, HD><<<(a.batch + kReq - 1) / kReq, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
};

hipError_t launch_decode_c4_store(kvc_dtype dtype, int head_dim, const DecodeArgs& a, hipStream_t stream) {
  return dispatch<C4StoreGo>(dtype, head_dim, a, stream);
}

hipError_t launch_decode_c4(kvc_dtype dtype, int head_dim, const DecodeArgs& a, hipStream_t stream) {
  return dispatch<C4Go>(dtype, head_dim, a, stream);
}

hipError_t launch_decode_c128(kvc_dtype dtype, int head_dim, const DecodeArgs& a, hipStream_t stream) {
  return dispatch<C128Go>(dtype, head_dim, a, stream);
}

}  // namespace kvc
