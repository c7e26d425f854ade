// kvc_compress.hip - prefill compress kernels (c4.cuh page, flash_c4_prefill
// with kWrite = false; compressor_v2.py page,
// _c128_compress_prefill_compress_kernel) and the state write (c4.cuh,
// c4_write; compressor_v2.py, _c128_compress_prefill_write_kernel).
//
// All three are HBM-streaming kernels (no dense contraction, so no MFMA):
//  - compress c4: 64 lanes x 16 B cover the 512 channels of one bf16 row, so a
//    lane group reads each of its 8 window entries' kv and score quarters
//    with one 16-byte load each, all 16 (+8 ape) loads in flight before the
//    first use; 512-thread workgroups hold 512 / lanes-per-row rows.
//  - compress c128: one workgroup per compressed row; its streams split the
//    128 window entries and merge their online-softmax partials in LDS.
//  - write: one wave per record, the whole row copied with 16-byte vectors.
// Grids are sized from the host-known capacities; threads past counts[0]
// (counts[1] for the write) return at once, so no host sync is needed.
#include "kvc_device.hpp"
#include "kvc_launch.hpp"
#include "kvc_pool.hpp"
#include "kvc_store.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;
// The ratio-4 pool runs 512-thread workgroups (8 rows of hd 512 bf16): against
// 256 threads, 4-5% less time on the mixed prefill (12 or 16 rows per
// workgroup are slower again).
constexpr int kC4Threads = 512;
// The ratio-128 pool runs 512 threads per row: 8 streams of 16 entries, so a row
// takes half as many rounds of loads as with 256 (with the pool's priority by
// progress, 6% faster on the mixed prefill).
constexpr int kC128Threads = 512;

// STORE = false: the pooled rows go to a.out as float32.  STORE = true: the
// row is normalised, rotated and stored as bf16 into the compressed cache
// (a.st) straight from registers.
template <typename T, int HD, bool STORE>
__global__ __launch_bounds__(kC4Threads) void compress_c4_kernel(CompressArgs a) {
  constexpr int V = Elem<T>::kVec;
  constexpr int kLanes = HD / V;
  constexpr int kRows = kC4Threads / kLanes;
  const int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes;
  const int c = (threadIdx.x % kLanes) * V;
  typedef typename Elem<T>::storage E;
  // The record and the count share one round trip: the record load is
  // unconditional, clamped into the buffer (every index below cap_c holds a
  // record: valid, padding or, after a planner error, stale), and only rows
  // below counts[0] use theirs.
  const kvc_plan_c rec = load_plan_c(a.plan_c + (row < a.cap_c ? row : a.cap_c - 1));
  bool live = (row < a.cap_c) & (row < a.counts[0]) & !plan_c_invalid(rec);
  float res[V];
#pragma unroll
  for (int v = 0; v < V; ++v) res[v] = 0.f;
  int32_t pos = 0, loc = -1;  // positions < 2^24, cache rows <= INT32_MAX
  StoreOperands<V> ops;
  if (live) {
    const int64_t ragged = rec.ragged_blen & 0xFFFFFFu;
    const int blen = (int)(rec.ragged_blen >> 24);
    const int64_t rp0 = rec.read_page_0, rp1 = rec.read_page_1;
    const bool first_block = rec.seq_len == 4u;
    if (!c4_record_ok(ragged, blen, rp0, rp1, first_block ? 4 : 0, a.num_q, a.num_state_rows)) {
      if (c == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
      live = false;
    }
    if (live) {
      const E* state = static_cast<const E*>(a.state);
      const E* input = static_cast<const E*>(a.input);
      const E* ape = static_cast<const E*>(a.ape);
      if constexpr (STORE) {
        // the store's own loads go out with the window's and are checked after the pool
        pos = rec.seq_len >= 4u ? (int32_t)rec.seq_len - 4 : 0;
        const auto pre = [&]() { loc = fetch_loc(a.st, ragged); };
        if (first_block) {
          c4_pool<T, HD, 4>(state, input, ape, ragged, blen, rp0, rp1, c, res, pre);
        } else {
          c4_pool<T, HD, 0>(state, input, ape, ragged, blen, rp0, rp1, c, res, pre);
        }
        if (store_ok(a.st, loc, pos)) {
          fetch_operands<V, HD>(a.st, c, pos, ops);  // cached loads, in flight during the row reduction
        } else {
          if (c == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
          live = false;
#pragma unroll
          for (int v = 0; v < V; ++v) res[v] = 0.f;
        }
      } else if (first_block) {
        c4_pool<T, HD, 4>(state, input, ape, ragged, blen, rp0, rp1, c, res);
      } else {
        c4_pool<T, HD, 0>(state, input, ape, ragged, blen, rp0, rp1, c, res);
      }
    }
  }
  if constexpr (STORE) {
    __shared__ float red[kC4Threads / kWave];
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) ss = fmaf(res[v], res[v], ss);
    ss = row_sum<kLanes>(ss, red);  // reached by every thread (rows wider than a wave sync)
    if (live) norm_rope_store<V, HD>(res, ss, c, loc, ops, a.st);
  } else {
    // A lane holds V adjacent channels, so storing them directly would write
    // 16-byte pieces at a 4*V-byte stride.  Staging the row in LDS lets every
    // store instruction write 64 x 16 contiguous bytes instead (2% faster in
    // the full step; with cold caches the two are even).
    __shared__ float stage[kC4Threads * V];  // the workgroup's output rows
    float* w = stage + (threadIdx.x / kLanes) * HD;
    store_floats<V>(w + c, res);
    __syncthreads();
    if (live) {
      const int lane = threadIdx.x % kLanes;
#pragma unroll
      for (int k = 0; k < V / 4; ++k) {
        const int ch = k * (kLanes * 4) + lane * 4;
        store16_stream(a.out + row * HD + ch, load16(w + ch));  // written once, read by a later kernel
      }
    }
  }
}

template <typename T, int HD, bool STORE>
__global__ __launch_bounds__(kC128Threads) void compress_c128_kernel(CompressArgs a) {
  typedef typename Elem<T>::storage E;
  typedef C128Pool<T, HD, kC128Threads> Pool;
  __shared__ typename Pool::A lds[Pool::kLdsElems];
  const int64_t row = blockIdx.x;  // < cap_c (the grid)
  const kvc_plan_c rec = load_plan_c(a.plan_c + row);  // in flight with the count (as in compress_c4)
  if ((row >= a.counts[0]) | plan_c_invalid(rec)) return;
  const int64_t ragged = rec.ragged_blen & 0xFFFFFFu;
  const int blen = (int)(rec.ragged_blen >> 24);
  const int64_t rp0 = rec.read_page_0;
  if (!c128_record_ok(ragged, blen, rp0, a.num_q, a.num_state_rows)) {
    if (threadIdx.x == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
    return;  // the whole workgroup leaves: nothing below is reached by part of it
  }
  const E* state = static_cast<const E*>(a.state);
  const E* input = static_cast<const E*>(a.input);
  const E* ape = static_cast<const E*>(a.ape);
  if constexpr (STORE) {
    // thread t ends with channels 2t, 2t+1 (a rotary pair); threads past HD/2 hold zeros.
    // The store's loads go out after the window's (holding them across the
    // pool would cost a wave per SIMD of occupancy).
    __shared__ float red[kC128Threads / kWave];
    const int c = 2 * threadIdx.x;
    const int32_t pos = rec.seq_len >= 128u ? (int32_t)rec.seq_len - 128 : 0;
    Pool::accumulate(state, input, ape, ragged, blen, rp0, 0, lds);
    const int32_t loc = fetch_loc(a.st, ragged);
    if (!store_ok(a.st, loc, pos)) {  // uniform over the workgroup
      if (threadIdx.x == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
      return;
    }
    StoreOperands<2> ops;
    if (c < HD) fetch_operands<2, HD>(a.st, c, pos, ops);  // cached loads, in flight during the merge
    float x[2] = {0.f, 0.f};
    if (c < HD) {
      x[0] = Pool::merged(lds, c);
      x[1] = Pool::merged(lds, c + 1);
    }
    const float ss = block_sum<kC128Threads>(fmaf(x[0], x[0], x[1] * x[1]), red);
    if (c < HD) norm_rope_store<2, HD>(x, ss, c, loc, ops, a.st);
  } else {
    Pool::run(state, input, ape, ragged, blen, rp0, 0, a.out + row * HD, lds);
  }
}

constexpr int kWriteRowsPerBlock = kThreads / kWave;

// One wave per record.  PER = 16-byte vectors per lane (a row holds up to
// 64 * PER vectors); the input row is read once and stored to the state, both
// streaming: the row is read back only by a later chunk's kernels, and a
// cached store would leave dirty lines that slow the next streaming kernel.
template <int PER>
__global__ __launch_bounds__(kThreads) void write_kernel(WriteArgs a) {
  const int64_t k = (int64_t)blockIdx.x * kWriteRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  // the record (clamped into the buffer, as in compress_c4) is in flight with the count
  const u32x2 rec = load8(a.plan_w + (k < a.cap_w ? k : a.cap_w - 1));
  __builtin_amdgcn_sched_barrier(0);  // keep the count's load (and its wait) after this one
  const int64_t ragged = rec.x;
  const int64_t loc = (int32_t)rec.y;
  const bool bad = (ragged >= a.num_q) | (loc < 0) | (loc >= a.num_state_rows);
  if ((k >= a.cap_w) | (k >= a.counts[1]) | (rec.x == 0xFFFFFFFFu)) return;
  if (bad) {
    if (lane == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
    return;
  }
  const int64_t rb = (int64_t)a.row_vecs * 16;
  const char* src = static_cast<const char*>(a.input) + ragged * rb;
  char* dst = static_cast<char*>(a.state) + loc * rb;
  if (PER == 1 && lane >= a.row_vecs) return;  // rows of 32 vectors (512 B)
  u32x4 buf[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) buf[u] = load16_stream(src + (int64_t)(lane + u * kWave) * 16);
#pragma unroll
  for (int u = 0; u < PER; ++u) store16_stream(dst + (int64_t)(lane + u * kWave) * 16, buf[u]);
}

template <typename T, int HD, bool STORE>
hipError_t c4_launch(const CompressArgs& a, hipStream_t stream) {
  constexpr int kRows = kC4Threads / (HD / Elem<T>::kVec);
  const int grid = (a.cap_c + kRows - 1) / kRows;
  compress_c4_kernel<T, HD, STORE><<<grid, kC4Threads, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int HD, bool STORE>
hipError_t c128_launch(const CompressArgs& a, hipStream_t stream) {
  compress_c128_kernel<T, HD, STORE><<<a.cap_c, kC128Threads, 0, stream>>>(a);
  return hipGetLastError();
}

template <template <typename, int> class F, typename Args>
hipError_t dispatch(kvc_dtype dtype, int hd, const Args& a, hipStream_t stream) {
  if (dtype == KVC_BF16) {
    if (hd == 128) return F<Bf16, 128>::go(a, stream);
    if (hd == 256) return F<Bf16, 256>::go(a, stream);
    return F<Bf16, 512>::go(a, stream);
  }
  if (hd == 128) return F<float, 128>::go(a, stream);
  if (hd == 256) return F<float, 256>::go(a, stream);
  return F<float, 512>::go(a, stream);
}

template <typename T, int HD>
struct C4Go {
  static hipError_t go(const CompressArgs& a, hipStream_t s) { return c4_launch<T, HD, false>(a, s); }
};
template <typename T, int HD>
struct C128Go {
  static hipError_t go(const CompressArgs& a, hipStream_t s) { return c128_launch<T, HD, false>(a, s); }
};
template <typename T, int HD>
struct C4StoreGo {
  static hipError_t go(const CompressArgs& a, hipStream_t s) { return c4_launch<T, HD, true>(a, s); }
};
template <typename T, int HD>
struct C128StoreGo {
  static hipError_t go(const CompressArgs& a, hipStream_t s) { return c128_launch<T, HD, true>(a, s); }
};

}  // namespace

hipError_t launch_compress_c4(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream) {
  return dispatch<C4Go>(dtype, head_dim, a, stream);
}

hipError_t launch_compress_c128(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream) {
  return dispatch<C128Go>(dtype, head_dim, a, stream);
}

hipError_t launch_compress_c4_store(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream) {
  return dispatch<C4StoreGo>(dtype, head_dim, a, stream);
}

hipError_t launch_compress_c128_store(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream) {
  return dispatch<C128StoreGo>(dtype, head_dim, a, stream);
}

hipError_t launch_write(const WriteArgs& a, hipStream_t stream) {
  // rows hold 32 (ratio 128, bf16, hd 128) to 512 (ratio 4, fp32, hd 512) vectors
  const int grid = (a.cap_w + kWriteRowsPerBlock - 1) / kWriteRowsPerBlock;
  switch (a.row_vecs) {
    case 32:
    case 64:
      write_kernel<1><<<grid, kThreads, 0, stream>>>(a);
      break;
    case 128:
      write_kernel<2><<<grid, kThreads, 0, stream>>>(a);
      break;
    case 256:
      write_kernel<4><<<grid, kThreads, 0, stream>>>(a);
      break;
    case 512:
      write_kernel<8><<<grid, kThreads, 0, stream>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvc
