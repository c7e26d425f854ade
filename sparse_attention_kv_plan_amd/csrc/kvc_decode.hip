// kvc_decode.hip - fused decode step: store the new token, pool on a block
// boundary (c4.cuh page, flash_c4_decode; compressor_v2.py page,
// _c128_compress_decode_kernel).
//
// The window's last entry is the new token itself.  Instead of reading it
// back through the state (a read-after-write across lanes), the pool takes it
// from the input row, which holds the same bits; the other entries are state
// rows that this step does not write (indices are distinct per call).
//  - ratio 4: one lane group (64 lanes for hd 512 bf16) per request; each lane
//    copies its 16-byte slice of the 4 quarters, then pools 8 entries.
//  - ratio 128: a few workgroups per request, each owning a slice of the
//    channels: it copies its slice of the row and, on a boundary, pools its
//    channels over the 128-entry page.
//  - ratio 4 with the store step (compressor_v2.py, compress_norm_rope_store):
//    the pooled row is normalised, rotated and stored as bf16 into the
//    compressed cache straight from registers; nothing else is written for it.
#include "kvc_device.hpp"
#include "kvc_launch.hpp"
#include "kvc_pool.hpp"
#include "kvc_store.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;

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
  const kvc_plan_d rec = load_plan_d(a.plan_d + b);
  if (plan_d_invalid(rec)) {
    store_zeros<V>(out);
    return;
  }
  const bool boundary = (rec.seq_len & 3u) == 0u;
  const bool first_block = rec.seq_len == 4u;
  const int64_t wl = rec.write_loc, rp0 = rec.read_page_0, rp1 = rec.read_page_1;
  bool ok = wl >= 0 && wl < a.num_state_rows;
  // the pool reads entries 0..6 from the state (7 = the new token, from the input)
  if (boundary) ok = ok && c4_record_ok(b, 7, rp0, rp1, first_block ? 4 : 0, a.batch, a.num_state_rows);
  if (!ok) {
    if (c == 0 && a.status) atomicOr(a.status, KVC_DERR_RECORD);
    store_zeros<V>(out);
    return;
  }
  E* state = static_cast<E*>(a.state);
  const E* input = static_cast<const E*>(a.input);
  u32x4 q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = load16(input + b * R + i * HD + c);
#pragma unroll
  for (int i = 0; i < 4; ++i) store16_stream(state + wl * R + i * HD + c, q[i]);
  if (!boundary) {
    store_zeros<V>(out);
    return;
  }
  float res[V];
  const E* ape = static_cast<const E*>(a.ape);
  if (first_block) {
    c4_pool<T, HD, 4>(state, input, ape, b, 7, rp0, rp1, c, res);
  } else {
    c4_pool<T, HD, 0>(state, input, ape, b, 7, rp0, rp1, c, res);
  }
  store_floats<V, true>(out, res);
}

// Ratio 4 with the store step.  No early return: a row of more than 64 lanes
// (fp32, hd 512) reduces its sum of squares across two waves with a barrier.
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
    const kvc_plan_d rec = load_plan_d(a.plan_d + b);
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
        const E* input = static_cast<const E*>(a.input);
        u32x4 q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = load16(input + b * R + i * HD + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) store16_stream(state + wl * R + i * HD + c, q[i]);
        if (boundary) {
          pos = (int32_t)rec.seq_len - 4;
          const auto pre = [&]() { loc = fetch_loc(a.st, b); };
          const E* ape = static_cast<const E*>(a.ape);
          if (first_block) {
            c4_pool<T, HD, 4>(state, input, ape, b, 7, rp0, rp1, c, res, pre);
          } else {
            c4_pool<T, HD, 0>(state, input, ape, b, 7, rp0, rp1, c, res, pre);
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

// Ratio 128: a workgroup of 128 threads owns a group of kDec128Group
// requests and one slice of HD / CS channels; CS workgroups cover a group.
// Every request's slice of the row is 16 vectors of 16 bytes, so each thread
// copies one vector of one request into the state (and zeroes its part of the
// output when the request closes no block).  The group's boundary requests
// are then pooled one after another, each by its CS workgroups at once on
// different CUs (8 lanes x 16 bytes per stream, 16 streams, 8 entries each).
// The copy phase leaves each request's verdict in LDS, so the pool loop loads
// no record again.
// One request per workgroup would make the light requests (a 768-byte copy
// each) a dispatch-bound stream of tiny workgroups at large batches.
constexpr int kDec128Threads = 128;
constexpr int kDec128SliceVecs = 16;  // 16-byte vectors of one request's row slice, for every T and HD
constexpr int kDec128Group = kDec128Threads / kDec128SliceVecs;

template <typename T, int HD>
struct Dec128Shape {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int CS = HD / (8 * V);  // channel slices per request
  static_assert((2 * HD / V) / CS == kDec128SliceVecs, "slice of 16 vectors");
};

// Whether decode record rec (request b) can run, and whether it pools.
__device__ __forceinline__ bool dec128_ok(const kvc_plan_d& rec, int64_t b, const DecodeArgs& a) {
  const bool boundary = (rec.seq_len & 127u) == 0u;
  bool ok = rec.write_loc >= 0 && rec.write_loc < a.num_state_rows;
  if (boundary) ok = ok && c128_record_ok(b, 127, rec.read_page_0, a.batch, a.num_state_rows);
  return ok;
}

template <typename T, int HD>
__global__ __launch_bounds__(kDec128Threads) void decode_c128_kernel(DecodeArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int V = Elem<T>::kVec;
  constexpr int CS = Dec128Shape<T, HD>::CS;
  typedef C128Pool<T, HD, kDec128Threads, CS> Pool;
  constexpr int64_t R = 2 * HD;
  constexpr int HDW = HD / CS;
  __shared__ typename Pool::A lds[Pool::kLdsElems];
  const int64_t b0 = (int64_t)(blockIdx.x / CS) * kDec128Group;
  const int cs = blockIdx.x % CS;
  __shared__ int32_t pool_page[kDec128Group];  // read page of a request that pools, else -1
  E* state = static_cast<E*>(a.state);
  const E* input = static_cast<const E*>(a.input);
  {
    // the copy: request b0 + t / 16, vector t % 16 of this slice
    const int j = threadIdx.x / kDec128SliceVecs;
    const int64_t b = b0 + j;
    const int v = threadIdx.x % kDec128SliceVecs;
    int32_t page = -1;
    if (b < a.batch) {
      const kvc_plan_d rec = load_plan_d(a.plan_d + b);
      const bool valid = !plan_d_invalid(rec);
      const bool ok = valid && dec128_ok(rec, b, a);
      const bool boundary = (rec.seq_len & 127u) == 0u;
      if (valid && !ok && cs == 0 && v == 0 && a.status) atomicOr(a.status, KVC_DERR_RECORD);
      if (ok) {
        const int64_t off = (int64_t)(cs * kDec128SliceVecs + v) * V;
        store16_stream(state + (int64_t)rec.write_loc * R + off, load16(input + b * R + off));
      }
      if ((!ok || !boundary) && v < HDW / 4) store_zeros<4>(a.out + b * HD + cs * HDW + v * 4);
      if (ok && boundary) page = rec.read_page_0;
    }
    if (v == 0) pool_page[j] = page;
  }
  __syncthreads();
  // the pools, one boundary request at a time (the loop is uniform over the workgroup)
  for (int j = 0; j < kDec128Group; ++j) {
    const int32_t page = pool_page[j];
    if (page < 0) continue;
    Pool::run(state, input, static_cast<const E*>(a.ape), b0 + j, 127, page, cs, a.out + (b0 + j) * HD, lds);
    __syncthreads();  // the next pool reuses lds
  }
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
    const int64_t grid = (a.batch + kDec128Group - 1) / kDec128Group * Dec128Shape<T, HD>::CS;
    decode_c128_kernel<T, HD><<<(unsigned)grid, kDec128Threads, 0, s>>>(a);
    return hipGetLastError();
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
