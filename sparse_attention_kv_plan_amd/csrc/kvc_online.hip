// kvc_online.hip - the ratio-128 pool with the online state (compressor_v2.py
// page, _use_online_compress: the state of a request is one slot of
// 3 * head_dim values).  A slot holds, per channel, the running maximum m,
// the running sum l = sum exp(t - m) and the running weighted sum
// acc = sum exp(t - m) kv of the request's unfinished block (fp32,
// [slots, 3, hd]: m, l, acc).  The ordinary ratio-128 plans drive it:
//  - compress: a C record pools window entries [buffer_len, 128) from the
//    input and, when buffer_len > 0, merges the slot's partial (the entries
//    before the chunk); out = acc / l;
//  - write: each request's run of W records (its positions after the last
//    completed block, consecutive records of one slot) is folded into the
//    slot, continuing it unless the run starts a block; a workgroup covers 16
//    records and one channel slice and folds the runs that start there;
//  - decode: one token folded per request; a request that closes a block
//    emits acc / l, the others a zero row.
// HBM-bound like the paged pool; a slot is 6 KiB at hd 512 instead of a
// 256 KiB page.
#include "kvc_device.hpp"
#include "kvc_launch.hpp"
#include "kvc_pool.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;
constexpr int kCompressThreads = 512;  // as the paged ratio-128 pool: 8 streams of 16 entries

// one workgroup per C record
template <typename T, int HD>
__global__ __launch_bounds__(kCompressThreads) void compress_online_kernel(OnlineArgs a) {
  typedef typename Elem<T>::storage E;
  typedef C128Pool<T, HD, kCompressThreads> Pool;
  __shared__ typename Pool::A lds[Pool::kLdsElems];
  const int64_t row = blockIdx.x;
  if (row >= a.counts[0] || row >= a.cap) return;
  const kvc_plan_c rec = load_plan_c(a.plan_c + row);
  if (plan_c_invalid(rec)) return;
  const int64_t ragged = rec.ragged_blen & 0xFFFFFFu;
  const int blen = (int)(rec.ragged_blen >> 24);
  const int64_t slot = rec.read_page_0;
  // buffer_len is an 8-bit field; a window holds at most 127 entries before its own token
  const bool ok = blen <= 127 && (blen == 0 || (slot >= 0 && slot < a.num_slots)) && ragged - 127 + blen >= 0 &&
                  ragged < a.num_q;
  if (!ok) {  // uniform over the workgroup
    if (threadIdx.x == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
    return;
  }
  Pool::accumulate_range(static_cast<const E*>(a.input), static_cast<const E*>(a.ape), ragged - 127, 0, blen, 128, 0,
                         lds);
  const float* st = blen > 0 ? a.state + slot * 3 * HD : nullptr;  // slot is read only when blen > 0
  for (int d = threadIdx.x; d < HD; d += kCompressThreads) {
    typename Pool::A M, L, Acc;
    Pool::merged_partial(lds, d, st != nullptr, st ? st[d] : 0.f, st ? st[HD + d] : 0.f, st ? st[2 * HD + d] : 0.f,
                         &M, &L, &Acc);
    __builtin_nontemporal_store((float)(Acc / L), a.out + row * HD + d);
  }
}

// Workgroup (g, cs) covers W records [32 g, 32 g + 32) and channel slice cs:
// it folds every run that starts among its records, one after another, each
// by 16 streams x 8 entries over its slice (one round of loads), so a
// request's run is spread over CS workgroups on different CUs.  The records
// it needs (one before its range to find run heads, 127 after it for run
// lengths) are staged in LDS (both loads of a thread in flight together), and
// a run's old slot values go out with its window.  A request has one run per
// chunk (its positions after the last completed block, at most 127), so most
// workgroups find no head and leave after the staging.  The launch is
// latency-bound: a run takes three dependent trips to memory (records; slot
// and window; the slot's store).  Measured by kernel trace on the mixed
// prefill (64 runs): 13.3 us with 32 records per workgroup, 14.6 us with 16,
// 17 and 20 us with 64 and 128 (more runs in sequence per workgroup); 256
// threads with 4 entries per stream, or the window's loads interleaved with
// the arithmetic, change nothing.  The count is read in the records' round
// trip and every argument at the start (an argument first read inside the
// run loop cost a trip of its own there).
constexpr int kWriteThreads = 128;
constexpr int kWriteGroup = 32;
constexpr int kWriteRecs = kWriteGroup + 128;  // records k0 - 1 .. k0 + 158

template <typename T, int HD>
struct WriteShape {
  static constexpr int CS = HD / (8 * Elem<T>::kVec);  // channel slices
};

__device__ __forceinline__ int64_t slot_of(uint2 r) {
  return (r.x == 0xFFFFFFFFu || (int32_t)r.y < 0) ? -1 : (int32_t)r.y / 128;
}

template <typename T, int HD>
__global__ __launch_bounds__(kWriteThreads) void write_online_kernel(OnlineArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int CS = WriteShape<T, HD>::CS;
  constexpr int HDW = HD / CS;
  static_assert(HDW <= kWriteThreads, "one channel of the slice per thread");
  typedef C128Pool<T, HD, kWriteThreads, CS, 8> Pool;  // a stream's 8 entries in one round of loads
  __shared__ typename Pool::A lds[Pool::kLdsElems];
  __shared__ uint2 recs[kWriteRecs];
  __shared__ int heads[kWriteGroup];
  __shared__ int n_heads, run_end[kWriteThreads / kWave];
  const int64_t k0 = (int64_t)(blockIdx.x / CS) * kWriteGroup;
  const int cs = blockIdx.x % CS;
  in_sgprs(a.state);  // the arguments a run needs, read with the first ones
  in_sgprs(a.input);
  in_sgprs(a.ape);
  in_sgprs(a.num_slots);
  in_sgprs(a.num_q);
  // The count and the records in one round trip: the record loads are
  // unconditional, their indices clamped into the buffer [0, cap) (cap >= 1),
  // and records at or past the count are replaced once both are in.
  const int32_t count = a.counts[1];
  constexpr int kPerThread = (kWriteRecs + kWriteThreads - 1) / kWriteThreads;
  uint2 r[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int64_t k = k0 - 1 + threadIdx.x + u * kWriteThreads;
    r[u] = *reinterpret_cast<const uint2*>(a.plan_w + min(max(k, (int64_t)0), (int64_t)a.cap - 1));
  }
  asm volatile("" ::: "memory");  // every load above goes out before the count is tested
  const int64_t n_w = min((int64_t)count, (int64_t)a.cap);
  if (k0 >= n_w) return;  // uniform: no record of this workgroup's range (n_w >= 1 below)
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int i = threadIdx.x + u * kWriteThreads;
    const int64_t k = k0 - 1 + i;
    if (i < kWriteRecs) recs[i] = (k >= 0 && k < n_w) ? r[u] : make_uint2(0xFFFFFFFFu, 0u);
  }
  if (threadIdx.x == 0) n_heads = 0;
  __syncthreads();
  if (threadIdx.x < kWriteGroup) {
    const uint2 r = recs[threadIdx.x + 1];
    if (r.x != 0xFFFFFFFFu && (slot_of(recs[threadIdx.x]) != slot_of(r) || slot_of(r) < 0))
      heads[atomicAdd(&n_heads, 1)] = (int)threadIdx.x;  // runs touch distinct slots: their order is free
  }
  __syncthreads();
  const int nh = n_heads;
  for (int h = 0; h < nh; ++h) {
    const int j0 = heads[h] + 1;  // the head's index in recs
    const uint2 head = recs[j0];
    const int64_t loc = (int32_t)head.y, ragged = head.x;
    const int64_t slot = loc >= 0 ? loc / 128 : -1;
    const int p0 = loc >= 0 ? (int)(loc % 128) : 0;
    if (loc < 0 || slot >= a.num_slots || ragged >= a.num_q) {  // uniform over the workgroup
      if (cs == 0 && threadIdx.x == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
      continue;
    }
    // the slot's old values go out before the run's length is known
    float* st = a.state + slot * 3 * HD + cs * HDW;
    const int d = threadIdx.x;
    const bool cont = p0 > 0;  // the block started before this chunk: continue the slot
    float m0 = 0.f, l0 = 0.f, a0 = 0.f;
    if (cont && d < HDW) {
      m0 = st[d];
      l0 = st[HD + d];
      a0 = st[2 * HD + d];
    }
    // run length: records j0 .. j0+n-1 continue the head's slot, rows and
    // positions; n is the first record that breaks the run (or the block's
    // end), found by a ballot in each wave and the waves' minimum.  (An LDS
    // atomicMin here became a scalar loop over the active lanes, 1.4 us.)
    bool brk = false;
    if (threadIdx.x > 0 && threadIdx.x < 128 - p0) {
      const uint2 r = recs[j0 + threadIdx.x];
      brk = !(r.x == (uint32_t)(ragged + threadIdx.x) && (int64_t)(int32_t)r.y == loc + threadIdx.x);
    }
    const unsigned long long breaks = __ballot(brk);
    if (threadIdx.x % kWave == 0)
      run_end[threadIdx.x / kWave] = breaks ? (int)(threadIdx.x + __ffsll(breaks) - 1) : 128 - p0;
    __syncthreads();
    int n = run_end[0];
#pragma unroll
    for (int w = 1; w < kWriteThreads / kWave; ++w) n = min(n, run_end[w]);
    __syncthreads();  // every thread has read run_end before the next run writes it
    if (ragged + n > a.num_q) {  // uniform
      if (cs == 0 && threadIdx.x == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
      continue;
    }
    // entries e in [p0, p0 + n) of the block: input row ragged - p0 + e, ape
    // row e.  (Issuing the window before n is known means loading the rows
    // past the run too, which costs more than the wait it saves.)
    Pool::accumulate_range(static_cast<const E*>(a.input), static_cast<const E*>(a.ape), ragged - p0, 0, p0, p0 + n,
                           cs, lds);
    if (d < HDW) {
      typename Pool::A M, L, Acc;  // M is already a value an fp32 slot holds exactly
      Pool::merged_partial(lds, d, cont, m0, l0, a0, &M, &L, &Acc);
      st[d] = (float)M;
      st[HD + d] = (float)L;
      st[2 * HD + d] = (float)Acc;
    }
    __syncthreads();  // lds is reused by the next run
  }
}

// one thread per V channels of one request
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void decode_online_kernel(OnlineArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int V = Elem<T>::kVec;
  constexpr int kLanes = HD / V;
  constexpr int64_t R = 2 * HD;
  const int64_t b = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kLanes;
  const int c = (threadIdx.x % kLanes) * V;
  if (b >= a.cap) return;
  float* out = a.out + b * HD + c;
  const kvc_plan_d rec = load_plan_d(a.plan_d + b);
  if (plan_d_invalid(rec)) {
    store_zeros<V>(out);
    return;
  }
  const int64_t slot = rec.read_page_0;
  if (slot < 0 || slot >= a.num_slots) {
    if (c == 0 && a.status) atomicOr(a.status, KVC_DERR_RECORD);
    store_zeros<V>(out);
    return;
  }
  const uint32_t pos = rec.seq_len - 1;
  const bool fresh = pos % 128u == 0u;
  const E* in = static_cast<const E*>(a.input) + b * R;
  float kv[V], t[V], ap[V];
  widen16<T>(load16(in + c), kv);
  widen16<T>(load16(in + HD + c), t);
  widen16<T>(load16(static_cast<const E*>(a.ape) + (int64_t)(pos % 128u) * HD + c), ap);
  float* st = a.state + slot * 3 * HD + c;
  float m[V], l[V], acc[V];
  if (!fresh) {
#pragma unroll
    for (int v = 0; v < V; v += 4) {
      widen16<float>(load16(st + v), m + v);
      widen16<float>(load16(st + HD + v), l + v);
      widen16<float>(load16(st + 2 * HD + v), acc + v);
    }
  }
  // the fold in the pool's arithmetic type (fp64 for fp32 inputs); the new
  // maximum is taken as the fp32 value the slot keeps, so the stored sums
  // are relative to exactly the stored maximum
  typedef typename Acc<T>::type A;
  const bool closes = rec.seq_len % 128u == 0u;
  float o[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const A tv = (A)t[v] + (A)ap[v];
    A nm, lv, av;
    if (fresh) {
      nm = slot_shift(tv);
      lv = softmax_exp(tv - nm);  // 1 unless the shift rounded tv
      av = lv * (A)kv[v];
    } else {
      nm = slot_shift(amax((A)m[v], tv));
      const A f = softmax_exp((A)m[v] - nm), w = softmax_exp(tv - nm);
      lv = (A)l[v] * f + w;
      av = afma((A)acc[v], f, w * (A)kv[v]);
    }
    m[v] = (float)nm;
    l[v] = (float)lv;
    acc[v] = (float)av;
    o[v] = closes ? (float)(av / lv) : 0.f;
  }
  store_floats<V>(st, m);
  store_floats<V>(st + HD, l);
  store_floats<V>(st + 2 * HD, acc);
  if (closes) {
    store_floats<V, true>(out, o);
  } else {
    store_zeros<V>(out);
  }
}

template <template <typename, int> class K>
struct Launch {
  template <typename T, int HD>
  static hipError_t go(const OnlineArgs& a, int64_t grid, hipStream_t s) {
    K<T, HD>::launch(a, grid, s);
    return hipGetLastError();
  }
};

#define KVC_ONLINE_KERNEL(NAME, KERNEL, NT)                                              \
  template <typename T, int HD>                                                          \
  struct NAME {                                                                          \
    static void launch(const OnlineArgs& a, int64_t grid, hipStream_t s) {               \
      KERNEL<T, HD><<<(unsigned)grid, NT, 0, s>>>(a);                                    \
    }                                                                                    \
  };
KVC_ONLINE_KERNEL(CompressK, compress_online_kernel, kCompressThreads)
template <typename T, int HD>
struct WriteK {
  static void launch(const OnlineArgs& a, int64_t grid, hipStream_t s) {
    write_online_kernel<T, HD><<<(unsigned)(grid * WriteShape<T, HD>::CS), kWriteThreads, 0, s>>>(a);
  }
};
KVC_ONLINE_KERNEL(DecodeK, decode_online_kernel, kThreads)
#undef KVC_ONLINE_KERNEL

template <template <typename, int> class K>
hipError_t dispatch(kvc_dtype dtype, int hd, const OnlineArgs& a, int64_t grid, hipStream_t stream) {
  typedef Launch<K> L;
  if (dtype == KVC_BF16) {
    if (hd == 128) return L::template go<Bf16, 128>(a, grid, stream);
    if (hd == 256) return L::template go<Bf16, 256>(a, grid, stream);
    return L::template go<Bf16, 512>(a, grid, stream);
  }
  if (hd == 128) return L::template go<float, 128>(a, grid, stream);
  if (hd == 256) return L::template go<float, 256>(a, grid, stream);
  return L::template go<float, 512>(a, grid, stream);
}

}  // namespace

hipError_t launch_compress_online(kvc_dtype dtype, int head_dim, const OnlineArgs& a, hipStream_t stream) {
  return dispatch<CompressK>(dtype, head_dim, a, a.cap, stream);
}

hipError_t launch_write_online(kvc_dtype dtype, int head_dim, const OnlineArgs& a, hipStream_t stream) {
  return dispatch<WriteK>(dtype, head_dim, a, ((int64_t)a.cap + kWriteGroup - 1) / kWriteGroup, stream);
}

hipError_t launch_decode_online(kvc_dtype dtype, int head_dim, const OnlineArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.cap * (head_dim / (dtype == KVC_BF16 ? 8 : 4));
  return dispatch<DecodeK>(dtype, head_dim, a, (threads + kThreads - 1) / kThreads, stream);
}

}  // namespace kvc
