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
//    slot, continuing it unless the run starts a block; a workgroup covers 32
//    records and one channel slice and folds the runs that start there, or,
//    given the prefill planner's run list, one request's run;
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

// Workgroup (g, cs) covers W records [32 g, 32 g + 32) and channel slice cs,
// and folds every run that starts among its records.  The records it needs
// (one before its range to find run heads, 127 after it for run lengths) are
// staged in LDS together with the count (one round trip); a ballot per wave
// marks the records that continue no run, and each head's length is the
// distance to the next such record.  Runs of up to 8 records (a few tokens
// per request per chunk, as when several tokens are verified at once) are
// folded side by side, 8 threads each (one 16-byte vector of the slice per
// thread, the run's entries in turn); longer runs one after another, each by
// 16 streams x 8 entries over the slice (one round of loads) merged in LDS,
// so a long run is spread over CS workgroups on different CUs.  A request has
// one run per chunk (its positions after the last completed block, at most
// 127), so most workgroups find no head and leave after the staging.
// Measured by kernel trace on the mixed prefill (64 runs of 1-127 records):
// 13.3 us with 32 records per workgroup, 14.6 us with 16, 17 and 20 us with
// 64 and 128; 256 threads with 4 entries per stream, or the window's loads
// interleaved with the arithmetic, change nothing.
constexpr int kWriteThreads = 128;
constexpr int kWriteGroup = 32;
constexpr int kWriteRecs = kWriteGroup + 128;  // records k0 - 1 .. k0 + 158
constexpr int kShortRun = 8;                   // runs folded side by side
constexpr int kShortChunk = 4;                 // entries per round of loads in a short run

template <typename T, int HD>
struct WriteShape {
  static constexpr int CS = HD / (8 * Elem<T>::kVec);  // channel slices
};

__device__ __forceinline__ int64_t slot_of(uint2 r) {
  return (r.x == 0xFFFFFFFFu || (int32_t)r.y < 0) ? -1 : (int32_t)r.y / 128;
}

// Whether record r continues the run of the record q before it: the next
// ragged row and the next state row of the same block.
__device__ __forceinline__ bool continues(uint2 q, uint2 r) {
  return r.x != 0xFFFFFFFFu && r.x == q.x + 1u && (int32_t)r.y == (int32_t)q.y + 1 && ((int32_t)r.y & 127) != 0;
}

// A run of n <= kShortRun records folded by one thread over V channels [c, c + V)
// of its slot: the block's entries p0 .. p0 + n - 1 (input rows ragged ..,
// ape rows p0 ..), onto the slot's partial when the block began earlier.
template <typename T, int HD>
__device__ __forceinline__ void fold_short_run(const OnlineArgs& a, int64_t ragged, int64_t slot, int p0, int n,
                                               int c) {
  typedef typename Elem<T>::storage E;
  typedef typename Acc<T>::type A;
  constexpr int V = Elem<T>::kVec;
  constexpr int64_t R = 2 * HD;
  const E* input = static_cast<const E*>(a.input);
  const E* ape = static_cast<const E*>(a.ape);
  float* st = a.state + slot * 3 * HD + c;
  A m[V], l[V], acc[V];
  if (p0 > 0) {  // continue the slot
    float m0[V], l0[V], a0[V];
#pragma unroll
    for (int v = 0; v < V; v += 4) {
      widen16<float>(load16(st + v), m0 + v);
      widen16<float>(load16(st + HD + v), l0 + v);
      widen16<float>(load16(st + 2 * HD + v), a0 + v);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      m[v] = m0[v];
      l[v] = l0[v];
      acc[v] = a0[v];
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      m[v] = -INFINITY;
      l[v] = 0;
      acc[v] = 0;
    }
  }
  for (int e0 = 0; e0 < n; e0 += kShortChunk) {
    u32x4 kv_raw[kShortChunk], sc_raw[kShortChunk], ap_raw[kShortChunk];
#pragma unroll
    for (int u = 0; u < kShortChunk; ++u) {  // entries past the run load its last one (not used)
      const int e = min(e0 + u, n - 1);
      kv_raw[u] = load16_stream(input + (ragged + e) * R + c);
      sc_raw[u] = load16_stream(input + (ragged + e) * R + HD + c);
      ap_raw[u] = load16(ape + (int64_t)(p0 + e) * HD + c);
    }
#pragma unroll
    for (int u = 0; u < kShortChunk; ++u) {
      if (e0 + u >= n) break;
      float kv[V], sc[V], ap[V];
      widen16<T>(kv_raw[u], kv);
      widen16<T>(sc_raw[u], sc);
      widen16<T>(ap_raw[u], ap);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const A t = (A)sc[v] + (A)ap[v];
        const A nm = amax(m[v], t);
        const A f = softmax_exp(m[v] - nm), w = softmax_exp(t - nm);  // f = 0 on a fresh block
        l[v] = afma(l[v], f, w);
        acc[v] = afma(acc[v], f, w * (A)kv[v]);
        m[v] = nm;
      }
    }
  }
  // stored relative to the fp32 value the slot keeps as its maximum
  float mo[V], lo[V], ao[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const A M = slot_shift(m[v]);
    const A f = softmax_exp(m[v] - M);
    mo[v] = (float)M;
    lo[v] = (float)(l[v] * f);
    ao[v] = (float)(acc[v] * f);
  }
  store_floats<V>(st, mo);
  store_floats<V>(st + HD, lo);
  store_floats<V>(st + 2 * HD, ao);
}

template <typename T, int HD>
__global__ __launch_bounds__(kWriteThreads) void write_online_kernel(OnlineArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int V = Elem<T>::kVec;
  constexpr int CS = WriteShape<T, HD>::CS;
  constexpr int HDW = HD / CS;
  constexpr int kVecs = HDW / V;                      // vectors of a slice (8)
  constexpr int kSide = kWriteThreads / kVecs;        // short runs folded at once (16)
  constexpr int kWords = 2 * kWriteThreads / kWave;   // break-mask words over 256 record places
  static_assert(HDW <= kWriteThreads && kWriteRecs <= 2 * kWriteThreads, "write shape");
  typedef C128Pool<T, HD, kWriteThreads, CS, 8> Pool;  // a stream's 8 entries in one round of loads
  __shared__ typename Pool::A lds[Pool::kLdsElems];
  __shared__ uint2 recs[kWriteRecs];
  __shared__ unsigned long long stop[kWords];  // bit k of word w: record 64 w + k continues no run
  __shared__ int run_j[2][kWriteGroup], run_n[2][kWriteGroup];  // [0] short runs, [1] long: head in recs, length
  __shared__ int n_runs[2];
  const int64_t k0 = (int64_t)(blockIdx.x / CS) * kWriteGroup;
  const int cs = blockIdx.x % CS;
  const int t = threadIdx.x;
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
    const int64_t k = k0 - 1 + t + u * kWriteThreads;
    r[u] = *reinterpret_cast<const uint2*>(a.plan_w + min(max(k, (int64_t)0), (int64_t)a.cap - 1));
  }
  asm volatile("" ::: "memory");  // every load above goes out before the count is tested
  const int64_t n_w = min((int64_t)count, (int64_t)a.cap);
  if (k0 >= n_w) return;  // uniform: no record of this workgroup's range (n_w >= 1 below)
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int i = t + u * kWriteThreads;
    const int64_t k = k0 - 1 + i;
    if (i < kWriteRecs) recs[i] = (k >= 0 && k < n_w) ? r[u] : make_uint2(0xFFFFFFFFu, 0u);
  }
  if (t < 2) n_runs[t] = 0;
  __syncthreads();
  // which records continue no run (a ballot per wave; places past the staged records count as stops)
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int k = p * kWriteThreads + t;
    const bool cont = k >= 1 && k < kWriteRecs && continues(recs[k - 1], recs[k]);
    const unsigned long long m = __ballot(!cont);
    if (t % kWave == 0) stop[p * (kWriteThreads / kWave) + t / kWave] = m;
  }
  __syncthreads();
  if (t < kWriteGroup) {
    const int j0 = t + 1;  // a head is a record whose slot differs from the one before
    const uint2 head = recs[j0];
    if (head.x != 0xFFFFFFFFu && (slot_of(recs[t]) != slot_of(head) || slot_of(head) < 0)) {
      // its run: records j0 .. j0+n-1, up to the next record that continues no run
      int k = j0 + 1;
      while (k < kWords * kWave) {  // ends by the staged records' end: every place past it stops
        const unsigned long long m = stop[k >> 6] >> (k & 63);
        if (m) {
          k += __ffsll(m) - 1;
          break;
        }
        k = ((k >> 6) + 1) << 6;
      }
      const int n = k - j0;
      const int64_t loc = (int32_t)head.y, ragged = head.x;
      if (loc < 0 || loc / 128 >= a.num_slots || ragged + n > a.num_q) {
        if (cs == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
      } else {
        const int kind = n > kShortRun;
        const int i = atomicAdd(&n_runs[kind], 1);  // runs touch distinct slots: their order is free
        run_j[kind][i] = j0;
        run_n[kind][i] = n;
      }
    }
  }
  __syncthreads();
  // short runs side by side: thread t folds vector t % kVecs of run t / kVecs
  const int ns = n_runs[0];
  for (int i0 = 0; i0 < ns; i0 += kSide) {
    const int i = i0 + t / kVecs;
    if (i < ns) {
      const uint2 head = recs[run_j[0][i]];
      const int64_t loc = (int32_t)head.y;
      fold_short_run<T, HD>(a, head.x, loc / 128, (int)(loc % 128), run_n[0][i], cs * HDW + (t % kVecs) * V);
    }
  }
  // long runs one after another, each by the whole workgroup
  const int nl = n_runs[1];
  for (int h = 0; h < nl; ++h) {
    const int j0 = run_j[1][h], n = run_n[1][h];
    const uint2 head = recs[j0];
    const int64_t loc = (int32_t)head.y, ragged = head.x;
    const int64_t slot = loc / 128;
    const int p0 = (int)(loc % 128);
    float* st = a.state + slot * 3 * HD + cs * HDW;
    const int d = t;
    const bool cont = p0 > 0;  // the block started before this chunk: continue the slot
    float m0 = 0.f, l0 = 0.f, a0 = 0.f;
    if (cont && d < HDW) {
      m0 = st[d];
      l0 = st[HD + d];
      a0 = st[2 * HD + d];
    }
    // entries e in [p0, p0 + n) of the block: input row ragged - p0 + e, ape row e
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

// The same fold driven by the planner's run list: workgroup (b, cs) folds
// request b's run (input rows ragged .., positions p0 .. p0 + n - 1 of slot
// loc / 128, p0 = loc % 128) over channel slice cs, by the same two paths as
// above (a run of up to kShortRun records by one thread per vector of the
// slice, a longer one by the whole workgroup), so the slots come out bit for
// bit as with the scan.  One round trip for the entry and the W count (0
// after a planner error), then the run's entries and the slot's partial; no
// staging or search.
template <typename T, int HD>
__global__ __launch_bounds__(kWriteThreads) void write_online_runs_kernel(OnlineArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int CS = WriteShape<T, HD>::CS;
  constexpr int HDW = HD / CS;
  typedef C128Pool<T, HD, kWriteThreads, CS, 8> Pool;
  __shared__ typename Pool::A lds[Pool::kLdsElems];
  const int64_t b = blockIdx.x / CS;
  const int cs = blockIdx.x % CS;
  const int d = threadIdx.x;
  const int4 run = *reinterpret_cast<const int4*>(a.runs + 4 * b);
  const int32_t n_w = a.counts[1];
  const int n = run.z;
  if (n == 0 || n_w <= 0) return;  // uniform over the workgroup
  const int64_t ragged = run.x, loc = run.y;
  const int64_t slot = loc / 128;
  const int p0 = (int)(loc % 128);
  if (loc < 0 || slot >= a.num_slots || n < 0 || p0 + n > 128 || ragged < 0 || ragged + n > a.num_q) {
    if (cs == 0 && d == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
    return;
  }
  if (n <= kShortRun) {
    constexpr int kVecs = HDW / Elem<T>::kVec;
    if (d < kVecs) fold_short_run<T, HD>(a, ragged, slot, p0, n, cs * HDW + d * Elem<T>::kVec);
    return;
  }
  float* st = a.state + slot * 3 * HD + cs * HDW;
  const bool cont = p0 > 0;  // the block started before this chunk: continue the slot
  float m0 = 0.f, l0 = 0.f, a0 = 0.f;
  if (cont && d < HDW) {
    m0 = st[d];
    l0 = st[HD + d];
    a0 = st[2 * HD + d];
  }
  Pool::accumulate_range(static_cast<const E*>(a.input), static_cast<const E*>(a.ape), ragged - p0, 0, p0, p0 + n, cs,
                         lds);
  if (d < HDW) {
    typename Pool::A M, L, Acc;
    Pool::merged_partial(lds, d, cont, m0, l0, a0, &M, &L, &Acc);
    st[d] = (float)M;
    st[HD + d] = (float)L;
    st[2 * HD + d] = (float)Acc;
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
    if (a.runs != nullptr) {
      write_online_runs_kernel<T, HD><<<(unsigned)(a.batch * WriteShape<T, HD>::CS), kWriteThreads, 0, s>>>(a);
    } else {
      write_online_kernel<T, HD><<<(unsigned)(grid * WriteShape<T, HD>::CS), kWriteThreads, 0, s>>>(a);
    }
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
