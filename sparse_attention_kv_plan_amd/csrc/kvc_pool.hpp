// kvc_pool.hpp - the softmax pool over a window (c4.cuh page, c4_forward;
// compressor_v2.py page, _c128_compress_prefill_compress_kernel), shared by
// the prefill compress and the fused decode kernels.
//
// For every channel d of a compressed row:
//   t_i = score_i[d] + ape[i][d]
//   out = sum_i exp(t_i - m) kv_i[d] / sum_i exp(t_i - m),   m = max_i t_i
// A lane owns one 16-byte group of channels (8 bf16 or 4 fp32) and keeps the
// maximum, the sum of weights and the weighted sum in registers of the
// pool's arithmetic type (Acc<T>: fp32 for bf16 inputs, where the weight is
// 2^((t - m) log2 e) on the hardware exp unit; fp64 for fp32 inputs).
#pragma once

#include "kvc_device.hpp"

namespace kvc {

// ---------------------------------------------------------------------------
// ratio 4: 8 window entries, one lane group per row
// ---------------------------------------------------------------------------
//
// Entry i of the row closing at seq_len comes from the state when
// i < blen (rows rp0*4 + i for i < 4, rp1*4 + i - 4 otherwise), else from
// input row ragged - 7 + i.  Entries 0..3 (the previous block) use the
// |kv overlap| and |score overlap| quarters of their row, entries 4..7 the
// |kv| and |score| quarters.  FIRST = 4 drops the entries before the start of
// the sequence (the first block); they are not loaded at all.  pre() runs
// right after the window's loads are issued, so a caller's own loads overlap
// them.
struct NoPre {
  __device__ void operator()() const {}
};

// The pool of one lane's channels [c, c + V) from the window's raw kv and
// score vectors (entries FIRST..7); ape_of(i) gives entry i's ape vector.
template <typename T, int FIRST, typename ApeOf>
__device__ __forceinline__ void c4_pool_math(const u32x4* kv_raw, const u32x4* sc_raw, const ApeOf& ape_of,
                                             float* res) {
  typedef typename Acc<T>::type A;
  constexpr int V = Elem<T>::kVec;
  A t[8][V];
#pragma unroll
  for (int i = FIRST; i < 8; ++i) {
    float sc[V], a[V];
    widen16<T>(sc_raw[i], sc);
    widen16<T>(ape_of(i), a);
#pragma unroll
    for (int v = 0; v < V; ++v) t[i][v] = (A)sc[v] + (A)a[v];
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    A m = t[FIRST][v];
#pragma unroll
    for (int i = FIRST + 1; i < 8; ++i) m = amax(m, t[i][v]);
    A den = 0, num = 0;
#pragma unroll
    for (int i = FIRST; i < 8; ++i) {
      float kv[V];
      widen16<T>(kv_raw[i], kv);  // widened per channel: keeps the raw 16-byte vectors as the only live copy
      const A w = softmax_exp(t[i][v] - m);
      den += w;
      num = afma(w, (A)kv[v], num);
    }
    res[v] = (float)(num / den);
  }
}

template <typename T, int HD, int FIRST, typename Pre = NoPre>
__device__ __forceinline__ void c4_pool(const typename Elem<T>::storage* __restrict__ state,
                                        const typename Elem<T>::storage* __restrict__ input,
                                        const typename Elem<T>::storage* __restrict__ ape, int64_t ragged, int blen,
                                        int64_t rp0, int64_t rp1, int c, float* res, const Pre& pre = Pre()) {
  constexpr int64_t R = 4 * HD;
  // all kv / score loads of the window are issued before any use
  u32x4 kv_raw[8], sc_raw[8];
#pragma unroll
  for (int i = FIRST; i < 8; ++i) {
    const int64_t srow = (i < 4) ? rp0 * 4 + i : rp1 * 4 + (i - 4);
    const typename Elem<T>::storage* row = (i < blen) ? state + srow * R : input + (ragged - 7 + i) * R;
    kv_raw[i] = load16_stream(row + ((i < 4) ? 0 : HD) + c);
    sc_raw[i] = load16_stream(row + ((i < 4) ? 2 * HD : 3 * HD) + c);
  }
  pre();
  // ape is reused by every row: cached loads, issued as the arithmetic needs them
  c4_pool_math<T, FIRST>(kv_raw, sc_raw, [&](int i) { return load16(ape + i * HD + c); }, res);
}

// The decode window: entries FIRST..6 from the state (pages rp0, rp1), entry 7
// (the new token) from the lane's own copy of its input row, q = the row's
// four quarters |kv overlap|kv|score overlap|score| at channels [c, c + V);
// the ape rows go out with the window's loads.
template <typename T, int HD, int FIRST>
__device__ __forceinline__ void c4_decode_window(const typename Elem<T>::storage* __restrict__ state,
                                                 const typename Elem<T>::storage* __restrict__ ape, int64_t rp0,
                                                 int64_t rp1, int c, const u32x4* q, u32x4* kv_raw, u32x4* sc_raw,
                                                 u32x4* ap_raw) {
  constexpr int64_t R = 4 * HD;
#pragma unroll
  for (int i = FIRST; i < 7; ++i) {
    const typename Elem<T>::storage* row = state + ((i < 4) ? rp0 * 4 + i : rp1 * 4 + (i - 4)) * R;
    kv_raw[i] = load16_stream(row + ((i < 4) ? 0 : HD) + c);
    sc_raw[i] = load16_stream(row + ((i < 4) ? 2 * HD : 3 * HD) + c);
  }
#pragma unroll
  for (int i = FIRST; i < 8; ++i) ap_raw[i] = load16(ape + i * HD + c);
  kv_raw[7] = q[1];
  sc_raw[7] = q[3];
}

// Rows the ratio-4 window of a record reads, checked against the buffers.
// Nearly every record reads the input only (blen = 0); its check is two
// compares, taken before the general form (whose 64-bit page arithmetic sits
// between the record load and the window loads, and cost ~4% of the pool).
__device__ __forceinline__ bool c4_record_ok(int64_t ragged, int blen, int64_t rp0, int64_t rp1, int first,
                                             int64_t num_q, int64_t num_state_rows) {
  if (blen == 0) return ragged - 7 + first >= 0 && ragged < num_q;
  const int s_hi = blen < 8 ? blen : 8;
  const int lo0 = first, hi0 = s_hi < 4 ? s_hi : 4;
  const int lo1 = first > 4 ? first : 4, hi1 = s_hi;
  const int in_lo = first > s_hi ? first : s_hi;
  bool ok = rows_ok(rp0 * 4 + lo0, rp0 * 4 + hi0, num_state_rows);
  ok = ok && rows_ok(rp1 * 4 + (lo1 - 4), rp1 * 4 + (hi1 - 4), num_state_rows);
  ok = ok && rows_ok(ragged - 7 + in_lo, ragged + 1, num_q);
  return ok;
}

// ---------------------------------------------------------------------------
// ratio 128: 128 window entries, one workgroup per row
// ---------------------------------------------------------------------------
//
// The workgroup's NT threads form S = NT / (HDW / V) streams over a slice of
// HDW = HD / CS channels (CS workgroups share a row when CS > 1; the softmax is
// per channel, so the slices need no merge).  Stream s owns entries s, s + S,
// s + 2S, ... (at any moment the streams read adjacent rows) and runs an online
// softmax over them in chunks of U entries, all loads of a chunk issued before
// any use.  U = 4 keeps the streams under 128 VGPRs (4 waves per SIMD).  The S
// partial (max, sum, weighted sum) triples are merged in LDS.
// Entry i is state row rp0*128 + i when i < blen, else input row
// ragged - 127 + i.
//
// Wave priority by progress: when a stream runs 4 or more chunks, its wave
// sets its issue priority from 3 (first quarter of its chunks) down to 0 (last
// quarter).  The waves sharing a SIMD belong to different rows; with equal
// priority the oldest wave wins the issue slots, so rows dispatched first
// finish far ahead of the rest and the last rows run with too few loads in
// flight to keep HBM busy.  Serving the waves that are behind first evens the
// rows out (on MI355X, 6% less time for the ratio-128 prefill pool).
__device__ __forceinline__ void progress_priority(int quarter) {
  if (quarter == 0) {
    __builtin_amdgcn_s_setprio(3);
  } else if (quarter == 1) {
    __builtin_amdgcn_s_setprio(2);
  } else if (quarter == 2) {
    __builtin_amdgcn_s_setprio(1);
  } else {
    __builtin_amdgcn_s_setprio(0);
  }
}

template <typename T, int HD, int NT, int CS = 1, int U = 4>
struct C128Pool {
  typedef typename Acc<T>::type A;        // the arithmetic type; LDS partials are kept in it too
  static constexpr int V = Elem<T>::kVec;
  static constexpr int HDW = HD / CS;     // channels of this workgroup
  static constexpr int kLanes = HDW / V;  // lanes per stream
  static constexpr int S = NT / kLanes;   // streams per workgroup
  static constexpr int PER = 128 / S;     // entries per stream
  static constexpr int kLdsElems = 3 * S * HDW;
  static constexpr bool kPrio = PER / U >= 4;  // priority by progress (see above)
  static_assert(HD % CS == 0 && NT % kLanes == 0 && 128 % S == 0 && PER % U == 0, "bad c128 pool shape");

  // Every stream's partial (max, sum, weighted sum) per channel of the slice,
  // left in lds (kLdsElems) behind a workgroup barrier.
  __device__ __forceinline__ static void accumulate(const typename Elem<T>::storage* __restrict__ state,
                                                    const typename Elem<T>::storage* __restrict__ input,
                                                    const typename Elem<T>::storage* __restrict__ ape,
                                                    int64_t ragged, int blen, int64_t rp0, int cs, A* lds) {
    constexpr int64_t R = 2 * HD;
    const int sid = threadIdx.x / kLanes;
    const int cl = (threadIdx.x % kLanes) * V;  // channel inside the slice
    const int c = cs * HDW + cl;
    A m[V], l[V], acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      m[v] = -INFINITY;
      l[v] = 0;
      acc[v] = 0;
    }
    for (int k0 = 0; k0 < PER; k0 += U) {
      if constexpr (kPrio) progress_priority(k0 * 4 / PER);
      u32x4 kv_raw[U], sc_raw[U], ap_raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = sid + S * (k0 + u);
        const typename Elem<T>::storage* row =
            (i < blen) ? state + (rp0 * 128 + i) * R : input + (ragged - 127 + i) * R;
        kv_raw[u] = load16_stream(row + c);
        sc_raw[u] = load16_stream(row + HD + c);
        ap_raw[u] = load16(ape + (int64_t)i * HD + c);
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        A t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float sc[V], ap[V];
          widen16<T>(sc_raw[u], sc);
          widen16<T>(ap_raw[u], ap);
          t[u] = (A)sc[v] + (A)ap[v];
        }
        A cm = t[0];
#pragma unroll
        for (int u = 1; u < U; ++u) cm = amax(cm, t[u]);
        const A nm = amax(m[v], cm);
        const A scale = softmax_exp(m[v] - nm);  // 0 on the first chunk (m = -inf)
        A lv = l[v] * scale, av = acc[v] * scale;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float kv[V];
          widen16<T>(kv_raw[u], kv);
          const A w = softmax_exp(t[u] - nm);
          lv += w;
          av = afma(w, (A)kv[v], av);
        }
        m[v] = nm;
        l[v] = lv;
        acc[v] = av;
      }
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    A* lm = lds;
    A* ll = lds + S * HDW;
    A* la = lds + 2 * S * HDW;
    store_acc<V>(lm + sid * HDW + cl, m);
    store_acc<V>(ll + sid * HDW + cl, l);
    store_acc<V>(la + sid * HDW + cl, acc);
    __syncthreads();
  }

  // The online-state form: entry e (0..127) is input row row0 + e with ape row
  // ape0 + e, and only entries lo <= e < hi take part (0 <= lo < hi <= 128).
  // Every entry is loaded (the load count stays fixed): an entry out of
  // [lo, hi) loads the nearest entry in range (the same few rows, so cache
  // hits) and is weighed 0.  A chunk whose entries are all out of range
  // leaves its stream's partial untouched.
  struct Chunk {
    u32x4 kv[U], sc[U], ap[U];
  };

  // the loads of chunk k0 (entries sid + S * (k0 + u) of this thread's stream)
  __device__ __forceinline__ static void load_chunk(const typename Elem<T>::storage* __restrict__ input,
                                                    const typename Elem<T>::storage* __restrict__ ape, int64_t row0,
                                                    int ape0, int lo, int hi, int k0, int cs, Chunk& ch) {
    constexpr int64_t R = 2 * HD;
    const int sid = threadIdx.x / kLanes;
    const int c = cs * HDW + (threadIdx.x % kLanes) * V;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = min(max(sid + S * (k0 + u), lo), hi - 1);
      const typename Elem<T>::storage* row = input + (row0 + e) * R;
      ch.kv[u] = load16_stream(row + c);
      ch.sc[u] = load16_stream(row + HD + c);
      ch.ap[u] = load16(ape + (int64_t)(ape0 + e) * HD + c);
    }
  }

  // folds chunk k0 into the running (m, l, acc) of this thread's channels
  __device__ __forceinline__ static void fold_chunk(const Chunk& ch, int lo, int hi, int k0, A* m, A* l, A* acc) {
    const int sid = threadIdx.x / kLanes;
    bool in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = sid + S * (k0 + u);
      in[u] = e >= lo && e < hi;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      A t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float sc[V], ap[V];
        widen16<T>(ch.sc[u], sc);
        widen16<T>(ch.ap[u], ap);
        t[u] = in[u] ? (A)sc[v] + (A)ap[v] : (A)-INFINITY;
      }
      A cm = t[0];
#pragma unroll
      for (int u = 1; u < U; ++u) cm = amax(cm, t[u]);
      const A nm = amax(m[v], cm);
      const A sh = nm == (A)-INFINITY ? (A)0 : nm;  // nothing in range yet: keep the zeros
      const A scale = softmax_exp(m[v] - sh);
      A lv = l[v] * scale, av = acc[v] * scale;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kv[V];
        widen16<T>(ch.kv[u], kv);
        const A w = softmax_exp(t[u] - sh);
        lv += w;
        av = afma(w, in[u] ? (A)kv[v] : (A)0, av);
      }
      m[v] = nm;
      l[v] = lv;
      acc[v] = av;
    }
  }

  // this thread's partial into lds, then a workgroup barrier
  __device__ __forceinline__ static void store_partial(const A* m, const A* l, const A* acc, A* lds) {
    const int sid = threadIdx.x / kLanes;
    const int cl = (threadIdx.x % kLanes) * V;
    store_acc<V>(lds + sid * HDW + cl, m);
    store_acc<V>(lds + S * HDW + sid * HDW + cl, l);
    store_acc<V>(lds + 2 * S * HDW + sid * HDW + cl, acc);
    __syncthreads();
  }

  __device__ __forceinline__ static void accumulate_range(const typename Elem<T>::storage* __restrict__ input,
                                                          const typename Elem<T>::storage* __restrict__ ape,
                                                          int64_t row0, int ape0, int lo, int hi, int cs, A* lds) {
    A m[V], l[V], acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      m[v] = -INFINITY;
      l[v] = 0;
      acc[v] = 0;
    }
    for (int k0 = 0; k0 < PER; k0 += U) {
      if constexpr (kPrio) progress_priority(k0 * 4 / PER);
      Chunk ch;
      load_chunk(input, ape, row0, ape0, lo, hi, k0, cs, ch);
      // every load of the chunk goes out before the first use (the scheduler
      // otherwise interleaves them with the arithmetic of earlier entries)
      __builtin_amdgcn_sched_barrier(0);
      fold_chunk(ch, lo, hi, k0, m, l, acc);
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    store_partial(m, l, acc, lds);
  }

  // The merged (max, sum, weighted sum) of channel d of the slice, with an
  // extra partial (m0, l0, a0) folded in when `extra` (an online slot).  The
  // sums are taken relative to slot_shift(max), the value an fp32 slot can
  // hold, which is returned as the maximum.
  __device__ __forceinline__ static void merged_partial(const A* lds, int d, bool extra, float m0, float l0,
                                                        float a0, A* M_out, A* L_out, A* A_out) {
    const A* lm = lds;
    const A* ll = lds + S * HDW;
    const A* la = lds + 2 * S * HDW;
    A M = extra ? (A)m0 : (A)-INFINITY;
#pragma unroll
    for (int s = 0; s < S; ++s) M = amax(M, lm[s * HDW + d]);
    M = slot_shift(M);
    A Lsum = 0, Asum = 0;
    if (extra) {
      const A f = softmax_exp((A)m0 - M);
      Lsum = (A)l0 * f;
      Asum = (A)a0 * f;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const A f = softmax_exp(lm[s * HDW + d] - M);  // 0 for a stream with nothing in range
      Lsum = afma(ll[s * HDW + d], f, Lsum);
      Asum = afma(la[s * HDW + d], f, Asum);
    }
    *M_out = M;
    *L_out = Lsum;
    *A_out = Asum;
  }

  // The pooled value of channel d of the slice, merged from the partials.
  __device__ __forceinline__ static float merged(const A* lds, int d) {
    const A* lm = lds;
    const A* ll = lds + S * HDW;
    const A* la = lds + 2 * S * HDW;
    A M = lm[d];
#pragma unroll 8
    for (int s = 1; s < S; ++s) M = amax(M, lm[s * HDW + d]);
    A Lsum = 0, Asum = 0;
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
      const A f = softmax_exp(lm[s * HDW + d] - M);
      Lsum = afma(ll[s * HDW + d], f, Lsum);
      Asum = afma(la[s * HDW + d], f, Asum);
    }
    return (float)(Asum / Lsum);
  }

  // The slice's channels into out_row (streaming stores), each channel merged
  // by P = NT / HDW consecutive lanes over S / P partials apiece and combined
  // with lane shuffles: with many streams (S >= 16) this keeps every wave of
  // the workgroup busy instead of one wave running all S steps per channel.
  __device__ __forceinline__ static void store_merged_par(const A* lds, int cs, float* __restrict__ out_row) {
    constexpr int P = NT / HDW;
    static_assert(P >= 1 && (P & (P - 1)) == 0 && P <= kWave && S % P == 0, "parallel merge shape");
    const A* lm = lds;
    const A* ll = lds + S * HDW;
    const A* la = lds + 2 * S * HDW;
    const int p = threadIdx.x % P, d = threadIdx.x / P;
    A M = lm[p * HDW + d];
#pragma unroll
    for (int s = p + P; s < S; s += P) M = amax(M, lm[s * HDW + d]);
#pragma unroll
    for (int o = 1; o < P; o <<= 1) M = amax(M, __shfl_xor(M, o, kWave));
    A Lsum = 0, Asum = 0;
#pragma unroll
    for (int s = p; s < S; s += P) {
      const A f = softmax_exp(lm[s * HDW + d] - M);
      Lsum = afma(ll[s * HDW + d], f, Lsum);
      Asum = afma(la[s * HDW + d], f, Asum);
    }
#pragma unroll
    for (int o = 1; o < P; o <<= 1) {
      Lsum += __shfl_xor(Lsum, o, kWave);
      Asum += __shfl_xor(Asum, o, kWave);
    }
    if (p == 0) __builtin_nontemporal_store((float)(Asum / Lsum), out_row + cs * HDW + d);
  }

  // accumulate, then the slice's channels into out_row (streaming stores)
  __device__ __forceinline__ static void run(const typename Elem<T>::storage* __restrict__ state,
                                             const typename Elem<T>::storage* __restrict__ input,
                                             const typename Elem<T>::storage* __restrict__ ape, int64_t ragged,
                                             int blen, int64_t rp0, int cs, float* __restrict__ out_row, A* lds) {
    accumulate(state, input, ape, ragged, blen, rp0, cs, lds);
    for (int d = threadIdx.x; d < HDW; d += NT) __builtin_nontemporal_store(merged(lds, d), out_row + cs * HDW + d);
  }
};

__device__ __forceinline__ bool c128_record_ok(int64_t ragged, int blen, int64_t rp0, int64_t num_q,
                                               int64_t num_state_rows) {
  const int s_hi = blen < 128 ? blen : 128;
  return rows_ok(rp0 * 128, rp0 * 128 + s_hi, num_state_rows) && rows_ok(ragged - 127 + s_hi, ragged + 1, num_q);
}

}  // namespace kvc
