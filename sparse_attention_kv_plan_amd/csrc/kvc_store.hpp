// kvc_store.hpp - the step after the pool (compressor_v2.py page,
// compress_norm_rope_store and _forward_unified_hip): RMSNorm over the row,
// rotary embedding of the row's last rope_dim channels at position
// seq_len - ratio, bf16 store into the compressed cache at out_loc[key].
//
// A thread owns K adjacent channels of a row (K even, so a rotary pair never
// straddles two threads, and rope_dim % 8 == 0 keeps a thread's K channels
// all rotated or all plain).  The row's sum of squares is reduced across
// the threads of the row first (row_sum / block_sum), so every thread of a
// row applies the same scale.
#pragma once

#include "kvc_device.hpp"

namespace kvc {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even; a NaN stays a NaN) packed
// low / high in one word.  gfx950 converts a pair in one instruction
// (v_cvt_pk_bf16_f32); rounding by integer arithmetic instead costs ~7 VALU
// operations per channel, and measurably slows the fused pool.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Sum over the kLanes consecutive lanes that hold one row (kLanes a power of
// two).  Rows of up to 64 lanes reduce inside the wave with an xor butterfly
// (every lane ends with the same bits); wider rows add their waves' partials
// through `red` (one float per wave of the workgroup).  Every thread of the
// workgroup must call it.
template <int kLanes>
__device__ __forceinline__ float row_sum(float v, float* red) {
  constexpr int kIn = kLanes < kWave ? kLanes : kWave;
#pragma unroll
  for (int o = kIn / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if constexpr (kLanes > kWave) {
    constexpr int kWaves = kLanes / kWave;
    const int wave = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) red[wave] = v;
    __syncthreads();
    const int w0 = wave / kWaves * kWaves;
    v = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) v += red[w0 + i];
  }
  return v;
}

// Sum over the whole workgroup of NT threads; `red` holds NT / 64 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  __syncthreads();  // red may still be read by a previous call
  return row_sum<NT>(v, red);
}

template <int K>
__device__ __forceinline__ void load_floats(const float* p, float* out) {
  static_assert(K == 2 || K % 4 == 0, "K");
  if constexpr (K == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    out[0] = v.x;
    out[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < K; i += 4) {
      const u32x4 v = load16(p + i);
      out[i + 0] = __uint_as_float(v.x);
      out[i + 1] = __uint_as_float(v.y);
      out[i + 2] = __uint_as_float(v.z);
      out[i + 3] = __uint_as_float(v.w);
    }
  }
}

// K channels -> K bf16 at dst (2K bytes, aligned to 2K), streaming store
template <int K>
__device__ __forceinline__ void store_bf16(uint16_t* dst, const float* y) {
  uint32_t w[K / 2];
#pragma unroll
  for (int i = 0; i < K / 2; ++i) w[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
  if constexpr (K == 2) {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(dst));
  } else if constexpr (K == 4) {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(dst));
    __builtin_nontemporal_store(w[1], reinterpret_cast<uint32_t*>(dst) + 1);
  } else {
#pragma unroll
    for (int i = 0; i < K / 2; i += 4) {
      const u32x4 v = {w[i], w[i + 1], w[i + 2], w[i + 3]};
      store16_stream(dst + 2 * i, v);
    }
  }
}

// The out_loc entry of a key, or -1 when the key has none.  Issued before the
// pool's loads and checked after them, so the lookup adds no latency.
__device__ __forceinline__ int32_t fetch_loc(const kvc_store_args& st, int64_t key) {
  return (key >= 0 && key < st.num_loc) ? st.out_loc[key] : -1;
}

// Whether the row of a record can be stored: its location (from fetch_loc)
// and rotary position are inside their tables.
__device__ __forceinline__ bool store_ok(const kvc_store_args& st, int32_t loc, int32_t pos) {
  return loc >= 0 && loc < st.num_cache_rows && (st.rope_dim == 0 || pos < st.max_position);
}

// Per-thread operands of the store: the norm weight of channels [c, c + K)
// and, for rotated channels, their (cos, sin) pairs at the row's position.
template <int K>
struct StoreOperands {
  float w[K];
  float cs[K];
};

template <int K, int HD>
__device__ __forceinline__ void fetch_operands(const kvc_store_args& st, int c, int32_t pos, StoreOperands<K>& o) {
  load_floats<K>(st.norm_weight + c, o.w);
  const int base = HD - st.rope_dim;
  if (c >= base && pos < st.max_position)
    load_floats<K>(st.freqs_cis + (int64_t)pos * st.rope_dim + (c - base), o.cs);
}

// Norm + rotation + store of channels [c, c + K) of one row whose sum of
// squares over all HD channels is ss.  x is modified in place.
template <int K, int HD>
__device__ __forceinline__ void norm_rope_store(float* x, float ss, int c, int32_t loc, const StoreOperands<K>& o,
                                                const kvc_store_args& st) {
  const float inv = 1.0f / sqrtf(ss * (1.0f / HD) + st.eps);
#pragma unroll
  for (int k = 0; k < K; ++k) x[k] = x[k] * inv * o.w[k];
  if (c >= HD - st.rope_dim) {
#pragma unroll
    for (int k = 0; k < K; k += 2) {
      const float re = x[k], im = x[k + 1];
      x[k] = re * o.cs[k] - im * o.cs[k + 1];
      x[k + 1] = re * o.cs[k + 1] + im * o.cs[k];
    }
  }
  store_bf16<K>(st.cache + (int64_t)loc * HD + c, x);
}

}  // namespace kvc
