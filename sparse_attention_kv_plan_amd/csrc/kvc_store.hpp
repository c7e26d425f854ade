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

// float -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
  for (int i = 0; i < K / 2; ++i) w[i] = bf16_bits(y[2 * i]) | (bf16_bits(y[2 * i + 1]) << 16);
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

// Whether the row of a record can be stored: its key, cache location and
// rotary position are inside their tables.  Sets *loc.
__device__ __forceinline__ bool store_target(const kvc_store_args& st, int64_t key, int64_t pos, int64_t* loc) {
  if (key < 0 || key >= st.num_loc) return false;
  const int64_t l = st.out_loc[key];
  if (l < 0 || l >= st.num_cache_rows) return false;
  if (st.rope_dim > 0 && pos >= st.max_position) return false;
  *loc = l;
  return true;
}

// Norm + rotation + store of channels [c, c + K) of one row whose sum of
// squares over all HD channels is ss.  x is modified in place.
template <int K, int HD>
__device__ __forceinline__ void norm_rope_store(float* x, float ss, int c, int64_t pos, int64_t loc,
                                                const kvc_store_args& st) {
  const float inv = 1.0f / sqrtf(ss * (1.0f / HD) + st.eps);
  float w[K];
  load_floats<K>(st.norm_weight + c, w);
#pragma unroll
  for (int k = 0; k < K; ++k) x[k] = x[k] * inv * w[k];
  const int base = HD - st.rope_dim;
  if (c >= base) {
    float cs[K];
    load_floats<K>(st.freqs_cis + pos * st.rope_dim + (c - base), cs);
#pragma unroll
    for (int k = 0; k < K; k += 2) {
      const float re = x[k], im = x[k + 1];
      x[k] = re * cs[k] - im * cs[k + 1];
      x[k + 1] = re * cs[k + 1] + im * cs[k];
    }
  }
  store_bf16<K>(st.cache + loc * HD + c, x);
}

}  // namespace kvc
