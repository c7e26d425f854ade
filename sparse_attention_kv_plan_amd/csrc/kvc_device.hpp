// kvc_device.hpp - device-side helpers shared by the gfx950 kernels.
//
// Element storage: fp32 as float, bf16 as its 16-bit pattern.  Every global
// access of tensor data is a 16-byte vector (4 fp32 or 8 bf16 channels), so a
// wave of 64 lanes moves 1 KiB per instruction and a row of a tensor is read
// by consecutive lanes (fully coalesced).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Bf16 {};  // tag type: bf16 stored as uint16_t bit patterns

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  typedef float storage;
  static constexpr int kVec = 4;  // channels per 16-byte vector
};
template <>
struct Elem<Bf16> {
  typedef uint16_t storage;
  static constexpr int kVec = 8;
};

// Puts a wave-uniform value (a kernel argument) in scalar registers at this
// point.  The compiler otherwise loads an argument where it is first used;
// one first used inside a branch or a loop then costs a trip to memory of its
// own there, after whatever the kernel waited for before.
template <typename T>
__device__ __forceinline__ void in_sgprs(T v) {
  asm volatile("" ::"s"(v));
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 load8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Streaming (non-temporal) 16-byte access for data touched once per launch: the
// line is not kept in L2 / the last-level cache, so a stream of kv/score rows
// neither evicts the small reused operands (ape, plans) nor forces write-backs
// of dirty lines left by earlier kernels.  On MI355X this lifts a plain read
// stream from about 6.1 to about 6.9 TB/s.  Every row that a kernel writes for
// a later kernel (state rows, compressed rows) is stored the same way: dirty
// cached lines left by a write kernel slow the next streaming kernel by ~25%.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// 16 bytes of elements -> kVec floats (bf16 -> fp32 is an exact 16-bit shift)
template <typename T>
__device__ __forceinline__ void widen16(u32x4 raw, float* out);

template <>
__device__ __forceinline__ void widen16<float>(u32x4 raw, float* out) {
  out[0] = __uint_as_float(raw.x);
  out[1] = __uint_as_float(raw.y);
  out[2] = __uint_as_float(raw.z);
  out[3] = __uint_as_float(raw.w);
}

template <>
__device__ __forceinline__ void widen16<Bf16>(u32x4 raw, float* out) {
  out[0] = __uint_as_float(raw.x << 16);
  out[1] = __uint_as_float(raw.x & 0xFFFF0000u);
  out[2] = __uint_as_float(raw.y << 16);
  out[3] = __uint_as_float(raw.y & 0xFFFF0000u);
  out[4] = __uint_as_float(raw.z << 16);
  out[5] = __uint_as_float(raw.z & 0xFFFF0000u);
  out[6] = __uint_as_float(raw.w << 16);
  out[7] = __uint_as_float(raw.w & 0xFFFF0000u);
}

// 2^x on the hardware exp unit; the softmax weights are exp(d) = 2^(d*log2 e)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// The arithmetic type of the pool for an input element type.
//  - bf16 inputs: fp32.  bf16 widens exactly, and the weights' relative error
//    of a few fp32 ulp is far inside the bf16 bar (2e-2 absolute).
//  - fp32 inputs: fp64.  score + ape, the shift by the window maximum, the
//    exponential and both sums are then exact to about 1e-15 relative for
//    any finite input, so the result is the pooled value rounded once to
//    fp32.  In fp32 arithmetic a weight carries a relative error of about
//    |score| * 2^-24 (the rounding of score + ape and of the scaled
//    exponent), which grows with the scores' magnitude.
template <typename T>
struct Acc;
template <>
struct Acc<Bf16> {
  typedef float type;
};
template <>
struct Acc<float> {
  typedef double type;
};

// exp(d) of a shifted score (d <= 0 apart from rounding of the shift)
__device__ __forceinline__ float softmax_exp(float d) { return exp2_hw(d * kLog2e); }
__device__ __forceinline__ double softmax_exp(double d) { return exp(d); }

__device__ __forceinline__ float amax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ double amax(double a, double b) { return fmax(a, b); }
__device__ __forceinline__ float afma(float a, float b, float c) { return fmaf(a, b, c); }
__device__ __forceinline__ double afma(double a, double b, double c) { return fma(a, b, c); }

// A running maximum as it is kept in an fp32 slot: the sums that go with it
// must be taken relative to exactly that value.  Identity in fp32.
__device__ __forceinline__ float slot_shift(float m) { return m; }
__device__ __forceinline__ double slot_shift(double m) { return (double)(float)m; }

// store n (a multiple of 4) floats as 16-byte vectors
template <int N, bool STREAM = false>
__device__ __forceinline__ void store_floats(float* dst, const float* v) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    u32x4 w;
    w.x = __float_as_uint(v[i + 0]);
    w.y = __float_as_uint(v[i + 1]);
    w.z = __float_as_uint(v[i + 2]);
    w.w = __float_as_uint(v[i + 3]);
    if constexpr (STREAM) {
      store16_stream(dst + i, w);
    } else {
      store16(dst + i, w);
    }
  }
}

// store n partials of the pool's arithmetic type (LDS)
template <int N>
__device__ __forceinline__ void store_acc(float* dst, const float* v) {
  store_floats<N>(dst, v);
}
template <int N>
__device__ __forceinline__ void store_acc(double* dst, const double* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) dst[i] = v[i];
}

template <int N>
__device__ __forceinline__ void store_zeros(float* dst) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < N; i += 4) store16_stream(dst + i, z);
}

__device__ __forceinline__ bool plan_c_invalid(const kvc_plan_c& r) { return r.seq_len == 0xFFFFFFFFu; }
__device__ __forceinline__ bool plan_d_invalid(const kvc_plan_d& r) { return r.seq_len == 0xFFFFFFFFu; }

__device__ __forceinline__ kvc_plan_c load_plan_c(const kvc_plan_c* p) {
  u32x4 v = load16(p);
  kvc_plan_c r;
  r.seq_len = v.x;
  r.ragged_blen = v.y;
  r.read_page_0 = (int32_t)v.z;
  r.read_page_1 = (int32_t)v.w;
  return r;
}

__device__ __forceinline__ kvc_plan_d load_plan_d(const kvc_plan_d* p) {
  u32x4 v = load16(p);
  kvc_plan_d r;
  r.seq_len = v.x;
  r.write_loc = (int32_t)v.y;
  r.read_page_0 = (int32_t)v.z;
  r.read_page_1 = (int32_t)v.w;
  return r;
}

// true iff rows [lo, hi) of a buffer with n rows are all in range (empty is fine)
__device__ __forceinline__ bool rows_ok(int64_t lo, int64_t hi, int64_t n) { return hi <= lo || (lo >= 0 && hi <= n); }

}  // namespace kvc
