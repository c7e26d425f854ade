// Same-box bandwidth ceilings: plain 16-byte-vector streams over flat buffers, which the benchmark
// times beside the pool kernels.  They are no part of the KV compressor and libkvc.so does not
// contain them; they live in libstream_probe.so.
//
//   int stream_probe(int kind, int nontemporal, const void* src, int64_t src_bytes,
//                    void* dst, int64_t dst_bytes, void* stream);
//
// kind 0  copy: every 16-byte vector of src is read once and written once to dst.
// kind 1  read 8, write 1: each vector written to dst is the xor of 8 vectors of src (the ratio-4
//         pool moves about 8 bytes in for each byte out).
// kind 2  read only: each thread xors 16 vectors of src and stores the result only when it is not
//         zero.  A src filled with one repeated value xors to zero, so nothing is written, but the
//         compiler cannot drop the loads.
// nontemporal != 0 loads src with streaming loads; stores are always ordinary.
// src_bytes must be a positive multiple of the kind's tile (stream_probe_tile(kind) bytes); dst must hold
// src_bytes (kind 0), src_bytes / 8 (kind 1) or src_bytes / 16 (kind 2) bytes; both pointers are
// device memory aligned to 16 bytes.  The launch goes to `stream` (a hipStream_t, NULL for the
// default stream) and is asynchronous.
// Returns 0, -EINVAL for a bad argument (nothing launched), or the HIP error of the launch.
#include <hip/hip_runtime.h>

#include <cerrno>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <bool NT>
__device__ inline u32x4 load(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Workgroup g reads the R*U*kThreads vectors starting at vector g*R*U*kThreads and writes the U*kThreads
// vectors starting at g*U*kThreads: thread t's vector u is the xor of its R reads
// ((g*U + u)*R + r)*kThreads + t, r < R.  The grid is exactly src vectors / (R*U*kThreads), so every
// index is in bounds.
template <int R, int U, bool NT, bool WRITE>
__global__ __launch_bounds__(kThreads) void stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  const int64_t g = blockIdx.x;
  u32x4 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[u] ^= load<NT>(src + ((g * U + u) * R + r) * kThreads + threadIdx.x);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u32x4 v = acc[u];
    if (WRITE || (v.x | v.y | v.z | v.w) != 0u) dst[(g * U + u) * kThreads + threadIdx.x] = v;
  }
}

struct Kind {
  int reads, unroll;  // R, U
};
constexpr Kind kKinds[3] = {{1, 4}, {8, 1}, {16, 1}};

template <int R, int U, bool WRITE>
void launch(bool nt, const u32x4* src, u32x4* dst, int64_t blocks, hipStream_t s) {
  if (nt) stream_kernel<R, U, true, WRITE><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(src, dst);
  else stream_kernel<R, U, false, WRITE><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(src, dst);
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int stream_probe(int kind, int nontemporal, const void* src,
                                                                   int64_t src_bytes, void* dst, int64_t dst_bytes,
                                                                   void* stream) {
  if (kind < 0 || kind > 2 || src == nullptr || dst == nullptr) return -EINVAL;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return -EINVAL;
  const Kind k = kKinds[kind];
  const int64_t tile = 16LL * k.reads * k.unroll * kThreads;
  if (src_bytes <= 0 || src_bytes % tile != 0) return -EINVAL;
  const int64_t blocks = src_bytes / tile;
  if (blocks > 0x7fffffffLL) return -EINVAL;
  if (dst_bytes < src_bytes / k.reads) return -EINVAL;
  const auto* s = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
  const auto hs = static_cast<hipStream_t>(stream);
  const bool nt = nontemporal != 0;
  if (kind == 0) launch<1, 4, true>(nt, s, d, blocks, hs);
  else if (kind == 1) launch<8, 1, true>(nt, s, d, blocks, hs);
  else launch<16, 1, false>(nt, s, d, blocks, hs);
  return static_cast<int>(hipGetLastError());
}

// The tile of each kind, in bytes: src_bytes must be a multiple of it.
extern "C" __attribute__((visibility("default"))) int64_t stream_probe_tile(int kind) {
  if (kind < 0 || kind > 2) return -EINVAL;
  return 16LL * kKinds[kind].reads * kKinds[kind].unroll * kThreads;
}
