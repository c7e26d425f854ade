// kvc_compress.hip - prefill compress kernels (c4.cuh page, flash_c4_prefill
// with kWrite = false; compressor_v2.py page,
// _c128_compress_prefill_compress_kernel) and the state write (c4.cuh,
// c4_write; compressor_v2.py, _c128_compress_prefill_write_kernel).
//
// All three are HBM-streaming kernels (no dense contraction, so no MFMA):
//  - compress c4: 64 lanes x 16 B cover one half-row of hd 512 bf16, so a
//    lane group reads each of its 8 window entries' kv and score quarters
//    with one 16-byte load each, all 16 (+8 ape) loads in flight before the
//    first use; 256-thread workgroups hold 256 / lanes-per-row rows.
//  - compress c128: one workgroup per compressed row; its streams split the
//    128 window entries and merge their online-softmax partials in LDS.
//  - write: one wave per record, the whole row copied with 16-byte vectors.
// Grids are sized from the host-known capacities; threads past counts[0]
// (counts[1] for the write) return at once, so no host sync is needed.
#include "kvc_device.hpp"
#include "kvc_launch.hpp"
#include "kvc_pool.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;

template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void compress_c4_kernel(CompressArgs a) {
  typedef typename Elem<T>::storage E;
  constexpr int V = Elem<T>::kVec;
  constexpr int kLanes = HD / V;
  constexpr int kRows = kThreads / kLanes;
  __shared__ float stage[kThreads * V];  // the workgroup's output rows
  const int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes;
  const int lane = threadIdx.x % kLanes;
  const int c = lane * V;
  bool live = row < a.counts[0] && row < a.cap_c;
  float res[V];
  if (live) {
    const kvc_plan_c rec = load_plan_c(a.plan_c + row);
    const int64_t ragged = rec.ragged_blen & 0xFFFFFFu;
    const int blen = (int)(rec.ragged_blen >> 24);
    const int64_t rp0 = rec.read_page_0, rp1 = rec.read_page_1;
    const bool first_block = rec.seq_len == 4u;
    live = !plan_c_invalid(rec);
    if (live && !c4_record_ok(ragged, blen, rp0, rp1, first_block ? 4 : 0, a.num_q, a.num_state_rows)) {
      if (c == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
      live = false;
    }
    if (live) {
      const E* state = static_cast<const E*>(a.state);
      const E* input = static_cast<const E*>(a.input);
      const E* ape = static_cast<const E*>(a.ape);
      if (first_block) {
        c4_pool<T, HD, 4>(state, input, ape, ragged, blen, rp0, rp1, c, res);
      } else {
        c4_pool<T, HD, 0>(state, input, ape, ragged, blen, rp0, rp1, c, res);
      }
    }
  }
  // A lane holds V adjacent channels, so storing them directly would write
  // 16-byte pieces at a 4*V-byte stride.  Staging the row in LDS lets every
  // store instruction write 64 x 16 contiguous bytes instead.
  float* w = stage + (threadIdx.x / kLanes) * HD;
  store_floats<V>(w + c, res);
  __syncthreads();
  if (live) {
#pragma unroll
    for (int k = 0; k < V / 4; ++k) {
      const int ch = k * (kLanes * 4) + lane * 4;
      store16_stream(a.out + row * HD + ch, load16(w + ch));  // written once, read by a later kernel
    }
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void compress_c128_kernel(CompressArgs a) {
  typedef typename Elem<T>::storage E;
  typedef C128Pool<T, HD, kThreads> Pool;
  __shared__ float lds[Pool::kLdsFloats];
  const int64_t row = blockIdx.x;
  if (row >= a.counts[0] || row >= a.cap_c) return;
  const kvc_plan_c rec = load_plan_c(a.plan_c + row);
  if (plan_c_invalid(rec)) return;
  const int64_t ragged = rec.ragged_blen & 0xFFFFFFu;
  const int blen = (int)(rec.ragged_blen >> 24);
  const int64_t rp0 = rec.read_page_0;
  if (!c128_record_ok(ragged, blen, rp0, a.num_q, a.num_state_rows)) {
    if (threadIdx.x == 0) atomicOr(a.counts + 3, KVC_DERR_RECORD);
    return;
  }
  Pool::run(static_cast<const E*>(a.state), static_cast<const E*>(a.input), static_cast<const E*>(a.ape), ragged,
            blen, rp0, 0, a.out + row * HD, lds);
}

constexpr int kWriteRowsPerBlock = kThreads / kWave;

// One wave per record.  PER = 16-byte vectors per lane (a row holds up to
// 64 * PER vectors); the input row is read once (streaming load) and stored
// to the state with ordinary stores, since the next chunk reads it back.
template <int PER>
__global__ __launch_bounds__(kThreads) void write_kernel(WriteArgs a) {
  const int64_t k = (int64_t)blockIdx.x * kWriteRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (k >= a.counts[1] || k >= a.cap_w) return;
  const uint2 rec = *reinterpret_cast<const uint2*>(a.plan_w + k);
  if (rec.x == 0xFFFFFFFFu) return;
  const int64_t ragged = rec.x;
  const int64_t loc = (int32_t)rec.y;
  if (ragged >= a.num_q || loc < 0 || loc >= a.num_state_rows) {
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

template <typename T, int HD>
hipError_t c4_launch(const CompressArgs& a, hipStream_t stream) {
  constexpr int kRows = kThreads / (HD / Elem<T>::kVec);
  const int grid = (a.cap_c + kRows - 1) / kRows;
  compress_c4_kernel<T, HD><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t c128_launch(const CompressArgs& a, hipStream_t stream) {
  compress_c128_kernel<T, HD><<<a.cap_c, kThreads, 0, stream>>>(a);
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
  static hipError_t go(const CompressArgs& a, hipStream_t s) { return c4_launch<T, HD>(a, s); }
};
template <typename T, int HD>
struct C128Go {
  static hipError_t go(const CompressArgs& a, hipStream_t s) { return c128_launch<T, HD>(a, s); }
};

}  // namespace

hipError_t launch_compress_c4(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream) {
  return dispatch<C4Go>(dtype, head_dim, a, stream);
}

hipError_t launch_compress_c128(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream) {
  return dispatch<C128Go>(dtype, head_dim, a, stream);
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
