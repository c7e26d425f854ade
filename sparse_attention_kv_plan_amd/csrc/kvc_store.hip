// kvc_store.hip - norm + rotary embedding + bf16 store of compressed rows
// that are already in HBM as float32 (compressor_v2.py page,
// compress_norm_rope_store).  HBM-bound: a row is read once (4*hd bytes) and
// stored once (2*hd bytes); 8 channels per lane, hd/8 lanes per row, the sum
// of squares reduced across the row's lanes inside the wave.
#include "kvc_device.hpp"
#include "kvc_launch.hpp"
#include "kvc_store.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;
constexpr int kK = 8;  // channels per lane

template <int HD, bool DECODE>
__global__ __launch_bounds__(kThreads) void norm_rope_store_kernel(NormRopeStoreArgs a) {
  constexpr int kLanes = HD / kK;  // 16, 32 or 64: a row never leaves its wave
  constexpr int kRows = kThreads / kLanes;
  const int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes;
  const int c = (threadIdx.x % kLanes) * kK;
  // the loads that depend on nothing go out first (the record, the row, the
  // norm weight), then the lookups that need the record
  bool live;
  uint32_t seq_len = 0;
  int64_t key = 0;
  int32_t* err;
  if constexpr (DECODE) {
    if (row >= a.n) return;
    const kvc_plan_d rec = load_plan_d(a.plan_d + row);
    live = !plan_d_invalid(rec) && rec.seq_len % (uint32_t)a.compress_ratio == 0;
    seq_len = rec.seq_len;
    key = row;
    err = a.status;
  } else {
    if (row >= a.counts[0] || row >= a.n) return;
    const kvc_plan_c rec = load_plan_c(a.plan_c + row);
    live = !plan_c_invalid(rec);
    seq_len = rec.seq_len;
    key = rec.ragged_blen & 0xFFFFFFu;
    err = a.counts + 3;
  }
  float x[kK];
  const float* src = a.rows + row * HD + c;  // row < a.n: inside the rows buffer whatever the record holds
#pragma unroll
  for (int i = 0; i < kK; i += 4) widen16<float>(load16_stream(src + i), x + i);
  const int32_t pos = seq_len >= (uint32_t)a.compress_ratio ? (int32_t)(seq_len - a.compress_ratio) : 0;
  StoreOperands<kK> ops;
  const int32_t loc = live ? fetch_loc(a.st, key) : -1;
  if (live) fetch_operands<kK, HD>(a.st, c, pos, ops);
  if (!live) return;
  if (!store_ok(a.st, loc, pos)) {
    if (c == 0 && err != nullptr) atomicOr(err, KVC_DERR_RECORD);
    return;  // the whole row leaves together: the reduction below stays inside live rows
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kK; ++k) ss = fmaf(x[k], x[k], ss);
  ss = row_sum<kLanes>(ss, nullptr);
  norm_rope_store<kK, HD>(x, ss, c, loc, ops, a.st);
}

template <int HD, bool DECODE>
hipError_t nrs_launch(const NormRopeStoreArgs& a, hipStream_t stream) {
  constexpr int kRows = kThreads / (HD / kK);
  norm_rope_store_kernel<HD, DECODE><<<(a.n + kRows - 1) / kRows, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_rope_store(int head_dim, bool decode, const NormRopeStoreArgs& a, hipStream_t stream) {
  if (head_dim == 128) return decode ? nrs_launch<128, true>(a, stream) : nrs_launch<128, false>(a, stream);
  if (head_dim == 256) return decode ? nrs_launch<256, true>(a, stream) : nrs_launch<256, false>(a, stream);
  return decode ? nrs_launch<512, true>(a, stream) : nrs_launch<512, false>(a, stream);
}

}  // namespace kvc
