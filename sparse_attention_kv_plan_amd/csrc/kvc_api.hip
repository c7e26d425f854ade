// kvc_api.hip - the C entry points declared in include/kvc.h: host argument
// checks, then one kernel launch each on the caller's stream.
#include <stdint.h>

#include <climits>
#include <cmath>

#include "kvc.h"
#include "kvc_launch.hpp"

#define KVC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool aligned4(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool ratio_ok(int cr) { return cr == 4 || cr == 128; }
bool dtype_ok(int dt) { return dt == KVC_F32 || dt == KVC_BF16; }
bool hd_ok(int hd) { return hd == 128 || hd == 256 || hd == 512; }
bool rows_ok(int64_t rows) { return rows >= 0 && rows <= INT32_MAX; }
int status_of(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_EHIP; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
// the ratio-128 boundary list: optional, 8-byte aligned; ratio 4 has none
bool boundaries_ok(int cr, const int32_t* list) { return list == nullptr || (cr == 128 && aligned8(list)); }

}  // namespace

KVC_EXPORT int kvc_plan_prefill(int compress_ratio, int batch, int num_q, const int32_t* seq_lens,
                                const int32_t* extend_lens, const int32_t* state_index, int64_t num_state_rows,
                                kvc_plan_c* plan_c, int cap_c, kvc_plan_w* plan_w, int cap_w, int32_t* counts,
                                int32_t* runs, void* stream) {
  if (!ratio_ok(compress_ratio) || batch < 1 || batch > KVC_MAX_PREFILL_BATCH) return KVC_EINVAL;
  if (runs != nullptr && (compress_ratio != 128 || !aligned16(runs))) return KVC_EINVAL;
  if (num_q < batch || num_q >= KVC_MAX_TOKENS || cap_c < 0 || cap_w < 0 || !rows_ok(num_state_rows))
    return KVC_EINVAL;
  if (!aligned4(seq_lens) || !aligned4(extend_lens) || !aligned4(state_index) || !aligned4(counts))
    return KVC_EINVAL;
  if ((cap_c > 0 && !aligned16(plan_c)) || (cap_w > 0 && !aligned8(plan_w)))
    return KVC_EINVAL;
  kvc::PlanPrefillArgs a{};
  a.seq_lens = seq_lens;
  a.extend_lens = extend_lens;
  a.state_index = state_index;
  a.num_state_rows = num_state_rows;
  a.plan_c = plan_c;
  a.plan_w = plan_w;
  a.counts = counts;
  a.batch = batch;
  a.num_q = num_q;
  a.cap_c = cap_c;
  a.cap_w = cap_w;
  a.runs = runs;
  return status_of(kvc::launch_plan_prefill(compress_ratio, kvc::kPlanRing, a, as_stream(stream)));
}

KVC_EXPORT int kvc_plan_decode(int compress_ratio, int batch, const int32_t* seq_lens, const int32_t* state_index,
                               int64_t num_state_rows, kvc_plan_d* plan_d, int32_t* boundaries, int32_t* status,
                               void* stream) {
  if (!ratio_ok(compress_ratio) || batch < 1 || batch > KVC_MAX_DECODE_BATCH || !rows_ok(num_state_rows))
    return KVC_EINVAL;
  if (!aligned4(seq_lens) || !aligned4(state_index) || !aligned16(plan_d)) return KVC_EINVAL;
  if (!boundaries_ok(compress_ratio, boundaries)) return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  kvc::PlanDecodeArgs a{};
  a.seq_lens = seq_lens;
  a.state_index = state_index;
  a.num_state_rows = num_state_rows;
  a.plan_d = plan_d;
  a.status = status;
  a.batch = batch;
  a.boundaries = boundaries;
  return status_of(kvc::launch_plan_decode(compress_ratio, kvc::kPlanRing, a, as_stream(stream)));
}

namespace {

// Host checks of the SWA tables; fills t on success.
bool swa_args_ok(int cr, const int32_t* req_to_token, int64_t r2t_stride, int64_t num_reqs,
                 const int32_t* full_to_swa, int64_t num_full, int swa_page_size, int ring_size, kvc::SwaTables* t) {
  if (swa_page_size <= 0 || ring_size <= 0 || swa_page_size % ring_size != 0 || ring_size % cr != 0) return false;
  if (cr == 4 && ring_size % 8 != 0) return false;  // both 4-row pages of a window must be distinct rows
  if (cr == 128 && ring_size != 128) return false;  // the ratio-128 consumer pools one 128-row page
  if (r2t_stride <= 0 || num_reqs <= 0 || num_full < 0 || num_full > INT32_MAX) return false;
  if (r2t_stride > INT64_MAX / num_reqs) return false;
  if (!aligned4(req_to_token) || (num_full > 0 && !aligned4(full_to_swa))) return false;
  *t = kvc::SwaTables{req_to_token, full_to_swa, r2t_stride, num_reqs, num_full, swa_page_size, ring_size};
  return true;
}

}  // namespace

KVC_EXPORT int kvc_plan_prefill_swa(int compress_ratio, int batch, int num_q, const int32_t* seq_lens,
                                    const int32_t* extend_lens, const int32_t* req_pool_indices,
                                    const int32_t* req_to_token, int64_t r2t_stride, int64_t num_reqs,
                                    const int32_t* full_to_swa, int64_t num_full, int swa_page_size, int ring_size,
                                    int64_t num_state_rows, kvc_plan_c* plan_c, int cap_c, kvc_plan_w* plan_w,
                                    int cap_w, int32_t* counts, int32_t* status, void* stream) {
  if (!ratio_ok(compress_ratio) || batch < 1 || batch > KVC_MAX_PREFILL_BATCH) return KVC_EINVAL;
  if (num_q < batch || num_q >= KVC_MAX_TOKENS || cap_c < 0 || cap_w < 0 || !rows_ok(num_state_rows))
    return KVC_EINVAL;
  if (!aligned4(seq_lens) || !aligned4(extend_lens) || !aligned4(req_pool_indices) || !aligned4(counts))
    return KVC_EINVAL;
  if ((cap_c > 0 && !aligned16(plan_c)) || (cap_w > 0 && !aligned8(plan_w)))
    return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  kvc::PlanPrefillArgs a{};
  if (!swa_args_ok(compress_ratio, req_to_token, r2t_stride, num_reqs, full_to_swa, num_full, swa_page_size,
                   ring_size, &a.swa))
    return KVC_EINVAL;
  a.seq_lens = seq_lens;
  a.extend_lens = extend_lens;
  a.state_index = req_pool_indices;
  a.num_state_rows = num_state_rows;
  a.plan_c = plan_c;
  a.plan_w = plan_w;
  a.counts = counts;
  a.status = status;
  a.batch = batch;
  a.num_q = num_q;
  a.cap_c = cap_c;
  a.cap_w = cap_w;
  return status_of(kvc::launch_plan_prefill(compress_ratio, kvc::kPlanSwa, a, as_stream(stream)));
}

KVC_EXPORT int kvc_plan_decode_swa(int compress_ratio, int batch, const int32_t* seq_lens,
                                   const int32_t* req_pool_indices, const int32_t* req_to_token, int64_t r2t_stride,
                                   int64_t num_reqs, const int32_t* full_to_swa, int64_t num_full, int swa_page_size,
                                   int ring_size, int64_t num_state_rows, kvc_plan_d* plan_d, int32_t* boundaries,
                                   int32_t* status, void* stream) {
  if (!ratio_ok(compress_ratio) || batch < 1 || batch > KVC_MAX_DECODE_BATCH || !rows_ok(num_state_rows))
    return KVC_EINVAL;
  if (!aligned4(seq_lens) || !aligned4(req_pool_indices) || !aligned16(plan_d)) return KVC_EINVAL;
  if (!boundaries_ok(compress_ratio, boundaries)) return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  kvc::PlanDecodeArgs a{};
  if (!swa_args_ok(compress_ratio, req_to_token, r2t_stride, num_reqs, full_to_swa, num_full, swa_page_size,
                   ring_size, &a.swa))
    return KVC_EINVAL;
  a.seq_lens = seq_lens;
  a.state_index = req_pool_indices;
  a.num_state_rows = num_state_rows;
  a.plan_d = plan_d;
  a.status = status;
  a.batch = batch;
  a.boundaries = boundaries;
  return status_of(kvc::launch_plan_decode(compress_ratio, kvc::kPlanSwa, a, as_stream(stream)));
}

KVC_EXPORT int kvc_plan_prefill_page4(int batch, int num_q, const int32_t* seq_lens, const int32_t* extend_lens,
                                      const int32_t* page_index, const int32_t* bundle, int64_t num_state_rows,
                                      kvc_plan_c* plan_c, int cap_c, kvc_plan_w* plan_w, int cap_w, int32_t* counts,
                                      int32_t* status, void* stream) {
  if (batch < 1 || batch > KVC_MAX_PREFILL_BATCH) return KVC_EINVAL;
  if (num_q < batch || num_q >= KVC_MAX_TOKENS || cap_c < 0 || cap_w < 0 || !rows_ok(num_state_rows))
    return KVC_EINVAL;
  if (!aligned4(seq_lens) || !aligned4(extend_lens) || !aligned4(page_index) || !aligned16(bundle) ||
      !aligned4(counts))
    return KVC_EINVAL;
  if ((cap_c > 0 && !aligned16(plan_c)) || (cap_w > 0 && !aligned8(plan_w)))
    return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  kvc::PlanPrefillArgs a{};
  a.seq_lens = seq_lens;
  a.extend_lens = extend_lens;
  a.state_index = page_index;
  a.num_state_rows = num_state_rows;
  a.plan_c = plan_c;
  a.plan_w = plan_w;
  a.counts = counts;
  a.status = status;
  a.batch = batch;
  a.num_q = num_q;
  a.cap_c = cap_c;
  a.cap_w = cap_w;
  a.bundle = bundle;
  return status_of(kvc::launch_plan_prefill(4, kvc::kPlanPage4, a, as_stream(stream)));
}

KVC_EXPORT int kvc_plan_decode_page4(int batch, const int32_t* seq_lens, const int32_t* page_index,
                                     const int32_t* prev_page, int64_t num_state_rows, kvc_plan_d* plan_d,
                                     int32_t* status, void* stream) {
  if (batch < 1 || batch > KVC_MAX_DECODE_BATCH || !rows_ok(num_state_rows)) return KVC_EINVAL;
  if (!aligned4(seq_lens) || !aligned4(page_index) || !aligned4(prev_page) || !aligned16(plan_d)) return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  kvc::PlanDecodeArgs a{};
  a.seq_lens = seq_lens;
  a.state_index = page_index;
  a.num_state_rows = num_state_rows;
  a.plan_d = plan_d;
  a.status = status;
  a.batch = batch;
  a.prev_page = prev_page;
  return status_of(kvc::launch_plan_decode(4, kvc::kPlanPage4, a, as_stream(stream)));
}

KVC_EXPORT int kvc_write(int compress_ratio, kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows,
                         const void* input, int num_q, const kvc_plan_w* plan_w, int cap_w, int32_t* counts,
                         void* stream) {
  if (!ratio_ok(compress_ratio) || !dtype_ok(dtype) || !hd_ok(head_dim) || !rows_ok(num_state_rows)) return KVC_EINVAL;
  if (num_q < 0 || num_q >= KVC_MAX_TOKENS || cap_w < 0 || !aligned4(counts)) return KVC_EINVAL;
  if (cap_w == 0) return KVC_OK;
  if (!aligned16(state) || !aligned16(input) || !aligned8(plan_w))
    return KVC_EINVAL;
  const int esize = dtype == KVC_BF16 ? 2 : 4;
  const int row_vecs = (compress_ratio == 4 ? 4 : 2) * head_dim * esize / 16;
  kvc::WriteArgs a{state, input, plan_w, counts, num_state_rows, num_q, cap_w, row_vecs};
  return status_of(kvc::launch_write(a, as_stream(stream)));
}

namespace {

// Host checks of the norm / rotary / store parameters.
bool store_args_ok(int hd, const kvc_store_args* st) {
  if (st == nullptr) return false;
  if (st->rope_dim < 0 || st->rope_dim > hd || st->rope_dim % 8 != 0) return false;
  if (!(st->eps >= 0.f) || !std::isfinite(st->eps)) return false;
  if (st->num_loc < 0 || st->num_loc > INT32_MAX || !rows_ok(st->num_cache_rows) || st->max_position < 0)
    return false;
  if (st->max_position > INT32_MAX) return false;
  if (!aligned16(st->norm_weight)) return false;
  if (st->num_cache_rows > 0 && !aligned16(st->cache)) return false;
  if (st->num_loc > 0 && !aligned4(st->out_loc)) return false;
  if (st->rope_dim > 0 && st->max_position > 0 && !aligned16(st->freqs_cis)) return false;
  return true;
}

// out != nullptr: pool into float32 rows; st != nullptr: pool + norm + rotary + store
int compress_common(bool c4, kvc_dtype dtype, int head_dim, const void* state, int64_t num_state_rows,
                    const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c, int cap_c,
                    int32_t* counts, float* out, const kvc_store_args* st, void* stream) {
  if (!dtype_ok(dtype) || !hd_ok(head_dim) || !rows_ok(num_state_rows)) return KVC_EINVAL;
  if (num_q < 0 || num_q >= KVC_MAX_TOKENS || cap_c < 0 || !aligned4(counts)) return KVC_EINVAL;
  if (st != nullptr && !store_args_ok(head_dim, st)) return KVC_EINVAL;
  if (cap_c == 0) return KVC_OK;
  if (!aligned16(input) || !aligned16(ape) || !aligned16(plan_c)) return KVC_EINVAL;
  if (st == nullptr && !aligned16(out)) return KVC_EINVAL;
  if (num_state_rows > 0 && !aligned16(state)) return KVC_EINVAL;
  kvc::CompressArgs a{state, input, ape, plan_c, counts, out, num_state_rows, num_q, cap_c, {}};
  hipError_t e;
  if (st != nullptr) {
    a.st = *st;
    e = c4 ? kvc::launch_compress_c4_store(dtype, head_dim, a, as_stream(stream))
           : kvc::launch_compress_c128_store(dtype, head_dim, a, as_stream(stream));
  } else {
    e = c4 ? kvc::launch_compress_c4(dtype, head_dim, a, as_stream(stream))
           : kvc::launch_compress_c128(dtype, head_dim, a, as_stream(stream));
  }
  return status_of(e);
}

// out != nullptr: pooled rows to float32; st != nullptr (ratio 4): pool + norm + rotary + store
int decode_common(bool c4, kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows, const void* input,
                  const void* ape, const kvc_plan_d* plan_d, const int32_t* boundaries, int batch, int32_t* status,
                  float* out, const kvc_store_args* st, void* stream) {
  if (!dtype_ok(dtype) || !hd_ok(head_dim) || !rows_ok(num_state_rows)) return KVC_EINVAL;
  if (batch < 1 || batch > KVC_MAX_DECODE_BATCH) return KVC_EINVAL;
  if (!aligned16(input) || !aligned16(ape) || !aligned16(plan_d)) return KVC_EINVAL;
  if (st == nullptr ? !aligned16(out) : !store_args_ok(head_dim, st)) return KVC_EINVAL;
  if (num_state_rows > 0 && !aligned16(state)) return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  if (!boundaries_ok(c4 ? 4 : 128, boundaries)) return KVC_EINVAL;
  kvc::DecodeArgs a{state, input, ape, plan_d, status, out, num_state_rows, batch, {}, boundaries};
  hipError_t e;
  if (st != nullptr) {
    a.st = *st;
    e = kvc::launch_decode_c4_store(dtype, head_dim, a, as_stream(stream));
  } else {
    e = c4 ? kvc::launch_decode_c4(dtype, head_dim, a, as_stream(stream))
           : kvc::launch_decode_c128(dtype, head_dim, a, as_stream(stream));
  }
  return status_of(e);
}

}  // namespace

KVC_EXPORT int kvc_compress_c4(kvc_dtype dtype, int head_dim, const void* state, int64_t num_state_rows,
                               const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c, int cap_c,
                               int32_t* counts, float* out, void* stream) {
  return compress_common(true, dtype, head_dim, state, num_state_rows, input, num_q, ape, plan_c, cap_c, counts, out,
                         nullptr, stream);
}

KVC_EXPORT int kvc_compress_c128(kvc_dtype dtype, int head_dim, const void* state, int64_t num_state_rows,
                                 const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c, int cap_c,
                                 int32_t* counts, float* out, void* stream) {
  return compress_common(false, dtype, head_dim, state, num_state_rows, input, num_q, ape, plan_c, cap_c, counts,
                         out, nullptr, stream);
}

KVC_EXPORT int kvc_compress_c4_norm_rope_store(kvc_dtype dtype, int head_dim, const void* state,
                                               int64_t num_state_rows, const void* input, int num_q, const void* ape,
                                               const kvc_plan_c* plan_c, int cap_c, int32_t* counts,
                                               const kvc_store_args* args, void* stream) {
  if (args == nullptr) return KVC_EINVAL;
  return compress_common(true, dtype, head_dim, state, num_state_rows, input, num_q, ape, plan_c, cap_c, counts,
                         nullptr, args, stream);
}

KVC_EXPORT int kvc_compress_c128_norm_rope_store(kvc_dtype dtype, int head_dim, const void* state,
                                                 int64_t num_state_rows, const void* input, int num_q, const void* ape,
                                                 const kvc_plan_c* plan_c, int cap_c, int32_t* counts,
                                                 const kvc_store_args* args, void* stream) {
  if (args == nullptr) return KVC_EINVAL;
  return compress_common(false, dtype, head_dim, state, num_state_rows, input, num_q, ape, plan_c, cap_c, counts,
                         nullptr, args, stream);
}

KVC_EXPORT int kvc_norm_rope_store_prefill(int compress_ratio, int head_dim, const float* rows,
                                           const kvc_plan_c* plan_c, int cap_c, int32_t* counts,
                                           const kvc_store_args* args, void* stream) {
  if (!ratio_ok(compress_ratio) || !hd_ok(head_dim) || cap_c < 0 || cap_c >= KVC_MAX_TOKENS || !aligned4(counts))
    return KVC_EINVAL;
  if (!store_args_ok(head_dim, args)) return KVC_EINVAL;
  if (cap_c == 0) return KVC_OK;
  if (!aligned16(rows) || !aligned16(plan_c)) return KVC_EINVAL;
  const kvc::NormRopeStoreArgs a{rows, plan_c, nullptr, counts, nullptr, cap_c, compress_ratio, *args};
  return status_of(kvc::launch_norm_rope_store(head_dim, false, a, as_stream(stream)));
}

KVC_EXPORT int kvc_norm_rope_store_decode(int compress_ratio, int head_dim, const float* rows,
                                          const kvc_plan_d* plan_d, int batch, int32_t* status,
                                          const kvc_store_args* args, void* stream) {
  if (!ratio_ok(compress_ratio) || !hd_ok(head_dim) || batch < 1 || batch > KVC_MAX_DECODE_BATCH) return KVC_EINVAL;
  if (!store_args_ok(head_dim, args)) return KVC_EINVAL;
  if (!aligned16(rows) || !aligned16(plan_d)) return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  const kvc::NormRopeStoreArgs a{rows, nullptr, plan_d, nullptr, status, batch, compress_ratio, *args};
  return status_of(kvc::launch_norm_rope_store(head_dim, true, a, as_stream(stream)));
}

KVC_EXPORT int kvc_decode_c4(kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows, const void* input,
                             const void* ape, const kvc_plan_d* plan_d, int batch, int32_t* status, float* out,
                             void* stream) {
  return decode_common(true, dtype, head_dim, state, num_state_rows, input, ape, plan_d, nullptr, batch, status, out,
                       nullptr, stream);
}

KVC_EXPORT int kvc_decode_c128(kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows, const void* input,
                               const void* ape, const kvc_plan_d* plan_d, const int32_t* boundaries, int batch,
                               int32_t* status, float* out, void* stream) {
  return decode_common(false, dtype, head_dim, state, num_state_rows, input, ape, plan_d, boundaries, batch, status,
                       out, nullptr, stream);
}

KVC_EXPORT int kvc_decode_c4_norm_rope_store(kvc_dtype dtype, int head_dim, void* state, int64_t num_state_rows,
                                             const void* input, const void* ape, const kvc_plan_d* plan_d, int batch,
                                             int32_t* status, const kvc_store_args* args, void* stream) {
  if (args == nullptr) return KVC_EINVAL;
  return decode_common(true, dtype, head_dim, state, num_state_rows, input, ape, plan_d, nullptr, batch, status,
                       nullptr, args, stream);
}

namespace {

bool online_common_ok(kvc_dtype dtype, int head_dim, const float* state, int64_t num_slots, const void* input,
                      const void* ape) {
  if (!dtype_ok(dtype) || !hd_ok(head_dim) || num_slots < 0 || num_slots > INT32_MAX / 128) return false;
  if (!aligned16(input) || !aligned16(ape)) return false;
  return num_slots == 0 || aligned16(state);
}

}  // namespace

KVC_EXPORT int kvc_compress_c128_online(kvc_dtype dtype, int head_dim, const float* state, int64_t num_slots,
                                        const void* input, int num_q, const void* ape, const kvc_plan_c* plan_c,
                                        int cap_c, int32_t* counts, float* out, void* stream) {
  if (!online_common_ok(dtype, head_dim, state, num_slots, input, ape)) return KVC_EINVAL;
  if (num_q < 0 || num_q >= KVC_MAX_TOKENS || cap_c < 0 || !aligned4(counts)) return KVC_EINVAL;
  if (cap_c == 0) return KVC_OK;
  if (!aligned16(plan_c) || !aligned16(out)) return KVC_EINVAL;
  kvc::OnlineArgs a{};
  a.state = const_cast<float*>(state);
  a.input = input;
  a.ape = ape;
  a.plan_c = plan_c;
  a.counts = counts;
  a.out = out;
  a.num_slots = num_slots;
  a.num_q = num_q;
  a.cap = cap_c;
  return status_of(kvc::launch_compress_online(dtype, head_dim, a, as_stream(stream)));
}

KVC_EXPORT int kvc_write_c128_online(kvc_dtype dtype, int head_dim, float* state, int64_t num_slots,
                                     const void* input, int num_q, const void* ape, const kvc_plan_w* plan_w,
                                     int cap_w, int32_t* counts, const int32_t* runs, int batch, void* stream) {
  if (!online_common_ok(dtype, head_dim, state, num_slots, input, ape)) return KVC_EINVAL;
  if (num_q < 0 || num_q >= KVC_MAX_TOKENS || cap_w < 0 || !aligned4(counts)) return KVC_EINVAL;
  if (runs != nullptr && (!aligned16(runs) || batch < 1 || batch > KVC_MAX_PREFILL_BATCH)) return KVC_EINVAL;
  if (cap_w == 0) return KVC_OK;
  if (!aligned8(plan_w)) return KVC_EINVAL;
  kvc::OnlineArgs a{};
  a.state = state;
  a.input = input;
  a.ape = ape;
  a.plan_w = plan_w;
  a.counts = counts;
  a.runs = runs;
  a.num_slots = num_slots;
  a.num_q = num_q;
  a.cap = cap_w;
  a.batch = batch;
  return status_of(kvc::launch_write_online(dtype, head_dim, a, as_stream(stream)));
}

KVC_EXPORT int kvc_decode_c128_online(kvc_dtype dtype, int head_dim, float* state, int64_t num_slots,
                                      const void* input, const void* ape, const kvc_plan_d* plan_d, int batch,
                                      int32_t* status, float* out, void* stream) {
  if (!online_common_ok(dtype, head_dim, state, num_slots, input, ape)) return KVC_EINVAL;
  if (batch < 1 || batch > KVC_MAX_DECODE_BATCH || !aligned16(plan_d) || !aligned16(out)) return KVC_EINVAL;
  if (status != nullptr && !aligned4(status)) return KVC_EINVAL;
  kvc::OnlineArgs a{};
  a.state = state;
  a.input = input;
  a.ape = ape;
  a.plan_d = plan_d;
  a.status = status;
  a.out = out;
  a.num_slots = num_slots;
  a.cap = batch;
  return status_of(kvc::launch_decode_online(dtype, head_dim, a, as_stream(stream)));
}

KVC_EXPORT const char* kvc_strerror(int code) {
  switch (code) {
    case KVC_OK:
      return "ok";
    case KVC_EINVAL:
      return "invalid argument (nothing was enqueued)";
    case KVC_EHIP:
      return "HIP launch failed";
    case KVC_DERR_EXTEND:
      return "device data: extend_len <= 0 or > seq_len (decode: seq_len <= 0)";
    case KVC_DERR_NUMQ:
      return "device data: sum of extend_len != num_q";
    case KVC_DERR_INDEX:
      return "device data: state index outside the state buffer";
    case KVC_DERR_CAPACITY:
      return "device data: plan needs more records than cap_c / cap_w";
    case KVC_DERR_RECORD:
      return "device data: record points outside the input or the state";
    case KVC_DERR_DUPLICATE:
      return "device data: two requests of a prefill chunk share a state slot";
    default:
      return "unknown kvc code";
  }
}
