// kvc_launch.hpp - internal launchers, one per kernel family.  The C entry
// points in kvc_api.hip check host arguments and call these; each launcher
// only enqueues its kernel and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// SWA-paged state tables (used by the *_swa planners only)
struct SwaTables {
  const int32_t* req_to_token;  // [num_reqs, stride]
  const int32_t* full_to_swa;   // [num_full]
  int64_t stride;
  int64_t num_reqs;
  int64_t num_full;
  int swa_page_size;
  int ring_size;
};

// how plan records name state rows: the per-request ring or page, the SWA
// pool's rings, or 4-row pages that the caller hands over (ratio 4)
enum PlanMap { kPlanRing = 0, kPlanSwa = 1, kPlanPage4 = 2 };

struct PlanPrefillArgs {
  const int32_t* seq_lens;
  const int32_t* extend_lens;
  const int32_t* state_index;  // request pool indices in SWA mode
  int64_t num_state_rows;
  kvc_plan_c* plan_c;
  kvc_plan_w* plan_w;
  int32_t* counts;
  int32_t* status;  // SWA mode: OR of record lookup errors (may be null)
  int batch;
  int num_q;
  int cap_c;
  int cap_w;
  SwaTables swa;
  const int32_t* bundle;  // page-4 mode: [batch, 4] load_first, load_second, write_first page, last position
  int32_t* runs;          // ratio 128, per-request pages, may be null: each request's W run (int32 [batch, 4])
};

struct PlanDecodeArgs {
  const int32_t* seq_lens;
  const int32_t* state_index;
  int64_t num_state_rows;
  kvc_plan_d* plan_d;
  int32_t* status;
  int batch;
  SwaTables swa;
  const int32_t* prev_page;  // page-4 mode: [batch] page of the block before the new token's
  int32_t* boundaries;       // ratio 128, may be null: the boundary list (int32 [2 * batch + 2])
};

struct WriteArgs {
  void* state;
  const void* input;
  const kvc_plan_w* plan_w;
  int32_t* counts;
  int64_t num_state_rows;
  int num_q;
  int cap_w;
  int row_vecs;  // 16-byte vectors per row
};

struct CompressArgs {
  const void* state;
  const void* input;
  const void* ape;
  const kvc_plan_c* plan_c;
  int32_t* counts;
  float* out;  // pool only
  int64_t num_state_rows;
  int num_q;
  int cap_c;
  kvc_store_args st;  // pool + norm + rotary + store only
};

struct DecodeArgs {
  void* state;
  const void* input;
  const void* ape;
  const kvc_plan_d* plan_d;
  int32_t* status;
  float* out;  // decode only
  int64_t num_state_rows;
  int batch;
  kvc_store_args st;               // decode + norm + rotary + store only
  const int32_t* boundaries;       // ratio 128, may be null: the planner's boundary list
};

// norm + rotary + store of float32 rows (prefill: plan_c / counts; decode: plan_d / status)
struct NormRopeStoreArgs {
  const float* rows;
  const kvc_plan_c* plan_c;
  const kvc_plan_d* plan_d;
  int32_t* counts;
  int32_t* status;
  int n;  // cap_c or batch
  int compress_ratio;
  kvc_store_args st;
};

// the ratio-128 online state: slots [num_slots, 3, hd] fp32 (m, l, acc)
struct OnlineArgs {
  float* state;
  const void* input;
  const void* ape;
  const kvc_plan_c* plan_c;  // compress
  const kvc_plan_w* plan_w;  // write
  const kvc_plan_d* plan_d;  // decode
  int32_t* counts;           // compress (counts[0], [3]) and write (counts[1], [3])
  int32_t* status;           // decode (may be null)
  float* out;                // compress and decode
  const int32_t* runs;       // write, may be null: the planner's run list (int32 [batch, 4])
  int64_t num_slots;
  int num_q;
  int cap;  // cap_c, cap_w or batch
  int batch;  // write with a run list: its entries
};

hipError_t launch_plan_prefill(int compress_ratio, int map, const PlanPrefillArgs& a, hipStream_t stream);
hipError_t launch_plan_decode(int compress_ratio, int map, const PlanDecodeArgs& a, hipStream_t stream);
hipError_t launch_write(const WriteArgs& a, hipStream_t stream);
hipError_t launch_compress_c4(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream);
hipError_t launch_compress_c128(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream);
hipError_t launch_compress_c4_store(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream);
hipError_t launch_compress_c128_store(kvc_dtype dtype, int head_dim, const CompressArgs& a, hipStream_t stream);
hipError_t launch_norm_rope_store(int head_dim, bool decode, const NormRopeStoreArgs& a, hipStream_t stream);
hipError_t launch_decode_c4(kvc_dtype dtype, int head_dim, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_c4_store(kvc_dtype dtype, int head_dim, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_compress_online(kvc_dtype dtype, int head_dim, const OnlineArgs& a, hipStream_t stream);
hipError_t launch_write_online(kvc_dtype dtype, int head_dim, const OnlineArgs& a, hipStream_t stream);
hipError_t launch_decode_online(kvc_dtype dtype, int head_dim, const OnlineArgs& a, hipStream_t stream);
hipError_t launch_decode_c128(kvc_dtype dtype, int head_dim, const DecodeArgs& a, hipStream_t stream);

}  // namespace kvc
