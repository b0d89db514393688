// mla_kernels.h -- kernel parameter blocks and launchers (library-internal).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/mla_decode.h"

namespace mla {

struct SplitParams {
  const uint16_t* q_nope;
  const uint16_t* q_pe;
  const void* kv;               // latent part of cache rows (16-bit, or E4M3 bytes)
  const void* kpe;              // RoPE part of cache rows
  const int32_t* block_table;   // paged only
  const int32_t* seqlens;
  int32_t* num_splits;          // planner mode: written by workgroup 0 for the combine
  int32_t* split_offset;        // planner mode: [B + 1], written by workgroup 0
  int32_t* work;                // planner mode: work list (4 ints per item), written by workgroup 0
  uint16_t* out;
  float* lse;
  uint16_t* part16;             // [max_work, H, 512] fp16 normalised partial rows (every row)
  float* part32;                // [max_work, H, 512] fp32 copies of rows with values beyond +-1
  float* part_lse;              // [max_work, H], base 2; low mantissa bit set: the row has an fp32 copy
  int64_t q_nope_sb, q_nope_sh, q_pe_sb, q_pe_sh;
  int64_t kv_sb, kv_sr, kpe_sb, kpe_sr;
  int64_t out_sb, out_sh;
  int32_t num_split;            // > 0 forced splits per sequence (the tail included), 0 planner mode,
                                // kPlanGiven: num_splits / split_offset / work hold a plan made
                                // beforehand (read only), num_cus its capacity in work items
  int32_t seqlen_q;             // query tokens per sequence (>= 1)
  int32_t heads_per_token;      // heads / seqlen_q
  int32_t batch, heads;
  int32_t page_size, bt_stride;
  int32_t num_pages;            // paged: page indices are clamped to [0, num_pages)
  int32_t row_cap;              // lengths are clamped to [0, row_cap]
  int32_t num_cus;              // planner mode: the planner's CU count; kPlanGiven: the plan's capacity
  float scale_log2;             // softmax_scale * log2(e) (* kv_scale for an FP8 cache)
  float out_scale;              // FP8 cache: kv_scale (values are decode(byte) * kv_scale); else 1
};

// SplitParams::num_split of a call with a plan made beforehand (one more
// field would cost the split kernel scalar registers inside its tile loop).
constexpr int32_t kPlanGiven = -1;

struct CombineParams {
  const uint16_t* part16;       // [max_work, H, 512] fp16 partial rows
  const float* part32;          // fp32 copies (rows whose lse has the low bit set)
  const float* part_lse;
  const int32_t* split_offset;  // planner mode
  uint16_t* out;
  float* lse;
  int64_t out_sb, out_sh;
  int32_t num_split;
  int32_t heads;
  int32_t max_work;             // split_offset values are clamped to [0, max_work]
};

struct PlanParams {
  const int32_t* seqlens;
  int32_t* num_splits;
  int32_t* split_offset;
  int32_t* work;
  int32_t batch, heads, num_split, num_cus, seqlen_q;
  int32_t row_cap;              // lengths are clamped to [0, row_cap]
};

struct BlockCheckParams {
  const int32_t* block_table;
  const int32_t* seqlens;
  int32_t* bad;                 // [B] out: entries read and outside [0, num_pages)
  int32_t page_size, bt_stride, num_pages;
  int32_t row_cap;              // lengths are clamped to [0, row_cap] (as in the split kernel)
};

hipError_t launch_plan(const PlanParams& p, hipStream_t stream);
hipError_t launch_check_block_table(const BlockCheckParams& p, int batch, hipStream_t stream);
// This device's no-allocation scratch array: its device address (taken once
// per device with hipGetSymbolAddress) and size (MLA_NOALLOC_SCRATCH_BYTES).
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
// t0 / t1: events that time the launch from its dispatch packet, or null.
// kv8: the cache holds E4M3 bytes (queries and output in `dtype`).
hipError_t launch_split(const SplitParams& p, int dtype, bool paged, bool kv8, int grid_x, int grid_y,
                        hipStream_t stream, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// mean_splits: splits per sequence, on average (forced count, or the plan's
// bound over the batch); from kCombineSplitkMin on, four waves share a head.
constexpr int kCombineSplitkMin = 16;
hipError_t launch_combine(const CombineParams& p, int dtype, int batch, int mean_splits, hipStream_t stream,
                          hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

}  // namespace mla
