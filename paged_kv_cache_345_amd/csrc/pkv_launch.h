// Host-side launch interface between the C ABI (api.hip) and the kernel
// translation units (decode.hip, plan.hip, cache_ops.hip).

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Work-list plan of one decode call, written by decode_plan_kernel into the
// caller's workspace and read by the decode kernels.  A work item is one
// segment (blocks_per_part consecutive blocks) of one row (sequence, unit).
// Int offsets into `plan`:
constexpr int kPlanFull = 0;         // F: full segments per unit
constexpr int kPlanPartial = 1;      // P: partial (last) segments per unit
constexpr int kPlanClasses = 32;     // list B classes: up to 16 partial-size buckets and the empties (power of 2)
constexpr int kPlanClassOff = 16;    // [16, 16 + kPlanClasses]: class offsets into list B
constexpr int kPlanHeaderInts = 512;
// list_A (F entries, packed s | g << 20) follows the header; list_B (one
// sequence id per partial segment or empty sequence, P entries) follows
// list_A's capacity of num_seqs * parts_max entries.
constexpr int kPlanSeqBits = 20;
constexpr int kPlanMaxSeqs = 4096;   // sequences one plan covers (LDS bound)
constexpr int kPlanMaxTasks = 6144;  // (segments + size classes) x 64-sequence chunks (LDS bound)

struct DecodeArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;     // [S, Hq, parts_max, 128] unnormalised partial outputs
  float* ws_ml;    // [S, Hq, parts_max, 2]   (running max in log2 units, Z)
  int* plan;       // work-list plan (planned mode) or null
  float scale_log2e;  // logit scale (times the one K scale of an fp8 cache) in log2 units
  float out_scale;    // 1, or the one V scale of an fp8 cache
  const float* k_head_scales;  // fp8 cache with per-KV-head K scales, else null: logits of head h * [h]
  const float* v_head_scales;  // fp8 cache with per-KV-head V scales, else null: outputs of head h * [h]
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;       // num_heads / num_kv_heads
  int head_tiles;  // ceil(group / 16)
  int units;       // work units per sequence: num_kv_heads * (group == 1 ? 1 : head_tiles)
  int max_blocks_per_seq;
  int num_blocks;
  int blocks_per_part;  // segment length in blocks (<= 4 x 64: each wave streams at most 64)
  int parts_max;        // segments of the longest possible row
  int planned;  // 1: items come from the plan's work list; 0: from blockIdx directly
};

// Chunked prefill: chunk query j of sequence s (output row query_start[s] + j)
// sits at position context_lens[s] - C_s + j and attends to cache tokens
// 0 .. that position.  A work-group takes kPrefillTiles x 4 tiles of 16 rows
// (query position, head) of one KV head: tile i of the work-group covers the
// positions [8 ppt qb + i ppt, + ppt) for heads_per_tile heads each; wave w
// holds tiles kPrefillTiles w .. + kPrefillTiles - 1, and the work-group
// stages the blocks it streams in LDS once for all its waves.
constexpr int kPrefillTiles = 2;  // 16-row tiles per wave
struct PrefillArgs {
  DecodeArgs d;                // out, q and the partials are per query token
  const int32_t* query_start;  // [num_seqs + 1]
  int heads_per_tile;          // hpt = min(group, 16)
  int pos_per_wave;            // ppt = 16 / hpt: positions per tile
  int q_blocks;                // ceil(max_query_len / (4 kPrefillTiles ppt))
  int num_query_tokens;
};

struct PlanArgs {
  const int32_t* context_lens;
  int* plan;
  int num_seqs;
  int num_heads;
  int units;
  int max_blocks_per_seq;
  int blocks_per_part;
  int parts_max;
  int scan;  // 1: at most one sequence per thread of the plan work-group (plan_body.h's wave-per-chunk path)
};

// The fused decode-step prologue (step.hip): copy_blocks, reshape_and_cache
// and the plan in one launch over a 16-bit cache.  Its plan work-group has 256
// threads and smaller LDS tables than decode_plan_kernel, so the launch keeps
// 7 work-groups per compute unit for the copy and write roles.
constexpr int kPlanThreads = 1024;  // decode_plan_kernel
constexpr int kStepThreads = 256;   // decode_step_prologue_kernel
constexpr int kStepPlanMaxSeqs = 1024;
constexpr int kStepPlanMaxTasks = 2048;
constexpr int kStepPlanMaxParts = 1024;
struct StepArgs {
  const uint16_t* k;  // [num_tokens, num_kv_heads, 128] new rows
  const uint16_t* v;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* slot_mapping;
  const int32_t* block_pairs;  // [num_pairs][2] (src, dst)
  int64_t num_tokens;
  int num_pairs;
  int num_kv_heads;
  int32_t num_blocks;
  int planned;      // 1: the plan work-group writes the plan
  PlanArgs plan;
  int64_t plan_wg;  // the plan work-group: after the write work-groups, before the copies (set by the launcher)
  // fp8 caches (k_cache / v_cache then hold E4M3 codes): the write's scales
  float k_scale, v_scale;
  const float* k_head_scales;  // [num_kv_heads] or null
  const float* v_head_scales;
};

// act_dtype: 0 fp16, 1 bf16 (q, out); fp8_cache: the pages hold E4M3 codes
hipError_t launch_decode(const DecodeArgs& a, int act_dtype, bool fp8_cache, hipStream_t stream);
hipError_t launch_decode_plan(const PlanArgs& a, hipStream_t stream);
hipError_t launch_decode_read_pages(const DecodeArgs& a, bool fp8_cache, uint32_t* sink, hipStream_t stream);
// fp8_cache: the pages hold E4M3 codes and the rows are act_dtype (0 fp16, 1 bf16)
hipError_t launch_decode_step_prologue(const StepArgs& a, bool fp8_cache, int act_dtype, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int act_dtype, bool fp8_cache, hipStream_t stream);
hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t num_blocks, hipStream_t stream);
hipError_t launch_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                        const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t num_blocks, int act_dtype, float k_scale, float v_scale,
                                        const float* k_head_scales, const float* v_head_scales,
                                        hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t num_blocks, int32_t page_bytes, hipStream_t stream);
hipError_t launch_swap_blocks(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k, const void* src_v,
                              int32_t src_blocks, const int32_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                              int32_t page_bytes, hipStream_t stream);
hipError_t launch_gather_cache(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, const int32_t* out_offsets, int32_t num_kv_heads,
                               int32_t num_blocks, bool fp8_cache, hipStream_t stream);

}  // namespace pkv
