// Host-side launch interface between the C ABI (api.hip) and the kernel
// translation units (decode.hip, cache_ops.hip).

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct DecodeArgs {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;   // [S, Hq, parts_max, 128] unnormalised partial outputs
  float* ws_ml;  // [S, Hq, parts_max, 2]   (running max in log2 units, Z)
  float scale_log2e;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;       // num_heads / num_kv_heads
  int head_tiles;  // ceil(group / 16)
  int max_blocks_per_seq;
  int num_blocks;
  int blocks_per_part;
  int parts_max;
};

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream);
hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t num_blocks, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t num_blocks, hipStream_t stream);
hipError_t launch_gather_cache(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, const int32_t* out_offsets, int32_t num_kv_heads,
                               int32_t num_blocks, hipStream_t stream);

}  // namespace pkv
