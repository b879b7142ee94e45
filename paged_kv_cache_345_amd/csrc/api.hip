// C ABI of libpagedkv: argument validation, partition choice, workspace
// sizing and kernel launches on the caller's stream.  See include/pagedkv.h
// for the contract of each entry point.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "pagedkv.h"
#include "pkv_device.h"
#include "pkv_launch.h"


namespace {

constexpr double kLog2e = 1.4426950408889634073599246810019;

pkv_status check_desc(const pkv_cache_desc* c) {
  if (!c) return PKV_ERR_INVALID;
  if (c->block_size != pkv::kBlockSize || c->head_size != pkv::kHeadSize) return PKV_ERR_UNSUPPORTED;
  if (c->dtype != PKV_F16 && c->dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PKV_ERR_INVALID;
  // every page offset must fit int64 comfortably and every slot an int32
  if (static_cast<int64_t>(c->num_blocks) * pkv::kBlockSize > INT32_MAX) return PKV_ERR_INVALID;
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Partition length in blocks.  Automatic choice: 16 blocks (256 tokens); 32
// blocks (512 tokens) once a row can hold more than 8192 tokens; doubled
// further only if the partition count would exceed the reduce kernel's bound.
pkv_status resolve_partition(int32_t max_blocks_per_seq, int32_t partition_tokens, int32_t* bpp_out,
                             int32_t* parts_out) {
  int32_t bpp;
  if (partition_tokens == 0) {
    bpp = max_blocks_per_seq > 512 ? 32 : 16;
    while ((max_blocks_per_seq + bpp - 1) / bpp > pkv::kMaxPartitions && bpp < pkv::kMaxBlocksPerPartition) bpp *= 2;
  } else {
    if (partition_tokens < pkv::kBlockSize || partition_tokens % pkv::kBlockSize != 0 ||
        partition_tokens > pkv::kBlockSize * pkv::kMaxBlocksPerPartition)
      return PKV_ERR_INVALID;
    bpp = partition_tokens / pkv::kBlockSize;
  }
  const int32_t parts = (max_blocks_per_seq + bpp - 1) / bpp;
  if (parts > pkv::kMaxPartitions) return PKV_ERR_UNSUPPORTED;
  *bpp_out = bpp;
  *parts_out = parts;
  return PKV_OK;
}

pkv_status check_decode_shape(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                              const pkv_cache_desc* cache) {
  pkv_status st = check_desc(cache);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_heads <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID;
  if (num_heads % cache->num_kv_heads != 0) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(max_blocks_per_seq) * pkv::kBlockSize > INT32_MAX) return PKV_ERR_INVALID;
  return PKV_OK;
}

size_t workspace_bytes_for(int32_t num_seqs, int32_t num_heads, int32_t parts) {
  if (parts <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * static_cast<size_t>(num_heads) * static_cast<size_t>(parts);
  return rows * (pkv::kHeadSize + 2) * sizeof(float);
}

pkv_status from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_DEVICE; }

}  // namespace

extern "C" {

size_t pkv_cache_bytes(const pkv_cache_desc* cache) {
  if (check_desc(cache) != PKV_OK) return 0;
  return static_cast<size_t>(cache->num_blocks) * static_cast<size_t>(cache->num_kv_heads) * pkv::kPageElems * 2;
}

int64_t pkv_k_index(const pkv_cache_desc* c, int32_t block, int32_t head, int32_t token, int32_t dim) {
  if (check_desc(c) != PKV_OK || block < 0 || block >= c->num_blocks || head < 0 || head >= c->num_kv_heads ||
      token < 0 || token >= pkv::kBlockSize || dim < 0 || dim >= pkv::kHeadSize)
    return -1;
  return (static_cast<int64_t>(block) * c->num_kv_heads + head) * pkv::kPageElems + pkv::k_page_offset(token, dim);
}

int64_t pkv_v_index(const pkv_cache_desc* c, int32_t block, int32_t head, int32_t token, int32_t dim) {
  if (check_desc(c) != PKV_OK || block < 0 || block >= c->num_blocks || head < 0 || head >= c->num_kv_heads ||
      token < 0 || token >= pkv::kBlockSize || dim < 0 || dim >= pkv::kHeadSize)
    return -1;
  return (static_cast<int64_t>(block) * c->num_kv_heads + head) * pkv::kPageElems + pkv::v_page_offset(token, dim);
}

int32_t paged_attn_decode_partition_tokens(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                           int32_t partition_tokens, const pkv_cache_desc* cache) {
  if (check_decode_shape(num_seqs, num_heads, max_blocks_per_seq, cache) != PKV_OK) return -1;
  int32_t bpp, parts;
  if (resolve_partition(max_blocks_per_seq, partition_tokens, &bpp, &parts) != PKV_OK) return -1;
  return bpp * pkv::kBlockSize;
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                        int32_t partition_tokens, const pkv_cache_desc* cache) {
  if (check_decode_shape(num_seqs, num_heads, max_blocks_per_seq, cache) != PKV_OK) return static_cast<size_t>(-1);
  int32_t bpp, parts;
  if (resolve_partition(max_blocks_per_seq, partition_tokens, &bpp, &parts) != PKV_OK) return static_cast<size_t>(-1);
  return workspace_bytes_for(num_seqs, num_heads, parts);
}

pkv_status paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, float scale,
                             int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                             const pkv_cache_desc* cache, int32_t partition_tokens, void* workspace,
                             size_t workspace_bytes, void* stream) {
  pkv_status st = check_decode_shape(num_seqs, num_heads, max_blocks_per_seq, cache);
  if (st != PKV_OK) return st;
  if (num_kv_heads != cache->num_kv_heads) return PKV_ERR_INVALID;
  if (!std::isfinite(scale)) return PKV_ERR_INVALID;
  int32_t bpp, parts;
  st = resolve_partition(max_blocks_per_seq, partition_tokens, &bpp, &parts);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  const size_t need = workspace_bytes_for(num_seqs, num_heads, parts);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return PKV_ERR_INVALID;

  pkv::DecodeArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t rows = static_cast<size_t>(num_seqs) * static_cast<size_t>(num_heads) * static_cast<size_t>(parts);
  a.ws_o = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = need ? static_cast<float*>(workspace) + rows * pkv::kHeadSize : nullptr;
  a.scale_log2e = static_cast<float>(static_cast<double>(scale) * kLog2e);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.head_tiles = (a.group + 15) / 16;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = cache->num_blocks;
  a.blocks_per_part = bpp;
  a.parts_max = parts;
  return from_hip(pkv::launch_decode(a, cache->dtype, static_cast<hipStream_t>(stream)));
}

pkv_status reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int32_t num_tokens, const pkv_cache_desc* cache,
                             void* stream) {
  pkv_status st = check_desc(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  // keep each launch's grid well inside 2^31 work-groups
  const int32_t chunk = static_cast<int32_t>(((int64_t{1} << 30) * 16) / (int64_t{16} * cache->num_kv_heads));
  for (int32_t t0 = 0; t0 < num_tokens; t0 += chunk) {
    const int32_t n = num_tokens - t0 < chunk ? num_tokens - t0 : chunk;
    const size_t row_off = static_cast<size_t>(t0) * static_cast<size_t>(cache->num_kv_heads) * pkv::kHeadSize;
    hipError_t e = pkv::launch_reshape_and_cache(static_cast<const uint16_t*>(k) + row_off,
                                                 static_cast<const uint16_t*>(v) + row_off, k_cache, v_cache,
                                                 slot_mapping + t0, n, cache->num_kv_heads, cache->num_blocks,
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PKV_ERR_DEVICE;
  }
  return PKV_OK;
}

pkv_status copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                       const pkv_cache_desc* cache, void* stream) {
  pkv_status st = check_desc(cache);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_ERR_INVALID;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_pairs) return PKV_ERR_INVALID;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(num_pairs) * 2 * cache->num_kv_heads > INT32_MAX) return PKV_ERR_INVALID;
  return from_hip(pkv::launch_copy_blocks(k_cache, v_cache, block_pairs, num_pairs, cache->num_kv_heads,
                                          cache->num_blocks, static_cast<hipStream_t>(stream)));
}

pkv_status gather_cache(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_blocks_per_seq, const int32_t* out_offsets, const pkv_cache_desc* cache,
                        void* stream) {
  pkv_status st = check_desc(cache);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!k_out || !v_out || !k_cache || !v_cache || !block_tables || !context_lens || !out_offsets)
    return PKV_ERR_INVALID;
  if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(num_seqs) * max_blocks_per_seq > INT32_MAX) return PKV_ERR_INVALID;
  return from_hip(pkv::launch_gather_cache(k_out, v_out, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                           max_blocks_per_seq, out_offsets, cache->num_kv_heads, cache->num_blocks,
                                           static_cast<hipStream_t>(stream)));
}

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_DEVICE: return "HIP launch or runtime failure";
    case PKV_ERR_OUT_OF_BLOCKS: return "out of free blocks";
  }
  return "unknown status";
}

const char* pkv_version(void) { return "pagedkv 0.1 (gfx950)"; }

}  // extern "C"
