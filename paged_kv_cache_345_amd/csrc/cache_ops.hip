// Cache data-movement kernels: slot-mapped write, copy-on-write block copy and
// the paged -> contiguous inspection gather, for 16-bit and fp8 (E4M3) pages.
// All of them move bits only, except the fp8 write, which encodes.
//
// Slot model from page "vLLM 部署与 PagedAttention 原理 · 检索整理（CSDN 频道批次）",
// item 2: tokens fill fixed-size blocks reached through a block table, and a
// block shared by parallel samples is copied before it is written.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "cache_write.h"

namespace pkv {

// 16-bit slot-mapped write: one work-group per write item (cache_write.h).
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int64_t num_tokens,
    int num_kv_heads, int64_t num_slots) {
  write_rows16(blockIdx.x, k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, num_slots);
}

// fp8 (E4M3) cache write: write_rows_fp8 (cache_write.h) per work-group.
template <class DT>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int64_t num_tokens, int num_kv_heads,
    int64_t num_slots, float k_scale, float v_scale, const float* __restrict__ k_head_scales,
    const float* __restrict__ v_head_scales) {
  write_rows_fp8<DT>(blockIdx.x, k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, num_slots, k_scale,
                     v_scale, k_head_scales, v_head_scales);
}

// One work-group copies one page, 16 bytes per thread (256 threads for a
// 4 KiB 16-bit page, 128 for a 2 KiB fp8 page).  Work-group index -> (pair,
// which of the 2*Hkv pages of the block).  The stores are non-temporal: with
// the default policy the copied lines are still dirty in the memory-side cache
// when the step's attention kernel runs and slow it by ~4 us on a 128-sequence
// batch (measured on MI355X); this kernel takes the same time either way.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                          const int32_t* __restrict__ block_pairs, int num_kv_heads,
                                                          int32_t num_blocks, int page_bytes) {
  const int64_t wg = blockIdx.x;
  const int pages = 2 * num_kv_heads;
  const int64_t pair = wg / pages;
  const int page = static_cast<int>(wg - pair * pages);
  const int32_t src = block_pairs[2 * pair];
  const int32_t dst = block_pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* base = page < num_kv_heads ? k_cache : v_cache;
  const int h = page < num_kv_heads ? page : page - num_kv_heads;
  const uint4* s = reinterpret_cast<const uint4*>(base + (static_cast<int64_t>(src) * num_kv_heads + h) * page_bytes);
  char* d = base + (static_cast<int64_t>(dst) * num_kv_heads + h) * page_bytes;
  store16<kNonTemporal>(range_rsrc(d, page_bytes), 16u * threadIdx.x, s[threadIdx.x]);
}

// Block swap between two caches (typically the device pool and a pool in
// pinned host memory, reached through its device mapping): one work-group per
// page, 16 bytes per thread; the work-group index -> (pair, which of the
// 2*Hkv pages of the block).  Pairs with a block outside its own pool are
// skipped.
__global__ __launch_bounds__(256) void swap_blocks_kernel(char* __restrict__ dst_k, char* __restrict__ dst_v,
                                                          int32_t dst_blocks, const char* __restrict__ src_k,
                                                          const char* __restrict__ src_v, int32_t src_blocks,
                                                          const int32_t* __restrict__ block_pairs, int num_kv_heads,
                                                          int page_bytes) {
  const int64_t wg = blockIdx.x;
  const int pages = 2 * num_kv_heads;
  const int64_t pair = wg / pages;
  const int page = static_cast<int>(wg - pair * pages);
  const int32_t src = block_pairs[2 * pair];
  const int32_t dst = block_pairs[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const bool is_k = page < num_kv_heads;
  const int h = is_k ? page : page - num_kv_heads;
  const uint4* s = reinterpret_cast<const uint4*>((is_k ? src_k : src_v) +
                                                  (static_cast<int64_t>(src) * num_kv_heads + h) * page_bytes);
  uint4* d = reinterpret_cast<uint4*>((is_k ? dst_k : dst_v) + (static_cast<int64_t>(dst) * num_kv_heads + h) * page_bytes);
  d[threadIdx.x] = s[threadIdx.x];
}

// One work-group per (sequence, logical block).  Thread -> (token, head, chunk).
__global__ __launch_bounds__(256) void gather_cache_kernel(
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ out_offsets, int max_blocks_per_seq,
    int num_kv_heads, int32_t num_blocks) {
  const int64_t wg = blockIdx.x;
  const int64_t s = wg / max_blocks_per_seq;
  const int j = static_cast<int>(wg - s * max_blocks_per_seq);
  int64_t L = context_lens[s];
  if (L > static_cast<int64_t>(max_blocks_per_seq) * kBlockSize) L = static_cast<int64_t>(max_blocks_per_seq) * kBlockSize;
  const int64_t first = static_cast<int64_t>(j) * kBlockSize;
  if (first >= L) return;
  const int32_t block = block_tables[s * max_blocks_per_seq + j];
  if (block < 0 || block >= num_blocks) return;
  const int ntok = static_cast<int>(L - first < kBlockSize ? L - first : kBlockSize);
  const int64_t row0 = static_cast<int64_t>(out_offsets[s]) + first;
  const int work = kBlockSize * num_kv_heads * 16;
  for (int idx = threadIdx.x; idx < work; idx += blockDim.x) {
    const int c = idx & 15;
    const int t = (idx >> 4) & 15;
    const int h = idx >> 8;
    if (t >= ntok) continue;
    const int64_t page = (static_cast<int64_t>(block) * num_kv_heads + h) * kPageElems;
    const int64_t out_row = (row0 + t) * num_kv_heads + h;
    reinterpret_cast<uint4*>(k_out + out_row * kHeadSize)[c] =
        *reinterpret_cast<const uint4*>(k_cache + page + k_page_offset(t, 8 * c));
    uint16_t e16[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e16[e] = v_cache[page + v_page_offset(t, 8 * c + e)];
    uint4 packed;
    packed.x = e16[0] | (static_cast<uint32_t>(e16[1]) << 16);
    packed.y = e16[2] | (static_cast<uint32_t>(e16[3]) << 16);
    packed.z = e16[4] | (static_cast<uint32_t>(e16[5]) << 16);
    packed.w = e16[6] | (static_cast<uint32_t>(e16[7]) << 16);
    reinterpret_cast<uint4*>(v_out + out_row * kHeadSize)[c] = packed;
  }
}

// fp8 pages -> contiguous rows of codes (one byte per element).
__global__ __launch_bounds__(256) void gather_cache_fp8_kernel(
    uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ out_offsets, int max_blocks_per_seq,
    int num_kv_heads, int32_t num_blocks) {
  const int64_t wg = blockIdx.x;
  const int64_t s = wg / max_blocks_per_seq;
  const int j = static_cast<int>(wg - s * max_blocks_per_seq);
  int64_t L = context_lens[s];
  if (L > static_cast<int64_t>(max_blocks_per_seq) * kBlockSize) L = static_cast<int64_t>(max_blocks_per_seq) * kBlockSize;
  const int64_t first = static_cast<int64_t>(j) * kBlockSize;
  if (first >= L) return;
  const int32_t block = block_tables[s * max_blocks_per_seq + j];
  if (block < 0 || block >= num_blocks) return;
  const int ntok = static_cast<int>(L - first < kBlockSize ? L - first : kBlockSize);
  const int64_t row0 = static_cast<int64_t>(out_offsets[s]) + first;
  const int work = kBlockSize * num_kv_heads * 16;
  for (int idx = threadIdx.x; idx < work; idx += blockDim.x) {
    const int c = idx & 15;
    const int t = (idx >> 4) & 15;
    const int h = idx >> 8;
    if (t >= ntok) continue;
    const int64_t page = (static_cast<int64_t>(block) * num_kv_heads + h) * kPageBytesFp8;
    const int64_t out_row = (row0 + t) * num_kv_heads + h;
    reinterpret_cast<uint2*>(k_out + out_row * kHeadSize)[c] =
        *reinterpret_cast<const uint2*>(k_cache + page + k_page_offset_fp8(t, 8 * c));
    uint2 packed = make_uint2(0u, 0u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      packed.x |= static_cast<uint32_t>(v_cache[page + v_page_offset_fp8(t, 8 * c + e)]) << (8 * e);
      packed.y |= static_cast<uint32_t>(v_cache[page + v_page_offset_fp8(t, 8 * c + 4 + e)]) << (8 * e);
    }
    reinterpret_cast<uint2*>(v_out + out_row * kHeadSize)[c] = packed;
  }
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t num_blocks, hipStream_t stream) {
  // one work-group per (window of 4 tokens, group of 4 KV heads), rounded up to the XCD count
  const int64_t items = (static_cast<int64_t>(num_tokens) + 3) / 4 * ((num_kv_heads + 3) / 4);
  const int64_t grid = (items + kNumXcd - 1) / kNumXcd * kNumXcd;
  reshape_and_cache_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(k_cache),
      static_cast<uint16_t*>(v_cache), slot_mapping, num_tokens, num_kv_heads,
      static_cast<int64_t>(num_blocks) * kBlockSize);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                        const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t num_blocks, int act_dtype, float k_scale, float v_scale,
                                        const float* k_head_scales, const float* v_head_scales,
                                        hipStream_t stream) {
  // one work-group per (window of 4 tokens, group of 4 KV heads), as above
  const int64_t items = (static_cast<int64_t>(num_tokens) + 3) / 4 * ((num_kv_heads + 3) / 4);
  const dim3 g(static_cast<uint32_t>((items + kNumXcd - 1) / kNumXcd * kNumXcd)), b(256);
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  const int64_t slots = static_cast<int64_t>(num_blocks) * kBlockSize;
  if (act_dtype == 0)
    reshape_and_cache_fp8_kernel<F16><<<g, b, 0, stream>>>(kk, vv, kc, vc, slot_mapping, num_tokens, num_kv_heads,
                                                            slots, k_scale, v_scale, k_head_scales, v_head_scales);
  else
    reshape_and_cache_fp8_kernel<BF16><<<g, b, 0, stream>>>(kk, vv, kc, vc, slot_mapping, num_tokens, num_kv_heads,
                                                             slots, k_scale, v_scale, k_head_scales, v_head_scales);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t num_blocks, int32_t page_bytes, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(num_pairs) * 2 * num_kv_heads;
  copy_blocks_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(page_bytes / 16), 0, stream>>>(
      static_cast<char*>(k_cache), static_cast<char*>(v_cache), block_pairs, num_kv_heads, num_blocks, page_bytes);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k, const void* src_v,
                              int32_t src_blocks, const int32_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                              int32_t page_bytes, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(num_pairs) * 2 * num_kv_heads;
  swap_blocks_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(page_bytes / 16), 0, stream>>>(
      static_cast<char*>(dst_k), static_cast<char*>(dst_v), dst_blocks, static_cast<const char*>(src_k),
      static_cast<const char*>(src_v), src_blocks, block_pairs, num_kv_heads, page_bytes);
  return hipGetLastError();
}

hipError_t launch_gather_cache(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, const int32_t* out_offsets, int32_t num_kv_heads,
                               int32_t num_blocks, bool fp8_cache, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(num_seqs) * max_blocks_per_seq;
  if (fp8_cache)
    gather_cache_fp8_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(
        static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out), static_cast<const uint8_t*>(k_cache),
        static_cast<const uint8_t*>(v_cache), block_tables, context_lens, out_offsets, max_blocks_per_seq,
        num_kv_heads, num_blocks);
  else
    gather_cache_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(
        static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out), static_cast<const uint16_t*>(k_cache),
        static_cast<const uint16_t*>(v_cache), block_tables, context_lens, out_offsets, max_blocks_per_seq,
        num_kv_heads, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
