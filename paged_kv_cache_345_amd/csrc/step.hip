// The decode-step prologue in one launch: the copy-on-write block copy, the
// slot-mapped write of the new tokens and the attention work-list plan, which
// a decode step otherwise runs as three kernels before the attention.
//
// Mechanism from page "vLLM 部署与 PagedAttention 原理 · 检索整理（CSDN 频道批次）",
// item 2: parallel samples share prompt blocks by reference count, and a
// shared block is copied before a sample writes into it.
//
// 16-bit and fp8 (E4M3) caches; the fp8 form encodes the new rows as the fp8
// write does.  Work-groups (256 threads each) take one of three roles by
// index, the longest-running first, since work-groups start in index order:
//   * from 0: the slot-mapped write (cache_write.h), in the write kernel's XCD
//     order (its first index is a multiple of 8);
//   * the next one: the plan (plan_body.h), when the call is planned;
//   * the next 2 * Hkv * num_pairs: one page of one copy pair each.  The copy
//     of (src, dst) must see dst's new tokens land after it, so the work-group
//     that copies a page also merges into it, in registers before its single
//     store, every new token whose slot lies in dst.  The write work-groups
//     store those tokens too: both writers store the same bytes, so the order
//     between them does not matter.
// The merge reads slot_mapping whole in every copy work-group (one coalesced
// pass), which suits a decode step's few tokens.
//
// What the one launch saves on a 128-sequence, 40-head step (MI355X): three
// kernel boundaries and the plan's and the copy's own durations (~7.6 and
// ~5.2 us), which now run beside the write.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cache_write.h"
#include "pkv_device.h"
#include "pkv_launch.h"
#include "plan_body.h"

namespace pkv {

namespace {

// The copy of one page of pair `pair` (page < Hkv: K of head page; else V of
// head page - Hkv), with every new token whose slot lies in dst merged in.
// The work-group finds those tokens with one coalesced pass over
// slot_mapping (each thread tests one entry per 256), collecting them in LDS;
// with unique slots at most 16 tokens land in one block.
__device__ inline void copy_page_merged(const StepArgs& a, int64_t pair, int page) {
  __shared__ int match[kBlockSize];
  __shared__ int n_match;
  const int hkv = a.num_kv_heads;
  const int32_t src = a.block_pairs[2 * pair];
  const int32_t dst = a.block_pairs[2 * pair + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;  // the whole work-group
  const bool is_k = page < hkv;
  const int h = is_k ? page : page - hkv;
  uint16_t* base = is_k ? a.k_cache : a.v_cache;
  const int tid = threadIdx.x;
  uint4 val = reinterpret_cast<const uint4*>(base + (static_cast<int64_t>(src) * hkv + h) * kPageElems)[tid];
  if (tid == 0) n_match = 0;
  __syncthreads();
  const int64_t slot_lo = static_cast<int64_t>(dst) * kBlockSize;
  for (int64_t i = tid; i < a.num_tokens; i += kStepThreads) {
    const int32_t sl = a.slot_mapping[i];
    if (sl >= slot_lo && sl < slot_lo + kBlockSize) {
      const int k = atomicAdd(&n_match, 1);
      if (k < kBlockSize) match[k] = static_cast<int>(i);
    }
  }
  __syncthreads();
  const int n = n_match < kBlockSize ? n_match : kBlockSize;
  // thread tid holds 8 elements of the page.  K: token tid % 16, dims
  // 8 (tid / 16) .. + 8.  V: element e is token 4 ((tid % 64) / 16) + e % 4,
  // dim 32 (tid / 64) + 16 (e / 4) + tid % 16 (the page layouts in pkv_device.h).
  for (int m = 0; m < n; ++m) {
    const int64_t i = match[m];
    const int t0 = a.slot_mapping[i] & 15;
    const uint16_t* row = (is_k ? a.k : a.v) + (i * hkv + h) * kHeadSize;
    if (is_k) {
      if ((tid & 15) == t0) val = reinterpret_cast<const uint4*>(row)[tid >> 4];
    } else if (((tid & 63) >> 4) == (t0 >> 2)) {
      const int d0 = 32 * (tid >> 6) + (tid & 15);
      const uint32_t lo = row[d0], hi = row[d0 + 16];
      const int e = t0 & 3;  // elements e (dim d0) and 4 + e (dim d0 + 16)
      const int sh = 16 * (e & 1);
      const uint32_t keep = ~(0xffffu << sh);
      if ((e >> 1) == 0) {
        val.x = (val.x & keep) | (lo << sh);
        val.z = (val.z & keep) | (hi << sh);
      } else {
        val.y = (val.y & keep) | (lo << sh);
        val.w = (val.w & keep) | (hi << sh);
      }
    }
  }
  uint16_t* d = base + (static_cast<int64_t>(dst) * hkv + h) * kPageElems;
  store16<kNonTemporal>(page_rsrc(d), 16u * tid, val);
}

// The fp8 form of copy_page_merged: a 2 KiB page of E4M3 codes, 8 bytes per
// thread.  Thread tid's bytes: K page: token (tid / 2) % 16, dims d0 .. d0 + 7
// with d0 = 64 (tid / 128) + 32 (tid % 2) + 8 ((tid / 32) % 4); V page: byte
// 4 j + e is token 4 ((tid / 32) % 4) + e, dim dl + 16 j with dl = 64 (tid /
// 128) + 32 (tid % 2) + (tid / 2) % 16 (the fp8 page layouts in pkv_device.h).
// A merged token's codes come from encode_fp8 with the row's scale, as in the
// write, so both writers store the same bytes.
template <class DT>
__device__ inline void copy_page_merged_fp8(const StepArgs& a, int64_t pair, int page) {
  __shared__ int match[kBlockSize];
  __shared__ int n_match;
  const int hkv = a.num_kv_heads;
  const int32_t src = a.block_pairs[2 * pair];
  const int32_t dst = a.block_pairs[2 * pair + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;  // the whole work-group
  const bool is_k = page < hkv;
  const int h = is_k ? page : page - hkv;
  uint8_t* base = reinterpret_cast<uint8_t*>(is_k ? a.k_cache : a.v_cache);
  const int tid = threadIdx.x;
  uint2 val = reinterpret_cast<const uint2*>(base + (static_cast<int64_t>(src) * hkv + h) * kPageBytesFp8)[tid];
  if (tid == 0) n_match = 0;
  __syncthreads();
  const int64_t slot_lo = static_cast<int64_t>(dst) * kBlockSize;
  for (int64_t i = tid; i < a.num_tokens; i += kStepThreads) {
    const int32_t sl = a.slot_mapping[i];
    if (sl >= slot_lo && sl < slot_lo + kBlockSize) {
      const int k = atomicAdd(&n_match, 1);
      if (k < kBlockSize) match[k] = static_cast<int>(i);
    }
  }
  __syncthreads();
  const int n = n_match < kBlockSize ? n_match : kBlockSize;
  const float* head_scales = is_k ? a.k_head_scales : a.v_head_scales;
  const float scale = head_scales ? head_scales[h] : (is_k ? a.k_scale : a.v_scale);
  for (int m = 0; m < n; ++m) {
    const int64_t i = match[m];
    const int t0 = a.slot_mapping[i] & 15;
    const uint4* row = reinterpret_cast<const uint4*>((is_k ? a.k : a.v) + (i * hkv + h) * kHeadSize);
    if (is_k) {
      if (((tid >> 1) & 15) == t0) {
        const uint4 r8 = row[8 * (tid >> 7) + 4 * (tid & 1) + ((tid >> 5) & 3)];  // dims d0 .. d0 + 7
        val = make_uint2(0u, 0u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          val.x |= encode_fp8<DT>(r8, e, scale) << (8 * e);
          val.y |= encode_fp8<DT>(r8, 4 + e, scale) << (8 * e);
        }
      }
    } else if (((tid >> 5) & 3) == (t0 >> 2)) {
      const int dl = 64 * (tid >> 7) + 32 * (tid & 1) + ((tid >> 1) & 15);
      const uint32_t lo = encode_fp8<DT>(row[dl >> 3], dl & 7, scale);
      const uint32_t hi = encode_fp8<DT>(row[(dl + 16) >> 3], dl & 7, scale);
      const int sh = 8 * (t0 & 3);
      val.x = (val.x & ~(0xffu << sh)) | (lo << sh);
      val.y = (val.y & ~(0xffu << sh)) | (hi << sh);
    }
  }
  uint8_t* d = base + (static_cast<int64_t>(dst) * hkv + h) * kPageBytesFp8;
  store8<kNonTemporal>(range_rsrc(d, kPageBytesFp8), 8u * tid, val);
}

// Cache formats of the fused launch: the write and the merged page copy.
struct Step16 {
  __device__ static void write(int64_t wg, const StepArgs& a) {
    write_rows16(wg, a.k, a.v, a.k_cache, a.v_cache, a.slot_mapping, a.num_tokens, a.num_kv_heads,
                 static_cast<int64_t>(a.num_blocks) * kBlockSize);
  }
  __device__ static void copy(const StepArgs& a, int64_t pair, int page) { copy_page_merged(a, pair, page); }
};
template <class DT>
struct StepFp8 {
  __device__ static void write(int64_t wg, const StepArgs& a) {
    write_rows_fp8<DT>(wg, a.k, a.v, reinterpret_cast<uint8_t*>(a.k_cache), reinterpret_cast<uint8_t*>(a.v_cache),
                       a.slot_mapping, a.num_tokens, a.num_kv_heads, static_cast<int64_t>(a.num_blocks) * kBlockSize,
                       a.k_scale, a.v_scale, a.k_head_scales, a.v_head_scales);
  }
  __device__ static void copy(const StepArgs& a, int64_t pair, int page) { copy_page_merged_fp8<DT>(a, pair, page); }
};

template <class Fmt>
__global__ __launch_bounds__(kStepThreads) void decode_step_prologue_kernel(StepArgs a) {
  const int64_t wg = blockIdx.x;
  if (wg < a.plan_wg) {  // the write: first, since it runs longest
    Fmt::write(wg, a);
    return;
  }
  if (wg == a.plan_wg) {
    if (a.planned) plan_body<kStepThreads, kStepPlanMaxSeqs, kStepPlanMaxTasks, kStepPlanMaxParts>(a.plan);
    return;
  }
  const int64_t c = wg - a.plan_wg - 1;
  const int pages = 2 * a.num_kv_heads;
  Fmt::copy(a, c / pages, static_cast<int>(c % pages));
}

}  // namespace

hipError_t launch_decode_step_prologue(const StepArgs& a_in, bool fp8_cache, int act_dtype, hipStream_t stream) {
  StepArgs a = a_in;
  // write work-groups from 0 (a multiple of 8, so the write keeps its XCD
  // order), then the plan work-group, then one per copied page
  const int64_t items = (a.num_tokens + 3) / 4 * ((a.num_kv_heads + 3) / 4);
  a.plan_wg = (items + kNumXcd - 1) / kNumXcd * kNumXcd;
  const int64_t copy_wgs = static_cast<int64_t>(a.num_pairs) * 2 * a.num_kv_heads;
  const dim3 grid(static_cast<uint32_t>(a.plan_wg + 1 + copy_wgs)), block(kStepThreads);
  if (!fp8_cache)
    decode_step_prologue_kernel<Step16><<<grid, block, 0, stream>>>(a);
  else if (act_dtype == 0)
    decode_step_prologue_kernel<StepFp8<F16>><<<grid, block, 0, stream>>>(a);
  else
    decode_step_prologue_kernel<StepFp8<BF16>><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
