// The decode-step prologue in one launch: the copy-on-write block copy, the
// slot-mapped write of the new tokens and the attention work-list plan, which
// a decode step otherwise runs as three kernels before the attention.
//
// Mechanism from page "vLLM 部署与 PagedAttention 原理 · 检索整理（CSDN 频道批次）",
// item 2: parallel samples share prompt blocks by reference count, and a
// shared block is copied before a sample writes into it.
//
// Work-groups (256 threads each) take one of three roles by index, the
// longest-running first, since work-groups start in index order:
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

__global__ __launch_bounds__(kStepThreads) void decode_step_prologue_kernel(StepArgs a) {
  const int64_t wg = blockIdx.x;
  if (wg < a.plan_wg) {  // the write: first, since it runs longest
    write_rows16(wg, a.k, a.v, a.k_cache, a.v_cache, a.slot_mapping, a.num_tokens, a.num_kv_heads,
                 static_cast<int64_t>(a.num_blocks) * kBlockSize);
    return;
  }
  if (wg == a.plan_wg) {
    if (a.planned) plan_body<kStepThreads, kStepPlanMaxSeqs, kStepPlanMaxTasks, kStepPlanMaxParts>(a.plan);
    return;
  }
  const int64_t c = wg - a.plan_wg - 1;
  const int pages = 2 * a.num_kv_heads;
  copy_page_merged(a, c / pages, static_cast<int>(c % pages));
}

}  // namespace

hipError_t launch_decode_step_prologue(const StepArgs& a_in, hipStream_t stream) {
  StepArgs a = a_in;
  // write work-groups from 0 (a multiple of 8, so the write keeps its XCD
  // order), then the plan work-group, then one per copied page
  const int64_t items = (a.num_tokens + 3) / 4 * ((a.num_kv_heads + 3) / 4);
  a.plan_wg = (items + kNumXcd - 1) / kNumXcd * kNumXcd;
  const int64_t copy_wgs = static_cast<int64_t>(a.num_pairs) * 2 * a.num_kv_heads;
  const int64_t grid = a.plan_wg + 1 + copy_wgs;
  decode_step_prologue_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(kStepThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
