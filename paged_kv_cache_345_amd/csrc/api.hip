// C ABI of libpagedkv: argument validation, partition choice, workspace
// sizing and kernel launches on the caller's stream.  See include/pagedkv.h
// for the contract of each entry point.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "pagedkv.h"
#include "pkv_device.h"
#include "pkv_launch.h"


namespace {

constexpr double kLog2e = 1.4426950408889634073599246810019;

pkv_status check_desc(const pkv_cache_desc* c) {
  if (!c) return PKV_ERR_INVALID;
  if (c->block_size != pkv::kBlockSize || c->head_size != pkv::kHeadSize) return PKV_ERR_UNSUPPORTED;
  if (c->dtype != PKV_F16 && c->dtype != PKV_BF16 && c->dtype != PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PKV_ERR_INVALID;
  // every page offset must fit int64 comfortably and every slot an int32
  if (static_cast<int64_t>(c->num_blocks) * pkv::kBlockSize > INT32_MAX) return PKV_ERR_INVALID;
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_fp8(const pkv_cache_desc* c) { return c->dtype == PKV_FP8_E4M3; }
int32_t page_bytes(const pkv_cache_desc* c) { return is_fp8(c) ? pkv::kPageBytesFp8 : 2 * pkv::kPageElems; }

// The scales of an fp8 call: act dtype fp16/bf16; each of K and V has either
// a per-head array (4-byte aligned device pointer) or a finite positive scalar.
pkv_status check_scales(const pkv_fp8_scales* f) {
  if (!f) return PKV_ERR_INVALID;
  if (f->act_dtype != PKV_F16 && f->act_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  auto ok = [](float x, const float* per_head) {
    if (per_head) return (reinterpret_cast<uintptr_t>(per_head) & 3u) == 0;
    return std::isfinite(x) && x > 0.f;
  };
  if (!ok(f->k_scale, f->k_head_scales) || !ok(f->v_scale, f->v_head_scales)) return PKV_ERR_INVALID;
  return PKV_OK;
}

// Logit scale (log2 units) and output scale of a decode or prefill call; the
// per-head arrays, when given, are applied in the kernels instead.
void set_scales(pkv::DecodeArgs& a, float scale, const pkv_fp8_scales* fp8) {
  const bool k_fold = fp8 && !fp8->k_head_scales;
  a.scale_log2e = static_cast<float>(static_cast<double>(scale) * kLog2e *
                                     (k_fold ? static_cast<double>(fp8->k_scale) : 1.0));
  a.out_scale = fp8 && !fp8->v_head_scales ? fp8->v_scale : 1.0f;
  a.k_head_scales = fp8 ? fp8->k_head_scales : nullptr;
  a.v_head_scales = fp8 ? fp8->v_head_scales : nullptr;
}

// MI355X: 256 compute units; work-groups of the decode kernels that fit on one
// compute unit at once (4 waves each: MHA fp16 runs 5 waves per SIMD, MHA bf16
// and MHA over an fp8 cache 4, the GQA kernels 2).
constexpr int64_t kComputeUnits = 256;
int64_t resident_work_groups(int32_t group, int32_t dtype) {
  return kComputeUnits * (group == 1 ? (dtype == PKV_F16 ? 5 : 4) : 2);
}

// Segment length in blocks.  Automatic choice: the largest power of two in
// [16, 256] blocks that is at most the work of one resident work-group at the
// row bound (rows x max_blocks over the resident work-groups) and at most the
// smallest power of two covering max_blocks; doubled (up to 256) only if the
// segment count would exceed the reduce kernel's bound.  Longer segments mean
// fewer partials to merge; measured on MI355X, this bound keeps the work
// balanced while removing most of the merge (GQA batch 3%, LLaMA-7B batch 3%
// faster than half as long).  The choice depends on the shapes only.
pkv_status resolve_partition(int32_t num_seqs, int32_t units, int32_t group, int32_t dtype, int32_t max_blocks_per_seq,
                             int32_t partition_tokens, int32_t* bpp_out, int32_t* parts_out) {
  int32_t bpp;
  if (partition_tokens == 0) {
    const int64_t rows = static_cast<int64_t>(num_seqs) * units;
    const int64_t per_wg = rows * max_blocks_per_seq / resident_work_groups(group, dtype);
    int32_t cover = 16;
    while (cover < max_blocks_per_seq && cover < pkv::kMaxSegmentBlocks) cover *= 2;
    bpp = 16;
    while (bpp < cover && 2 * bpp <= per_wg) bpp *= 2;
    while ((max_blocks_per_seq + bpp - 1) / bpp > pkv::kMaxPartitions && bpp < pkv::kMaxSegmentBlocks) bpp *= 2;
  } else {
    if (partition_tokens < pkv::kBlockSize || partition_tokens % pkv::kBlockSize != 0 ||
        partition_tokens > pkv::kBlockSize * pkv::kMaxSegmentBlocks)
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

size_t round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace sections of one decode call, in bytes from its base.
struct DecodeLayout {
  int32_t bpp = 0, parts = 0, units = 0, group = 0;
  bool planned = false;
  size_t plan = 0, partial_o = 0, partial_ml = 0, total = 0;
};

pkv_status decode_layout(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq, int32_t partition_tokens,
                         const pkv_cache_desc* cache, DecodeLayout* out) {
  pkv_status st = check_decode_shape(num_seqs, num_heads, max_blocks_per_seq, cache);
  if (st != PKV_OK) return st;
  DecodeLayout L;
  L.group = num_heads / cache->num_kv_heads;
  L.units = cache->num_kv_heads * (L.group == 1 ? 1 : (L.group + 15) / 16);
  st = resolve_partition(num_seqs, L.units, L.group, cache->dtype, max_blocks_per_seq, partition_tokens, &L.bpp,
                         &L.parts);
  if (st != PKV_OK) return st;
  const int64_t chunks = (static_cast<int64_t>(num_seqs) + 63) / 64;
  L.planned = num_seqs <= pkv::kPlanMaxSeqs && (static_cast<int64_t>(L.parts) + L.bpp) * chunks <= pkv::kPlanMaxTasks &&
              static_cast<int64_t>(L.units) * num_seqs * L.parts < (int64_t{1} << 31);
  const size_t S = static_cast<size_t>(num_seqs);
  size_t off = 0;
  if (L.planned) {
    L.plan = off;
    off += round_up((pkv::kPlanHeaderInts + S * static_cast<size_t>(L.parts) + S) * sizeof(int32_t));
  }
  if (L.parts > 1) {
    const size_t rows = S * static_cast<size_t>(num_heads) * static_cast<size_t>(L.parts);
    L.partial_o = off;
    off += round_up(rows * pkv::kHeadSize * sizeof(float));
    L.partial_ml = off;
    off += round_up(rows * 2 * sizeof(float));
  }
  L.total = off;
  *out = L;
  return PKV_OK;
}

pkv_status from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_DEVICE; }

}  // namespace

extern "C" {

size_t pkv_cache_bytes(const pkv_cache_desc* cache) {
  if (check_desc(cache) != PKV_OK) return 0;
  return static_cast<size_t>(cache->num_blocks) * static_cast<size_t>(cache->num_kv_heads) *
         static_cast<size_t>(page_bytes(cache));
}

int64_t pkv_k_index(const pkv_cache_desc* c, int32_t block, int32_t head, int32_t token, int32_t dim) {
  if (check_desc(c) != PKV_OK || block < 0 || block >= c->num_blocks || head < 0 || head >= c->num_kv_heads ||
      token < 0 || token >= pkv::kBlockSize || dim < 0 || dim >= pkv::kHeadSize)
    return -1;
  return (static_cast<int64_t>(block) * c->num_kv_heads + head) * pkv::kPageElems +
         (is_fp8(c) ? pkv::k_page_offset_fp8(token, dim) : pkv::k_page_offset(token, dim));
}

int64_t pkv_v_index(const pkv_cache_desc* c, int32_t block, int32_t head, int32_t token, int32_t dim) {
  if (check_desc(c) != PKV_OK || block < 0 || block >= c->num_blocks || head < 0 || head >= c->num_kv_heads ||
      token < 0 || token >= pkv::kBlockSize || dim < 0 || dim >= pkv::kHeadSize)
    return -1;
  return (static_cast<int64_t>(block) * c->num_kv_heads + head) * pkv::kPageElems +
         (is_fp8(c) ? pkv::v_page_offset_fp8(token, dim) : pkv::v_page_offset(token, dim));
}

int32_t paged_attn_decode_partition_tokens(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                           int32_t partition_tokens, const pkv_cache_desc* cache) {
  DecodeLayout L;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, partition_tokens, cache, &L) != PKV_OK) return -1;
  return L.bpp * pkv::kBlockSize;
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                        int32_t partition_tokens, const pkv_cache_desc* cache) {
  DecodeLayout L;
  if (decode_layout(num_seqs, num_heads, max_blocks_per_seq, partition_tokens, cache, &L) != PKV_OK)
    return static_cast<size_t>(-1);
  return L.total;
}

}  // extern "C"

namespace {

// The plan's wave-per-chunk path applies (plan_body.h): one sequence per thread.
bool plan_scan_fits(int32_t num_seqs, const DecodeLayout&, int threads) { return num_seqs <= threads; }

// Checks shared by the plan and the run entry points.
pkv_status check_workspace(const DecodeLayout& L, const void* workspace, size_t workspace_bytes) {
  if (L.total > 0 && (!workspace || workspace_bytes < L.total || !aligned16(workspace))) return PKV_ERR_INVALID;
  return PKV_OK;
}

pkv_status launch_plan(const DecodeLayout& L, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t max_blocks_per_seq, void* workspace, hipStream_t stream) {
  if (!L.planned) return PKV_OK;
  pkv::PlanArgs pa;
  pa.context_lens = context_lens;
  pa.plan = reinterpret_cast<int*>(static_cast<char*>(workspace) + L.plan);
  pa.num_seqs = num_seqs;
  pa.num_heads = num_heads;
  pa.units = L.units;
  pa.max_blocks_per_seq = max_blocks_per_seq;
  pa.blocks_per_part = L.bpp;
  pa.parts_max = L.parts;
  pa.scan = plan_scan_fits(num_seqs, L, pkv::kPlanThreads) ? 1 : 0;
  return from_hip(pkv::launch_decode_plan(pa, stream));
}

pkv_status decode_impl(bool plan_first, void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, float scale, int32_t num_kv_heads,
                       int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                       const pkv_fp8_scales* fp8, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                       void* stream, uint32_t* read_probe_sink = nullptr) {
  pkv_status st = check_decode_shape(num_seqs, num_heads, max_blocks_per_seq, cache);
  if (st != PKV_OK) return st;
  // an fp8 cache comes only with its scales, and scales only with an fp8 cache
  if (is_fp8(cache) != (fp8 != nullptr)) return fp8 ? PKV_ERR_INVALID : PKV_ERR_UNSUPPORTED;
  if (fp8) {
    st = check_scales(fp8);
    if (st != PKV_OK) return st;
  }
  const int32_t act_dtype = fp8 ? fp8->act_dtype : cache->dtype;
  if (num_kv_heads != cache->num_kv_heads) return PKV_ERR_INVALID;
  if (!std::isfinite(scale)) return PKV_ERR_INVALID;
  DecodeLayout L;
  st = decode_layout(num_seqs, num_heads, max_blocks_per_seq, partition_tokens, cache, &L);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  st = check_workspace(L, workspace, workspace_bytes);
  if (st != PKV_OK) return st;

  char* ws = static_cast<char*>(workspace);
  pkv::DecodeArgs a;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws_o = L.parts > 1 ? reinterpret_cast<float*>(ws + L.partial_o) : nullptr;
  a.ws_ml = L.parts > 1 ? reinterpret_cast<float*>(ws + L.partial_ml) : nullptr;
  a.plan = L.planned ? reinterpret_cast<int*>(ws + L.plan) : nullptr;
  set_scales(a, scale, fp8);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = L.group;
  a.head_tiles = (L.group + 15) / 16;
  a.units = L.units;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = cache->num_blocks;
  a.blocks_per_part = L.bpp;
  a.parts_max = L.parts;
  a.planned = L.planned ? 1 : 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (plan_first) {
    st = launch_plan(L, context_lens, num_seqs, num_heads, max_blocks_per_seq, workspace, hs);
    if (st != PKV_OK) return st;
  }
  if (read_probe_sink) return from_hip(pkv::launch_decode_read_pages(a, fp8 != nullptr, read_probe_sink, hs));
  return from_hip(pkv::launch_decode(a, act_dtype == PKV_F16 ? 0 : 1, fp8 != nullptr, hs));
}

}  // namespace

extern "C" {

pkv_status paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, float scale,
                             int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                             const pkv_cache_desc* cache, int32_t partition_tokens, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_impl(true, out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, num_seqs,
                     num_heads, max_blocks_per_seq, cache, nullptr, partition_tokens, workspace, workspace_bytes,
                     stream);
}

pkv_status paged_attn_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                 int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                 const pkv_cache_desc* cache, const pkv_fp8_scales* scales, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!scales) return PKV_ERR_INVALID;
  return decode_impl(true, out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, num_seqs,
                     num_heads, max_blocks_per_seq, cache, scales, partition_tokens, workspace, workspace_bytes,
                     stream);
}

pkv_status paged_attn_decode_run_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                     int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                     const pkv_fp8_scales* scales, int32_t partition_tokens, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!scales) return PKV_ERR_INVALID;
  return decode_impl(false, out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, num_seqs,
                     num_heads, max_blocks_per_seq, cache, scales, partition_tokens, workspace, workspace_bytes,
                     stream);
}

}  // extern "C"

namespace {

// Workspace of paged_attn_decode_noalloc: one copy per GPU (the code object's
// device globals are placed on every device the library is loaded on).  Host
// code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per device, and is kept per device below.
static_assert(PKV_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address on the current device, looked up on the first call.
pkv_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_DEVICE;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                     int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                     int32_t partition_tokens, void* stream) {
  DecodeLayout L;
  pkv_status st = decode_layout(num_seqs, num_heads, max_blocks_per_seq, partition_tokens, cache, &L);
  if (st != PKV_OK) return st;
  if (L.total > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_INVALID;
  void* ws = nullptr;
  if (num_seqs > 0 && L.total > 0) {
    st = scratch_on_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_impl(true, out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, num_seqs,
                     num_heads, max_blocks_per_seq, cache, nullptr, partition_tokens, ws,
                     ws ? PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}

pkv_status paged_attn_decode_read_pages(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                        int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                        int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                        uint32_t* sink, void* stream) {
  if (!sink || cache == nullptr) return PKV_ERR_INVALID;
  // q and out are never touched: any aligned non-null pointers pass the shared checks
  void* const unused = sink;
  const bool fp8 = cache->dtype == PKV_FP8_E4M3;
  pkv_fp8_scales ones{PKV_F16, 1.f, 1.f, nullptr, nullptr};
  if ((reinterpret_cast<uintptr_t>(sink) & 15u) != 0) return PKV_ERR_INVALID;
  return decode_impl(false, unused, unused, k_cache, v_cache, block_tables, context_lens, 1.f, cache->num_kv_heads,
                     num_seqs, num_heads, max_blocks_per_seq, cache, fp8 ? &ones : nullptr, partition_tokens,
                     workspace, workspace_bytes, stream, sink);
}

pkv_status paged_attn_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                  int32_t max_blocks_per_seq, const pkv_cache_desc* cache, int32_t partition_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  DecodeLayout L;
  pkv_status st = decode_layout(num_seqs, num_heads, max_blocks_per_seq, partition_tokens, cache, &L);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens) return PKV_ERR_INVALID;
  st = check_workspace(L, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  return launch_plan(L, context_lens, num_seqs, num_heads, max_blocks_per_seq, workspace,
                     static_cast<hipStream_t>(stream));
}

pkv_status paged_attn_decode_run(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                 int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pkv_cache_desc* cache, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(false, out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, num_seqs,
                     num_heads, max_blocks_per_seq, cache, nullptr, partition_tokens, workspace, workspace_bytes,
                     stream);
}

}  // extern "C"

namespace {

pkv_status write_impl(const void* k, const void* v, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                      int32_t num_tokens, const pkv_cache_desc* cache, const pkv_fp8_scales* fp8, void* stream) {
  pkv_status st = check_desc(cache);
  if (st != PKV_OK) return st;
  if (is_fp8(cache) != (fp8 != nullptr)) return fp8 ? PKV_ERR_INVALID : PKV_ERR_UNSUPPORTED;
  if (fp8) {
    st = check_scales(fp8);
    if (st != PKV_OK) return st;
  }
  if (num_tokens < 0) return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  // keep each launch's grid well inside 2^31 work-groups
  const int32_t chunk = static_cast<int32_t>(((int64_t{1} << 30) * 16) / (int64_t{16} * cache->num_kv_heads));
  for (int32_t t0 = 0; t0 < num_tokens; t0 += chunk) {
    const int32_t n = num_tokens - t0 < chunk ? num_tokens - t0 : chunk;
    const size_t row_off = static_cast<size_t>(t0) * static_cast<size_t>(cache->num_kv_heads) * pkv::kHeadSize;
    const uint16_t* kt = static_cast<const uint16_t*>(k) + row_off;
    const uint16_t* vt = static_cast<const uint16_t*>(v) + row_off;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = fp8 ? pkv::launch_reshape_and_cache_fp8(kt, vt, k_cache, v_cache, slot_mapping + t0, n,
                                                          cache->num_kv_heads, cache->num_blocks,
                                                          fp8->act_dtype == PKV_F16 ? 0 : 1, fp8->k_scale,
                                                          fp8->v_scale, fp8->k_head_scales, fp8->v_head_scales, hs)
                       : pkv::launch_reshape_and_cache(kt, vt, k_cache, v_cache, slot_mapping + t0, n,
                                                      cache->num_kv_heads, cache->num_blocks, hs);
    if (e != hipSuccess) return PKV_ERR_DEVICE;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int32_t num_tokens, const pkv_cache_desc* cache,
                             void* stream) {
  return write_impl(k, v, k_cache, v_cache, slot_mapping, num_tokens, cache, nullptr, stream);
}

pkv_status reshape_and_cache_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                 const int32_t* slot_mapping, int32_t num_tokens, const pkv_cache_desc* cache,
                                 const pkv_fp8_scales* scales, void* stream) {
  if (!scales) return PKV_ERR_INVALID;
  return write_impl(k, v, k_cache, v_cache, slot_mapping, num_tokens, cache, scales, stream);
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
                                          cache->num_blocks, page_bytes(cache), static_cast<hipStream_t>(stream)));
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
                                           is_fp8(cache), static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The plan of a call fits the fused prologue's plan work-group (its LDS tables).
bool step_plan_fits(const DecodeLayout& L, int32_t num_seqs) {
  const int64_t chunks = (static_cast<int64_t>(num_seqs) + 63) / 64;
  return num_seqs <= pkv::kStepPlanMaxSeqs && L.parts <= pkv::kStepPlanMaxParts &&
         (static_cast<int64_t>(L.parts) + L.bpp) * chunks <= pkv::kStepPlanMaxTasks;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// decode_step_prologue and its fp8 form (fp8: the write's scales, null for a
// 16-bit cache).
pkv_status prologue_impl(const void* k, const void* v, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                         int32_t num_tokens, const int32_t* block_pairs, int32_t num_pairs,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                         const pkv_cache_desc* cache, const pkv_fp8_scales* fp8, int32_t partition_tokens,
                         void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status st = check_desc(cache);
  if (st != PKV_OK) return st;
  if (is_fp8(cache) != (fp8 != nullptr)) return fp8 ? PKV_ERR_INVALID : PKV_ERR_UNSUPPORTED;
  if (fp8) {
    st = check_scales(fp8);
    if (st != PKV_OK) return st;
  }
  if (num_tokens < 0 || num_pairs < 0) return PKV_ERR_INVALID;
  DecodeLayout L;
  st = decode_layout(num_seqs, num_heads, max_blocks_per_seq, partition_tokens, cache, &L);
  if (st != PKV_OK) return st;
  if (!k_cache || !v_cache || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  if (num_tokens > 0 && (!k || !v || !slot_mapping || !aligned16(k) || !aligned16(v))) return PKV_ERR_INVALID;
  if (num_pairs > 0 && !block_pairs) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(num_pairs) * 2 * cache->num_kv_heads > INT32_MAX / 4) return PKV_ERR_INVALID;
  const bool plan = num_seqs > 0 && L.planned;
  if (plan) {
    if (!context_lens) return PKV_ERR_INVALID;
    st = check_workspace(L, workspace, workspace_bytes);
    if (st != PKV_OK) return st;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // a bulk write keeps the separate kernels: the merge scans every token per copied page
  if (num_tokens > 65536) {
    st = copy_blocks(k_cache, v_cache, block_pairs, num_pairs, cache, stream);
    if (st == PKV_OK) st = write_impl(k, v, k_cache, v_cache, slot_mapping, num_tokens, cache, fp8, stream);
    if (st == PKV_OK && plan) st = launch_plan(L, context_lens, num_seqs, num_heads, max_blocks_per_seq, workspace, hs);
    return st;
  }
  const bool fused_plan = plan && step_plan_fits(L, num_seqs);
  pkv::StepArgs a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.block_pairs = block_pairs;
  a.num_tokens = num_tokens;
  a.num_pairs = num_pairs;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_blocks = cache->num_blocks;
  a.planned = fused_plan ? 1 : 0;
  if (fp8) {
    a.k_scale = fp8->k_scale;
    a.v_scale = fp8->v_scale;
    a.k_head_scales = fp8->k_head_scales;
    a.v_head_scales = fp8->v_head_scales;
  }
  if (fused_plan) {
    a.plan.context_lens = context_lens;
    a.plan.plan = reinterpret_cast<int*>(static_cast<char*>(workspace) + L.plan);
    a.plan.num_seqs = num_seqs;
    a.plan.num_heads = num_heads;
    a.plan.units = L.units;
    a.plan.max_blocks_per_seq = max_blocks_per_seq;
    a.plan.blocks_per_part = L.bpp;
    a.plan.parts_max = L.parts;
    a.plan.scan = plan_scan_fits(num_seqs, L, pkv::kStepThreads) ? 1 : 0;
  }
  st = from_hip(pkv::launch_decode_step_prologue(a, fp8 != nullptr, fp8 && fp8->act_dtype == PKV_BF16 ? 1 : 0, hs));
  if (st == PKV_OK && plan && !fused_plan)
    st = launch_plan(L, context_lens, num_seqs, num_heads, max_blocks_per_seq, workspace, hs);
  return st;
}

}  // namespace

extern "C" {

pkv_status decode_step_prologue(const void* k, const void* v, void* k_cache, void* v_cache,
                                const int32_t* slot_mapping, int32_t num_tokens, const int32_t* block_pairs,
                                int32_t num_pairs, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t max_blocks_per_seq, const pkv_cache_desc* cache, int32_t partition_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return prologue_impl(k, v, k_cache, v_cache, slot_mapping, num_tokens, block_pairs, num_pairs, context_lens,
                       num_seqs, num_heads, max_blocks_per_seq, cache, nullptr, partition_tokens, workspace,
                       workspace_bytes, stream);
}

pkv_status decode_step_prologue_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int32_t num_tokens, const int32_t* block_pairs,
                                    int32_t num_pairs, const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_heads, int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                    const pkv_fp8_scales* scales, int32_t partition_tokens, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!scales) return PKV_ERR_INVALID;
  return prologue_impl(k, v, k_cache, v_cache, slot_mapping, num_tokens, block_pairs, num_pairs, context_lens,
                       num_seqs, num_heads, max_blocks_per_seq, cache, scales, partition_tokens, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Workspace and tiling of one prefill call.
struct PrefillLayout {
  int32_t hpt = 0, ppt = 0, q_blocks = 0, units = 0, group = 0, bpp = 0, parts = 0;
  size_t partial_o = 0, partial_ml = 0, total = 0;
};

pkv_status prefill_layout(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq, int32_t num_query_tokens,
                          int32_t max_query_len, int32_t partition_tokens, const pkv_cache_desc* cache,
                          PrefillLayout* out) {
  pkv_status st = check_decode_shape(num_seqs, num_heads, max_blocks_per_seq, cache);
  if (st != PKV_OK) return st;
  if (num_query_tokens < 0 || max_query_len < 0) return PKV_ERR_INVALID;
  if (num_query_tokens > 0 && (max_query_len < 1 || max_query_len > num_query_tokens)) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(max_query_len) > static_cast<int64_t>(max_blocks_per_seq) * pkv::kBlockSize)
    return PKV_ERR_INVALID;
  PrefillLayout P;
  P.group = num_heads / cache->num_kv_heads;
  P.hpt = P.group < 16 ? P.group : 16;
  P.ppt = 16 / P.hpt;
  const int32_t per_wg = pkv::kWavesPerGroup * pkv::kPrefillTiles * P.ppt;
  P.q_blocks = max_query_len > 0 ? (max_query_len + per_wg - 1) / per_wg : 0;
  P.units = cache->num_kv_heads * ((P.group + 15) / 16);
  // Segment length.  Automatic: the whole key range (the smallest power of
  // two of blocks covering max_blocks_per_seq) while the query blocks alone
  // give every resident work-group two items, halved down to 16 blocks while
  // they do not; every wave of a prefill work-group streams the whole segment.
  if (partition_tokens == 0) {
    const int64_t items = static_cast<int64_t>(num_seqs) * P.units * (P.q_blocks > 0 ? P.q_blocks : 1);
    const int64_t want = 2 * kComputeUnits * 3;  // 3 prefill work-groups fit a compute unit
    int32_t cover = 16;
    while (cover < max_blocks_per_seq) cover *= 2;
    P.bpp = cover;
    while (P.bpp > 16 && items * ((max_blocks_per_seq + P.bpp - 1) / P.bpp) < want) P.bpp /= 2;
    P.parts = (max_blocks_per_seq + P.bpp - 1) / P.bpp;
  } else {
    st = resolve_partition(num_seqs, P.units, 2, PKV_BF16, max_blocks_per_seq, partition_tokens, &P.bpp, &P.parts);
    if (st != PKV_OK) return st;
  }
  const int64_t items = static_cast<int64_t>(P.units) * num_seqs * P.q_blocks * P.parts;
  if (items > (int64_t{1} << 31) - 64) return PKV_ERR_UNSUPPORTED;
  size_t off = 0;
  if (P.parts > 1) {
    const size_t rows = static_cast<size_t>(num_query_tokens) * static_cast<size_t>(num_heads) *
                        static_cast<size_t>(P.parts);
    P.partial_o = off;
    off += round_up(rows * pkv::kHeadSize * sizeof(float));
    P.partial_ml = off;
    off += round_up(rows * 2 * sizeof(float));
  }
  P.total = off;
  *out = P;
  return PKV_OK;
}

pkv_status prefill_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                        float scale, int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                        int32_t max_blocks_per_seq, int32_t num_query_tokens, int32_t max_query_len,
                        const pkv_cache_desc* cache, const pkv_fp8_scales* fp8, int32_t partition_tokens,
                        void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status st = check_decode_shape(num_seqs, num_heads, max_blocks_per_seq, cache);
  if (st != PKV_OK) return st;
  if (is_fp8(cache) != (fp8 != nullptr)) return fp8 ? PKV_ERR_INVALID : PKV_ERR_UNSUPPORTED;
  if (fp8) {
    st = check_scales(fp8);
    if (st != PKV_OK) return st;
  }
  if (num_kv_heads != cache->num_kv_heads) return PKV_ERR_INVALID;
  if (!std::isfinite(scale)) return PKV_ERR_INVALID;
  PrefillLayout P;
  st = prefill_layout(num_seqs, num_heads, max_blocks_per_seq, num_query_tokens, max_query_len, partition_tokens,
                      cache, &P);
  if (st != PKV_OK) return st;
  if (num_seqs == 0 || num_query_tokens == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start) return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  if (P.total > 0 && (!workspace || workspace_bytes < P.total || !aligned16(workspace))) return PKV_ERR_INVALID;

  char* ws = static_cast<char*>(workspace);
  pkv::PrefillArgs pa;
  pkv::DecodeArgs& a = pa.d;
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws_o = P.parts > 1 ? reinterpret_cast<float*>(ws + P.partial_o) : nullptr;
  a.ws_ml = P.parts > 1 ? reinterpret_cast<float*>(ws + P.partial_ml) : nullptr;
  a.plan = nullptr;
  set_scales(a, scale, fp8);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = P.group;
  a.head_tiles = (P.group + 15) / 16;
  a.units = P.units;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = cache->num_blocks;
  a.blocks_per_part = P.bpp;
  a.parts_max = P.parts;
  a.planned = 0;
  pa.query_start = query_start;
  pa.heads_per_tile = P.hpt;
  pa.pos_per_wave = P.ppt;
  pa.q_blocks = P.q_blocks;
  pa.num_query_tokens = num_query_tokens;
  const int32_t act = fp8 ? fp8->act_dtype : cache->dtype;
  return from_hip(pkv::launch_prefill(pa, act == PKV_F16 ? 0 : 1, fp8 != nullptr, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

size_t paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                         int32_t num_query_tokens, int32_t max_query_len, int32_t partition_tokens,
                                         const pkv_cache_desc* cache) {
  PrefillLayout P;
  if (prefill_layout(num_seqs, num_heads, max_blocks_per_seq, num_query_tokens, max_query_len, partition_tokens,
                     cache, &P) != PKV_OK)
    return static_cast<size_t>(-1);
  return P.total;
}

pkv_status paged_attn_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                              float scale, int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                              int32_t max_blocks_per_seq, int32_t num_query_tokens, int32_t max_query_len,
                              const pkv_cache_desc* cache, int32_t partition_tokens, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale, num_kv_heads,
                      num_seqs, num_heads, max_blocks_per_seq, num_query_tokens, max_query_len, cache, nullptr,
                      partition_tokens, workspace, workspace_bytes, stream);
}

pkv_status paged_attn_prefill_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start, float scale, int32_t num_kv_heads, int32_t num_seqs,
                                  int32_t num_heads, int32_t max_blocks_per_seq, int32_t num_query_tokens,
                                  int32_t max_query_len, const pkv_cache_desc* cache, const pkv_fp8_scales* scales,
                                  int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (!scales) return PKV_ERR_INVALID;
  return prefill_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale, num_kv_heads,
                      num_seqs, num_heads, max_blocks_per_seq, num_query_tokens, max_query_len, cache, scales,
                      partition_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The address a kernel on the current device uses for p: p itself for device
// memory, the device mapping for pinned host memory.  Anything else (pageable
// host memory, unknown pointers) is refused, so no kernel ever touches an
// address the device cannot reach.
pkv_status device_address(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error this query leaves behind
    return PKV_ERR_INVALID;
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = p;
    return PKV_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    *out = attr.devicePointer;
    return PKV_OK;
  }
  return PKV_ERR_INVALID;
}

}  // namespace

extern "C" {

pkv_status swap_blocks(void* dst_k, void* dst_v, const pkv_cache_desc* dst_cache, const void* src_k,
                       const void* src_v, const pkv_cache_desc* src_cache, const int32_t* block_pairs,
                       int32_t num_pairs, void* stream) {
  pkv_status st = check_desc(dst_cache);
  if (st != PKV_OK) return st;
  st = check_desc(src_cache);
  if (st != PKV_OK) return st;
  if (dst_cache->num_kv_heads != src_cache->num_kv_heads || dst_cache->dtype != src_cache->dtype)
    return PKV_ERR_INVALID;
  if (num_pairs < 0) return PKV_ERR_INVALID;
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs) return PKV_ERR_INVALID;
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v)) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(num_pairs) * 2 * src_cache->num_kv_heads > INT32_MAX) return PKV_ERR_INVALID;
  const void* p[5] = {dst_k, dst_v, src_k, src_v, block_pairs};
  const void* d[5];
  for (int i = 0; i < 5; ++i) {
    st = device_address(p[i], &d[i]);
    if (st != PKV_OK) return st;
  }
  return from_hip(pkv::launch_swap_blocks(const_cast<void*>(d[0]), const_cast<void*>(d[1]), dst_cache->num_blocks, d[2],
                                          d[3], src_cache->num_blocks, static_cast<const int32_t*>(d[4]), num_pairs,
                                          src_cache->num_kv_heads, page_bytes(src_cache),
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
