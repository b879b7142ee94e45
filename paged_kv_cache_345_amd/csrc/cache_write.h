// Slot-mapped write of new rows into the paged cache (16-bit pages, and fp8
// pages with encoding): the work split and the body of one work-group, shared
// by reshape_and_cache_kernel / reshape_and_cache_fp8_kernel (cache_ops.hip)
// and the fused decode-step prologue (step.hip).
//
// Slot model from page "vLLM 部署与 PagedAttention 原理 · 检索整理（CSDN 频道批次）",
// item 2: tokens fill fixed-size blocks reached through a block table.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {

// Work split: a work-group per (window of 4 consecutive slot_mapping entries,
// group of 4 KV heads); wave w takes window token w, lane l head l/16 of the
// group and 8-dim chunk l%16.  K lands as one 16-byte store per lane (8
// consecutive dims of one token are contiguous in the K page).  In the V page
// the 4 tokens of an aligned quad (slots 4m .. 4m+3) sit side by side for every
// dim, so a quad written whole becomes, after a transpose through LDS, one
// 16-byte store per (dims d, d+16) pair, made by the wave of the matching head;
// a token outside any complete quad falls back to eight 2-byte stores.  A quad
// whose first token lies in a window is written by that window's work-group (a
// quad may reach up to 3 tokens past the window; at most one quad starts in a
// window).  Measured on MI355X, a 64-prompt write (85 K tokens x 40 heads,
// 3.5 GB moved): 2.68 ms with 2-byte V stores only, 0.97 ms with whole quads,
// 0.85 ms (4.1 TB/s) with the XCD-contiguous order of write_item below; the
// decode-step write (128 lone tokens) is unchanged in effect.
//
// Store policy, measured on MI355X with the attention kernel that follows in a
// decode step: a decode step writes every touched page in small pieces, and
// with the default policy those partly written lines are still dirty in the
// memory-side cache when attention streams the cache, which then runs ~15 us
// (5%) slower on a 128-sequence, 40-head batch.  Non-temporal K stores remove
// most of that at no cost here; non-temporal 2-byte V stores would make this
// kernel 2.4x slower, so V keeps the default policy.  A token whose neighbour
// in slot_mapping lies in the same block (a prefill writing consecutive
// tokens) keeps the default policy for K too: there the cache merges the
// tokens' pieces into whole lines, which non-temporal stores would bypass
// (measured: a 64 Ki-token bulk write takes 1.7x as long with them).
// The window's slots and per-token flags.  Every array index below is a
// compile-time constant and per-lane picks are selects: an index that varies
// across lanes would put the array in per-lane scratch memory, whose stores
// (4 KiB per wave) slow this kernel and leave dirty lines that slow the
// attention kernel after it.
struct WriteWindow {
  int32_t s[10];       // slot_mapping[4Q - 3 .. 4Q + 6]; -1 outside [0, num_tokens) or [0, num_slots)
  int lead;            // window token (0..3) that starts a complete quad, or -1
  int32_t lead_slot;   // its slot
  uint32_t quad_mask;  // bit k: window token k belongs to a complete quad (its V is written whole)
  uint32_t lone_mask;  // bit k: window token k shares its block with neither slot_mapping neighbour
  int64_t first;       // 4Q

  __device__ WriteWindow(const int32_t* __restrict__ slot_mapping, int64_t q, int64_t num_tokens, int64_t num_slots) {
    first = 4 * q;
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const int64_t i = first - 3 + j;
      const int32_t x = (i >= 0 && i < num_tokens) ? slot_mapping[i] : -1;
      s[j] = (x >= 0 && x < num_slots) ? x : -1;
    }
    // entries j .. j+3 hold the slots 4m .. 4m+3 (one block, since 16 % 4 == 0)
    bool quad[7];
#pragma unroll
    for (int j = 0; j < 7; ++j)
      quad[j] = s[j] >= 0 && (s[j] & 3) == 0 && s[j + 1] == s[j] + 1 && s[j + 2] == s[j] + 2 && s[j + 3] == s[j] + 3;
    lead = -1;
    lead_slot = -1;
    quad_mask = 0;
    lone_mask = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 3 + k;
      if (lead < 0 && quad[j]) {  // at most one quad starts in a window: its next 3 slots are not multiples of 4
        lead = k;
        lead_slot = s[j];
      }
      if (quad[j] || quad[j - 1] || quad[j - 2] || quad[j - 3]) quad_mask |= 1u << k;
      const int32_t b = s[j] >> 4;
      if ((s[j - 1] < 0 || (s[j - 1] >> 4) != b) && (s[j + 1] < 0 || (s[j + 1] >> 4) != b)) lone_mask |= 1u << k;
    }
  }
  __device__ int32_t slot(int k) const { return k == 0 ? s[3] : k == 1 ? s[4] : k == 2 ? s[5] : s[6]; }
  __device__ bool in_quad(int k) const { return (quad_mask >> k) & 1u; }
  __device__ bool lone(int k) const { return (lone_mask >> k) & 1u; }
};

// Work-group -> (window q, head group hg).  The items are ordered (hg, q), q
// fastest, and dealt to the 8 XCDs in contiguous chunks (work-groups are
// dispatched round-robin over the XCDs), so neighbouring windows of one head
// group, which write the two halves of each 128-byte line of a K page, meet in
// one L2.  `wg` is the work-group's index among the write work-groups; its
// XCD is wg mod 8 as long as the first write work-group's blockIdx is a
// multiple of 8.  Returns false for a work-group past the last item (the grid
// is rounded up to a multiple of the XCD count).
__device__ inline bool write_item(int64_t wg, int64_t num_tokens, int num_kv_heads, int64_t& q, int& hg) {
  const int64_t nwin = (num_tokens + 3) / 4;
  const int groups = (num_kv_heads + 3) / 4;
  const int64_t total = nwin * groups;
  const int64_t per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int64_t lam = (wg % kNumXcd) * per_xcd + wg / kNumXcd;
  if (lam >= total) return false;
  hg = static_cast<int>(lam / nwin);
  q = lam - static_cast<int64_t>(hg) * nwin;
  return true;
}

// The 16-bit write of one work-group (256 threads), write work-group `wg`.
__device__ inline void write_rows16(int64_t wg, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                    const int32_t* __restrict__ slot_mapping, int64_t num_tokens, int num_kv_heads,
                                    int64_t num_slots) {
  __shared__ uint4 stage[4][4][16];  // [quad token][head in group][chunk]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t q;
  int hg;
  if (!write_item(wg, num_tokens, num_kv_heads, q, hg)) return;  // the whole work-group: no barrier is skipped
  const WriteWindow w(slot_mapping, q, num_tokens, num_slots);
  const int hh = lane >> 4, c = lane & 15;
  const int h = 4 * hg + hh;
  const int32_t slot = w.slot(wave);
  const int64_t token = w.first + wave;

  if (slot >= 0 && h < num_kv_heads) {
    const int64_t row = token * num_kv_heads + h;
    const int t = slot & 15;
    const int64_t page = (static_cast<int64_t>(slot >> 4) * num_kv_heads + h) * kPageElems;
    const uint4 kv = reinterpret_cast<const uint4*>(k + row * kHeadSize)[c];
    const __amdgpu_buffer_rsrc_t kr = page_rsrc(k_cache + page);
    if (w.lone(wave))
      store16<kNonTemporal>(kr, 2u * k_page_offset(t, 8 * c), kv);
    else
      store16(kr, 2u * k_page_offset(t, 8 * c), kv);
    if (!w.in_quad(wave)) {
      const uint4 vv = reinterpret_cast<const uint4*>(v + row * kHeadSize)[c];
      const __amdgpu_buffer_rsrc_t vr = page_rsrc(v_cache + page);
      const uint32_t e32[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t bits = static_cast<uint16_t>((e & 1) ? (e32[e >> 1] >> 16) : (e32[e >> 1] & 0xffffu));
        store2(vr, 2u * v_page_offset(t, 8 * c + e), bits);
      }
    }
  }
  if (w.lead >= 0 && h < num_kv_heads) {
    const int64_t row = (w.first + w.lead + wave) * num_kv_heads + h;
    stage[wave][hh][c] = reinterpret_cast<const uint4*>(v + row * kHeadSize)[c];
  }
  __syncthreads();
  const int hw = 4 * hg + wave;
  if (w.lead >= 0 && hw < num_kv_heads) {
    const int a = lane >> 4, b = lane & 15;
    uint32_t x[4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int d = 32 * a + 16 * p + b;
      const uint16_t* s0 = reinterpret_cast<const uint16_t*>(stage[0][wave]);
      const uint16_t* s1 = reinterpret_cast<const uint16_t*>(stage[1][wave]);
      const uint16_t* s2 = reinterpret_cast<const uint16_t*>(stage[2][wave]);
      const uint16_t* s3 = reinterpret_cast<const uint16_t*>(stage[3][wave]);
      x[2 * p] = static_cast<uint32_t>(s0[d]) | (static_cast<uint32_t>(s1[d]) << 16);
      x[2 * p + 1] = static_cast<uint32_t>(s2[d]) | (static_cast<uint32_t>(s3[d]) << 16);
    }
    const int32_t sl = w.lead_slot;
    const int64_t page = (static_cast<int64_t>(sl >> 4) * num_kv_heads + hw) * kPageElems;
    store16(page_rsrc(v_cache + page), 2u * v_page_offset(sl & 15, 32 * a + b), make_uint4(x[0], x[1], x[2], x[3]));
  }
}

// E4M3 code of element e of 8 16-bit values, divided by the row's scale: the
// one encoding of the fp8 write, used by every kernel that stores a new row's
// codes, so that all of them store the same bytes.
template <class DT>
__device__ inline uint32_t encode_fp8(const uint4& row8, int e, float scale) {
  return e4m3_encode(elem<DT>(row8, e) / scale);
}

// The fp8 (E4M3) write of one work-group, write work-group `wg`: the same
// work split; each element is encoded by encode_fp8 above (one correctly
// rounded float division by the call's one K (V) scale or that of the
// element's KV head, then e4m3_encode).  K lands as one 8-byte store per lane
// (8 consecutive dims of one token are contiguous in the fp8 K page).  A
// complete quad's V codes are staged in LDS and leave as 32 16-byte stores per
// head page (dims 64a + b + {0, 16, 32, 48} of the 4 tokens each); other
// tokens' V as eight 1-byte stores.  The K store policy follows write_rows16
// above.
template <class DT>
__device__ inline void write_rows_fp8(int64_t wg, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                      uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                      const int32_t* __restrict__ slot_mapping, int64_t num_tokens, int num_kv_heads,
                                      int64_t num_slots, float k_scale, float v_scale,
                                      const float* __restrict__ k_head_scales,
                                      const float* __restrict__ v_head_scales) {
  __shared__ uint2 stage[4][4][16];  // [quad token][head in group][chunk]: V codes
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t q;
  int hg;
  if (!write_item(wg, num_tokens, num_kv_heads, q, hg)) return;  // the whole work-group: no barrier is skipped
  const WriteWindow w(slot_mapping, q, num_tokens, num_slots);
  const int hh = lane >> 4, c = lane & 15;
  const int h = 4 * hg + hh;
  const int32_t slot = w.slot(wave);
  const int64_t token = w.first + wave;
  // this lane's head: its scales (per cache, or per KV head)
  const bool head_ok = h < num_kv_heads;
  if (head_ok && k_head_scales) k_scale = k_head_scales[h];
  if (head_ok && v_head_scales) v_scale = v_head_scales[h];

  if (slot >= 0 && head_ok) {
    const int64_t row = token * num_kv_heads + h;
    const int t = slot & 15;
    const int64_t page = (static_cast<int64_t>(slot >> 4) * num_kv_heads + h) * kPageBytesFp8;
    const uint4 kv = reinterpret_cast<const uint4*>(k + row * kHeadSize)[c];
    uint2 kq = make_uint2(0u, 0u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kq.x |= encode_fp8<DT>(kv, e, k_scale) << (8 * e);
      kq.y |= encode_fp8<DT>(kv, 4 + e, k_scale) << (8 * e);
    }
    const __amdgpu_buffer_rsrc_t kr = range_rsrc(k_cache + page, kPageBytesFp8);
    if (w.lone(wave))
      store8<kNonTemporal>(kr, k_page_offset_fp8(t, 8 * c), kq);
    else
      store8(kr, k_page_offset_fp8(t, 8 * c), kq);
    if (!w.in_quad(wave)) {
      const uint4 vv = reinterpret_cast<const uint4*>(v + row * kHeadSize)[c];
      const __amdgpu_buffer_rsrc_t vr = range_rsrc(v_cache + page, kPageBytesFp8);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        store1(vr, v_page_offset_fp8(t, 8 * c + e), static_cast<uint8_t>(encode_fp8<DT>(vv, e, v_scale)));
    }
  }
  if (w.lead >= 0 && h < num_kv_heads) {  // quad token `wave`, head h, chunk c: encode into LDS
    const int64_t row = (w.first + w.lead + wave) * num_kv_heads + h;
    const uint4 vv = reinterpret_cast<const uint4*>(v + row * kHeadSize)[c];
    uint2 vq = make_uint2(0u, 0u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vq.x |= encode_fp8<DT>(vv, e, v_scale) << (8 * e);
      vq.y |= encode_fp8<DT>(vv, 4 + e, v_scale) << (8 * e);
    }
    stage[wave][hh][c] = vq;
  }
  __syncthreads();
  const int hw = 4 * hg + wave;  // this wave stores the quad's V page of head hw
  if (w.lead >= 0 && hw < num_kv_heads && lane < 32) {
    // lane (a = lane / 16, b = lane % 16): byte 8p + 4r + t of its chunk holds
    // dim 64a + 32p + 16r + b of quad token t
    const int a = lane >> 4, b = lane & 15;
    uint32_t x[4];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {  // pr = 2p + r
      const int d = 64 * a + 16 * pr + b;
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        word |= static_cast<uint32_t>(reinterpret_cast<const uint8_t*>(stage[t][wave])[d]) << (8 * t);
      x[pr] = word;
    }
    const int64_t page = (static_cast<int64_t>(w.lead_slot >> 4) * num_kv_heads + hw) * kPageBytesFp8;
    store16(range_rsrc(v_cache + page, kPageBytesFp8), v_page_offset_fp8(w.lead_slot & 15, 64 * a + b),
            make_uint4(x[0], x[1], x[2], x[3]));
  }
}

}  // namespace pkv
