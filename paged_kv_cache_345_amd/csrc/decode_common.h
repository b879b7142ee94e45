// Device code shared by the attention kernels (decode.hip, prefill.hip):
// page formats and the block stream, stale-slot masking of V fragments, and
// the log-sum-exp merge of segment partials.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// Tokens of a sequence, clamped to what its block-table row can address.
__device__ inline int clamped_len(const DecodeArgs& a, int s) {
  int L = a.context_lens[s];
  const int cap = a.max_blocks_per_seq * kBlockSize;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Masks that zero the 16-bit elements of a V fragment whose token is not
// valid.  Word k of a lane's 16-byte V fragment holds tokens 4G + (2k & 3) and
// 4G + (2k+1 & 3), so words x,z share one mask and y,w the other.
__device__ inline void mask_v(uint4 (&vv)[4], int grp, int nvalid) {
  const int t0 = 4 * grp;
  const uint32_t m01 = (t0 + 0 < nvalid ? 0x0000ffffu : 0u) | (t0 + 1 < nvalid ? 0xffff0000u : 0u);
  const uint32_t m23 = (t0 + 2 < nvalid ? 0x0000ffffu : 0u) | (t0 + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vv[i].x &= m01;
    vv[i].y &= m23;
    vv[i].z &= m01;
    vv[i].w &= m23;
  }
}

// Page formats.  Each holds the raw bytes of one block's K page and V page as
// loaded by a wave, and widens them to the 16-bit fragments the math consumes
// (kv[i]: lane (grp, col) -> token col, dims 8*(4i + grp) .. +8; vv[p]: tokens
// 4grp .. 4grp+3 of dims 16*(2p) + col and 16*(2p+1) + col).
//
// Each page is read with raw buffer loads: one buffer descriptor per page
// (wave-uniform, scalar registers, with the page as its record limit) and a
// single per-lane byte offset shared by K and V.  The K loads carry the
// non-temporal hint and the V loads the default policy.  Measured on MI355X
// over every decode batch: splitting the page traffic evenly between the two
// policies streams 5-9% faster than either policy alone, and a 3:5 to 6:2
// split is as good.

// 16-bit pages (fp16 / bf16 cache): four contiguous 1 KiB wave loads per page.
struct Page16 {
  static constexpr int kPageBytes = 2 * kPageElems;
  struct Raw {
    uint4 k[4], v[4];
  };
  __device__ static inline void load(Raw& r, const char* kp, const char* vp, uint32_t lane_bytes) {
    const __amdgpu_buffer_rsrc_t kr = range_rsrc(kp, kPageBytes);
    const __amdgpu_buffer_rsrc_t vr = range_rsrc(vp, kPageBytes);
    r.k[0] = load16<0, kNonTemporal>(kr, lane_bytes);
    r.k[1] = load16<1024, kNonTemporal>(kr, lane_bytes);
    r.k[2] = load16<2048, kNonTemporal>(kr, lane_bytes);
    r.k[3] = load16<3072, kNonTemporal>(kr, lane_bytes);
    r.v[0] = load16<0>(vr, lane_bytes);
    r.v[1] = load16<1024>(vr, lane_bytes);
    r.v[2] = load16<2048>(vr, lane_bytes);
    r.v[3] = load16<3072>(vr, lane_bytes);
  }
  __device__ static inline void expand(const Raw& r, uint4 (&kv)[4], uint4 (&vv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kv[i] = r.k[i];
      vv[i] = r.v[i];
    }
  }
};

// fp8 (E4M3) pages: two contiguous 1 KiB wave loads per page; lane l's 16
// bytes of load i are its 16-bit fragments 2i and 2i+1, one byte per element,
// widened exactly to the activation type DT (every E4M3 value is an fp16 and a
// bf16 value).  The cache scales are applied outside: to the logit scale (K)
// and to the output (V).
template <class DT>
struct PageFp8 {
  static constexpr int kPageBytes = kPageBytesFp8;
  struct Raw {
    uint4 k[2], v[2];
  };
  __device__ static inline void load(Raw& r, const char* kp, const char* vp, uint32_t lane_bytes) {
    const __amdgpu_buffer_rsrc_t kr = range_rsrc(kp, kPageBytes);
    const __amdgpu_buffer_rsrc_t vr = range_rsrc(vp, kPageBytes);
    r.k[0] = load16<0, kNonTemporal>(kr, lane_bytes);
    r.k[1] = load16<1024, kNonTemporal>(kr, lane_bytes);
    r.v[0] = load16<0>(vr, lane_bytes);
    r.v[1] = load16<1024>(vr, lane_bytes);
  }
  __device__ static inline void widen(uint4 w, uint4& lo, uint4& hi) {
    lo = make_uint4(DT::template from_e4m3x2<false>(w.x), DT::template from_e4m3x2<true>(w.x),
                    DT::template from_e4m3x2<false>(w.y), DT::template from_e4m3x2<true>(w.y));
    hi = make_uint4(DT::template from_e4m3x2<false>(w.z), DT::template from_e4m3x2<true>(w.z),
                    DT::template from_e4m3x2<false>(w.w), DT::template from_e4m3x2<true>(w.w));
  }
  __device__ static inline void expand(const Raw& r, uint4 (&kv)[4], uint4 (&vv)[4]) {
    widen(r.k[0], kv[0], kv[1]);
    widen(r.k[1], kv[2], kv[3]);
    widen(r.v[0], vv[0], vv[1]);
    widen(r.v[1], vv[2], vv[3]);
  }
};

// Streams blocks j0 .. j0 + nb - 1 (nb >= 1) of one sequence's pages of one KV
// head through `process`, two register sets deep: one block in flight while
// the other is consumed.  Only the last block takes the masked path.  Block
// ids are wave-uniform scalar loads (16 per scalar-cache line).
template <class PF, class Process>
__device__ __attribute__((always_inline)) inline void stream_blocks(const DecodeArgs& a, int s, int kvh, int j0, int nb,
                                                                    int lane, Process&& process) {
  const int32_t* row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq + j0;
  const int64_t page_stride = static_cast<int64_t>(a.num_kv_heads) * PF::kPageBytes;
  const int64_t head_off = static_cast<int64_t>(kvh) * PF::kPageBytes;
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  auto issue = [&](typename PF::Raw& r, int jj) __attribute__((always_inline)) {
    const int bid = row[jj];
    const bool bad = static_cast<unsigned>(bid) >= static_cast<unsigned>(a.num_blocks);
    const int64_t off = static_cast<int64_t>(bad ? 0 : bid) * page_stride + head_off;
    PF::load(r, kc + off, vc + off, static_cast<uint32_t>(lane) * 16u);
  };
  // the widened fragments are built when a block is consumed, never held in flight
  auto consume = [&]<bool kTail>(const typename PF::Raw& r, int j) __attribute__((always_inline)) {
    uint4 kv[4], vv[4];
    PF::expand(r, kv, vv);
    process.template operator()<kTail>(kv, vv, j);
  };
  typename PF::Raw ra, rb;
  issue(ra, 0);
  int jj = 0;
  // steady state: full blocks only and no conditional loads, so each wait
  // leaves the other register set in flight
  for (; jj + 2 < nb; jj += 2) {
    issue(rb, jj + 1);
    consume.template operator()<false>(ra, j0 + jj);
    issue(ra, jj + 2);
    consume.template operator()<false>(rb, j0 + jj + 1);
  }
  if (jj + 1 < nb) {
    issue(rb, jj + 1);
    consume.template operator()<false>(ra, j0 + jj);
    consume.template operator()<true>(rb, j0 + jj + 1);
  } else {
    consume.template operator()<true>(ra, j0 + jj);
  }
}

// The logit scale (log2 units) and the output scale of the rows of KV head
// kvh: the call's scalars, or the fp8 cache's per-head K / V scales.
__device__ inline float head_logit_scale(const DecodeArgs& a, int kvh) {
  return a.k_head_scales ? a.scale_log2e * a.k_head_scales[kvh] : a.scale_log2e;
}
__device__ inline float head_out_scale(const DecodeArgs& a, int kvh) {
  return a.v_head_scales ? a.v_head_scales[kvh] : a.out_scale;
}

// Merge of the n >= 2 segment partials of one output row by one wave:
//   M = max_p m_p,  c_p = 2^(m_p - M),  out = sum_p c_p O_p / sum_p c_p Z_p.
// ml: (m_p, Z_p) pairs; o: the partial rows, 128 floats each.  A segment in
// which the row saw no key has m_p = -1e30 and contributes c_p = 0.  Up to 4
// segments, lane l merges output dims 2l and 2l+1 over all of them.  Longer
// rows: lane l = 16 sg + dg takes the segments p = sg (mod 4) for dims
// 8 dg .. 8 dg + 7, so 4 segments are in flight per step, and the 4 segment
// groups are summed across the wave at the end.
template <class DT>
__device__ inline void lse_merge_row(const float* ml, const float* o, int n, uint16_t* out, float out_scale,
                                     int lane) {
  float mx = -__builtin_inff();
  for (int p = lane; p < n; p += kWave) mx = fmaxf(mx, ml[2 * p]);
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));

  if (n <= 4) {
    const float2* o2 = reinterpret_cast<const float2*>(o) + lane;
    float z = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p = 0; p < n; ++p) {
      const float c = exp2_fast(ml[2 * p] - mx);
      const float2 v = o2[p * (kHeadSize / 2)];
      z = fmaf(c, ml[2 * p + 1], z);
      o0 = fmaf(c, v.x, o0);
      o1 = fmaf(c, v.y, o1);
    }
    reinterpret_cast<uint32_t*>(out)[lane] = DT::pack2(o0 / z * out_scale, o1 / z * out_scale);
    return;
  }

  const int sg = lane >> 4;
  const int dg = lane & 15;
  float z = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 2
  for (int p = sg; p < n; p += 4) {
    const float c = exp2_fast(ml[2 * p] - mx);
    const float4* op = reinterpret_cast<const float4*>(o + p * kHeadSize) + 2 * dg;
    const float4 v0 = op[0];
    const float4 v1 = op[1];
    z = fmaf(c, ml[2 * p + 1], z);
    acc[0] = fmaf(c, v0.x, acc[0]);
    acc[1] = fmaf(c, v0.y, acc[1]);
    acc[2] = fmaf(c, v0.z, acc[2]);
    acc[3] = fmaf(c, v0.w, acc[3]);
    acc[4] = fmaf(c, v1.x, acc[4]);
    acc[5] = fmaf(c, v1.y, acc[5]);
    acc[6] = fmaf(c, v1.z, acc[6]);
    acc[7] = fmaf(c, v1.w, acc[7]);
  }
  z = cross_row_sum(z);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = cross_row_sum(acc[i]);
  if (sg == 0) {
    uint4 packed;
    packed.x = DT::pack2(acc[0] / z * out_scale, acc[1] / z * out_scale);
    packed.y = DT::pack2(acc[2] / z * out_scale, acc[3] / z * out_scale);
    packed.z = DT::pack2(acc[4] / z * out_scale, acc[5] / z * out_scale);
    packed.w = DT::pack2(acc[6] / z * out_scale, acc[7] / z * out_scale);
    reinterpret_cast<uint4*>(out)[dg] = packed;
  }
}

}  // namespace pkv
