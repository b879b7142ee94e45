// Chunked-prefill paged attention for gfx950: multi-token queries, causal by
// position, on the matrix cores, and the log-sum-exp merge of its segment
// partials.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Chunked prefill: 4 waves x 16 (query position, head) rows of one KV head per
// work-group, on the matrix cores.  Each wave streams the work-group's whole
// segment of blocks for its own 16 rows (the 4 waves read the same pages at
// about the same time, so the repeats hit the compute unit's cache), masks
// every key beyond its row's position, and writes its rows itself.
// ---------------------------------------------------------------------------

// Blocks that the work-group holding chunk query qi streams: up to the block
// of its last query's position.  Shared by the prefill kernel and its reduce.
__device__ inline int prefill_wg_blocks(const PrefillArgs& pa, int L, int C, int qi) {
  const int per_wg = kWavesPerGroup * pa.pos_per_wave;
  const int last_q = min(C, (qi / per_wg + 1) * per_wg) - 1;
  return (L - C + last_q) / kBlockSize + 1;
}

template <class DT, class PF>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs pa) {
  const DecodeArgs& a = pa.d;
  // item (unit, sequence, query block, segment), segment fastest; XCD-aware
  // chunks as in decode's direct mode
  const int64_t total = static_cast<int64_t>(a.units) * a.num_seqs * pa.q_blocks * a.parts_max;
  const int64_t per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int64_t lam = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
  if (lam >= total) return;
  const int g = static_cast<int>(lam % a.parts_max);
  int64_t rest = lam / a.parts_max;
  const int qb = static_cast<int>(rest % pa.q_blocks);
  rest /= pa.q_blocks;
  const int s = static_cast<int>(rest % a.num_seqs);
  const int u = static_cast<int>(rest / a.num_seqs);
  const int kvh = u / a.head_tiles;
  const int tile = u - kvh * a.head_tiles;
  const int h0 = kvh * a.group + tile * 16;
  const int nh = min(pa.heads_per_tile, a.group - tile * 16);

  const int L = clamped_len(a, s);
  const int q0 = pa.query_start[s];
  const int C = min(max(pa.query_start[s + 1] - q0, 0), L);
  const int ppt = pa.pos_per_wave;
  const int wg_q0 = qb * kWavesPerGroup * ppt;
  if (wg_q0 >= C) return;  // uniform over the work-group
  const int nblk = prefill_wg_blocks(pa, L, C, wg_q0);
  const int nseg = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  if (g >= nseg) return;
  const int j0 = g * a.blocks_per_part;
  const int nb = min(a.blocks_per_part, nblk - j0);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int hpt = pa.heads_per_tile;
  // tile row r of this wave: position index r / hpt, head index r % hpt
  auto row_query = [&](int r) { return wg_q0 + wave * ppt + r / hpt; };
  auto row_valid = [&](int r) { return r / hpt < ppt && r % hpt < nh && row_query(r) < C; };
  const int pos_col = row_valid(col) ? L - C + row_query(col) : -1;  // -1: every key masked
  if (__ballot(pos_col >= 0) == 0) return;  // no row of this wave is a query (no barrier follows)

  float m = kInitMax;
  float z = 0.f;
  float4_t O[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) O[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  uint4 qf[4];
  if (pos_col >= 0) {
    const uint4* qrow = reinterpret_cast<const uint4*>(
        a.q + (static_cast<int64_t>(q0 + row_query(col)) * a.num_heads + h0 + col % hpt) * kHeadSize);
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[i] = qrow[4 * i + grp];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[i] = make_uint4(0, 0, 0, 0);
  }

  auto process = [&]<bool kTail>(uint4 (&kv)[4], uint4 (&vv)[4], int j) __attribute__((always_inline)) {
    const int nvalid = kTail ? min(kBlockSize, L - j * kBlockSize) : kBlockSize;
    float4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) S = DT::mfma_qk(kv[i], qf[i], S);
    float x[4];
    const int t0 = j * kBlockSize + 4 * grp;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = t0 + r <= pos_col ? S[r] * a.scale_log2e : kMaskedLogit;

    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = cross_row_max(bm);
    const float m_new = fmaxf(m, bm);
    const float alpha = exp2_fast(m - m_new);
    m = m_new;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = DT::round(exp2_fast(x[r] - m_new));
    z = z * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = lane_from(alpha, 4 * grp + r);
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O[jd][r] *= ar[r];
    }
    uint2 pa2;
    pa2.x = DT::pack2(pr[0], pr[1]);
    pa2.y = DT::pack2(pr[2], pr[3]);
    if (kTail && nvalid < kBlockSize) mask_v(vv, grp, nvalid);  // stale slots past the context
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      const uint4& f = vv[jd >> 1];
      const uint2 b = (jd & 1) ? make_uint2(f.z, f.w) : make_uint2(f.x, f.y);
      O[jd] = DT::mfma_pv(pa2, b, O[jd]);
    }
  };
  stream_blocks<PF>(a, s, kvh, j0, nb, lane, process);

  // O[jd][r]: row 4grp + r, dim 16 jd + col; lane c (< 16) holds row c's max and sum
  const float Zc = cross_row_sum(z);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tr = 4 * grp + r;
    const float Zr = lane_from(Zc, tr);
    const float mr = lane_from(m, tr);
    if (!row_valid(tr)) continue;
    const int64_t orow = static_cast<int64_t>(q0 + row_query(tr)) * a.num_heads + h0 + tr % hpt;
    if (nseg == 1) {
      uint16_t* dst = a.out + orow * kHeadSize + col;
      const float inv = a.out_scale / Zr;
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) dst[16 * jd] = DT::from_f32(O[jd][r] * inv);
    } else {
      const int64_t slot = orow * a.parts_max + g;
      float* dst = a.ws_o + slot * kHeadSize + col;
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) dst[16 * jd] = O[jd][r];
      if (col == 0) {
        a.ws_ml[2 * slot] = mr;
        a.ws_ml[2 * slot + 1] = Zr;
      }
    }
  }
}

// One wave per (query token, head) output row whose work-group streamed more
// than one segment.
template <class DT>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillArgs pa) {
  const DecodeArgs& a = pa.d;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + wave_id_uniform();
  if (row >= static_cast<int64_t>(pa.num_query_tokens) * a.num_heads) return;
  const int tq = static_cast<int>(row / a.num_heads);
  // sequence of query token tq: the last s with query_start[s] <= tq
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pa.query_start[mid] <= tq) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int L = clamped_len(a, s);
  const int q0 = pa.query_start[s];
  const int C = min(max(pa.query_start[s + 1] - q0, 0), L);
  const int qi = tq - q0;
  // no such query (a chunk longer than its context), or one past the grid
  // (a chunk longer than max_query_len): the prefill kernel wrote nothing for it
  if (qi >= C || qi >= pa.q_blocks * kWavesPerGroup * pa.pos_per_wave) return;
  const int nblk = prefill_wg_blocks(pa, L, C, qi);
  const int n = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  if (n <= 1) return;  // written directly by the prefill kernel
  const int64_t base = row * a.parts_max;
  lse_merge_row<DT>(a.ws_ml + 2 * base, a.ws_o + base * kHeadSize, n, a.out + row * kHeadSize, a.out_scale,
                    threadIdx.x & (kWave - 1));
}

template <class DT, class PF>
static hipError_t launch_prefill_t(const PrefillArgs& pa, hipStream_t stream) {
  const DecodeArgs& a = pa.d;
  const int64_t total = static_cast<int64_t>(a.units) * a.num_seqs * pa.q_blocks * a.parts_max;
  const int64_t grid = (total + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid > 0x7fffffff || grid <= 0) return hipErrorInvalidValue;
  prefill_kernel<DT, PF><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(pa);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.parts_max > 1) {
    const int64_t rows = static_cast<int64_t>(pa.num_query_tokens) * a.num_heads;
    const int64_t rgrid = (rows + kWavesPerGroup - 1) / kWavesPerGroup;
    if (rgrid > 0x7fffffff) return hipErrorInvalidValue;
    prefill_reduce_kernel<DT><<<dim3(static_cast<uint32_t>(rgrid)), dim3(256), 0, stream>>>(pa);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_prefill(const PrefillArgs& pa, int act_dtype, bool fp8_cache, hipStream_t stream) {
  if (fp8_cache)
    return act_dtype == 0 ? launch_prefill_t<F16, PageFp8<F16>>(pa, stream)
                          : launch_prefill_t<BF16, PageFp8<BF16>>(pa, stream);
  return act_dtype == 0 ? launch_prefill_t<F16, Page16>(pa, stream) : launch_prefill_t<BF16, Page16>(pa, stream);
}

}  // namespace pkv
