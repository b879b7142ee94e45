// Paged decode attention for gfx950.
//
// What is computed (page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐
// LLM 推理引擎", §2.1: QK dot products, softmax normalisation, weighted sum of
// V): for each sequence s and query head h, one query row attends to the
// context_lens[s] tokens whose K/V pages are found through the block table
// (page "vLLM 部署与 PagedAttention 原理 · 检索整理", item 2).
//
// How (this library's design, not the pages'):
//   * a row is (sequence, unit), where a unit is a KV head (MHA) or a tile of
//     up to 16 query heads of one KV head (GQA).  A row's blocks are cut into
//     segments of blocks_per_part blocks; a work item is one segment, and one
//     work-group of 4 waves owns it: each wave streams an equal share of the
//     segment's pages (four contiguous 1 KiB loads per K page and per V page,
//     one block ahead), and the 4 partial softmax states are merged through
//     LDS.  A row of one segment is written directly; a longer row writes one
//     (m, Z, unnormalised O) partial per segment and decode_reduce_kernel
//     merges them with the log-sum-exp identity.
//   * planned mode: a one-work-group pre-pass (plan.hip) lists the non-empty
//     segments, full ones first and partial ones by size, largest first.
//     Work-groups take their items from it by index, per XCD, so no
//     work-group in the body of the grid is dispatched just to exit, the
//     longest items run first and the shortest last, and neighbouring items
//     (parallel samples sharing prompt pages) run together on one XCD's L2.
//     The grid is an upper bound: work-groups past the end of the list,
//     dispatched last, exit at once.  Direct mode (very large batches) maps
//     blockIdx to items directly.
//   * softmax is online in base 2: logits are pre-multiplied by
//     scale * log2(e) and exponentiated with v_exp_f32.
//   * MHA (one query head per KV head): the dot products run on the vector
//     ALU (v_dot2), reduced across the four 16-lane rows; the running max is
//     wave-uniform (DPP row max), and the weights of tokens 4G..4G+3 are
//     handed to row G with ds_bpermute for the V accumulation.
//   * GQA (g query heads per KV head): S = K Q^T on v_mfma_f32_16x16x32 and
//     O += P V on v_mfma_f32_16x16x16, up to 16 heads per tile, per-head
//     running max.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"

namespace pkv {

// Direct mode: work-group -> item, XCD-aware.  Work-groups are dispatched to
// the 8 XCDs round-robin (XCD = blockIdx.x % 8), each XCD with its own L2.
// The item space is ordered (unit, segment, sequence) and cut into 8
// contiguous chunks, one per XCD, so consecutive sequences (parallel samples
// sharing prompt blocks) run together on one L2.  Returns false for padding
// work-groups.
__device__ inline bool direct_item(const DecodeArgs& a, int& s, int& u, int& g) {
  const int64_t total = static_cast<int64_t>(a.units) * a.parts_max * a.num_seqs;
  const int64_t per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int64_t w = blockIdx.x;
  const int64_t lam = (w % kNumXcd) * per_xcd + w / kNumXcd;
  if (lam >= total) return false;
  s = static_cast<int>(lam % a.num_seqs);
  const int64_t rest = lam / a.num_seqs;
  g = static_cast<int>(rest % a.parts_max);
  u = static_cast<int>(rest / a.parts_max);
  return true;
}

// Planned mode: item x of XCD xcd's work list, from the plan (plan.hip).  The
// XCD's list is its eighth of list A (full segments, all units, unit-major)
// followed by its share of list B (partial segments, size descending), dealt
// to the XCDs in runs of 4 consecutive items.  Work-group w runs on XCD w % 8
// and takes item w / 8 of that XCD's list; returns false past its end.
__device__ inline bool planned_item(const DecodeArgs& a, int xcd, uint32_t x, int& s, int& u, int& g) {
  // all item counts fit 31 bits (the host plans only such calls), so 32-bit
  // unsigned arithmetic is exact here
  const int* plan = a.plan;
  const uint32_t units = static_cast<uint32_t>(a.units);
  const uint32_t F = static_cast<uint32_t>(plan[kPlanFull]);
  const uint32_t na = units * F;
  const uint32_t a0 = static_cast<uint32_t>((static_cast<uint64_t>(xcd) * na) >> 3);
  const uint32_t a1 = static_cast<uint32_t>((static_cast<uint64_t>(xcd + 1) * na) >> 3);
  if (x < a1 - a0) {
    const uint32_t gi = a0 + x;
    const uint32_t uu = gi / F;
    const uint32_t packed = static_cast<uint32_t>(plan[kPlanHeaderInts + (gi - uu * F)]);
    u = static_cast<int>(uu);
    s = static_cast<int>(packed & ((1u << kPlanSeqBits) - 1));
    g = static_cast<int>(packed >> kPlanSeqBits);
    return true;
  }
  const uint32_t y = x - (a1 - a0);
  const uint32_t b = ((y >> 2) * kNumXcd + xcd) * 4 + (y & 3);
  const uint32_t np = static_cast<uint32_t>(plan[kPlanPartial]);
  if (b >= units * np) return false;
  // size class c: b in [units * off[c], units * off[c + 1])
  const int* off = plan + kPlanClassOff;
  int c = 0;
#pragma unroll
  for (int step = kPlanClasses / 2; step > 0; step >>= 1)
    if (units * static_cast<uint32_t>(off[c + step]) <= b) c += step;
  const uint32_t kc = static_cast<uint32_t>(off[c + 1] - off[c]);
  const uint32_t r = b - units * static_cast<uint32_t>(off[c]);
  const uint32_t uu = r / kc;
  u = static_cast<int>(uu);
  s = plan[kPlanHeaderInts + static_cast<int64_t>(a.num_seqs) * a.parts_max + off[c] + (r - uu * kc)];
  const int nblk = (clamped_len(a, s) + kBlockSize - 1) / kBlockSize;
  g = nblk / a.blocks_per_part;  // the partial segment is the last one
  return true;
}

__device__ inline bool work_group_item(const DecodeArgs& a, int& s, int& u, int& g) {
  return a.planned ? planned_item(a, blockIdx.x % kNumXcd, blockIdx.x / kNumXcd, s, u, g) : direct_item(a, s, u, g);
}

__host__ inline int64_t item_grid(const DecodeArgs& a) {
  const int64_t total = static_cast<int64_t>(a.units) * a.parts_max * a.num_seqs;
  // Planned: the lists of the 8 XCDs differ in length by at most 5 items from
  // an even split, so 8 spare work-groups per XCD cover any list.
  return ((total + kNumXcd - 1) / kNumXcd + (a.planned ? 8 : 0)) * kNumXcd;
}

// Block range of wave `wave` inside segment g of a row with nblk blocks.
struct WaveRange {
  int j0, nb, nseg;
};
__device__ inline WaveRange wave_range(const DecodeArgs& a, int nblk, int g, int wave) {
  const int bpp = a.blocks_per_part;
  const int nseg = (nblk + bpp - 1) / bpp;
  const int s0 = g * bpp;
  const int n = min(bpp, nblk - s0);
  const int lo = s0 + (wave * n) / kWavesPerGroup;
  const int hi = s0 + ((wave + 1) * n) / kWavesPerGroup;
  return WaveRange{lo, hi - lo, nseg};
}

// ---------------------------------------------------------------------------
// MHA: one query head per KV head.
// ---------------------------------------------------------------------------
template <class DT, class PF>
__global__ __launch_bounds__(256, DT::kMhaWavesPerSimd) void decode_mha_kernel(DecodeArgs a) {
  __shared__ float red_o[kWavesPerGroup][kHeadSize];
  __shared__ float red_m[kWavesPerGroup];
  __shared__ float red_z[kWavesPerGroup];

  int s, h, g;
  if (!work_group_item(a, s, h, g)) return;  // uniform over the work-group
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int nblk = (clamped_len(a, s) + kBlockSize - 1) / kBlockSize;
  const WaveRange wr = wave_range(a, nblk, g, wave);
  if (g >= wr.nseg) {  // direct mode past the row's end (uniform over the work-group)
    if (g == 0 && threadIdx.x < kHeadSize)  // empty context: zero row
      a.out[(static_cast<int64_t>(s) * a.num_heads + h) * kHeadSize + threadIdx.x] = 0;
    return;
  }
  const int row_s = s, j_begin = wr.j0, j_count = wr.nb, nseg = wr.nseg;
  const int L = clamped_len(a, row_s);
  const float sl2e = head_logit_scale(a, h);  // MHA: the unit is the KV head
  uint16_t* out_row = a.out + (static_cast<int64_t>(row_s) * a.num_heads + h) * kHeadSize;
  const int grp = lane >> 4;
  const int col = lane & 15;

  float m = kInitMax;
  float z = 0.f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  if (j_count > 0) {
    const uint4* qrow =
        reinterpret_cast<const uint4*>(a.q + (static_cast<int64_t>(row_s) * a.num_heads + h) * kHeadSize);
    uint4 qf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[i] = qrow[4 * i + grp];
    const int src_row_lane = 20 * grp;  // lane 16*grp + 4*grp holds token 4*grp's weight in row grp

    // One block: QK, online softmax, V accumulation.  kTail: the last block of
    // the range, which may be the sequence's partial last block; every other
    // block is full and needs no masking.
    auto process = [&]<bool kTail>(uint4 (&kv)[4], uint4 (&vv)[4], int j) __attribute__((always_inline)) {
      const int nvalid = kTail ? min(kBlockSize, L - j * kBlockSize) : kBlockSize;

      // QK: lane (grp, col) holds 32 of token col's 128 dims
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) part = dot8<DT>(qf[i], kv[i], part);
      part = cross_row_sum(part);
      const float x = (!kTail || col < nvalid) ? part * sl2e : kMaskedLogit;

      // online softmax with a wave-uniform running max
      const float m_new = fmaxf(m, row_max16(x));
      const float alpha = exp2_fast(m - m_new);
      const float w = exp2_fast(x - m_new);
      m = m_new;
      z = z * alpha + w;

      float wi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wi[i] = lane_from(w, src_row_lane + i);
      if (kTail && nvalid < kBlockSize) mask_v(vv, grp, nvalid);

      // V: lane (grp, col) holds tokens 4grp..4grp+3 of dims 16j + col, j = 0..7
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int jd = 2 * pp + half;
          float a_j = acc[jd] * alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) a_j = fmaf(wi[i], elem<DT>(vv[pp], 4 * half + i), a_j);
          acc[jd] = a_j;
        }
      }
    };
    stream_blocks<PF>(a, row_s, h, j_begin, j_count, lane, process);
    z = row_sum16(z);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = cross_row_sum(acc[j]);
  }

  // lane (grp, col) holds dims 32grp + col and 32grp + 16 + col
  const int d_a = 32 * grp + col;
  red_o[wave][d_a] = grp == 0 ? acc[0] : grp == 1 ? acc[2] : grp == 2 ? acc[4] : acc[6];
  red_o[wave][d_a + 16] = grp == 0 ? acc[1] : grp == 1 ? acc[3] : grp == 2 ? acc[5] : acc[7];
  if (lane == 0) {
    red_m[wave] = m;
    red_z[wave] = z;
  }
  __syncthreads();

  // merge the 4 waves: M = max m_w, c_w = 2^(m_w - M), O = sum c_w O_w / sum c_w Z_w
  const int d = threadIdx.x;
  if (d < kHeadSize) {
    const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    float Z = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      const float c = exp2_fast(red_m[w] - M);
      Z = fmaf(c, red_z[w], Z);
      O = fmaf(c, red_o[w][d], O);
    }
    if (nseg == 1) {
      out_row[d] = DT::from_f32(O / Z * head_out_scale(a, h));
    } else {
      const int64_t slot = (static_cast<int64_t>(s) * a.num_heads + h) * a.parts_max + g;
      a.ws_o[slot * kHeadSize + d] = O;
      if (d == 0) {
        a.ws_ml[2 * slot] = M;
        a.ws_ml[2 * slot + 1] = Z;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GQA: up to 16 query heads of one KV head per work-group, on the matrix cores.
// ---------------------------------------------------------------------------
template <class DT, class PF>
__global__ __launch_bounds__(256) void decode_gqa_kernel(DecodeArgs a) {
  __shared__ float red_o[kWavesPerGroup][16][kHeadSize];
  __shared__ float red_m[kWavesPerGroup][16];
  __shared__ float red_z[kWavesPerGroup][16];

  int s, ht, g;
  if (!work_group_item(a, s, ht, g)) return;  // uniform over the work-group
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int kvh = ht / a.head_tiles;
  const int tile = ht - kvh * a.head_tiles;
  const int h0 = kvh * a.group + tile * 16;
  const int nh = min(16, a.group - tile * 16);
  const int grp = lane >> 4;
  const int col = lane & 15;
  const float sl2e = head_logit_scale(a, kvh);

  const int L = clamped_len(a, s);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const WaveRange wr = wave_range(a, nblk, g, wave);
  uint16_t* out_seq = a.out + static_cast<int64_t>(s) * a.num_heads * kHeadSize;
  if (g >= wr.nseg) {  // direct mode past the row's end (uniform over the work-group)
    if (g == 0)        // empty context: zero rows
      for (int e = threadIdx.x; e < nh * kHeadSize; e += 256) out_seq[static_cast<int64_t>(h0) * kHeadSize + e] = 0;
    return;
  }

  float m = kInitMax;  // running max of head `col`
  float z = 0.f;       // this lane's share of head `col`'s softmax sum
  float4_t O[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) O[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  if (wr.nb > 0) {
    // B operand of S = K Q^T: lane (grp, col) holds head col, dims 8*(4i + grp) .. +8
    uint4 qf[4];
    if (col < nh) {
      const uint4* qrow =
          reinterpret_cast<const uint4*>(a.q + (static_cast<int64_t>(s) * a.num_heads + h0 + col) * kHeadSize);
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = qrow[4 * i + grp];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = make_uint4(0, 0, 0, 0);
    }

    auto process = [&]<bool kTail>(uint4 (&kv)[4], uint4 (&vv)[4], int j) __attribute__((always_inline)) {
      const int nvalid = kTail ? min(kBlockSize, L - j * kBlockSize) : kBlockSize;

      // S[token 4grp + r][head col]
      float4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) S = DT::mfma_qk(kv[i], qf[i], S);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = (!kTail || 4 * grp + r < nvalid) ? S[r] * sl2e : kMaskedLogit;

      float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bm = cross_row_max(bm);
      const float m_new = fmaxf(m, bm);
      const float alpha = exp2_fast(m - m_new);
      m = m_new;
      // weights rounded to the operand type once; the sum uses the same values
      // the matrix op multiplies with
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = DT::round(exp2_fast(x[r] - m_new));
      z = z * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));

      // rows of O are heads 4grp + r: fetch their rescale factors
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = lane_from(alpha, 4 * grp + r);
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[jd][r] *= ar[r];
      }

      // A operand of O += P V: lane (grp, col) holds P[head col][tokens 4grp..4grp+3]
      uint2 pa;
      pa.x = DT::pack2(pr[0], pr[1]);
      pa.y = DT::pack2(pr[2], pr[3]);
      if (kTail && nvalid < kBlockSize) mask_v(vv, grp, nvalid);
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
        const uint4& f = vv[jd >> 1];
        const uint2 b = (jd & 1) ? make_uint2(f.z, f.w) : make_uint2(f.x, f.y);
        O[jd] = DT::mfma_pv(pa, b, O[jd]);
      }
    };
    stream_blocks<PF>(a, s, kvh, wr.j0, wr.nb, lane, process);
  }

  // this wave's state: O[j][r] is head 4grp + r, dim 16j + col; m and the
  // full sum of head col
  const float Zc = cross_row_sum(z);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red_o[wave][4 * grp + r][16 * j + col] = O[j][r];
  }
  if (grp == 0) {
    red_m[wave][col] = m;
    red_z[wave][col] = Zc;
  }
  __syncthreads();

  // merge the 4 waves: thread -> head t / 16, dims 8 (t % 16) .. + 8
  const int hh = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * 8;
  if (hh < nh) {
    const float M = fmaxf(fmaxf(red_m[0][hh], red_m[1][hh]), fmaxf(red_m[2][hh], red_m[3][hh]));
    float c[kWavesPerGroup];
    float Z = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      c[w] = exp2_fast(red_m[w][hh] - M);
      Z = fmaf(c[w], red_z[w][hh], Z);
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kWavesPerGroup; ++w) t = fmaf(c[w], red_o[w][hh][d0 + e], t);
      o[e] = t;
    }
    if (wr.nseg == 1) {
      uint16_t* orow = out_seq + static_cast<int64_t>(h0 + hh) * kHeadSize + d0;
      uint4 packed;
      const float os = head_out_scale(a, kvh);
      packed.x = DT::pack2(o[0] / Z * os, o[1] / Z * os);
      packed.y = DT::pack2(o[2] / Z * os, o[3] / Z * os);
      packed.z = DT::pack2(o[4] / Z * os, o[5] / Z * os);
      packed.w = DT::pack2(o[6] / Z * os, o[7] / Z * os);
      *reinterpret_cast<uint4*>(orow) = packed;
    } else {
      const int64_t slot = (static_cast<int64_t>(s) * a.num_heads + h0 + hh) * a.parts_max + g;
      float4* dst = reinterpret_cast<float4*>(a.ws_o + slot * kHeadSize + d0);
      dst[0] = make_float4(o[0], o[1], o[2], o[3]);
      dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      if (d0 == 0) {
        a.ws_ml[2 * slot] = M;
        a.ws_ml[2 * slot + 1] = Z;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of segment partials.
// ---------------------------------------------------------------------------
// One wave per (sequence, head) row with more than one segment; 4 rows per
// work-group.
template <class DT>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + wave_id_uniform();
  if (row >= static_cast<int64_t>(a.num_seqs) * a.num_heads) return;
  const int s = static_cast<int>(row / a.num_heads);
  const int L = clamped_len(a, s);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int n = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  if (n <= 1) return;  // written directly by the decode kernel
  const int64_t base = row * a.parts_max;
  const int kvh = static_cast<int>(row % a.num_heads) / a.group;
  lse_merge_row<DT>(a.ws_ml + 2 * base, a.ws_o + base * kHeadSize, n, a.out + row * kHeadSize,
                    head_out_scale(a, kvh), threadIdx.x & (kWave - 1));
}

// The decode call's page reads alone: the same work items, wave ranges, block
// stream and load instructions as the decode kernels, with no arithmetic
// beyond folding the loaded words together.  Its duration is the ceiling the
// memory system puts on the decode call for a batch (a diagnostic).
template <class PF>
__global__ __launch_bounds__(256) void decode_read_pages_kernel(DecodeArgs a, uint32_t* sink) {
  int s, u, g;
  if (!work_group_item(a, s, u, g)) return;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int kvh = a.group == 1 ? u : u / a.head_tiles;
  const int nblk = (clamped_len(a, s) + kBlockSize - 1) / kBlockSize;
  const WaveRange wr = wave_range(a, nblk, g, wave);
  if (g >= wr.nseg || wr.nb <= 0) return;
  uint32_t acc = 0;
  auto process = [&]<bool kTail>(uint4 (&kv)[4], uint4 (&vv)[4], int) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= kv[i].x ^ kv[i].y ^ kv[i].z ^ kv[i].w ^ vv[i].x ^ vv[i].y ^ vv[i].z ^ vv[i].w;
  };
  stream_blocks<PF>(a, s, kvh, wr.j0, wr.nb, lane, process);
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; a store only on that exact value
}

hipError_t launch_decode_read_pages(const DecodeArgs& a, bool fp8_cache, uint32_t* sink, hipStream_t stream) {
  const int64_t grid = item_grid(a);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (fp8_cache)
    decode_read_pages_kernel<PageFp8<F16>><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a, sink);
  else
    decode_read_pages_kernel<Page16><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a, sink);
  return hipGetLastError();
}

template <class DT, class PF>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t grid = item_grid(a);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (a.group == 1)
    decode_mha_kernel<DT, PF><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a);
  else
    decode_gqa_kernel<DT, PF><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.parts_max > 1) {
    const int64_t rgrid = (static_cast<int64_t>(a.num_seqs) * a.num_heads + kWavesPerGroup - 1) / kWavesPerGroup;
    decode_reduce_kernel<DT><<<dim3(static_cast<uint32_t>(rgrid)), dim3(256), 0, stream>>>(a);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_decode(const DecodeArgs& a, int act_dtype, bool fp8_cache, hipStream_t stream) {
  if (fp8_cache)
    return act_dtype == 0 ? launch_decode_t<F16, PageFp8<F16>>(a, stream) : launch_decode_t<BF16, PageFp8<BF16>>(a, stream);
  return act_dtype == 0 ? launch_decode_t<F16, Page16>(a, stream) : launch_decode_t<BF16, Page16>(a, stream);
}

}  // namespace pkv
