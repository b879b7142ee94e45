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

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// Tokens of a sequence, clamped to what its block-table row can address.
__device__ inline int clamped_len(const DecodeArgs& a, int s) {
  int L = a.context_lens[s];
  const int cap = a.max_blocks_per_seq * kBlockSize;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

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
      const float x = (!kTail || col < nvalid) ? part * a.scale_log2e : kMaskedLogit;

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
      out_row[d] = DT::from_f32(O / Z * a.out_scale);
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
      for (int r = 0; r < 4; ++r) x[r] = (!kTail || 4 * grp + r < nvalid) ? S[r] * a.scale_log2e : kMaskedLogit;

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
      const float os = a.out_scale;
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
  lse_merge_row<DT>(a.ws_ml + 2 * base, a.ws_o + base * kHeadSize, n, a.out + row * kHeadSize, a.out_scale,
                    threadIdx.x & (kWave - 1));
}

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
