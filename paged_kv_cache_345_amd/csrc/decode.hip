// Paged decode attention for gfx950.
//
// What is computed (page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐
// LLM 推理引擎", §2.1: QK dot products, softmax normalisation, weighted sum of
// V): for each sequence s and query head h, one query row attends to the
// context_lens[s] tokens whose K/V pages are found through the block table
// (page "vLLM 部署与 PagedAttention 原理 · 检索整理", item 2).
//
// How (this library's design, not the pages'):
//   * work item = (sequence, KV head [, 16-head tile], partition of
//     blocks_per_part blocks).  One 64-lane wave owns one item; a work-group is
//     four independent waves.  Each wave streams its pages with four
//     contiguous 1 KiB loads per K page and per V page, one block ahead.
//   * softmax is online in base 2: logits are pre-multiplied by
//     scale * log2(e) and exponentiated with v_exp_f32.
//   * MHA (one query head per KV head): the dot products run on the vector
//     ALU (v_dot2), reduced across the four 16-lane rows; the running max is
//     wave-uniform (DPP row max), and the weights of tokens 4G..4G+3 are
//     handed to row G with ds_bpermute for the V accumulation.
//   * GQA (g query heads per KV head): S = K Q^T on v_mfma_f32_16x16x32 and
//     O += P V on v_mfma_f32_16x16x16, up to 16 heads per tile, per-head
//     running max.
//   * a sequence with more than one partition writes (m, Z, unnormalised O)
//     partials; decode_reduce_kernel merges them with the log-sum-exp
//     identity, staging the partition weights in LDS.

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

// Work-group -> work items, XCD-aware.  Work-groups are dispatched to the 8
// XCDs round-robin (XCD = blockIdx.x % 8), each XCD with its own L2.  The
// logical work space is ordered (head [x tile], partition, group of 4
// consecutive sequences) and cut into 8 contiguous chunks, one per XCD: each
// XCD walks a few heads, partition by partition, through the sequences in
// order, and the 4 waves of a work-group take 4 consecutive sequences.
// Sequences that share prompt blocks (parallel samples, numbered
// consecutively) thus read the same pages on the same CU and L2 at about the
// same time.  Returns false for padding work-groups and missing sequences.
__device__ inline bool xcd_item(const DecodeArgs& a, int heads, int& s, int& h, int& p) {
  const int64_t n_sb = (a.num_seqs + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t total = static_cast<int64_t>(heads) * a.parts_max * n_sb;
  const int64_t per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int64_t w = blockIdx.x;
  const int64_t lam = (w % kNumXcd) * per_xcd + w / kNumXcd;
  if (lam >= total) return false;
  const int64_t sb = lam % n_sb;
  const int64_t rest = lam / n_sb;
  p = static_cast<int>(rest % a.parts_max);
  h = static_cast<int>(rest / a.parts_max);
  s = static_cast<int>(sb * kWavesPerGroup) + wave_id_uniform();
  return s < a.num_seqs;
}

__host__ inline int64_t xcd_grid(int64_t heads, int64_t parts, int64_t num_seqs) {
  const int64_t n_sb = (num_seqs + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t total = heads * parts * n_sb;
  return ((total + kNumXcd - 1) / kNumXcd) * kNumXcd;
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

// Four contiguous 1 KiB wave loads per K page and per V page, as raw buffer
// loads: one buffer descriptor per page (wave-uniform, scalar registers, with a
// 4 KiB record limit) and a single per-lane byte offset shared by K and V.
__device__ inline void load_page(uint4 (&kv)[4], uint4 (&vv)[4], const uint16_t* kp, const uint16_t* vp,
                                 uint32_t lane_bytes) {
  const __amdgpu_buffer_rsrc_t kr = page_rsrc(kp);
  const __amdgpu_buffer_rsrc_t vr = page_rsrc(vp);
  kv[0] = load16<0>(kr, lane_bytes);
  kv[1] = load16<1024>(kr, lane_bytes);
  kv[2] = load16<2048>(kr, lane_bytes);
  kv[3] = load16<3072>(kr, lane_bytes);
  vv[0] = load16<0>(vr, lane_bytes);
  vv[1] = load16<1024>(vr, lane_bytes);
  vv[2] = load16<2048>(vr, lane_bytes);
  vv[3] = load16<3072>(vr, lane_bytes);
}

// ---------------------------------------------------------------------------
// MHA: one query head per KV head.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(256, 4) void decode_mha_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int H = a.num_kv_heads;
  int s, h, p;
  if (!xcd_item(a, H, s, h, p)) return;

  const int L = clamped_len(a, s);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int n_parts = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  uint16_t* out_row = a.out + (static_cast<int64_t>(s) * a.num_heads + h) * kHeadSize;
  if (p >= n_parts) {
    if (p == 0) {  // empty context: defined zero output
      out_row[2 * lane] = 0;
      out_row[2 * lane + 1] = 0;
    }
    return;
  }
  const int j0 = p * a.blocks_per_part;
  const int nb = min(a.blocks_per_part, nblk - j0);
  const int grp = lane >> 4;
  const int col = lane & 15;

  int my_bid = 0;
  if (lane < nb) my_bid = a.block_tables[static_cast<int64_t>(s) * a.max_blocks_per_seq + j0 + lane];

  const uint4* qrow = reinterpret_cast<const uint4*>(a.q + (static_cast<int64_t>(s) * a.num_heads + h) * kHeadSize);
  uint4 qf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qf[i] = qrow[4 * i + grp];

  const int64_t page_stride = static_cast<int64_t>(H) * kPageElems;
  const int64_t head_off = static_cast<int64_t>(h) * kPageElems;
  const int src_row_lane = 20 * grp;  // lane 16*grp + 4*grp holds token 4*grp's weight in row grp

  float m = kInitMax;
  float z = 0.f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  // One block of this partition: QK, online softmax, V accumulation.
  // kTail: the sequence's last block, which may hold fewer than 16 tokens;
  // every other block is full and needs no masking.
  auto process = [&]<bool kTail>(uint4 (&kv)[4], uint4 (&vv)[4], int jj) __attribute__((always_inline)) {
    const int nvalid = kTail ? min(kBlockSize, L - (j0 + jj) * kBlockSize) : kBlockSize;

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
        const int j = 2 * pp + half;
        float a_j = acc[j] * alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) a_j = fmaf(wi[i], elem<DT>(vv[pp], 4 * half + i), a_j);
        acc[j] = a_j;
      }
    }
  };
  auto issue = [&](uint4 (&kv)[4], uint4 (&vv)[4], int jj) __attribute__((always_inline)) {
    const int bid = __builtin_amdgcn_readlane(my_bid, jj);
    const bool bad = static_cast<unsigned>(bid) >= static_cast<unsigned>(a.num_blocks);
    const int64_t off = static_cast<int64_t>(bad ? 0 : bid) * page_stride + head_off;
    load_page(kv, vv, a.k_cache + off, a.v_cache + off, static_cast<uint32_t>(lane) * 16u);
  };

  // two register sets: one block in flight while the other is consumed
  uint4 ka[4], va[4], kb[4], vb[4];
  issue(ka, va, 0);
  int jj = 0;
  // steady state: full blocks only and no conditional loads, so each wait
  // leaves the other register set in flight
  for (; jj + 2 < nb; jj += 2) {
    issue(kb, vb, jj + 1);
    process.template operator()<false>(ka, va, jj);
    issue(ka, va, jj + 2);
    process.template operator()<false>(kb, vb, jj + 1);
  }
  if (jj + 1 < nb) {
    issue(kb, vb, jj + 1);
    process.template operator()<false>(ka, va, jj);
    process.template operator()<true>(kb, vb, jj + 1);
  } else {
    process.template operator()<true>(ka, va, jj);
  }

  z = row_sum16(z);
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = cross_row_sum(acc[j]);
  // lane (grp, col) stores dims 16*(2grp) + col and 16*(2grp+1) + col
  const float o_a = grp == 0 ? acc[0] : grp == 1 ? acc[2] : grp == 2 ? acc[4] : acc[6];
  const float o_b = grp == 0 ? acc[1] : grp == 1 ? acc[3] : grp == 2 ? acc[5] : acc[7];
  const int d_a = 32 * grp + col;
  const int d_b = d_a + 16;
  if (n_parts == 1) {
    out_row[d_a] = DT::from_f32(o_a / z);
    out_row[d_b] = DT::from_f32(o_b / z);
  } else {
    const int64_t slot = (static_cast<int64_t>(s) * a.num_heads + h) * a.parts_max + p;
    float* o = a.ws_o + slot * kHeadSize;
    o[d_a] = o_a;
    o[d_b] = o_b;
    if (lane == 0) {
      a.ws_ml[2 * slot] = m;
      a.ws_ml[2 * slot + 1] = z;
    }
  }
}

// ---------------------------------------------------------------------------
// GQA: up to 16 query heads of one KV head per wave, on the matrix cores.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(256) void decode_gqa_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int Hkv = a.num_kv_heads;
  int s, ht, p;
  if (!xcd_item(a, Hkv * a.head_tiles, s, ht, p)) return;
  const int kvh = ht / a.head_tiles;
  const int tile = ht - kvh * a.head_tiles;

  const int h0 = kvh * a.group + tile * 16;
  const int nh = min(16, a.group - tile * 16);
  const int grp = lane >> 4;
  const int col = lane & 15;

  const int L = clamped_len(a, s);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int n_parts = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  uint16_t* out_seq = a.out + static_cast<int64_t>(s) * a.num_heads * kHeadSize;
  if (p >= n_parts) {
    if (p == 0) {  // empty context: defined zero output
      for (int e = lane; e < nh * kHeadSize; e += kWave) out_seq[static_cast<int64_t>(h0) * kHeadSize + e] = 0;
    }
    return;
  }
  const int j0 = p * a.blocks_per_part;
  const int nb = min(a.blocks_per_part, nblk - j0);

  int my_bid = 0;
  if (lane < nb) my_bid = a.block_tables[static_cast<int64_t>(s) * a.max_blocks_per_seq + j0 + lane];

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

  const int64_t page_stride = static_cast<int64_t>(Hkv) * kPageElems;
  const int64_t head_off = static_cast<int64_t>(kvh) * kPageElems;

  float m = kInitMax;  // running max of head `col`
  float z = 0.f;       // this lane's share of head `col`'s softmax sum
  float4_t O[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) O[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto process = [&]<bool kTail>(uint4 (&kv)[4], uint4 (&vv)[4], int jj) __attribute__((always_inline)) {
    const int nvalid = kTail ? min(kBlockSize, L - (j0 + jj) * kBlockSize) : kBlockSize;

    // S[token 4grp + r][head col]
    float4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) S = DT::mfma_qk(kv[i], qf[i], S);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      x[r] = (!kTail || 4 * grp + r < nvalid) ? S[r] * a.scale_log2e : kMaskedLogit;

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
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O[j][r] *= ar[r];
    }

    // A operand of O += P V: lane (grp, col) holds P[head col][tokens 4grp..4grp+3]
    uint2 pa;
    pa.x = DT::pack2(pr[0], pr[1]);
    pa.y = DT::pack2(pr[2], pr[3]);
    if (kTail && nvalid < kBlockSize) mask_v(vv, grp, nvalid);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4& f = vv[j >> 1];
      const uint2 b = (j & 1) ? make_uint2(f.z, f.w) : make_uint2(f.x, f.y);
      O[j] = DT::mfma_pv(pa, b, O[j]);
    }
  };
  auto issue = [&](uint4 (&kv)[4], uint4 (&vv)[4], int jj) __attribute__((always_inline)) {
    const int bid = __builtin_amdgcn_readlane(my_bid, jj);
    const bool bad = static_cast<unsigned>(bid) >= static_cast<unsigned>(a.num_blocks);
    const int64_t off = static_cast<int64_t>(bad ? 0 : bid) * page_stride + head_off;
    load_page(kv, vv, a.k_cache + off, a.v_cache + off, static_cast<uint32_t>(lane) * 16u);
  };

  uint4 ka[4], va[4], kb[4], vb[4];
  issue(ka, va, 0);
  int jj = 0;
  // steady state: full blocks only and no conditional loads, so each wait
  // leaves the other register set in flight
  for (; jj + 2 < nb; jj += 2) {
    issue(kb, vb, jj + 1);
    process.template operator()<false>(ka, va, jj);
    issue(ka, va, jj + 2);
    process.template operator()<false>(kb, vb, jj + 1);
  }
  if (jj + 1 < nb) {
    issue(kb, vb, jj + 1);
    process.template operator()<false>(ka, va, jj);
    process.template operator()<true>(kb, vb, jj + 1);
  } else {
    process.template operator()<true>(ka, va, jj);
  }

  const float Z = cross_row_sum(z);  // head col's total
  float zr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) zr[r] = lane_from(Z, 4 * grp + r);
  if (n_parts == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = 4 * grp + r;
      if (hr < nh) {
        uint16_t* orow = out_seq + static_cast<int64_t>(h0 + hr) * kHeadSize;
#pragma unroll
        for (int j = 0; j < 8; ++j) orow[16 * j + col] = DT::from_f32(O[j][r] / zr[r]);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = 4 * grp + r;
      if (hr < nh) {
        const int64_t slot = (static_cast<int64_t>(s) * a.num_heads + h0 + hr) * a.parts_max + p;
        float* o = a.ws_o + slot * kHeadSize;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[16 * j + col] = O[j][r];
      }
    }
    if (grp == 0 && col < nh) {
      const int64_t slot = (static_cast<int64_t>(s) * a.num_heads + h0 + col) * a.parts_max + p;
      a.ws_ml[2 * slot] = m;
      a.ws_ml[2 * slot + 1] = Z;
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partition partials: one work-group per (seq, head).
//   M = max_p m_p,  c_p = 2^(m_p - M),  out = sum_p c_p O_p / sum_p c_p Z_p
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  __shared__ float wts[kMaxPartitions];
  __shared__ float red[8 * kHeadSize];
  __shared__ float scal[8];
  const int tid = threadIdx.x;
  const int s = blockIdx.x / a.num_heads;
  const int h = blockIdx.x - s * a.num_heads;
  const int L = clamped_len(a, s);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int n = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  if (n <= 1) return;  // written directly by the decode kernel
  const int64_t base = (static_cast<int64_t>(s) * a.num_heads + h) * a.parts_max;
  const float* ml = a.ws_ml + 2 * base;

  float mx = -__builtin_inff();
  for (int p = tid; p < n; p += 256) mx = fmaxf(mx, ml[2 * p]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  if ((tid & 63) == 0) scal[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(scal[0], scal[1]), fmaxf(scal[2], scal[3]));

  float zs = 0.f;
  for (int p = tid; p < n; p += 256) {
    const float w = exp2_fast(ml[2 * p] - mx);
    wts[p] = w;
    zs += w * ml[2 * p + 1];
  }
  zs += __shfl_xor(zs, 32, 64);
  zs += __shfl_xor(zs, 16, 64);
  zs += __shfl_xor(zs, 8, 64);
  zs += __shfl_xor(zs, 4, 64);
  zs += __shfl_xor(zs, 2, 64);
  zs += __shfl_xor(zs, 1, 64);
  if ((tid & 63) == 0) scal[4 + (tid >> 6)] = zs;
  __syncthreads();
  const float Z = (scal[4] + scal[5]) + (scal[6] + scal[7]);

  // thread -> (partition group pg of 8, dims 4*dl .. 4*dl+3)
  const int pg = tid >> 5;
  const int dl = tid & 31;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = pg; p < n; p += 8) {
    const float w = wts[p];
    const float4 o = reinterpret_cast<const float4*>(a.ws_o + (base + p) * kHeadSize)[dl];
    acc.x = fmaf(w, o.x, acc.x);
    acc.y = fmaf(w, o.y, acc.y);
    acc.z = fmaf(w, o.z, acc.z);
    acc.w = fmaf(w, o.w, acc.w);
  }
  reinterpret_cast<float4*>(red + pg * kHeadSize)[dl] = acc;
  __syncthreads();
  if (tid < kHeadSize) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) t += red[g * kHeadSize + tid];
    a.out[(static_cast<int64_t>(s) * a.num_heads + h) * kHeadSize + tid] = DT::from_f32(t / Z);
  }
}

template <class DT>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t heads = static_cast<int64_t>(a.num_kv_heads) * (a.group == 1 ? 1 : a.head_tiles);
  const int64_t grid = xcd_grid(heads, a.parts_max, a.num_seqs);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (a.group == 1)
    decode_mha_kernel<DT><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a);
  else
    decode_gqa_kernel<DT><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.parts_max > 1) {
    const int64_t rgrid = static_cast<int64_t>(a.num_seqs) * a.num_heads;
    decode_reduce_kernel<DT><<<dim3(static_cast<uint32_t>(rgrid)), dim3(256), 0, stream>>>(a);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
  return dtype == 0 ? launch_decode_t<F16>(a, stream) : launch_decode_t<BF16>(a, stream);
}

}  // namespace pkv
