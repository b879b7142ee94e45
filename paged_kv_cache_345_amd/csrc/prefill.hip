// Chunked-prefill paged attention for gfx950: multi-token queries, causal by
// position, on the matrix cores, and the log-sum-exp merge of its segment
// partials.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Chunked prefill on the matrix cores.  A work-group takes 8 tiles of 16
// (query position, head) rows of one KV head, two tiles per wave, and streams
// the blocks of its segment in steps of kStageBlocks blocks.  Each step's K
// and V pages go straight from the cache into LDS (buffer loads with the LDS
// destination bit), kStageBufs - 1 steps ahead of the one being computed, and
// every wave reads its fragments from there for both of its tiles.  Per step
// and tile: S = K Q^T (16x16x32 products), one online-softmax update over the
// step's keys (the causal mask by row position is evaluated only in steps
// that reach past some row's position; the other steps keep a lazy softmax
// reference that moves only when a score passes it by 2^8), then O += P V
// (16x16x32 products over the step's two blocks).
// A block wholly past every position of a wave is skipped by that wave.  Each
// wave writes its own rows.
//
// The step loads are issued from inline assembly: with the compiler's own LDS
// loads, it waits for every load in flight before each LDS read and each
// barrier, which leaves no load ahead of the step being computed (measured on
// MI355X: staging one step ahead through registers instead gave 1.6x longer
// calls on both prefill batches).  The kernel therefore keeps the vector-memory
// counter itself: no other vector memory access happens in the step loop
// (block ids are scalar loads, q is taken before the loop), each wave waits
// for its own loads of the next step, and the work-group barrier follows.
// M0, which the loads take their LDS address from, has no other use in this
// kernel's code.
// ---------------------------------------------------------------------------

// Step geometry, measured on MI355X over both prefill batches and the
// prefix-cached admission: 2-block steps with 3 buffers (48 KiB of LDS, at
// most 168 VGPRs, so 3 work-groups per compute unit) against 2 per unit with 4 buffers:
// 7%, 13% and 19% shorter calls; 1-block steps or 4-block steps, 4 tiles per
// wave (1 work-group per unit) and 1 tile per wave (4 per unit) were slower.
constexpr int kStageBlocks = 2;  // blocks per LDS step
constexpr int kStageBufs = 3;    // LDS step buffers: up to kStageBufs - 1 steps in flight
constexpr int kPrefillGroupsPerCu = 3;
// Lazy softmax reference of the mask-free update: 2^8 bounds P well inside the
// 16-bit range of its operand (fp16 max 65504).
constexpr float kLazyShift = 8.f;

// Blocks that the work-group holding chunk query qi streams: up to the block
// of its last query's position.  Shared by the prefill kernel and its reduce.
__device__ inline int prefill_wg_blocks(const PrefillArgs& pa, int L, int C, int qi) {
  const int per_wg = kWavesPerGroup * kPrefillTiles * pa.pos_per_wave;
  const int last_q = min(C, (qi / per_wg + 1) * per_wg) - 1;
  return (L - C + last_q) / kBlockSize + 1;
}

// Work order.  Work-groups differ in length by the number of blocks they
// stream, and about three rounds of them fill the chip, so the dispatch order
// decides how long the last ones run alone.  Up to kPrefillSortSeqs sequences,
// each unit's sequences go out longest first: a group is (unit, sequence)
// with its q_blocks x parts_max items (latest query block first, so the
// longest item of the group leads), groups run in the order (unit, sequences
// by block count descending, ties by index), and the XCDs take 8 contiguous
// chunks of that order.  An XCD thus works on one or two units at a time, and
// sequences that share prompt blocks read the shared pages in one L2 at about
// the same time (dealing consecutive groups to different XCDs instead put
// five units on each XCD at once and made a batch of prompts that share a
// 1024-token prefix 9% slower).  Longer batches keep the plain order (unit,
// sequence, query block, segment) in 8 contiguous XCD chunks.
constexpr int kPrefillSortSeqs = 256;

__host__ __device__ inline int64_t prefill_grid(const PrefillArgs& pa) {
  const DecodeArgs& a = pa.d;
  const int64_t per_group = static_cast<int64_t>(pa.q_blocks) * a.parts_max;
  const int64_t groups = static_cast<int64_t>(a.units) * a.num_seqs;
  if (a.num_seqs <= kPrefillSortSeqs) return (groups + kNumXcd - 1) / kNumXcd * per_group * kNumXcd;
  return (groups * per_group + kNumXcd - 1) / kNumXcd * kNumXcd;
}

// The item of this work-group in the longest-first order: false when the
// work-group has none (uniform).  Every thread of the work-group calls it.
__device__ inline bool prefill_sorted_item(const PrefillArgs& pa, int& g, int& qb, int& s, int& u) {
  const DecodeArgs& a = pa.d;
  __shared__ __attribute__((aligned(16))) int keys[kPrefillSortSeqs];
  __shared__ int pick;
  const int S = a.num_seqs;
  const int per_group = pa.q_blocks * a.parts_max;
  const int64_t groups = static_cast<int64_t>(S) * a.units;
  const int64_t per_xcd = (groups + kNumXcd - 1) / kNumXcd;  // groups per XCD chunk
  const int64_t xcd = blockIdx.x % kNumXcd;
  const int i = static_cast<int>(blockIdx.x / kNumXcd);      // item index within the XCD's chunk
  if (i / per_group >= per_xcd) return false;
  const int64_t group = xcd * per_xcd + i / per_group;
  if (group >= groups) return false;
  u = static_cast<int>(group / S);
  const int rank = static_cast<int>(group % S);
  const int m = i % per_group;
  qb = pa.q_blocks - 1 - m / a.parts_max;
  g = m % a.parts_max;
  // sort key of sequence t: blocks of its key range (0 without a chunk);
  // slots S .. 4 ceil(S/4) - 1 hold -1, which no sequence ranks behind
  const int t = threadIdx.x;
  int key = -1;
  if (t < S) {
    const int Lt = clamped_len(a, t);
    const int q0t = pa.query_start[t];
    const int Ct = min(max(pa.query_start[t + 1] - q0t, 0), Lt);
    key = Ct > 0 ? (Lt - 1) / kBlockSize + 1 : 0;
  }
  if (t < ((S + 3) & ~3)) keys[t] = key;
  if (t == 0) pick = 0;
  __syncthreads();
  // rank of sequence t: the sequences with a larger key, or an equal key and
  // a lower index, come first; the ranks are a permutation of 0 .. S-1
  if (t < S) {
    int r = 0;
    for (int j = 0; j < S; j += 4) {
      const int4 k4 = *reinterpret_cast<const int4*>(&keys[j]);
      r += (k4.x > key) | ((k4.x == key) & (j + 0 < t));
      r += (k4.y > key) | ((k4.y == key) & (j + 1 < t));
      r += (k4.z > key) | ((k4.z == key) & (j + 2 < t));
      r += (k4.w > key) | ((k4.w == key) & (j + 3 < t));
    }
    if (r == rank) pick = t;
  }
  __syncthreads();
  s = pick;
  return true;
}

// Fragment reads from a page copy in LDS, in the page formats' register layout
// (lane l's 16 bytes of wave load i sit at byte 1024 i + 16 l of the page).
template <class PF>
struct LdsPage;
template <>
struct LdsPage<Page16> {
  __device__ static inline void k(const char* pg, int lane, uint4 (&kv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kv[i] = *reinterpret_cast<const uint4*>(pg + 1024 * i + 16 * lane);
  }
  __device__ static inline void v(const char* pg, int lane, uint4 (&vv)[4]) { k(pg, lane, vv); }
  // V fragments 2 h and 2 h + 1
  __device__ static inline void v_half(const char* pg, int lane, int h, uint4& f0, uint4& f1) {
    f0 = *reinterpret_cast<const uint4*>(pg + 2048 * h + 16 * lane);
    f1 = *reinterpret_cast<const uint4*>(pg + 2048 * h + 1024 + 16 * lane);
  }
};
template <class DT>
struct LdsPage<PageFp8<DT>> {
  __device__ static inline void k(const char* pg, int lane, uint4 (&kv)[4]) {
    const uint4 w0 = *reinterpret_cast<const uint4*>(pg + 16 * lane);
    const uint4 w1 = *reinterpret_cast<const uint4*>(pg + 1024 + 16 * lane);
    PageFp8<DT>::widen(w0, kv[0], kv[1]);
    PageFp8<DT>::widen(w1, kv[2], kv[3]);
  }
  __device__ static inline void v(const char* pg, int lane, uint4 (&vv)[4]) { k(pg, lane, vv); }
  __device__ static inline void v_half(const char* pg, int lane, int h, uint4& f0, uint4& f1) {
    PageFp8<DT>::widen(*reinterpret_cast<const uint4*>(pg + 1024 * h + 16 * lane), f0, f1);
  }
};

// s_waitcnt vmcnt(min(n, kMax) * kPerStep): at most n steps of kPerStep loads
// each still in flight (the count must be an immediate)
template <int kPerStep, int kMax>
__device__ __attribute__((always_inline)) inline void wait_vm_steps(int n) {
  if constexpr (kMax > 0) {
    if (n >= kMax) {
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kMax * kPerStep) : "memory");
      return;
    }
    wait_vm_steps<kPerStep, kMax - 1>(n);
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

template <class DT, class PF>
__global__ __launch_bounds__(256, kPrefillGroupsPerCu) void prefill_kernel(PrefillArgs pa) {
  constexpr int kPage = PF::kPageBytes;
  constexpr int kPieces = kPage / 1024;                          // 1 KiB wave loads per page
  constexpr int kLoads = 2 * kStageBlocks * kPieces / kWavesPerGroup;  // wave loads per wave per step
  __shared__ __attribute__((aligned(16))) char lds[kStageBufs][2][kStageBlocks][kPage];  // [buffer][K, V][block]

  const DecodeArgs& a = pa.d;
  int g, qb, s, u;  // item: segment, query block, sequence, unit
  if (a.num_seqs <= kPrefillSortSeqs) {
    if (!prefill_sorted_item(pa, g, qb, s, u)) return;  // uniform over the work-group
  } else {
    // (unit, sequence, query block, segment), segment fastest, in XCD-aware
    // chunks as in decode's direct mode
    const int64_t total = static_cast<int64_t>(a.units) * a.num_seqs * pa.q_blocks * a.parts_max;
    const int64_t per_xcd = (total + kNumXcd - 1) / kNumXcd;
    const int64_t lam = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
    if (lam >= total) return;  // uniform over the work-group
    g = static_cast<int>(lam % a.parts_max);
    int64_t rest = lam / a.parts_max;
    qb = static_cast<int>(rest % pa.q_blocks);
    rest /= pa.q_blocks;
    s = static_cast<int>(rest % a.num_seqs);
    u = static_cast<int>(rest / a.num_seqs);
  }
  const int kvh = u / a.head_tiles;
  const int tile = u - kvh * a.head_tiles;
  const int h0 = kvh * a.group + tile * 16;
  const int nh = min(pa.heads_per_tile, a.group - tile * 16);

  const int L = clamped_len(a, s);
  const int q0 = pa.query_start[s];
  const int C = min(max(pa.query_start[s + 1] - q0, 0), L);
  const int ppt = pa.pos_per_wave;
  const int wg_q0 = qb * kWavesPerGroup * kPrefillTiles * ppt;
  if (wg_q0 >= C) return;  // uniform over the work-group
  const int nblk = prefill_wg_blocks(pa, L, C, wg_q0);
  const int nseg = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  if (g >= nseg) return;  // uniform over the work-group
  const int j0 = g * a.blocks_per_part;
  const int nb = min(a.blocks_per_part, nblk - j0);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int hpt = pa.heads_per_tile;
  // row r of tile T of this wave: position index r / hpt, head index r % hpt
  auto row_query = [&](int T, int r) { return wg_q0 + (kPrefillTiles * wave + T) * ppt + r / hpt; };
  auto row_valid = [&](int T, int r) { return r / hpt < ppt && r % hpt < nh && row_query(T, r) < C; };
  int pos[kPrefillTiles];  // position of row col of each tile; -1: no query (every key masked)
#pragma unroll
  for (int T = 0; T < kPrefillTiles; ++T) pos[T] = row_valid(T, col) ? L - C + row_query(T, col) : -1;
  // the wave's position range over its valid rows (wave-uniform)
  int hi_pos = max(pos[0], pos[kPrefillTiles - 1]);
  int lo_pos = pos[0] >= 0 ? pos[0] : 0x7fffffff;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    hi_pos = max(hi_pos, __shfl_xor(hi_pos, d, kWave));
    lo_pos = min(lo_pos, __shfl_xor(lo_pos, d, kWave));
  }

  float m[kPrefillTiles], z[kPrefillTiles];
  float4_t O[kPrefillTiles][8];
  uint4 qf[kPrefillTiles][4];
#pragma unroll
  for (int T = 0; T < kPrefillTiles; ++T) {
    m[T] = kInitMax;
    z[T] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) O[T][j] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (pos[T] >= 0) {
      const uint4* qrow = reinterpret_cast<const uint4*>(
          a.q + (static_cast<int64_t>(q0 + row_query(T, col)) * a.num_heads + h0 + col % hpt) * kHeadSize);
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[T][i] = qrow[4 * i + grp];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[T][i] = make_uint4(0, 0, 0, 0);
    }
  }
  // Take the q loads' results here: the step loads below go to LDS behind the
  // compiler's back, and a wait for q left inside the loop would also wait for
  // every step load in flight.
#pragma unroll
  for (int T = 0; T < kPrefillTiles; ++T)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      asm volatile("" : "+v"(qf[T][i].x), "+v"(qf[T][i].y), "+v"(qf[T][i].z), "+v"(qf[T][i].w));
  // A negative scale is carried by the queries: with q negated (sign bits
  // flipped, exact) the scores change sign exactly, and S sc = (-S)(-sc), so
  // every logit keeps its bits while the scale the steps use is >= 0 and the
  // row maximum of the logits is sc times the row maximum of the scores.
  const float sl2e = head_logit_scale(a, kvh);
  const bool neg_scale = sl2e < 0.f;
  const float sc = neg_scale ? -sl2e : sl2e;
  if (neg_scale) {
#pragma unroll
    for (int T = 0; T < kPrefillTiles; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qf[T][i].x ^= 0x80008000u;
        qf[T][i].y ^= 0x80008000u;
        qf[T][i].z ^= 0x80008000u;
        qf[T][i].w ^= 0x80008000u;
      }
  }

  // step loads, straight from the cache into LDS: wave w loads page w of the
  // step (the K pages of its blocks first, then the V pages) as kLoads 1 KiB
  // pieces; lane l's 16 bytes of piece i land at byte 1024 i + 16 l of the copy
  const int32_t* brow = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq + j0;
  const int64_t page_stride = static_cast<int64_t>(a.num_kv_heads) * kPage;
  const int64_t head_off = static_cast<int64_t>(kvh) * kPage;
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  static_assert(kLoads == kPieces, "each wave loads one whole page per step");
  // waves 0, 1: the K pages of the step's blocks; waves 2, 3: the V pages
  const char* const cache_base = (wave < kStageBlocks ? kc : vc) + head_off;
  const int wave_blk = wave % kStageBlocks;  // the step's block this wave loads
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int jj = st * kStageBlocks + wave_blk;
    // block id by a scalar load (the asm memory clobbers below keep the
    // compiler from proving the table unchanged, so it would use a vector
    // load and a wait that also drains the step loads in flight)
    int bid;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=s"(bid) : "s"(brow + min(jj, nb - 1)) : "memory");
    const bool bad = jj >= nb || static_cast<unsigned>(bid) >= static_cast<unsigned>(a.num_blocks);
    const __amdgpu_buffer_rsrc_t r =
        range_rsrc(cache_base + (bad ? 0 : bid) * page_stride, bad ? 0 : kPage);  // a bad id reads zeros
    // LDS byte address of the page copy (the low 32 bits of its generic address)
    const uint32_t dst = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>(&lds[st % kStageBufs][wave / kStageBlocks][wave_blk][0])));
    // Every page load takes the default cache policy.  Unlike decode, where a
    // page is read once, the work-groups of the other query blocks of the same
    // sequence and head read the same pages at about the same time, and a
    // non-temporal hint on the K pages (decode's split) cost those re-reads
    // their L2 hits (measured on MI355X, LLaMA-13B-shaped prefill batch: L2
    // hit rate 52% -> 62%, HBM reads 1.62 -> 1.27 GB, 6.5% shorter calls; GQA
    // and fp8 batches 4%).  Load i goes to LDS (lane l's 16 bytes at dst +
    // 1024 i + 16 l) and is counted by the vector-memory counter, which
    // wait_steps below checks.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is written here and read by nothing else
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(dst + 1024u * i), "v"(1024u * i + 16u * lane), "s"(r) : "memory", "m0");
#pragma clang diagnostic pop
  };
  // Work-group barrier between steps.  Before it each wave has waited for its
  // own loads of the step about to be read (wait_steps) and for its own LDS
  // reads (their data is consumed before the barrier, and the buffer they read
  // is refilled after it).  __syncthreads() would also drain every load still
  // in flight for the later steps.
  auto step_barrier = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // wait until at most n steps' loads of this wave are still in flight
  auto wait_steps = [&](int n) __attribute__((always_inline)) {
    wait_vm_steps<kLoads, kStageBufs - 2>(n);
  };

  const uint32_t ones = DT::pack2(1.f, 1.f);
  // One step over blocks jstep .. jstep + n - 1 (n >= 1, wave-uniform).  kFast:
  // n == kStageBlocks and every valid row of the wave sees every key, so no
  // mask is evaluated (rows without a query compute garbage they never write).
  auto step = [&]<bool kFast>(int buf, int jstep, int n) __attribute__((always_inline)) {
    float4_t S[kPrefillTiles][kStageBlocks];
#pragma unroll
    for (int b = 0; b < kStageBlocks; ++b) {
#pragma unroll
      for (int T = 0; T < kPrefillTiles; ++T) S[T][b] = float4_t{0.f, 0.f, 0.f, 0.f};
      if (kFast || b < n) {
        uint4 kv[4];
        LdsPage<PF>::k(lds[buf][0][b], lane, kv);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int T = 0; T < kPrefillTiles; ++T) S[T][b] = DT::mfma_qk(kv[i], qf[T][i], S[T][b]);
        }
      }
    }

    uint2 P[kPrefillTiles][kStageBlocks];
    float alpha[kPrefillTiles];
    // O[T] *= alpha of its rows when some row's reference moved (alpha == 1
    // exactly otherwise); the alpha of row c sits in lane c, and lane (grp, col)
    // holds rows 4 grp .. 4 grp + 3
    auto rescale = [&](int T) __attribute__((always_inline)) {
      if (__ballot(alpha[T] != 1.f) == 0) return;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = lane_from(alpha[T], 4 * grp + r);
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[T][jd][r] *= ar[r];
      }
    };
    if (kFast) {
      // Lazy reference: a row's m moves only when the row maximum of the step
      // passes it by more than kLazyShift (log2 units), so P = 2^(x - m) stays
      // below 2^kLazyShift and O is rescaled rarely; O, z and m keep their
      // meaning.  Each lane first tests its own 8 scores (sc >= 0: the max of
      // S sc is sc times the max of S); only when some lane of the wave passes
      // is the row maximum reduced across the 4 rows and the reference moved.
      float e[kPrefillTiles];
#pragma unroll
      for (int T = 0; T < kPrefillTiles; ++T) {
        e[T] = S[T][0][0];
#pragma unroll
        for (int b = 0; b < kStageBlocks; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) e[T] = fmaxf(e[T], S[T][b][r]);
      }
      bool pass = false;
#pragma unroll
      for (int T = 0; T < kPrefillTiles; ++T) {
        alpha[T] = 1.f;
        pass |= e[T] * sc > m[T] + kLazyShift;
      }
      if (__ballot(pass) != 0) {  // rare: one branch for both tiles keeps the common path straight
#pragma unroll
        for (int T = 0; T < kPrefillTiles; ++T) {
          const float mx = cross_row_max(e[T]) * sc;
          const bool move = mx > m[T] + kLazyShift;
          alpha[T] = move ? exp2_fast(m[T] - mx) : 1.f;
          m[T] = move ? mx : m[T];
          rescale(T);
        }
      }
#pragma unroll
      for (int T = 0; T < kPrefillTiles; ++T) {
        const float neg = -m[T];
        float zs = 0.f;
#pragma unroll
        for (int b = 0; b < kStageBlocks; ++b) {
          P[T][b].x = DT::pack2(exp2_fast(fmaf(S[T][b][0], sc, neg)), exp2_fast(fmaf(S[T][b][1], sc, neg)));
          P[T][b].y = DT::pack2(exp2_fast(fmaf(S[T][b][2], sc, neg)), exp2_fast(fmaf(S[T][b][3], sc, neg)));
          zs = DT::dot2(P[T][b].x, ones, zs);
          zs = DT::dot2(P[T][b].y, ones, zs);
        }
        z[T] = fmaf(z[T], alpha[T], zs);
      }
    } else {
#pragma unroll
      for (int T = 0; T < kPrefillTiles; ++T) {
        float x[kStageBlocks][4];
        float bm = kMaskedLogit;
#pragma unroll
        for (int b = 0; b < kStageBlocks; ++b) {
          const int t0 = (jstep + b) * kBlockSize + 4 * grp;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[b][r] = b < n && t0 + r <= pos[T] ? S[T][b][r] * sc : kMaskedLogit;
            bm = fmaxf(bm, x[b][r]);
          }
        }
        bm = cross_row_max(bm);
        const float m_new = fmaxf(m[T], bm);
        alpha[T] = exp2_fast(m[T] - m_new);
        float zs = 0.f;
#pragma unroll
        for (int b = 0; b < kStageBlocks; ++b) {
          P[T][b].x = DT::pack2(exp2_fast(x[b][0] - m_new), exp2_fast(x[b][1] - m_new));
          P[T][b].y = DT::pack2(exp2_fast(x[b][2] - m_new), exp2_fast(x[b][3] - m_new));
          zs = DT::dot2(P[T][b].x, ones, zs);
          zs = DT::dot2(P[T][b].y, ones, zs);
        }
        m[T] = m_new;
        z[T] = fmaf(z[T], alpha[T], zs);
      }
    }
    if (!kFast) {
#pragma unroll
      for (int T = 0; T < kPrefillTiles; ++T) rescale(T);
    }

    // O += P V over both blocks of the step in one 16x16x32 product per
    // (tile, 16 dims): lane (grp, col) gives k slots 8 grp .. 8 grp + 3 to
    // tokens 4 grp .. 4 grp + 3 of the first block and k slots 8 grp + 4 ..
    // 8 grp + 7 to the same tokens of the second, in P and in V alike.  A block
    // outside the step's live prefix has P = 0 and V = 0 (its LDS copy may hold
    // stale slots of the sequence's last block, NaN included).
    static_assert(kStageBlocks == 2, "one 16x16x32 product spans the step's two blocks");
    // word masks of the V fragments (mask_v's): stale slots past the context and
    // a dead second block read as zeros
    uint32_t mk01[kStageBlocks], mk23[kStageBlocks];
#pragma unroll
    for (int b = 0; b < kStageBlocks; ++b) {
      const int nvalid = (kFast || b < n) ? L - (jstep + b) * kBlockSize : 0;
      const int t0 = 4 * grp;
      mk01[b] = (kFast || t0 + 0 < nvalid ? 0x0000ffffu : 0u) | (kFast || t0 + 1 < nvalid ? 0xffff0000u : 0u);
      mk23[b] = (kFast || t0 + 2 < nvalid ? 0x0000ffffu : 0u) | (kFast || t0 + 3 < nvalid ? 0xffff0000u : 0u);
    }
    uint4 pk[kPrefillTiles];  // P of both blocks in the k-slot order above
#pragma unroll
    for (int T = 0; T < kPrefillTiles; ++T) pk[T] = make_uint4(P[T][0].x, P[T][0].y, P[T][1].x, P[T][1].y);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 f[kStageBlocks][2];
#pragma unroll
      for (int b = 0; b < kStageBlocks; ++b) {
        LdsPage<PF>::v_half(lds[buf][1][b], lane, h, f[b][0], f[b][1]);
        if (!kFast) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            f[b][e].x &= mk01[b];
            f[b][e].y &= mk23[b];
            f[b][e].z &= mk01[b];
            f[b][e].w &= mk23[b];
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jd = 4 * h + jj;
        const uint4& f0 = f[0][jj >> 1];
        const uint4& f1 = f[1][jj >> 1];
        const uint4 bv = (jj & 1) ? make_uint4(f0.z, f0.w, f1.z, f1.w) : make_uint4(f0.x, f0.y, f1.x, f1.y);
#pragma unroll
        for (int T = 0; T < kPrefillTiles; ++T) O[T][jd] = DT::mfma_pv32(pk[T], bv, O[T][jd]);
      }
    }
  };

  const int nsteps = (nb + kStageBlocks - 1) / kStageBlocks;
  // The mask-free steps form a prefix of the segment: step st is one exactly
  // when its kStageBlocks blocks all lie in the segment and below the wave's
  // first position, j0 + (st + 1) kStageBlocks <= (lo_pos + 1) / 16 (which
  // also puts them below its last one).  Counted once.
  const int fast_steps =
      hi_pos < 0 ? 0 : min(nb / kStageBlocks, max(0, (min(lo_pos, 0x7ffffff0) + 1) / kBlockSize - j0) / kStageBlocks);
  for (int st = 0; st < min(nsteps, kStageBufs - 1); ++st) issue(st);
  wait_steps(min(nsteps, kStageBufs - 1) - 1);
  step_barrier();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st % kStageBufs;
    // the buffer of step st + kStageBufs - 1 was last read in step st - 1, before the barrier that ended it
    if (st + kStageBufs - 1 < nsteps) issue(st + kStageBufs - 1);

    const int jstep = j0 + st * kStageBlocks;
    if (st < fast_steps) {
      step.template operator()<true>(buf, jstep, kStageBlocks);
    } else {
      // live blocks of the step for this wave: a prefix (the step's blocks
      // inside the segment, up to the wave's last position)
      const int nlive =
          hi_pos < 0 ? 0 : max(0, min(min(kStageBlocks, nb - st * kStageBlocks), hi_pos / kBlockSize - jstep + 1));
      if (nlive > 0) step.template operator()<false>(buf, jstep, nlive);
    }

    if (st + 1 < nsteps) {
      // step st + 1 landed; the steps after it that were issued may stay in flight
      wait_steps(min(nsteps - 1, st + kStageBufs - 1) - (st + 1));
      step_barrier();
    }
  }

  // O[T][jd][r]: row 4grp + r, dim 16 jd + col; lane c (< 16) holds row c's max and sum
#pragma unroll
  for (int T = 0; T < kPrefillTiles; ++T) {
    const float Zc = cross_row_sum(z[T]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 4 * grp + r;
      const float Zr = lane_from(Zc, tr);
      const float mr = lane_from(m[T], tr);
      if (!row_valid(T, tr)) continue;
      const int64_t orow = static_cast<int64_t>(q0 + row_query(T, tr)) * a.num_heads + h0 + tr % hpt;
      if (nseg == 1) {
        uint16_t* dst = a.out + orow * kHeadSize + col;
        const float inv = head_out_scale(a, kvh) / Zr;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) dst[16 * jd] = DT::from_f32(O[T][jd][r] * inv);
      } else {
        const int64_t slot = orow * a.parts_max + g;
        float* dst = a.ws_o + slot * kHeadSize + col;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) dst[16 * jd] = O[T][jd][r];
        if (col == 0) {
          a.ws_ml[2 * slot] = mr;
          a.ws_ml[2 * slot + 1] = Zr;
        }
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
  if (qi >= C || qi >= pa.q_blocks * kWavesPerGroup * kPrefillTiles * pa.pos_per_wave) return;
  const int nblk = prefill_wg_blocks(pa, L, C, qi);
  const int n = (nblk + a.blocks_per_part - 1) / a.blocks_per_part;
  if (n <= 1) return;  // written directly by the prefill kernel
  const int64_t base = row * a.parts_max;
  const int kvh = static_cast<int>(row % a.num_heads) / a.group;
  lse_merge_row<DT>(a.ws_ml + 2 * base, a.ws_o + base * kHeadSize, n, a.out + row * kHeadSize,
                    head_out_scale(a, kvh), threadIdx.x & (kWave - 1));
}

template <class DT, class PF>
static hipError_t launch_prefill_t(const PrefillArgs& pa, hipStream_t stream) {
  const DecodeArgs& a = pa.d;
  const int64_t grid = prefill_grid(pa);
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
