// Work-list planning for paged decode attention: the body run by one
// work-group, shared by decode_plan_kernel (plan.hip) and the fused decode-step
// prologue (step.hip).
//
// A decode work item is one segment (blocks_per_part consecutive blocks) of
// one sequence for one work unit (a KV head, or a 16-head tile of one KV head).
// The plan orders the items so that
//   * the large items come first and the small ones last: every full
//     segment (list A) precedes the sequences' partial last segments
//     (list B), and list B runs from the largest partial sizes to the
//     smallest, so the kernel's tail consists of the shortest items;
//   * parallel samples, which are consecutive sequences with equal lengths and
//     shared prompt blocks, sit next to each other in both lists and are read
//     by neighbouring waves at about the same time;
//   * no empty item exists, so no work-group is dispatched only to exit.
//
// List A, per unit, in the order (segment p, sequence s) over the pairs with
// p < f_s = nblk_s / blocks_per_part.  List B, per class of partial size r =
// nblk_s % blocks_per_part (largest first), the sequences of that class in
// order, then the sequences with an empty context.  The
// positions come from per-(segment, 64-sequence chunk) counts and a prefix
// over chunks; a wave ballot gives each sequence its rank inside a chunk.
//
// A sequence with an empty context gets one item in the last class of list
// B, which writes its defined zero output rows.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace plan_detail {

constexpr int kRBits = 8;  // blocks_per_part <= 256, so a remainder fits 8 bits

// List B classes, in order: partial segments by size, largest first, in
// kSizeBuckets buckets (one size per bucket when blocks_per_part <= 16), then
// the empty sequences (no blocks: their item writes the defined zero output
// row).
constexpr int kSizeBuckets = kPlanClasses / 2;
__device__ inline int num_classes(int bpp) { return (bpp - 1 < kSizeBuckets ? bpp - 1 : kSizeBuckets) + 1; }
__device__ inline int class_of(int r, int bpp) {
  const int nb = num_classes(bpp) - 1;
  return r ? ((bpp - 1 - r) * nb) / (bpp - 1) : nb;
}

// Exclusive prefix sum of x[0..n) in place, by one wave; returns the total.
__device__ inline int wave_exclusive_scan(int* x, int n, int lane) {
  const int per = (n + kWave - 1) / kWave;
  const int lo = min(n, lane * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += x[i];
  // inclusive scan of the lane sums across the wave
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  const int total = __shfl(incl, kWave - 1, kWave);
  int run = incl - sum;
  for (int i = lo; i < hi; ++i) {
    const int v = x[i];
    x[i] = run;
    run += v;
  }
  return total;
}

}  // namespace plan_detail

// One work-group of kThreads threads writes the plan of `a`.  Capacities (LDS
// sizes): kMaxSeqs sequences, kMaxTasks (segment | class, 64-sequence chunk)
// counters, kMaxParts segments per row; the caller checks them.
template <int kThreads, int kMaxSeqs, int kMaxTasks, int kMaxParts>
__device__ inline void plan_body(const PlanArgs& a) {
  constexpr int kPlanWaves = kThreads / kWave;
  __shared__ int fr[kMaxSeqs];            // f << plan_detail::kRBits | r per sequence
  __shared__ int8_t cls[kMaxSeqs];        // list B class per sequence, -1 if none
  __shared__ int hist_f[kMaxParts + 2];  // count of f, then prefix data
  __shared__ int cnt[kMaxTasks];          // per (segment | class, chunk) counts
  __shared__ int cls_off[kPlanClasses + 1];   // partial classes, size descending
  __shared__ int f_max;
  __shared__ int full_total;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int S = a.num_seqs;
  const int bpp = a.blocks_per_part;
  const int cap = a.max_blocks_per_seq;
  const int nch = (S + kWave - 1) / kWave;
  int* list_a = a.plan + kPlanHeaderInts;
  int* list_b = list_a + static_cast<int64_t>(S) * a.parts_max;

  if (a.scan) {
    // At most kThreads sequences: wave w owns the 64-sequence chunk w, so a
    // sequence's rank inside its chunk comes from a ballot in its own wave,
    // with no task loop across waves and four barriers in all.  The same lists
    // and header as below, entry for entry.
    static_assert(kMaxSeqs >= kThreads, "one sequence per thread");
    const int s = tid;
    int f = 0, c = -1;
    if (s < S) {
      const int L = a.context_lens[s] < 0 ? 0 : a.context_lens[s];
      const int nblk = min((L + kBlockSize - 1) / kBlockSize, cap);
      f = nblk / bpp;
      const int r = nblk - f * bpp;
      c = (r || nblk == 0) ? plan_detail::class_of(r, bpp) : -1;
    }
    if (tid == 0) f_max = 0;
    __syncthreads();
    if (s < S && f > 0) atomicMax(&f_max, f);
    const int nclass = plan_detail::num_classes(bpp);
    const uint64_t below = (uint64_t{1} << lane) - 1;
    __syncthreads();
    const int P = f_max;
    // per (key, chunk) counts, key = segment p < P or P + class: the layout of cnt below
    if (wave < nch) {
      for (int p = 0; p < P; ++p) {
        const uint64_t m = __ballot(f > p);
        if (lane == 0) cnt[p * nch + wave] = __popcll(m);
      }
      for (int k = 0; k < nclass; ++k) {
        const uint64_t m = __ballot(c == k);
        if (lane == 0) cnt[(P + k) * nch + wave] = __popcll(m);
      }
    }
    __syncthreads();
    // totals per key and their exclusive prefixes: C_p in hist_f, class offsets in cls_off
    if (wave == 0) {
      for (int p = lane; p < P; p += kWave) {
        int t = 0;
        for (int w = 0; w < nch; ++w) t += cnt[p * nch + w];
        hist_f[p] = t;
      }
      if (lane < nclass) {
        int t = 0;
        for (int w = 0; w < nch; ++w) t += cnt[(P + lane) * nch + w];
        cls_off[lane] = t;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int F = plan_detail::wave_exclusive_scan(hist_f, P, lane);
      if (lane == 0) full_total = F;
    } else if (wave == 1) {
      const int NB = plan_detail::wave_exclusive_scan(cls_off, nclass, lane);
      if (lane == 0) cls_off[nclass] = NB;
    }
    __syncthreads();
    if (wave < nch) {
      for (int p = 0; p < P; ++p) {
        const uint64_t m = __ballot(f > p);
        if (f > p) {
          int pos = hist_f[p] + __popcll(m & below);
          for (int w = 0; w < wave; ++w) pos += cnt[p * nch + w];
          list_a[pos] = s | (p << kPlanSeqBits);
        }
      }
      for (int k = 0; k < nclass; ++k) {
        const uint64_t m = __ballot(c == k);
        if (c == k) {
          int pos = cls_off[k] + __popcll(m & below);
          for (int w = 0; w < wave; ++w) pos += cnt[(P + k) * nch + w];
          list_b[pos] = s;
        }
      }
    }
    if (tid <= kPlanClasses) a.plan[kPlanClassOff + tid] = cls_off[min(tid, nclass)];
    if (tid == 0) {
      a.plan[kPlanFull] = full_total;
      a.plan[kPlanPartial] = cls_off[nclass];
    }
    return;
  }

  // the context lengths are the kernel's longest wait: load them first
  constexpr int kSeqsPerThread = kMaxSeqs / kThreads;
  int lens[kSeqsPerThread];
#pragma unroll
  for (int k = 0; k < kSeqsPerThread; ++k) {
    const int s = tid + k * kThreads;
    lens[k] = s < S ? a.context_lens[s] : 0;
  }
  for (int i = tid; i <= a.parts_max + 1; i += kThreads) hist_f[i] = 0;
  for (int i = tid; i <= kPlanClasses; i += kThreads) cls_off[i] = 0;
  if (tid == 0) f_max = 0;

  __syncthreads();

  // per-sequence segment counts and list B class
#pragma unroll
  for (int k = 0; k < kSeqsPerThread; ++k) {
    const int s = tid + k * kThreads;
    if (s < S) {
      const int L = lens[k] < 0 ? 0 : lens[k];
      const int nblk = min((L + kBlockSize - 1) / kBlockSize, cap);
      const int f = nblk / bpp;
      const int r = nblk - f * bpp;
      fr[s] = (f << plan_detail::kRBits) | r;
      const int c = (r || nblk == 0) ? plan_detail::class_of(r, bpp) : -1;
      cls[s] = static_cast<int8_t>(c);
      atomicAdd(&hist_f[f], 1);
      if (c >= 0) atomicAdd(&cls_off[c], 1);
      atomicMax(&f_max, f);
    }
  }
  __syncthreads();

  const int P = f_max;
  const int nclass = plan_detail::num_classes(bpp);
  // c_p = #{s : f_s > p} = S - #{s : f_s <= p}, and list A offsets C_p = prefix of c_p
  if (wave == 0) plan_detail::wave_exclusive_scan(hist_f, P + 1, lane);  // hist_f[x] = #{s : f_s < x}
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) cnt[p] = S - hist_f[p + 1];
  __syncthreads();
  if (wave == 0) {
    const int F = plan_detail::wave_exclusive_scan(cnt, P, lane);  // cnt[p] = C_p
    if (lane == 0) full_total = F;
  } else if (wave == 1) {
    const int NB = plan_detail::wave_exclusive_scan(cls_off, nclass, lane);
    if (lane == 0) cls_off[nclass] = NB;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) hist_f[p] = cnt[p];  // keep C_p in hist_f
  if (tid <= kPlanClasses) a.plan[kPlanClassOff + tid] = cls_off[min(tid, nclass)];
  if (tid == 0) {
    a.plan[kPlanFull] = full_total;
    a.plan[kPlanPartial] = cls_off[nclass];
  }
  __syncthreads();

  // per (segment, chunk) and (class, chunk) counts
  const int ta = P * nch;
  const int tasks = ta + nclass * nch;
  for (int t = wave; t < tasks; t += kPlanWaves) {
    const int chunk = t % nch;
    const int key = t / nch;
    const int s = chunk * kWave + lane;
    bool pred = false;
    if (s < S) pred = t < ta ? (fr[s] >> plan_detail::kRBits) > key : cls[s] == key - P;
    const uint64_t m = __ballot(pred);
    if (lane == 0) cnt[t] = __popcll(m);
  }
  __syncthreads();
  // exclusive prefix over chunks, one thread per segment index / class
  for (int key = tid; key < P + nclass; key += kThreads) {
    int run = 0;
    for (int c = 0; c < nch; ++c) {
      const int v = cnt[key * nch + c];
      cnt[key * nch + c] = run;
      run += v;
    }
  }
  __syncthreads();
  for (int t = wave; t < tasks; t += kPlanWaves) {
    const int chunk = t % nch;
    const int key = t / nch;
    const int s = chunk * kWave + lane;
    bool pred = false;
    if (s < S) pred = t < ta ? (fr[s] >> plan_detail::kRBits) > key : cls[s] == key - P;
    const uint64_t m = __ballot(pred);
    const int rank = __popcll(m & ((uint64_t{1} << lane) - 1));
    if (pred) {
      if (t < ta)
        list_a[hist_f[key] + cnt[t] + rank] = s | (key << kPlanSeqBits);
      else
        list_b[cls_off[key - P] + cnt[t] + rank] = s;
    }
  }
}

}  // namespace pkv
