// Work-list planning for paged decode attention (one work-group, 1024 threads).
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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
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
__device__ int wave_exclusive_scan(int* x, int n, int lane) {
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

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(PlanArgs a) {
  __shared__ int fr[kPlanMaxSeqs];            // f << kRBits | r per sequence
  __shared__ int8_t cls[kPlanMaxSeqs];        // list B class per sequence, -1 if none
  __shared__ int hist_f[kMaxPartitions + 2];  // count of f, then prefix data
  __shared__ int cnt[kPlanMaxTasks];          // per (segment | class, chunk) counts
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

  // the context lengths are the kernel's longest wait: load them first
  constexpr int kSeqsPerThread = kPlanMaxSeqs / kPlanThreads;
  int lens[kSeqsPerThread];
#pragma unroll
  for (int k = 0; k < kSeqsPerThread; ++k) {
    const int s = tid + k * kPlanThreads;
    lens[k] = s < S ? a.context_lens[s] : 0;
  }
  for (int i = tid; i <= a.parts_max + 1; i += kPlanThreads) hist_f[i] = 0;
  for (int i = tid; i <= kPlanClasses; i += kPlanThreads) cls_off[i] = 0;
  if (tid == 0) f_max = 0;

  __syncthreads();

  // per-sequence segment counts and list B class
#pragma unroll
  for (int k = 0; k < kSeqsPerThread; ++k) {
    const int s = tid + k * kPlanThreads;
    if (s < S) {
      const int L = lens[k] < 0 ? 0 : lens[k];
      const int nblk = min((L + kBlockSize - 1) / kBlockSize, cap);
      const int f = nblk / bpp;
      const int r = nblk - f * bpp;
      fr[s] = (f << kRBits) | r;
      const int c = (r || nblk == 0) ? class_of(r, bpp) : -1;
      cls[s] = static_cast<int8_t>(c);
      atomicAdd(&hist_f[f], 1);
      if (c >= 0) atomicAdd(&cls_off[c], 1);
      atomicMax(&f_max, f);
    }
  }
  __syncthreads();

  const int P = f_max;
  const int nclass = num_classes(bpp);
  // c_p = #{s : f_s > p} = S - #{s : f_s <= p}, and list A offsets C_p = prefix of c_p
  if (wave == 0) wave_exclusive_scan(hist_f, P + 1, lane);  // hist_f[x] = #{s : f_s < x}
  __syncthreads();
  for (int p = tid; p < P; p += kPlanThreads) cnt[p] = S - hist_f[p + 1];
  __syncthreads();
  if (wave == 0) {
    const int F = wave_exclusive_scan(cnt, P, lane);  // cnt[p] = C_p
    if (lane == 0) full_total = F;
  } else if (wave == 1) {
    const int NB = wave_exclusive_scan(cls_off, nclass, lane);
    if (lane == 0) cls_off[nclass] = NB;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kPlanThreads) hist_f[p] = cnt[p];  // keep C_p in hist_f
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
    if (s < S) pred = t < ta ? (fr[s] >> kRBits) > key : cls[s] == key - P;
    const uint64_t m = __ballot(pred);
    if (lane == 0) cnt[t] = __popcll(m);
  }
  __syncthreads();
  // exclusive prefix over chunks, one thread per segment index / class
  for (int key = tid; key < P + nclass; key += kPlanThreads) {
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
    if (s < S) pred = t < ta ? (fr[s] >> kRBits) > key : cls[s] == key - P;
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

}  // namespace

hipError_t launch_decode_plan(const PlanArgs& a, hipStream_t stream) {
  decode_plan_kernel<<<dim3(1), dim3(kPlanThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
