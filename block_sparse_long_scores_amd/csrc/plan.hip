// Tile plan of a continuous batch: the (sequence, KV head, query block) tasks
// ordered by their work, longest first, for the persistent attention kernel.
//
// In a batch of prompts of very different lengths (and chunked prefills that
// start deep in a sequence) the work of a task is not a function of its
// query-block index within its sequence, so the order the contiguous path
// uses (last query block first) would start some of the longest tasks last
// and leave the end of the launch to a few CUs.  One workgroup counting-sorts
// the tasks by an estimate of their work, in 32-key chunks: kept blocks x
// (block / 32) + dropped blocks / 32 (the mean-correction pseudo-keys) + 2
// (the fixed cost of a tile).  Ties keep no particular order; the outputs do
// not depend on the order.  The kernel also zeroes the attention launch's
// tile-queue counters, which live in the same caller workspace.
#include "fp2_device.h"
#include "fp2_internal.h"
#include "geometry.h"

namespace fp2 {

constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 4096;  // work estimates are clamped to kPlanBins - 1

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int hist[kPlanBins];
  __shared__ int wsum[kPlanThreads / 64];
  const int tid = threadIdx.x;
  const int per_seq = a.Hkv * a.seq.nqb_stride;
  const int ntask_all = a.seq.batch * per_seq;
  for (int b = tid; b < kPlanBins; b += kPlanThreads) hist[b] = 0;
  // the attention launch that follows on the same stream starts its tile
  // queues from these counters (each on its own 128-byte line)
  if (tid < 8) a.sched[32 * tid] = 0u;
  __syncthreads();

  // work estimate of task t (-1: no query block there)
  auto work = [&](int t) -> int {
    const int s = t / per_seq;
    const int r = t - s * per_seq;
    const int il = r % a.seq.nqb_stride;
    const SeqGeo g = seq_geo(a.seq, s, a.block);
    if (il >= g.nqb) return -1;
    const int i = g.first_qb + il;
    const int kept = a.block_cnt[t];
    const int dropped = a.mean_correction ? (i + 1 - kept) : 0;
    const int w = kept * (a.block / 32) + (dropped + 31) / 32 + 2;
    return w < kPlanBins ? w : kPlanBins - 1;
  };
  for (int t = tid; t < ntask_all; t += kPlanThreads) {
    const int w = work(t);
    if (w >= 0) atomicAdd(&hist[w], 1);
  }
  __syncthreads();

  // exclusive prefix over bins in descending order: bin b starts after every
  // task of a larger estimate.  Thread tid owns bins [4 tid, 4 tid + 4) of the
  // reversed order.
  constexpr int PER = kPlanBins / kPlanThreads;
  int loc[PER];
  int tot = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    loc[k] = hist[kPlanBins - 1 - (PER * tid + k)];
    tot += loc[k];
  }
  const int lane = tid & 63, wv = tid >> 6;
  int incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wv; ++w2) before += wsum[w2];
  int run = before + incl - tot;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int b = kPlanBins - 1 - (PER * tid + k);
    const int c = loc[k];
    hist[b] = run;  // becomes the running cursor of bin b
    run += c;
  }
  if (tid == kPlanThreads - 1) a.plan_count[0] = run;  // all valid tasks
  __syncthreads();

  for (int t = tid; t < ntask_all; t += kPlanThreads) {
    const int w = work(t);
    if (w >= 0) a.plan[atomicAdd(&hist[w], 1)] = t;
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace fp2
