// Pattern discovery and max-based dynamic thresholding on gfx950.
//
// Source: "FlashPrefill V2: block-sparse prefill attention for long-context LLM
// serving", abstract (instantaneous pattern discovery, max-based dynamic
// thresholding, mean correction), and the papers.ananclaw.com explainer §2.1
// (Supp(q), the dropped blocks' average value).  Pattern discovery is read as
// block mean-pooling with unscaled pooled-Q . pooled-K block scores; a key
// block is kept when its score is at least the row maximum minus tau, and the
// sink block 0 and the diagonal block are always kept.
//
// pool_kernel   : one workgroup per query block (all KV groups at once) or
//                 per key block (K and V at once).  Streams the rows once from
//                 HBM with 16-byte coalesced loads, accumulates in fp32.
// select_kernel : one workgroup per (sequence, KV head, run of query blocks).
//                 Scores every visible key block against the run's pooled
//                 queries, reduces each row's maximum across the wavefront and
//                 compacts the kept blocks into an ascending index list with
//                 a ballot prefix count.
#include "fp2_device.h"
#include "fp2_internal.h"
#include "geometry.h"

#include <algorithm>

namespace fp2 {

constexpr int kPoolThreads = 256;
constexpr int kMaxChunksPerThread = 4;
static_assert(kPoolThreads * kMaxChunksPerThread == kPoolMaxTasks, "pool task capacity");

// Accumulate one 16-byte chunk of a row into acc[EPC] (fp32).
template <int ESZ>
__device__ __forceinline__ void acc_chunk(float* acc, const uint4& w) {
  if constexpr (ESZ == 2) {
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float lo, hi;
      unpack_bf16x2(ws[e], lo, hi);
      acc[2 * e] += lo;
      acc[2 * e + 1] += hi;
    }
  } else {
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[4 * e + b] += fp8_byte_to_f32(ws[e], b);
    }
  }
}

// NC: 16-byte chunk slots per thread (a row of W elements is W / EPC chunks
// over kPoolThreads threads), chosen at launch from the head counts so that
// no register is held for slots no thread uses; rows are loaded in groups of
// kRows (fewer when more slots are live), every load of a group in flight
// before the first is added, in row order.
template <int ESZ, int NC>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolArgs a) {
  constexpr int kRows = NC == 1 ? 8 : NC == 2 ? 4 : 2;
  constexpr int EPC = 16 / ESZ;  // elements per 16-byte chunk
  extern __shared__ float red[];
  const int s = blockIdx.y;
  const SeqGeo g = seq_geo(a.seq, s, a.block);
  const int t = threadIdx.x;
  const int x = blockIdx.x;
  const int D = a.D;

  if (x < a.seq.nqb_stride) {
    // ---- query block: mean over the G heads of each group and the rows present
    const int il = x;
    if (il >= g.nqb) return;
    const int i = g.first_qb + il;
    const int r0 = max(i * a.block, g.P) - g.P;
    const int r1 = min((i + 1) * a.block, g.Sk) - g.P;
    const int W = a.Hq * D;
    const int nch = W / EPC;
    const char* base = (const char*)a.q + (long)(g.qrow0 + r0) * W * ESZ;
    float acc[NC][EPC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[c][e] = 0.f;
    const int nr = r1 - r0;
    int r = 0;
    for (; r + kRows <= nr; r += kRows) {
      uint4 w[kRows][NC];
#pragma unroll
      for (int u = 0; u < kRows; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          int ch = t + c * kPoolThreads;
          if (ch < nch) w[u][c] = *(const uint4*)(base + (long)(r + u) * W * ESZ + ch * 16);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kRows; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (t + c * kPoolThreads < nch) acc_chunk<ESZ>(acc[c], w[u][c]);
    }
    for (; r < nr; ++r) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        int ch = t + c * kPoolThreads;
        if (ch < nch) acc_chunk<ESZ>(acc[c], *(const uint4*)(base + (long)r * W * ESZ + ch * 16));
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      int ch = t + c * kPoolThreads;
      if (ch < nch) {
        int e0 = ch * EPC;
        float sc = (ESZ == 1) ? a.q_scale[e0 / D] : 1.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) red[e0 + e] = acc[c][e] * sc;
      }
    }
    __syncthreads();
    if (a.select_mode != 0) {  // union and head-max selection: one mean per query head
      const float inv1 = 1.f / (float)nr;
      for (int o = t; o < a.Hq * D; o += kPoolThreads) {
        const int hq = o / D, dd = o - hq * D;
        a.qbar[(((long)s * a.Hq + hq) * a.seq.nqb_stride + il) * D + dd] = red[o] * inv1;
      }
      return;
    }
    const int G = a.Hq / a.Hkv;
    const float inv = 1.f / (float)(G * nr);
    for (int o = t; o < a.Hkv * D; o += kPoolThreads) {
      int h = o / D, dd = o - h * D;
      float sum = 0.f;
      for (int gg = 0; gg < G; ++gg) sum += red[(h * G + gg) * D + dd];
      a.qbar[(((long)s * a.Hkv + h) * a.seq.nqb_stride + il) * D + dd] = sum * inv;
    }
    return;
  }

  // ---- key block: means of K and V over the keys of block j
  const int j = x - a.seq.nqb_stride;
  if (j >= g.nkb) return;
  const int c0 = j * a.block;
  const int c1 = min(c0 + a.block, g.Sk);
  const int W = a.Hkv * D;
  const int nch = W / EPC;
  const int ntask = a.vbar ? 2 * nch : nch;
  const int rowbytes = W * ESZ;
  float acc[NC][EPC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[c][e] = 0.f;
  // block-sum cache (paged): the entry of a full block sits at the physical
  // id of its first page and holds the same fp32 sums, in the same order, as
  // the row loop below
  float* csk = nullptr;
  float* csv = nullptr;
  bool from_cache = false;
  // (a cache without V sums serves only calls that pool no V: the V tasks
  // would otherwise read or write through a NULL pointer)
  if (a.bsum_k && (a.bsum_v || !a.vbar) && c1 - c0 == a.block) {
    const long pg = a.kv.page_table[(long)s * a.kv.max_pages + (c0 >> a.kv.page_log2)];
    csk = a.bsum_k + pg * W;
    csv = a.bsum_v ? a.bsum_v + pg * W : nullptr;
    from_cache = j < a.cached_blocks[s];
  }
  if (from_cache) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int task = t + c * kPoolThreads;
      if (task < ntask) {
        const bool isv = task >= nch;
        const float* src = (isv ? csv : csk) + (isv ? task - nch : task) * EPC;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[c][e] = src[e];
      }
    }
  }
  // rows in groups of kRows: every load of a group is issued before the
  // first is added (the adds keep the row order, so the sums are the same)
  int cc = from_cache ? c1 : c0;
  for (; cc + kRows <= c1; cc += kRows) {
    uint4 w[kRows][NC];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const char* krow = kv_row(a.kv, a.kv.k, s, a.seq.seqlen_k, cc + u, rowbytes);
      const char* vrow = kv_row(a.kv, a.kv.v, s, a.seq.seqlen_k, cc + u, rowbytes);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int task = t + c * kPoolThreads;
        if (task < ntask) {
          const char* row = task < nch ? krow : vrow;
          const int ch = task < nch ? task : task - nch;
          w[u][c] = *(const uint4*)(row + ch * 16);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRows; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (t + c * kPoolThreads < ntask) acc_chunk<ESZ>(acc[c], w[u][c]);
  }
  for (; cc < c1; ++cc) {
    const char* krow = kv_row(a.kv, a.kv.k, s, a.seq.seqlen_k, cc, rowbytes);
    const char* vrow = kv_row(a.kv, a.kv.v, s, a.seq.seqlen_k, cc, rowbytes);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int task = t + c * kPoolThreads;
      if (task < ntask) {
        const char* row = task < nch ? krow : vrow;
        const int ch = task < nch ? task : task - nch;
        acc_chunk<ESZ>(acc[c], *(const uint4*)(row + ch * 16));
      }
    }
  }
  if (csk && !from_cache) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int task = t + c * kPoolThreads;
      if (task < ntask) {
        const bool isv = task >= nch;
        float* dst = (isv ? csv : csk) + (isv ? task - nch : task) * EPC;
#pragma unroll
        for (int e = 0; e < EPC; ++e) dst[e] = acc[c][e];
      }
    }
  }
  const float inv = 1.f / (float)(c1 - c0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    int task = t + c * kPoolThreads;
    if (task < ntask) {
      bool isv = task >= nch;
      int ch = isv ? task - nch : task;
      int e0 = ch * EPC;
      int h = e0 / D, dd = e0 - h * D;
      float sc = inv;
      if (ESZ == 1) sc *= (isv ? a.v_scale : a.k_scale)[h];
      float* dst = (isv ? a.vbar : a.kbar) + (((long)s * a.Hkv + h) * a.seq.nkb_stride + j) * D + dd;
#pragma unroll
      for (int e = 0; e < EPC; ++e) dst[e] = acc[c][e] * sc;
    }
  }
}

constexpr int kSelThreads = 256;

// Block selection of TQ consecutive query blocks of one (sequence, KV head)
// per workgroup: scores against every visible pooled key block in LDS, the
// max-threshold rule per row, then the kept list in ascending order (with
// the sink and diagonal blocks).  Group-mean mode scores the group's pooled
// query once; union mode scores each query head of the group and keeps a
// block when any head keeps it; head-max mode scores each query head and
// thresholds the largest of the group's scores.
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  extern __shared__ float smem[];
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const SeqGeo g = seq_geo(a.seq, s, a.block);
  const int TQ = a.rows_per_wg;
  const int il0 = blockIdx.x * TQ;
  if (il0 >= g.nqb) return;
  const int nrows = min(TQ, g.nqb - il0);
  const int D = a.D;
  const int jmax = g.first_qb + il0 + nrows - 1;  // last visible key block of the run
  const int ncols = jmax + 1;
  const int nw = (ncols + 31) >> 5;
  float* qb = smem;                           // [TQ][D]
  float* sc = smem + TQ * D;                  // [TQ][ncols]
  uint32_t* kb = (uint32_t*)(sc + TQ * ncols);  // union mode: [TQ][nw] keep bits
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const float* kbh = a.kbar + ((long)s * a.Hkv + h) * a.seq.nkb_stride * D;
  // group mean: one pass over the group's pooled query; union: one pass per
  // query head of the group, each OR-ing its kept blocks into kb; head max:
  // one pass per query head, each raising the row's scores to its own
  const bool uni = a.select_mode == 1;
  const bool hmax = a.select_mode == 2;
  const int npass = a.select_mode != 0 ? a.Hq / a.Hkv : 1;
  if (uni)
    for (int o = t; o < nrows * nw; o += kSelThreads) kb[o] = 0u;

  for (int pass = 0; pass < npass; ++pass) {
    const float* qsrc = a.select_mode != 0 ? a.qbar + (((long)s * a.Hq + h * npass + pass) * a.seq.nqb_stride + il0) * D
                            : a.qbar + (((long)s * a.Hkv + h) * a.seq.nqb_stride + il0) * D;
    __syncthreads();
    for (int o = t; o < nrows * D; o += kSelThreads) qb[o] = qsrc[o];
    __syncthreads();

    // scores S[r][j] = <qbar_r, kbar_j> for all j <= jmax (fp32, fma over d
    // in order).  A column's kbar row is loaded eight float4 at a time, all
    // eight in flight before the first is used; rows past nrows compute on
    // row 0's query (in bounds, results dropped) so that the fma chain has
    // no branches.
    for (int j = t; j < ncols; j += kSelThreads) {
      float acc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const float4* krow = (const float4*)(kbh + (long)j * D);
      for (int d0 = 0; d0 < D / 4; d0 += 8) {  // D / 4 is 16 or 32
        float4 kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = krow[d0 + u];
        __builtin_amdgcn_sched_barrier(0);  // keep the eight loads ahead of their use
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float4 qv = *(const float4*)(qb + (r < nrows ? r : 0) * D + 4 * (d0 + u));
            acc[r] = fmaf(qv.x, kv[u].x, acc[r]);
            acc[r] = fmaf(qv.y, kv[u].y, acc[r]);
            acc[r] = fmaf(qv.z, kv[u].z, acc[r]);
            acc[r] = fmaf(qv.w, kv[u].w, acc[r]);
          }
        }
      }
      // each thread owns the same columns j in every pass
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < nrows) sc[r * ncols + j] = (hmax && pass > 0) ? fmaxf(sc[r * ncols + j], acc[r]) : acc[r];
    }
    __syncthreads();
    if (hmax && pass + 1 < npass) continue;  // threshold once every head has scored

    // per row: max over j <= i, threshold; group mean and head max:
    // ascending compaction right away; union: this head's kept blocks into
    // the row's keep bits
    for (int r = wave; r < nrows; r += kSelThreads / 64) {
      const int il = il0 + r;
      const int i = g.first_qb + il;
      const float* row = sc + r * ncols;
      float m = -INFINITY;
      for (int j = lane; j <= i; j += 64) m = fmaxf(m, row[j]);
      m = wave_max(m);
      const float thr = m - a.tau;
      if (uni) {
        for (int j0 = 0; j0 <= i; j0 += 64) {
          const int j = j0 + lane;
          const uint64_t mask = __ballot(j <= i && row[j] >= thr);
          if (lane == 0) {
            kb[r * nw + (j0 >> 5)] |= (uint32_t)mask;
            if ((j0 >> 5) + 1 < nw) kb[r * nw + (j0 >> 5) + 1] |= (uint32_t)(mask >> 32);
          }
        }
        continue;
      }
      int* dst = a.block_idx + (((long)s * a.Hkv + h) * a.seq.nqb_stride + il) * (long)a.seq.nkb_stride;
      int base = 0;
      for (int j0 = 0; j0 <= i; j0 += 64) {
        int j = j0 + lane;
        bool keep = false;
        if (j <= i) keep = (row[j] >= thr) || j == 0 || j == i;
        uint64_t mask = __ballot(keep);
        if (keep) dst[base + __popcll(mask & lt_mask)] = j;
        base += __popcll(mask);
      }
      if (lane == 0) a.block_cnt[((long)s * a.Hkv + h) * a.seq.nqb_stride + il] = base;
    }
  }
  if (!uni) return;

  // union: ascending compaction of the keep bits, plus sink and diagonal
  __syncthreads();
  for (int r = wave; r < nrows; r += kSelThreads / 64) {
    const int il = il0 + r;
    const int i = g.first_qb + il;
    int* dst = a.block_idx + (((long)s * a.Hkv + h) * a.seq.nqb_stride + il) * (long)a.seq.nkb_stride;
    int base = 0;
    for (int j0 = 0; j0 <= i; j0 += 64) {
      const int j = j0 + lane;
      bool keep = false;
      if (j <= i) keep = ((kb[r * nw + (j >> 5)] >> (j & 31)) & 1u) || j == 0 || j == i;
      const uint64_t mask = __ballot(keep);
      if (keep) dst[base + __popcll(mask & lt_mask)] = j;
      base += __popcll(mask);
    }
    if (lane == 0) a.block_cnt[((long)s * a.Hkv + h) * a.seq.nqb_stride + il] = base;
  }
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t st) {
  dim3 grid(a.seq.nqb_stride + a.seq.nkb_stride, a.seq.batch);
  size_t lds = (size_t)a.Hq * a.D * sizeof(float);
  // chunk slots per thread: the larger of the query row (Hq D elements) and
  // the key block's K (and V) rows, in 16-byte chunks over kPoolThreads
  const int epc = a.fp8 ? 16 : 8;
  const int tasks = std::max(a.Hq * a.D / epc, (a.vbar ? 2 : 1) * a.Hkv * a.D / epc);
  const int nc = (tasks + kPoolThreads - 1) / kPoolThreads;
  if (nc < 1 || nc > kMaxChunksPerThread) return hipErrorInvalidValue;
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kPoolThreads), lds, st, a); };
  if (a.fp8) {
    if (nc == 1) go(pool_kernel<1, 1>);
    else if (nc == 2) go(pool_kernel<1, 2>);
    else if (nc == 3) go(pool_kernel<1, 3>);
    else go(pool_kernel<1, 4>);
  } else {
    if (nc == 1) go(pool_kernel<2, 1>);
    else if (nc == 2) go(pool_kernel<2, 2>);
    else if (nc == 3) go(pool_kernel<2, 3>);
    else go(pool_kernel<2, 4>);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  dim3 grid((a.seq.nqb_stride + a.rows_per_wg - 1) / a.rows_per_wg, a.Hkv, a.seq.batch);
  size_t lds = (size_t)a.rows_per_wg * (a.D + a.seq.nkb_stride + (a.seq.nkb_stride + 31) / 32) * sizeof(float);
  const hipError_t e =
      hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace fp2
