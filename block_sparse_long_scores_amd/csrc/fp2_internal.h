// Internal interface between the C ABI layer (api.cpp) and the kernel
// launchers (*.hip).  Plain structs of device pointers and sizes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp2 {

// Geometry of the sequences of one call.  Contiguous calls have `batch`
// sequences of equal length; paged calls read per-sequence lengths from the
// device arrays cu_seqlens_q / seqlens_k.
struct SeqDesc {
  int batch;          // number of sequences
  int seqlen_q;       // contiguous: query rows per sequence
  int seqlen_k;       // contiguous: keys per sequence
  const int* cu_seqlens_q;  // paged: [batch+1] (device) or nullptr
  const int* seqlens_k;     // paged: [batch] (device) or nullptr
  int nqb_stride;     // query blocks per sequence in the mask / qbar arrays
  int nkb_stride;     // key blocks per sequence in the mask / pooled arrays
};

// K/V addressing: contiguous [B, Sk, Hkv, D] or paged [pages, page, Hkv, D].
struct KVDesc {
  const void* k;
  const void* v;
  const int* page_table;    // paged: [batch, max_pages] or nullptr
  int max_pages;
  int page_log2;            // log2(page_size) when paged
};

// The pooling kernel streams one row of a query block (all Hq heads) or of a
// key block (K and V of all Hkv heads) per step, 16 bytes per task and at
// most this many tasks per row (256 threads x 4 chunks each).
constexpr int kPoolMaxTasks = 1024;

struct PoolArgs {
  SeqDesc seq;
  KVDesc kv;
  const void* q;            // contiguous [B, Sq, Hq, D] or packed [total_q, Hq, D]
  float* qbar;              // [B, Hkv, nqb_stride, D]
  float* kbar;              // [B, Hkv, nkb_stride, D]
  float* vbar;              // [B, Hkv, nkb_stride, D] or nullptr
  const float* q_scale;     // fp8 only
  const float* k_scale;
  const float* v_scale;
  int Hq, Hkv, D, block, fp8;
  // Paged calls with a block-sum cache (or nullptr): fp32 row sums of full
  // key blocks, [num_pages, Hkv * D] each, at the physical id of the block's
  // first page; blocks below cached_blocks[s] are read from it, every other
  // full block is summed and written to it.
  float* bsum_k;
  float* bsum_v;
  const int* cached_blocks;
  int select_mode;          // 1, 2: qbar per query head [B, Hq, nqb_stride, D]
};

struct SelectArgs {
  SeqDesc seq;
  const float* qbar;
  const float* kbar;
  int* block_idx;           // [B, Hkv, nqb_stride, nkb_stride]
  int* block_cnt;           // [B, Hkv, nqb_stride]
  int Hkv, D, block;
  float tau;
  int rows_per_wg;          // query blocks per workgroup
  int select_mode;          // 0: group-mean qbar; 1: union over the group's query heads;
                            // 2: largest of the group's per-head scores
  int Hq;
};

// Work-ordered task list of a continuous batch (plan.hip).
struct PlanArgs {
  SeqDesc seq;
  const int* block_cnt;     // [B, Hkv, nqb_stride]
  int* plan;                // out: task ids (s*Hkv + h)*nqb_stride + il, longest first
  int* plan_count;          // out: number of tasks
  unsigned* sched;          // out: the attention launch's tile-queue counters, zeroed
  int Hkv, block, mean_correction;
};

struct AttnArgs {
  SeqDesc seq;
  KVDesc kv;
  const void* q;
  void* out;
  float* lse;
  int lse_stride;           // contiguous: Sq per (b, hq) row; paged layout [total_q, Hq] ignores it
  const int* block_idx;     // sparse only
  const int* block_cnt;
  const float* kbar;        // mean correction only
  const float* vbar;
  const float* q_scale;     // fp8 only
  const float* k_scale;
  const float* v_scale;
  int Hq, Hkv, G;
  float scale_log2;         // softmax_scale * log2(e)
  int sparse;               // 1: block list + optional correction; 0: dense
  int mean_correction;
  int out_mode;             // output dtype: 0 bf16, 1 fp32, 2 e4m3 (codes of out / *o_scale)
  const float* o_scale;     // e4m3 output: per-tensor scale (device)
  int parts;                // workgroups per (seq, head, q-block) tile
  int waves;                // waves per workgroup
  int nqb_grid;             // query-block extent of the tile space
  int head_group;           // KV heads per group of the tile order (divides Hkv; no plan)
  const int* plan;          // optional work-ordered task list (PlanArgs) or nullptr
  const int* plan_count;
  // tile-queue counters (8 x 32 unsigned, zeroed before the launch) in caller
  // memory, or nullptr: the launcher then takes one of the library's sets
  unsigned* sched;
  // set by the launcher
  int ntiles;               // Hkv * batch * parts * nqb_grid
  int sched_slot;           // the library's counter set used when sched is nullptr
  int lds_sched;            // LDS byte offset of the next-tile broadcast
  int lds_dtab;             // LDS byte offset of the copy-offset table
};

hipError_t launch_pool(const PoolArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int D, int block, int fp8, hipStream_t s);
// Dynamic LDS bytes of the attention kernel (0 for an unsupported shape).
size_t attention_lds_bytes(int D, int block, int nkb, int fp8);
hipError_t launch_attention_bf16(const AttnArgs& a, int D, int block, hipStream_t s);
hipError_t launch_attention_fp8(const AttnArgs& a, int D, int block, hipStream_t s);
size_t attention_lds_bytes_bf16(int D, int block, int nkb);
size_t attention_lds_bytes_fp8(int D, int block, int nkb);

// Records msg as the calling thread's last error (fp2_last_error) and
// returns st; for entry points defined outside api.cpp.
int set_last_error(int st, const char* msg);

}  // namespace fp2
