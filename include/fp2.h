/*
 * fp2.h -- C ABI of the MI355X (gfx950) block-sparse causal prefill attention
 * library: block selection, sparse attention with mean correction, the dense
 * causal baseline, and the paged-KV / chunked-prefill path.
 *
 * The operation (sources are cited by page title and section):
 *  - "FlashPrefill V2: block-sparse prefill attention for long-context LLM
 *    serving", abstract: instantaneous pattern discovery and max-based dynamic
 *    thresholding select the key blocks each query block attends to; a mean
 *    correction term suppresses the error of the dropped blocks; the operator
 *    supports GQA (PackGQA), FP8, paged KV cache and continuous batching.
 *  - papers.ananclaw.com explainer, §2.1: for query block q only the
 *    threshold-selected keys Supp(q) are computed; V2 adds the mean
 *    correction Out_q^V2 built from mu_q and the dropped blocks' average value.
 *    §2.2: PackGQA (the query heads of one GQA group share a K/V tile).
 *    §2.3: FP8 E4M3 with scale calibration; paged KV whose block size matches
 *    the page table; continuous batching.
 *
 * What the library computes, per sequence, KV head h and query block i
 * (blocks numbered by absolute position, block size b):
 *  1. qbar_i = mean of Q over the G = Hq/Hkv query heads of group h and the
 *     rows of block i present in the call; kbar_j, vbar_j = means of K, V over
 *     the keys of block j (fp32 accumulation).
 *  2. S_ij = <qbar_i, kbar_j> (unscaled), 0 <= j <= i; m_i = max_j S_ij;
 *     block j is kept iff S_ij >= m_i - tau; blocks 0 and i are always kept.
 *  3. Each query row attends causally to the keys of the kept blocks.
 *  4. With mean_correction != 0 every dropped block j enters the same softmax
 *     as one pseudo-key with logit softmax_scale*<q, kbar_j> + ln(n_j) and
 *     value vbar_j (n_j = keys in block j).
 *  5. out = normalised sum; lse = natural log of the softmax denominator.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers, scalars and the params struct are
 *    host memory.  The caller owns every buffer, the workspace included; the
 *    library allocates no device memory and keeps no pointer after a call.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  Buffers must stay valid until the stream has run it.
 *    Only kernels are enqueued (no memset, copy or host synchronisation), so
 *    a call can be captured into a HIP graph.  The attention kernel pulls
 *    its tiles from 8 device-side counters that no concurrent launch may
 *    share.  The paged entry points keep them in the caller's workspace
 *    (with the call's pooled blocks, mask and task list), so a workspace,
 *    like any output buffer, must not be shared by calls that overlap in
 *    time; calls on one stream run in order and may reuse it.
 *    fp2_sparse_prefill and fp2_dense_prefill use one of the library's sets:
 *    each of the first 192 streams a process launches them on gets a set of
 *    its own (reused by that stream's later launches, which run in order;
 *    beyond 192 streams the oldest stream's set is handed on; each host
 *    thread's hipStreamPerThread counts as a stream of its own), and a launch
 *    captured into a HIP graph gets the next of 64 further sets, which no
 *    eager launch uses.  So launches on different streams may run at once,
 *    and graph replays may run next to eager launches on any stream; one
 *    graph must not be replayed concurrently with itself, or with a graph
 *    whose launch was captured a multiple of 64 captured launches later.
 *  - Layouts are row-major.  Contiguous tensors are BSHD: q [B, Sq, Hq, d],
 *    k and v [B, Sk, Hkv, d], out [B, Sq, Hq, d].  Query head hq reads KV
 *    head hq / G.  Query row r of a sequence sits at absolute position
 *    Sk - Sq + r (Sq < Sk is a chunked prefill over a cached prefix).
 *  - Host-side validation runs before anything is enqueued; on any error the
 *    call returns a negative fp2_status, enqueues nothing, and
 *    fp2_last_error() (thread-local) describes the problem.  A failed launch
 *    returns FP2_EDEVICE.  No C++ exception crosses this interface.
 *  - With FP2_LOG=1 in the environment every call prints one line of its
 *    launch shape to stderr; results are unchanged.
 *  - Numerical range: each query row's softmax runs against a fixed
 *    reference (the largest logit over the first 32 keys of the row's first
 *    kept block, plus a margin) instead of a running maximum.  A row whose
 *    normaliser leaves fp32's range against it (logits far above that
 *    reference) makes its workgroup recompute the tile with the reference
 *    moved up (to the pass's normaliser, its largest fp8 superchunk maximum,
 *    or found by a doubling-then-bisecting search when the normaliser
 *    overflowed), so results are those of the exact softmax for logits up
 *    to 4e6 log2 units above the reference; a row beyond that is written as
 *    NaN (and its lse as NaN).  Logits must be finite in fp32.
 *  - Supported shapes: head_dim in {64, 128}; block_size in {64, 128};
 *    num_q_heads a positive multiple of num_kv_heads, with num_q_heads *
 *    head_dim <= 8192 and num_kv_heads * head_dim <= 4096 for bf16 inputs
 *    (16384 and 8192 for fp8; e.g. up to 64 query and 32 KV heads at d 128
 *    in bf16); in_dtype FP2_BF16 or FP2_FP8_E4M3; out_dtype FP2_BF16,
 *    FP2_FP32 or FP2_FP8_E4M3 (with o_scale); seqlen_k up to
 *    fp2_max_seqlen_k.
 */
#ifndef FP2_H
#define FP2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP2_OK = 0,
  FP2_EINVAL = -1,        /* bad argument (null pointer, bad size, NaN tau) */
  FP2_EUNSUPPORTED = -2,  /* valid request outside the supported shapes     */
  FP2_EWORKSPACE = -3,    /* workspace missing or smaller than required     */
  FP2_EDEVICE = -4        /* HIP runtime or launch error                    */
} fp2_status;

typedef enum { FP2_BF16 = 0, FP2_FP8_E4M3 = 1, FP2_FP32 = 2 } fp2_dtype;

typedef struct {
  int32_t num_q_heads;     /* Hq                                               */
  int32_t num_kv_heads;    /* Hkv; G = Hq / Hkv                                */
  int32_t head_dim;        /* d: 64 or 128                                     */
  int32_t block_size;      /* b: 64 or 128 (the selection granularity)         */
  float softmax_scale;     /* <= 0 means 1/sqrt(head_dim)                      */
  float tau;               /* threshold on the unscaled block scores S_ij;
                            * +INFINITY keeps every block; NaN is an error.
                            * A threshold tau_s on softmax-scaled scores
                            * (s * S_ij) is tau = tau_s / s.                  */
  int32_t mean_correction; /* 0: drop blocks outright; 1: pseudo-key correction */
  int32_t in_dtype;        /* fp2_dtype of q, k, v: FP2_BF16 or FP2_FP8_E4M3   */
  int32_t out_dtype;       /* fp2_dtype of out: FP2_BF16, FP2_FP32 or FP2_FP8_E4M3 */
  /* FP8 only (E4M3, OCP "e4m3fn" encoding): per-head dequantization scales,
   * DEVICE fp32 arrays q_scale [Hq], k_scale [Hkv], v_scale [Hkv]; a value is
   * code * scale.  Ignored for bf16 inputs.                                   */
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  /* FP8 output only (out_dtype FP2_FP8_E4M3, any in_dtype): DEVICE pointer to
   * one fp32 per-tensor scale; the output value is code * (*o_scale).  Codes
   * are round-to-nearest-even of out / o_scale, saturated to +-448 (e4m3fn
   * has no infinity).  Must be a positive finite value; ignored otherwise.  */
  const float* o_scale;
  /* Selection rule under GQA packing (explainer §2.2 PackGQA, with the
   * block selection of §2.1; the pages leave open how the group's heads
   * share one mask): 0 = the group-mean qbar of step 1 above;
   * 1 = per query head: qbar_{hq,i} = mean of head hq's rows of block i,
   * each head applies step 2 to <qbar_{hq,i}, kbar_j>, and the group keeps
   * the union of its heads' blocks (plus sink and diagonal);
   * 2 = per query head scores <qbar_{hq,i}, kbar_j> as in mode 1, the
   * group's score is their maximum over the group's heads, and step 2 runs
   * once on that score (mode 0 is the same with the mean over the heads in
   * place of the maximum, since the score is linear in qbar).  The masks
   * stay per KV head, since the group shares one K/V tile.  Modes 1 and 2
   * need Hq/Hkv times the pooled-query workspace of mode 0.  Other values
   * are FP2_EINVAL.                                                        */
  int32_t select_mode;
} fp2_params;

/* Number of query blocks a sequence touches: blocks of absolute positions
 * [Sk - Sq, Sk), i.e. (Sk-1)/b - (Sk-Sq)/b + 1.  Key blocks: ceil(Sk / b). */
int32_t fp2_num_q_blocks(int32_t seqlen_q, int32_t seqlen_k, int32_t block_size);
int32_t fp2_num_k_blocks(int32_t seqlen_k, int32_t block_size);

/* Largest seqlen_k (per sequence, max_seqlen_k for the paged entry points)
 * that the kernels accept for these parameters: the selection keeps a row of
 * scores over every key block in LDS, the attention kernel the dropped-block
 * list of a query block.  Longer calls return FP2_EUNSUPPORTED.  Returns 0
 * for invalid parameters.                                                    */
int32_t fp2_max_seqlen_k(const fp2_params* p);

/* Workspace bytes needed by fp2_select_blocks for this problem size (the
 * pooled query blocks, fp32).  Returns 0 for invalid parameters.             */
size_t fp2_select_workspace_size(const fp2_params* p, int32_t batch,
                                 int32_t seqlen_q, int32_t seqlen_k);

/* One workspace size for every entry point that takes a workspace: at least
 * fp2_select_workspace_size(p, b, sq, sk) for every b <= batch, sq <=
 * max_seqlen_q, sk <= max_seqlen_k (sq <= sk), and at least
 * fp2_paged_workspace_size(p, n, max_seqlen_q, max_seqlen_k) for every
 * n <= batch.  A caller that sizes one buffer for the largest call it will
 * make can use it for both paths.  Returns 0 for invalid parameters.        */
size_t fp2_workspace_size(const fp2_params* p, int32_t batch,
                          int32_t max_seqlen_q, int32_t max_seqlen_k);

/* Block selection (steps 1-2 above; abstract: pattern discovery and max-based
 * dynamic thresholding; explainer §2.1: Supp(q)).
 *   q, k, v    : contiguous BSHD inputs (in_dtype).
 *   block_idx  : int32 [B, Hkv, nqb, nkb]; row (b, h, il) receives the kept
 *                key blocks of query block il (local index; absolute block
 *                (Sk-Sq)/b + il) in ascending order in entries [0, cnt);
 *                entries [cnt, nkb) are left undefined.
 *   block_cnt  : int32 [B, Hkv, nqb], the number of kept blocks per row.
 *   pooled_k   : fp32 [B, Hkv, nkb, d], the key-block means kbar.
 *   pooled_v   : fp32 [B, Hkv, nkb, d], the value-block means vbar; may be
 *                NULL (then not written).
 *   workspace  : device scratch of at least fp2_select_workspace_size bytes. */
fp2_status fp2_select_blocks(const fp2_params* p, int32_t batch,
                             int32_t seqlen_q, int32_t seqlen_k,
                             const void* q, const void* k, const void* v,
                             int32_t* block_idx, int32_t* block_cnt,
                             float* pooled_k, float* pooled_v,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* fp2_select_blocks without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing: the pooled query
 * blocks go to a static 16 MiB device array of the library (one copy per
 * GPU, held until the process ends).  Same arguments, kernels and results as
 * fp2_select_blocks.
 *   Limit: fp2_select_workspace_size(p, batch, seqlen_q, seqlen_k) must be at
 *   most 16 MiB (16777216 bytes), e.g. batch 4 at 128K tokens with 8 KV
 *   heads, d = 128, group-mean selection; larger calls return
 *   FP2_EUNSUPPORTED before anything is enqueued.  Other errors as
 *   fp2_select_blocks; FP2_EDEVICE if the array's device address cannot be
 *   obtained on the current device.
 *   All calls on one GPU share the array: calls that overlap in time on one
 *   GPU (different streams, or a captured graph replayed next to another
 *   call) race and give undefined results.  Calls in stream order are safe. */
fp2_status fp2_select_blocks_noalloc(const fp2_params* p, int32_t batch,
                                     int32_t seqlen_q, int32_t seqlen_k,
                                     const void* q, const void* k, const void* v,
                                     int32_t* block_idx, int32_t* block_cnt,
                                     float* pooled_k, float* pooled_v,
                                     void* stream);

/* Block-sparse causal attention with mean correction (steps 3-5; explainer
 * §2.1 Out_q^V2, §2.2 PackGQA).  Takes the mask and pooled blocks in the
 * layout fp2_select_blocks produces.  Any mask is accepted whose rows are
 * strictly ascending lists of blocks in [0, i] that contain the diagonal
 * block i; the dropped set of a row is the complement of its list in [0, i].
 * pooled_k and pooled_v are read only when mean_correction != 0 (then both
 * must be non-NULL).
 *   out : [B, Sq, Hq, d] in out_dtype.   lse : fp32 [B, Hq, Sq] or NULL.    */
fp2_status fp2_sparse_prefill(const fp2_params* p, int32_t batch,
                              int32_t seqlen_q, int32_t seqlen_k,
                              const void* q, const void* k, const void* v,
                              const int32_t* block_idx, const int32_t* block_cnt,
                              const float* pooled_k, const float* pooled_v,
                              void* out, float* lse, void* stream);

/* Dense causal attention softmax(scale * Q K^T) V over every key up to the
 * query's position (explainer §1.1; the abstract's dense baseline): the same
 * kernel as fp2_sparse_prefill with every block kept and no correction.
 * tau and mean_correction are ignored.                                       */
fp2_status fp2_dense_prefill(const fp2_params* p, int32_t batch,
                             int32_t seqlen_q, int32_t seqlen_k,
                             const void* q, const void* k, const void* v,
                             void* out, float* lse, void* stream);

/* Paged KV cache + continuous batch (abstract: paged KV cache and continuous
 * batching; explainer §2.3: KV block size matches the page table).
 *   q            : [total_q, Hq, d] packed new query rows of all sequences.
 *   cu_seqlens_q : int32 [num_seqs + 1] device, row offsets into q (and out).
 *   seqlens_k    : int32 [num_seqs] device, tokens in the cache per sequence,
 *                  the new chunk included (its K/V must already be written).
 *                  Sequence s has q_len = cu[s+1] - cu[s] <= seqlens_k[s]; its
 *                  query row r sits at position seqlens_k[s] - q_len + r.
 *                  q_len may be 0 (a slot with cached tokens and no new rows:
 *                  it gets no output rows and no attention tiles, and the
 *                  exported mask holds no row for it); seqlens_k[s] >= 1.
 *   max_seqlen_q, max_seqlen_k : host upper bounds of q_len and seqlens_k.
 *   k_cache, v_cache : [num_pages, page_size, Hkv, d] (in_dtype).
 *   page_size    : a power of two dividing block_size, at least
 *                  block_size / 64 (a block spans at most 64 pages).
 *   page_table   : int32 [num_seqs, max_pages_per_seq] device; token t of
 *                  sequence s lives in page page_table[s][t / page_size], row
 *                  t % page_size.  Entries must be in [0, num_pages); with
 *                  FP2_VALIDATE=1 in the environment the call copies the
 *                  lengths and the table to the host (synchronising the
 *                  stream) and rejects out-of-range values, otherwise they
 *                  are undefined behaviour.
 *   out          : [total_q, Hq, d] out_dtype.  lse: fp32 [total_q, Hq] or NULL.
 *   block_idx, block_cnt : optional mask export (both NULL or both set), laid
 *                  out [num_seqs, Hkv, max_nqb, max_nkb] and
 *                  [num_seqs, Hkv, max_nqb] with the sizes given by
 *                  fp2_paged_mask_dims; row il of sequence s is its il-th
 *                  query block, as in fp2_select_blocks.
 *   workspace    : at least fp2_paged_workspace_size bytes; holds the
 *                  call's pooled blocks, mask, task list and tile-queue
 *                  counters until the call has run (see the conventions).    */
void fp2_paged_mask_dims(const fp2_params* p, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, int32_t* max_nqb, int32_t* max_nkb);
size_t fp2_paged_workspace_size(const fp2_params* p, int32_t num_seqs,
                                int32_t max_seqlen_q, int32_t max_seqlen_k);
fp2_status fp2_sparse_prefill_paged(const fp2_params* p, int32_t num_seqs,
                                    const void* q, const int32_t* cu_seqlens_q,
                                    const int32_t* seqlens_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    const void* k_cache, const void* v_cache,
                                    int32_t num_pages, int32_t page_size,
                                    const int32_t* page_table, int32_t max_pages_per_seq,
                                    void* out, float* lse,
                                    int32_t* block_idx, int32_t* block_cnt,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/* fp2_sparse_prefill_paged with a caller-kept cache of key-block sums, for
 * chunked prefill ([EXP] §2.3: paged KV with chunked prefill; the pooled
 * statistics of a cached prefix do not change between its chunks, so they
 * are kept next to the KV cache instead of re-read from it every chunk).
 *   block_sums_k, block_sums_v : fp32 [num_pages, Hkv, d] (DEVICE, caller
 *       owned, kept across calls).  The entry of a FULL key block (block_size
 *       keys) of a sequence sits at the physical id of the block's first page
 *       and holds the fp32 row sums of its K (and V) rows, in code units for
 *       fp8 inputs.  block_sums_v may be NULL when mean_correction is 0.
 *   cached_blocks : int32 [num_seqs] (DEVICE): key blocks [0, cached_blocks[s])
 *       of sequence s are read from the cache (they must be full and unchanged
 *       since they were written); every other full block of the call is summed
 *       from the pages and written to the cache.  After the call, the full
 *       blocks of sequence s are its first seqlens_k[s] / block_size blocks,
 *       which is what cached_blocks[s] may be set to for its next chunk.  A
 *       page freed or rewritten invalidates the entry of the block it starts.
 * Results are bit-identical to fp2_sparse_prefill_paged on the same inputs
 * (the cached sums are the same fp32 sums in the same order).  Errors as
 * fp2_sparse_prefill_paged, plus FP2_EINVAL for a NULL cache argument.        */
fp2_status fp2_sparse_prefill_paged_pooled(const fp2_params* p, int32_t num_seqs,
                                           const void* q, const int32_t* cu_seqlens_q,
                                           const int32_t* seqlens_k,
                                           int32_t max_seqlen_q, int32_t max_seqlen_k,
                                           const void* k_cache, const void* v_cache,
                                           int32_t num_pages, int32_t page_size,
                                           const int32_t* page_table, int32_t max_pages_per_seq,
                                           void* out, float* lse,
                                           int32_t* block_idx, int32_t* block_cnt,
                                           void* workspace, size_t workspace_bytes,
                                           float* block_sums_k, float* block_sums_v,
                                           const int32_t* cached_blocks, void* stream);

/* Human-readable name of a status code (static string). */
const char* fp2_status_string(fp2_status s);
/* Description of the last error raised on the calling thread ("" if none). */
const char* fp2_last_error(void);
/* Library version string. */
const char* fp2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP2_H */
