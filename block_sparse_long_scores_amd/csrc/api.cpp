// C ABI of the library (declared in include/fp2.h): argument validation,
// workspace carving and kernel launches.  Nothing here allocates device
// memory; every error is reported before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "fp2.h"
#include "fp2_internal.h"

using namespace fp2;

namespace {

thread_local std::string g_err;

fp2_status fail(fp2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

fp2_status ok() {
  g_err.clear();
  return FP2_OK;
}

fp2_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FP2_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int nq_blocks(int sq, int sk, int b) { return (sk - 1) / b - (sk - sq) / b + 1; }
int nk_blocks(int sk, int b) { return (sk + b - 1) / b; }

bool env_validate() {
  const char* v = std::getenv("FP2_VALIDATE");
  return v && v[0] == '1';
}

bool env_log() {
  const char* v = std::getenv("FP2_LOG");
  return v && v[0] == '1';
}

fp2_status check_params(const fp2_params* p) {
  if (!p) return fail(FP2_EINVAL, "params is NULL");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(FP2_EINVAL, "num_q_heads=%d num_kv_heads=%d must be positive", p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(FP2_EINVAL, "num_q_heads=%d is not a multiple of num_kv_heads=%d", p->num_q_heads, p->num_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(FP2_EUNSUPPORTED, "head_dim=%d not in {64, 128}", p->head_dim);
  if (p->block_size != 64 && p->block_size != 128)
    return fail(FP2_EUNSUPPORTED, "block_size=%d not in {64, 128}", p->block_size);
  if (std::isnan(p->tau)) return fail(FP2_EINVAL, "tau is NaN");
  if (std::isnan(p->softmax_scale) || std::isinf(p->softmax_scale))
    return fail(FP2_EINVAL, "softmax_scale is not finite");
  if (p->in_dtype != FP2_BF16 && p->in_dtype != FP2_FP8_E4M3)
    return fail(FP2_EUNSUPPORTED, "in_dtype=%d not supported", p->in_dtype);
  if (p->out_dtype != FP2_BF16 && p->out_dtype != FP2_FP32 && p->out_dtype != FP2_FP8_E4M3)
    return fail(FP2_EUNSUPPORTED, "out_dtype=%d not supported", p->out_dtype);
  if (p->out_dtype == FP2_FP8_E4M3 && !p->o_scale)
    return fail(FP2_EINVAL, "out_dtype FP8_E4M3 needs o_scale");
  if (p->in_dtype == FP2_FP8_E4M3 && (!p->q_scale || !p->k_scale || !p->v_scale))
    return fail(FP2_EINVAL, "fp8 inputs need q_scale, k_scale and v_scale");
  if (p->mean_correction != 0 && p->mean_correction != 1)
    return fail(FP2_EINVAL, "mean_correction=%d must be 0 or 1", p->mean_correction);
  if (p->select_mode < 0 || p->select_mode > 2)
    return fail(FP2_EINVAL, "select_mode=%d must be 0, 1 or 2", p->select_mode);
  // the pooling kernel's 16-byte tasks per row: a query row of all Hq heads,
  // a key row of K and V of all Hkv heads
  const long esz = p->in_dtype == FP2_FP8_E4M3 ? 1 : 2;
  if ((long)p->num_q_heads * p->head_dim * esz > 16L * kPoolMaxTasks ||
      2L * p->num_kv_heads * p->head_dim * esz > 16L * kPoolMaxTasks)
    return fail(FP2_EUNSUPPORTED, "num_q_heads=%d / num_kv_heads=%d too many for head_dim=%d (at most %ld q and %ld kv heads)",
                p->num_q_heads, p->num_kv_heads, p->head_dim, 16L * kPoolMaxTasks / (p->head_dim * esz),
                8L * kPoolMaxTasks / (p->head_dim * esz));
  return FP2_OK;
}

fp2_status check_lengths(int batch, int sq, int sk) {
  if (batch <= 0) return fail(FP2_EINVAL, "batch=%d must be positive", batch);
  if (sq <= 0 || sk < sq) return fail(FP2_EINVAL, "need 0 < seqlen_q=%d <= seqlen_k=%d", sq, sk);
  return FP2_OK;
}

// Query blocks per select workgroup such that the score rows fit in LDS.
int select_rows_per_wg(int D, int nkb) {
  for (int tq = 16; tq >= 1; tq >>= 1)
    if ((size_t)tq * (D + nkb + (nkb + 31) / 32) * sizeof(float) <= 160 * 1024) return tq;
  return 0;
}

bool attn_lds_ok(int D, int block, int nkb, int fp8) {
  const size_t need = attention_lds_bytes(D, block, nkb, fp8);
  return need > 0 && need <= 160 * 1024;
}

float scale_of(const fp2_params* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.f / std::sqrt((float)p->head_dim);
}

// KV heads per group in a dense launch's tile order.  Every dense tile
// streams its head's whole K/V prefix, so the heads in flight at once set the
// read working set.  When the K and V of all heads (over the batch) exceed
// 128 MiB, half of the 256 MB last-level cache in front of HBM, the heads go
// two at a time: at 128K keys, d 128 and 8 KV heads this measured 5% faster
// in bf16 and 2% in fp8 than all heads at once, and one or four heads at a
// time were slower than two.  Sparse launches read only their kept blocks;
// they keep every head in flight, which measured the same or better.
static int dense_head_group(int Hkv, int batch, long seqlen_k, int D, int esz) {
  const double kv_bytes = 2.0 * batch * (double)seqlen_k * D * esz * Hkv;
  if (kv_bytes <= 128.0 * 1024 * 1024 || Hkv % 2 != 0) return Hkv;
  return 2;
}

void fill_attn_common(AttnArgs& a, const fp2_params* p) {
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.scale_log2 = scale_of(p) * 1.4426950408889634f;
  a.out_mode = p->out_dtype == FP2_FP32 ? 1 : p->out_dtype == FP2_FP8_E4M3 ? 2 : 0;
  a.o_scale = p->out_dtype == FP2_FP8_E4M3 ? p->o_scale : nullptr;
  a.q_scale = p->q_scale;
  a.k_scale = p->k_scale;
  a.v_scale = p->v_scale;
  // packed query rows of a GQA tile: 64 per wavefront, at most 4 wavefronts
  // (256 rows) per workgroup
  const int rows = a.G * p->block_size;
  a.parts = (rows + 255) / 256;
  const int rows_part = rows < 256 ? rows : 256;
  a.waves = (rows_part + 63) / 64;
}

}  // namespace

namespace fp2 {
int set_last_error(int st, const char* msg) { return fail((fp2_status)st, "%s", msg); }
}  // namespace fp2

extern "C" {

int32_t fp2_num_q_blocks(int32_t seqlen_q, int32_t seqlen_k, int32_t block_size) {
  if (block_size <= 0 || seqlen_q <= 0 || seqlen_k < seqlen_q) return 0;
  return nq_blocks(seqlen_q, seqlen_k, block_size);
}

int32_t fp2_num_k_blocks(int32_t seqlen_k, int32_t block_size) {
  if (block_size <= 0 || seqlen_k <= 0) return 0;
  return nk_blocks(seqlen_k, block_size);
}

int32_t fp2_max_seqlen_k(const fp2_params* p) {
  if (check_params(p) != FP2_OK) return 0;
  const int D = p->head_dim, b = p->block_size;
  const int fp8 = p->in_dtype == FP2_FP8_E4M3;
  // both limits fall as nkb grows: the selection's score rows and the
  // attention kernel's correction buffers (dropped-block list) in LDS
  auto fits = [&](int nkb) { return select_rows_per_wg(D, nkb) > 0 && attn_lds_ok(D, b, nkb, fp8); };
  if (!fits(1)) return 0;
  int lo = 1, hi = (1 << 30) / b;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (fits(mid)) lo = mid;
    else hi = mid - 1;
  }
  return lo * b;
}

size_t fp2_select_workspace_size(const fp2_params* p, int32_t batch, int32_t seqlen_q, int32_t seqlen_k) {
  if (check_params(p) != FP2_OK || check_lengths(batch, seqlen_q, seqlen_k) != FP2_OK) return 0;
  const int nqb = nq_blocks(seqlen_q, seqlen_k, p->block_size);
  const int qh = p->select_mode != 0 ? p->num_q_heads : p->num_kv_heads;  // pooled query rows per block
  return align_up((size_t)batch * qh * nqb * p->head_dim * sizeof(float));
}

fp2_status fp2_select_blocks(const fp2_params* p, int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                             const void* q, const void* k, const void* v, int32_t* block_idx,
                             int32_t* block_cnt, float* pooled_k, float* pooled_v, void* workspace,
                             size_t workspace_bytes, void* stream) {
  fp2_status st = check_params(p);
  if (st != FP2_OK) return st;
  if ((st = check_lengths(batch, seqlen_q, seqlen_k)) != FP2_OK) return st;
  if (!q || !k || !v || !block_idx || !block_cnt || !pooled_k)
    return fail(FP2_EINVAL, "q, k, v, block_idx, block_cnt and pooled_k must be non-NULL");
  const int D = p->head_dim, b = p->block_size;
  const int nqb = nq_blocks(seqlen_q, seqlen_k, b);
  const int nkb = nk_blocks(seqlen_k, b);
  const int tq = select_rows_per_wg(D, nkb);
  if (tq == 0) return fail(FP2_EUNSUPPORTED, "seqlen_k=%d: %d key blocks exceed the selection kernel's LDS", seqlen_k, nkb);
  const size_t need = fp2_select_workspace_size(p, batch, seqlen_q, seqlen_k);
  if (!workspace || workspace_bytes < need)
    return fail(FP2_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);

  SeqDesc sd{batch, seqlen_q, seqlen_k, nullptr, nullptr, nqb, nkb};
  PoolArgs pa{};
  pa.seq = sd;
  pa.kv = KVDesc{k, v, nullptr, 0, 0};
  pa.q = q;
  pa.qbar = (float*)workspace;
  pa.kbar = pooled_k;
  pa.vbar = pooled_v;
  pa.q_scale = p->q_scale;
  pa.k_scale = p->k_scale;
  pa.v_scale = p->v_scale;
  pa.Hq = p->num_q_heads;
  pa.Hkv = p->num_kv_heads;
  pa.D = D;
  pa.block = b;
  pa.fp8 = p->in_dtype == FP2_FP8_E4M3;
  pa.select_mode = p->select_mode;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_pool(pa, s);
  if (e != hipSuccess) return device_status(e, "pool kernel launch");
  SelectArgs sa{};
  sa.seq = sd;
  sa.qbar = pa.qbar;
  sa.kbar = pooled_k;
  sa.block_idx = block_idx;
  sa.block_cnt = block_cnt;
  sa.Hkv = p->num_kv_heads;
  sa.D = D;
  sa.block = b;
  sa.tau = p->tau;
  sa.rows_per_wg = tq;
  sa.select_mode = p->select_mode;
  sa.Hq = p->num_q_heads;
  e = launch_select(sa, s);
  if (e != hipSuccess) return device_status(e, "select kernel launch");
  if (env_log())
    fprintf(stderr, "[fp2] select B=%d Sq=%d Sk=%d Hq=%d Hkv=%d d=%d b=%d nqb=%d nkb=%d rows/wg=%d tau=%g\n", batch,
            seqlen_q, seqlen_k, p->num_q_heads, p->num_kv_heads, D, b, nqb, nkb, tq, p->tau);
  return ok();
}

static fp2_status attention_common(const fp2_params* p, int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                                   const void* q, const void* k, const void* v, const int32_t* block_idx,
                                   const int32_t* block_cnt, const float* pooled_k, const float* pooled_v,
                                   void* out, float* lse, void* stream, bool sparse) {
  fp2_status st = check_params(p);
  if (st != FP2_OK) return st;
  if ((st = check_lengths(batch, seqlen_q, seqlen_k)) != FP2_OK) return st;
  if (!q || !k || !v || !out) return fail(FP2_EINVAL, "q, k, v and out must be non-NULL");
  const bool corr = sparse && p->mean_correction;
  if (sparse && (!block_idx || !block_cnt)) return fail(FP2_EINVAL, "block_idx and block_cnt must be non-NULL");
  if (corr && (!pooled_k || !pooled_v))
    return fail(FP2_EINVAL, "mean_correction needs pooled_k and pooled_v");
  const int D = p->head_dim, b = p->block_size;
  const int nqb = nq_blocks(seqlen_q, seqlen_k, b);
  const int nkb = nk_blocks(seqlen_k, b);
  if (!attn_lds_ok(D, b, nkb, p->in_dtype == FP2_FP8_E4M3)) return fail(FP2_EUNSUPPORTED, "seqlen_k=%d too long for the attention kernel", seqlen_k);
  AttnArgs a{};
  fill_attn_common(a, p);
  a.seq = SeqDesc{batch, seqlen_q, seqlen_k, nullptr, nullptr, nqb, nkb};
  a.kv = KVDesc{k, v, nullptr, 0, 0};
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.lse_stride = seqlen_q;
  a.block_idx = block_idx;
  a.block_cnt = block_cnt;
  a.kbar = pooled_k;
  a.vbar = pooled_v;
  a.sparse = sparse;
  a.mean_correction = corr;
  a.nqb_grid = nqb;
  a.head_group = sparse ? a.Hkv : dense_head_group(a.Hkv, batch, seqlen_k, D, p->in_dtype == FP2_FP8_E4M3 ? 1 : 2);
  hipError_t e = launch_attention(a, D, b, p->in_dtype == FP2_FP8_E4M3, (hipStream_t)stream);
  if (e != hipSuccess) return device_status(e, "attention kernel launch");
  if (env_log())
    fprintf(stderr, "[fp2] %s attention B=%d Sq=%d Sk=%d Hq=%d Hkv=%d d=%d b=%d parts=%d waves=%d grid=%ld\n",
            sparse ? "sparse" : "dense", batch, seqlen_q, seqlen_k, a.Hq, a.Hkv, D, b, a.parts, a.waves,
            (long)a.Hkv * batch * a.parts * nqb);
  return ok();
}

fp2_status fp2_sparse_prefill(const fp2_params* p, int32_t batch, int32_t seqlen_q, int32_t seqlen_k, const void* q,
                              const void* k, const void* v, const int32_t* block_idx, const int32_t* block_cnt,
                              const float* pooled_k, const float* pooled_v, void* out, float* lse, void* stream) {
  return attention_common(p, batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt, pooled_k, pooled_v, out, lse,
                          stream, true);
}

fp2_status fp2_dense_prefill(const fp2_params* p, int32_t batch, int32_t seqlen_q, int32_t seqlen_k, const void* q,
                             const void* k, const void* v, void* out, float* lse, void* stream) {
  return attention_common(p, batch, seqlen_q, seqlen_k, q, k, v, nullptr, nullptr, nullptr, nullptr, out, lse, stream,
                          false);
}

void fp2_paged_mask_dims(const fp2_params* p, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t* max_nqb,
                         int32_t* max_nkb) {
  int nq = 0, nk = 0;
  if (p && p->block_size > 0 && max_seqlen_q > 0 && max_seqlen_k >= max_seqlen_q) {
    nk = nk_blocks(max_seqlen_k, p->block_size);
    nq = (max_seqlen_q + p->block_size - 1) / p->block_size + 1;
    if (nq > nk) nq = nk;
  }
  if (max_nqb) *max_nqb = nq;
  if (max_nkb) *max_nkb = nk;
}

namespace {
struct PagedLayout {
  size_t qbar, kbar, vbar, idx, cnt, plan, sched, total;
};
PagedLayout paged_layout(const fp2_params* p, int n, int max_nqb, int max_nkb) {
  PagedLayout L{};
  const size_t H = p->num_kv_heads, D = p->head_dim;
  size_t off = 0;
  L.qbar = off;
  const size_t QH = p->select_mode != 0 ? p->num_q_heads : p->num_kv_heads;
  off += align_up((size_t)n * QH * max_nqb * D * 4);
  L.kbar = off;
  off += align_up((size_t)n * H * max_nkb * D * 4);
  L.vbar = off;
  off += align_up((size_t)n * H * max_nkb * D * 4);
  L.idx = off;
  off += align_up((size_t)n * H * max_nqb * max_nkb * 4);
  L.cnt = off;
  off += align_up((size_t)n * H * max_nqb * 4);
  L.plan = off;  // task count, then the work-ordered task list
  off += align_up(16 + (size_t)n * H * max_nqb * 4);
  L.sched = off;  // the attention launch's 8 tile-queue counters, 128 bytes apart
  off += align_up(8 * 128);
  L.total = off;
  return L;
}
}  // namespace

size_t fp2_paged_workspace_size(const fp2_params* p, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k) {
  if (check_params(p) != FP2_OK || check_lengths(num_seqs, max_seqlen_q, max_seqlen_k) != FP2_OK) return 0;
  int nq, nk;
  fp2_paged_mask_dims(p, max_seqlen_q, max_seqlen_k, &nq, &nk);
  return paged_layout(p, num_seqs, nq, nk).total;
}

static fp2_status paged_impl(const fp2_params* p, int32_t num_seqs, const void* q, const int32_t* cu_seqlens_q,
                             const int32_t* seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                             const void* k_cache, const void* v_cache, int32_t num_pages, int32_t page_size,
                             const int32_t* page_table, int32_t max_pages_per_seq, void* out, float* lse,
                             int32_t* block_idx, int32_t* block_cnt, void* workspace, size_t workspace_bytes,
                             void* stream, float* bsum_k, float* bsum_v, const int32_t* cached_blocks) {
  fp2_status st = check_params(p);
  if (st != FP2_OK) return st;
  if ((st = check_lengths(num_seqs, max_seqlen_q, max_seqlen_k)) != FP2_OK) return st;
  if (!q || !cu_seqlens_q || !seqlens_k || !k_cache || !v_cache || !page_table || !out)
    return fail(FP2_EINVAL, "q, cu_seqlens_q, seqlens_k, k_cache, v_cache, page_table and out must be non-NULL");
  if ((block_idx == nullptr) != (block_cnt == nullptr))
    return fail(FP2_EINVAL, "block_idx and block_cnt must be both NULL or both set");
  if (page_size <= 0 || (page_size & (page_size - 1)) || p->block_size % page_size ||
      p->block_size / page_size > 64)
    return fail(FP2_EUNSUPPORTED, "page_size=%d must be a power of two dividing block_size=%d, at least %d",
                page_size, p->block_size, p->block_size / 64);
  if (num_pages <= 0) return fail(FP2_EINVAL, "num_pages=%d must be positive", num_pages);
  const int b = p->block_size, D = p->head_dim;
  if ((long)max_pages_per_seq * page_size < max_seqlen_k)
    return fail(FP2_EINVAL, "max_pages_per_seq=%d * page_size=%d < max_seqlen_k=%d", max_pages_per_seq, page_size,
                max_seqlen_k);
  int max_nqb, max_nkb;
  fp2_paged_mask_dims(p, max_seqlen_q, max_seqlen_k, &max_nqb, &max_nkb);
  const int tq = select_rows_per_wg(D, max_nkb);
  if (tq == 0 || !attn_lds_ok(D, b, max_nkb, p->in_dtype == FP2_FP8_E4M3))
    return fail(FP2_EUNSUPPORTED, "max_seqlen_k=%d too long for this build", max_seqlen_k);
  const PagedLayout L = paged_layout(p, num_seqs, max_nqb, max_nkb);
  if (!workspace || workspace_bytes < L.total)
    return fail(FP2_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, L.total);
  hipStream_t s = (hipStream_t)stream;

  if (env_validate()) {
    std::vector<int32_t> cu(num_seqs + 1), sk(num_seqs), tab((size_t)num_seqs * max_pages_per_seq);
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemcpy(cu.data(), cu_seqlens_q, cu.size() * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(sk.data(), seqlens_k, sk.size() * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(tab.data(), page_table, tab.size() * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return device_status(e, "FP2_VALIDATE copy");
    if (cu[0] != 0) return fail(FP2_EINVAL, "cu_seqlens_q[0]=%d must be 0", cu[0]);
    for (int i = 0; i < num_seqs; ++i) {
      const int lq = cu[i + 1] - cu[i];
      if (lq < 0 || lq > max_seqlen_q || sk[i] < lq || sk[i] > max_seqlen_k || sk[i] <= 0)
        return fail(FP2_EINVAL, "sequence %d: q_len=%d seqlen_k=%d inconsistent with the maxima", i, lq, sk[i]);
      const int npg = (sk[i] + page_size - 1) / page_size;
      for (int pg = 0; pg < npg; ++pg) {
        const int id = tab[(size_t)i * max_pages_per_seq + pg];
        if (id < 0 || id >= num_pages)
          return fail(FP2_EINVAL, "sequence %d page %d: page id %d outside [0, %d)", i, pg, id, num_pages);
      }
    }
  }

  char* ws = (char*)workspace;
  float* qbar = (float*)(ws + L.qbar);
  float* kbar = (float*)(ws + L.kbar);
  float* vbar = (float*)(ws + L.vbar);
  int32_t* idx = block_idx ? block_idx : (int32_t*)(ws + L.idx);
  int32_t* cnt = block_cnt ? block_cnt : (int32_t*)(ws + L.cnt);
  int plog = 0;
  while ((1 << plog) < page_size) ++plog;
  const SeqDesc sd{num_seqs, 0, 0, cu_seqlens_q, seqlens_k, max_nqb, max_nkb};
  const KVDesc kv{k_cache, v_cache, page_table, max_pages_per_seq, plog};

  PoolArgs pa{};
  pa.seq = sd;
  pa.kv = kv;
  pa.q = q;
  pa.qbar = qbar;
  pa.kbar = kbar;
  // the value means (and their cached sums) are needed only by the mean
  // correction; without it the pool kernel reads and writes no V at all
  pa.vbar = p->mean_correction ? vbar : nullptr;
  pa.q_scale = p->q_scale;
  pa.k_scale = p->k_scale;
  pa.v_scale = p->v_scale;
  pa.Hq = p->num_q_heads;
  pa.Hkv = p->num_kv_heads;
  pa.D = D;
  pa.block = b;
  pa.fp8 = p->in_dtype == FP2_FP8_E4M3;
  pa.select_mode = p->select_mode;
  pa.bsum_k = bsum_k;
  pa.bsum_v = bsum_v;
  pa.cached_blocks = cached_blocks;
  hipError_t e = launch_pool(pa, s);
  if (e != hipSuccess) return device_status(e, "pool kernel launch");
  SelectArgs sa{};
  sa.seq = sd;
  sa.qbar = qbar;
  sa.kbar = kbar;
  sa.block_idx = idx;
  sa.block_cnt = cnt;
  sa.Hkv = p->num_kv_heads;
  sa.D = D;
  sa.block = b;
  sa.tau = p->tau;
  sa.rows_per_wg = tq;
  sa.select_mode = p->select_mode;
  sa.Hq = p->num_q_heads;
  e = launch_select(sa, s);
  if (e != hipSuccess) return device_status(e, "select kernel launch");
  PlanArgs pl{};
  pl.seq = sd;
  pl.block_cnt = cnt;
  pl.plan_count = (int32_t*)(ws + L.plan);
  pl.plan = (int32_t*)(ws + L.plan + 16);
  pl.sched = (unsigned*)(ws + L.sched);
  pl.Hkv = p->num_kv_heads;
  pl.block = b;
  pl.mean_correction = p->mean_correction;
  e = launch_plan(pl, s);
  if (e != hipSuccess) return device_status(e, "plan kernel launch");
  AttnArgs a{};
  fill_attn_common(a, p);
  a.plan = pl.plan;
  a.plan_count = pl.plan_count;
  a.sched = pl.sched;
  a.seq = sd;
  a.kv = kv;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.lse_stride = 0;
  a.block_idx = idx;
  a.block_cnt = cnt;
  a.kbar = kbar;
  a.vbar = vbar;
  a.sparse = 1;
  a.head_group = a.Hkv;  // unused: the plan orders paged tiles
  a.mean_correction = p->mean_correction;
  a.nqb_grid = max_nqb;
  e = launch_attention(a, D, b, p->in_dtype == FP2_FP8_E4M3, s);
  if (e != hipSuccess) return device_status(e, "attention kernel launch");
  if (env_log())
    fprintf(stderr, "[fp2] paged n=%d max_sq=%d max_sk=%d page=%d max_nqb=%d max_nkb=%d\n", num_seqs, max_seqlen_q,
            max_seqlen_k, page_size, max_nqb, max_nkb);
  return ok();
}

size_t fp2_workspace_size(const fp2_params* p, int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k) {
  if (check_params(p) != FP2_OK || check_lengths(batch, max_seqlen_q, max_seqlen_k) != FP2_OK) return 0;
  int nq, nk;
  fp2_paged_mask_dims(p, max_seqlen_q, max_seqlen_k, &nq, &nk);
  // the pooled-query region of the paged layout is the select workspace of
  // the largest query-block count any (sq <= max_sq, sk <= max_sk) reaches
  const size_t paged = paged_layout(p, batch, nq, nk).total;
  const size_t qh = p->select_mode != 0 ? p->num_q_heads : p->num_kv_heads;
  const size_t sel = align_up((size_t)batch * qh * nq * p->head_dim * sizeof(float));
  return paged > sel ? paged : sel;
}

fp2_status fp2_sparse_prefill_paged(const fp2_params* p, int32_t num_seqs, const void* q, const int32_t* cu_seqlens_q,
                                    const int32_t* seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    const void* k_cache, const void* v_cache, int32_t num_pages, int32_t page_size,
                                    const int32_t* page_table, int32_t max_pages_per_seq, void* out, float* lse,
                                    int32_t* block_idx, int32_t* block_cnt, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return paged_impl(p, num_seqs, q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k, k_cache, v_cache, num_pages,
                    page_size, page_table, max_pages_per_seq, out, lse, block_idx, block_cnt, workspace,
                    workspace_bytes, stream, nullptr, nullptr, nullptr);
}

fp2_status fp2_sparse_prefill_paged_pooled(const fp2_params* p, int32_t num_seqs, const void* q,
                                           const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                           int32_t max_seqlen_q, int32_t max_seqlen_k, const void* k_cache,
                                           const void* v_cache, int32_t num_pages, int32_t page_size,
                                           const int32_t* page_table, int32_t max_pages_per_seq, void* out,
                                           float* lse, int32_t* block_idx, int32_t* block_cnt, void* workspace,
                                           size_t workspace_bytes, float* block_sums_k, float* block_sums_v,
                                           const int32_t* cached_blocks, void* stream) {
  if (!p) return fail(FP2_EINVAL, "params is NULL");
  if (!block_sums_k || !cached_blocks || (p->mean_correction && !block_sums_v))
    return fail(FP2_EINVAL, "block_sums_k, cached_blocks (and block_sums_v with mean correction) must be non-NULL");
  return paged_impl(p, num_seqs, q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k, k_cache, v_cache, num_pages,
                    page_size, page_table, max_pages_per_seq, out, lse, block_idx, block_cnt, workspace,
                    workspace_bytes, stream, block_sums_k, p->mean_correction ? block_sums_v : nullptr,
                    cached_blocks);
}

const char* fp2_status_string(fp2_status s) {
  switch (s) {
    case FP2_OK: return "FP2_OK";
    case FP2_EINVAL: return "FP2_EINVAL";
    case FP2_EUNSUPPORTED: return "FP2_EUNSUPPORTED";
    case FP2_EWORKSPACE: return "FP2_EWORKSPACE";
    case FP2_EDEVICE: return "FP2_EDEVICE";
  }
  return "FP2_UNKNOWN";
}

const char* fp2_last_error(void) { return g_err.c_str(); }

const char* fp2_version(void) { return "fp2-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
