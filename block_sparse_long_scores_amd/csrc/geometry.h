// Per-sequence block geometry and K/V row addressing, device side.
#pragma once

#include "fp2_device.h"
#include "fp2_internal.h"

namespace fp2 {

// Blocks are numbered by absolute position.  Query row r of a sequence sits at
// position P + r with P = Sk - Sq (a chunked prefill when P > 0).
struct SeqGeo {
  int Sq, Sk, P;
  int first_qb;  // absolute index of the first query block touched
  int nqb;       // query blocks touched
  int nkb;       // key blocks
  int qrow0;     // first row of this sequence in q / out
};

__device__ __forceinline__ SeqGeo seq_geo(const SeqDesc& d, int s, int block) {
  SeqGeo g;
  if (d.cu_seqlens_q) {
    int a = d.cu_seqlens_q[s];
    int b = d.cu_seqlens_q[s + 1];
    g.Sq = b - a;
    g.qrow0 = a;
    g.Sk = d.seqlens_k[s];
  } else {
    g.Sq = d.seqlen_q;
    g.Sk = d.seqlen_k;
    g.qrow0 = s * d.seqlen_q;
  }
  g.P = g.Sk - g.Sq;
  g.first_qb = g.P / block;
  g.nqb = g.Sq > 0 ? (g.Sk - 1) / block - g.first_qb + 1 : 0;
  g.nkb = (g.Sk + block - 1) / block;
  return g;
}

// Byte address of key/value row c (all heads) of sequence s.
__device__ __forceinline__ const char* kv_row(const KVDesc& kv, const void* base, int s,
                                              int seqlen_k_contig, int c, int rowbytes) {
  if (kv.page_table) {
    int pg = kv.page_table[(long)s * kv.max_pages + (c >> kv.page_log2)];
    long row = ((long)pg << kv.page_log2) + (c & ((1 << kv.page_log2) - 1));
    return (const char*)base + row * rowbytes;
  }
  return (const char*)base + ((long)s * seqlen_k_contig + c) * (long)rowbytes;
}

}  // namespace fp2
