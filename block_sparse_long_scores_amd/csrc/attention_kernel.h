// Block-sparse (and dense) causal prefill attention with mean correction, gfx950.
// The kernel template; attention_bf16.hip and attention_fp8.hip instantiate it.
//
// Source: "FlashPrefill V2: block-sparse prefill attention for long-context LLM
// serving", abstract (sparse attention operator with PackGQA memory access,
// FP8, paged KV cache, mean correction term), and the papers.ananclaw.com
// explainer §2.1 (query block q computes only Supp(q); Out_q^V2 adds the
// dropped blocks' mass through mu_q and their average value) and §2.2
// (PackGQA).  The pages' kernel targets Hopper (warp specialization, pingpong);
// this one is laid out for CDNA4 instead:
//
//  * One workgroup per (sequence, KV head h, query block i, part): its 4
//    wavefronts hold 256 of the G query heads x b rows of the GQA group, 64
//    packed query rows per wave (PackGQA: every query head of the group reads
//    the same K/V tile from LDS; a 512-row group takes two workgroups, which
//    land on the same XCD and share its L2).
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys on the M side, queries on
//    the N side, so each lane owns 2 query columns and the row max / row sum
//    of the online softmax are lane-local plus one permlane32 exchange.
//  * The accumulator registers of S^T, in order, are the B-operand slots of
//    the P V MFMA (4 consecutive keys per half-slot), so P^T feeds
//    v_mfma_f32_32x32x16_bf16 straight from registers; O^T = V^T P^T
//    accumulates in the AGPR file.  The V^T operand comes from
//    ds_read_b64_tr_b16 (LDS transpose read: 4 consecutive keys of one d per
//    lane) on the natural [key][d] tile.
//  * K and V both travel HBM -> LDS with global_load_lds_dwordx4 (no register
//    staging), double-buffered: block n+1 streams in while block n is
//    computed.  LDS rows are padded (row + 32 B for d = 128) so that the
//    operand reads are bank-conflict-free and every operand address is one
//    base register plus a compile-time offset.
//  * Softmax in the log2 domain against a fixed per-row reference m: before
//    the block loop each query row takes the max of its logits over the first
//    32 keys of its first kept block (the sink block) plus kRefMargin.  The
//    loop then needs one FMA, one exp2, one add and half a convert per score
//    and never rescales the AGPR-resident O^T.  m is at most kRefMargin above
//    the row's true max, so the largest term keeps full precision; a row whose
//    normaliser reaches 2^kRefOverflow (a logit ~80 nats above the sink chunk)
//    makes the workgroup recompute the tile with m moved up by log2 of that
//    normaliser, which bounds every term by 1 (exact, just slower).
//  * Mean correction: after the kept blocks, the dropped blocks of the row
//    (the complement of the kept list in [0, i)) are processed 32 at a time
//    as pseudo-keys: K row = kbar_j, V row = vbar_j (bf16 in LDS), logit bias
//    log2(n_j), no causal mask (dropped blocks lie strictly before i).
#pragma once

#include "fp2_device.h"
#include "fp2_internal.h"
#include "geometry.h"

#include <atomic>
#include <map>
#include <mutex>
#include <thread>
#include <tuple>
#include <type_traits>
#include <utility>

namespace fp2 {
namespace {  // internal: every precision's translation unit has its own copy

constexpr int kRowsPerWave = 64;
constexpr int kRowsPerPart = 256;
constexpr int NT = kRowsPerWave / 32;  // 32-query column groups per wave
constexpr float kRefMargin = 16.0f;     // log2 units above the sink-chunk max
constexpr float kRefOverflow = 100.0f;  // log2 units above the reference that force a rerun
// Passes of a tile (see the rerun rule at the end of attn_tile): a row whose
// normaliser overflowed is searched for (steps doubling from 128 log2 units,
// then bisected), which reaches logits up to ~8e6 log2 units above the first
// reference within 32 passes; a row still unresolved after the last pass is
// written as NaN.
constexpr int kMaxPasses = 32;
constexpr float kFirstStep = 128.0f;
// A normaliser below 2^-kRefUnder after a step up means the reference
// overshot: its largest terms sit near fp32's denormal range and lose
// precision (the first pass's normaliser is at least 2^-kRefMargin).
constexpr float kRefUnder = 60.0f;
// fp8 P codes: the e4m3 code of 2^x is taken as RNE(8 (x + 7) - kCodeShift),
// the exponent-and-mantissa bits read as one fixed-point number of x + 7
// (a log-linear, Mitchell-style approximation of 2^x: the mantissa is
// linear in the fraction of x).  The shift centres its error: the decoded
// code is within a factor exp(+-0.0728) of 2^x over the normal range.
constexpr float kCodeShift = 0.34f;
// The code c is converted two scores at a time as the unorm16 fraction
// (256 c + 127.5) / 65535: the high byte of round(65535 y) is then c rounded
// to nearest, and one byte permute gathers four such high bytes into the
// packed P operand (two packed converts and a permute per four scores, in
// place of four single-byte converts).
constexpr float kU16 = 256.0f / 65535.0f;
constexpr float kU16Half = 127.5f / 65535.0f;

template <int D, int BLK, bool F8>
struct Cfg {
  static constexpr int ESZ = F8 ? 1 : 2;       // bytes per K/V element
  static constexpr int KS = D / 16;            // k-steps of a bf16 QK chain (32x32x16)
  static constexpr int KS8 = D / 64;           // k-steps of an fp8 QK chain (32x32x64)
  static constexpr int MT = D / 32;            // 32-row tiles of O^T along d
  static constexpr int KC = BLK / 32;          // 32-key chunks per block
  static constexpr int NSC = BLK / 64;         // 64-key superchunks per block (fp8 P V)
  static constexpr int ROWB = D * ESZ;         // bytes of one K/V row of one head
  // LDS row stride: rows are padded so that the rows read by one LDS read
  // phase (consecutive rows for the K operand, the 4/8-key groups of the
  // transpose reads for V) land on distinct banks.
  static constexpr int RS = F8 ? ROWB + 16 : ROWB + (D == 128 ? 32 : 16);
  static constexpr int TILE = ((BLK * RS + 1023) / 1024) * 1024;  // one K or V tile
  static constexpr int NLD = TILE / 1024;      // global_load_lds wave ops per tile
  static constexpr int RS16 = 2 * D + (D == 128 ? 32 : 16);  // bf16 pseudo-key rows
  static constexpr int PSB = BLK * RS16;       // one pseudo-key tile of BLK rows (bf16)
  static constexpr int NPW = (NLD + 3) / 4;    // copy ops per wave and tile with 4 waves
  static constexpr int NPWP = (NPW + 3) & ~3;  // table entries per thread (16-byte rows)
  static constexpr int DTAB = NPWP * 256 * 4;  // LDS bytes of the copy-offset table
};

// LDS bytes of the correction phase: pseudo-K and pseudo-V tiles, the
// dropped count, the kept-block bitmap and the dropped-block list.
template <int D, int BLK, bool F8>
__host__ __device__ constexpr int corr_lds_bytes(int nkb) {
  return 2 * Cfg<D, BLK, F8>::PSB + 4 + 4 * ((nkb + 31) / 32) + 4 * nkb;
}

// fp8 S^T chunk (32 keys x 32 queries, K on the A side) as a chain of
// v_mfma_f32_32x32x64_f8f6f4 (e4m3 A and B, no block scale) with the
// accumulator in VGPRs, where the softmax reads it (a compiler-placed result
// would land in AGPRs next to the O^T accumulators and need a copy per
// register).  Hazards the compiler cannot see through the asm are covered
// inside it: 2 wait states before the first MFMA (VALU write -> MFMA source
// read) and 20 after the last (16-pass MFMA result -> VALU access).
__device__ __forceinline__ f32x16 qk8_chain(const i32x8 (&k)[2], const i32x8 (&q)[2]) {
  f32x16 S;
  asm("s_nop 1\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %0, %1, %3, 0\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %0, %2, %4, %0\n\t"
      "s_nop 15\n\t"
      "s_nop 3"
      : "=&v"(S)
      : "v"(k[0]), "v"(k[1]), "v"(q[0]), "v"(q[1]));
  return S;
}

__device__ __forceinline__ f32x16 qk8_chain(const i32x8 (&k)[1], const i32x8 (&q)[1]) {
  f32x16 S;
  asm("s_nop 1\n\t"
      "v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0\n\t"
      "s_nop 15\n\t"
      "s_nop 3"
      : "=&v"(S)
      : "v"(k[0]), "v"(q[0]));
  return S;
}

// The same chain split into one asm statement per MFMA, so that the
// compiler can issue independent VALU work between them: the first writes
// S (C = 0), the last accumulates into it.  Nothing may touch S between the
// two (the second MFMA reads it as its exactly overlapping accumulator,
// which needs no wait states).
__device__ __forceinline__ void qk8_first(f32x16& S, const i32x8& k, const i32x8& q) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(S) : "v"(k), "v"(q));
}
// The last MFMA of a chain in the pipelined stages, whose S the VALU first
// reads at least 14 instructions later (the rest of the stage's last slot,
// the next stage's operand reads, and a slot with an MFMA and a max-tree
// piece): the 8 wait states here make up the 19 that a 16-pass MFMA result
// needs before a VALU read.
__device__ __forceinline__ void qk8_last(f32x16& S, const i32x8& k, const i32x8& q) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\ts_nop 7"
               : "+v"(S)
               : "v"(k), "v"(q));
}

// LDS transpose reads.  The K/V tiles a block reads were completed by an
// explicit s_waitcnt + barrier at the start of that block, while the copies
// in flight during it fill the other buffer.  The restrict-qualified pointer
// gives the read alias-scope information after inlining, which keeps the
// compiler from waiting on those in-flight LDS-DMA copies before each read
// (plain LDS loads carry type-based alias information and are not held).
__device__ __forceinline__ i16x4 lds_read_tr16(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)p);
}

__device__ __forceinline__ u32x4 lds_read_u32x4(const unsigned* __restrict__ p) { return *(const u32x4*)p; }

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// One tile: the G*b packed query rows of (sequence, KV head, query block) or
// the 256-row part `part` of them, over its kept key blocks (or all blocks
// j <= i when dense), then the mean correction and the epilogue.  PG: a
// paged launch (K/V rows through the page table, tiles in the plan's work
// order); contiguous launches get an instance without any of the page-table
// code, which leaves their block loop shorter and their registers freer.
template <int D, int BLK, bool F8, bool PG>
__device__ __forceinline__ void attn_tile(const AttnArgs& a, const int q, const int pos, char* smem) {
  using C = Cfg<D, BLK, F8>;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nwaves = nthr >> 6;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int l32 = lane & 31;

  // ---- tile (q, pos): position pos of queue q (see attn_kernel).
  //  Without a plan, tile t = 8*pos + q: the KV heads go in groups of
  //  head_group (all heads at once in sparse launches), and within a group
  //  query blocks go from the last (longest) down; the G2 =
  //  head_group*batch*parts tiles of one query block are rotated by the
  //  query-block rank, so that queue t % 8 serves every head of the group in
  //  turn (kept-block counts differ between heads) while the parts of one
  //  tile share a queue.
  //  With a plan: task k = 8*(pos / parts) + q of the work-ordered list,
  //  part pos % parts.
  int h, s, part, il;
  if constexpr (PG) {
    part = pos % a.parts;
    const int task = a.plan[8 * (pos / a.parts) + q];
    const int per_seq = a.Hkv * a.seq.nqb_stride;
    s = task / per_seq;
    const int r = task - s * per_seq;
    h = r / a.seq.nqb_stride;
    il = r - h * a.seq.nqb_stride;
  } else {
    const int HG = a.head_group;
    const int G2 = HG * a.seq.batch * a.parts;
    const int per_group = G2 * a.nqb_grid;
    const int tile0 = 8 * pos + q;
    const int grp = tile0 / per_group;
    const int tile = tile0 - grp * per_group;
    const int rank = tile / G2;
    int t = (tile - rank * G2 + rank) % G2;
    h = grp * HG + t % HG;
    t /= HG;
    s = t % a.seq.batch;
    t /= a.seq.batch;
    part = t;
    il = a.nqb_grid - 1 - rank;
  }
  const SeqGeo g = seq_geo(a.seq, s, BLK);
  if (il < 0 || il >= g.nqb) return;
  const int i = g.first_qb + il;
  const int G = a.G;
  const int pr0 = part * kRowsPerPart + wave * kRowsPerWave;

  // query column nt of this lane: packed row pr = pr0 + l32 + 32*nt, i.e.
  // query head h*G + pr/BLK, row pr%BLK of block i.
  auto qinfo = [&](int nt, int& rb, long& off) __attribute__((always_inline)) -> bool {
    const int pr = pr0 + l32 + 32 * nt;
    const int gq = pr / BLK;
    rb = pr - gq * BLK;
    const int r = i * BLK + rb - g.P;
    off = ((long)(g.qrow0 + r) * a.Hq + (h * G + gq)) * D;
    return (pr < G * BLK) && r >= 0 && r < g.Sq;
  };

  // Q operands (B side of S^T) and the log2-domain scale of a raw score.
  //  bf16: k-step ks of lane (n, hh) holds d in [16ks + 8hh, +8).
  //  fp8:  k-step ks of lane (n, hh) holds d in [64ks + 32hh, +32) (the
  //        32x32x64 MFMA pairs byte e of A lane (x, hh) with byte e of B
  //        lane (n, hh)); a raw score is in code units and takes the
  //        per-head dequantization scales q_s * k_s.
  using QT = typename std::conditional<F8, i32x8, bf16x8>::type;
  constexpr int QKS = F8 ? C::KS8 : C::KS;
  int rib[NT];
  float cs[NT];
  QT qop[NT][QKS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    long off;
    const bool ok = qinfo(nt, rib[nt], off);
    if constexpr (F8) {
      const unsigned char* qp = (const unsigned char*)a.q + off + 32 * hh;
#pragma unroll
      for (int ks = 0; ks < QKS; ++ks) {
        if (ok) {
          const i32x4 lo = *(const i32x4*)(qp + 64 * ks);
          const i32x4 hi = *(const i32x4*)(qp + 64 * ks + 16);
          qop[nt][ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          qop[nt][ks] = i32x8{};
        }
      }
      const int gq = (pr0 + l32 + 32 * nt) / BLK;
      cs[nt] = ok ? a.scale_log2 * a.q_scale[h * G + gq] * a.k_scale[h] : a.scale_log2;
    } else {
#pragma unroll
      for (int ks = 0; ks < QKS; ++ks) {
        if (ok) {
          qop[nt][ks] = *(const bf16x8*)((const __bf16*)a.q + off + 16 * ks + 8 * hh);
        } else {
          qop[nt][ks] = bf16x8{};
        }
      }
      cs[nt] = a.scale_log2;
    }
  }

  f32x16 O[C::MT][NT];
  f32x16 Lacc[F8 ? NT : 1];  // fp8: row sums of P, accumulated by MFMA
  float mref[NT], lsum[NT];
  // fp8: 8 * logit scale and 112 - kCodeShift - 8 * mref (the code offset
  // of the pass's reference, before the superchunk's 8 fx), both in unorm16
  // units (times kU16, the offset plus kU16Half); the largest superchunk maximum above mref (log2 units)
  // seen in the pass, which sets the exact reference of a rerun.
  float cs8[F8 ? NT : 1], base8[F8 ? NT : 1], rmax[F8 ? NT : 1];
  // rerun search step per row (log2 units; negative once bracketed)
  float rstep[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) rstep[nt] = kFirstStep;
  if constexpr (F8) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) cs8[nt] = (8.f * kU16) * cs[nt];
  }

  // LDS: K tiles at [0, 2*TILE), V tiles at [2*TILE, 4*TILE) (double buffer)
  char* const lds = smem;
  const int rowbytes = a.Hkv * C::ROWB;
  const int Skm1 = g.Sk - 1;
  const int plog = a.kv.page_log2;
  const int* ptab = PG ? a.kv.page_table + (long)s * a.kv.max_pages : nullptr;
  // true in the paged instance as a constant (the entry point rejects a NULL
  // table), the pointer test in the contiguous one (where it folds away)
  const bool paged = PG ? true : ptab != nullptr;

  // Paged caches: page ids of key block j, lane i holding the id of its i-th
  // page (a block spans BLK / page_size <= 64 pages; page_size divides BLK).
  // The page-table branches below test `paged`, a constant in the paged
  // instance: a run-time test of the pointer left a branch around every
  // page-id read, and the wait the compiler puts before a read of freshly
  // loaded ids was then repeated after each copy pair (both paths of each
  // branch merge), so the first block of a tile was issued one copy round
  // trip at a time.
  // They are loaded one block ahead of the K/V copies that use them, so that
  // no copy address waits on a load (vmcnt drains in order: a wait for the
  // page table would also wait for every copy already in flight).
  auto load_pids = [&](int j) __attribute__((always_inline)) -> int {
    if (!paged) return 0;
    const int p0 = (j * BLK) >> plog;
    const int npg = max(1, BLK >> plog);
    return lane < npg ? ptab[min(p0 + lane, Skm1 >> plog)] : 0;
  };

  // K and V tile of key block j -> LDS buffer bb (async, global_load_lds).
  // Wave op `it` (it = wave, wave + nwaves, ...) fills tile bytes [1024*it,
  // 1024*it + 1024) with 16 bytes per lane: lane bytes o = 1024*it + 16*lane
  // fall in row o / RS at byte o % RS; bytes in a row pad (or past the last
  // row) reload chunk 0 of a valid row.  The (row, byte) pair of each lane is
  // advanced by a fixed step per op instead of being divided out; the copy
  // address is a wave-uniform block base plus a 32-bit lane offset; rows past
  // the last key reload the last key.  The copies go through a cursor
  // (dma_begin, then dma_step per op); run_tile can advance it by `dq` ops
  // per chunk (0 everywhere now: interleaving the copies of the next block
  // with the compute measured slower than issuing them before it).
  const int step = 1024 * nwaves;
  const int drow = step / C::RS, dbyte = step - drow * C::RS;
  const int o0 = 1024 * wave + 16 * lane;
  const int row0 = o0 / C::RS, byte0 = o0 - row0 * C::RS;
  int dq_it = C::NLD, dq_row = 0, dq_byte = 0, dq_kb0 = 0, dq_rlast = 0, dq_bb = 0, dq_pids = 0;
  const char* dq_kp = nullptr;
  const char* dq_vp = nullptr;
  auto dma_begin = [&](int j, int bb, int pids) __attribute__((always_inline)) {
    dq_kb0 = j * BLK;
    dq_rlast = min(Skm1 - dq_kb0, BLK - 1);  // last row holding a key of this block
    dq_row = row0;
    dq_byte = byte0;
    dq_it = wave;
    dq_bb = bb;
    dq_pids = pids;
    const long b0 = paged ? (long)h * C::ROWB : ((long)s * a.seq.seqlen_k + dq_kb0) * rowbytes + h * C::ROWB;
    dq_kp = (const char*)a.kv.k + b0;
    dq_vp = (const char*)a.kv.v + b0;
  };
  auto dma_step = [&]() __attribute__((always_inline)) {
    if (dq_it >= C::NLD) return;
    const bool inrow = dq_byte < C::ROWB && dq_row <= dq_rlast;
    long off;
    if (!paged) {
      off = (unsigned)(min(dq_row, dq_rlast) * rowbytes + (inrow ? dq_byte : 0));
    } else {
      const int key = dq_kb0 + min(dq_row, dq_rlast);
      const int pg = __builtin_amdgcn_ds_bpermute(((key >> plog) - (dq_kb0 >> plog)) << 2, dq_pids);
      off = (((long)pg << plog) + (key & ((1 << plog) - 1))) * rowbytes + (inrow ? dq_byte : 0);
    }
    __builtin_amdgcn_global_load_lds((const void*)(dq_kp + off), (lds_void*)(lds + dq_bb * C::TILE + dq_it * 1024),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(dq_vp + off),
                                     (lds_void*)(lds + (2 + dq_bb) * C::TILE + dq_it * 1024), 16, 0, 0);
    dq_it += nwaves;
    dq_row += drow;
    dq_byte += dbyte;
    if (dq_byte >= C::RS) {
      dq_byte -= C::RS;
      dq_row += 1;
    }
  };
  auto dma_some = [&](int n) __attribute__((always_inline)) {
    for (int k = 0; k < n; ++k) dma_step();
  };
  auto dma_rest = [&]() __attribute__((always_inline)) {
    while (dq_it < C::NLD) dma_step();
  };
  // With 4 waves, the lane offsets of a wave's copies are the same for every
  // full key block, relative to the block's first row (contiguous caches) or
  // to the first row of the page that holds the op (paged caches whose pages
  // fill a whole number of 1 KB copy ops in LDS, so that no op straddles two
  // pages).  They are computed once per tile into an LDS table (thread tid's
  // entries at dtab[NPWP tid, +NPWP), read back with 16-byte loads before the
  // first copy is issued) and each copy of a full block is a wave-uniform base
  // plus that 32-bit offset.  Other paged layouts and a sequence's last,
  // partial block take the cursor above.  Copy op k of the wave exists for
  // every wave when k < NLD / 4.
  const bool dfast = nwaves == 4 && (!paged || ((C::RS << plog) & 1023) == 0);
  const int rowmask = paged ? (1 << plog) - 1 : BLK - 1;
  unsigned* const dtab = (unsigned*)(smem + a.lds_dtab) + C::NPWP * tid;
  if (dfast) {
#pragma unroll
    for (int k = 0; k < C::NPW; ++k) {
      const int it = wave + 4 * k;
      if (k < C::NLD / 4 || it < C::NLD) {
        const int o = 1024 * it + 16 * lane;
        const int row = o / C::RS, byte = o - row * C::RS;
        const bool inrow = byte < C::ROWB && row < BLK;
        dtab[k] = (unsigned)((min(row, BLK - 1) & rowmask) * rowbytes + (inrow ? byte : 0));
      }
    }
  }
  auto issue_fast = [&](int j, int bb, int pids) __attribute__((always_inline)) {
    const long b0 = paged ? (long)h * C::ROWB : ((long)s * a.seq.seqlen_k + (long)j * BLK) * rowbytes + h * C::ROWB;
    u32x4 offv[C::NPWP / 4];
#pragma unroll
    for (int r = 0; r < C::NPWP / 4; ++r) offv[r] = lds_read_u32x4(dtab + 4 * r);
#pragma unroll
    for (int k = 0; k < C::NPW; ++k) {
      const int it = wave + 4 * k;
      if (k < C::NLD / 4 || it < C::NLD) {
        long pb = b0;
        if (paged) {  // page of the op's first row (every row of the op is in it)
          const int pi = min((1024 * it) / C::RS, BLK - 1) >> plog;
          pb += ((long)__builtin_amdgcn_readlane(pids, pi) << plog) * rowbytes;
        }
        const unsigned off = offv[k >> 2][k & 3];
        __builtin_amdgcn_global_load_lds((const void*)((const char*)a.kv.k + pb + off),
                                         (lds_void*)(lds + bb * C::TILE + it * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)((const char*)a.kv.v + pb + off),
                                         (lds_void*)(lds + (2 + bb) * C::TILE + it * 1024), 16, 0, 0);
      }
    }
  };
  auto issue_load = [&](int j, int bb, int pids) __attribute__((always_inline)) {
    if (dfast && (j + 1) * BLK <= g.Sk) {
      issue_fast(j, bb, pids);
    } else {
      dma_begin(j, bb, pids);
      dma_rest();
    }
  };

  // ===================== bf16 operand path (32x32x16 MFMA) =================
  // Used for the bf16 K/V tiles and, in both precisions, for the bf16
  // pseudo-key tiles of the mean correction (row stride RS16).
  //  K (A side of S^T): row l32 of the chunk; the d-range of k-step ks
  //  matches the Q operand: bf16 Q [16ks + 8hh, +8); fp8 Q converted to bf16
  //  [64(ks/4) + 32hh + 8(ks%4), +8).
  //  V (A side of O^T, transpose read): group g = lane/16 reads rows
  //  K0 + (lane%16)/4 at d = 32*mt + 16*(g%2) + 4*(lane%4), K0 = 16*ks2 +
  //  8*sec + 4*hh within the chunk.
  const int koff16 = l32 * C::RS16 + (F8 ? 64 : 16) * hh;
  const int voff16 = (4 * hh + ((lane & 15) >> 2)) * C::RS16 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  auto kofs16 = [](int ks) constexpr -> int { return F8 ? 128 * (ks >> 2) + 16 * (ks & 3) : 32 * ks; };

  auto load_kop = [&](const char* kt, int kc, bf16x8 (&kop)[C::KS]) __attribute__((always_inline)) {
    const char* kb = kt + kc * 32 * C::RS16 + koff16;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kop[ks] = *(const bf16x8*)(kb + kofs16(ks));
  };
  auto load_vop = [&](const char* vt, int kc, bf16x8 (&vop)[C::MT][2]) __attribute__((always_inline)) {
    const char* vb = vt + kc * 32 * C::RS16 + voff16;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const i16x4 v0 = lds_read_tr16(vb + 64 * mt + 16 * ks2 * C::RS16);
        const i16x4 v1 = lds_read_tr16(vb + 64 * mt + (16 * ks2 + 8) * C::RS16);
        vop[mt][ks2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  auto qk = [&](const bf16x8 (&kop)[C::KS], const bf16x8 (&qq)[C::KS]) __attribute__((always_inline)) -> f32x16 {
    f32x16 S = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qq[ks], S, 0, 0, 0);
    return S;
  };
  auto pv = [&](const bf16x8 (&vop)[C::MT][2], const bf16x8 (&pk)[2], int nt) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
        O[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[mt][ks2], pk[ks2], O[mt][nt], 0, 0, 0);
  };

  // Interleave hint for one pipeline stage: nmfma MFMAs, each followed by a
  // slice of the stage's VALU work (the softmax of the other column set).
  auto interleave = [&](int nmfma, auto nvalu) __attribute__((always_inline)) {
    for (int k = 0; k < nmfma; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(nvalu)::value, 0);  // VALU
    }
  };
  // The same for the bf16 chunk stages, with the stage's LDS operand reads
  // placed first (they feed the next chunk's QK or P V) and each MFMA
  // followed by one exp (a transcendental, its own scheduling class) and
  // NV other VALU ops, which keeps every gap between MFMAs under one MFMA's
  // issue time.
  auto interleave2 = [&](auto nds, int nmfma, auto nv) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, decltype(nds)::value, 0);  // DS read
    for (int k = 0; k < nmfma; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x402, decltype(nv)::value, 0);  // VALU or TRANS
    }
  };
  using V4 = std::integral_constant<int, 4>;
  using V8 = std::integral_constant<int, 8>;
  using V5 = std::integral_constant<int, 5>;
  using V16 = std::integral_constant<int, 16>;

  // One pipeline stage, written in issue order: the P V MFMAs of one column
  // set first (operands in registers), then the QK chain of the next chunk
  // (its K operand, read at the start of the chunk, arrives meanwhile); after
  // every MFMA slot the softmax of the next score(s) of the other column set
  // (fma, exp2, add; every second score the bf16 pair convert), so that each
  // gap between MFMAs holds a few VALU ops that issue under the MFMA in
  // flight.  Scores are tied to slots statically, whether or not the slot's
  // MFMA exists in this stage.  mode 0: plain; 1: diagonal block (causal
  // mask); 2: pseudo-keys (slots >= nvalid masked).  Key-in-chunk of
  // accumulator register r: 8*(r/4) + 4*hh + r%4.
  auto stage_mix = [&](const f32x16& Sin, int nts, int kc, int mode, int nvalid, float bias, bf16x8 (&pk)[2],
                       bool pv_on, const bf16x8 (&vv)[C::MT][2], const bf16x8 (&pp)[2], int ntp, bool qk_on,
                       const bf16x8 (&kk)[C::KS], const bf16x8 (&qs)[C::KS], f32x16& Sout)
      __attribute__((always_inline)) {
    constexpr int NPV = 2 * C::MT, NSLOT = NPV + C::KS, PER = 16 / NSLOT;
    const float mb = mref[nts] - bias;
    const float sc = F8 ? cs[nts] : a.scale_log2;
    float sum = 0.f;
    float ph[16];
#pragma unroll
    for (int g = 0; g < NSLOT; ++g) {
      if (g < NPV) {
        if (pv_on) O[g >> 1][ntp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[g >> 1][g & 1], pp[g & 1], O[g >> 1][ntp], 0, 0, 0);
      } else if (qk_on) {
        Sout = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[g - NPV], qs[g - NPV], g == NPV ? f32x16{} : Sout, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int r = g * PER + e;
        const int kic = 8 * (r >> 2) + 4 * hh + (r & 3);
        float x = __builtin_fmaf(Sin[r], sc, -mb);
        if (mode == 1 && kc * 32 + kic > rib[nts]) x = -INFINITY;
        if (mode == 2 && kc * 32 + kic >= nvalid) x = -INFINITY;
        ph[r] = __builtin_amdgcn_exp2f(x);
        sum += ph[r];
        if (r & 1) {
          pk[r >> 3][(r & 7) - 1] = (__bf16)ph[r - 1];
          pk[r >> 3][r & 7] = (__bf16)ph[r];
        }
      }
    }
    lsum[nts] += sum;
  };

  // The NCH 32-key chunks of one bf16 K/V tile (or of one pseudo-key tile),
  // software-pipelined in two stages per chunk c:
  //   stage 1: PV(c-1, columns 1), QK(c+1, columns 0)  ||  softmax(S_c, columns 0)
  //   stage 2: PV(c, columns 0), QK(c+1, columns 1)    ||  softmax(S_c, columns 1)
  // so the exp/sum/convert VALU work of one column set runs under the MFMAs of
  // the other; PV(last, columns 1) closes the tile.  Operand buffers are
  // indexed by chunk parity (no register copies after unrolling), and the
  // tile base offsets go through readfirstlane so every LDS operand address
  // is one base register plus a 16-bit immediate.
  auto run_tile = [&](const char* kt, const char* vt, int nch, int mode, int nvalid, float bias,
                      const bf16x8 (&qq)[NT][C::KS], int dq) __attribute__((always_inline)) {
    const int kbo = __builtin_amdgcn_readfirstlane((int)(kt - lds));
    const int vbo = __builtin_amdgcn_readfirstlane((int)(vt - lds));
    const char* kbase = lds + kbo;
    const char* vbase = lds + vbo;
    bf16x8 kop[C::KS];
    bf16x8 vop[2][C::MT][2];
    bf16x8 p0[2], p1[2][2];
    f32x16 S[2][2];
    load_kop(kbase, 0, kop);
    load_vop(vbase, 0, vop[0]);
    S[0][0] = qk(kop, qq[0]);
    S[0][1] = qk(kop, qq[1]);
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
      if (c >= nch) break;
      const int cp = c & 1, np = cp ^ 1;
      const bool more = c + 1 < nch;
      if (more) load_kop(kbase, c + 1, kop);
      dma_some(dq);
      // stage 1
      stage_mix(S[cp][0], 0, c, mode, nvalid, bias, p0, c > 0, vop[np], p1[np], 1, more, kop, qq[0], S[np][0]);
      interleave2(std::integral_constant<int, C::KS>{}, (c > 0 ? 2 * C::MT : 0) + (more ? C::KS : 0), V4{});
      __builtin_amdgcn_sched_barrier(0);
      // stage 2
      if (more) load_vop(vbase, c + 1, vop[np]);
      stage_mix(S[cp][1], 1, c, mode, nvalid, bias, p1[cp], true, vop[cp], p0, 0, more, kop, qq[1], S[np][1]);
      interleave2(std::integral_constant<int, 4 * C::MT>{}, 2 * C::MT + (more ? C::KS : 0), V4{});
      __builtin_amdgcn_sched_barrier(0);
    }
    const int lp = (nch - 1) & 1;
    pv(vop[lp], p1[lp], 1);
  };

  // ===================== fp8 operand path (32x32x64 MFMA) ==================
  //  K (A side of S^T): lane (x, hh) reads 32 bytes of key row x at d =
  //  64ks + 32hh, matching the Q operand.
  //  P^T (B side of O^T): for a 64-key superchunk, bytes 0..15 of lane (n,
  //  hh) are the accumulator registers of its first 32-key chunk, bytes
  //  16..31 those of the second, i.e. byte e is key 32(e/16) + 8((e%16)/4) +
  //  4hh + e%4.  The MFMA's k-block 0 (bytes 0..15 of both lane halves) is
  //  thus exactly the first chunk and k-block 1 the second, and the E8M0
  //  scale of k-block kb of column n is read from lane n + 32kb: P is stored
  //  per (query, superchunk) as P' = P * 2^-b with b chosen from the
  //  superchunk's max, so that P' lies in [128, 256) at the max, and 2^b is
  //  applied inside the MFMA (no fp8 overflow, full e4m3 precision for the
  //  largest terms; both k-blocks carry the same scale byte).
  //  V^T (A side of O^T): ds_read_b64_tr_b8 returns to lane i of a 16-lane
  //  group byte e = byte i%8 of the row addressed by source lane 2e + i/8, so
  //  source lanes 2e, 2e+1 address the same key (the P byte order above) at d
  //  and d + 8; four reads (+16 keys each) fill the 32 bytes.
  const int koff8 = l32 * C::RS + 32 * hh;
  const int L16 = lane & 15;
  const int voff8 = (8 * (L16 >> 3) + 4 * hh + ((L16 >> 1) & 3)) * C::RS + 16 * ((lane >> 4) & 1) + 8 * (L16 & 1);
  auto load_kop8 = [&](const char* kt, int kc, i32x8 (&kop)[C::KS8]) __attribute__((always_inline)) {
    const char* kb = kt + kc * 32 * C::RS + koff8;
#pragma unroll
    for (int ks = 0; ks < C::KS8; ++ks) {
      const i32x4 lo = *(const i32x4*)(kb + 64 * ks);
      const i32x4 hi = *(const i32x4*)(kb + 64 * ks + 16);
      kop[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto load_vop8 = [&](const char* vt, int sc, i32x8 (&vop)[C::MT]) __attribute__((always_inline)) {
    const char* vb = vt + sc * 64 * C::RS + voff8;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      i32x2 r[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
        r[t4] = lds_read_tr8(vb + 32 * mt + 16 * t4 * C::RS);
      vop[mt] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    }
  };
  auto qk8 = [&](const i32x8 (&kop)[C::KS8], int nt) __attribute__((always_inline)) -> f32x16 {
    f32x16 S = f32x16{};
    if constexpr (F8) S = qk8_chain(kop, qop[nt]);
    return S;
  };
  // Superchunk softmax of column set nt (Sn[q] is the S^T chunk 2sc + q), in
  // pieces: sm8_scale(q) for q = 0, 1 applies the causal mask (mode 1) to
  // chunk q and folds its max into mh, and for q = 2 takes the other lane
  // half's max and sets the superchunk's power-of-two scale (one scale per
  // 64 keys: the max-tree tail and the scale arithmetic run once instead of
  // per chunk, in a slot of their own, as they are a chain of dependent
  // ops); sm8_exp(q, j) turns registers 4j..4j+3 of chunk q into 4 scaled
  // e4m3 bytes of P.
  auto sm8_scale = [&](f32x16 (&Sn)[2], int q, int nt, int sc, int mode, float& mh, int& bq, float& bias)
      __attribute__((always_inline)) {
    if (q < 2) {
      if (mode == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kic = 8 * (r >> 2) + 4 * hh + (r & 3);
          if ((2 * sc + q) * 32 + kic > rib[nt]) Sn[q][r] = -INFINITY;
        }
      }
      // NaN-propagating maximum (v_maximum3_f32, no canonicalizing copies
      // of the MFMA results, which fmaxf needs in IEEE mode): 16 values in 8
      // ops; chunk 1 folds in chunk 0's
      const f32x16& v = Sn[q];
      const float m0 = maximum3(v[0], v[1], v[2]), m1 = maximum3(v[3], v[4], v[5]);
      const float m2 = maximum3(v[6], v[7], v[8]), m3 = maximum3(v[9], v[10], v[11]);
      const float m4 = maximum3(v[12], v[13], v[14]);
      mh = maximum3(maximum3(m0, m1, m2), maximum3(m3, m4, v[15]), q == 0 ? v[15] : mh);
      return;
    }
    // the other lane half's 16 keys of the same query column, then the scale
    const float m = max_partner32(mh);
    const float rel = __builtin_fmaf(m, cs[nt], -mref[nt]);
    rmax[nt] = fmaxf(rmax[nt], rel);
    float fx = floorf(rel);
    fx = fminf(fmaxf(fx, -110.f), 120.f);
    bq = (int)fx - 7;
    // code offset 8 (7 - mref - bq) - kCodeShift = base8 - 8 fx in unorm16
    // units (fx is integral, so no integer-to-float convert is needed)
    bias = __builtin_fmaf(-8.f * kU16, fx, base8[nt]);
  };
  // The e4m3 code of P = 2^x, x = S cs - mref - bq, is the round-to-nearest
  // byte of c = 8 (x + 7) - kCodeShift, clamped at 0: y = S cs8 + bias is
  // (256 c + 127.5) / 65535, whose unorm16 convert (clamped to [0, 1]) holds
  // the code in its high byte.  One FMA per score, one packed convert per two
  // and a byte permute per four, no exponential (a superchunk's largest x is
  // below 8, so the largest code is 0x78 = 256; masked scores give 0).
  auto sm8_exp = [&](const f32x16 (&Sn)[2], int q, int j, int nt, const float bias, i32x8& pk)
      __attribute__((always_inline)) {
    const float y0 = __builtin_fmaf(Sn[q][4 * j + 0], cs8[nt], bias);
    const float y1 = __builtin_fmaf(Sn[q][4 * j + 1], cs8[nt], bias);
    const float y2 = __builtin_fmaf(Sn[q][4 * j + 2], cs8[nt], bias);
    const float y3 = __builtin_fmaf(Sn[q][4 * j + 3], cs8[nt], bias);
    const unsigned lo = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pknorm_u16(y0, y1));
    const unsigned hi = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pknorm_u16(y2, y3));
    // bytes 0-3 of the result: the high bytes of y0, y1 (lo) and y2, y3 (hi)
    pk[4 * q + j] = (int)__builtin_amdgcn_perm(hi, lo, 0x07050301u);
  };
  // e4m3 1.0 in every byte: the A operand of the row-sum MFMA.  Defined by
  // vector moves so that it lives in vector registers (as a uniform constant
  // the compiler keeps it in scalar registers, spills those, and rebuilds the
  // operand with 12 lane reads and moves at every use).
  i32x8 ones8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int one;
    asm volatile("v_mov_b32 %0, 0x38383838" : "=v"(one));
    ones8[e] = one;
  }
  auto pv8 = [&](const i32x8 (&vop)[C::MT], const i32x8& pk, int sbyte, int nt) __attribute__((always_inline)) {
    if constexpr (F8) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        O[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mt], pk, O[mt][nt], 0, 0, 0, 127, 0, sbyte);
      Lacc[nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, pk, Lacc[nt], 0, 0, 0, 127, 0, sbyte);
    }
  };
  // One fp8 stage in issue order, each slot pinned by a scheduling barrier:
  // the P V MFMAs of column set ntp (its O tiles, then the row-sum MFMA),
  // then the two QK chains of column set ntq (first MFMAs, then last ones);
  // after each slot one or two pieces of the softmax of column set nts (the
  // two max trees and the scale first, then the eight 4-score groups).
  auto stage8 = [&](f32x16 (&Sn)[2], int nts, int sc, int mode, i32x8& pk, int& sbyte, bool pv_on,
                    const i32x8 (&vv)[C::MT], const i32x8& pp, int psb, int ntp, bool qk_on,
                    const i32x8 (&k0)[C::KS8], const i32x8 (&k1)[C::KS8], int ntq, f32x16 (&So)[2])
      __attribute__((always_inline)) {
    constexpr int NPVS = C::MT + 1, NSLOT = NPVS + 2 * C::KS8, NPIECE = 11;
    static_assert(NSLOT == 2 * NPVS - 1, "a stage without QK chains spreads its P V MFMAs over every other slot");
    int bq;
    float bias, mh;
#pragma unroll
    for (int g = 0; g < NSLOT; ++g) {
      if constexpr (F8) {
        // MFMA of slot g; a stage without QK chains (NSLOT = 2 NPVS - 1) puts
        // its P V MFMAs in every other slot, so that the softmax pieces of
        // the slots between them issue under an MFMA as well
        const bool has = qk_on || g % 2 == 0;
        const int mi = qk_on ? g : g / 2;
        if (!has) {
        } else if (mi < C::MT) {
          if (pv_on)
            O[mi][ntp] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vv[mi], pp, O[mi][ntp], 0, 0, 0, 127, 0, psb);
        } else if (mi == C::MT) {
          if (pv_on) Lacc[ntp] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, pp, Lacc[ntp], 0, 0, 0, 127, 0, psb);
        } else if (qk_on) {
          const int t = mi - NPVS;
          if constexpr (C::KS8 == 2) {
            if (t == 0) qk8_first(So[0], k0[0], qop[ntq][0]);
            if (t == 1) qk8_first(So[1], k1[0], qop[ntq][0]);
            if (t == 2) qk8_last(So[0], k0[1], qop[ntq][1]);
            if (t == 3) qk8_last(So[1], k1[1], qop[ntq][1]);
          } else {
            if (t == 0) So[0] = qk8(k0, ntq);
            if (t == 1) So[1] = qk8(k1, ntq);
          }
        }
      }
      // pieces 0-2 (the two max trees, then the scale) in slots 0-2, the 8
      // code pieces spread over the remaining slots, the later slots taking
      // two where there are more pieces than slots
#pragma unroll
      for (int pc = 0; pc < NPIECE; ++pc) {
        if ((pc < 3 ? pc : NSLOT - 1 - (10 - pc) * (NSLOT - 3) / 8) == g) {
          if (pc < 3) {
            sm8_scale(Sn, pc, nts, sc, mode, mh, bq, bias);
          } else {
            sm8_exp(Sn, (pc - 3) >> 2, (pc - 3) & 3, nts, bias, pk);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sbyte = 127 + bq;
  };
  // The NSC superchunks of one fp8 K/V tile, two stages per superchunk sc:
  //   stage X: PV(sc-1, columns 1), QK(sc, columns 1)    ||  softmax(S_sc, columns 0)
  //   stage Y: PV(sc, columns 0),   QK(sc+1, columns 0)  ||  softmax(S_sc, columns 1)
  // so that only two S sets (one per column set) are ever live.  The K
  // operands of superchunk sc+1 are read at the start of stage Y, behind its
  // P V MFMAs; the V operands are double-buffered by superchunk parity.
  //
  // With an even NSC the closing P V of a tile (its last superchunk, column
  // set 1) is carried into the next tile's first stage X, whose P V slots
  // are otherwise empty: the V operands, P and its scale byte stay in the
  // registers below across the block boundary (stage X of superchunk 0
  // reads exactly the parity the last superchunk wrote).  The first tile of
  // a pass takes a zero P (and zero V) there, which adds nothing.
  constexpr bool CARRY8 = C::NSC % 2 == 0;
  i32x8 vop8[2][C::MT];
  i32x8 pp8_0, pp8_1;
  int sb8_0 = 127, sb8_1 = 127;
  auto run_tile8 = [&](const char* kt, const char* vt, int mode, int dq, bool carry_out) __attribute__((always_inline)) {
    const int kbo = __builtin_amdgcn_readfirstlane((int)(kt - lds));
    const int vbo = __builtin_amdgcn_readfirstlane((int)(vt - lds));
    const char* kbase = lds + kbo;
    const char* vbase = lds + vbo;
    i32x8 kop[2][C::KS8];
    auto& vop = vop8;
    auto& pp0 = pp8_0;
    auto& pp1 = pp8_1;
    int& sb0 = sb8_0;
    int& sb1 = sb8_1;
    f32x16 S0[2], S1[2];
    load_kop8(kbase, 0, kop[0]);
    load_kop8(kbase, 1, kop[1]);
    S0[0] = qk8(kop[0], 0);
    S0[1] = qk8(kop[1], 0);
#pragma unroll
    for (int sc = 0; sc < C::NSC; ++sc) {
      const int cp = sc & 1;
      const bool more = sc + 1 < C::NSC;
      // stage X
      load_vop8(vbase, sc, vop[cp]);
      dma_some(dq);
      __builtin_amdgcn_sched_barrier(0);
      stage8(S0, 0, sc, mode, pp0, sb0, sc > 0 || CARRY8, vop[cp ^ 1], pp1, sb1, 1, true, kop[0], kop[1], 1, S1);
      // stage Y
      if (more) {
        load_kop8(kbase, 2 * sc + 2, kop[0]);
        load_kop8(kbase, 2 * sc + 3, kop[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      stage8(S1, 1, sc, mode, pp1, sb1, true, vop[cp], pp0, sb0, 0, more, kop[0], kop[1], 0, S0);
    }
    if (!CARRY8 || !carry_out) pv8(vop[(C::NSC - 1) & 1], pp1, sb1, 1);
  };

  // dq: next-block copy ops to issue per chunk (per superchunk in fp8)
  auto run_main = [&](const char* kt, const char* vt, int mode, int dq) __attribute__((always_inline)) {
    if constexpr (F8) {
      run_tile8(kt, vt, mode, dq, mode == 0);  // the diagonal block (last) closes its own P V
    } else {
      run_tile(kt, vt, C::KC, mode, 0, 0.f, qop, dq);
    }
  };


  // ---- kept blocks (sparse) or all blocks j <= i (dense)
  const long mrow = ((long)s * a.Hkv + h) * a.seq.nqb_stride + il;
  const int* list = a.sparse ? a.block_idx + mrow * a.seq.nkb_stride : nullptr;
  const int nblk = a.sparse ? a.block_cnt[mrow] : i + 1;
  const int j0 = a.sparse ? list[0] : 0;

  // Reference max per query row: max logit over the first 32 keys of the
  // first block (causally masked if that block is the diagonal), + margin.
  issue_load(j0, 0, load_pids(j0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  {
    f32x16 S0[NT];
    if constexpr (F8) {
      i32x8 kop[C::KS8];
      load_kop8(lds, 0, kop);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S0[nt] = qk8(kop, nt);
    } else {
      bf16x8 kop[C::KS];
      load_kop(lds, 0, kop);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S0[nt] = qk(kop, qop[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kic = 8 * (r >> 2) + 4 * hh + (r & 3);
        float x = S0[nt][r] * cs[nt];
        if (j0 == i && kic > rib[nt]) x = -INFINITY;
        m = fmaxf(m, x);
      }
      m = fmaxf(m, partner32(m));
      mref[nt] = (m > -INFINITY ? m : 0.f) + kRefMargin;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll 1
  for (int pass = 0; pass < kMaxPasses; ++pass) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) O[mt][nt] = f32x16{};
      lsum[nt] = 0.f;
      if constexpr (F8) {
        Lacc[nt] = f32x16{};
        base8[nt] = __builtin_fmaf(-8.f * kU16, mref[nt], (112.f - kCodeShift) * kU16 + kU16Half);
        rmax[nt] = -INFINITY;
      }
    }
    if constexpr (F8 && CARRY8) {  // the carried P V of the pass's first block adds nothing
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) vop8[1][mt] = i32x8{};
      pp8_1 = i32x8{};
      sb8_1 = 127;
    }
    if (pass > 0) {
      __syncthreads();
      issue_load(j0, 0, load_pids(j0));
    }
    // Blocks 0 .. nblk-2 are strictly below the diagonal (the list is
    // ascending and ends with block i): one unmasked loop, the diagonal block
    // peeled after it.  List entries are read three blocks ahead so that the
    // address of the next K/V prefetch never waits on memory.
    // Paged: the page ids of the block after next are loaded together with
    // the copies of the next block.
    int jnext = nblk > 1 ? (a.sparse ? list[1] : 1) : 0;
    int jafter = nblk > 2 ? (a.sparse ? list[2] : 2) : 0;
    int pnext = load_pids(jnext);
    for (int n = 0; n + 1 < nblk; ++n) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const int jafter2 = n + 3 < nblk ? (a.sparse ? list[n + 3] : n + 3) : 0;
      const int pafter = load_pids(jafter);
      issue_load(jnext, (n + 1) & 1, pnext);
      const char* kt = lds + (n & 1) * C::TILE;
      const char* vt = lds + (2 + (n & 1)) * C::TILE;
      run_main(kt, vt, 0, 0);
      jnext = jafter;
      jafter = jafter2;
      pnext = pafter;
    }
    {
      const int n = nblk - 1;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const char* kt = lds + (n & 1) * C::TILE;
      const char* vt = lds + (2 + (n & 1)) * C::TILE;
      run_main(kt, vt, 1, 0);
    }

    // ---- mean correction: dropped blocks as pseudo-keys
    // LDS during this phase: pseudo-K tile (BLK rows, bf16) | pseudo-V tile |
    // ndrop | kept-block bitmap | dropped-block list.  The dropped blocks are
    // gathered BLK at a time: each thread loads its share of their fp32
    // kbar/vbar rows with plain loads (TPP issued before any is converted)
    // and writes them as bf16 into the padded tiles, which are then taken 32
    // pseudo-keys at a time.  In
    // fp8 the pseudo rows are divided by the head's k / v scale so that they
    // share the code units of the fp8 K and V (the logit scale cs and the
    // output scale v_s then apply to both), and Q is widened to bf16 (exact
    // for e4m3 values).
    if (a.sparse && a.mean_correction && i > 0) {
      __syncthreads();
      char* pk_t = lds;
      char* pv_t = lds + C::PSB;
      int* ndrop_slot = (int*)(lds + 2 * C::PSB);
      uint32_t* bm = (uint32_t*)(ndrop_slot + 1);
      const int nwords = (i + 31) >> 5;
      int* drop = (int*)(bm + nwords);
      for (int w = tid; w < nwords; w += nthr) bm[w] = 0u;
      __syncthreads();
      for (int n = tid; n < nblk; n += nthr) {
        const int j = list[n];
        if (j < i) atomicOr(&bm[j >> 5], 1u << (j & 31));
      }
      __syncthreads();
      if (wave == 0) {
        int total = 0;
        for (int w0 = 0; w0 < nwords; w0 += 64) {
          const int w = w0 + lane;
          uint32_t bits = 0u;
          if (w < nwords) {
            const uint32_t valid = (w < (i >> 5)) ? 0xffffffffu : ((1u << (i & 31)) - 1u);
            bits = ~bm[w] & valid;
          }
          const int cnt = __popc(bits);
          const int incl = wave_incl_scan(cnt);
          int off = total + incl - cnt;
          while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            drop[off++] = w * 32 + b;
          }
          total += __shfl(incl, 63, 64);
        }
        if (lane == 0) *ndrop_slot = total;
      }
      __syncthreads();
      const int ndrop = *ndrop_slot;
      const float* kbr = a.kbar + ((long)s * a.Hkv + h) * a.seq.nkb_stride * D;
      const float* vbr = a.vbar + ((long)s * a.Hkv + h) * a.seq.nkb_stride * D;
      const float bias = log2f((float)BLK);  // ln(n_j) in log2 units; dropped blocks are full
      const float kmul = F8 ? 1.f / a.k_scale[h] : 1.f;
      const float vmul = F8 ? 1.f / a.v_scale[h] : 1.f;
      bf16x8 q16[NT][C::KS];
      if constexpr (F8) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const i32x8 w = qop[nt][ks >> 2];
            const uint32_t w0 = (uint32_t)w[2 * (ks & 3)], w1 = (uint32_t)w[2 * (ks & 3) + 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              q16[nt][ks][e] = (__bf16)fp8_byte_to_f32(w0, e);
              q16[nt][ks][4 + e] = (__bf16)fp8_byte_to_f32(w1, e);
            }
          }
      }
      constexpr int CH8 = D / 8;              // 8-element pieces per row
      constexpr int TASKS = 2 * BLK * CH8;    // pieces of a round (K rows, then V rows)
      constexpr int TPP = 4;                  // pieces per thread held in registers at once
      for (int c0 = 0; c0 < ndrop; c0 += BLK) {
        for (int base = 0; base < TASKS; base += nthr * TPP) {
          float4 x[TPP][2];
#pragma unroll
          for (int u = 0; u < TPP; ++u) {
            const int task = base + u * nthr + tid;
            if (task < TASKS) {
              const int rr = task / CH8;        // 0 .. 2*BLK-1: K rows then V rows
              const int c = task - rr * CH8;
              const int pidx = c0 + (rr & (BLK - 1));
              const int id = drop[pidx < ndrop ? pidx : 0];  // past the end: any finite row (masked)
              const float* src = (rr < BLK ? kbr : vbr) + (long)id * D + c * 8;
              x[u][0] = *(const float4*)src;
              x[u][1] = *(const float4*)(src + 4);
            }
          }
#pragma unroll
          for (int u = 0; u < TPP; ++u) {
            const int task = base + u * nthr + tid;
            if (task < TASKS) {
              const int rr = task / CH8;
              const int c = task - rr * CH8;
              const float f = rr < BLK ? kmul : vmul;
              const uint4 w = make_uint4(pack_bf16x2(x[u][0].x * f, x[u][0].y * f),
                                         pack_bf16x2(x[u][0].z * f, x[u][0].w * f),
                                         pack_bf16x2(x[u][1].x * f, x[u][1].y * f),
                                         pack_bf16x2(x[u][1].z * f, x[u][1].w * f));
              *(uint4*)((rr < BLK ? pk_t : pv_t) + (rr & (BLK - 1)) * C::RS16 + c * 16) = w;
            }
          }
        }
        __syncthreads();
        const int nv = min(BLK, ndrop - c0);
#pragma unroll 1
        for (int cc = 0; cc * 32 < nv; ++cc) {
          if constexpr (F8) {
            run_tile(pk_t + cc * 32 * C::RS16, pv_t + cc * 32 * C::RS16, 1, 2, nv - cc * 32, bias, q16, 0);
          } else {
            run_tile(pk_t + cc * 32 * C::RS16, pv_t + cc * 32 * C::RS16, 1, 2, nv - cc * 32, bias, qop, 0);
          }
        }
        __syncthreads();
      }
    }

    // A row whose normaliser overflowed the range reruns the tile with its
    // reference moved up (all rows of the workgroup take part in the rerun;
    // rows that were fine recompute the same values).
    // Rerun rule, per row (both lane halves of a query column see the same
    // normaliser lt and take the same decision):
    //  * fp8: a superchunk maximum more than kRefOverflow above the reference
    //    (its codes may have left e4m3's range): the reference moves up to
    //    that maximum, after which every code of the rerun is in range;
    //  * a finite normaliser of 2^kRefOverflow or more: the reference moves up
    //    by log2(lt), which is at least the largest exponent, so every term
    //    of the rerun is at most 1;
    //  * an overflowed normaliser (some exponent beyond fp32's range): the
    //    reference moves up by a step that doubles from kFirstStep until a
    //    pass's normaliser falls below 2^-kRefUnder (the reference overshot)
    //    and is bisected from then on; the window of references that give a
    //    normaliser in [2^-kRefUnder, 2^kRefOverflow) is 160 log2 units wide,
    //    so the search ends there with every term at full precision.
    // All rows of the workgroup rerun; rows that were fine recompute the
    // same values.  A row still unresolved after the last pass is written
    // as NaN (its logits exceed the first reference by more than ~8e6).
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float lt = (F8 ? Lacc[nt][0] : 0.f) + lsum[nt] + partner32(lsum[nt]);
      const float st = rstep[nt];
      bool bad_nt = false;
      if (F8 && rmax[F8 ? nt : 0] > kRefOverflow) {
        bad_nt = true;
        mref[nt] += rmax[F8 ? nt : 0];
      } else if (lt >= __builtin_exp2f(kRefOverflow) && lt < INFINITY) {
        bad_nt = true;
        mref[nt] += log2f(lt);
      } else if (lt == INFINITY) {  // overflow: step up
        bad_nt = true;
        mref[nt] += fabsf(st) * (st < 0.f ? 0.5f : 1.f);
        rstep[nt] = st < 0.f ? 0.5f * st : 2.f * st;
      } else if (lt < __builtin_exp2f(-kRefUnder) && st != kFirstStep) {  // overshot a step up: bisect back
        bad_nt = true;
        const float half = st < 0.f ? -0.5f * st : 0.25f * st;
        mref[nt] -= half;
        rstep[nt] = -half;
      }
      if (bad_nt && pass + 1 == kMaxPasses) lsum[nt] = __builtin_nanf("");  // unresolved row: NaN
      bad |= bad_nt;
    }
    if (!__syncthreads_or(bad)) break;
  }

  // ---- epilogue: O = O^T / l (fp8: times the head's v scale), LSE
  // output: fp32, bf16, or e4m3 codes of out / o_scale (RNE, saturated)
  const int omode = a.out_mode;
  const float oscale = (F8 ? a.v_scale[h] : 1.f) * (omode == 2 ? 1.f / *a.o_scale : 1.f);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int rb;
    long off;
    const bool ok = qinfo(nt, rb, off);
    const float lt = (F8 ? Lacc[nt][0] : 0.f) + lsum[nt] + partner32(lsum[nt]);
    const float inv = oscale / lt;
    if (ok) {
      if (a.lse && hh == 0) {
        const int gq = (pr0 + l32 + 32 * nt) / BLK;
        const int r = i * BLK + rb - g.P;
        const long li = a.seq.cu_seqlens_q ? (long)(g.qrow0 + r) * a.Hq + h * G + gq
                                           : ((long)s * a.Hq + h * G + gq) * a.lse_stride + r;
        a.lse[li] = (mref[nt] + log2f(lt)) * kLn2;
      }
      if (omode == 2) {
        unsigned char* dst = (unsigned char*)a.out + off + 4 * hh;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(O[mt][nt][4 * q4 + e] * inv, -448.f), 448.f);
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
            *(int*)(dst + 32 * mt + 8 * q4) = w;
          }
      } else if (omode == 1) {
        float* dst = (float*)a.out + off + 4 * hh;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(float4*)(dst + 32 * mt + 8 * q4) =
                make_float4(O[mt][nt][4 * q4] * inv, O[mt][nt][4 * q4 + 1] * inv, O[mt][nt][4 * q4 + 2] * inv,
                            O[mt][nt][4 * q4 + 3] * inv);
      } else {
        __bf16* dst = (__bf16*)a.out + off + 4 * hh;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(uint2*)(dst + 32 * mt + 8 * q4) =
                make_uint2(pack_bf16x2(O[mt][nt][4 * q4] * inv, O[mt][nt][4 * q4 + 1] * inv),
                           pack_bf16x2(O[mt][nt][4 * q4 + 2] * inv, O[mt][nt][4 * q4 + 3] * inv));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Persistent tile scheduler.  The tiles form 8 queues, one per XCD under the
// round-robin workgroup -> XCD dispatch, each ordered longest first (see
// attn_tile).  The gridDim.x <= #CU workgroups stay resident; workgroup w
// starts at position w / 8 of its home queue w % 8 and then pulls the next
// position of its queue from a device-scope counter, moving on to the other
// queues in turn once its own is drained.  Workgroups never wait for the
// hardware dispatcher between tiles (with tiles of very different lengths that
// dispatcher leaves CUs idle), while the two parts of one tile and the tiles
// of one head in a query-block rank stay in one XCD's L2.
//
// The 8 counters (each on its own 128-byte line) must be zero when the
// launch starts and must belong to no launch that can run at the same time.
// Paged launches keep them in the caller's workspace (zeroed by the plan
// kernel before them on the stream).  Contiguous launches, which take no
// workspace, use one of the sets in g_sched, zeroed by sched_reset_kernel on
// the launch's stream right before it: the first kStreamSlots streams a
// process launches on each get a set of their own (a stream's launches run
// in order, so they can share it), and a launch captured into a HIP graph
// takes the next of kCaptureSlots further sets, which no eager launch uses.
constexpr int kStreamSlots = 192;
constexpr int kCaptureSlots = 64;
constexpr int kSchedSlots = kStreamSlots + kCaptureSlots;
__device__ unsigned int g_sched[kSchedSlots][8][32];

__global__ void sched_reset_kernel(int slot) {
  if (threadIdx.x < 8) atomicExch(&g_sched[slot][threadIdx.x][0], 0u);
}

template <int D, int BLK, bool F8, bool PG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int nwg = gridDim.x;
  const int home = blockIdx.x & 7;
  unsigned int(*ctr)[32] = a.sched ? (unsigned int(*)[32])a.sched : g_sched[a.sched_slot];
  // tiles in queue q: all positions below it are tiles
  const int ntask = PG ? __builtin_amdgcn_readfirstlane(a.plan_count[0]) : a.ntiles;
  auto queue_len = [&](int q) -> int {
    if (!PG) return (ntask - q + 7) >> 3;
    return q < ntask ? ((ntask - q + 7) >> 3) * a.parts : 0;
  };
  // next-tile broadcast, double-buffered: the slot written at iteration k is
  // rewritten at k+2, after every thread has passed the barrier of k+1
  volatile int* next_slot = (volatile int*)(smem + a.lds_sched);
  int qi = 0;        // thread 0: queues drained so far
  unsigned pre = 0;  // thread 0: position fetched from queue (home + qi) % 8
  // thread 0: the next tile, encoded q | pos << 3, or -1 when every queue is
  // drained; `pre` holds a fetch from queue (home + qi) % 8 on entry
  auto next_tile = [&]() -> int {
    while (qi < 8) {
      const int q = (home + qi) & 7;
      const int pos = (nwg - q + 7) / 8 + (int)pre;  // the home workgroups took positions [0, nhome)
      if (pos < queue_len(q)) return q | (pos << 3);
      if (++qi < 8) pre = atomicAdd(&ctr[(home + qi) & 7][0], 1u);
    }
    return -1;
  };
  int tile = (int)(blockIdx.x >> 3) < queue_len(home) ? home | ((blockIdx.x >> 3) << 3) : -2;
  if (tile == -2) {  // no tile at the home position: start by fetching
    if (threadIdx.x == 0) {
      pre = atomicAdd(&ctr[home][0], 1u);
      next_slot[1] = next_tile();
    }
    __syncthreads();
    tile = __builtin_amdgcn_readfirstlane(next_slot[1]);
  }
  for (int k = 0; tile >= 0; ++k) {
    if (threadIdx.x == 0 && qi < 8) pre = atomicAdd(&ctr[(home + qi) & 7][0], 1u);
    attn_tile<D, BLK, F8, PG>(a, tile & 7, tile >> 3, smem);
    if (threadIdx.x == 0) next_slot[k & 1] = next_tile();
    __syncthreads();
    tile = __builtin_amdgcn_readfirstlane(next_slot[k & 1]);
  }
}

// LDS of the attention kernel for a given key-block count: the K/V tiles or
// the correction phase's buffers (whichever is larger), then the copy-offset
// table, then the next-tile broadcast slots.  The compiler reserves a static
// segment in front of the 1 KB-aligned dynamic buffer, which counts against
// the workgroup's 160 KB as well.
constexpr int kSchedLdsBytes = 16;
constexpr int kStaticLdsBytes = 1024;

template <int D, int BLK, bool F8>
static size_t attn_lds_dtab(int nkb) {
  using C = Cfg<D, BLK, F8>;
  size_t lds = 4 * (size_t)C::TILE;
  const size_t corr = (size_t)corr_lds_bytes<D, BLK, F8>(nkb);
  return corr > lds ? corr : lds;
}

// the dynamic LDS of a launch
template <int D, int BLK, bool F8>
static size_t attn_dyn_lds_bytes(int nkb) {
  return attn_lds_dtab<D, BLK, F8>(nkb) + Cfg<D, BLK, F8>::DTAB + kSchedLdsBytes;
}

// the workgroup's whole LDS, static segment included (checked against 160 KB)
template <int D, int BLK, bool F8>
static size_t attn_lds_bytes(int nkb) {
  return attn_dyn_lds_bytes<D, BLK, F8>(nkb) + kStaticLdsBytes;
}

static int compute_units() {
  static std::atomic<int> cache[64];  // zero-initialised (static storage); calls may come from several threads
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev >= 64) dev = 63;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The library's counter set for a contiguous launch on stream st (see the
// scheduler above): a captured launch takes the next capture set in turn;
// otherwise the stream keeps the set it got at its first launch on this
// device, sets being handed out in first-use order (past kStreamSlots
// streams the oldest assignment is taken over).  hipStreamPerThread is one
// handle for a different stream in every host thread, so there the calling
// thread is part of the key.
static int sched_slot_for(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t ce = hipStreamIsCapturing(st, &cs);
  if (ce == hipSuccess && cs == hipStreamCaptureStatusActive) {
    static std::atomic<unsigned> next_capture{0};
    return kStreamSlots + (int)(next_capture.fetch_add(1) % kCaptureSlots);
  }
  if (ce != hipSuccess) (void)hipGetLastError();  // a refused capture query leaves no error behind
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  using Key = std::tuple<int, hipStream_t, std::thread::id>;
  static std::mutex mu;
  static std::map<Key, int> slot_of;
  static Key owner[64][kStreamSlots];
  static int next[64];
  const int dv = dev & 63;
  std::lock_guard<std::mutex> lock(mu);
  const Key key(dev, st, st == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id());
  const auto it = slot_of.find(key);
  if (it != slot_of.end()) return it->second;
  const int slot = next[dv]++ % kStreamSlots;
  if (next[dv] > kStreamSlots) slot_of.erase(owner[dv][slot]);
  owner[dv][slot] = key;
  slot_of[key] = slot;
  return slot;
}

// Once per kernel instance and device (a kernel's attributes belong to the
// device it runs on): whether the static segment fits the allowance (1) or
// not (-1), after raising the dynamic-LDS limit to everything the allowance
// leaves (launches then pass their own size, which never lowers the limit);
// 0 when the attributes cannot be read.  Devices past the first 64 redo this
// at every launch, which sets the same value again.
template <int D, int BLK, bool F8, bool PG>
static int lds_attr_ok() {
  static std::atomic<int> static_ok[64];  // zero-initialised (static storage)
  static std::mutex init_mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>* const okp = dev < 64 ? &static_ok[dev] : nullptr;
  int ok = okp ? okp->load(std::memory_order_acquire) : 0;
  if (ok != 0) return ok;
  std::lock_guard<std::mutex> lock(init_mu);
  ok = okp ? okp->load(std::memory_order_relaxed) : 0;
  if (ok != 0) return ok;
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, (const void*)attn_kernel<D, BLK, F8, PG>) != hipSuccess) return 0;
  ok = fa.sharedSizeBytes <= (size_t)kStaticLdsBytes ? 1 : -1;
  if (ok > 0 && hipFuncSetAttribute((const void*)attn_kernel<D, BLK, F8, PG>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    160 * 1024 - kStaticLdsBytes) != hipSuccess)
    return 0;
  if (okp) okp->store(ok, std::memory_order_release);
  return ok;
}

template <int D, int BLK, bool F8>
static hipError_t launch_t(const AttnArgs& a0, hipStream_t st) {
  const long ntiles = (long)a0.Hkv * a0.seq.batch * a0.parts * a0.nqb_grid;
  if (attn_lds_bytes<D, BLK, F8>(a0.seq.nkb_stride) > 160 * 1024) return hipErrorInvalidValue;
  if (ntiles > 0x7fffffffL) return hipErrorInvalidValue;
  // the tile order maps every tile to a head below Hkv only for a divisor
  if (!a0.plan && (a0.head_group < 1 || a0.Hkv % a0.head_group != 0)) return hipErrorInvalidValue;
  const bool pg = a0.kv.page_table != nullptr;
  if (pg != (a0.plan != nullptr)) return hipErrorInvalidValue;  // paged launches come with their plan
  const int ok = pg ? lds_attr_ok<D, BLK, F8, true>() : lds_attr_ok<D, BLK, F8, false>();
  if (ok <= 0) return hipErrorInvalidValue;
  const size_t lds_total = attn_dyn_lds_bytes<D, BLK, F8>(a0.seq.nkb_stride);
  if (ntiles == 0) return hipSuccess;
  AttnArgs a = a0;
  a.ntiles = (int)ntiles;
  a.lds_dtab = (int)attn_lds_dtab<D, BLK, F8>(a0.seq.nkb_stride);
  a.lds_sched = (int)(lds_total - kSchedLdsBytes);
  const long grid = ntiles < compute_units() ? ntiles : compute_units();
  if (!a.sched) {
    a.sched_slot = sched_slot_for(st);
    hipLaunchKernelGGL(sched_reset_kernel, dim3(1), dim3(64), 0, st, a.sched_slot);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pg)
    hipLaunchKernelGGL((attn_kernel<D, BLK, F8, true>), dim3((unsigned)grid), dim3(64 * a.waves), lds_total, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, BLK, F8, false>), dim3((unsigned)grid), dim3(64 * a.waves), lds_total, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp2
