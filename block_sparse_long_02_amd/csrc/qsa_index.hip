// Indexer block scores (a2) and the deterministic top-K_B block select (a3).
//
// Method (page "Qwen3.8-Flash-Next 没有缩小模型，它重写了每个参数何时上场",
// section "03 · Attention", BLOCK SCORE and CAUSAL SPARSE SET equations, third
// and fourth QSA steps): for query i at position p the candidates are the
// completed blocks b < n_c = (p+1)/4; each gets
//     s_b = sum_h w_h * ReLU(q_h . kbar_b / sqrt(128))          (float32)
// and the K = min(budget, n_c) best under (score desc, block asc) are kept.
//
// Design (gfx950).  Scores are never materialised for all candidates: at 1M
// tokens that would be 1 MB per query, and writing then re-reading them costs
// more HBM time than the score GEMM itself.  Instead:
//   1. sample pass   -- the score GEMM over every 32nd block writes those
//                       scores (1/32 of the work) for rows with > 4096 candidates;
//   2. threshold     -- per row, tau = the r-th largest sampled score, with r
//                       chosen so that about K + 1280 candidates score >= tau;
//   3. filter pass   -- the full score GEMM (bf16 MFMA 16x16x32, indexer query
//                       rows in registers, block keys streamed) appends every
//                       (score, block) with score >= tau to a per-row list
//                       (wave-aggregated atomics);
//   4. final select  -- per row, an exact LDS radix select over that list under
//                       the total order, then the ids sorted ascending.
// Exactness does not depend on the sample: if the list holds >= K entries it
// contains the true top K (all of them score >= the K-th score >= tau).  A row
// whose list is short or overflows is selected inside step 4 by an exact
// radix select that recomputes its scores on every pass (slow, needs no score
// storage, rare).
#include <math.h>

#include <type_traits>

#include "qsa_common.hpp"

namespace qsa {

// m-tiles (of 4 queries x 4 heads) per wave in the prefill score GEMM
#ifndef QSA_PREFILL_MT
#define QSA_PREFILL_MT 2
#endif
constexpr int kPrefillMT = QSA_PREFILL_MT;
// workgroups per CU the prefill score GEMM is compiled for
#ifndef QSA_SCORE_WGS
#define QSA_SCORE_WGS 3
#endif
constexpr int kCandCap = 4096;      // list capacity per row
constexpr int kSampleStride = 16;   // decode (dense) path: every 16th score is a sample
// prefill sample pass: every kPrefillSampleStride-th block is scored
#ifndef QSA_PREFILL_SAMPLE_STRIDE
#define QSA_PREFILL_SAMPLE_STRIDE 32
#endif
constexpr int kPrefillSampleStride = QSA_PREFILL_SAMPLE_STRIDE;
// aimed-for surplus of prefill list entries over K
#ifndef QSA_SAMPLE_EXTRA
#define QSA_SAMPLE_EXTRA 1280
#endif
constexpr int kSampleExtra = QSA_SAMPLE_EXTRA;
constexpr int kBins = 2048;         // 11-bit radix digits / histogram bins
constexpr int kFinishCap = 256;     // keys ranked one by one in a boundary bin
// 1/sqrt(128) rounded once to float32
constexpr float kScoreScale = 0x1.6a09e6p-4f;

// Row geometry shared by all kernels: which sequence, position, candidates.
struct RowGeom {
  int seq, pos, n_c;
  bool ok;
};

__device__ __forceinline__ RowGeom row_geom(const int32_t* __restrict__ cu_q,
                                            const int32_t* __restrict__ seq_len, int n_seq,
                                            int row, int max_blocks) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  RowGeom r;
  const int qb = cu_q[lo], qe = cu_q[lo + 1];
  r.seq = lo;
  r.pos = seq_len[lo] - (qe - qb) + (row - qb);
  r.n_c = (r.pos + 1) >> 2;
  r.ok = row >= qb && row < qe && r.pos >= 0 && r.n_c <= max_blocks;
  return r;
}

// max(x, +0) on the bit pattern: negative floats (sign bit set) are negative
// int32 values, so a signed integer max gives +0 for them and x otherwise
// (-0 also maps to +0).  One instruction instead of a NaN-quieting fmaxf.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// The float32 epilogue shared by every pass: heads in acc[0..3].
__device__ __forceinline__ float block_score(f32x4 acc, const float* __restrict__ w) {
#pragma clang fp contract(off)
  const float u0 = relu_bits(acc[0]) * kScoreScale;
  const float u1 = relu_bits(acc[1]) * kScoreScale;
  const float u2 = relu_bits(acc[2]) * kScoreScale;
  const float u3 = relu_bits(acc[3]) * kScoreScale;
  float s = w[0] * u0;
  s = s + w[1] * u1;
  s = s + w[2] * u2;
  s = s + w[3] * u3;
  return s == 0.f ? 0.f : s;   // canonical +0
}

// ----------------------------------------------------- dense scores (decode)
// Small tiles (at most 4 queries per sequence, i.e. decode and multi-token
// decode): the score of every candidate is written out.  That costs 4 bytes
// per block against the 256-byte block key the kernel must stream anyway, and
// lets the select read scores instead of recomputing them; every 16th score
// also goes to a contiguous sample row.  Workgroup = one
// sequence's queries (m-tile rows 4*query + head) x one chunk of columns; wave
// w takes the 16-column tiles w, w+4, ...  The tile loop is fully unrolled so
// that kDenseDepth tiles of keys stay in flight with exact wait counts, and
// the scores are stored after the last tile.
//
// Chunk size.  A launch whose 1024-column chunks fill the chip's workgroup
// slots streams best in those chunks: each wave keeps 4 tiles in flight
// through 16 tiles without a gap between workgroup rounds.  A launch whose
// rows are few or mostly short (a ragged batch with one long row) leaves
// most CUs with one such workgroup or none, and the long row's chunks each
// take 4 memory round trips; 256-column chunks put 4 times as many of its
// bytes in flight at once.  The kernel picks the size itself from the
// sequence lengths (the host knows only the longest): every workgroup counts
// the launch's active 1024-column chunks the same way and so takes the same
// decision.
constexpr int kDenseChunk = 1024;
constexpr int kDenseChunkSmall = 256;
constexpr int kDenseDepth = 4;
// workgroup slots of the chip for this kernel (256 CUs x 4)
constexpr int kDenseSlots = 1024;
// launches of up to this many sequences choose their chunk size (one wave
// counts the chunks, one sequence per lane)
constexpr int kDenseAdaptSeqs = 64;

// Rows of sequence s scored by the dense pass: n_rows (<= 4) rows ending at
// its last position, candidates up to nc_last; false if it has no query row.
struct DenseSeq {
  int qb, qe, qe_raw, pos0, n_rows, nc_last;
};
__device__ __forceinline__ bool dense_seq(const int32_t* __restrict__ cu_q,
                                          const int32_t* __restrict__ seq_len, int n_q,
                                          int max_blocks, int s, DenseSeq& d) {
  d.qb = cu_q[s];
  d.qe_raw = cu_q[s + 1];
  d.qe = min(d.qe_raw, n_q);
  if (d.qb >= d.qe || d.qb < 0) return false;
  d.pos0 = seq_len[s] - (d.qe_raw - d.qb);
  d.n_rows = min(4, d.qe - d.qb);
  // rows with more than max_blocks candidates are reported by the select;
  // the others still need every score
  d.nc_last = min((d.pos0 + d.n_rows) >> 2, max_blocks);
  return true;
}

template <bool kPaged, int kChunk>
__device__ __forceinline__ void dense_chunk(const uint16_t* __restrict__ idx_q,
                                            const float* __restrict__ w, const DenseSeq& d, int s,
                                            int chunk, const uint16_t* __restrict__ bk,
                                            int64_t bk_stride, uint32_t* __restrict__ dense,
                                            int64_t dense_stride, uint32_t* __restrict__ dsmp,
                                            int64_t dsmp_stride, const Pages& pg,
                                            float (&s_w)[4][4], int (&s_nc)[4]) {
  constexpr int kTiles = kChunk / 64;   // tiles per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int qb = d.qb, qe = d.qe, n_rows = d.n_rows;
  const int v0 = chunk * kChunk;
  if (v0 >= d.nc_last) return;
  const int v1 = min(v0 + kChunk, d.nc_last);
  if (threadIdx.x < 4) {
    const int j = threadIdx.x;
    const bool ok = j < n_rows;
    const int rj = min(qb + j, qe - 1);
    s_nc[j] = ok ? (d.pos0 + j + 1) >> 2 : 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float wv = w[(int64_t)rj * 4 + h];
      s_w[j][h] = ok ? wv : 0.f;
    }
  }
  // A fragment: row col = 4*query + head, dims 32*ks + 8*grp .. +7
  u32x4 af[4];
  {
    const int j = col >> 2;
    const int rj = min(qb + j, qe - 1);
    const uint16_t* src = idx_q + ((int64_t)rj * 4 + (col & 3)) * kIdxDim + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 v = ldg16(src + 32 * ks);
      af[ks] = j < n_rows ? v : u32x4{0, 0, 0, 0};
    }
  }
  const uint16_t* bseq = bk + (kPaged ? 0 : (int64_t)s * bk_stride);
  // paged: lane l holds the physical page of the chunk's l-th page (a chunk
  // of 1024 blocks spans at most 17 pages of >= 64 blocks); only pages that
  // hold blocks below v1 are read from the table
  const int p0 = kPaged ? (v0 >> pg.shift) : 0;
  int tabv = 0;
  if (kPaged && p0 + lane <= ((v1 - 1) >> pg.shift))
    tabv = pg.table[(int64_t)s * pg.stride + p0 + lane];
  const int c0 = v0 + wave * 16;
#ifndef QSA_DENSE_SKEW
#define QSA_DENSE_SKEW 1
#endif
  // Workgroups start at different tiles of their chunk (rotated order) so
  // that the ones running together do not stream the same address offsets.
  const int rot = QSA_DENSE_SKEW ? (int)(((unsigned)s * 7u + (unsigned)chunk * 3u) & (kTiles - 1)) : 0;
  auto tcol = [&](int t) { return c0 + 64 * ((t + rot) & (kTiles - 1)); };
  // B fragment of tile t: column tcol(t) + col (clamped in bounds past v1)
  auto load_tile = [&](u32x4 (&bf)[4], int t) {
    const int b = min(tcol(t) + col, v1 - 1);
    int64_t pb = b;
    if constexpr (kPaged) {
      const int pp = __shfl(tabv, (b >> pg.shift) - p0, 64);
      pb = ((int64_t)pp << pg.shift) + (b & ((1 << pg.shift) - 1));
    }
    const uint16_t* src = bseq + pb * kIdxDim + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bf[ks] = ldg16(src + 32 * ks);
  };
  u32x4 buf[kDenseDepth][4];
#pragma unroll
  for (int dd = 0; dd < kDenseDepth; ++dd) load_tile(buf[dd], dd);
  __syncthreads();
  // lane holds the 4 heads of query grp for block c0 + 64t + col
  const int j = grp;
  const float wr[4] = {s_w[j][0], s_w[j][1], s_w[j][2], s_w[j][3]};
  const int nc_j = min(s_nc[j], v1);
  float sc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma_16x16x32(af[ks], buf[t % kDenseDepth][ks], acc);
    if (t + kDenseDepth < kTiles) load_tile(buf[t % kDenseDepth], t + kDenseDepth);
    sc[t] = block_score(acc, wr);
  }
  if (j < n_rows) {
    uint32_t* drow = dense + (int64_t)(qb + j) * dense_stride;
    uint32_t* srow = dsmp + (int64_t)(qb + j) * dsmp_stride;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int b = tcol(t) + col;
      if (b < nc_j) {
        drow[b] = __float_as_uint(sc[t]);
        if ((b & (kSampleStride - 1)) == 0) srow[b / kSampleStride] = __float_as_uint(sc[t]);
      }
    }
  }
}

// Grid: n_seq x n_small workgroups (n_small = 256-column chunks of the
// longest row) when adapt is set, else n_seq x 1024-column chunks.  One
// linear grid, sequence-major: a sequence's chunks take consecutive
// workgroup ids, which the dispatcher spreads over the XCDs (a grid of
// (sequences, chunks) would put every chunk of a sequence on one XCD
// whenever the sequence count is a multiple of 8).  With 1024-column chunks
// in an adaptive launch the working workgroups are the first n_seq x
// n_big ids and the rest exit at once.
template <bool kPaged>
__global__ void __launch_bounds__(256, 4)
score_dense_kernel(const uint16_t* __restrict__ idx_q, const float* __restrict__ w,
                   const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len,
                   int n_seq, int n_q, int max_blocks, const uint16_t* __restrict__ bk,
                   int64_t bk_stride, uint32_t* __restrict__ dense, int64_t dense_stride,
                   uint32_t* __restrict__ dsmp, int64_t dsmp_stride, int adapt, Pages pg) {
  __shared__ float s_w[4][4];
  __shared__ int s_nc[4];
  const int n_big = (max_blocks + kDenseChunk - 1) / kDenseChunk;
  const int id = blockIdx.x;
  bool big = true;
  // adaptive launches: lane i of every wave holds sequence i's geometry,
  // from which the workgroup's own sequence is then taken by a shuffle
  DenseSeq e = {};
  bool e_ok = false;
  if (adapt) {
    // active 1024-column chunks of the launch (every wave of every
    // workgroup computes the same sum)
    const int lane = threadIdx.x & 63;
    int n = 0;
    if (lane < n_seq) {
      e_ok = dense_seq(cu_q, seq_len, n_q, max_blocks, lane, e);
      if (e_ok && e.nc_last > 0) n = (e.nc_last + kDenseChunk - 1) / kDenseChunk;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
    big = n >= kDenseSlots;
  }
  const int n_ch = big ? n_big : (max_blocks + kDenseChunkSmall - 1) / kDenseChunkSmall;
  if (id >= n_seq * n_ch) return;
  const int s = id / n_ch, chunk = id % n_ch;
  DenseSeq d;
  if (adapt) {
    if (!__shfl((int)e_ok, s, 64)) return;
    d.qb = __shfl(e.qb, s, 64);
    d.qe = __shfl(e.qe, s, 64);
    d.qe_raw = __shfl(e.qe_raw, s, 64);
    d.pos0 = __shfl(e.pos0, s, 64);
    d.n_rows = __shfl(e.n_rows, s, 64);
    d.nc_last = __shfl(e.nc_last, s, 64);
  } else if (!dense_seq(cu_q, seq_len, n_q, max_blocks, s, d)) {
    return;
  }
  if (big)
    dense_chunk<kPaged, kDenseChunk>(idx_q, w, d, s, chunk, bk, bk_stride, dense, dense_stride,
                                     dsmp, dsmp_stride, pg, s_w, s_nc);
  else
    dense_chunk<kPaged, kDenseChunkSmall>(idx_q, w, d, s, chunk, bk, bk_stride, dense,
                                          dense_stride, dsmp, dsmp_stride, pg, s_w, s_nc);
}

// ------------------------------------------------------- prefill GEMM
// Prefill variant of the score GEMM: workgroup = 4*MT*NW queries (NW waves,
// each owning MT m-tiles of 16 rows = 4 queries x 4 heads) x a chunk of
// columns.  The sample pass uses 4 waves, the filter pass 8 (64 queries, two
// workgroups and 4 waves per SIMD, at most 128 VGPRs).  Block keys go through
// a 2-stage LDS ring of 64 columns (16 KB) shared by the waves: every thread
// loads 16/NW chunks of 16 bytes of the next stage into registers while the
// current stage is multiplied, then writes them to LDS (each wave
// instruction covers a 1 KB run of 4 columns).  Inside a stage, columns sit
// 272 bytes apart (256 + 16 of padding), which makes the MFMA B-fragment
// reads (16 columns x one 16-byte chunk) hit 16 distinct bank groups.
//
// Filter epilogue.  About 1% of candidates reach the threshold, so almost
// every stage has a hit somewhere; handling hits in the SIMT stream would cost
// more than the MFMAs.  The stream therefore only (1) evaluates the cheap
// pre-filter and takes its compare mask as a wave ballot, and (2) for the few
// (tile, m-tile) pairs with a set bit, appends the raw 4-head accumulators and
// the block id to a per-row LDS pending list.  The defined float32 score and
// the exact tau test run once per workgroup over the pending lists, one entry
// per lane.
constexpr int kStageCols = 64;
// bf16 elements per LDS column: 256 bytes of key plus 16 of padding, so the
// 16 lanes of a 128-bit B-fragment read (16 columns, the same dims) hit 16
// distinct bank groups
constexpr int kColStride = kIdxDim + 8;

// v_dot2_f32_bf16 with a destination of its own: for a loop-invariant
// accumulator the compiler picks the accumulating form plus a register copy
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
// pending pre-filter passes per row and workgroup: 32 for 8-wave workgroups
// (the most that two per CU leave room for), 24 for 4-wave ones
template <int NW>
constexpr int kPending = NW == 8 ? 32 : 24;

// Largest column chunk a workgroup takes (host-side chunks are <= this).
constexpr int kMaxChunkCols = 2048;

// (the second launch bound is the minimum number of waves per SIMD: 4-wave
// workgroups at QSA_SCORE_WGS per CU, 8-wave workgroups at 2 per CU)
template <int MT, int NW, bool kSample, bool kPaged>
__global__ void __launch_bounds__(64 * NW, NW == 4 ? QSA_SCORE_WGS : 4)
score_gemm_kernel(const uint16_t* __restrict__ idx_q, const float* __restrict__ w,
                  const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len,
                  int n_seq, int n_q, int tiles_per_seq, int max_blocks,
                  const uint16_t* __restrict__ bk, int64_t bk_stride, int chunk_cols,
                  const uint32_t* __restrict__ thresh, int32_t* __restrict__ cnt,
                  u32x2* __restrict__ cand, uint16_t* __restrict__ samples, int ns_stride,
                  Pages pg) {
  constexpr int QT = 4 * MT * NW;   // queries per workgroup
  constexpr int CPT = 16 / NW;      // 16-byte chunks of a stage per thread
  constexpr int kWaveCols = 4 * CPT;   // stage columns each wave loads
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int stride = kSample ? kPrefillSampleStride : 1;
  constexpr int kPend = kSample ? 1 : kPending<NW>;
  // paged: the physical pages of the chunk's blocks (pages hold >= 64 blocks)
  constexpr int kPgSlots = kPaged ? kMaxChunkCols * stride / 64 + 1 : 1;
  __shared__ int s_pg[kPgSlots];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][kStageCols * kColStride];
  __shared__ float s_w[QT][4];
  __shared__ f32x4 s_wc[QT];
  __shared__ float s_tlo[QT];
  __shared__ int s_nc[QT];
  __shared__ uint32_t s_th[QT];
  __shared__ int s_pcnt[QT];
  __shared__ f32x4 s_pacc[QT][kPend];
  __shared__ int s_pidx[QT][kPend];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int s = blockIdx.x / tiles_per_seq, t = blockIdx.x % tiles_per_seq;
  const int qb = cu_q[s], qe_raw = cu_q[s + 1];
  const int qe = min(qe_raw, n_q);
  const int row0 = qb + t * QT;
  if (row0 >= qe || row0 < 0) return;
  const int pos0 = seq_len[s] - (qe_raw - qb) + t * QT;
  const int n_rows = min(QT, qe - row0);
  // rows beyond max_blocks are reported by the select; the others proceed
  const int nc_last = min((pos0 + n_rows) >> 2, max_blocks);
  const int max_cols = kSample ? (nc_last + stride - 1) / stride : nc_last;
  const int v0 = blockIdx.y * chunk_cols;
  if (v0 >= max_cols) return;
  if (kSample && nc_last <= kCandCap) return;
  const int v1 = min(v0 + chunk_cols, max_cols);
  const bool collect_all = !kSample && nc_last <= kCandCap;
  int pg0 = 0;
  if constexpr (kPaged) {
    pg0 = (int)(((int64_t)v0 * stride) >> pg.shift);
    const int pn = (int)((((int64_t)(v1 - 1) * stride) >> pg.shift) - pg0 + 1);
    for (int i = threadIdx.x; i < pn; i += 256)
      s_pg[i] = pg.table[(int64_t)s * pg.stride + pg0 + i];
  }

  if (threadIdx.x < QT) {
    const int j = threadIdx.x;
    const bool ok = j < n_rows;
    const int rj = min(row0 + j, qe - 1);
    const int nc = ok ? (pos0 + j + 1) >> 2 : 0;
    s_nc[j] = (kSample && nc <= kCandCap) ? 0 : nc;
    const uint32_t th = kSample ? 0u : thresh[rj];
    s_th[j] = ok && !kSample ? th : 0xFFFFFFFFu;
    s_pcnt[j] = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float wv = w[(int64_t)rj * 4 + h];
      s_w[j][h] = ok ? wv : 0.f;
      s_wc[j][h] = ok ? wv * kScoreScale : 0.f;
    }
    // Pre-filter bound.  The defined score lies within 2^-21 (relative) of
    // the real c * sum_h w_h ReLU(t_h).  The fast score rounds each ReLU(t_h)
    // and each w_h*c to bf16 (RNE, relative error <= 2^-9 each; bf16 keeps
    // float32's exponent range), multiplies exactly and sums in float32, so
    // it is >= (1 - 2^-8) times the real value.  A candidate with score >=
    // tau therefore has fast score >= tau * (1 - 2^-7); the absolute 2^-100
    // covers rounding at subnormal scale.  Rows that keep every candidate
    // pass everything (-1).
    const float tau = __uint_as_float(s_th[j]);
    s_tlo[j] = (!ok || kSample) ? INFINITY
                                : (nc <= kCandCap ? -1.f : tau * (1.f - 0x1p-7f) - 0x1p-100f);
  }

  // A fragments of this wave's m-tiles (rows (wave*MT + mt)*16 + col)
  u32x4 af[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int j = (wave * MT + mt) * 4 + (col >> 2);
    const bool ok = j < n_rows;
    const int rj = min(row0 + j, qe - 1);
    const uint16_t* src = idx_q + ((int64_t)rj * 4 + (col & 3)) * kIdxDim + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 v = ldg16(src + 32 * ks);
      af[mt][ks] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  __syncthreads();
  bf16x2 r_wc01[MT], r_wc23[MT];   // w_h * c as packed bf16 pairs
  float r_ntlo[MT];   // -tau_lo
  int r_nc[MT];
  // pending entries of this lane's row (uniform over its 16-lane group):
  // each row belongs to exactly one wave, so the count needs no atomics
  int r_pc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const f32x4 wc = s_wc[(wave * MT + mt) * 4 + grp];
    r_wc01[mt] = __builtin_convertvector((f32x2){wc[0], wc[1]}, bf16x2);
    r_wc23[mt] = __builtin_convertvector((f32x2){wc[2], wc[3]}, bf16x2);
    r_ntlo[mt] = -s_tlo[(wave * MT + mt) * 4 + grp];
    r_nc[mt] = min(s_nc[(wave * MT + mt) * 4 + grp], v1);
    r_pc[mt] = 0;
  }

  const uint16_t* bseq = bk + (kPaged ? 0 : (int64_t)s * bk_stride);
  const int n_stages = (v1 - v0 + kStageCols - 1) / kStageCols;
  // The sequence's block keys as a buffer resource whose range ends after
  // virtual column v1 - 1: loads past it return zeros (such columns are
  // never emitted).  Offsets stay below 2^28 bytes (2^20 blocks x 256 B).
  const int nrec = ((v1 - 1) * stride + 1) * kIdxDim * 2;
  const __amdgpu_buffer_rsrc_t bk_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)bseq, (short)0, nrec, 0x00020000);
  // This thread carries CPT chunks of a stage: column c = kWaveCols*wave +
  // 4*i + lane/16, 16-byte chunk lane%16; its byte offsets relative to the
  // stage's first column are fixed.
  int loff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = kWaveCols * wave + 4 * i + (lane >> 4);
    loff[i] = (c * stride * kIdxDim + (lane & 15) * 8) * 2;
  }
  auto load_stage = [&](u32x4 (&r)[CPT], int st) {
    if constexpr (kPaged && !kSample) {
      // a 64-column stage lies inside one page (pages hold >= 64 blocks and
      // stages start at multiples of 64): the contiguous path's offsets from
      // a per-stage buffer resource at the stage's first physical block
      const int c0 = v0 + st * kStageCols;
      const int pidx = __builtin_amdgcn_readfirstlane((c0 >> pg.shift) - pg0);
      const int64_t pb = ((int64_t)s_pg[pidx] << pg.shift) + (c0 & ((1 << pg.shift) - 1));
      const int nrec_st = (min(v1 - c0, kStageCols) - 1) * kIdxDim * 2 + kIdxDim * 2;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(bseq + pb * kIdxDim), (short)0, nrec_st, 0x00020000);
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, loff[i], 0, 0));
    } else if constexpr (kPaged) {
      // sample pass: each column is its own block (32 apart), looked up in
      // the LDS page slice; columns past v1 - 1 read column v1 - 1 and are zeroed
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = kWaveCols * wave + 4 * i + (lane >> 4);
        const int vcol = v0 + st * kStageCols + c;
        const int64_t blk = (int64_t)min(vcol, v1 - 1) * stride;
        const int64_t pb = ((int64_t)s_pg[(int)(blk >> pg.shift) - pg0] << pg.shift) +
                           (blk & (((int64_t)1 << pg.shift) - 1));
        const u32x4 v = ldg16(bseq + pb * kIdxDim + (lane & 15) * 8);
        r[i] = vcol < v1 ? v : u32x4{0, 0, 0, 0};
      }
    } else {
      const int base = (v0 + st * kStageCols) * stride * kIdxDim * 2;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        r[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(bk_rsrc, base + loff[i], 0, 0));
      }
    }
  };
  auto store_stage = [&](const u32x4 (&r)[CPT], int st) {
    uint16_t* dst = s_b[st & 1];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = kWaveCols * wave + 4 * i + (lane >> 4);
      *(u32x4*)(dst + c * kColStride + (lane & 15) * 8) = r[i];
    }
  };
  // the defined score of row j for block b, and where it goes
  auto emit_exact = [&](const f32x4& acc, int j, int vcol, int b) {
    const int nc = s_nc[j];
    if (!(vcol < v1 && b < nc)) return;
    const uint32_t key = __float_as_uint(block_score(acc, s_w[j]));
    const int64_t rbase = (int64_t)(row0 + j) * kCandCap;
    if (kSample) {
      samples[(int64_t)(row0 + j) * ns_stride + vcol] = (uint16_t)(key >> 16);
    } else if (nc <= kCandCap) {
      cand[rbase + b] = u32x2{key, (uint32_t)b};
    } else if (key >= s_th[j]) {
      const int g = atomicAdd(&cnt[row0 + j], 1);
      if (g < kCandCap) cand[rbase + g] = u32x2{key, (uint32_t)b};
    }
  };

  // One stage = 4 column tiles, explicitly pipelined: the B fragments of
  // tile t+1 are read from LDS before the MFMAs of tile t are issued, and the
  // epilogue of tile t runs after the MFMAs of tile t+1 are in flight.
  // B fragment of column tile ct: column 16 ct + col, dims 32 ks + 8 grp ..
  // +7; the lane's base address plus a constant per (ct, ks)
  const int b_lane = col * kColStride + 8 * grp;
  auto read_b = [&](const uint16_t* sb, int ct, u32x4 (&bf)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bf[ks] = *(const u32x4*)(sb + b_lane + 16 * ct * kColStride + 32 * ks);
  };
  auto mfma_b = [&](const u32x4 (&bf)[4], f32x4 (&acc)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc[mt] = mfma_16x16x32(af[mt][ks], bf[ks], acc[mt]);
    }
  };
  // mode 0: every score emitted exactly (sample pass, rows that keep all
  // candidates); 1: pre-filter; 2: pre-filter in a chunk whose columns all
  // lie below every row's candidate count and inside whole stages, so the
  // column test is dropped and the pass mask is the pre-filter's ballot
  auto epi = [&](auto mode_tag, const f32x4 (&acc)[MT], int vbase) {
    constexpr int kMode = decltype(mode_tag)::value;
    constexpr bool kFilter = kMode != 0;
    const int vcol = vbase + col;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int j = (wave * MT + mt) * 4 + grp;
      if (!kFilter) {
        emit_exact(acc[mt], j, vcol, vcol * stride);
        continue;
      }
      // fast score on packed bf16: ReLU as a 16-bit integer max (negative
      // patterns, -0 included, become +0), then two bf16 dot2s into float32
      const bf16x2 p01 = __builtin_convertvector((f32x2){acc[mt][0], acc[mt][1]}, bf16x2);
      const bf16x2 p23 = __builtin_convertvector((f32x2){acc[mt][2], acc[mt][3]}, bf16x2);
      const s16x2 z = {0, 0};
      const bf16x2 r01 = __builtin_bit_cast(bf16x2, __builtin_elementwise_max(__builtin_bit_cast(s16x2, p01), z));
      const bf16x2 r23 = __builtin_bit_cast(bf16x2, __builtin_elementwise_max(__builtin_bit_cast(s16x2, p23), z));
      // margin = fast - tau_lo (the sum starts at -tau_lo; its float32
      // rounding, ~2^-24 of tau, is far inside the 2^-7 slack)
      float margin = dot2_bf16(r23, r_wc23[mt], r_ntlo[mt]);
      margin = __builtin_amdgcn_fdot2_f32_bf16(r01, r_wc01[mt], margin, false);
      const uint64_t hit = __ballot(margin >= 0.f);
      if (hit) {         // a few lanes: append raw accumulators
        const bool pass = kMode == 2 ? margin >= 0.f : (margin >= 0.f && vcol < r_nc[mt]);
        // this lane's 16-lane group is its row: rank among the group's passes
        const uint32_t gm = (uint32_t)((kMode == 2 ? hit : __ballot(pass)) >> (16 * grp)) & 0xFFFFu;
        const int slot = r_pc[mt] + __popc(gm & ((1u << col) - 1u));
        if (pass) {
          if (slot < kPend) {
            s_pacc[j][slot] = acc[mt];
            s_pidx[j][slot] = vcol;
          } else {
            // rare: list full.  The row index goes through an empty asm so
            // that the path's addresses are formed here instead of being
            // kept live (spilled) across the loop.
            int jr = j;
            asm volatile("" : "+v"(jr));
            emit_exact(acc[mt], jr, vcol, vcol);
          }
        }
        r_pc[mt] += __popc(gm);
      }
    }
  };
  // The epilogue of a stage's last tile runs in the next stage, behind the
  // MFMAs of its first tile (it reads only registers and this wave's rows).
  auto run = [&](auto mode_tag) {
    u32x4 stage_regs[CPT];
    load_stage(stage_regs, 0);
    store_stage(stage_regs, 0);
    __syncthreads();
    f32x4 a1[MT];
    for (int st = 0; st < n_stages; ++st) {
      const bool more = st + 1 < n_stages;
      if (more) load_stage(stage_regs, st + 1);          // in flight during this stage
      const uint16_t* sb = s_b[st & 1];
      const int cbase = v0 + st * kStageCols;
      u32x4 b0[4], b1[4];
      f32x4 a0[MT];
      read_b(sb, 0, b0);
      read_b(sb, 1, b1);
      mfma_b(b0, a0);                       // tile 0
      if (st > 0) epi(mode_tag, a1, cbase - 16);   // tile 3 of the previous stage
      read_b(sb, 2, b0);
      mfma_b(b1, a1);                       // tile 1
      epi(mode_tag, a0, cbase);
      read_b(sb, 3, b1);
      mfma_b(b0, a0);                       // tile 2
      epi(mode_tag, a1, cbase + 16);
      mfma_b(b1, a1);                       // tile 3
      epi(mode_tag, a0, cbase + 32);
      if (more) store_stage(stage_regs, st + 1);
      __syncthreads();   // stage st+1 visible; stage st's buffer free for st+2
    }
    epi(mode_tag, a1, v0 + n_stages * kStageCols - 16);
  };
  // rows are in position order, so the first row has the fewest candidates
  const bool full_chunk = v1 <= min((pos0 + 1) >> 2, max_blocks) && (v1 - v0) % kStageCols == 0;
  if (kSample || collect_all) run(std::integral_constant<int, 0>{});
  else if (full_chunk) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 1>{});

  if (!kSample && !collect_all) {
    if (col == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) s_pcnt[(wave * MT + mt) * 4 + grp] = r_pc[mt];
    }
    __syncthreads();
    // exact score of every pending entry; each wave takes rows wave, wave+NW, ...
    for (int j = wave; j < QT; j += NW) {
      const int n = min(s_pcnt[j], kPend);
      uint32_t key = 0;
      bool take = false;
      int b = 0;
      if (lane < n) {
        key = __float_as_uint(block_score(s_pacc[j][lane], s_w[j]));
        b = s_pidx[j][lane];
        take = key >= s_th[j];
      }
      if (s_nc[j] <= kCandCap) {
        // a row that keeps every candidate (mixed tile): slot = block id
        if (lane < n) cand[(int64_t)(row0 + j) * kCandCap + b] = u32x2{key, (uint32_t)b};
        continue;
      }
      const unsigned long long m = __ballot(take);
      if (m) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&cnt[row0 + j], __popcll(m));
        base = __shfl(base, 0, 64);
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        if (take && base + rank < kCandCap)
          cand[(int64_t)(row0 + j) * kCandCap + base + rank] = u32x2{key, (uint32_t)b};
      }
    }
  }
}

// ------------------------------------------------------ LDS radix select
// k-th largest value (1-based) among the participating elements, where
// each(f) calls f(participates, value) for every element this thread holds
// and values have `nbits` bits.  11-bit digits from the top.  Needs kBins
// ints of LDS in `hist`.
template <class Each>
__device__ uint32_t block_kth_largest_each(Each each, int k, int nbits, int* hist, int* tmp,
                                           int* res) {
  uint32_t prefix = 0, pmask = 0;
  for (int top = nbits; top > 0;) {
    const int width = top >= 11 ? 11 : top;
    const int shift = top - width;
    const int bins = 1 << width;
    for (int i = threadIdx.x; i < bins; i += 256) hist[i] = 0;
    __syncthreads();
    each([&](bool in, uint32_t v) {
      if (in && (v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & (bins - 1)], 1);
    });
    __syncthreads();
    // thread t owns bins [per*t, per*t + per)
    const int per = (bins + 255) / 256;
    const int b0 = threadIdx.x * per;
    int local = 0;
    for (int b = b0; b < b0 + per && b < bins; ++b) local += hist[b];
    int total;
    const int excl = block_excl_scan_256(local, tmp, total);
    int run = total - excl - local;   // elements in bins above mine
    for (int b = min(b0 + per, bins) - 1; b >= b0; --b) {
      const int h = hist[b];
      if (run < k && run + h >= k) { res[0] = b; res[1] = run; }
      run += h;
    }
    __syncthreads();
    const uint32_t d = (uint32_t)res[0];
    k -= res[1];
    prefix |= d << shift;
    pmask |= (uint32_t)(bins - 1) << shift;
    top = shift;
    __syncthreads();
  }
  return prefix;
}

// The same over get(i) -> {participates, value} for i < n, thread t taking
// i = t, t + 256, ...
template <class Get>
__device__ uint32_t block_kth_largest(Get get, int n, int k, int nbits, int* hist, int* tmp,
                                      int* res) {
  return block_kth_largest_each(
      [&](auto f) {
        for (int i = threadIdx.x; i < n; i += 256) {
          bool in;
          const uint32_t v = get(i, in);
          f(in, v);
        }
      },
      k, nbits, hist, tmp, res);
}

// Block-wide min and max of one value per thread (ends with a barrier).
__device__ void block_min_max(uint32_t lo, uint32_t hi, int* tmp, uint32_t& out_lo,
                              uint32_t& out_hi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
  }
  if (lane == 0) { tmp[wave] = (int)lo; tmp[4 + wave] = (int)hi; }
  __syncthreads();
  out_lo = min(min((uint32_t)tmp[0], (uint32_t)tmp[1]), min((uint32_t)tmp[2], (uint32_t)tmp[3]));
  out_hi = max(max((uint32_t)tmp[4], (uint32_t)tmp[5]), max((uint32_t)tmp[6], (uint32_t)tmp[7]));
  __syncthreads();
}

// k-th largest (1 <= k <= n) of n keys < 2^31, where each(f) calls f(key)
// for every key this thread holds (the workgroup's threads hold all n
// between them, each key once).  Range-adaptive
// histogram passes: the current key range [lo, hi] (first the keys' min and
// max) is cut into at most 2048 bins of 2^s keys, bin = (key - lo) >> s, so
// that keys crowded in a narrow range still spread over many bins.  Each pass
// finds the bin holding the k-th largest and narrows the range to it; a bin
// of single values (s = 0) is the answer, and a bin of at most kFinishCap
// keys is ranked exactly (each thread holds one key and counts the others).
// Ends with a barrier.
struct KthLds {
  int* hist;       // kBins
  uint32_t* bin;   // kFinishCap
  int* tmp;        // 8
  int* res;        // 2
  int* bin_n;      // 1
};

template <class Each>
__device__ uint32_t kth_largest_each(Each each, int k, const KthLds& sh) {
  const int tid = threadIdx.x;
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  each([&](uint32_t v) { lo = min(lo, v); hi = max(hi, v); });
  block_min_max(lo, hi, sh.tmp, lo, hi);
  for (;;) {
    const uint32_t span = hi - lo;
    const int s = span < (uint32_t)kBins ? 0 : 32 - __clz((int)(span >> 11));   // span >> s < 2048
    for (int i = tid; i < kBins; i += 256) sh.hist[i] = 0;
    if (tid == 0) *sh.bin_n = 0;
    __syncthreads();
    each([&](uint32_t v) {
      if (v >= lo && v <= hi) atomicAdd(&sh.hist[(v - lo) >> s], 1);
    });
    __syncthreads();
    constexpr int per = kBins / 256;
    const int b0 = tid * per;
    int local = 0;
#pragma unroll
    for (int b = 0; b < per; ++b) local += sh.hist[b0 + b];
    int total;
    const int excl = block_excl_scan_256(local, sh.tmp, total);
    int run = total - excl - local;   // keys in the bins above this thread's
#pragma unroll
    for (int b = per - 1; b >= 0; --b) {
      const int h = sh.hist[b0 + b];
      if (run < k && run + h >= k) { sh.res[0] = b0 + b; sh.res[1] = run; }
      run += h;
    }
    __syncthreads();
    const uint32_t B = (uint32_t)sh.res[0];
    k -= sh.res[1];
    const int hb = sh.hist[B];
    __syncthreads();
    const uint32_t blo = lo + (B << s);
    if (s == 0) return blo;
    if (hb <= kFinishCap) {
      const uint32_t bhi = blo + ((1u << s) - 1u);
      each([&](uint32_t v) {
        if (v >= blo && v <= bhi) sh.bin[atomicAdd(sh.bin_n, 1)] = v;
      });
      __syncthreads();
      if (tid < hb) {
        const uint32_t x = sh.bin[tid];
        int gt = 0, ge = 0;
        for (int j = 0; j < hb; ++j) {
          const uint32_t y = sh.bin[j];
          gt += y > x;
          ge += y >= x;
        }
        if (gt < k && k <= ge) sh.res[0] = (int)x;   // every writer has the same x
      }
      __syncthreads();
      const uint32_t T = (uint32_t)sh.res[0];
      __syncthreads();
      return T;
    }
    lo = blo;
    hi = blo + ((1u << s) - 1u);
  }
}

// kth_largest_each over get(0..n), thread t taking i = t, t + 256, ...
template <class Get>
__device__ uint32_t kth_largest_fast(Get get, int n, int k, const KthLds& sh) {
  return kth_largest_each(
      [&](auto f) {
        for (int i = threadIdx.x; i < n; i += 256) f(get(i));
      },
      k, sh);
}

// f(v) for each of the n uint32 values at p (16-byte aligned, readable up
// to n rounded up to 4) by a 256-thread workgroup, 8 16-byte loads in flight
// per thread: a pass over values in global memory then costs a few memory
// round trips instead of one per 256 values.
template <class F>
__device__ __forceinline__ void for_each_u32(const uint32_t* __restrict__ p, int n, F f) {
  const u32x4* p4 = reinterpret_cast<const u32x4*>(p);
  const int nq = (n + 3) >> 2;
  for (int q0 = 0; q0 < nq; q0 += 256 * 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + 256 * u + threadIdx.x;
      v[u] = q < nq ? p4[q] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + 256 * u + threadIdx.x;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e < n) f(v[u][e]);
    }
  }
}

// kth_largest_each for values in global memory, each pass through
// for_each_u32.  Ends with a barrier.
__device__ uint32_t kth_largest_global(const uint32_t* __restrict__ p, int n, int k,
                                       const KthLds& sh) {
  return kth_largest_each([&](auto f) { for_each_u32(p, n, f); }, k, sh);
}

// The k (<= kMaxBudget) distinct ids in ids[] (each < n), written to
// out[0..k) in ascending order by a 256-thread workgroup: ids are bucketed on
// their top 11 bits (counts, a scan, a scatter through LDS atomics), and an
// id's place is its bucket's start plus the number of smaller ids in its
// bucket (a bucket holds a few ids).  hist: kBins ints; tmp: k ints.
__device__ void sort_ids_to(const int* ids, int k, int n, int* hist, int* tmp, int* scan_tmp,
                            int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const int top = 32 - __clz((n - 1) | 1);          // bits of the largest id
  const int shift = top > 11 ? top - 11 : 0;
  const int nb = ((n - 1) >> shift) + 1;            // <= kBins
  for (int b = tid; b < nb; b += 256) hist[b] = 0;
  __syncthreads();
  for (int i = tid; i < k; i += 256) atomicAdd(&hist[ids[i] >> shift], 1);
  __syncthreads();
  // bucket starts: thread t owns buckets [per*t, per*t + per)
  constexpr int per = kBins / 256;
  const int b0 = tid * per;
  int local = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) local += b0 + j < nb ? hist[b0 + j] : 0;
  int total;
  int run = block_excl_scan_256(local, scan_tmp, total);
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (b0 + j < nb) {
      const int h = hist[b0 + j];
      hist[b0 + j] = run;
      run += h;
    }
  }
  __syncthreads();
  for (int i = tid; i < k; i += 256) {
    const int id = ids[i];
    tmp[atomicAdd(&hist[id >> shift], 1)] = id;   // hist[b] ends as bucket b's end
  }
  __syncthreads();
  for (int p = tid; p < k; p += 256) {
    const int id = tmp[p];
    const int b = id >> shift;
    const int s0 = b > 0 ? hist[b - 1] : 0, s1 = hist[b];
    int rank = s0;
    for (int q = s0; q < s1; ++q) rank += tmp[q] < id ? 1 : 0;
    out[rank] = id;
  }
}

// ------------------------------------------------------------ threshold
// Per row: rows with <= kCandCap candidates keep them all (count preset to
// n_c, tau = 0); other rows get tau = the r-th largest sampled score.
// Samples are the top 16 bits of the sampled score keys; tau is the lower edge
// of the r-th largest one, so at least r*32 candidates are expected above it.
//
// Up to 8192 samples (rows to about 1M tokens): each thread holds 32 samples
// as packed 16-bit pairs and tau16 = max{v : #(samples >= v) >= r} is found by
// a binary search on v; each step counts two samples per 32-bit word (a
// borrow test and a population count) and does one block reduction.  Scores cluster in a few exponents, so radix
// histograms would serialise on a few bins; counting has no contention.
// Longer rows use the LDS radix select over the samples in global memory.
constexpr int kBsearchSamples = 32 * 256;

__global__ void __launch_bounds__(256)
threshold_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len, int n_seq,
                 int max_blocks, int budget, const uint16_t* __restrict__ samples, int ns_stride,
                 uint32_t* __restrict__ thresh, int32_t* __restrict__ cnt) {
  __shared__ int hist[kBins];
  __shared__ int tmp[8];
  __shared__ int res[2];
  __shared__ int red[2][4];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowGeom g = row_geom(cu_q, seq_len, n_seq, row, max_blocks);
  if (!g.ok) {
    if (threadIdx.x == 0) { thresh[row] = 0xFFFFFFFFu; cnt[row] = 0; }
    return;
  }
  if (g.n_c <= kCandCap) {
    if (threadIdx.x == 0) { thresh[row] = 0u; cnt[row] = g.n_c; }
    return;
  }
  if (threadIdx.x == 0) cnt[row] = 0;
  const int k = min(budget, g.n_c);
  const int ns = (g.n_c + kPrefillSampleStride - 1) / kPrefillSampleStride;
  const int r = min(ns, (k + kSampleExtra + kPrefillSampleStride - 1) / kPrefillSampleStride);
  const uint16_t* sp = samples + (int64_t)row * ns_stride;
  uint32_t t16;
  if (ns <= kBsearchSamples) {
    // samples 32t .. 32t+31 as 16 words of two; rows are 16-byte aligned and
    // padded to a multiple of 8, so a run that starts below ns is readable
    // whole.  Samples are scores >= 0, so bit 15 of each half is clear:
    // with xs = w | 0x80008000, bit 15 of each half of xs - mid*0x10001 is
    // set exactly when that sample is >= mid (no borrow crosses halves, as
    // 1 <= mid <= 0x8000).  Samples past ns become 0 (never >= mid).
    uint32_t xs[16];
    int mx = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i0 = 32 * threadIdx.x + 8 * v;
      u32x4 q = {0u, 0u, 0u, 0u};
      if (i0 < ns) q = ldg16(sp + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 2 * e;
        const uint32_t lo16 = i < ns ? (q[e] & 0xFFFFu) : 0u;
        const uint32_t hi16 = i + 1 < ns ? (q[e] >> 16) : 0u;
        mx = max(mx, (int)max(lo16, hi16));
        xs[4 * v + e] = (lo16 | (hi16 << 16)) | 0x80008000u;
      }
    }
    auto block_sum = [&](int c, int it) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
      if (lane == 0) red[it & 1][wave] = c;
      __syncthreads();   // double-buffered: the next step writes the other half
      return red[it & 1][0] + red[it & 1][1] + red[it & 1][2] + red[it & 1][3];
    };
    // hi = one past the largest sample (block maximum)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) red[1][wave] = mx;
    __syncthreads();
    int lo = 0, hi = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3])) + 1;
    for (int it = 0; hi - lo > 1; ++it) {
      const int mid = (lo + hi) >> 1;
      const uint32_t mm = (uint32_t)mid * 0x10001u;
      int c = 0;
#pragma unroll
      for (int p = 0; p < 16; ++p) c += __popc((xs[p] - mm) & 0x80008000u);
      if (block_sum(c, it) >= r) lo = mid;
      else hi = mid;
    }
    t16 = (uint32_t)lo;
  } else {
    t16 = block_kth_largest([&](int i, bool& in) { in = true; return (uint32_t)sp[i]; }, ns, r, 16,
                            hist, tmp, res);
  }
  if (threadIdx.x == 0) thresh[row] = t16 << 16;
}

// ------------------------------------------------------------- fallback
// Exact select for a row whose list came out short or overflowed: recompute
// the score of every candidate on every radix pass (VALU dot products, one
// block per thread), then emit in ascending block order.  Slow but needs no
// score storage; the sampled threshold makes it rare.
__device__ __forceinline__ uint32_t recompute_key(const uint16_t* __restrict__ q4,
                                                  const float* __restrict__ w4,
                                                  const uint16_t* __restrict__ kb) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int d8 = 0; d8 < kIdxDim / 8; ++d8) {
    const u32x4 kv = ldg16(kb + 8 * d8);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 qv = ldg16(q4 + h * kIdxDim + 8 * d8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[h] += bf16_lo(qv[e]) * bf16_lo(kv[e]);
        acc[h] += bf16_hi(qv[e]) * bf16_hi(kv[e]);
      }
    }
  }
  return __float_as_uint(block_score(acc, w4));
}

__device__ void exact_select_recompute(const uint16_t* __restrict__ q4, const float* __restrict__ w4,
                                       const uint16_t* __restrict__ bseq, const Pages& pg,
                                       int seq, int n_c, int k,
                                       int32_t* __restrict__ out, int budget, int* hist, int* tmp,
                                       int* res) {
  auto key_of = [&](int b, bool& in) {
    in = true;
    const int64_t pb = pg.table ? phys_block(pg, seq, b) : b;
    return recompute_key(q4, w4, bseq + pb * kIdxDim);
  };
  const uint32_t tau = block_kth_largest(key_of, n_c, k, 31, hist, tmp, res);
  int above = 0;
  for (int b = threadIdx.x; b < n_c; b += 256) { bool in; above += key_of(b, in) > tau; }
  int tot_above;
  block_excl_scan_256(above, tmp, tot_above);
  const int need = k - tot_above;   // ties to take, lowest block ids first
  int ties_run = 0, out_run = 0;
  for (int b0 = 0; b0 < n_c; b0 += 256) {
    const int b = b0 + threadIdx.x;
    bool in;
    const uint32_t key = b < n_c ? key_of(b, in) : 0u;
    const bool is_tie = b < n_c && key == tau;
    const bool is_above = b < n_c && key > tau;
    int tie_tot;
    const int tie_rank = ties_run + block_excl_scan_256(is_tie ? 1 : 0, tmp, tie_tot);
    const bool take = is_above || (is_tie && tie_rank < need);
    int take_tot;
    const int slot = out_run + block_excl_scan_256(take ? 1 : 0, tmp, take_tot);
    if (take && slot < k) out[slot] = b;
    ties_run += tie_tot;
    out_run += take_tot;
  }
  for (int i = k + threadIdx.x; i < budget; i += 256) out[i] = -1;
}

// ------------------------------------------------------ list selection
// A row's candidate list as the workgroup holds it: thread t keeps the
// entries 2q and 2q + 1, q = t + 256 u (u < kPairsPer), as one 16-byte pair
// {key, id, key, id} in registers; entries at or past c are not part of it.
constexpr int kPairsPer = kCandCap / 2 / 256;
struct RegList {
  u32x4 e[kPairsPer];
  int c;
  // f(key, id) for every entry this thread holds
  template <class F>
  __device__ __forceinline__ void each(F f) const {
#pragma unroll
    for (int u = 0; u < kPairsPer; ++u) {
      const int i = 2 * ((int)threadIdx.x + 256 * u);
      if (i < c) f(e[u][0], (int)e[u][1]);
      if (i + 1 < c) f(e[u][2], (int)e[u][3]);
    }
  }
};

// Exact top-k (score desc, block asc) of a list of c >= k candidates, written
// to out[0..k) in ascending block order and -1 up to budget.  Radix select
// on the score key, then on the block id among ties at the threshold; the k
// ids sorted by buckets.
__device__ void select_from_list(const RegList& L, int k, int* ids, int* ids_tmp, int n_ids,
                                 int* n_out, const KthLds& lds, int32_t* __restrict__ out,
                                 int budget) {
  int* hist = lds.hist;
  int* tmp = lds.tmp;
  int* res = lds.res;
  uint32_t tau = 0, iota_cut = 0xFFFFFFFFu;
  const bool all = L.c == k;
  if (threadIdx.x == 0) *n_out = 0;
  if (!all) {
    tau = kth_largest_each([&](auto f) { L.each([&](uint32_t key, int) { f(key); }); }, k, lds);
    int above = 0, ties = 0;
    L.each([&](uint32_t key, int) {
      above += key > tau;
      ties += key == tau;
    });
    int tot_above, tot_ties;
    block_excl_scan_256(above, tmp, tot_above);
    block_excl_scan_256(ties, tmp, tot_ties);
    const int need = k - tot_above;
    if (need < tot_ties) {
      // the `need` lowest block ids among the ties: k-th largest of (2^22-1-id)
      const uint32_t v = block_kth_largest_each(
          [&](auto f) {
            L.each([&](uint32_t key, int id) { f(key == tau, 0x3FFFFFu - (uint32_t)id); });
          },
          need, 22, hist, tmp, res);
      iota_cut = 0x3FFFFFu - v;
    }
  }
  __syncthreads();
  L.each([&](uint32_t key, int id) {
    const bool take = all || key > tau || (key == tau && (uint32_t)id <= iota_cut);
    if (take) {
      const int slot = atomicAdd(n_out, 1);
      if (slot < kMaxBudget) ids[slot] = id;
    }
  });
  __syncthreads();
  if (k > 0) sort_ids_to(ids, k, n_ids, hist, ids_tmp, tmp, out);
  for (int i = k + threadIdx.x; i < budget; i += 256) out[i] = -1;
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exact top-k over keys get(0..n) of items id(0..n) listed in ascending
// block order: threshold tau = k-th largest key, then every key > tau and the
// first ties in list order, emitted in that order (so ids stay ascending).
// The 4 waves take contiguous quarters; ranks come from wave ballots.
template <class Get, class Id>
__device__ void select_ordered(Get get, Id id, int n, int k, int* hist, int* tmp, int* res,
                               int* wcnt, int32_t* __restrict__ out, int budget) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t tau =
      k >= n ? 0u : block_kth_largest([&](int i, bool& in) { in = true; return get(i); }, n, k, 31,
                                      hist, tmp, res);
  const int per = (n + 3) / 4;
  const int s0 = min(n, wave * per), s1 = min(n, s0 + per);
  int a = 0, t = 0;
  for (int i = s0 + lane; i < s1; i += 64) {
    const uint32_t key = get(i);
    a += key > tau;
    t += key == tau;
  }
  a = wave_sum(a);
  t = wave_sum(t);
  if (lane == 0) { wcnt[2 * wave] = a; wcnt[2 * wave + 1] = t; }
  __syncthreads();
  int need = k;   // ties to take, in list order: k - #above overall
  for (int w2 = 0; w2 < 4; ++w2) need -= wcnt[2 * w2];
  int tie_base = 0, out_base = 0;
  for (int w2 = 0; w2 < wave; ++w2) {
    const int tw = wcnt[2 * w2 + 1];
    out_base += wcnt[2 * w2] + min(max(need - tie_base, 0), tw);
    tie_base += tw;
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r0 = s0; r0 < s1; r0 += 64) {
    const int i = r0 + lane;
    const bool valid = i < s1;
    const uint32_t key = valid ? get(i) : 0u;
    const bool is_above = valid && key > tau;
    const bool is_tie = valid && key == tau;
    const unsigned long long mt = __ballot(is_tie);
    const bool take = is_above || (is_tie && tie_base + __popcll(mt & below) < need);
    const unsigned long long mk = __ballot(take);
    if (take) {
      const int slot = out_base + __popcll(mk & below);
      if (slot < k) out[slot] = id(i);
    }
    tie_base += __popcll(mt);
    out_base += __popcll(mk);
  }
  for (int i = k + threadIdx.x; i < budget; i += 256) out[i] = -1;
  __syncthreads();
}

// --------------------------------------------------------- final select
struct SelectShared {
  int hist[kBins];
  uint32_t bin[kFinishCap];
  int ids[kMaxBudget];
  int ids_tmp[kMaxBudget];
  int tmp[8];
  int res[2];
  int n_out;
  int bin_n;
};

__global__ void __launch_bounds__(256)
final_select_kernel(const uint16_t* __restrict__ idx_q, const float* __restrict__ w,
                    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len,
                    int n_seq, int max_blocks, int budget, const uint16_t* __restrict__ bk,
                    int64_t bk_stride, const int32_t* __restrict__ cnt,
                    const u32x2* __restrict__ cand, int32_t* __restrict__ sel,
                    int32_t* __restrict__ sel_count, Pages pg) {
  __shared__ SelectShared sh;
  const int row = blockIdx.x;
  const RowGeom g = row_geom(cu_q, seq_len, n_seq, row, max_blocks);
  int32_t* out = sel + (int64_t)row * budget;
  if (!g.ok) {
    for (int i = threadIdx.x; i < budget; i += 256) out[i] = -1;
    if (threadIdx.x == 0) sel_count[row] = -1;
    return;
  }
  const int k = min(budget, g.n_c);
  const int c = cnt[row];
  if (k > 0 && (c < k || c > kCandCap)) {
    exact_select_recompute(idx_q + (int64_t)row * 4 * kIdxDim, w + (int64_t)row * 4,
                           bk + (pg.table ? 0 : (int64_t)g.seq * bk_stride), pg, g.seq, g.n_c, k,
                           out, budget, sh.hist, sh.tmp, sh.res);
    if (threadIdx.x == 0) sel_count[row] = k;
    return;
  }
  // the list into registers, every 16-byte load (two entries) in flight at
  // once: one memory round trip per row.  Rows start 16-byte aligned and hold
  // kCandCap (even) slots, so the pair holding entry c - 1 is readable whole.
  RegList L;
  L.c = c;
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(cand + (int64_t)row * kCandCap);
    const int n_pairs = (c + 1) >> 1;
#pragma unroll
    for (int u = 0; u < kPairsPer; ++u) {
      const int q = threadIdx.x + 256 * u;
      L.e[u] = q < n_pairs ? src[q] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  select_from_list(L, k, sh.ids, sh.ids_tmp, g.n_c, &sh.n_out,
                   KthLds{sh.hist, sh.bin, sh.tmp, sh.res, &sh.bin_n}, out, budget);
  if (threadIdx.x == 0) sel_count[row] = k;
}

// ---------------------------------------------------- dense select (decode)
// One workgroup per row over the dense scores of score_dense_kernel:
//   1. tau_s = the r-th largest sample (every 16th score), r chosen so that
//      about K + 768 scores reach it (the samples are loaded first, so this
//      overlaps the loads of the row);
//   2. the scores >= tau_s are compacted, in block order, into an LDS list:
//      32768 scores per pass are staged in LDS so that each thread owns 128
//      consecutive scores; a block scan of the per-thread hit counts gives
//      each thread its list offset;
//   3. if the list holds >= K entries it holds the true top K (all of them
//      score >= the K-th score >= tau_s); they are found exactly and emitted
//      in list order, i.e. ascending block order;
//   4. a short or overflowing list falls back to an exact ordered select
//      over all scores of the row.
// The k-th largest values come from one 11-bit histogram pass plus an exact
// finish inside the boundary bin (or the full radix select when that bin is
// crowded).
constexpr int kDenseList = 2560;
constexpr int kDenseExtra = 768;
constexpr int kDensePassQ = 8192;   // quads per pass (32768 scores; 32 per thread)
// Rows longer than kLongRow scores are compacted in pieces of one pass each,
// one workgroup per piece, into per-piece segments of the row's list (in
// block order, so the list needs no sort); a second launch selects from the
// segments.  A piece's workgroup finds tau_s from the samples itself.
constexpr int kPieceScores = 4 * kDensePassQ;
constexpr int kLongRow = 2 * kPieceScores;
constexpr int kMaxPieces = 64;
// rows with up to this many samples find their threshold in LDS
constexpr int kLdsSamples = 4096;

struct DenseShared {
  u32x4 rowq[kDensePassQ];
  union {
    struct {
      uint32_t key[kDenseList];
      int pos[kDenseList];
    } l;
    uint32_t smp[2048];
  } u;
  int hist[kBins];
  uint32_t bin[kFinishCap];
  int tmp[8];
  int res[2];
  int wcnt[8];
  int bin_n;
};

// Exact top-k of the LDS list (key, pos) of c entries in block order,
// emitted in list order to out[0..k), -1 up to budget.
__device__ void select_dense_list(int c, int k, DenseShared& sh, int32_t* __restrict__ out,
                                  int budget) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t tau =
      k >= c ? 0u : kth_largest_fast([&](int i) { return sh.u.l.key[i]; }, c, k,
                                     KthLds{sh.hist, sh.bin, sh.tmp, sh.res, &sh.bin_n});
  const int per = (c + 255) / 256 * 64;
  const int s0 = min(c, wave * per), s1 = min(c, s0 + per);
  int a = 0, t = 0;
  for (int i = s0 + lane; i < s1; i += 64) {
    const uint32_t v = sh.u.l.key[i];
    a += v > tau;
    t += v == tau;
  }
  a = wave_sum(a);
  t = wave_sum(t);
  if (lane == 0) { sh.wcnt[2 * wave] = a; sh.wcnt[2 * wave + 1] = t; }
  __syncthreads();
  int need = k;
  for (int w2 = 0; w2 < 4; ++w2) need -= sh.wcnt[2 * w2];
  int tie_base = 0, out_base = 0;
  for (int w2 = 0; w2 < wave; ++w2) {
    const int tw = sh.wcnt[2 * w2 + 1];
    out_base += sh.wcnt[2 * w2] + min(max(need - tie_base, 0), tw);
    tie_base += tw;
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r0 = s0; r0 < s1; r0 += 64) {
    const int i = r0 + lane;
    const bool ok = i < s1;
    const uint32_t v = ok ? sh.u.l.key[i] : 0u;
    const bool is_tie = ok && v == tau;
    const unsigned long long mt = __ballot(is_tie);
    const bool take = (ok && v > tau) || (is_tie && tie_base + __popcll(mt & below) < need);
    const unsigned long long mk = __ballot(take);
    if (take) {
      const int slot = out_base + __popcll(mk & below);
      if (slot < k) out[slot] = sh.u.l.pos[i];
    }
    tie_base += __popcll(mt);
    out_base += __popcll(mk);
  }
  for (int i = k + threadIdx.x; i < budget; i += 256) out[i] = -1;
}

__global__ void __launch_bounds__(256)
select_dense_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len,
                    int n_seq, int max_blocks, int budget, const uint32_t* __restrict__ dense,
                    int64_t dense_stride, const uint32_t* __restrict__ dsmp,
                    int64_t dsmp_stride, int32_t* __restrict__ sel,
                    int32_t* __restrict__ sel_count, int n_pieces, u32x2* __restrict__ seg,
                    int32_t* __restrict__ segcnt) {
  __shared__ DenseShared sh;
  const int tid = threadIdx.x;
  const int row = blockIdx.x / n_pieces, piece = blockIdx.x - row * n_pieces;
  const RowGeom g = row_geom(cu_q, seq_len, n_seq, row, max_blocks);
  // split rows: this workgroup compacts one piece; other rows: piece 0 does all
  const bool split = seg != nullptr && g.ok && g.n_c > kLongRow;
  if (split ? piece * kPieceScores >= g.n_c : piece != 0) return;
  int32_t* out = sel + (int64_t)row * budget;
  if (!g.ok) {
    for (int i = tid; i < budget; i += 256) out[i] = -1;
    if (tid == 0) sel_count[row] = -1;
    return;
  }
  const int n = g.n_c;
  const int k = min(budget, n);
  // 16-byte aligned; readable up to the row stride (a multiple of 64 >= n)
  const uint32_t* drow = dense + (int64_t)row * dense_stride;
  const u32x4* drow4 = reinterpret_cast<const u32x4*>(drow);
  const uint32_t* srow = dsmp + (int64_t)row * dsmp_stride;
  if (tid == 0 && !split) sel_count[row] = k;

  if (n <= kDenseList) {   // short rows: the whole row is the list
    for (int i = tid; i < n; i += 256) { sh.u.l.key[i] = drow[i]; sh.u.l.pos[i] = i; }
    __syncthreads();
    select_dense_list(n, k, sh, out, budget);
    return;
  }

  const int nq = (n + 3) >> 2;
  const int ns = (n + kSampleStride - 1) / kSampleStride;
  const int r = min(ns, (k + kDenseExtra + kSampleStride - 1) / kSampleStride);
  // samples first (the threshold waits only for them), then the row
  uint32_t sv[8];
  if (ns <= 2048) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sv[j] = srow[min(256 * j + tid, ns - 1)];
  }
  constexpr int kQ = kDensePassQ / 256;
  u32x4 kv[kQ];
  auto load_pass = [&](int q0) {
#pragma unroll
    for (int u = 0; u < kQ; ++u) kv[u] = drow4[min(q0 + 256 * u + tid, nq - 1)];
  };
  // quads of this workgroup: the whole row, or one piece of a split row
  const int q_first = split ? piece * kDensePassQ : 0;
  const int q_end = split ? min(nq, q_first + kDensePassQ) : nq;
  load_pass(q_first);
  uint32_t tau_s;
  if (ns <= 2048) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (256 * j + tid < ns) sh.u.smp[256 * j + tid] = sv[j];
    __syncthreads();
    tau_s = kth_largest_fast([&](int i) { return sh.u.smp[i]; }, ns, r,
                             KthLds{sh.hist, sh.bin, sh.tmp, sh.res, &sh.bin_n});
  } else if (ns <= kLdsSamples) {
    // up to kLdsSamples samples (rows up to 65,536 blocks, e.g. multi-token
    // rows one block past 32,768): staged in the pass buffer, which is free
    // until the compaction, and searched in LDS
    uint32_t* smp = reinterpret_cast<uint32_t*>(sh.rowq);
    uint32_t tv[kLdsSamples / 256];
#pragma unroll
    for (int j = 0; j < kLdsSamples / 256; ++j) {
      const int i = tid + 256 * j;
      tv[j] = i < ns ? srow[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kLdsSamples / 256; ++j) {
      const int i = tid + 256 * j;
      if (i < ns) smp[i] = tv[j];
    }
    __syncthreads();
    tau_s = kth_largest_fast([&](int i) { return smp[i]; }, ns, r,
                             KthLds{sh.hist, sh.bin, sh.tmp, sh.res, &sh.bin_n});
    __syncthreads();   // the pass buffer is rewritten by the compaction
  } else {
    tau_s = kth_largest_global(srow, ns, r, KthLds{sh.hist, sh.bin, sh.tmp, sh.res, &sh.bin_n});
  }

  // compaction; tau_s = 0 would pass every score (more than the list holds)
  int run = tau_s == 0 ? kDenseList + 1 : 0;
  for (int q0 = q_first; q0 < q_end && tau_s != 0; q0 += kDensePassQ) {
    if (q0 > q_first) load_pass(q0);
    // stage: quad ql of the pass goes to thread ql/32's run, slot swizzled by
    // the owner so that both the writes here and the reads below are free of
    // bank conflicts; scores past n become 0 (never >= tau_s >= 1)
#pragma unroll
    for (int u = 0; u < kQ; ++u) {
      const int ql = 256 * u + tid;
      u32x4 v = kv[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = 4 * (q0 + ql) + e < n ? v[e] : 0u;
      const int seg = ql >> 5;
      sh.rowq[(seg << 5) | ((ql & 31) ^ (seg & 31))] = v;
    }
    __syncthreads();
    // this thread's 128 consecutive scores: hit mask and count
    uint32_t hm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const u32x4 v = sh.rowq[(tid << 5) | (j ^ (tid & 31))];
#pragma unroll
      for (int e = 0; e < 4; ++e) hm[j >> 3] |= (v[e] >= tau_s ? 1u : 0u) << (4 * (j & 7) + e);
    }
    const int c = __popc(hm[0]) + __popc(hm[1]) + __popc(hm[2]) + __popc(hm[3]);
    int total;
    int slot = run + block_excl_scan_256(c, sh.tmp, total);
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      uint32_t m = hm[w4];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        const int j = 8 * w4 + (bit >> 2), e = bit & 3;
        if (slot < kDenseList) {
          const uint32_t* qv = reinterpret_cast<const uint32_t*>(&sh.rowq[(tid << 5) | (j ^ (tid & 31))]);
          sh.u.l.key[slot] = qv[e];
          sh.u.l.pos[slot] = 4 * (q0 + 32 * tid + j) + e;
        }
        ++slot;
      }
    }
    run += total;
    __syncthreads();   // rowq is rewritten by the next pass
  }

  if (split) {
    // the piece's entries, in block order, and their count (above
    // kDenseList: the list cannot hold the row's candidates)
    u32x2* sp = seg + ((int64_t)row * n_pieces + piece) * kDenseList;
    const int m = run <= kDenseList ? run : 0;
    for (int i = tid; i < m; i += 256) sp[i] = u32x2{sh.u.l.key[i], (uint32_t)sh.u.l.pos[i]};
    if (tid == 0) segcnt[(int64_t)row * n_pieces + piece] = run;
    return;
  }
  if (run >= k && run <= kDenseList) {
    select_dense_list(run, k, sh, out, budget);
  } else {
    select_ordered([&](int i) { return drow[i]; }, [](int i) { return i; }, n, k, sh.hist, sh.tmp,
                   sh.res, sh.wcnt, out, budget);
  }
}

// Second step for split rows: the pieces' segments, concatenated in piece
// order, form the row's list of scores >= tau_s in block order; its exact
// top K is emitted as for an unsplit row.  A piece that overflowed, or a
// list short of K or longer than kDenseList, falls back to the exact ordered
// select over the row's dense scores.
__global__ void __launch_bounds__(256)
dense_list_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len,
                  int n_seq, int max_blocks, int budget, const uint32_t* __restrict__ dense,
                  int64_t dense_stride, int n_pieces, const u32x2* __restrict__ seg,
                  const int32_t* __restrict__ segcnt, int32_t* __restrict__ sel,
                  int32_t* __restrict__ sel_count) {
  __shared__ DenseShared sh;
  __shared__ int s_off[kMaxPieces + 1];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const RowGeom g = row_geom(cu_q, seq_len, n_seq, row, max_blocks);
  if (!g.ok || g.n_c <= kLongRow) return;   // done by select_dense_kernel
  const int n = g.n_c;
  const int k = min(budget, n);
  const int np = (n + kPieceScores - 1) / kPieceScores;
  int32_t* out = sel + (int64_t)row * budget;
  if (tid == 0) {
    int tot = 0;
    bool ok = true;
    for (int p = 0; p < np; ++p) {
      const int c = segcnt[(int64_t)row * n_pieces + p];
      ok = ok && c >= 0 && c <= kDenseList;
      s_off[p] = tot;
      tot += ok ? c : 0;
    }
    s_off[np] = (ok && tot >= k && tot <= kDenseList) ? tot : -1;
    sel_count[row] = k;
  }
  __syncthreads();
  const int c = s_off[np];
  if (c >= 0) {
    for (int p = 0; p < np; ++p) {
      const int b0 = s_off[p], cnt = s_off[p + 1] - b0;   // s_off[np] = c
      const u32x2* sp = seg + ((int64_t)row * n_pieces + p) * kDenseList;
      for (int i = tid; i < cnt; i += 256) {
        const u32x2 e = sp[i];
        sh.u.l.key[b0 + i] = e[0];
        sh.u.l.pos[b0 + i] = (int)e[1];
      }
    }
    __syncthreads();
    select_dense_list(c, k, sh, out, budget);
  } else {
    const uint32_t* drow = dense + (int64_t)row * dense_stride;
    select_ordered([&](int i) { return drow[i]; }, [](int i) { return i; }, n, k, sh.hist, sh.tmp,
                   sh.res, sh.wcnt, out, budget);
  }
}

// ------------------------------------------------------------ workspace
struct IndexWs {
  uint32_t* thresh;
  int32_t* cnt;
  u32x2* cand;
  uint16_t* samples;
  uint32_t* dense;
  uint32_t* dsmp;
  u32x2* seg;          // split decode rows: per-piece list segments
  int32_t* segcnt;
  int n_pieces;
  int ns_stride;
  int64_t dense_stride, dsmp_stride;
  size_t bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Small tiles (<= 4 queries per sequence) use dense scores; otherwise the
// sampled-threshold path with per-row candidate lists.
inline bool use_dense(int max_q_len) { return max_q_len <= 4; }

// Pieces per row of a dense select launch: 1 unless rows may exceed kLongRow
// scores (and the pieces fit the list kernel's table).
inline int dense_pieces(int max_blocks) {
  if (max_blocks <= kLongRow) return 1;
  const int np = (max_blocks + kPieceScores - 1) / kPieceScores;
  return np <= kMaxPieces ? np : 1;
}

inline IndexWs index_ws_layout(void* base, int n_q, int max_q_len, int max_blocks) {
  IndexWs ws = {};
  char* p = (char*)base;
  size_t off = 0;
  // sample rows padded to a multiple of 8 (16 bytes)
  ws.ns_stride = ((max_blocks + kPrefillSampleStride - 1) / kPrefillSampleStride + 7) & ~7;
  ws.dense_stride = ((int64_t)max_blocks + 63) / 64 * 64;
  ws.dsmp_stride = ((int64_t)((max_blocks + kSampleStride - 1) / kSampleStride) + 63) / 64 * 64;
  if (use_dense(max_q_len)) {
    ws.dense = (uint32_t*)(p + off);
    off = align256(off + (size_t)n_q * ws.dense_stride * 4);
    ws.dsmp = (uint32_t*)(p + off);
    off = align256(off + (size_t)n_q * ws.dsmp_stride * 4);
    ws.n_pieces = dense_pieces(max_blocks);
    if (ws.n_pieces > 1) {
      ws.seg = (u32x2*)(p + off);
      off = align256(off + (size_t)n_q * ws.n_pieces * kDenseList * 8);
      ws.segcnt = (int32_t*)(p + off);
      off = align256(off + (size_t)n_q * ws.n_pieces * 4);
    }
  } else {
    ws.thresh = (uint32_t*)(p + off); off = align256(off + (size_t)n_q * 4);
    ws.cnt = (int32_t*)(p + off); off = align256(off + (size_t)n_q * 4);
    ws.cand = (u32x2*)(p + off); off = align256(off + (size_t)n_q * kCandCap * 8);
    ws.samples = (uint16_t*)(p + off);
    off = align256(off + (max_blocks > kCandCap ? (size_t)n_q * ws.ns_stride * 2 : 0));
  }
  ws.bytes = off < 256 ? (size_t)256 : off;   // (HIP's host max() is int-only)
  return ws;
}

}  // namespace qsa

extern "C" {

size_t qsa_index_select_workspace(int32_t n_q, int32_t max_q_len, int32_t max_blocks) {
  if (n_q <= 0 || max_q_len <= 0 || max_blocks < 0) return 0;
  return qsa::index_ws_layout(nullptr, n_q, max_q_len, max_blocks).bytes;
}

int qsa_index_select(const void* idx_q, const float* w, const int32_t* cu_q,
                     const int32_t* seq_len, int32_t n_seq, int32_t n_q, int32_t max_q_len,
                     int32_t max_blocks, const void* block_keys, int64_t bk_seq_stride,
                     int32_t budget, int32_t* sel, int32_t* sel_count, void* workspace,
                     size_t ws_bytes, const int32_t* block_table, int64_t table_stride,
                     int32_t page_tokens, void* stream) {
  using namespace qsa_host;
  using namespace qsa;
  if (n_q < 0 || n_seq < 0 || max_q_len < 0 || max_blocks < 0) return QSA_ERR_INVALID_ARG;
  Pages pg;
  if (!make_pages(block_table, table_stride, page_tokens, pg)) return QSA_ERR_INVALID_ARG;
  if (budget < 1 || budget > QSA_MAX_BUDGET) return QSA_ERR_INVALID_ARG;
  if (n_q == 0) return QSA_OK;
  if (n_seq == 0 || max_q_len == 0) return QSA_ERR_INVALID_ARG;
  if (!idx_q || !w || !cu_q || !seq_len || !block_keys || !sel || !sel_count || !workspace)
    return QSA_ERR_INVALID_ARG;
  if (!aligned16(idx_q) || !aligned16(w) || !aligned16(block_keys) || !aligned16(workspace))
    return QSA_ERR_INVALID_ARG;
  if (!stride_ok(bk_seq_stride)) return QSA_ERR_INVALID_ARG;
  if (max_blocks > QSA_MAX_TOKENS / QSA_BLOCK) return QSA_ERR_UNSUPPORTED;
  if (n_seq > 0x7FFFFFFF / 8) return QSA_ERR_UNSUPPORTED;
  const IndexWs ws = index_ws_layout(workspace, n_q, max_q_len, max_blocks);
  if (ws_bytes < ws.bytes) return QSA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;

  if (use_dense(max_q_len)) {
    // decode: dense scores, then one select per row
    if (max_blocks > 0) {
      // launches of few sequences pick their chunk size in the kernel (the
      // grid then holds the 256-column chunks of every row)
      const int adapt = n_seq <= kDenseAdaptSeqs ? 1 : 0;
      const int chunk_cols = adapt ? kDenseChunkSmall : kDenseChunk;
      const int n_chunks = (max_blocks + chunk_cols - 1) / chunk_cols;
      const int64_t n_wg = (int64_t)n_seq * n_chunks;
      if (n_wg > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
      auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(256), 0, st, (const uint16_t*)idx_q, w,
                           cu_q, seq_len, n_seq, n_q, max_blocks, (const uint16_t*)block_keys,
                           bk_seq_stride, ws.dense, ws.dense_stride, ws.dsmp, ws.dsmp_stride,
                           adapt, pg);
      };
      if (pg.table) launch(score_dense_kernel<true>);
      else launch(score_dense_kernel<false>);
    }
    const int np = ws.n_pieces;
    if ((int64_t)n_q * np > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(select_dense_kernel, dim3((unsigned)((int64_t)n_q * np)), dim3(256), 0, st,
                       cu_q, seq_len, n_seq, max_blocks, budget, (const uint32_t*)ws.dense,
                       ws.dense_stride, (const uint32_t*)ws.dsmp, ws.dsmp_stride, sel, sel_count,
                       np, np > 1 ? ws.seg : (u32x2*)nullptr, ws.segcnt);
    if (np > 1)
      hipLaunchKernelGGL(dense_list_kernel, dim3(n_q), dim3(256), 0, st, cu_q, seq_len, n_seq,
                         max_blocks, budget, (const uint32_t*)ws.dense, ws.dense_stride, np,
                         (const u32x2*)ws.seg, (const int32_t*)ws.segcnt, sel, sel_count);
    return launch_status();
  }

#ifndef QSA_FILTER_WAVES
#define QSA_FILTER_WAVES 8
#endif
  constexpr int kFilterWaves = QSA_FILTER_WAVES;   // waves per filter-pass workgroup
  auto row_tiles = [&](int nw) { return (max_q_len + 4 * kPrefillMT * nw - 1) / (4 * kPrefillMT * nw); };
  const int64_t gx = (int64_t)row_tiles(4) * n_seq;
  if (gx > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
#ifndef QSA_PREFILL_CHUNK
#define QSA_PREFILL_CHUNK 2048
#endif
  constexpr int chunk = QSA_PREFILL_CHUNK;   // candidate blocks per workgroup
  static_assert(chunk <= kMaxChunkCols && chunk % kStageCols == 0, "prefill chunk");
  auto gemm = [&](auto sample_tag, auto waves_tag, unsigned gy, int chunk_cols) {
    constexpr bool kS = decltype(sample_tag)::value;
    constexpr int kNW = decltype(waves_tag)::value;
    const int tiles = row_tiles(kNW);
    const dim3 grid((unsigned)((int64_t)tiles * n_seq), gy);
    auto launch = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(64 * kNW), 0, st, (const uint16_t*)idx_q, w, cu_q,
                         seq_len, n_seq, n_q, tiles, max_blocks, (const uint16_t*)block_keys,
                         bk_seq_stride, chunk_cols, ws.thresh, ws.cnt, ws.cand, ws.samples,
                         ws.ns_stride, pg);
    };
    if (pg.table) launch(score_gemm_kernel<kPrefillMT, kNW, kS, true>);
    else launch(score_gemm_kernel<kPrefillMT, kNW, kS, false>);
  };
  // 1. sample pass (only rows with more than kCandCap candidates need it)
  if (max_blocks > kCandCap) {
    gemm(std::true_type{}, std::integral_constant<int, 4>{}, (ws.ns_stride + chunk - 1) / chunk,
         chunk);
  }
  // 2. thresholds (also preset the list counters)
  hipLaunchKernelGGL(threshold_kernel, dim3(n_q), dim3(256), 0, st, cu_q, seq_len, n_seq,
                     max_blocks, budget, ws.samples, ws.ns_stride, ws.thresh, ws.cnt);
  // 3. filter pass.  About K + kSampleExtra of a row's n_c candidates pass
  //    the pre-filter, spread over its n_c / chunk workgroups; the chunk is
  //    halved (down to one stage) until the longest row expects at most
  //    kPassTarget passes per workgroup, so that short rows (a larger share
  //    passes) rarely fill their pending lists.
  if (max_blocks > 0) {
#ifndef QSA_PASS_TARGET
#define QSA_PASS_TARGET 24
#endif
    constexpr int kPassTarget = QSA_PASS_TARGET;
    int fchunk = chunk;
    while (fchunk > kStageCols &&
           (int64_t)fchunk * (budget + kSampleExtra) > (int64_t)kPassTarget * max_blocks)
      fchunk >>= 1;
    const int gy = (max_blocks + fchunk - 1) / fchunk;
    if (gy > 65535) return QSA_ERR_UNSUPPORTED;
    gemm(std::false_type{}, std::integral_constant<int, kFilterWaves>{}, (unsigned)gy, fchunk);
  }
  // 4. exact select per row (rows whose list came out short or overflowed
  //    are selected exactly by recomputing their scores)
  hipLaunchKernelGGL(final_select_kernel, dim3(n_q), dim3(256), 0, st, (const uint16_t*)idx_q, w,
                     cu_q, seq_len, n_seq, max_blocks, budget, (const uint16_t*)block_keys,
                     bk_seq_stride, ws.cnt, ws.cand, sel, sel_count, pg);
  return launch_status();
}

}  // extern "C"
