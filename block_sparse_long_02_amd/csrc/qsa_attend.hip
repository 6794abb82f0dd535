// Sparse attention over the QSA token set (a4 expand + tail, a5 query RoPE,
// a6 prefill, a7 split-K decode with a combine pass).
//
// Method (page "Qwen3.8-Flash-Next 没有缩小模型，它重写了每个参数何时上场",
// section "03 · Attention", CAUSAL SPARSE SET equation and fifth QSA step):
// query i attends exactly over S_i = its selected micro-blocks expanded to
// their 4 tokens plus the unfinished tail {4 n_c, ..., i}; 24 query heads share
// 2 KV heads (head h reads KV head h/12); width 256, rotary on dims 0..63.
//
// Design (gfx950): a wave walks a row's selected micro-blocks in tiles of 8
// (32 tokens); a micro-block of one KV head is a single 2 KB run in both
// caches.  Per tile it computes S^T = K Q^T with bf16 MFMA 16x16x32 (tokens
// as rows, the 12 heads of the KV group padded to 16 as columns).  The MFMA
// output gives each lane the 4 tokens of one micro-block for one head, which
// is exactly the k-slice the P V product needs from P, so P never leaves
// registers; the V cache is laid out [block][dim][4 tokens] so the matching V
// operand is one 8-byte run per (block, dim).  Online softmax in float32
// (base-2 exponent), output accumulators in float32.
//   prefill (attend_rows_kernel): one wave per query row and KV head, 4 rows
//     per workgroup; the next tile's keys come through the LDS DMA, the next
//     tile's values into registers, while the current tile computes.
//   decode (attend_split_kernel + combine_kernel): a row's tiles are split
//     over several workgroups that write (m, l, O) partials, merged after.
#include <math.h>

#include <mutex>

#include "qsa_common.hpp"

namespace qsa {

constexpr int kTileMB = 8;                    // micro-blocks per tile (two 16-token halves)
constexpr int kHalves = kTileMB / 4;
constexpr int kWaves = 4;
constexpr int kMaxList = kMaxBudget + 1;      // selected blocks + tail block
constexpr int kPartFloats = kGroup * kHeadDim + 2 * 16;  // O[12][256], m[16], l[16]
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Largest s with cu_q[s] <= row.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu_q, int n_seq, int row) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float bf16_elem(const u32x4& v, int e) {
  uint32_t w = v[e >> 1];
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8; a field at its maximum waits for nothing)
constexpr int kWaitVmem16 = 0x4F70;   // vector memory loads in flight <= 16
constexpr int kWaitVmem0 = 0x0F70;    // no vector memory load in flight
constexpr int kWaitLds0 = 0xC07F;     // no LDS access in flight

// split decode: one row's list and rotary angles, and the 4 waves' partial
// results merged at the end
struct SplitShared {
  int list[kMaxList + 8];            // micro-block ids, tail block last
  float cs[kRopeDim / 2][2];         // cos, sin of the query position
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][kGroup][kHeadDim];
};

// prefill: one wave's row (its list, rotary angles and next-tile key slots)
struct RowShared {
  int list[kMaxList + 8];
  float cs[kRopeDim / 2][2];
  u32x4 kst[kHalves][8][64];
};

// ---- the per-tile arithmetic shared by the prefill and the split decode
// kernels.  A tile is 8 micro-blocks (32 tokens) in two halves; in half hv,
// lane (col, grp) holds K rows of token `col` (micro-block 4 hv + col / 4)
// and the V / P k-slice of micro-block 4 hv + grp.

// Query fragment: the B operand of S^T = K Q^T.  The lane holds head `col`
// of this KV group (heads 12..15 are zero padding), dims 32 ks + 8 grp ..
// +7.  Rotate-half RoPE on dims 0..63 (pair j = 8 grp + e sits in qf[0] (x1)
// and qf[1] (x2)); the rotated dims are carried as two bf16 terms (value in
// qf, residual in ql), so the rotation adds no bf16 rounding to the logits;
// dims 64..255 are the bf16 inputs themselves.
__device__ __forceinline__ void rotate_query(u32x4 (&qf)[8], u32x4 (&ql)[2],
                                             const float (*cs)[2], int col, int grp) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    if (col >= kGroup) qf[ks] = u32x4{0, 0, 0, 0};
  ql[0] = u32x4{0u, 0u, 0u, 0u};
  ql[1] = u32x4{0u, 0u, 0u, 0u};
  u32x4 r0, r1, l0, l1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float y1[2], y2[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int e = 2 * w + h2, j = 8 * grp + e;
      const float c = cs[j][0], sn = cs[j][1];
      const float x1 = bf16_elem(qf[0], e), x2 = bf16_elem(qf[1], e);
      y1[h2] = x1 * c - x2 * sn;
      y2[h2] = x2 * c + x1 * sn;
    }
    r0[w] = pack_bf16x2(y1[0], y1[1]);
    r1[w] = pack_bf16x2(y2[0], y2[1]);
    l0[w] = pack_bf16x2(y1[0] - bf16_lo(r0[w]), y1[1] - bf16_hi(r0[w]));
    l1[w] = pack_bf16x2(y2[0] - bf16_lo(r1[w]), y2[1] - bf16_hi(r1[w]));
  }
  if (col < kGroup) { qf[0] = r0; qf[1] = r1; ql[0] = l0; ql[1] = l1; }
}

// S^T = K Q^T on MFMA 16x16x32: sc[hv][i] is token 4 grp + i of half hv for
// head col (the rotated dims twice: value and residual of the query).
__device__ __forceinline__ void tile_logits(const u32x4 (&kh)[kHalves][8], const u32x4 (&qf)[8],
                                            const u32x4 (&ql)[2], f32x4 (&sc)[kHalves]) {
#pragma unroll
  for (int hv = 0; hv < kHalves; ++hv) {
    sc[hv] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sc[hv] = mfma_16x16x32(kh[hv][ks], qf[ks], sc[hv]);
    sc[hv] = mfma_16x16x32(kh[hv][0], ql[0], sc[hv]);
    sc[hv] = mfma_16x16x32(kh[hv][1], ql[1], sc[hv]);
  }
}

// Online softmax of one tile and O += P V.  Logits in log2 units (scale);
// slots past the list (padding) and the tail block's tokens past the query
// are masked.  Lazy rescale: the reference max m_run only moves when a
// head's tile max exceeds it by more than 2^8, so p <= 256 and the float32
// sums stay exact-enough; the 64 output rescales run only on those tiles.
// P goes into the P V product as two bf16 terms (value and residual), so the
// product carries no bf16 rounding of the weights.
__device__ __forceinline__ void tile_softmax_pv(const f32x4 (&sc)[kHalves], u32x4 (&vh)[kHalves][8],
                                                f32x4 (&o)[16], float& m_run, float& l_run,
                                                int base, int cnt, int n_mb, int tail_slot,
                                                int tail_len, float scale, int grp) {
  float x[4 * kHalves];
#pragma unroll
  for (int hv = 0; hv < kHalves; ++hv)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * hv + i] = sc[hv][i] * scale;
  if (base + kTileMB > cnt) {
    // the tile holds the tail block and/or padding slots (uniform branch)
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
      const int sv = base + 4 * hv + grp;
      const int nv = sv >= n_mb ? 0 : (sv == tail_slot ? tail_len : 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * hv + i] = i < nv ? x[4 * hv + i] : -INFINITY;
      // cache rows past the query inside the tail block (and padding slots)
      // may hold anything: zero their V so that p = 0 cannot meet a NaN
      const uint32_t m01 = (nv > 0 ? 0xFFFFu : 0u) | (nv > 1 ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (nv > 2 ? 0xFFFFu : 0u) | (nv > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        vh[hv][c][0] &= m01; vh[hv][c][1] &= m23; vh[hv][c][2] &= m01; vh[hv][c][3] &= m23;
      }
    }
  }
  float mt = x[0];
#pragma unroll
  for (int i = 1; i < 4 * kHalves; ++i) mt = fmaxf(mt, x[i]);
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  if (__ballot(mt > m_run + 8.f)) {
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
    l_run *= alpha;
    m_run = m_new;
    float a_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_row[i] = __shfl(alpha, 4 * grp + i, 64);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= a_row[i];
    }
  }
  float p[4 * kHalves], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4 * kHalves; ++i) { p[i] = __builtin_amdgcn_exp2f(x[i] - m_run); ps += p[i]; }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  l_run += ps;
  // P k-slice of 8 tokens (2 micro-blocks) per lane: MFMA 16x16x32
  u32x4 pa, pl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pa[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    pl[e] = pack_bf16x2(p[2 * e] - bf16_lo(pa[e]), p[2 * e + 1] - bf16_hi(pa[e]));
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // dims 32c + 2*col (even tile) and 32c + 2*col + 1 (odd tile)
    u32x4 be = {vh[0][c][0], vh[0][c][1], vh[1][c][0], vh[1][c][1]};
    u32x4 bo = {vh[0][c][2], vh[0][c][3], vh[1][c][2], vh[1][c][3]};
    o[2 * c] = mfma_16x16x32(pa, be, o[2 * c]);
    o[2 * c + 1] = mfma_16x16x32(pa, bo, o[2 * c + 1]);
    o[2 * c] = mfma_16x16x32(pl, be, o[2 * c]);
    o[2 * c + 1] = mfma_16x16x32(pl, bo, o[2 * c + 1]);
  }
}

// The row's geometry: its sequence, position, candidate count and tail, and
// whether its selection is usable (a row with a bad selection gets NaN).
struct RowGeo {
  int s, pos, n_c, tail_len, cnt, n_mb, n_tiles;
  bool bad;
};
__device__ __forceinline__ RowGeo row_geo(const int32_t* __restrict__ cu_q,
                                          const int32_t* __restrict__ seq_len, int n_seq,
                                          const int32_t* __restrict__ sel_count, int budget,
                                          int row, bool one_per_seq) {
  RowGeo r;
  // one_per_seq: row s is the single query of sequence s (decode)
  r.s = one_per_seq ? row : find_seq(cu_q, n_seq, row);
  const int q_begin = one_per_seq ? row : cu_q[r.s];
  const int q_end = one_per_seq ? row + 1 : cu_q[r.s + 1];
  r.pos = seq_len[r.s] - (q_end - q_begin) + (row - q_begin);
  r.n_c = (r.pos + 1) >> 2;
  r.tail_len = (r.pos + 1) & 3;
  r.cnt = sel_count[row];
  r.bad = row >= q_end || r.pos < 0 || r.cnt < 0 || r.cnt > budget || r.cnt > r.n_c ||
          (r.cnt < min(budget, r.n_c));
  r.n_mb = r.cnt + (r.tail_len > 0 ? 1 : 0);
  r.n_tiles = (r.n_mb + kTileMB - 1) / kTileMB;
  return r;
}

// ---- prefill: one row per wave ---------------------------------------------
// Each wave attends one query row for one KV head on its own: its block list,
// rotary angles and key slots live in its own LDS region, it walks all of the
// row's tiles in order, and it normalises and writes the row's output itself
// (no workgroup barrier, no merge between waves).  A workgroup of 4 waves
// takes 4 consecutive rows of one KV head; the dispatcher deals workgroups to
// the 8 XCDs in turn, so each XCD holds one KV head and 256 rows of it in
// flight.  Rows of the same chunk select many of the same blocks, and the 4
// rows of a workgroup walk their ascending lists side by side, so a shared
// block is often still in L2 when the next row needs it.
// The keys of the next tile go straight from global memory into the wave's
// LDS slots (the LDS DMA puts lane i's 16 bytes in slot i) while the current
// tile computes, without the registers a second kh would take; the values of
// the next tile are loaded into registers once P V has consumed vh.
__global__ void __launch_bounds__(256, 2)
attend_rows_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
                   const int32_t* __restrict__ seq_len, int n_seq, int n_rows,
                   const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                   int64_t seq_stride, int64_t head_stride,
                   const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count,
                   int budget, uint16_t* __restrict__ out, float* __restrict__ lse, RopeFreq fr,
                   float sm_scale, Pages pg) {
  __shared__ RowShared shw[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x & 1;
  const int row = (int)(blockIdx.x >> 1) * kWaves + wave;
  if (row >= n_rows) return;   // waves are independent: no workgroup barrier below
  RowShared& sh = shw[wave];

  const RowGeo r = row_geo(cu_q, seq_len, n_seq, sel_count, budget, row, false);
  if (r.bad) {
    for (int i = lane; i < kGroup * kHeadDim; i += 64)
      out[((int64_t)row * kQHeads + g * kGroup) * kHeadDim + i] = 0x7FC0;  // NaN
    if (lse && lane < kGroup)
      lse[(int64_t)row * kQHeads + g * kGroup + lane] = __int_as_float(0x7FC00000);
    return;
  }
  const int cnt = r.cnt, n_mb = r.n_mb, n_tiles = r.n_tiles;
  const int tail_slot = r.tail_len > 0 ? cnt : -1;
  // paged caches: one pool per KV head, the list below holds physical blocks
  const int64_t seq_off = pg.table ? 0 : (int64_t)r.s * seq_stride;
  const uint16_t* kbase = kc + seq_off + (int64_t)g * head_stride;
  const uint16_t* vbase = vc + seq_off + (int64_t)g * head_stride;
  const float scale = kLog2e * sm_scale;   // logits in log2 units

  // query fragment first, so that its latency overlaps the list load
  u32x4 qf[8], ql[2];
  const int head = g * kGroup + min(col, kGroup - 1);
  const uint16_t* qrow = q + ((int64_t)row * kQHeads + head) * kHeadDim + 8 * grp;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = ldg16(qrow + 32 * ks);

  // block list (ascending ids from the selection, the tail block last) and
  // the query's rotary angles into this wave's LDS
  for (int i = lane; i < cnt; i += 64) {
    int id = sel[(int64_t)row * budget + i];
    id = min(max(id, 0), r.n_c - 1);
    sh.list[i] = pg.table ? (int)phys_block(pg, r.s, id) : id;
  }
  if (lane == 0 && r.tail_len > 0)
    sh.list[cnt] = pg.table ? (int)phys_block(pg, r.s, r.n_c) : r.n_c;
  if (lane < kRopeDim / 2) {
    double sd, cd;
    sincos((double)r.pos * freq_at(fr, lane), &sd, &cd);
    sh.cs[lane][0] = (float)cd;
    sh.cs[lane][1] = (float)sd;
  }
  __builtin_amdgcn_s_waitcnt(kWaitLds0);   // the wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  rotate_query(qf, ql, sh.cs, col, grp);

  u32x4 kh[kHalves][8], vh[kHalves][8];
  auto load_v = [&](int t) {
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
      const int idv = sh.list[min(t * kTileMB + 4 * hv + grp, n_mb - 1)];
      const uint16_t* vp = vbase + (int64_t)idv * (kBlock * kHeadDim) + 8 * col;
#pragma unroll
      for (int c = 0; c < 8; ++c) vh[hv][c] = ldg16(vp + 128 * c);
    }
  };
  auto dma_k = [&](int t) {
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
      const int idk = sh.list[min(t * kTileMB + 4 * hv + (col >> 2), n_mb - 1)];
      const uint16_t* kp = kbase + ((int64_t)idk * kBlock + (col & 3)) * kHeadDim + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        __builtin_amdgcn_global_load_lds(
            (const void*)(kp + 32 * ks),
            (__attribute__((address_space(3))) void*)&sh.kst[hv][ks][0], 16, 0, 0);
    }
  };

  f32x4 o[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (n_tiles > 0) {
    dma_k(0);
    asm volatile("" ::: "memory");   // keep the DMA ahead of the value loads
    load_v(0);
  }
  for (int t = 0; t < n_tiles; ++t) {
    // outstanding here: this tile's key DMA, then its 16 value loads
    __builtin_amdgcn_s_waitcnt(kWaitVmem16);   // the keys have landed
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kh[hv][ks] = sh.kst[hv][ks][lane];
    f32x4 sc[kHalves];
    tile_logits(kh, qf, ql, sc);
    // kh is consumed, so the slots can take the next tile's keys.  This
    // tile's values are waited for first, on every path: the compiler counts
    // an LDS DMA conservatively, and a wait for an older load behind it would
    // become a wait for the DMA too.
    __builtin_amdgcn_s_waitcnt(kWaitLds0);
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    if (t + 1 < n_tiles) dma_k(t + 1);
    asm volatile("" ::: "memory");
    tile_softmax_pv(sc, vh, o, m_run, l_run, t * kTileMB, cnt, n_mb, tail_slot, r.tail_len,
                    scale, grp);
    if (t + 1 < n_tiles) load_v(t + 1);
  }

  // output: the lane holds heads 4 grp + i, dims 32c + 2col and + 1; the
  // softmax denominator and max of head h sit in lane h
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hr = 4 * grp + i;
    const float inv = 1.f / __shfl(l_run, hr, 64);
    if (hr < kGroup) {
      uint16_t* op = out + ((int64_t)row * kQHeads + g * kGroup + hr) * kHeadDim + 2 * col;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *(uint32_t*)(op + 32 * c) = (uint32_t)f32_to_bf16_bits(o[2 * c][i] * inv) |
                                    ((uint32_t)f32_to_bf16_bits(o[2 * c + 1][i] * inv) << 16);
    }
  }
  if (lse && grp == 0 && col < kGroup)
    lse[(int64_t)row * kQHeads + g * kGroup + col] = (m_run + log2f(l_run)) * kLn2;
}

// ---- split decode -----------------------------------------------------------
// n_splits workgroups per (row, KV head) write (m, l, O) partials; 4 waves
// split each workgroup's contiguous range of tiles and merge in LDS.  The K
// and V loads are staggered by half a tile: the keys of tile t + 1 are
// requested as soon as the logits of tile t are formed, the values of tile
// t + 1 once P V of tile t has consumed vh, so each wave always has one of the
// two operands in flight while it computes (256 VGPRs: one wave per SIMD).
__global__ void __launch_bounds__(256, 1)
attend_split_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
                    const int32_t* __restrict__ seq_len, int n_seq, int n_rows,
                    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                    int64_t seq_stride, int64_t head_stride,
                    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count,
                    int budget, int n_splits, int one_per_seq, float* __restrict__ part,
                    RopeFreq fr, float sm_scale, Pages pg) {
  __shared__ SplitShared sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;

  // Each XCD takes a contiguous range of (row, KV head, split) items: the
  // dispatcher deals consecutive workgroup ids to the 8 XCDs in turn, so
  // without this the rows of one sequence (the query tokens of a multi-token
  // decode) would each run on another XCD and could not share the blocks
  // they have in common through one L2.
  const int wg = (gridDim.x & 7) ? (int)blockIdx.x
                                 : (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3));
  const int split = wg % n_splits;
  const int g = (wg / n_splits) & 1;
  const int row = wg / (2 * n_splits);
  if (row >= n_rows) return;

  const RowGeo r = row_geo(cu_q, seq_len, n_seq, sel_count, budget, row, one_per_seq != 0);
  float* pp = part + ((int64_t)(row * 2 + g) * n_splits + split) * kPartFloats;
  if (r.bad) {
    for (int i = threadIdx.x; i < kPartFloats; i += 256) pp[i] = __int_as_float(0x7FC00000);
    return;
  }
  const int cnt = r.cnt, n_mb = r.n_mb;
  const int tail_slot = r.tail_len > 0 ? cnt : -1;
  // part p of this (row, KV head) takes tiles [p*n/parts, (p+1)*n/parts)
  const int parts = n_splits * kWaves;
  const int my_part = split * kWaves + wave;
  const int t_begin = (int)((int64_t)my_part * r.n_tiles / parts);
  const int t_end = (int)((int64_t)(my_part + 1) * r.n_tiles / parts);
  const int64_t seq_off = pg.table ? 0 : (int64_t)r.s * seq_stride;
  const uint16_t* kbase = kc + seq_off + (int64_t)g * head_stride;
  const uint16_t* vbase = vc + seq_off + (int64_t)g * head_stride;
  const float scale = kLog2e * sm_scale;

  u32x4 qf[8], ql[2];
  const int head = g * kGroup + min(col, kGroup - 1);
  const uint16_t* qrow = q + ((int64_t)row * kQHeads + head) * kHeadDim + 8 * grp;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = ldg16(qrow + 32 * ks);

  for (int i = threadIdx.x; i < cnt; i += 256) {
    int id = sel[(int64_t)row * budget + i];
    id = min(max(id, 0), r.n_c - 1);   // ids come ascending from the selection
    sh.list[i] = pg.table ? (int)phys_block(pg, r.s, id) : id;
  }
  if (threadIdx.x == 0 && r.tail_len > 0)
    sh.list[cnt] = pg.table ? (int)phys_block(pg, r.s, r.n_c) : r.n_c;
  if (threadIdx.x < kRopeDim / 2) {
    double sd, cd;
    sincos((double)r.pos * freq_at(fr, threadIdx.x), &sd, &cd);
    sh.cs[threadIdx.x][0] = (float)cd;
    sh.cs[threadIdx.x][1] = (float)sd;
  }
  __syncthreads();

  u32x4 kh[kHalves][8], vh[kHalves][8];
  auto load_k = [&](int t) {
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
      const int idk = sh.list[min(t * kTileMB + 4 * hv + (col >> 2), n_mb - 1)];
      const uint16_t* kp = kbase + ((int64_t)idk * kBlock + (col & 3)) * kHeadDim + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kh[hv][ks] = ldg16(kp + 32 * ks);
    }
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
      const int idv = sh.list[min(t * kTileMB + 4 * hv + grp, n_mb - 1)];
      const uint16_t* vp = vbase + (int64_t)idv * (kBlock * kHeadDim) + 8 * col;
#pragma unroll
      for (int c = 0; c < 8; ++c) vh[hv][c] = ldg16(vp + 128 * c);
    }
  };
  if (t_begin < t_end) {
    load_k(t_begin);
    load_v(t_begin);
  }
  rotate_query(qf, ql, sh.cs, col, grp);

  f32x4 o[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  for (int t = t_begin; t < t_end; ++t) {
    f32x4 sc[kHalves];
    tile_logits(kh, qf, ql, sc);
    if (t + 1 < t_end) load_k(t + 1);
    tile_softmax_pv(sc, vh, o, m_run, l_run, t * kTileMB, cnt, n_mb, tail_slot, r.tail_len,
                    scale, grp);
    if (t + 1 < t_end) load_v(t + 1);
  }

  // ---- merge the 4 waves in LDS and write this split's partial
  if (grp == 0) { sh.m[wave][col] = m_run; sh.l[wave][col] = l_run; }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hr = 4 * grp + i;
    if (hr < kGroup) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        sh.o[wave][hr][32 * c + 2 * col] = o[2 * c][i];
        sh.o[wave][hr][32 * c + 2 * col + 1] = o[2 * c + 1][i];
      }
    }
  }
  __syncthreads();
  const int d = threadIdx.x;   // one output dim per thread
  for (int h = 0; h < kGroup; ++h) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sh.m[w][h]);
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = sh.l[w][h] > 0.f ? exp2f(sh.m[w][h] - mx) : 0.f;
      lsum += sh.l[w][h] * f;
      acc += sh.o[w][h][d] * f;
    }
    pp[h * kHeadDim + d] = acc;
    if (d == 0) { pp[kGroup * kHeadDim + h] = mx; pp[kGroup * kHeadDim + 16 + h] = lsum; }
  }
}

// Combine the NS partials of every (row, KV head, head): one workgroup per
// (row, query head), one output dim per thread.  All NS (max, sum, output)
// triples are loaded at once, then merged: one round trip to memory.
template <int NS>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ part, int n_rows, uint16_t* __restrict__ out,
               float* __restrict__ lse) {
  const int h = blockIdx.x % kGroup;
  const int g = (blockIdx.x / kGroup) & 1;
  const int row = blockIdx.x / (2 * kGroup);
  if (row >= n_rows) return;
  const int d = threadIdx.x;
  const float* base = part + (int64_t)(row * 2 + g) * NS * kPartFloats;
  float m[NS], l[NS], o[NS];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const float* pp = base + sp * kPartFloats;
    m[sp] = pp[kGroup * kHeadDim + h];
    l[sp] = pp[kGroup * kHeadDim + 16 + h];
    o[sp] = pp[h * kHeadDim + d];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) mx = fmaxf(mx, m[sp]);
  float lsum = 0.f, acc = 0.f;
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    const float f = l[sp] > 0.f ? exp2f(m[sp] - mx) : 0.f;
    lsum += l[sp] * f;
    acc += o[sp] * f;
  }
  out[((int64_t)row * kQHeads + g * kGroup + h) * kHeadDim + d] = (uint16_t)f32_to_bf16_bits(acc / lsum);
  if (lse && d == 0) lse[(int64_t)row * kQHeads + g * kGroup + h] = (mx + log2f(lsum)) * kLn2;
}

}  // namespace qsa

namespace {

// Splits per (query row, KV head) of a split-K decode launch: the largest
// power of two up to 16 that keeps the launch at most kDecodeSlots
// (row, KV head, split) workgroups.  Few rows (a ragged batch dominated by one
// long sequence) get many splits, many rows (multi-token decode) few: the
// per-workgroup setup (list, angles, merge, partials) is then paid as few
// times as the GPU's workgroup slots allow.
#ifndef QSA_DECODE_SLOTS
#define QSA_DECODE_SLOTS 256
#endif
constexpr int kDecodeSlots = QSA_DECODE_SLOTS;
constexpr int kMaxDecodeSplits = 16;

inline int decode_splits(int64_t n_rows) {
  int sp = kMaxDecodeSplits;
  while (sp > 1 && 2 * n_rows * sp > kDecodeSlots) sp >>= 1;
  return sp;
}

inline size_t decode_partials_bytes(int64_t n_rows) {
  return (size_t)n_rows * 2 * decode_splits(n_rows) * qsa::kPartFloats * sizeof(float);
}

// The split workgroups of a decode launch write (m, l, O) partials to part;
// the combine pass merges each (row, KV head)'s splits.
void launch_split_decode(const void* q, const int32_t* cu_q, const int32_t* seq_len, int n_seq,
                         int n_rows, int one_per_seq, const void* k_cache, const void* v_cache,
                         int64_t kv_seq_stride, int64_t kv_head_stride, const int32_t* sel,
                         const int32_t* sel_count, int budget, void* out, float* lse,
                         float* part, const qsa::RopeFreq& fr, float softmax_scale,
                         const qsa::Pages& pg, hipStream_t st) {
  const int sp = decode_splits(n_rows);
  hipLaunchKernelGGL(qsa::attend_split_kernel, dim3(n_rows * 2 * sp), dim3(256), 0, st,
                     (const uint16_t*)q, cu_q, seq_len, n_seq, n_rows, (const uint16_t*)k_cache,
                     (const uint16_t*)v_cache, kv_seq_stride, kv_head_stride, sel, sel_count,
                     budget, sp, one_per_seq, part, fr, softmax_scale, pg);
  const dim3 g(n_rows * 2 * qsa::kGroup);
  const float* cp = part;
  switch (sp) {
    case 1: hipLaunchKernelGGL(qsa::combine_kernel<1>, g, dim3(256), 0, st, cp, n_rows, (uint16_t*)out, lse); break;
    case 2: hipLaunchKernelGGL(qsa::combine_kernel<2>, g, dim3(256), 0, st, cp, n_rows, (uint16_t*)out, lse); break;
    case 4: hipLaunchKernelGGL(qsa::combine_kernel<4>, g, dim3(256), 0, st, cp, n_rows, (uint16_t*)out, lse); break;
    case 8: hipLaunchKernelGGL(qsa::combine_kernel<8>, g, dim3(256), 0, st, cp, n_rows, (uint16_t*)out, lse); break;
    default: hipLaunchKernelGGL(qsa::combine_kernel<16>, g, dim3(256), 0, st, cp, n_rows, (uint16_t*)out, lse); break;
  }
}

int check_attend_common(const void* q, const void* k_cache, const void* v_cache,
                        int64_t kv_seq_stride, int64_t kv_head_stride, const int32_t* sel,
                        const int32_t* sel_count, int32_t budget, const void* out) {
  using namespace qsa_host;
  if (!q || !k_cache || !v_cache || !sel || !sel_count || !out) return QSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return QSA_ERR_INVALID_ARG;
  if (!stride_ok(kv_seq_stride) || !stride_ok(kv_head_stride)) return QSA_ERR_INVALID_ARG;
  if (budget < 1 || budget > QSA_MAX_BUDGET) return QSA_ERR_INVALID_ARG;
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_attend_prefill(const void* q, const int32_t* cu_q, const int32_t* seq_len, int32_t n_seq,
                       int32_t n_q, int32_t max_q_len, const void* k_cache, const void* v_cache,
                       int64_t kv_seq_stride, int64_t kv_head_stride, const int32_t* sel,
                       const int32_t* sel_count, int32_t budget, void* out, float* lse,
                       const double* inv_freq, float softmax_scale, const int32_t* block_table,
                       int64_t table_stride, int32_t page_tokens, void* stream) {
  if (n_q < 0 || n_seq < 0 || max_q_len < 0) return QSA_ERR_INVALID_ARG;
  qsa::RopeFreq fr;
  if (!qsa_host::make_rope_freq(inv_freq, fr) || !qsa_host::softmax_scale_ok(softmax_scale))
    return QSA_ERR_INVALID_ARG;
  qsa::Pages pg;
  if (!qsa_host::make_pages(block_table, table_stride, page_tokens, pg)) return QSA_ERR_INVALID_ARG;
  if (n_q == 0) return QSA_OK;
  if (n_seq == 0 || !cu_q || !seq_len) return QSA_ERR_INVALID_ARG;
  int st = check_attend_common(q, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel, sel_count,
                               budget, out);
  if (st != QSA_OK) return st;
  // 4 rows (one per wave) of one KV head per workgroup
  const int64_t n_wg = (((int64_t)n_q + qsa::kWaves - 1) / qsa::kWaves) * 2;
  if (n_wg > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(qsa::attend_rows_kernel, dim3((unsigned)n_wg), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)q, cu_q, seq_len, n_seq, n_q,
                     (const uint16_t*)k_cache, (const uint16_t*)v_cache, kv_seq_stride,
                     kv_head_stride, sel, sel_count, budget, (uint16_t*)out, lse, fr,
                     softmax_scale, pg);
  return qsa_host::launch_status();
}

size_t qsa_attend_decode_multi_workspace(int32_t n_q) {
  if (n_q <= 0) return 0;
  return decode_partials_bytes(n_q);
}

int qsa_attend_decode_multi(const void* q, const int32_t* cu_q, const int32_t* seq_len,
                            int32_t n_seq, int32_t n_q, const void* k_cache, const void* v_cache,
                            int64_t kv_seq_stride, int64_t kv_head_stride, const int32_t* sel,
                            const int32_t* sel_count, int32_t budget, void* out, float* lse,
                            void* workspace, size_t ws_bytes, const double* inv_freq,
                            float softmax_scale, const int32_t* block_table,
                            int64_t table_stride, int32_t page_tokens, void* stream) {
  using namespace qsa_host;
  if (n_q < 0 || n_seq < 0) return QSA_ERR_INVALID_ARG;
  qsa::RopeFreq fr;
  if (!make_rope_freq(inv_freq, fr) || !softmax_scale_ok(softmax_scale)) return QSA_ERR_INVALID_ARG;
  qsa::Pages pg;
  if (!make_pages(block_table, table_stride, page_tokens, pg)) return QSA_ERR_INVALID_ARG;
  if (n_q == 0) return QSA_OK;
  if (n_seq == 0 || !cu_q || !seq_len) return QSA_ERR_INVALID_ARG;
  int st = check_attend_common(q, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel, sel_count,
                               budget, out);
  if (st != QSA_OK) return st;
  if (!workspace || !aligned16(workspace)) return QSA_ERR_INVALID_ARG;
  if (ws_bytes < qsa_attend_decode_multi_workspace(n_q)) return QSA_ERR_WORKSPACE_TOO_SMALL;
  if ((int64_t)n_q * 2 * qsa::kGroup > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  launch_split_decode(q, cu_q, seq_len, n_seq, n_q, 0, k_cache, v_cache, kv_seq_stride,
                      kv_head_stride, sel, sel_count, budget, out, lse, (float*)workspace, fr,
                      softmax_scale, pg, (hipStream_t)stream);
  return launch_status();
}

size_t qsa_attend_decode_workspace(int32_t n_seq) {
  if (n_seq <= 0) return 0;
  return decode_partials_bytes(n_seq);
}

}  // extern "C"

namespace {

// Host checks shared by qsa_attend_decode and qsa_attend_decode_noalloc
// (everything but the partials buffer).
int check_decode(const void* q, const int32_t* seq_len, int32_t n_seq, const void* k_cache,
                 const void* v_cache, int64_t kv_seq_stride, int64_t kv_head_stride,
                 const int32_t* sel, const int32_t* sel_count, int32_t budget, const void* out,
                 const double* inv_freq, float softmax_scale, const int32_t* block_table,
                 int64_t table_stride, int32_t page_tokens, qsa::RopeFreq& fr, qsa::Pages& pg) {
  using namespace qsa_host;
  if (n_seq < 0) return QSA_ERR_INVALID_ARG;
  if (!make_rope_freq(inv_freq, fr) || !softmax_scale_ok(softmax_scale)) return QSA_ERR_INVALID_ARG;
  if (!make_pages(block_table, table_stride, page_tokens, pg)) return QSA_ERR_INVALID_ARG;
  if (n_seq == 0) return QSA_OK;
  if (!seq_len) return QSA_ERR_INVALID_ARG;
  int st = check_attend_common(q, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel, sel_count,
                               budget, out);
  if (st != QSA_OK) return st;
  if ((int64_t)n_seq * 2 * qsa::kGroup > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  return QSA_OK;
}

// The split-K partials and the combine pass of a decode step; `part` holds
// decode_partials_bytes(n_seq).
int launch_decode(const void* q, const int32_t* seq_len, int32_t n_seq, const void* k_cache,
                  const void* v_cache, int64_t kv_seq_stride, int64_t kv_head_stride,
                  const int32_t* sel, const int32_t* sel_count, int32_t budget, void* out,
                  float* lse, float* part, const qsa::RopeFreq& fr, float softmax_scale,
                  const qsa::Pages& pg, void* stream) {
  launch_split_decode(q, nullptr, seq_len, n_seq, n_seq, 1, k_cache, v_cache, kv_seq_stride,
                      kv_head_stride, sel, sel_count, budget, out, lse, part, fr, softmax_scale,
                      pg, (hipStream_t)stream);
  return qsa_host::launch_status();
}

// ---------------------------------------------------- allocation-free decode
// The partials of qsa_attend_decode_noalloc live in this file-scope device
// array instead of a caller's workspace: every GPU the library runs on holds
// its own copy until the process ends.  A launch of up to
// QSA_NOALLOC_MAX_SEQ = 128 rows writes at most kDecodeSlots partials
// (3.2 MB).  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in symbol); it asks the runtime for the array's
// address on each device once, with that device current, and uses that.
static_assert(2 * QSA_NOALLOC_MAX_SEQ <= kDecodeSlots, "the array holds every split of 128 rows");
constexpr size_t kNoAllocFloats = (size_t)kDecodeSlots * qsa::kPartFloats;

}  // namespace

static __device__ __align__(256) float scratch[kNoAllocFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The address of the current device's copy of `scratch`, looked up on the
// first call on that device.  The stream must belong to the current device.
int scratch_on_current_device(void* stream, float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_INTERNAL;
  if (dev < 0 || dev >= kMaxDevices) return QSA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return QSA_ERR_INVALID_ARG;
    if ((int)sdev != dev) return QSA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QSA_ERR_INTERNAL;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_attend_decode(const void* q, const int32_t* seq_len, int32_t n_seq, const void* k_cache,
                      const void* v_cache, int64_t kv_seq_stride, int64_t kv_head_stride,
                      const int32_t* sel, const int32_t* sel_count, int32_t budget, void* out,
                      float* lse, void* workspace, size_t ws_bytes, const double* inv_freq,
                      float softmax_scale, const int32_t* block_table, int64_t table_stride,
                      int32_t page_tokens, void* stream) {
  qsa::RopeFreq fr;
  qsa::Pages pg;
  int st = check_decode(q, seq_len, n_seq, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel,
                        sel_count, budget, out, inv_freq, softmax_scale, block_table,
                        table_stride, page_tokens, fr, pg);
  if (st != QSA_OK || n_seq == 0) return st;
  if (!workspace || !qsa_host::aligned16(workspace)) return QSA_ERR_INVALID_ARG;
  if (ws_bytes < qsa_attend_decode_workspace(n_seq)) return QSA_ERR_WORKSPACE_TOO_SMALL;
  return launch_decode(q, seq_len, n_seq, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel,
                       sel_count, budget, out, lse, (float*)workspace, fr, softmax_scale, pg,
                       stream);
}

int qsa_attend_decode_noalloc(const void* q, const int32_t* seq_len, int32_t n_seq,
                              const void* k_cache, const void* v_cache, int64_t kv_seq_stride,
                              int64_t kv_head_stride, const int32_t* sel,
                              const int32_t* sel_count, int32_t budget, void* out, float* lse,
                              const double* inv_freq, float softmax_scale,
                              const int32_t* block_table, int64_t table_stride,
                              int32_t page_tokens, void* stream) {
  qsa::RopeFreq fr;
  qsa::Pages pg;
  int st = check_decode(q, seq_len, n_seq, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel,
                        sel_count, budget, out, inv_freq, softmax_scale, block_table,
                        table_stride, page_tokens, fr, pg);
  if (st != QSA_OK || n_seq == 0) return st;
  if (n_seq > QSA_NOALLOC_MAX_SEQ) return QSA_ERR_UNSUPPORTED;
  float* part = nullptr;
  st = scratch_on_current_device(stream, &part);
  if (st != QSA_OK) return st;
  return launch_decode(q, seq_len, n_seq, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel,
                       sel_count, budget, out, lse, part, fr, softmax_scale, pg, stream);
}

}  // extern "C"
