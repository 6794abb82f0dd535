// Sparse attention over the QSA token set (a4 expand + tail, a5 query RoPE,
// a6 prefill, a7 split-K decode with a combine pass).
//
// Method (page "Qwen3.8-Flash-Next 没有缩小模型，它重写了每个参数何时上场",
// section "03 · Attention", CAUSAL SPARSE SET equation and fifth QSA step):
// query i attends exactly over S_i = its selected micro-blocks expanded to
// their 4 tokens plus the unfinished tail {4 n_c, ..., i}; 24 query heads share
// 2 KV heads (head h reads KV head h/12); width 256, rotary on dims 0..63.
//
// Design (gfx950): one wave streams tiles of 8 micro-blocks (32 tokens)
// straight from HBM into registers -- no LDS staging, since a micro-block of
// one KV head is a single 2 KB run in both caches.  Per tile it computes
// S^T = K Q^T with bf16 MFMA 16x16x32 (tokens as rows, the 12 heads of the
// KV group padded to 16 as columns).  The MFMA output gives each lane the 4
// tokens of one micro-block for one head, which is exactly the k-slice the
// P V product needs from P, so P never leaves registers; the V cache is laid
// out [block][dim][4 tokens] so the matching V operand is one 8-byte run per
// (block, dim).  Online softmax in float32 (base-2 exponent), output
// accumulators in float32.
#include <math.h>

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

struct AttnShared {
  int list[kMaxList + 8];            // micro-block ids, tail block last
  float cs[kRopeDim / 2][2];         // cos, sin of the query position
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][kGroup][kHeadDim];
};

// mode kFinal: one workgroup per (row, KV head) writes out / lse.
// otherwise: n_splits workgroups per (row, KV head) write partials.
template <bool kFinal>
__global__ void __launch_bounds__(256, 2)
attend_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q,
              const int32_t* __restrict__ seq_len, int n_seq, int n_rows,
              const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
              int64_t seq_stride, int64_t head_stride,
              const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int budget,
              int n_splits, int one_per_seq, uint16_t* __restrict__ out,
              float* __restrict__ lse, float* __restrict__ part, RopeFreq fr, float sm_scale,
              Pages pg) {
  __shared__ AttnShared sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;

  const int wg = blockIdx.x;
  const int split = wg % n_splits;
  const int g = (wg / n_splits) & 1;
  const int row = wg / (2 * n_splits);
  if (row >= n_rows) return;

  // ---- which sequence / position, and is the selection usable?
  // one_per_seq: row s is the single query of sequence s (decode)
  const int s = one_per_seq ? row : find_seq(cu_q, n_seq, row);
  const int q_begin = one_per_seq ? row : cu_q[s], q_end = one_per_seq ? row + 1 : cu_q[s + 1];
  const int L = seq_len[s];
  const int pos = L - (q_end - q_begin) + (row - q_begin);
  const int n_c = (pos + 1) >> 2;
  const int tail_len = (pos + 1) & 3;
  const int cnt = sel_count[row];
  const bool bad = row >= q_end || pos < 0 || cnt < 0 || cnt > budget || cnt > n_c ||
                   (cnt < min(budget, n_c));
  if (bad) {
    if (kFinal) {
      for (int i = threadIdx.x; i < kGroup * kHeadDim; i += 256)
        out[((int64_t)row * kQHeads + g * kGroup) * kHeadDim + i] = 0x7FC0;  // NaN
      if (lse && threadIdx.x < kGroup) lse[(int64_t)row * kQHeads + g * kGroup + threadIdx.x] = __int_as_float(0x7FC00000);
    } else {
      float* pp = part + ((int64_t)(row * 2 + g) * n_splits + split) * kPartFloats;
      for (int i = threadIdx.x; i < kPartFloats; i += 256) pp[i] = __int_as_float(0x7FC00000);
    }
    return;
  }
  const int n_mb = cnt + (tail_len > 0 ? 1 : 0);

  // ---- this wave's tiles
  const int n_tiles = (n_mb + kTileMB - 1) / kTileMB;
  const int parts = n_splits * kWaves;
  const int my_part = split * kWaves + wave;
  // even split: part p takes tiles [p*n/parts, (p+1)*n/parts)
  const int t_begin = (int)((int64_t)my_part * n_tiles / parts);
  const int t_end = (int)((int64_t)(my_part + 1) * n_tiles / parts);
  const int tail_slot = tail_len > 0 ? cnt : -1;

  // paged caches: one pool per KV head, the list below holds physical blocks
  const int64_t seq_off = pg.table ? 0 : (int64_t)s * seq_stride;
  const uint16_t* kbase = kc + seq_off + (int64_t)g * head_stride;
  const uint16_t* vbase = vc + seq_off + (int64_t)g * head_stride;
  const float scale = kLog2e * sm_scale;   // logits in log2 units

  f32x4 o[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Half hv of tile t covers micro-blocks t*kTileMB + 4hv .. +3.  K rows:
  // lane is token row `col` of the half; V / P k-slices: micro-block
  // t*kTileMB + 4hv + grp.
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
  // ---- block list and the query's rotary angles into LDS
  for (int i = threadIdx.x; i < cnt; i += 256) {
    int id = sel[(int64_t)row * budget + i];
    id = min(max(id, 0), n_c - 1);   // ids come ascending from the selection
    sh.list[i] = pg.table ? (int)phys_block(pg, s, id) : id;
  }
  if (threadIdx.x == 0 && tail_len > 0) sh.list[cnt] = pg.table ? (int)phys_block(pg, s, n_c) : n_c;
  if (threadIdx.x < kRopeDim / 2) {
    double sd, cd;
    sincos((double)pos * freq_at(fr, threadIdx.x), &sd, &cd);
    sh.cs[threadIdx.x][0] = (float)cd;
    sh.cs[threadIdx.x][1] = (float)sd;
  }
  __syncthreads();

  // ---- query fragment: B operand of S^T = K Q^T.  Lane holds head `col` of
  // this KV group, dims 32*ks + 8*grp .. +7.  Heads 12..15 are zero padding.
  u32x4 qf[8];
  // heads 12..15 of the tile are padding: their address is clamped to a real
  // head and the value replaced by zero
  const int head = g * kGroup + min(col, kGroup - 1);
  const uint16_t* qrow = q + ((int64_t)row * kQHeads + head) * kHeadDim + 8 * grp;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const u32x4 v = ldg16(qrow + 32 * ks);
    qf[ks] = col < kGroup ? v : u32x4{0, 0, 0, 0};
  }
  // The rotated dims 0..63 are carried as two bf16 terms (value and
  // residual), so the rotation adds no bf16 rounding to the logits; dims
  // 64..255 are the bf16 inputs themselves.
  u32x4 ql[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  {
    // rotate-half on dims 0..63: pair j = 8*grp + e sits in qf[0] (x1) and qf[1] (x2)
    u32x4 r0, r1, l0, l1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float y1[2], y2[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int e = 2 * w + h2, j = 8 * grp + e;
        const float c = sh.cs[j][0], sn = sh.cs[j][1];
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

  for (int t = t_begin; t < t_end; ++t) {
    const int base = t * kTileMB;
    load_k(t);
    load_v(t);

    // sc[hv][i]: token i of micro-block slot base + 4hv + grp, head col
    f32x4 sc[kHalves];
#pragma unroll
    for (int hv = 0; hv < kHalves; ++hv) {
      sc[hv] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sc[hv] = mfma_16x16x32(kh[hv][ks], qf[ks], sc[hv]);
      sc[hv] = mfma_16x16x32(kh[hv][0], ql[0], sc[hv]);
      sc[hv] = mfma_16x16x32(kh[hv][1], ql[1], sc[hv]);
    }
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
        // Cache rows past the query inside the tail block (and padding
        // slots) may hold anything: zero their V so that p = 0 cannot meet a
        // NaN.
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
    // Lazy rescale: the reference max m_run only moves when a head's tile max
    // exceeds it by more than 2^8, so p <= 256 and the float32 sums stay
    // exact-enough; the 64 output rescales run only on those tiles.
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

    {
      // P k-slice of 8 tokens (2 micro-blocks) per lane: MFMA 16x16x32.  P
      // goes in as two bf16 terms (value and residual), so the product with
      // V carries no bf16 rounding of the weights.
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
  }

  // ---- merge the 4 waves in LDS
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
  float* pp = kFinal ? nullptr : part + ((int64_t)(row * 2 + g) * n_splits + split) * kPartFloats;
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
    if (kFinal) {
      out[((int64_t)row * kQHeads + g * kGroup + h) * kHeadDim + d] =
          (uint16_t)f32_to_bf16_bits(acc / lsum);
      if (lse && d == 0) lse[(int64_t)row * kQHeads + g * kGroup + h] = (mx + log2f(lsum)) * kLn2;
    } else {
      pp[h * kHeadDim + d] = acc;
      if (d == 0) { pp[kGroup * kHeadDim + h] = mx; pp[kGroup * kHeadDim + 16 + h] = lsum; }
    }
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

// splits per (row, KV head) in decode
#ifndef QSA_DECODE_SPLITS
#define QSA_DECODE_SPLITS 8
#endif
constexpr int kDecodeSplits = QSA_DECODE_SPLITS;

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
  if ((int64_t)n_q * 2 > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(qsa::attend_kernel<true>, dim3(n_q * 2), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)q, cu_q, seq_len, n_seq, n_q, (const uint16_t*)k_cache,
                     (const uint16_t*)v_cache, kv_seq_stride, kv_head_stride, sel, sel_count,
                     budget, 1, 0, (uint16_t*)out, lse, (float*)nullptr, fr, softmax_scale, pg);
  return qsa_host::launch_status();
}

size_t qsa_attend_decode_multi_workspace(int32_t n_q) {
  if (n_q <= 0) return 0;
  return (size_t)n_q * 2 * kDecodeSplits * qsa::kPartFloats * sizeof(float);
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
  if ((int64_t)n_q * 2 * kDecodeSplits > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  float* part = (float*)workspace;
  hipLaunchKernelGGL(qsa::attend_kernel<false>, dim3(n_q * 2 * kDecodeSplits), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)q, cu_q, seq_len, n_seq, n_q,
                     (const uint16_t*)k_cache, (const uint16_t*)v_cache, kv_seq_stride,
                     kv_head_stride, sel, sel_count, budget, kDecodeSplits, 0,
                     (uint16_t*)nullptr, (float*)nullptr, part, fr, softmax_scale, pg);
  hipLaunchKernelGGL(qsa::combine_kernel<kDecodeSplits>, dim3(n_q * 2 * qsa::kGroup), dim3(256), 0,
                     (hipStream_t)stream, (const float*)part, n_q, (uint16_t*)out, lse);
  return launch_status();
}

size_t qsa_attend_decode_workspace(int32_t n_seq) {
  if (n_seq <= 0) return 0;
  return (size_t)n_seq * 2 * kDecodeSplits * qsa::kPartFloats * sizeof(float);
}

int qsa_attend_decode(const void* q, const int32_t* seq_len, int32_t n_seq, const void* k_cache,
                      const void* v_cache, int64_t kv_seq_stride, int64_t kv_head_stride,
                      const int32_t* sel, const int32_t* sel_count, int32_t budget, void* out,
                      float* lse, void* workspace, size_t ws_bytes, const double* inv_freq,
                      float softmax_scale, const int32_t* block_table, int64_t table_stride,
                      int32_t page_tokens, void* stream) {
  using namespace qsa_host;
  if (n_seq < 0) return QSA_ERR_INVALID_ARG;
  qsa::RopeFreq fr;
  if (!make_rope_freq(inv_freq, fr) || !softmax_scale_ok(softmax_scale)) return QSA_ERR_INVALID_ARG;
  qsa::Pages pg;
  if (!make_pages(block_table, table_stride, page_tokens, pg)) return QSA_ERR_INVALID_ARG;
  if (n_seq == 0) return QSA_OK;
  if (!seq_len) return QSA_ERR_INVALID_ARG;
  int st = check_attend_common(q, k_cache, v_cache, kv_seq_stride, kv_head_stride, sel, sel_count,
                               budget, out);
  if (st != QSA_OK) return st;
  if (!workspace || !aligned16(workspace)) return QSA_ERR_INVALID_ARG;
  if (ws_bytes < qsa_attend_decode_workspace(n_seq)) return QSA_ERR_WORKSPACE_TOO_SMALL;
  if ((int64_t)n_seq * 2 * qsa::kGroup > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  float* part = (float*)workspace;
  hipLaunchKernelGGL(qsa::attend_kernel<false>, dim3(n_seq * 2 * kDecodeSplits), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)q, (const int32_t*)nullptr, seq_len,
                     n_seq, n_seq, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                     kv_seq_stride, kv_head_stride, sel, sel_count, budget, kDecodeSplits, 1,
                     (uint16_t*)nullptr, (float*)nullptr, part, fr, softmax_scale, pg);
  hipLaunchKernelGGL(qsa::combine_kernel<kDecodeSplits>, dim3(n_seq * 2 * qsa::kGroup), dim3(256), 0,
                     (hipStream_t)stream, (const float*)part, n_seq, (uint16_t*)out, lse);
  return launch_status();
}

}  // extern "C"
