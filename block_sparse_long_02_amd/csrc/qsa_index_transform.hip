// The pages' indexer transforms, applied before the block scores.
//
// Page "Qwen3.8-Flash-Next 没有缩小模型，它重写了每个参数何时上场", the
// indexer figure caption and its note on the order of operations, and the
// second QSA step of section "03 · Attention":
//   key side   -- each 4-token micro-block is average-pooled, then
//                 RMS-normalised, then rotated (partial RoPE, 64 of the 128
//                 dims) at the block's position;
//   query side -- each projected indexer head is RMS-normalised, then rotated
//                 at the query token's position.
// Arithmetic (the same on both sides): the block mean is the float32
// ((k0 + k1) + k2) + k3 times 0.25 of the plain block key, without its bf16
// rounding; then, in float64, x * (mean(x^2) + eps)^(-1/2) * gamma[d], and the
// rotate-half rotation of the pairs (j, j+32), j < 32, by theta_j = pos * f_j;
// the result is rounded to float32, then to bf16 (both ties-to-even).  Keys
// take pos = p_b = 4b, the block's first token.  float64 makes the result
// independent of the order of the 128-term sum of squares except when the
// exact value lies within ~2^-50 (relative) of a rounding boundary.
//
// Layout of the work: 16 lanes hold one 128-dim vector, 8 dims (16 bytes)
// each; the sum of squares is a 16-lane butterfly; lane t (< 4) rotates dims
// 8t..8t+7 against lane t+4's dims 8t+32..8t+39 (one xor-4 exchange).
#include <math.h>

#include <cmath>

#include "qsa_common.hpp"

namespace qsa {

constexpr int kIdxRopeHalf = kRopePairs;   // pairs (j, j + 32) over dims 0..63

__device__ __forceinline__ double sum16(double v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v += __shfl_xor(v, m, 16);
  return v;
}

// x[0..7]: this lane's 8 dims (part = lane % 16 holds dims 8*part..8*part+7),
// already in float; g[0..7] and gp[0..7]: gamma at this lane's dims and at
// its xor-4 partner's; c[i], sn[i]: cos and sin of theta_j for the pair
// j = 8*(part % 4) + i (used by parts 0..7).  Returns the 8 bf16 results as
// 4 packed pairs.
__device__ __forceinline__ u32x4 norm_rope_8(const float (&x)[8], const float (&g)[8],
                                             const float (&gp)[8], int part, double eps,
                                             const double (&c)[8], const double (&sn)[8]) {
#pragma clang fp contract(off)
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += (double)x[i] * (double)x[i];
  ss = sum16(ss);
  const double r = 1.0 / sqrt(ss / (double)kIdxDim + eps);
  // the partner's raw values; every lane exchanges, only parts 0..7 use them
  float xp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xp[i] = __shfl_xor(x[i], 4, 16);
  double y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double n = ((double)x[i] * r) * (double)g[i];
    const double np = ((double)xp[i] * r) * (double)gp[i];
    // dims j (x1) and j + 32 (x2): y1 = x1 c - x2 s, y2 = x2 c + x1 s
    y[i] = part >= 8 ? n : part < 4 ? n * c[i] - np * sn[i] : n * c[i] + np * sn[i];
  }
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2((float)y[2 * e], (float)y[2 * e + 1]);
  return o;
}

__device__ __forceinline__ void load_gamma(const float* __restrict__ gamma, int part, float (&g)[8],
                                            float (&gp)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    g[i] = gamma ? gamma[part * 8 + i] : 1.f;
    gp[i] = gamma ? gamma[(part ^ 4) * 8 + i] : 1.f;
  }
}

// Key side: pooling as in the plain block key (16 lanes per block, 16 blocks
// per 256-thread workgroup and trip), then the transform.
__global__ void __launch_bounds__(256)
pool_block_keys_normed_kernel(const uint16_t* __restrict__ idx_k, int64_t ik_stride,
                              uint16_t* __restrict__ bk, int64_t bk_stride,
                              const int32_t* __restrict__ blk_begin,
                              const int32_t* __restrict__ blk_end,
                              const float* __restrict__ gamma, double eps, RopeFreq fr,
                              Pages pg) {
  const int s = blockIdx.y;
  const int64_t b0 = blk_begin[s], b1 = blk_end[s];
  const int part = threadIdx.x & 15;
  const int sub = threadIdx.x >> 4;
  float g[8], gp[8];
  load_gamma(gamma, part, g, gp);
  const double f0 = freq_at(fr, 2 * part), f1 = freq_at(fr, 2 * part + 1);
  const uint16_t* src_seq = idx_k + (pg.table ? 0 : (int64_t)s * ik_stride);
  uint16_t* dst_seq = bk + (pg.table ? 0 : (int64_t)s * bk_stride);
  // every lane of a 16-lane group takes the same trips (the butterfly needs
  // all 16): the loop bound depends on the group's block only
  for (int64_t lb = b0 + (int64_t)blockIdx.x * 16 + sub; lb < b1; lb += (int64_t)gridDim.x * 16) {
    // the rotation uses the logical position; paged caches store at the physical block
    const int64_t b = pg.table ? phys_block(pg, s, lb) : lb;
    const uint16_t* src = src_seq + b * (kBlock * kIdxDim) + part * 8;
    const u32x4 t0 = ldg16(src), t1 = ldg16(src + kIdxDim), t2 = ldg16(src + 2 * kIdxDim),
                t3 = ldg16(src + 3 * kIdxDim);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float lo = bf16_lo(t0[e]) + bf16_lo(t1[e]);
      lo = lo + bf16_lo(t2[e]);
      lo = lo + bf16_lo(t3[e]);
      float hi = bf16_hi(t0[e]) + bf16_hi(t1[e]);
      hi = hi + bf16_hi(t2[e]);
      hi = hi + bf16_hi(t3[e]);
      x[2 * e] = lo * 0.25f;
      x[2 * e + 1] = hi * 0.25f;
    }
    // the block's 32 angles, two per lane (j = 2*part, 2*part + 1), then
    // gathered: pair j = 8*(part % 4) + i sits in lane j/2, slot j%2
    const double pos = (double)(lb * kBlock);
    double c2[2], s2[2];
    sincos(pos * f0, &s2[0], &c2[0]);
    sincos(pos * f1, &s2[1], &c2[1]);
    double c[8], sn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int src = (part & 3) * 4 + (i >> 1);
      c[i] = __shfl(c2[i & 1], src, 16);
      sn[i] = __shfl(s2[i & 1], src, 16);
    }
    *(u32x4*)(dst_seq + b * kIdxDim + part * 8) = norm_rope_8(x, g, gp, part, eps, c, sn);
  }
}

// Query side: 16 lanes per (row, head), so one wave holds the 4 heads of one
// row (the stride over vectors is a multiple of 4) and lanes 0..31 compute
// the row's 32 angles once.  grid.y = sequence, grid.x strides over that
// sequence's rows x 4 heads.  q_out may alias q_raw: each lane reads its 16
// bytes before it writes them, and the exchanges are in registers.
__global__ void __launch_bounds__(256)
index_query_transform_kernel(const uint16_t* q_raw, uint16_t* q_out,
                             const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len,
                             int n_q, const float* __restrict__ gamma, double eps, RopeFreq fr) {
  const int s = blockIdx.y;
  const int qb = cu_q[s], qe_raw = cu_q[s + 1];
  const int qe = min(qe_raw, n_q);
  const int first_pos = seq_len[s] - (qe_raw - qb);   // position of row qb
  const int part = threadIdx.x & 15;
  float g[8], gp[8];
  load_gamma(gamma, part, g, gp);
  const int lane = threadIdx.x & 63;
  const double fl = freq_at(fr, lane & 31);
  const int64_t n_vec = (int64_t)max(qe - qb, 0) * kIdxHeads;
  for (int64_t v = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); v < n_vec;
       v += (int64_t)gridDim.x * 16) {
    const int row = qb + (int)(v / kIdxHeads);
    const int pos = first_pos + (row - qb);
    if (pos < 0) continue;   // uniform over the wave (one row)
    const int64_t off = ((int64_t)qb * kIdxHeads + v) * kIdxDim + part * 8;
    const u32x4 t = ldg16(q_raw + off);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(t[e]);
      x[2 * e + 1] = bf16_hi(t[e]);
    }
    double cl = 1.0, sl = 0.0;
    if (lane < kIdxRopeHalf) sincos((double)pos * fl, &sl, &cl);
    double c[8], sn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = (part & 3) * 8 + i;
      c[i] = __shfl(cl, j, 64);
      sn[i] = __shfl(sl, j, 64);
    }
    *(u32x4*)(q_out + off) = norm_rope_8(x, g, gp, part, eps, c, sn);
  }
}

}  // namespace qsa

namespace {

bool eps_ok(double eps) { return std::isfinite(eps) && eps >= 0.0; }

}  // namespace

extern "C" {

int qsa_pool_block_keys_normed(const void* idx_k, int64_t ik_seq_stride, void* block_keys,
                               int64_t bk_seq_stride, const int32_t* blk_begin,
                               const int32_t* blk_end, int32_t n_seq, int32_t max_span,
                               const float* gamma, double eps, const double* inv_freq,
                               const int32_t* block_table, int64_t table_stride,
                               int32_t page_tokens, void* stream) {
  using namespace qsa_host;
  if (n_seq < 0 || max_span < 0 || !eps_ok(eps)) return QSA_ERR_INVALID_ARG;
  qsa::Pages pg;
  if (!make_pages(block_table, table_stride, page_tokens, pg)) return QSA_ERR_INVALID_ARG;
  qsa::RopeFreq fr;
  if (!make_rope_freq(inv_freq, fr)) return QSA_ERR_INVALID_ARG;
  if (n_seq == 0 || max_span == 0) return QSA_OK;
  if (!idx_k || !block_keys || !blk_begin || !blk_end) return QSA_ERR_INVALID_ARG;
  if (!aligned16(idx_k) || !aligned16(block_keys)) return QSA_ERR_INVALID_ARG;
  if (!stride_ok(ik_seq_stride) || !stride_ok(bk_seq_stride)) return QSA_ERR_INVALID_ARG;
  if (n_seq > 65535) return QSA_ERR_UNSUPPORTED;
  int gx = (max_span + 15) / 16;
  if (gx > 65536) gx = 65536;
  hipLaunchKernelGGL(qsa::pool_block_keys_normed_kernel, dim3(gx, n_seq), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)idx_k, ik_seq_stride,
                     (uint16_t*)block_keys, bk_seq_stride, blk_begin, blk_end, gamma, eps, fr, pg);
  return launch_status();
}

int qsa_index_query_transform(const void* q_raw, void* q_out, const int32_t* cu_q,
                              const int32_t* seq_len, int32_t n_seq, int32_t n_q,
                              int32_t max_q_len, const float* gamma, double eps,
                              const double* inv_freq, void* stream) {
  using namespace qsa_host;
  if (n_seq < 0 || n_q < 0 || max_q_len < 0 || !eps_ok(eps)) return QSA_ERR_INVALID_ARG;
  qsa::RopeFreq fr;
  if (!make_rope_freq(inv_freq, fr)) return QSA_ERR_INVALID_ARG;
  if (n_seq == 0 || n_q == 0 || max_q_len == 0) return QSA_OK;
  if (!q_raw || !q_out || !cu_q || !seq_len) return QSA_ERR_INVALID_ARG;
  if (!aligned16(q_raw) || !aligned16(q_out)) return QSA_ERR_INVALID_ARG;
  if (n_seq > 65535) return QSA_ERR_UNSUPPORTED;
  int64_t gx = ((int64_t)max_q_len * qsa::kIdxHeads + 15) / 16;
  if (gx > 65536) gx = 65536;
  hipLaunchKernelGGL(qsa::index_query_transform_kernel, dim3((unsigned)gx, n_seq), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)q_raw, (uint16_t*)q_out, cu_q, seq_len,
                     n_q, gamma, eps, fr);
  return launch_status();
}

}  // extern "C"
