// Block-key pooling (a1), the cache-write partial RoPE helper (a5) and the
// ABI's status / version calls.
//
// Pooling follows the first QSA step of section "03 · Attention" on the page
// "Qwen3.8-Flash-Next 没有缩小模型，它重写了每个参数何时上场": the shared
// indexer key is averaged over non-overlapping 4-token micro-blocks.  The RoPE
// helper implements the 64-of-256-dim rotary embedding of the core heads
// (same page, config table and second QSA step).
#include "qsa_common.hpp"

namespace qsa {

// One thread pools 8 dims (16 bytes) of one block: 16 threads per block,
// 16 blocks per 256-thread workgroup and loop trip.  Reads of the 4 token
// rows are 256-byte coalesced segments; the store is one 256-byte segment.
__global__ void __launch_bounds__(256)
pool_block_keys_kernel(const uint16_t* __restrict__ idx_k, int64_t ik_stride,
                       uint16_t* __restrict__ bk, int64_t bk_stride,
                       const int32_t* __restrict__ blk_begin, const int32_t* __restrict__ blk_end,
                       Pages pg) {
  const int s = blockIdx.y;
  const int64_t b0 = blk_begin[s], b1 = blk_end[s];
  const int part = threadIdx.x & 15;   // which 8-dim slice
  const int sub = threadIdx.x >> 4;    // which block of the 16
  // paged: the pools' bases, and physical blocks (a page holds whole blocks)
  const uint16_t* src_seq = idx_k + (pg.table ? 0 : (int64_t)s * ik_stride);
  uint16_t* dst_seq = bk + (pg.table ? 0 : (int64_t)s * bk_stride);
  for (int64_t lb = b0 + (int64_t)blockIdx.x * 16 + sub; lb < b1; lb += (int64_t)gridDim.x * 16) {
    const int64_t b = pg.table ? phys_block(pg, s, lb) : lb;
    const uint16_t* src = src_seq + b * (kBlock * kIdxDim) + part * 8;
    u32x4 t0 = ldg16(src), t1 = ldg16(src + kIdxDim), t2 = ldg16(src + 2 * kIdxDim),
          t3 = ldg16(src + 3 * kIdxDim);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // float32 adds in token order, then the scale, then one bf16 rounding.
      float lo = bf16_lo(t0[e]) + bf16_lo(t1[e]);
      lo = lo + bf16_lo(t2[e]);
      lo = lo + bf16_lo(t3[e]);
      float hi = bf16_hi(t0[e]) + bf16_hi(t1[e]);
      hi = hi + bf16_hi(t2[e]);
      hi = hi + bf16_hi(t3[e]);
      o[e] = pack_bf16x2(lo * 0.25f, hi * 0.25f);
    }
    *(u32x4*)(dst_seq + b * kIdxDim + part * 8) = o;
  }
}

// One thread per rotation pair: 32 threads per (row, head), 8 (row, head)
// pairs per 256-thread workgroup.
__global__ void __launch_bounds__(256)
rope_apply_kernel(uint16_t* __restrict__ x, int64_t row_stride, int64_t head_stride,
                  int32_t n_heads, const int32_t* __restrict__ pos, int32_t pos0,
                  int64_t n_pairs, RopeFreq fr) {
  const int j = threadIdx.x & 31;
  const double fj = freq_at(fr, j);
  for (int64_t rh = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5); rh < n_pairs;
       rh += (int64_t)gridDim.x * 8) {
    const int64_t r = rh / n_heads;
    const int h = (int)(rh - r * n_heads);
    const int32_t p = pos ? pos[r] : pos0 + (int32_t)r;
    double theta = (double)p * fj;
    double sd, cd;
    sincos(theta, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    uint16_t* row = x + r * row_stride + (int64_t)h * head_stride;
    const float x1 = bf16_bits_to_f32(row[j]);
    const float x2 = bf16_bits_to_f32(row[j + kRopeDim / 2]);
    const float y1 = x1 * c - x2 * s;
    const float y2 = x2 * c + x1 * s;
    row[j] = (uint16_t)f32_to_bf16_bits(y1);
    row[j + kRopeDim / 2] = (uint16_t)f32_to_bf16_bits(y2);
  }
}

}  // namespace qsa


extern "C" {

const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_INVALID_ARG: return "QSA_ERR_INVALID_ARG";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED";
    case QSA_ERR_WORKSPACE_TOO_SMALL: return "QSA_ERR_WORKSPACE_TOO_SMALL";
    case QSA_ERR_LAUNCH_FAILED: return "QSA_ERR_LAUNCH_FAILED";
    case QSA_ERR_INTERNAL: return "QSA_ERR_INTERNAL";
    default: return "QSA_ERR_UNKNOWN";
  }
}

int qsa_abi_version(void) { return 4; }

int qsa_pool_block_keys(const void* idx_k, int64_t ik_seq_stride, void* block_keys,
                        int64_t bk_seq_stride, const int32_t* blk_begin, const int32_t* blk_end,
                        int32_t n_seq, int32_t max_span, const int32_t* block_table,
                        int64_t table_stride, int32_t page_tokens, void* stream) {
  using namespace qsa_host;
  if (n_seq < 0 || max_span < 0) return QSA_ERR_INVALID_ARG;
  qsa::Pages pg;
  if (!make_pages(block_table, table_stride, page_tokens, pg)) return QSA_ERR_INVALID_ARG;
  if (n_seq == 0 || max_span == 0) return QSA_OK;
  if (!idx_k || !block_keys || !blk_begin || !blk_end) return QSA_ERR_INVALID_ARG;
  if (!aligned16(idx_k) || !aligned16(block_keys)) return QSA_ERR_INVALID_ARG;
  if (!stride_ok(ik_seq_stride) || !stride_ok(bk_seq_stride)) return QSA_ERR_INVALID_ARG;
  if (n_seq > 65535) return QSA_ERR_UNSUPPORTED;
  const int per_wg = 16;
  int gx = (max_span + per_wg - 1) / per_wg;
  if (gx > 65536) gx = 65536;
  dim3 grid(gx, n_seq);
  hipLaunchKernelGGL(qsa::pool_block_keys_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)idx_k, ik_seq_stride, (uint16_t*)block_keys, bk_seq_stride,
                     blk_begin, blk_end, pg);
  return launch_status();
}

int qsa_rope_apply(void* x, int64_t row_stride, int64_t head_stride, int32_t n_heads,
                   const int32_t* pos, int32_t pos0, int32_t n_rows, const double* inv_freq,
                   void* stream) {
  using namespace qsa_host;
  if (n_rows < 0 || n_heads < 0) return QSA_ERR_INVALID_ARG;
  qsa::RopeFreq fr;
  if (!make_rope_freq(inv_freq, fr)) return QSA_ERR_INVALID_ARG;
  if (n_rows == 0 || n_heads == 0) return QSA_OK;
  if (!x || !aligned16(x)) return QSA_ERR_INVALID_ARG;
  if (!stride_ok(row_stride) || !stride_ok(head_stride)) return QSA_ERR_INVALID_ARG;
  if (pos0 < 0 || (int64_t)pos0 + n_rows > QSA_MAX_TOKENS) {
    if (!pos) return QSA_ERR_UNSUPPORTED;
  }
  const int64_t n_pairs = (int64_t)n_rows * n_heads;
  int64_t gx = (n_pairs + 7) / 8;
  if (gx > 1 << 20) gx = 1 << 20;
  hipLaunchKernelGGL(qsa::rope_apply_kernel, dim3((unsigned)gx), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)x, row_stride, head_stride, n_heads, pos, pos0, n_pairs, fr);
  return launch_status();
}

// YaRN (Peng et al., 2023) for the 32 rotary pairs: a pair of frequency
// theta turns r = orig_ctx / (2 pi / theta) times over the native window;
// gamma = clamp((r - alpha) / (beta - alpha), 0, 1); the new frequency is
// (1 - gamma) theta / factor + gamma theta.  The logit multiplier is
// (0.1 ln factor + 1)^2 (the paper's temperature, sqrt(1/t) = 0.1 ln s + 1).
int qsa_yarn_rope(double base, double factor, double orig_ctx, double alpha, double beta,
                  double* inv_freq, float* softmax_scale) {
  if (!inv_freq) return QSA_ERR_INVALID_ARG;
  if (!std::isfinite(base) || base <= 1.0 || !std::isfinite(factor) || factor < 1.0 ||
      !std::isfinite(orig_ctx) || orig_ctx <= 0.0 || !std::isfinite(alpha) ||
      !std::isfinite(beta) || !(alpha >= 0.0) || !(beta > alpha))
    return QSA_ERR_INVALID_ARG;
  const double two_pi = 2.0 * 3.14159265358979323846;
  for (int j = 0; j < qsa::kRopePairs; ++j) {
    const double theta = std::pow(base, -2.0 * (double)j / (double)qsa::kRopeDim);
    const double wavelength = two_pi / theta;
    const double r = orig_ctx / wavelength;
    double gamma = (r - alpha) / (beta - alpha);
    gamma = gamma < 0.0 ? 0.0 : (gamma > 1.0 ? 1.0 : gamma);
    inv_freq[j] = (1.0 - gamma) * theta / factor + gamma * theta;
  }
  if (softmax_scale) {
    const double t = 0.1 * std::log(factor) + 1.0;
    *softmax_scale = (float)(t * t / 16.0);
  }
  return QSA_OK;
}

}  // extern "C"
