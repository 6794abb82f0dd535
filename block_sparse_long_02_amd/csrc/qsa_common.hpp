// Shared device and host helpers for the QSA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "qsa.h"

namespace qsa {

// ----------------------------------------------------------------- types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = QSA_BLOCK;
constexpr int kIdxHeads = QSA_IDX_HEADS;
constexpr int kIdxDim = QSA_IDX_DIM;
constexpr int kQHeads = QSA_Q_HEADS;
constexpr int kKVHeads = QSA_KV_HEADS;
constexpr int kGroup = kQHeads / kKVHeads;  // 12 query heads per KV head
constexpr int kHeadDim = QSA_HEAD_DIM;
constexpr int kRopeDim = QSA_ROPE_DIM;
constexpr int kMaxBudget = QSA_MAX_BUDGET;

// -------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float32 -> bf16 bits (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------------- MFMA
// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies
// A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16]; it receives
// D[4*(l/16) + i][l%16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The 32 rotary frequencies f_j of the rotate-half pairs (j, j+32), passed to
// kernels by value (256 bytes of kernel arguments).
constexpr int kRopePairs = kRopeDim / 2;
struct RopeFreq {
  double f[kRopePairs];
};

// f_k for a lane-dependent k < 32, from the uniform table (a select chain,
// no indexed load of a kernel argument)
__device__ __forceinline__ double freq_at(const RopeFreq& fr, int k) {
  double f = 0.0;
#pragma unroll
  for (int t = 0; t < kRopePairs; ++t) f = (k == t) ? fr.f[t] : f;
  return f;
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

// Paged caches: a sequence's caches live in pages of 2^shift micro-blocks
// (4 * 2^shift tokens) inside shared pools; logical page p of sequence s is
// physical page table[s * stride + p].  table == nullptr: the contiguous
// per-sequence layout (the kernels then add their sequence strides).
struct Pages {
  const int32_t* table;
  int64_t stride;
  int shift;
};

// physical micro-block of logical micro-block b of sequence s (paged only)
__device__ __forceinline__ int64_t phys_block(const Pages& pg, int s, int64_t b) {
  const int64_t pi = b >> pg.shift;
  return ((int64_t)pg.table[(int64_t)s * pg.stride + pi] << pg.shift) +
         (b & (((int64_t)1 << pg.shift) - 1));
}

// --------------------------------------------------------- block helpers
// Exclusive prefix sum over a 256-thread workgroup.  `tmp` holds >= 4 ints of
// LDS.  Returns the exclusive prefix of `v`; `total` receives the sum.
__device__ __forceinline__ int block_excl_scan_256(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int t = tmp[w];
    if (w < wave) base += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

}  // namespace qsa

// ------------------------------------------------------------ host helpers
namespace qsa_host {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool stride_ok(int64_t s) { return s >= 0 && (s % 8) == 0; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH_FAILED;
}

// The caller's host table of 32 frequencies, or by default the core heads'
// 1e7^(-j/32) (float64).  False if an entry is not finite.
inline bool make_rope_freq(const double* inv_freq, qsa::RopeFreq& fr) {
  for (int j = 0; j < qsa::kRopePairs; ++j) {
    fr.f[j] = inv_freq ? inv_freq[j] : std::pow(1.0e7, -(double)j / (double)qsa::kRopePairs);
    if (!std::isfinite(fr.f[j])) return false;
  }
  return true;
}

inline bool softmax_scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// block_table == NULL: contiguous caches.  Otherwise page_tokens must be a
// power of two in [256, 2^22] (a page then holds whole 64-block GEMM stages)
// and table_stride >= 1.
inline bool make_pages(const int32_t* block_table, int64_t table_stride, int32_t page_tokens,
                       qsa::Pages& pg) {
  pg.table = block_table;
  pg.stride = table_stride;
  pg.shift = 0;
  if (!block_table) return true;
  if (table_stride < 1 || page_tokens < 256 || page_tokens > (1 << 22) ||
      (page_tokens & (page_tokens - 1)) != 0)
    return false;
  int sh = 0;
  while ((qsa::kBlock << sh) < page_tokens) ++sh;
  pg.shift = sh;
  return true;
}

}  // namespace qsa_host
