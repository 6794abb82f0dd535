// Micro-benchmarks of the sustained MFMA rate and HBM bandwidth (see
// include/qsa_probe.h).  Measurement only: no QSA arithmetic here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"
#include "qsa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NC independent accumulator chains per wave hide the MFMA latency.  Thread
// 0 of workgroup 0 also records its loop's shader-clock cycles (s_memtime)
// and 100 MHz reference ticks (s_memrealtime) in sink[0..3], so the clock
// the MFMAs ran at can be read back.
template <int NC>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
    b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
  }
  f32x4 acc[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    uint32_t* u = reinterpret_cast<uint32_t*>(sink);
    const uint64_t dc = c1 - c0, dr = r1 - r0;
    u[0] = (uint32_t)dc;
    u[1] = (uint32_t)(dc >> 32);
    u[2] = (uint32_t)dr;
    u[3] = (uint32_t)(dr >> 32);
  }
  if (s == -1.f) sink[4 + threadIdx.x % 252] = s;   // never true: the sums are >= 0
}

__global__ void __launch_bounds__(256) read_probe_kernel(const u32x4* __restrict__ src, int64_t n,
                                                         u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; i < n; i += stride) acc ^= src[i];
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) sink[0] = acc;   // practically never
}

__global__ void __launch_bounds__(256) copy_probe_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Reads n_runs runs of (1 << run_shift) 16-byte chunks; run r starts at
// chunk idx[r] << run_shift.  Consecutive threads read consecutive chunks of
// a run, four loads in flight per thread.
__global__ void __launch_bounds__(256) gather_probe_kernel(const u32x4* __restrict__ src,
                                                           const int32_t* __restrict__ idx,
                                                           int64_t n_runs, int run_shift,
                                                           u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t total = n_runs << run_shift, mask = ((int64_t)1 << run_shift) - 1;
  const int64_t stride = (int64_t)gridDim.x * 256;
  auto at = [&](int64_t c) { return ((int64_t)idx[c >> run_shift] << run_shift) + (c & mask); };
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < total; i += 4 * stride) {
    const int64_t a0 = at(i), a1 = at(i + stride), a2 = at(i + 2 * stride), a3 = at(i + 3 * stride);
    acc ^= src[a0] ^ src[a1] ^ src[a2] ^ src[a3];
  }
  for (; i < total; i += stride) acc ^= src[at(i)];
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) sink[0] = acc;   // practically never
}

int status() { return hipGetLastError() == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH_FAILED; }

bool bytes_ok(const void* p, int64_t bytes) {
  return p && ((uintptr_t)p & 15) == 0 && bytes > 0 && bytes % 64 == 0;
}

}  // namespace

extern "C" {

int qsa_probe_mfma_bf16(int32_t n_wg, int32_t iters, int32_t chains, float* sink, void* stream) {
  if (n_wg < 1 || iters < 1 || !sink || (chains != 8 && chains != 16)) return QSA_ERR_INVALID_ARG;
  if (chains == 8)
    hipLaunchKernelGGL(mfma_probe_kernel<8>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<16>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return status();
}

int qsa_probe_read(const void* src, int64_t bytes, int32_t n_wg, void* sink, void* stream) {
  if (!bytes_ok(src, bytes) || n_wg < 1 || !sink) return QSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(read_probe_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, (u32x4*)sink);
  return status();
}

int qsa_probe_gather(const void* src, int64_t bytes, const int32_t* idx, int64_t n_runs,
                     int32_t run_bytes, int32_t n_wg, void* sink, void* stream) {
  if (!bytes_ok(src, bytes) || !idx || n_runs < 1 || n_wg < 1 || !sink) return QSA_ERR_INVALID_ARG;
  if (run_bytes < 16 || run_bytes > (1 << 20) || (run_bytes & (run_bytes - 1))) return QSA_ERR_INVALID_ARG;
  if (bytes / run_bytes > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  int shift = 0;
  while ((16 << shift) < run_bytes) ++shift;
  hipLaunchKernelGGL(gather_probe_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, idx, n_runs, shift, (u32x4*)sink);
  return status();
}

int qsa_probe_copy(const void* src, void* dst, int64_t bytes, int32_t n_wg, void* stream) {
  if (!bytes_ok(src, bytes) || !bytes_ok(dst, bytes) || n_wg < 1) return QSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return status();
}

}  // extern "C"
