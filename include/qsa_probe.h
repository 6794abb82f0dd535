/*
 * qsa_probe.h -- micro-benchmarks that measure what an MI355X actually
 * sustains, to read the QSA kernels' roofline fractions against: a dense
 * bf16 MFMA loop (v_mfma_f32_16x16x32_bf16, the instruction the score GEMM
 * and the attention use), a streaming HBM read, a streaming copy and a
 * gather of fixed-size runs at random places.  Not
 * part of the QSA path; libqsa_probe.so is loaded only by the measurement
 * tool.  Same conventions as qsa.h (device pointers, void* stream, status
 * codes of qsa.h, validation before any HIP call).
 */
#ifndef QSA_PROBE_H_
#define QSA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_wg workgroups of 4 waves; each wave issues iters x `chains` (8 or 16)
 * independent 16x16x32 bf16 MFMAs (16,384 flop each).  sink: device
 * float[256]; words 0..3 receive workgroup 0's shader-clock cycles and
 * 100 MHz reference ticks over its loop (two uint64, low word first), the
 * rest is written only under a condition the data never meets.
 * Errors: 1 (INVALID_ARG) for n_wg < 1, iters < 1, other chain counts or a
 * NULL sink. */
int qsa_probe_mfma_bf16(int32_t n_wg, int32_t iters, int32_t chains, float* sink, void* stream);

/* Reads `bytes` (a multiple of 64, 16-byte aligned) from src with 16-byte
 * loads, grid-striding over n_wg workgroups of 256 threads; sink as above
 * (device, 16 bytes). */
int qsa_probe_read(const void* src, int64_t bytes, int32_t n_wg, void* sink, void* stream);

/* Gathers n_runs runs of run_bytes (a power of two, 16 .. 2^20) from src
 * (`bytes` long, as above): run r is src[idx[r] * run_bytes ..
 * (idx[r] + 1) * run_bytes).  idx: device int32[n_runs], each in
 * [0, bytes / run_bytes) -- the caller guarantees this; it is not checked on
 * the device.  The attention kernels' gathers are runs of 2 KB (one
 * micro-block of one KV head); this measures what such a pattern sustains.
 * Errors: 1 for bad pointers, sizes or run_bytes; 2 (UNSUPPORTED) when
 * bytes / run_bytes exceeds 2^31 - 1. */
int qsa_probe_gather(const void* src, int64_t bytes, const int32_t* idx, int64_t n_runs,
                     int32_t run_bytes, int32_t n_wg, void* sink, void* stream);

/* Copies `bytes` (as above) from src to dst (non-overlapping). */
int qsa_probe_copy(const void* src, void* dst, int64_t bytes, int32_t n_wg, void* stream);

#ifdef __cplusplus
}
#endif

#endif  // QSA_PROBE_H_
