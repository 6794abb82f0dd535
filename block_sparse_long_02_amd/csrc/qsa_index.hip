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
//   1. sample pass   -- the score GEMM over every 16th block writes those
//                       scores (1/16 of the work) for rows with > 4096 candidates;
//   2. threshold     -- per row, tau = the r-th largest sampled score, with r
//                       chosen so that about K + 1536 candidates score >= tau;
//   3. filter pass   -- the full score GEMM (bf16 MFMA 16x16x32, indexer query
//                       rows in registers, block keys streamed) appends every
//                       (score, block) with score >= tau to a per-row list
//                       (wave-aggregated atomics);
//   4. final select  -- per row, an exact LDS radix select over that list under
//                       the total order, then the ids sorted ascending.
// Exactness does not depend on the sample: if the list holds >= K entries it
// contains the true top K (all of them score >= the K-th score >= tau).  A row
// whose list is short or overflows goes to
//   5. fallback      -- an exact radix select that recomputes its scores on
//                       every pass (slow, needs no score storage).
#include <math.h>

#include "qsa_common.hpp"

namespace qsa {

constexpr int kCandCap = 4096;      // list capacity per row
constexpr int kSampleStride = 16;   // every 16th block is sampled
constexpr int kSampleExtra = 1536;  // aimed-for surplus of list entries over K
constexpr int kBins = 2048;         // 11-bit radix digits
constexpr int kFallbackWGs = 64;
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

// The float32 epilogue shared by every pass: heads in acc[0..3].
__device__ __forceinline__ float block_score(f32x4 acc, const float* __restrict__ w) {
#pragma clang fp contract(off)
  const float u0 = fmaxf(acc[0], 0.f) * kScoreScale;
  const float u1 = fmaxf(acc[1], 0.f) * kScoreScale;
  const float u2 = fmaxf(acc[2], 0.f) * kScoreScale;
  const float u3 = fmaxf(acc[3], 0.f) * kScoreScale;
  float s = w[0] * u0;
  s = s + w[1] * u1;
  s = s + w[2] * u2;
  s = s + w[3] * u3;
  return s == 0.f ? 0.f : s;   // canonical +0
}

// ----------------------------------------------------------- score GEMM
// Workgroup = one tile of 4*MT query rows of one sequence x a chunk of
// `chunk_cols` virtual columns.  Virtual column v is block v*stride (stride 16
// in the sample pass, 1 in the filter pass).  A row r = 4*(query) + head of the
// tile is MFMA row r%16 of m-tile r/16; each wave takes 16-column tiles
// round-robin, U tiles per trip so that U*4 KB of block keys are in flight.
template <int MT, int U, bool kSample>
__global__ void __launch_bounds__(256)
score_kernel(const uint16_t* __restrict__ idx_q, const float* __restrict__ w,
             const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len, int n_seq,
             int n_q, int tiles_per_seq, int max_blocks, const uint16_t* __restrict__ bk,
             int64_t bk_stride, int chunk_cols, const uint32_t* __restrict__ thresh,
             int32_t* __restrict__ cnt, u32x2* __restrict__ cand,
             uint32_t* __restrict__ samples, int ns_stride) {
  constexpr int QT = 4 * MT;
  constexpr int stride = kSample ? kSampleStride : 1;
  __shared__ float s_w[QT][4];
  __shared__ int s_nc[QT];
  __shared__ uint32_t s_th[QT];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int s = blockIdx.x / tiles_per_seq, t = blockIdx.x % tiles_per_seq;
  const int qb = cu_q[s], qe_raw = cu_q[s + 1];
  const int qe = min(qe_raw, n_q);                    // rows past n_q are never touched
  const int row0 = qb + t * QT;
  if (row0 >= qe || row0 < 0) return;
  const int pos0 = seq_len[s] - (qe_raw - qb) + t * QT;   // position of row0
  const int n_rows = min(QT, qe - row0);
  // candidates of the tile's last row bound every row's
  const int nc_last = (pos0 + n_rows) >> 2;
  if (nc_last > max_blocks) return;                   // reported by the final select
  const int max_cols = kSample ? (nc_last + stride - 1) / stride : nc_last;
  const int v0 = blockIdx.y * chunk_cols;
  if (v0 >= max_cols) return;
  if (kSample && nc_last <= kCandCap) return;          // no row of the tile samples
  const int v1 = min(v0 + chunk_cols, max_cols);

  if (threadIdx.x < QT) {
    const int j = threadIdx.x;
    const bool ok = j < n_rows;
    const int rj = min(row0 + j, qe - 1);             // in-bounds address for padding rows
    const int nc = ok ? (pos0 + j + 1) >> 2 : 0;
    s_nc[j] = (kSample && nc <= kCandCap) ? 0 : nc;    // sample only rows that need it
    const uint32_t th = kSample ? 0u : thresh[rj];
    s_th[j] = ok && !kSample ? th : 0xFFFFFFFFu;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float wv = w[(int64_t)rj * 4 + h];
      s_w[j][h] = ok ? wv : 0.f;
    }
  }

  // A fragments: m-tile mt, k-step ks -> row mt*16 + col (query mt*4 + col/4,
  // head col%4), dims 32*ks + 8*grp .. +7.
  u32x4 af[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int j = mt * 4 + (col >> 2);
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

  const uint16_t* bseq = bk + (int64_t)s * bk_stride;
  for (int c0 = v0 + wave * 16 * U; c0 < v1; c0 += 64 * U) {
    u32x4 bf[U][4];
    int vcol[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vcol[u] = c0 + u * 16 + col;
      const int b = min(vcol[u], v1 - 1) * stride;     // in-bounds row for masked columns
      const uint16_t* src = bseq + (int64_t)b * kIdxDim + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bf[u][ks] = ldg16(src + 32 * ks);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = vcol[u] * stride;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma_16x16x32(af[mt][ks], bf[u][ks], acc);
        // lane holds the 4 heads of query j = mt*4 + grp for block b
        const int j = mt * 4 + grp;
        const bool live = vcol[u] < v1 && b < s_nc[j];
        const float sc = block_score(acc, s_w[j]);
        const uint32_t key = __float_as_uint(sc);
        if (kSample) {
          if (live) samples[(int64_t)(row0 + j) * ns_stride + vcol[u]] = key;
        } else {
          const bool hit = live && key >= s_th[j];
          const unsigned long long mask = __ballot(hit);
          if (mask) {
            const uint32_t gm = (uint32_t)(mask >> (16 * grp)) & 0xFFFFu;
            const int n = __popc(gm);
            const int rank = __popc(gm & ((1u << col) - 1u));
            int base = 0;
            if (hit && rank == 0) base = atomicAdd(&cnt[row0 + j], n);
            const int leader = 16 * grp + (gm ? __ffs(gm) - 1 : 0);
            base = __shfl(base, leader, 64);
            if (hit) {
              const int slot = base + rank;
              if (slot < kCandCap) cand[(int64_t)(row0 + j) * kCandCap + slot] = u32x2{key, (uint32_t)b};
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------ LDS radix select
// k-th largest value (1-based) among the participating elements, where
// get(i) -> {participates, value} for i < n and values have `nbits` bits.
// 11-bit digits from the top.  Needs kBins ints of LDS in `hist`.
template <class Get>
__device__ uint32_t block_kth_largest(Get get, int n, int k, int nbits, int* hist, int* tmp,
                                      int* res) {
  uint32_t prefix = 0, pmask = 0;
  for (int top = nbits; top > 0;) {
    const int width = top >= 11 ? 11 : top;
    const int shift = top - width;
    const int bins = 1 << width;
    for (int i = threadIdx.x; i < bins; i += 256) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) {
      bool in;
      uint32_t v = get(i, in);
      if (in && (v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & (bins - 1)], 1);
    }
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

// Ascending bitonic sort of 512 ints in LDS by 256 threads.
__device__ void bitonic_sort_512(int* a) {
  for (int k2 = 2; k2 <= 512; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      const int t = threadIdx.x;
      const int i = 2 * t - (t & (j - 1));
      const int p = i + j;
      const bool up = (i & k2) == 0;
      const int x = a[i], y = a[p];
      if ((x > y) == up) { a[i] = y; a[p] = x; }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------ threshold
__global__ void __launch_bounds__(256)
threshold_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len, int n_seq,
                 int max_blocks, int budget, const uint32_t* __restrict__ samples, int ns_stride,
                 uint32_t* __restrict__ thresh, int32_t* __restrict__ cnt,
                 int32_t* __restrict__ fb_count) {
  __shared__ int hist[kBins];
  __shared__ int tmp[8];
  __shared__ int res[2];
  const int row = blockIdx.x;
  if (row == 0 && threadIdx.x == 0) *fb_count = 0;
  const RowGeom g = row_geom(cu_q, seq_len, n_seq, row, max_blocks);
  if (threadIdx.x == 0) cnt[row] = 0;
  if (!g.ok) { if (threadIdx.x == 0) thresh[row] = 0xFFFFFFFFu; return; }
  if (g.n_c <= kCandCap) { if (threadIdx.x == 0) thresh[row] = 0u; return; }
  const int k = min(budget, g.n_c);
  const int ns = (g.n_c + kSampleStride - 1) / kSampleStride;
  const int r = min(ns, (k + kSampleExtra + kSampleStride - 1) / kSampleStride);
  const uint32_t* sp = samples + (int64_t)row * ns_stride;
  const uint32_t tau = block_kth_largest(
      [&](int i, bool& in) { in = true; return sp[i]; }, ns, r, 31, hist, tmp, res);
  if (threadIdx.x == 0) thresh[row] = tau;
}

// --------------------------------------------------------- final select
struct SelectShared {
  uint32_t key[kCandCap];
  int idx[kCandCap];
  int hist[kBins];
  int ids[kMaxBudget];
  int tmp[8];
  int res[2];
  int n_out;
};

__global__ void __launch_bounds__(256)
final_select_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len,
                    int n_seq, int max_blocks, int budget, const int32_t* __restrict__ cnt,
                    const u32x2* __restrict__ cand, int32_t* __restrict__ sel,
                    int32_t* __restrict__ sel_count, int32_t* __restrict__ fb_count,
                    int32_t* __restrict__ fb_list) {
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
    if (threadIdx.x == 0) fb_list[atomicAdd(fb_count, 1)] = row;
    return;
  }
  for (int i = threadIdx.x; i < c; i += 256) {
    const u32x2 e = cand[(int64_t)row * kCandCap + i];
    sh.key[i] = e[0];
    sh.idx[i] = (int)e[1];
  }
  if (threadIdx.x == 0) sh.n_out = 0;
  __syncthreads();

  uint32_t tau = 0, iota_cut = 0xFFFFFFFFu;
  bool all = c == k;
  if (!all) {
    tau = block_kth_largest([&](int i, bool& in) { in = true; return sh.key[i]; }, c, k, 31,
                            sh.hist, sh.tmp, sh.res);
    // how many strictly above tau, how many equal
    int above = 0, ties = 0;
    for (int i = threadIdx.x; i < c; i += 256) {
      above += sh.key[i] > tau;
      ties += sh.key[i] == tau;
    }
    int tot_above, tot_ties;
    block_excl_scan_256(above, sh.tmp, tot_above);
    block_excl_scan_256(ties, sh.tmp, tot_ties);
    const int need = k - tot_above;
    if (need < tot_ties) {
      // the `need` lowest block ids among the ties: k-th largest of (2^22-1-id)
      const uint32_t v = block_kth_largest(
          [&](int i, bool& in) { in = sh.key[i] == tau; return 0x3FFFFFu - (uint32_t)sh.idx[i]; },
          c, need, 22, sh.hist, sh.tmp, sh.res);
      iota_cut = 0x3FFFFFu - v;
    }
  }
  for (int i = threadIdx.x; i < c; i += 256) {
    const uint32_t kk = sh.key[i];
    const bool take = all || kk > tau || (kk == tau && (uint32_t)sh.idx[i] <= iota_cut);
    if (take) {
      const int slot = atomicAdd(&sh.n_out, 1);
      if (slot < kMaxBudget) sh.ids[slot] = sh.idx[i];
    }
  }
  __syncthreads();
  for (int i = k + threadIdx.x; i < kMaxBudget; i += 256) sh.ids[i] = 0x7FFFFFFF;
  __syncthreads();
  bitonic_sort_512(sh.ids);
  for (int i = threadIdx.x; i < budget; i += 256) out[i] = i < k ? sh.ids[i] : -1;
  if (threadIdx.x == 0) sel_count[row] = k;
}

// ------------------------------------------------------------- fallback
// Exact select for rows whose list was short or overflowed: recompute the
// score of every candidate on every radix pass (VALU dot products; one block
// per thread), then emit in ascending block order.
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

__global__ void __launch_bounds__(256)
fallback_kernel(const uint16_t* __restrict__ idx_q, const float* __restrict__ w,
                const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_len, int n_seq,
                int max_blocks, int budget, const uint16_t* __restrict__ bk, int64_t bk_stride,
                const int32_t* __restrict__ fb_count, const int32_t* __restrict__ fb_list,
                int32_t* __restrict__ sel, int32_t* __restrict__ sel_count) {
  __shared__ int hist[kBins];
  __shared__ int tmp[8];
  __shared__ int res[2];
  const int n_fb = *fb_count;
  for (int e = blockIdx.x; e < n_fb; e += gridDim.x) {
    const int row = fb_list[e];
    const RowGeom g = row_geom(cu_q, seq_len, n_seq, row, max_blocks);
    const int k = min(budget, g.n_c);
    const uint16_t* q4 = idx_q + (int64_t)row * 4 * kIdxDim;
    const float* w4 = w + (int64_t)row * 4;
    const uint16_t* bseq = bk + (int64_t)g.seq * bk_stride;
    auto key_of = [&](int b, bool& in) {
      in = true;
      return recompute_key(q4, w4, bseq + (int64_t)b * kIdxDim);
    };
    const uint32_t tau = block_kth_largest(key_of, g.n_c, k, 31, hist, tmp, res);
    int above = 0;
    for (int b = threadIdx.x; b < g.n_c; b += 256) { bool in; above += key_of(b, in) > tau; }
    int tot_above;
    block_excl_scan_256(above, tmp, tot_above);
    const int need = k - tot_above;   // ties to take, lowest block ids first
    int32_t* out = sel + (int64_t)row * budget;
    int ties_run = 0, out_run = 0;
    for (int b0 = 0; b0 < g.n_c; b0 += 256) {
      const int b = b0 + threadIdx.x;
      bool in;
      const uint32_t key = b < g.n_c ? key_of(b, in) : 0u;
      const bool is_tie = b < g.n_c && key == tau;
      const bool is_above = b < g.n_c && key > tau;
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
    if (threadIdx.x == 0) sel_count[row] = k;
    __syncthreads();
  }
}

// ------------------------------------------------------------ workspace
struct IndexWs {
  uint32_t* thresh;
  int32_t* cnt;
  u32x2* cand;
  uint32_t* samples;
  int32_t* fb_count;
  int32_t* fb_list;
  int ns_stride;
  size_t bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline IndexWs index_ws_layout(void* base, int n_q, int max_blocks) {
  IndexWs ws;
  char* p = (char*)base;
  size_t off = 0;
  ws.ns_stride = (max_blocks + kSampleStride - 1) / kSampleStride;
  ws.thresh = (uint32_t*)(p + off); off = align256(off + (size_t)n_q * 4);
  ws.cnt = (int32_t*)(p + off); off = align256(off + (size_t)n_q * 4);
  ws.fb_count = (int32_t*)(p + off); off = align256(off + 4);
  ws.fb_list = (int32_t*)(p + off); off = align256(off + (size_t)n_q * 4);
  ws.cand = (u32x2*)(p + off); off = align256(off + (size_t)n_q * kCandCap * 8);
  ws.samples = (uint32_t*)(p + off);
  off = align256(off + (max_blocks > kCandCap ? (size_t)n_q * ws.ns_stride * 4 : 0));
  ws.bytes = off;
  return ws;
}

}  // namespace qsa

extern "C" {

size_t qsa_index_select_workspace(int32_t n_q, int32_t max_blocks) {
  if (n_q <= 0 || max_blocks < 0) return 0;
  return qsa::index_ws_layout(nullptr, n_q, max_blocks).bytes;
}

int qsa_index_select(const void* idx_q, const float* w, const int32_t* cu_q,
                     const int32_t* seq_len, int32_t n_seq, int32_t n_q, int32_t max_q_len,
                     int32_t max_blocks, const void* block_keys, int64_t bk_seq_stride,
                     int32_t budget, int32_t* sel, int32_t* sel_count, void* workspace,
                     size_t ws_bytes, void* stream) {
  using namespace qsa_host;
  using namespace qsa;
  if (n_q < 0 || n_seq < 0 || max_q_len < 0 || max_blocks < 0) return QSA_ERR_INVALID_ARG;
  if (budget < 1 || budget > QSA_MAX_BUDGET) return QSA_ERR_INVALID_ARG;
  if (n_q == 0) return QSA_OK;
  if (n_seq == 0 || max_q_len == 0) return QSA_ERR_INVALID_ARG;
  if (!idx_q || !w || !cu_q || !seq_len || !block_keys || !sel || !sel_count || !workspace)
    return QSA_ERR_INVALID_ARG;
  if (!aligned16(idx_q) || !aligned16(w) || !aligned16(block_keys) || !aligned16(workspace))
    return QSA_ERR_INVALID_ARG;
  if (!stride_ok(bk_seq_stride)) return QSA_ERR_INVALID_ARG;
  if (max_blocks > QSA_MAX_TOKENS / QSA_BLOCK) return QSA_ERR_UNSUPPORTED;
  const IndexWs ws = index_ws_layout(workspace, n_q, max_blocks);
  if (ws_bytes < ws.bytes) return QSA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;

  const bool small_tiles = max_q_len <= 4;
  const int qt = small_tiles ? 4 : 32;
  const int64_t tiles_per_seq = (max_q_len + qt - 1) / qt;
  const int64_t gx = tiles_per_seq * n_seq;
  if (gx > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  const int chunk = small_tiles ? 512 : 2048;

  // 1. sample pass (only rows with more than kCandCap candidates need it)
  if (max_blocks > kCandCap) {
    const int cols = ws.ns_stride;
    dim3 grid((unsigned)gx, (cols + chunk - 1) / chunk);
    if (small_tiles)
      hipLaunchKernelGGL((score_kernel<1, 4, true>), grid, dim3(256), 0, st, (const uint16_t*)idx_q,
                         w, cu_q, seq_len, n_seq, n_q, (int)tiles_per_seq, max_blocks,
                         (const uint16_t*)block_keys, bk_seq_stride, chunk, ws.thresh, ws.cnt,
                         ws.cand, ws.samples, ws.ns_stride);
    else
      hipLaunchKernelGGL((score_kernel<8, 1, true>), grid, dim3(256), 0, st, (const uint16_t*)idx_q,
                         w, cu_q, seq_len, n_seq, n_q, (int)tiles_per_seq, max_blocks,
                         (const uint16_t*)block_keys, bk_seq_stride, chunk, ws.thresh, ws.cnt,
                         ws.cand, ws.samples, ws.ns_stride);
  }
  // 2. thresholds (also zero the list counters and the fallback counter)
  hipLaunchKernelGGL(threshold_kernel, dim3(n_q), dim3(256), 0, st, cu_q, seq_len, n_seq,
                     max_blocks, budget, ws.samples, ws.ns_stride, ws.thresh, ws.cnt, ws.fb_count);
  // 3. filter pass
  if (max_blocks > 0) {
    dim3 grid((unsigned)gx, (max_blocks + chunk - 1) / chunk);
    if (grid.y > 65535) return QSA_ERR_UNSUPPORTED;
    if (small_tiles)
      hipLaunchKernelGGL((score_kernel<1, 4, false>), grid, dim3(256), 0, st,
                         (const uint16_t*)idx_q, w, cu_q, seq_len, n_seq, n_q, (int)tiles_per_seq,
                         max_blocks, (const uint16_t*)block_keys, bk_seq_stride, chunk, ws.thresh,
                         ws.cnt, ws.cand, ws.samples, ws.ns_stride);
    else
      hipLaunchKernelGGL((score_kernel<8, 1, false>), grid, dim3(256), 0, st,
                         (const uint16_t*)idx_q, w, cu_q, seq_len, n_seq, n_q, (int)tiles_per_seq,
                         max_blocks, (const uint16_t*)block_keys, bk_seq_stride, chunk, ws.thresh,
                         ws.cnt, ws.cand, ws.samples, ws.ns_stride);
  }
  // 4. exact select per row
  hipLaunchKernelGGL(final_select_kernel, dim3(n_q), dim3(256), 0, st, cu_q, seq_len, n_seq,
                     max_blocks, budget, ws.cnt, ws.cand, sel, sel_count, ws.fb_count, ws.fb_list);
  // 5. fallback for rows whose list was short or overflowed
  hipLaunchKernelGGL(fallback_kernel, dim3(kFallbackWGs), dim3(256), 0, st, (const uint16_t*)idx_q,
                     w, cu_q, seq_len, n_seq, max_blocks, budget, (const uint16_t*)block_keys,
                     bk_seq_stride, ws.fb_count, ws.fb_list, sel, sel_count);
  return launch_status();
}

}  // extern "C"
