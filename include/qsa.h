/*
 * qsa.h -- C ABI of libqsa: the Qwen Sparse Attention (QSA) hot path on one
 * AMD MI355X (gfx950).
 *
 * Pages cited (titles as published):
 *   [card]    "Qwen3.8-Flash-Next - 面向 Qwen4 架构的实验性预览权重发布"
 *             (aiboss88.com), model-card structure paragraph.
 *   [ailearn] "Qwen3.8-Flash-Next 没有缩小模型，它重写了每个参数何时上场"
 *             (ailearn.mscapital.top): config table, section "03 · Attention"
 *             (indexer figure caption, BLOCK SCORE and CAUSAL SPARSE SET
 *             equations, the five-step QSA list, the performance box).
 *
 * The QSA layer: an indexer with 4 query heads over one shared key (width
 * 128) mean-pools the keys of each sequence into 4-token micro-blocks, scores
 * every completed block for every query, keeps at most 512 blocks (2048
 * tokens) plus the query's unfinished tail block, and the core GQA attention
 * (24 query heads, 2 KV heads, width 256, rotary on 64 dims) reads exactly
 * those tokens ([card]; [ailearn] config table and §03).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers unless stated.  "bf16" buffers
 *    hold IEEE bfloat16 bit patterns (uint16).  The caller owns every buffer;
 *    the library allocates no device memory and keeps no pointer after a call
 *    returns.  Scratch space is passed in as `workspace`, sized by the matching
 *    *_workspace() query; the one exception, qsa_attend_decode_noalloc, uses a
 *    fixed-size array inside the library instead.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Every
 *    call only enqueues work on it and returns; results are ready once the
 *    stream is synchronised.  Device-side faults surface at that sync.
 *  - Arguments are validated on the host before any HIP call; a non-zero
 *    status means nothing was enqueued.  No C++ exception crosses the ABI.
 *  - Base pointers must be 16-byte aligned, strides (in elements) multiples
 *    of 8.  Tensor contents must be finite.
 *  - Batch layout ("varlen"): sequence s has seq_len[s] tokens in its caches;
 *    its queries are rows cu_q[s] .. cu_q[s+1]-1 of the query tensors and sit
 *    at the LAST positions of the sequence: row cu_q[s]+j has position
 *    seq_len[s] - (cu_q[s+1] - cu_q[s]) + j.  A prefill chunk is one sequence
 *    with many rows; a decode step is one row per sequence.  cu_q and seq_len
 *    are device int32 arrays; max_q_len (host) must be >= every
 *    cu_q[s+1]-cu_q[s] and max_blocks (host) >= every seq_len[s]/4.
 *  - Cache layouts (per sequence s and KV head g, strides in elements):
 *      idx_k       bf16 [n_seq][cap][128]           token-major indexer keys
 *      block_keys  bf16 [n_seq][cap/4][128]         pooled micro-block keys
 *      k_cache     bf16 [n_seq][2][cap][256]        rotated keys, token-major:
 *                  element (s,g,t,d) at s*kv_seq_stride + g*kv_head_stride + t*256 + d
 *      v_cache     bf16 [n_seq][2][cap/4][256][4]   values, micro-block-major and
 *                  dim-major inside a block: element (s,g,t,d) at
 *                  s*kv_seq_stride + g*kv_head_stride + (t/4)*1024 + d*4 + (t%4)
 *    `cap` is a multiple of 4 and covers every token of the sequence, so the
 *    unfinished tail block is always in bounds; cache rows at positions
 *    >= seq_len[s] inside that block may hold anything and are never used.
 *  - Paged caches (f3: prefix-cache reuse, [ailearn] performance box): every
 *    call that reads or writes a cache takes (block_table, table_stride,
 *    page_tokens).  block_table == NULL selects the contiguous layouts above.
 *    Otherwise the caches are pools of pages of page_tokens tokens (a power of
 *    two, 256 <= page_tokens <= 2^22); logical page p = t / page_tokens of
 *    sequence s is physical page P = block_table[s*table_stride + p] (device
 *    int32; table_stride >= 1), and the sequence strides are ignored:
 *      idx_k       bf16 [n_pages*page_tokens][128]      token row P*page_tokens + t%page_tokens
 *      block_keys  bf16 [n_pages*page_tokens/4][128]    block row P*page_tokens/4 + b%(page_tokens/4)
 *      k_cache     bf16 [2][n_pages*page_tokens][256]   kv_head_stride apart per KV head
 *      v_cache     bf16 [2][n_pages*page_tokens/4][256][4]   (same head stride, same block order)
 *    A sequence's table row must name a valid page for every page that holds
 *    one of its positions < seq_len[s]; sequences may share pages (a common
 *    prefix).  A page holds whole micro-blocks, so a chunk may start at any
 *    position: the block it completes is pooled from its page.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARG = 1,          /* null / misaligned pointer or stride, bad count or budget */
  QSA_ERR_UNSUPPORTED = 2,          /* shape outside the fixed QSA layer (e.g. > 2^22 tokens)  */
  QSA_ERR_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below the matching *_workspace() query         */
  QSA_ERR_LAUNCH_FAILED = 4,        /* a kernel launch reported an error                        */
  QSA_ERR_INTERNAL = 5
};

/* Fixed shapes of the QSA layer ([card]; [ailearn] config table and
 * CAUSAL SPARSE SET equation). */
#define QSA_BLOCK 4            /* micro-block ratio r                     */
#define QSA_IDX_HEADS 4        /* indexer query heads                     */
#define QSA_IDX_DIM 128        /* indexer head width                      */
#define QSA_Q_HEADS 24         /* core query heads                        */
#define QSA_KV_HEADS 2         /* core KV heads                           */
#define QSA_HEAD_DIM 256       /* core head width                         */
#define QSA_ROPE_DIM 64        /* rotated dims of a core head             */
#define QSA_MAX_BUDGET 512     /* K_B = ceil(2048 / 4)                    */
#define QSA_MAX_TOKENS (1 << 22)
#define QSA_NOALLOC_MAX_SEQ 128   /* sequences per qsa_attend_decode_noalloc call */

/* Human-readable name of a status code (static string, never NULL). */
const char* qsa_status_string(int status);

/* ABI version: bumped whenever a signature or a layout above changes. */
int qsa_abi_version(void);

/*
 * a1 -- block-key pooling.  [ailearn] §03, first QSA step and indexer figure
 * caption: the indexer keys of every non-overlapping 4-token micro-block are
 * averaged.  The block key is the plain mean (no RMSNorm, no block RoPE):
 *   kbar_b[d] = bf16_rne( (((k[4b][d] + k[4b+1][d]) + k[4b+2][d]) + k[4b+3][d]) * 0.25f )
 * with float32 adds in that order.  Bit-exact.
 *
 * For every sequence s, pools blocks blk_begin[s] <= b < blk_end[s] (device
 * int32 arrays) of idx_k into block_keys; other blocks are untouched.  The
 * caller guarantees 4*blk_end[s] <= tokens written for s.  max_span (host) is
 * an upper bound on blk_end[s]-blk_begin[s] used to size the launch; larger
 * spans are still pooled completely, only with fewer workgroups than ideal.
 * n_seq == 0 or max_span == 0 enqueues nothing.
 */
int qsa_pool_block_keys(const void* idx_k, int64_t ik_seq_stride,
                        void* block_keys, int64_t bk_seq_stride,
                        const int32_t* blk_begin, const int32_t* blk_end,
                        int32_t n_seq, int32_t max_span,
                        const int32_t* block_table, int64_t table_stride, int32_t page_tokens,
                        void* stream);

/*
 * a5 helper -- partial RoPE of cache keys at write time.  [card] and
 * [ailearn] config table: rotary on 64 of the 256 dims of a core head;
 * [ailearn] §03 second QSA step.  Rotate-half on dims 0..63 with pairs
 * (j, j+32), theta_j = pos * f_j taken in float64, cos/sin in float64
 * rounded to float32, rotation in float32, result rounded to bf16; dims
 * 64..255 are untouched.  In place.
 *
 * Row r, head h occupies x + r*row_stride + h*head_stride (bf16, 256 dims).
 * Its position is pos[r] (device int32) or, when pos == NULL, pos0 + r.
 * Used on the K cache once per token; queries are rotated inside the
 * attention kernels instead, which must be given the same frequencies.
 * inv_freq: HOST float64 [32] table of f_j, copied at the call; NULL gives
 * the native 1e7^(-j/32); qsa_yarn_rope fills the YaRN table.
 */
int qsa_rope_apply(void* x, int64_t row_stride, int64_t head_stride, int32_t n_heads,
                   const int32_t* pos, int32_t pos0, int32_t n_rows,
                   const double* inv_freq, void* stream);

/*
 * f4 -- YaRN context extension (host only, enqueues nothing).  [card]
 * structure paragraph and [ailearn] headline figures and §07 Deployment: the
 * native 262,144-token window is extended statically to 1M with YaRN.  The
 * pages give no constants; this is the YaRN paper's formula (Peng et al.,
 * 2023).  For pair j with theta = base^(-2j/64) and wavelength 2 pi / theta,
 *   r = orig_ctx / wavelength,  gamma = clamp((r - alpha) / (beta - alpha), 0, 1),
 *   inv_freq[j] = (1 - gamma) * theta / factor + gamma * theta      (float64)
 * and *softmax_scale = (0.1 ln factor + 1)^2 / 16 (float32; may be NULL), the
 * paper's temperature applied to the core logits.  The model's values are
 * base 1e7, factor 4, orig_ctx 262144, alpha 1, beta 32.  Give the table to
 * qsa_rope_apply, the attention calls and the indexer transforms, and the
 * scale to the attention calls.
 * Errors: QSA_ERR_INVALID_ARG for inv_freq == NULL, base <= 1, factor < 1,
 * orig_ctx <= 0, alpha < 0, beta <= alpha, or non-finite values.
 */
int qsa_yarn_rope(double base, double factor, double orig_ctx, double alpha, double beta,
                  double* inv_freq, float* softmax_scale);

/*
 * The pages' indexer transforms (optional; the plain path above omits them).
 * [ailearn] indexer figure caption and its note on the order of operations,
 * and §03 second QSA step: the key side average-pools each 4-token block,
 * then RMS-normalises it and rotates it at the block's position (partial
 * RoPE on 64 of the 128 dims); the query side RMS-normalises each projected
 * head and rotates it at the query's token position.  Feed the results to
 * qsa_index_select in place of the plain block keys and queries.
 *
 * Arithmetic, identical for both calls (x = one 128-dim vector):
 *   keys:    x[d] = float32 ((k0[d] + k1[d]) + k2[d]) + k3[d], times 0.25
 *            (the plain block key before its bf16 rounding);
 *   queries: x[d] = the bf16 input;
 *   then in float64: n[d] = (x[d] * (sum_d' x[d']^2 / 128 + eps)^(-1/2)) * gamma[d];
 *   for j < 32, with theta_j = pos * f_j:
 *            y[j]    = n[j] cos(theta_j) - n[j+32] sin(theta_j)
 *            y[j+32] = n[j+32] cos(theta_j) + n[j] sin(theta_j);
 *            y[d] = n[d] for d >= 64;
 *   out[d] = bf16_rne(float32_rne(y[d])).
 * pos = 4b for block b (the block's first token); the token position for a
 * query row (see the varlen convention).  Readings where the pages are
 * silent: eps (1e-6 is the usual choice), gamma (NULL = all ones; trained
 * weights replace it), f_j (NULL = 1e7^(-j/32), the core heads' frequencies).
 *
 *   gamma     float32 [128] device, or NULL
 *   eps       finite, >= 0 (eps = 0 turns an all-zero vector into NaN)
 *   inv_freq  float64 [32] HOST array of f_j, copied at the call, or NULL
 * Errors: QSA_ERR_INVALID_ARG for a negative count, a bad eps or a
 * non-finite f_j, and as for the plain calls.
 */

/* Key side: pools and transforms blocks blk_begin[s] <= b < blk_end[s] of
 * every sequence s exactly like qsa_pool_block_keys (same arguments, same
 * launch sizing); other blocks are untouched. */
int qsa_pool_block_keys_normed(const void* idx_k, int64_t ik_seq_stride,
                               void* block_keys, int64_t bk_seq_stride,
                               const int32_t* blk_begin, const int32_t* blk_end,
                               int32_t n_seq, int32_t max_span,
                               const float* gamma, double eps, const double* inv_freq,
                               const int32_t* block_table, int64_t table_stride,
                               int32_t page_tokens, void* stream);

/* Query side: q_raw and q_out are bf16 [n_q][4][128] (q_out may equal q_raw;
 * other overlaps are not allowed).  Row cu_q[s] + j of sequence s is
 * transformed at its position; rows that no sequence covers, or whose
 * position would be negative, are not written.  max_q_len as for
 * qsa_index_select. */
int qsa_index_query_transform(const void* q_raw, void* q_out,
                              const int32_t* cu_q, const int32_t* seq_len,
                              int32_t n_seq, int32_t n_q, int32_t max_q_len,
                              const float* gamma, double eps, const double* inv_freq,
                              void* stream);

/*
 * a2 + a3 -- indexer block scores and deterministic top-K_B block selection.
 * [ailearn] §03 BLOCK SCORE and CAUSAL SPARSE SET equations, third and fourth
 * QSA steps.  For query row i at position p (batch layout above), the
 * candidates are the completed blocks b < n_c = (p+1)/4 (a block counts once
 * its last token 4b+3 <= p), scored
 *   s_b = sum_h w[i][h] * ReLU( (q[i][h] . kbar_b) / sqrt(128) )   (float32)
 * The selection B_i is the K = min(budget, n_c) best candidates under the
 * order (score descending, block index ascending).
 *
 *   idx_q  bf16 [n_q][4][128]   indexer queries
 *   w      fp32 [n_q][4]        per-head weights, finite and >= 0 (scores are
 *                               then >= 0 and the kernels order them by their
 *                               float32 bit patterns; other weights give an
 *                               unspecified selection)
 *   sel    int32 [n_q][budget]  OUT: B_i in ascending block order, then -1 padding
 *   count  int32 [n_q]          OUT: K = min(budget, n_c); -1 for a row that no
 *                               sequence covers or whose n_c exceeds max_blocks
 * budget in 1..512.  The selection is exact with respect to the float32
 * scores the kernels compute (accumulation in MFMA order).  Needs workspace of
 * qsa_index_select_workspace(n_q, max_q_len, max_blocks) bytes, queried with
 * the same n_q, max_q_len and max_blocks as the call (the method differs for
 * max_q_len <= 4, where every score is kept); returns 0 for n_q <= 0,
 * max_q_len <= 0 or max_blocks < 0.
 */
size_t qsa_index_select_workspace(int32_t n_q, int32_t max_q_len, int32_t max_blocks);
int qsa_index_select(const void* idx_q, const float* w,
                     const int32_t* cu_q, const int32_t* seq_len,
                     int32_t n_seq, int32_t n_q, int32_t max_q_len, int32_t max_blocks,
                     const void* block_keys, int64_t bk_seq_stride,
                     int32_t budget, int32_t* sel, int32_t* sel_count,
                     void* workspace, size_t ws_bytes,
                     const int32_t* block_table, int64_t table_stride, int32_t page_tokens,
                     void* stream);

/*
 * a4 + a5 + a6 -- sparse prefill attention.  [ailearn] §03 CAUSAL SPARSE SET
 * equation (S_i = the selected blocks expanded to their 4 tokens, plus the
 * unfinished tail {4*n_c, ..., p}) and fifth QSA step (exact attention of the
 * 24 query heads / 2 KV heads over the original tokens of S_i).
 *
 * For every row i and head h (KV head g = h/12), with c = softmax_scale:
 *   out[i][h] = sum_{t in S_i} softmax_t( c * RoPE(q[i][h], p) . k_cache[g][t] ) v_cache[g][t]
 *   lse[i][h] = natural log of the softmax denominator (logits already scaled)
 * q is the raw (unrotated) query; k_cache holds keys already rotated at their
 * positions (qsa_rope_apply with the same inv_freq).  sel / sel_count as
 * written by qsa_index_select (ascending ids; a row with count < 0 gets NaN
 * output).
 *   q    bf16 [n_q][24][256]   out bf16 [n_q][24][256]   lse fp32 [n_q][24] or NULL
 *   inv_freq       HOST float64 [32] rotary frequencies, or NULL (1e7^(-j/32))
 *   softmax_scale  finite, > 0: 1/16 = 1/sqrt(256) natively; YaRN's from qsa_yarn_rope
 */
int qsa_attend_prefill(const void* q, const int32_t* cu_q, const int32_t* seq_len,
                       int32_t n_seq, int32_t n_q, int32_t max_q_len,
                       const void* k_cache, const void* v_cache,
                       int64_t kv_seq_stride, int64_t kv_head_stride,
                       const int32_t* sel, const int32_t* sel_count, int32_t budget,
                       void* out, float* lse, const double* inv_freq, float softmax_scale,
                       const int32_t* block_table, int64_t table_stride, int32_t page_tokens,
                       void* stream);

/*
 * a7 -- split-K decode attention plus combine.  Same mathematics as
 * qsa_attend_prefill for one query per sequence at position seq_len[s]-1
 * (row s of q, sel, out, lse).  The selected set is split across workgroups
 * (1 to 16 per row and KV head, fewer for larger batches); partial (max,
 * sum, output) triples go to the workspace and a combine pass merges them.
 * Needs qsa_attend_decode_workspace(n_seq) bytes.
 */
size_t qsa_attend_decode_workspace(int32_t n_seq);
int qsa_attend_decode(const void* q, const int32_t* seq_len, int32_t n_seq,
                      const void* k_cache, const void* v_cache,
                      int64_t kv_seq_stride, int64_t kv_head_stride,
                      const int32_t* sel, const int32_t* sel_count, int32_t budget,
                      void* out, float* lse, void* workspace, size_t ws_bytes,
                      const double* inv_freq, float softmax_scale,
                      const int32_t* block_table, int64_t table_stride, int32_t page_tokens,
                      void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the split-K
 * decode of qsa_attend_decode with no workspace argument.  Same arguments,
 * mathematics, kernels and results (bit for bit) as qsa_attend_decode.
 *
 * The partials live in a device array inside the library, one copy per GPU
 * it runs on, held until the process ends: 256 partials of 12,416 bytes
 * (3.2 MB), enough for every split of QSA_NOALLOC_MAX_SEQ = 128 sequences.
 * The call allocates nothing.  Its first call on a device looks the array up with that device
 * current, so `stream` must belong to the current device (or be NULL).  Every
 * call on one GPU shares that array: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race, so
 * order them.  Nothing in the array needs clearing between calls.
 * Errors: QSA_ERR_UNSUPPORTED for n_seq > QSA_NOALLOC_MAX_SEQ (checked on
 * the host before any HIP call); QSA_ERR_INVALID_ARG for a stream of another
 * device; otherwise as qsa_attend_decode.
 */
int qsa_attend_decode_noalloc(const void* q, const int32_t* seq_len, int32_t n_seq,
                              const void* k_cache, const void* v_cache,
                              int64_t kv_seq_stride, int64_t kv_head_stride,
                              const int32_t* sel, const int32_t* sel_count, int32_t budget,
                              void* out, float* lse, const double* inv_freq,
                              float softmax_scale, const int32_t* block_table,
                              int64_t table_stride, int32_t page_tokens, void* stream);

/*
 * f1 (multi-token decode) -- the split-K decode of qsa_attend_decode for a
 * varlen batch with a few query tokens per sequence, e.g. a new token plus
 * speculative (MTP) tokens: [ailearn] performance box (decode measured with 3
 * MTP steps).  Batch layout, mathematics and outputs as qsa_attend_prefill
 * (rows cu_q[s] .. cu_q[s+1]-1 at the last positions of sequence s); each
 * row's selected set is split across workgroups and combined as in
 * qsa_attend_decode.  Needs qsa_attend_decode_multi_workspace(n_q) bytes.
 */
size_t qsa_attend_decode_multi_workspace(int32_t n_q);
int qsa_attend_decode_multi(const void* q, const int32_t* cu_q, const int32_t* seq_len,
                            int32_t n_seq, int32_t n_q,
                            const void* k_cache, const void* v_cache,
                            int64_t kv_seq_stride, int64_t kv_head_stride,
                            const int32_t* sel, const int32_t* sel_count, int32_t budget,
                            void* out, float* lse, void* workspace, size_t ws_bytes,
                            const double* inv_freq, float softmax_scale,
                            const int32_t* block_table, int64_t table_stride,
                            int32_t page_tokens, void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* QSA_H_ */
