"""CPU oracle for the QSA (Qwen Sparse Attention) hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and this module imports
nothing from the product package.

Plain, slow and direct: numpy in float64, except at the rounding points the
method defines (listed per function).  No blocking, fusion or reordering
beyond what each definition states.

Pages cited (titles as published):
  [card]    "Qwen3.8-Flash-Next - 面向 Qwen4 架构的实验性预览权重发布"
            (aiboss88.com), model-card paragraph on the structure.
  [ailearn] "Qwen3.8-Flash-Next 没有缩小模型，它重写了每个参数何时上场"
            (ailearn.mscapital.top): the config table "公开 Config 的结构快照",
            section "03 · Attention" with the BLOCK SCORE and CAUSAL SPARSE SET
            equations and the five-step QSA list.
  [sysgeek] "Qwen3.8-Flash-Next：全新架构，迈向极致性价比" (sysgeek.cn),
            the QSA paragraph of the Attention section.

Readings where the pages leave a step open (each also stated where it is used):
  * block key = plain mean of the 4 token keys (no RMSNorm, no block RoPE);
  * score = sum_h w_h * ReLU(q_h . kbar_b / sqrt(128)); with w = 1 this ranks
    blocks exactly like the pages' unweighted, unscaled score;
  * ties in the top-K go to the lower block index;
  * core RoPE: rotate-half on dims 0..63, pairs (j, j+32), base 1e7, angles in
    float64;
  * softmax scale 1/sqrt(256) = 1/16; Q head h reads KV head floor(h/12).

Readings for YaRN (yarn_inv_freq, yarn_softmax_scale), which the pages name
without constants: the YaRN paper's published ramp with alpha = 1, beta = 32,
s = 4 over the native 262,144 tokens, and its temperature applied to the whole
logit; the indexer rotation takes the same table.

Readings for the pages' full indexer transforms (transform_block_keys,
transform_queries), which the plain path above leaves out:
  * RMSNorm over the 128 dims: x / sqrt(mean(x^2) + eps) * gamma, eps = 1e-6
    unless given, gamma = 1 unless given; on the query side per head;
  * the pooled mean enters the norm as the float32 sum-and-scale of the plain
    block key, before its bf16 rounding;
  * indexer RoPE: rotate-half on dims 0..63 of 128, pairs (j, j+32), the core's
    frequencies 1e7^(-j/32); keys at the block position p_b = 4b, queries at
    their token position;
  * everything after the float32 mean is float64; the result goes to float32
    (RNE), then to bf16 (RNE).

Arrays holding bf16 data are passed as float64 arrays whose values are exactly
representable in bf16 (the caller decodes bf16 losslessly).

Parity pins: every function here is checked against facts that do not come
from this file (closed forms, invariants, brute force, library routines); see
the tests whose names start with test_oracle_.  Two functions are comparison
allowances rather than steps of the method, and are pinned the same way:
selection_gap (a hand-worked boundary gap and allowance, and the allowance
against float32 scores summed in other orders) and attend_error_bound
(brute force over bf16-rounded and worst-case perturbed keys, and a
two-token case where it is nearly reached).
"""
from __future__ import annotations

import numpy as np

# Shapes of the QSA layer ([card] structure paragraph; [ailearn] config table).
R = 4                 # micro-block ratio r: tokens per block
TOKEN_BUDGET = 2048   # K, tokens kept from completed blocks
K_B = 512             # block budget ceil(K / r)   ([ailearn] CAUSAL SPARSE SET)
H_I, D_I = 4, 128     # indexer: 4 query heads over 1 shared key, width 128
H_Q, H_KV, D = 24, 2, 256
GROUP = H_Q // H_KV   # 12 query heads per KV head
D_ROPE = 64           # rotated dims of the core heads
ROPE_BASE = 1.0e7
SOFTMAX_SCALE = 1.0 / 16.0                       # 1/sqrt(256), a power of two
SCORE_SCALE = np.float32(1.0 / np.sqrt(128.0))   # 1/sqrt(d_I), rounded once to fp32


# ---------------------------------------------------------------- bf16 helper

def round_to_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float64.

    bf16 keeps the upper 16 bits of the IEEE-754 binary32 pattern.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if np.isnan(f).any():
        raise ValueError("NaN reached a bf16 rounding point")
    u = f.view(np.uint32).astype(np.uint64)
    half = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    hi = ((u + half) >> np.uint64(16)) & np.uint64(0xFFFF)
    return (hi.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------- indexer: pooling

def pool_block_keys(idx_k: np.ndarray, n_blocks: int) -> np.ndarray:
    """Mean of each non-overlapping 4-token micro-block of the indexer key.

    [ailearn] §03, first QSA step (average-pool the keys over non-overlapping
    4-token micro-blocks) and the indexer figure caption (pooling on the key
    side).  Reading: the block key is the plain mean; the pages' RMSNorm and
    block RoPE that follow need trained weights and are not applied.

    Rounding points: the sum is taken in float32 in token order
    ((k0 + k1) + k2) + k3, multiplied by 0.25 in float32, then rounded to bf16.

    idx_k: [L][128] token keys (bf16 values).  Returns [n_blocks][128].
    """
    k = np.asarray(idx_k, dtype=np.float64)
    assert k.shape[0] >= R * n_blocks
    # t[j] holds token j of every block; the arithmetic is elementwise per block.
    t = k[:R * n_blocks].reshape(n_blocks, R, D_I).astype(np.float32)
    s = t[:, 0] + t[:, 1]
    s = s + t[:, 2]
    s = s + t[:, 3]
    return round_to_bf16(s * np.float32(0.25))


# -------------------------------------------------------- indexer: scoring

def completed_blocks(i: int) -> int:
    """n_c(i): blocks b whose last token p_b + r - 1 = 4b + 3 is at or before i.

    [ailearn] §03, BLOCK SCORE equation: a block is scored only when
    p_b + r - 1 <= i (reading p_b = r*b, the block's first token); every other
    block scores minus infinity and is never a candidate.
    """
    return (i + 1) // R


def block_scores(q_i: np.ndarray, w_i: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Indexer score of each candidate block for one query.

    [ailearn] §03 BLOCK SCORE equation and third QSA step: the 4 indexer query
    heads each take a dot product with the shared pooled key, ReLU is applied,
    and the heads are summed.  Reading: each head is also weighted by w_h and
    the dot is scaled by 1/sqrt(128); with w = 1 this orders blocks as the
    unweighted form does.

    Rounding points (float32 decides the selection on both sides):
      dot_h = sum_d q_h[d] kbar[d]              in float64
      t_h   = float32(dot_h)
      u_h   = float32(max(t_h, 0) * SCORE_SCALE)
      s     = ((w0*u0 + w1*u1) + w2*u2) + w3*u3 each product and sum rounded to float32
      -0 is returned as +0.

    q_i: [4][128], w_i: [4] float32, kbar: [n][128] (the n candidate blocks).
    Returns float32 [n].
    """
    q = np.asarray(q_i, dtype=np.float64)
    kb = np.asarray(kbar, dtype=np.float64).reshape(-1, D_I)
    w = np.asarray(w_i, dtype=np.float32)
    dots = q @ kb.T                                   # [4][n] float64
    t = dots.astype(np.float32)
    u = np.maximum(t, np.float32(0.0)) * SCORE_SCALE  # float32
    acc = np.zeros(kb.shape[0], dtype=np.float32)
    for h in range(H_I):
        acc = acc + w[h] * u[h]
    acc[acc == 0] = np.float32(0.0)
    return acc


# ------------------------------------------------------ indexer: selection

def select_blocks(scores: np.ndarray, budget: int) -> np.ndarray:
    """B_i: the min(budget, n_c) best candidates, returned in ascending block order.

    [ailearn] §03 CAUSAL SPARSE SET equation (top-K_B of the block scores,
    K_B = ceil(K/r) = 512) and fourth QSA step (at most 512 complete blocks).
    Reading: the order is score descending, then block index ascending, so
    equal scores keep the lower block; fewer candidates than the budget means
    all of them are kept.
    """
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)
    n = s.shape[0]
    k_eff = min(int(budget), n)
    order = np.lexsort((np.arange(n), -s))
    return np.sort(order[:k_eff]).astype(np.int64)


def sparse_token_set(blocks: np.ndarray, i: int) -> np.ndarray:
    """S_i = Expand(B_i) united with the current unfinished tail {r*n_c(i), ..., i}.

    [ailearn] §03 CAUSAL SPARSE SET equation and its note that the unfinished
    current block is kept because it is causally visible.  Returns token
    positions in ascending order of block, then the tail.
    """
    b = np.asarray(blocks, dtype=np.int64)
    expanded = (R * b[:, None] + np.arange(R)[None, :]).reshape(-1)
    tail = np.arange(R * completed_blocks(i), i + 1, dtype=np.int64)
    return np.concatenate([expanded, tail])


# ----------------------------------------- indexer: the pages' transforms

RMS_EPS = 1.0e-6      # reading: the pages give no epsilon
D_I_ROPE = 64         # [ailearn] §03 second QSA step: the indexer rotates 64 of its 128 dims


def index_inv_freq() -> np.ndarray:
    """The 32 rotary frequencies 1e7^(-j/32) of the indexer's 64 rotated dims.

    [ailearn] §03 second QSA step (partial RoPE, 64 of 128 indexer dims).
    Reading: the same base and spacing as the core heads' rotary dims.
    """
    j = np.arange(D_I_ROPE // 2, dtype=np.float64)
    return ROPE_BASE ** (-2.0 * j / D_I_ROPE)


def rms_norm(x: np.ndarray, gamma=None, eps: float = RMS_EPS) -> np.ndarray:
    """RMS normalisation over the last axis, in float64.

    [ailearn] indexer figure caption and its note on the order of operations
    (the pooled key, and each projected query, are RMS-normalised).
    y = (x * (mean(x^2) + eps)^(-1/2)) * gamma.
    """
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    g = np.ones(x.shape[-1]) if gamma is None else np.asarray(gamma, dtype=np.float64)
    return (x * r) * g


def index_rope(x: np.ndarray, pos, inv_freq=None) -> np.ndarray:
    """Partial rotary embedding on the first 64 of the 128 indexer dims, float64.

    [ailearn] §03 second QSA step.  Rotate-half with pairs (j, j+32):
      y_j = x_j cos(theta_j) - x_{j+32} sin(theta_j)
      y_{j+32} = x_{j+32} cos(theta_j) + x_j sin(theta_j),  theta_j = pos * f_j;
    dims 64..127 pass through.  x: [..., 128]; pos broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    f = index_inv_freq() if inv_freq is None else np.asarray(inv_freq, dtype=np.float64)
    theta = np.asarray(pos, dtype=np.float64)[..., None] * f
    c, s = np.cos(theta), np.sin(theta)
    h = D_I_ROPE // 2
    y = x.copy()
    y[..., :h] = x[..., :h] * c - x[..., h:D_I_ROPE] * s
    y[..., h:D_I_ROPE] = x[..., h:D_I_ROPE] * c + x[..., :h] * s
    return y


def _to_bf16_via_f32(y: np.ndarray) -> np.ndarray:
    return round_to_bf16(np.asarray(y, dtype=np.float64).astype(np.float32))


def transform_block_keys(idx_k: np.ndarray, n_blocks: int, gamma=None, eps: float = RMS_EPS,
                         inv_freq=None, rounded: bool = True, first_block: int = 0) -> np.ndarray:
    """The pages' block key: pool, then RMSNorm, then block-position partial RoPE.

    [ailearn] indexer figure caption and its note on the order (key side:
    average-pool each 4 tokens, then RMSNorm and block-level partial RoPE);
    §03 first and second QSA steps.  Block b is rotated at p_b = 4b, the
    block's first token (the p_b of the BLOCK SCORE condition).

    The mean is the float32 ((k0 + k1) + k2) + k3, times 0.25, as for the plain
    block key but not rounded to bf16; the rest is float64, then float32, then
    bf16 (skipped with rounded=False, which returns the float64 values).
    idx_k: [L][128] token keys (bf16 values), token 0 being the first token of
    block first_block.  Returns [n_blocks][128].
    """
    k = np.asarray(idx_k, dtype=np.float64)
    assert k.shape[0] >= R * n_blocks
    t = k[:R * n_blocks].reshape(n_blocks, R, D_I).astype(np.float32)
    m = ((t[:, 0] + t[:, 1]) + t[:, 2]) + t[:, 3]
    m = (m * np.float32(0.25)).astype(np.float64)
    y = index_rope(rms_norm(m, gamma, eps), R * (first_block + np.arange(n_blocks)), inv_freq)
    return _to_bf16_via_f32(y) if rounded else y


def transform_queries(q_raw: np.ndarray, pos, gamma=None, eps: float = RMS_EPS,
                      inv_freq=None, rounded: bool = True) -> np.ndarray:
    """The pages' indexer query: per-head RMSNorm, then token-position RoPE.

    [ailearn] indexer figure caption and its note on the order (query side:
    independent projections, normalisation, then the current position's
    rotary embedding).  q_raw: [..., 4, 128] projected queries (bf16 values);
    pos: the token position of each row, broadcast against q_raw[..., 0, 0].
    float64, then float32, then bf16 (skipped with rounded=False).
    """
    q = np.asarray(q_raw, dtype=np.float64)
    p = np.asarray(pos, dtype=np.float64)[..., None]      # one position per row, all heads
    y = index_rope(rms_norm(q, gamma, eps), p, inv_freq)
    return _to_bf16_via_f32(y) if rounded else y


# -------------------------------------------------- YaRN context extension

NATIVE_CTX = 262144      # [card]; [ailearn] §07: native context, extended to 1M with YaRN
YARN_FACTOR = 4.0        # reading: s = 4 makes 4 * 262144 = 1,048,576 positions
YARN_ALPHA, YARN_BETA = 1.0, 32.0   # reading: the YaRN paper's ramp bounds


def yarn_inv_freq(factor: float = YARN_FACTOR, orig_ctx: int = NATIVE_CTX, base: float = ROPE_BASE,
                  alpha: float = YARN_ALPHA, beta: float = YARN_BETA) -> np.ndarray:
    """YaRN-scaled frequencies of the 32 rotary pairs (64 rotated dims).

    [ailearn] headline figures (262K -> 1M, YaRN) and §07 Deployment, [card]
    structure paragraph: the native 262,144-token window is extended
    statically to 1M with YaRN.  The pages give no
    constants, so this follows the YaRN paper (Peng et al., 2023) as
    published: for the pair with frequency theta (wavelength 2 pi / theta),
    r = orig_ctx / wavelength counts the rotations over the native window;
    gamma(r) = 0 below alpha, 1 above beta, linear in between; the new
    frequency is (1 - gamma) theta / s + gamma theta.  float64.
    """
    j = np.arange(D_ROPE // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / D_ROPE)
    wavelength = 2.0 * np.pi / theta
    r = orig_ctx / wavelength
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / factor + gamma * theta


def yarn_softmax_scale(factor: float = YARN_FACTOR) -> float:
    """Softmax scale of the core attention under YaRN: the logits q.k / 16 are
    divided by the paper's temperature t, with sqrt(1/t) = 0.1 ln(s) + 1.
    Reading: the whole logit is scaled (the paper's form for full RoPE)."""
    return SOFTMAX_SCALE * (0.1 * np.log(factor) + 1.0) ** 2


# ------------------------------------------------------------ core attention

def rope(x: np.ndarray, pos, inv_freq=None) -> np.ndarray:
    """Partial rotary embedding on the first 64 of 256 dims.

    [card] structure paragraph and [ailearn] config table (rotary dim 64) and
    second QSA step (the core uses 64 of 256 dims).  Reading: rotate-half with
    pairs (j, j+32), angle theta_j = pos * f_j with f_j = 1e7^(-j/32) unless a
    table is given (yarn_inv_freq), everything in float64; dims 64..255 pass
    through.

    x: [..., 256]; pos: scalar or array broadcast against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    p = np.asarray(pos, dtype=np.float64)[..., None]
    j = np.arange(D_ROPE // 2, dtype=np.float64)
    f = ROPE_BASE ** (-2.0 * j / D_ROPE) if inv_freq is None else np.asarray(inv_freq, np.float64)
    theta = p * f
    c, s = np.cos(theta), np.sin(theta)
    y = x.copy()
    x1, x2 = x[..., :D_ROPE // 2], x[..., D_ROPE // 2:D_ROPE]
    y[..., :D_ROPE // 2] = x1 * c - x2 * s
    y[..., D_ROPE // 2:D_ROPE] = x2 * c + x1 * s
    return y


def attend(q_i: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, tokens: np.ndarray,
           i: int, inv_freq=None, scale=None, k_bf16: bool = False):
    """Exact GQA softmax attention of query i over the token set S_i.

    [ailearn] §03 fifth QSA step: the 24-query / 2-KV core attends exactly over
    the original tokens of S_i.  Q and K are rotated at their own positions
    (with the frequency table inv_freq, default 1e7^(-j/32)); logits are
    scaled by `scale` (default 1/16); head h reads KV head floor(h/12).

    q_i: [24][256] raw query; tokens: the positions of S_i; k_rows, v_rows:
    [len(tokens)][2][256] the raw cache rows of those tokens (K not rotated).
    Returns (O [24][256], lse [24]) in float64, lse = log sum exp of the
    scaled logits.

    k_bf16=True rounds the rotated keys to bf16 (through float32): the
    values of a K cache that stores each key once, rotated at its position,
    in bf16.  The method's result is k_bf16=False (exact rotated keys);
    k_bf16=True gives the exact attention over such a cache's stored values,
    for checking a kernel that is handed that cache.
    """
    S = np.asarray(tokens, dtype=np.int64)
    qr = rope(np.asarray(q_i, dtype=np.float64), i, inv_freq)
    kr = rope(np.asarray(k_rows, dtype=np.float64), S[:, None], inv_freq)     # [n][2][256]
    if k_bf16:
        kr = _to_bf16_via_f32(kr)
    sm = SOFTMAX_SCALE if scale is None else float(scale)
    vs = np.asarray(v_rows, dtype=np.float64)                       # [n][2][256]
    assert kr.shape[0] == S.shape[0] and vs.shape[0] == S.shape[0]
    out = np.empty((H_Q, D), dtype=np.float64)
    lse = np.empty(H_Q, dtype=np.float64)
    for h in range(H_Q):
        g = h // GROUP
        logits = (kr[:, g, :] @ qr[h]) * sm
        m = logits.max()
        p = np.exp(logits - m)
        l = p.sum()
        out[h] = (p @ vs[:, g, :]) / l
        lse[h] = m + np.log(l)
    return out, lse


# ---------------------------------------------------------------- pipeline

def qsa_query(idx_q_i, w_i, kbar, q_i, k_raw, v, i: int, budget: int):
    """All steps for one query at position i: score, select, expand, attend.

    kbar must hold at least n_c(i) pooled block keys of the query's sequence;
    k_raw and v hold the raw cache rows of that sequence ([L][2][256]).
    Returns (blocks, out, lse).
    """
    n_c = completed_blocks(i)
    s = block_scores(idx_q_i, w_i, np.asarray(kbar)[:n_c])
    blocks = select_blocks(s, budget)
    tokens = sparse_token_set(blocks, i)
    out, lse = attend(q_i, np.asarray(k_raw)[tokens], np.asarray(v)[tokens], tokens, i)
    return blocks, out, lse


def selection_gap(scores: np.ndarray, q_i, w_i, kbar, budget: int):
    """Boundary gap and rounding allowance used to compare a float32 selection.

    Returns (gap, delta, s_k): gap = s_(K) - s_(K+1) of the sorted scores (inf
    when every candidate is kept), s_k = s_(K), and delta = 2^-15 * max_b
    sum_h w_h sum_d |q_h[d] kbar_b[d]| / sqrt(128), an upper bound on how far
    a float32-accumulated score can sit from this oracle's score (128-term
    dot products carry a relative error below 2^-17; 4x slack).
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    k_eff = min(int(budget), n)
    srt = np.sort(s)[::-1]
    gap = np.inf if k_eff >= n else srt[k_eff - 1] - srt[k_eff]
    s_k = srt[k_eff - 1] if k_eff > 0 else np.inf
    absdots = np.abs(np.asarray(q_i, np.float64)) @ np.abs(np.asarray(kbar, np.float64)).T
    mag = (np.asarray(w_i, np.float64)[:, None] * absdots).sum(0) / np.sqrt(128.0)
    delta = 2.0 ** -15 * (mag.max() if mag.size else 0.0)
    return gap, delta, s_k


# Error model of an attention that reads a bf16 cache of rotated keys and
# computes in float32 (used by attend_error_bound).
BF16_U = 2.0 ** -8       # bf16 unit roundoff: |bf16(x) - x| <= 2^-8 |x| (8-bit significand, RNE)
F32_ROTATION = 2.0 ** -21   # float32 cos/sin and rotation, relative to |x_j| + |x_{j+32}|
F32_LOGIT = 2.0 ** -14      # float32 logits, relative to sum_d |q_d k_d| (256 terms, 4x slack)
F32_WEIGHTED_SUM = 2.0 ** -12   # float32 softmax weights and sum_j p_j v_j, relative to sum_j p_j |v_j|


def k_cache_rounding_allowance(k_rows: np.ndarray, tokens: np.ndarray, inv_freq=None) -> np.ndarray:
    """Per-element bound on |stored key - exact rotated key| for a cache that
    stores each key rotated at its position in bf16 ([ailearn] §03: the fifth
    QSA step attends over the original tokens, the second rotates 64 dims).

    Rotated dims (pair j, j+32) go through float32 cos/sin and arithmetic,
    then bf16 RNE:  e_d = 2^-8 |k~_d| + 2^-21 (|k_j| + |k_{j+32}|), with k~
    the exact rotation and k the raw key; dims 64..255 are stored as given
    (e = 0).  k_rows: raw keys [n][2][256] at positions `tokens`.
    """
    S = np.asarray(tokens, dtype=np.int64)
    k = np.asarray(k_rows, dtype=np.float64)
    kr = rope(k, S[:, None], inv_freq)
    e = np.zeros_like(kr)
    h = D_ROPE // 2
    pair = np.abs(k[..., :h]) + np.abs(k[..., h:D_ROPE])            # |x_j| + |x_{j+32}|
    e[..., :h] = BF16_U * np.abs(kr[..., :h]) + F32_ROTATION * pair
    e[..., h:D_ROPE] = BF16_U * np.abs(kr[..., h:D_ROPE]) + F32_ROTATION * pair
    return e


def attend_error_bound(q_i: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                       tokens: np.ndarray, i: int, inv_freq=None, scale=None,
                       k_stored: bool = False):
    """Per-element bound on how far an attention computed from a bf16 cache of
    rotated keys, in float32, can sit from attend()'s float64 result (before
    the output's own bf16 rounding).  Not a step of the method: the tolerance
    the parity tests derive from the cache format.

    Stored key element d differs from the exact rotated one by at most e_d
    (k_cache_rounding_allowance); with k_stored=True the reference itself
    attends over the stored values (attend(k_bf16=True)) and e = 0.  Logit t
    of head h then moves by eps_t, |eps_t| <= beta_t with
        beta_t = c * ( sum_{d<64} |q~_d| e_td + 2^-14 sum_d |q~_d| |k~_td| ),
    the second term for float32 dot products.  The weights become
    p'_t = p_t exp(eps_t - L), L = log sum_u p_u exp(eps_u) in [L-, L+] =
    [log sum_u p_u exp(-beta_u), log sum_u p_u exp(beta_u)], so
        |p'_t / p_t - 1| <= r_t = max(exp(beta_t - L-) - 1, 1 - exp(-beta_t - L+)),
    and since sum_t (p'_t - p_t) = 0, for every dim
        |O' - O| <= sum_t p_t r_t |v_t - O| + 2^-12 sum_t p_t |v_t|,
    the last term for float32 weights and accumulation.  lse moves by L:
    at most max(L+, -L-) plus the same float32 slack.

    Same arguments as attend().  Returns (bound [24][256], lse_bound [24]).
    """
    S = np.asarray(tokens, dtype=np.int64)
    qr = rope(np.asarray(q_i, dtype=np.float64), i, inv_freq)
    kr = rope(np.asarray(k_rows, dtype=np.float64), S[:, None], inv_freq)   # [n][2][256]
    if k_stored:
        kr = _to_bf16_via_f32(kr)
        ek = np.zeros_like(kr)
    else:
        ek = k_cache_rounding_allowance(k_rows, S, inv_freq)
    sm = SOFTMAX_SCALE if scale is None else float(scale)
    vs = np.asarray(v_rows, dtype=np.float64)
    bound = np.empty((H_Q, D), dtype=np.float64)
    lse_bound = np.empty(H_Q, dtype=np.float64)
    for hq in range(H_Q):
        g = hq // GROUP
        aq = np.abs(qr[hq])
        logits = (kr[:, g, :] @ qr[hq]) * sm
        beta = sm * (ek[:, g, :] @ aq + F32_LOGIT * (np.abs(kr[:, g, :]) @ aq))
        p = np.exp(logits - logits.max())
        p /= p.sum()
        o = p @ vs[:, g, :]
        l_hi = np.log(p @ np.exp(beta))
        l_lo = np.log(p @ np.exp(-beta))
        r = np.maximum(np.expm1(beta - l_lo), -np.expm1(-beta - l_hi))
        bound[hq] = (p * r) @ np.abs(vs[:, g, :] - o) + F32_WEIGHTED_SUM * (p @ np.abs(vs[:, g, :]))
        lse_bound[hq] = max(l_hi, -l_lo) + F32_WEIGHTED_SUM
    return bound, lse_bound


def dense_causal_gqa(q_i: np.ndarray, k_raw: np.ndarray, v: np.ndarray, i: int):
    """Textbook causal GQA attention of query i over every token 0..i.

    Deliberately separate from attend(): token-by-token loops, no token set.
    Used to pin the sparse path, which must equal this whenever the budget
    covers every completed block.
    """
    qr = rope(np.asarray(q_i, dtype=np.float64), i)
    out = np.zeros((H_Q, D), dtype=np.float64)
    lse = np.zeros(H_Q, dtype=np.float64)
    k_raw = np.asarray(k_raw, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    for h in range(H_Q):
        g = h // GROUP
        logits = [float(rope(k_raw[j, g], j) @ qr[h]) / 16.0 for j in range(i + 1)]
        m = max(logits)
        weights = [np.exp(x - m) for x in logits]
        total = sum(weights)
        acc = np.zeros(D)
        for j in range(i + 1):
            acc += weights[j] * v[j, g]
        out[h] = acc / total
        lse[h] = m + np.log(total)
    return out, lse
