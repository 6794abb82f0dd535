"""Helpers shared by the parity tests: feed a generated batch to the oracle
and compare the HIP path's results with it.  Only tests import this."""
from __future__ import annotations

import numpy as np
import torch

from oracle import qsa_oracle as O

# attention tolerance (bf16 in/out, float32 accumulation)
MAX_ABS = 1e-2
REL_L2 = 5e-3


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


class OracleView:
    """Oracle-side view of one QSABatch (float64 arrays, per sequence)."""

    def __init__(self, b, transforms=False, gamma_k=None, gamma_q=None, eps=O.RMS_EPS,
                 yarn=False):
        """transforms=True: block keys and indexer queries as the pages'
        transforms make them (gamma_* are numpy arrays or None).  yarn=True:
        every rotation takes the oracle's YaRN table and the core attention
        its softmax scale."""
        self.b = b
        self.inv_freq = O.yarn_inv_freq() if yarn else None
        self.scale = O.yarn_softmax_scale() if yarn else None
        self.lens = b.seq_lens_host()
        self.cu = b.cu_q_host()
        self.pos = b.q_pos_host()
        self.seq = b.q_seq_host()
        self.transforms, self.gamma_k, self.gamma_q, self.eps = transforms, gamma_k, gamma_q, eps
        self._kb = {}

    def kbar(self, s):
        if s not in self._kb:
            k, n = np64(self.b.idx_k[s]), self.lens[s] // O.R
            self._kb[s] = (O.transform_block_keys(k, n, self.gamma_k, self.eps, self.inv_freq)
                           if self.transforms else O.pool_block_keys(k, n))
        return self._kb[s]

    def query(self, row):
        """The indexer query heads [4][128] of a row, as scored."""
        q = np64(self.b.idx_q[row])
        if self.transforms:
            q = O.transform_queries(q, self.pos[row], self.gamma_q, self.eps, self.inv_freq)
        return q

    def rows(self, s, tokens):
        """Raw K and V rows [n][2][256] of the listed tokens of sequence s."""
        t = torch.as_tensor(np.asarray(tokens), dtype=torch.long, device=self.b.k.device)
        k = np64(self.b.k[s][:, t, :]).transpose(1, 0, 2)
        v = np64(self.b.v[s][:, t, :]).transpose(1, 0, 2)
        return k, v

    def scores(self, row):
        s, p = self.seq[row], self.pos[row]
        n_c = O.completed_blocks(p)
        return O.block_scores(self.query(row), self.b.w[row].cpu().numpy(), self.kbar(s)[:n_c])

    def select(self, row):
        return O.select_blocks(self.scores(row), self.b.budget)

    def attend(self, row, blocks, k_stored=False):
        """The oracle's attention of a row over its selected blocks and tail:
        (out, lse, bound, lse_bound).  k_stored=False is the method's result
        (exactly rotated keys) with the allowance for a bf16 cache of rotated
        keys; k_stored=True attends over that cache's stored values, for
        tests whose input is the stored cache itself."""
        s, p = self.seq[row], self.pos[row]
        tokens = O.sparse_token_set(np.asarray(blocks, dtype=np.int64), p)
        return self._attend_tokens(row, s, p, tokens, k_stored)

    def _attend_tokens(self, row, s, p, tokens, k_stored):
        k, v = self.rows(s, tokens)
        q = np64(self.b.q[row])
        out, lse = O.attend(q, k, v, tokens, p, self.inv_freq, self.scale, k_bf16=k_stored)
        bound, lse_bound = O.attend_error_bound(q, k, v, tokens, p, self.inv_freq, self.scale,
                                                k_stored=k_stored)
        return out, lse, bound, lse_bound

    def dense(self, row):
        """Textbook causal GQA over every token 0..pos (for budget >= n_c),
        with the same allowance as attend()."""
        s, p = self.seq[row], self.pos[row]
        k, v = self.rows(s, np.arange(p + 1))
        q = np64(self.b.q[row])
        out, lse = O.dense_causal_gqa(q, k, v, p)
        bound, lse_bound = O.attend_error_bound(q, k, v, np.arange(p + 1), p)
        return out, lse, bound, lse_bound


def check_selection(view: OracleView, row: int, gpu_ids, gpu_count: int, exact: bool = False):
    """Rule for float32 selections: bit-exact when the oracle's boundary gap
    exceeds the rounding allowance delta (always, for exact-grid inputs);
    otherwise every choice must lie within delta of the boundary score.
    Returns 'exact' or 'near'."""
    b = view.b
    s, p = view.seq[row], view.pos[row]
    n_c = O.completed_blocks(p)
    k_eff = min(b.budget, n_c)
    assert gpu_count == k_eff, (row, gpu_count, k_eff)
    ids = np.asarray(gpu_ids[:gpu_count], dtype=np.int64)
    assert np.all(np.asarray(gpu_ids[gpu_count:]) == -1), row
    assert np.all(np.diff(ids) > 0), ("not strictly ascending", row)
    assert k_eff == 0 or (ids[0] >= 0 and ids[-1] < n_c), row
    sc = view.scores(row)
    want = O.select_blocks(sc, b.budget)
    gap, delta, s_k = O.selection_gap(sc, view.query(row), b.w[row].cpu().numpy(),
                                      view.kbar(s)[:n_c], b.budget)
    if exact or gap > delta:
        assert np.array_equal(ids, want), (row, np.setdiff1d(ids, want)[:8], np.setdiff1d(want, ids)[:8])
        return "exact"
    chosen = np.zeros(n_c, bool)
    chosen[ids] = True
    assert np.all(sc[chosen] >= s_k - delta), row
    assert np.all(sc[~chosen] <= s_k + delta), row
    return "near"


def allowed_error(ref_out, bound):
    """Per-element limit on |gpu - oracle| for a bf16 output: MAX_ABS, or,
    where that is exceeded, the oracle's allowance for the bf16 K cache and
    float32 arithmetic (`bound`, from O.attend_error_bound) plus half a bf16
    ulp of the output's own rounding at that magnitude."""
    a = np.abs(np.asarray(ref_out, dtype=np.float64)) + np.asarray(bound, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    half_ulp = np.exp2(e - 8.0)
    return np.maximum(MAX_ABS, bound + half_ulp)


def check_attention(gpu_out, gpu_lse, ref, label=""):
    """One row's [24][256] output against the oracle's ref = (out, lse, bound,
    lse_bound): every element within MAX_ABS or, failing that, within the
    derived allowance (allowed_error); relative L2 within REL_L2; lse within
    1e-2 or its allowance.  Returns (max-abs error, relative L2, number of
    elements that needed the allowance)."""
    ref_out, ref_lse, bound, lse_bound = ref
    o = np64(gpu_out)
    err = np.abs(o - ref_out)
    assert np.isfinite(o).all(), label
    lim = allowed_error(ref_out, bound)
    bad = err > lim
    assert not bad.any(), (label, float(err[bad].max()), float(lim[bad].min()),
                           float(np.abs(ref_out).max()))
    rel = np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out)
    assert rel <= REL_L2, (label, rel)
    if gpu_lse is not None:
        lerr = np.abs(np64(gpu_lse) - ref_lse)
        assert (lerr <= np.maximum(1e-2, lse_bound)).all(), (label, lerr.max())
    return err.max(), rel, int((err > MAX_ABS).sum())
