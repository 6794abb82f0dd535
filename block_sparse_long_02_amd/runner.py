"""One QSA layer's device state and the ABI calls of a prefill or decode step.

The runner owns the caches and output buffers of one batch (torch device
memory) and issues, per step, exactly the libqsa calls of the hot path:
pool the newly completed blocks, select blocks for every query, attend.
It does no arithmetic of its own.
"""
from __future__ import annotations

import copy

import torch

from . import qsa
from .workloads import QSABatch, R, v_cache_layout


def piece_bounds(n: int, parts: int) -> list[int]:
    """Row boundaries [0, ..., n] of a chunk cut into `parts` consecutive
    pieces: the first an eighth of the rows, so that the attention starts
    early; with three or more pieces the last an eighth too, so that the
    attention left running alone at the end is short; the pieces between
    equal (some pieces may be empty when n < parts)."""
    if parts <= 1:
        return [0, n]
    first = (n + 7) // 8
    last = n // 8 if parts >= 3 else 0
    mid = parts - 1 - (1 if parts >= 3 else 0)
    span = n - first - last
    return [0] + [first + span * i // mid for i in range(mid + 1)] + ([n] if parts >= 3 else [])


class QSARunner:
    def __init__(self, batch: QSABatch, decode: bool | None = None, transforms: bool = False,
                 gamma_k=None, gamma_q=None, eps: float = 1e-6, yarn: bool = False,
                 paged: int | None = None, page_seed: int = 0, shared_pages=None):
        """transforms=True applies the pages' indexer transforms: block keys are
        pooled, RMS-normalised and rotated; each step first normalises and
        rotates the indexer queries into a buffer of its own.  yarn=True
        extends the native 262,144-token window with YaRN (factor 4): every
        rotation (K cache, queries, indexer transforms) takes the YaRN
        frequencies and the core attention its softmax scale.  paged=P keeps
        every cache in pools of P-token pages, in a seeded random physical
        order; shared_pages = {dst: (src, n)} maps the first n pages of
        sequence dst onto those of src (the caller makes their tokens equal),
        as a prefix cache would."""
        b = batch
        assert b.idx_q.is_cuda, "batch must live on the GPU"
        self.b = b
        self.decode = (b.meta.get("kind") == "decode") if decode is None else decode
        # several query tokens per sequence, attended with the split-K decode
        self.mtp = b.meta.get("kind") == "mtp_decode" and not self.decode
        dev = b.idx_q.device
        lens = b.seq_lens_host()
        cu = b.cu_q_host()
        self.n_seq, self.n_q = b.n_seq, b.n_q
        self.max_q_len = b.max_q_len()
        self.max_blocks = b.max_blocks()
        self.budget = b.budget
        cap = b.l_cap
        self.transforms, self.gamma_k, self.gamma_q, self.eps = transforms, gamma_k, gamma_q, eps
        self.idx_q_t = torch.empty_like(b.idx_q) if transforms else None
        self.inv_freq, self.softmax_scale = qsa.yarn_rope() if yarn else (None, qsa.SOFTMAX_SCALE)

        # caches: K rotated once at its positions (cache-write time), V re-laid out
        self.k_cache = b.k.clone()
        for s in range(self.n_seq):
            qsa.rope_apply(self.k_cache[s], row_stride=256, head_stride=cap * 256, n_heads=2,
                           n_rows=lens[s], pos0=0, inv_freq=self.inv_freq)
        self.v_cache = v_cache_layout(b.v)
        self.idx_k = b.idx_k
        self.block_keys = torch.zeros((self.n_seq, cap // R, 128), dtype=torch.bfloat16, device=dev)
        self.pages = None
        if paged:
            self._to_pages(int(paged), page_seed, shared_pages or {})

        # blocks already in the cache before this step, and the ones the step completes
        before = [(lens[s] - (cu[s + 1] - cu[s])) // R for s in range(self.n_seq)]
        after = [lens[s] // R for s in range(self.n_seq)]
        zero = torch.zeros(self.n_seq, dtype=torch.int32, device=dev)
        t_before = torch.tensor(before, dtype=torch.int32, device=dev)
        if max(before) > 0:
            self._pool(zero, t_before, max(before))
        self.pool_begin = t_before
        self.pool_end = torch.tensor(after, dtype=torch.int32, device=dev)
        self.pool_span = max(a - c for a, c in zip(after, before))

        self.sel = torch.empty((self.n_q, self.budget), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((self.n_q,), dtype=torch.int32, device=dev)
        self.out = torch.empty((self.n_q, 24, 256), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((self.n_q, 24), dtype=torch.float32, device=dev)
        ws = qsa.index_select_workspace(self.n_q, self.max_q_len, self.max_blocks)
        self.ws_index = torch.empty((max(ws, 16),), dtype=torch.uint8, device=dev)
        wsd = (qsa.attend_decode_workspace(self.n_seq) if self.decode else
               qsa.attend_decode_multi_workspace(self.n_q) if self.mtp else 16)
        self.ws_decode = torch.empty((max(wsd, 16),), dtype=torch.uint8, device=dev)

    def _to_pages(self, P, seed, shared):
        """Move the caches into page pools (the layouts of the paged ABI)."""
        dev, cap = self.idx_k.device, self.b.l_cap
        npg = -(-cap // P)
        g = torch.Generator().manual_seed(seed)
        table = torch.randperm(self.n_seq * npg, generator=g).to(torch.int32).view(self.n_seq, npg)
        for dst, (src, n) in shared.items():
            table[dst, :n] = table[src, :n]
        self.block_table = table.contiguous().to(dev)
        self.pages = (self.block_table, P)
        n_tok = self.n_seq * npg * P
        t = torch.arange(cap, device=dev)
        tok = (self.block_table[:, t // P].long() * P + t % P).reshape(-1)
        tb = torch.arange(cap // R, device=dev)
        blk = (self.block_table[:, (R * tb) // P].long() * (P // R) + tb % (P // R)).reshape(-1)
        idx_k = torch.zeros((n_tok, 128), dtype=torch.bfloat16, device=dev)
        idx_k[tok] = self.idx_k.reshape(-1, 128)
        k = torch.zeros((2, n_tok, 256), dtype=torch.bfloat16, device=dev)
        k[:, tok] = self.k_cache.permute(1, 0, 2, 3).reshape(2, -1, 256)
        v = torch.zeros((2, n_tok // R, 256, R), dtype=torch.bfloat16, device=dev)
        v[:, blk] = self.v_cache.permute(1, 0, 2, 3, 4).reshape(2, -1, 256, R)
        self.idx_k, self.k_cache, self.v_cache = idx_k, k, v
        self.block_keys = torch.zeros((n_tok // R, 128), dtype=torch.bfloat16, device=dev)

    def _pool(self, begin, end, span, stream=None):
        if self.transforms:
            qsa.pool_block_keys_normed(self.idx_k, self.block_keys, begin, end, span,
                                       gamma=self.gamma_k, eps=self.eps, inv_freq=self.inv_freq,
                                       pages=self.pages, stream=stream)
        else:
            qsa.pool_block_keys(self.idx_k, self.block_keys, begin, end, span, pages=self.pages,
                                stream=stream)

    # the three calls of a step ------------------------------------------
    def pool(self, stream=None):
        if self.pool_span > 0:
            self._pool(self.pool_begin, self.pool_end, self.pool_span, stream)

    def select(self, stream=None):
        b = self.b
        idx_q = b.idx_q
        if self.transforms:
            qsa.index_query_transform(b.idx_q, self.idx_q_t, b.cu_q, b.seq_len, self.max_q_len,
                                      gamma=self.gamma_q, eps=self.eps, inv_freq=self.inv_freq,
                                      stream=stream)
            idx_q = self.idx_q_t
        qsa.index_select(idx_q, b.w, b.cu_q, b.seq_len, self.max_q_len, self.max_blocks,
                         self.block_keys, self.budget, self.sel, self.sel_count, self.ws_index,
                         pages=self.pages, stream=stream)

    def attend(self, stream=None):
        b = self.b
        rope = dict(inv_freq=self.inv_freq, softmax_scale=self.softmax_scale, pages=self.pages,
                    stream=stream)
        if self.decode:
            qsa.attend_decode(b.q, b.seq_len, self.k_cache, self.v_cache, self.sel, self.sel_count,
                              self.budget, self.out, self.lse, self.ws_decode, **rope)
        elif self.mtp:
            qsa.attend_decode_multi(b.q, b.cu_q, b.seq_len, self.k_cache, self.v_cache, self.sel,
                                    self.sel_count, self.budget, self.out, self.lse, self.ws_decode,
                                    **rope)
        else:
            qsa.attend_prefill(b.q, b.cu_q, b.seq_len, self.max_q_len, self.k_cache, self.v_cache,
                               self.sel, self.sel_count, self.budget, self.out, self.lse, **rope)

    def step(self, stream=None):
        self.pool(stream)
        self.select(stream)
        self.attend(stream)

    # pipelined prefill ----------------------------------------------------
    def _rows(self, a: int, c: int) -> "QSARunner":
        """Query rows [a, c) of a one-sequence prefill chunk as a chunk of its
        own (the sequence then ends at position prefix + c - 1): the same
        caches and outputs (views)."""
        b = self.b
        L = b.seq_lens_host()[0]
        dev = b.idx_q.device
        v = copy.copy(self)
        v.b = QSABatch(seq_len=torch.tensor([L - self.n_q + c], dtype=torch.int32, device=dev),
                       cu_q=torch.tensor([0, c - a], dtype=torch.int32, device=dev),
                       idx_q=b.idx_q[a:c], w=b.w[a:c], idx_k=b.idx_k, q=b.q[a:c], k=b.k, v=b.v,
                       budget=b.budget, meta=dict(b.meta))
        v.n_q = v.max_q_len = c - a
        v.idx_q_t = self.idx_q_t[a:c] if self.idx_q_t is not None else None
        v.sel, v.sel_count = self.sel[a:c], self.sel_count[a:c]
        v.out, v.lse = self.out[a:c], self.lse[a:c]
        return v

    def step_pipelined(self, parts: int = 4):
        """One prefill step with the chunk's query rows in `parts` consecutive
        pieces: piece i's attention runs on a second stream while piece i+1
        is selected, so the memory-bound attention overlaps the MFMA-bound
        score GEMM (pieces as piece_bounds cuts them).  Same calls on the same
        rows, so the same results as step().  One-sequence prefill batches
        only."""
        assert not (self.decode or self.mtp) and self.n_seq == 1, "one-sequence prefill"
        key = ("pipe", parts)
        if getattr(self, "_pipe_key", None) != key:
            bounds = piece_bounds(self.n_q, parts)
            self._pipe_parts = [self._rows(a, c) for a, c in zip(bounds[:-1], bounds[1:]) if c > a]
            self._pipe_streams = (torch.cuda.Stream(), torch.cuda.Stream())
            self._pipe_key = key
        sa, sb = self._pipe_streams
        main = torch.cuda.current_stream()
        sa.wait_stream(main)
        sb.wait_stream(main)
        done = []
        with torch.cuda.stream(sa):
            self.pool()
            for u in self._pipe_parts:
                u.select()
                e = torch.cuda.Event()
                e.record(sa)
                done.append(e)
        with torch.cuda.stream(sb):
            for u, e in zip(self._pipe_parts, done):
                sb.wait_event(e)
                u.attend()
        main.wait_stream(sa)
        main.wait_stream(sb)

    # HIP graphs ----------------------------------------------------------
    def capture(self, parts=("pool", "select", "attend")) -> torch.cuda.CUDAGraph:
        """Record the listed calls of a step as one HIP graph (the library
        issues no allocations or memsets, so the calls capture as they are).
        Replaying it redoes those calls on the runner's buffers."""
        calls = [getattr(self, p) for p in parts]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in calls:
                c()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        return g
