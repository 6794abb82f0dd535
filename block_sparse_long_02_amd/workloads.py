"""Seeded synthetic inputs for the QSA layer (Qwen Sparse Attention).

Shapes and value structure follow the workloads named for the Qwen3.8-Flash-Next
QSA layer (page "Qwen3.8-Flash-Next ... 实验性预览权重发布", model-card
paragraph; page "ailearn ... 03 Attention", config table): 4 indexer query heads
over one shared indexer key of width 128, 24 query heads over 2 KV heads of
width 256, 4-token micro-blocks.

This module only draws random numbers and lays them out.  It holds no step of
the attention method (no pooling, scoring, selection, RoPE or softmax), so the
HIP path and the CPU oracle can both be fed from it.  Every draw comes from a
seeded ``torch.Generator``; CPU and GPU generators give different streams, so
a test always feeds one generated batch to both sides.

Structure of the draws:

* indexer q/k, core q/k/v: N(0,1) in fp32, rounded to bf16 by torch.
* head weights w: softmax of N(0,1) logits per query, fp32.
* prefill planting: queries are cut into segments; segment g has a random unit
  direction u_g, its indexer queries are N(0,1) + 8 u_g, and n_plant blocks
  completed before the segment starts get token keys sqrt(128) u_g + 0.1 N(0,1).
* decode planting: u = normalise(sum_h w_h q_h); n_plant blocks spread over the
  context get token keys sqrt(128) u + 0.1 N(0,1).
* near ties: 513 blocks with noise-free keys alpha sqrt(128) u, 512 at alpha=1
  and one at alpha=0.99 placed below some of the alpha=1 blocks.
* exact grid: indexer q/k snapped to round(8x)/8 clipped to [-4, 4] and w to
  positive multiples of 2^-8, so every indexer dot product is exact in fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

H_I, D_I = 4, 128          # indexer query heads, indexer head width
H_Q, H_KV, D = 24, 2, 256  # core query heads, KV heads, head width
R = 4                      # tokens per micro-block

_KV_CHUNK = 1 << 18        # tokens generated per step for large caches


@dataclass
class QSABatch:
    """One batch of QSA inputs (torch tensors, all on one device).

    Queries of sequence s are rows cu_q[s] .. cu_q[s+1]-1 and sit at the last
    positions of the sequence: row cu_q[s]+j has position
    seq_len[s] - (cu_q[s+1]-cu_q[s]) + j.
    """
    seq_len: torch.Tensor   # int32 [n_seq]
    cu_q: torch.Tensor      # int32 [n_seq+1]
    idx_q: torch.Tensor     # bf16 [n_q][4][128]
    w: torch.Tensor         # fp32 [n_q][4]
    idx_k: torch.Tensor     # bf16 [n_seq][L_cap][128]
    q: torch.Tensor         # bf16 [n_q][24][256]
    k: torch.Tensor         # bf16 [n_seq][2][L_cap][256], not rotated
    v: torch.Tensor         # bf16 [n_seq][2][L_cap][256]
    budget: int
    planted: list = field(default_factory=list)  # per segment / sequence: list of block ids
    meta: dict = field(default_factory=dict)

    @property
    def n_q(self) -> int:
        return int(self.idx_q.shape[0])

    @property
    def n_seq(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def l_cap(self) -> int:
        return int(self.idx_k.shape[1])

    def seq_lens_host(self) -> list[int]:
        return [int(x) for x in self.seq_len.cpu().tolist()]

    def cu_q_host(self) -> list[int]:
        return [int(x) for x in self.cu_q.cpu().tolist()]

    def q_pos_host(self) -> list[int]:
        """Absolute position of every query row."""
        lens, cu = self.seq_lens_host(), self.cu_q_host()
        pos = []
        for s in range(len(lens)):
            ql = cu[s + 1] - cu[s]
            pos.extend(range(lens[s] - ql, lens[s]))
        return pos

    def q_seq_host(self) -> list[int]:
        cu = self.cu_q_host()
        out = []
        for s in range(len(cu) - 1):
            out.extend([s] * (cu[s + 1] - cu[s]))
        return out

    def max_q_len(self) -> int:
        cu = self.cu_q_host()
        return max(cu[s + 1] - cu[s] for s in range(len(cu) - 1))

    def max_blocks(self) -> int:
        return max(self.seq_lens_host()) // R

    def to(self, device) -> "QSABatch":
        """Copy every tensor to `device` (same values)."""
        names = ["seq_len", "cu_q", "idx_q", "w", "idx_k", "q", "k", "v"]
        kw = {n: getattr(self, n).to(device) for n in names}
        return QSABatch(budget=self.budget, planted=self.planted, meta=dict(self.meta), **kw)


def _cap(n_tokens: int) -> int:
    """Cache capacity in tokens: whole micro-blocks, at least one."""
    return max(R, (n_tokens + R - 1) // R * R)


def _snap_grid(x: torch.Tensor) -> torch.Tensor:
    return torch.clamp(torch.round(x * 8.0) / 8.0, -4.0, 4.0)


def _head_weights(n: int, g: torch.Generator, device, exact_grid: bool) -> torch.Tensor:
    z = torch.randn((n, H_I), generator=g, device=device, dtype=torch.float32)
    w = torch.softmax(z.double(), dim=-1).float()
    if exact_grid:
        w = torch.clamp(torch.round(w * 256.0), min=1.0) / 256.0
    return w.contiguous()


def _fill_normal_bf16(out: torch.Tensor, n_valid: int, g: torch.Generator):
    """out: bf16 [L_cap][width]; rows < n_valid get N(0,1), the rest zero."""
    out.zero_()
    for t0 in range(0, n_valid, _KV_CHUNK):
        t1 = min(n_valid, t0 + _KV_CHUNK)
        out[t0:t1] = torch.randn((t1 - t0, out.shape[1]), generator=g,
                                 device=out.device, dtype=torch.float32).to(torch.bfloat16)


def _core_tensors(n_q, lens, l_cap, g, device):
    n_seq = len(lens)
    q = torch.randn((n_q, H_Q, D), generator=g, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    k = torch.empty((n_seq, H_KV, l_cap, D), dtype=torch.bfloat16, device=device)
    v = torch.empty((n_seq, H_KV, l_cap, D), dtype=torch.bfloat16, device=device)
    for s in range(n_seq):
        for h in range(H_KV):
            _fill_normal_bf16(k[s, h], lens[s], g)
            _fill_normal_bf16(v[s, h], lens[s], g)
    return q, k, v


def _plant_tokens(idx_k_f: torch.Tensor, blocks, direction: torch.Tensor, scale: float,
                  noise: float, g: torch.Generator):
    """Set the 4 token keys of each listed block to scale*direction + noise*N(0,1)."""
    if len(blocks) == 0:
        return
    dev = idx_k_f.device
    b = torch.as_tensor(sorted(blocks), dtype=torch.long, device=dev)
    tok = (b[:, None] * R + torch.arange(R, device=dev)[None, :]).reshape(-1)
    val = scale * direction.to(dev)[None, :].expand(tok.numel(), D_I)
    if noise:
        val = val + noise * torch.randn((tok.numel(), D_I), generator=g, device=dev,
                                        dtype=torch.float32)
    idx_k_f[tok] = val


def _unit(vec: torch.Tensor) -> torch.Tensor:
    v = vec.double()
    return (v / v.norm()).float()


def make_prefill(*, prefix: int, chunk: int, budget: int, seg: int, n_plant: int,
                 seed: int, device="cpu", distance: str = "uniform",
                 exact_grid: bool = False) -> QSABatch:
    """One sequence: `prefix` cached tokens, then a chunk of `chunk` query tokens."""
    device = torch.device(device)
    gh = torch.Generator(device="cpu")
    gh.manual_seed(seed)
    gd = torch.Generator(device=device)
    gd.manual_seed(seed + 7919)
    total = prefix + chunk
    l_cap = _cap(total)

    idx_k_f = torch.zeros((l_cap, D_I), dtype=torch.float32, device=device)
    for t0 in range(0, total, _KV_CHUNK):
        t1 = min(total, t0 + _KV_CHUNK)
        idx_k_f[t0:t1] = torch.randn((t1 - t0, D_I), generator=gd, device=device,
                                     dtype=torch.float32)
    idx_q_f = torch.randn((chunk, H_I, D_I), generator=gd, device=device, dtype=torch.float32)

    n_segments = (chunk + seg - 1) // seg
    used: set[int] = set()
    planted = []
    for sg in range(n_segments):
        u = _unit(torch.randn((D_I,), generator=gh, dtype=torch.float64))
        j0, j1 = sg * seg, min(chunk, (sg + 1) * seg)
        idx_q_f[j0:j1] += 8.0 * u.to(device)[None, None, :]
        first_pos = prefix + j0
        n_avail = (first_pos + 1) // R
        chosen = []
        if n_avail > 0 and n_plant > 0:
            if distance == "uniform":
                perm = torch.randperm(n_avail, generator=gh).tolist()
                for b in perm:
                    if b not in used:
                        chosen.append(b)
                        if len(chosen) == n_plant:
                            break
            else:  # log-uniform distance (in tokens) back from the segment start
                lo, hi = math.log(R), math.log(max(first_pos, R + 1))
                tries = 0
                while len(chosen) < n_plant and tries < 64 * n_plant:
                    tries += 1
                    d = math.exp(lo + (hi - lo) * float(torch.rand((), generator=gh)))
                    b = int((first_pos - d) // R)
                    if 0 <= b < n_avail and b not in used and b not in chosen:
                        chosen.append(b)
        used.update(chosen)
        planted.append(sorted(chosen))
        _plant_tokens(idx_k_f, chosen, u, math.sqrt(D_I), 0.1, gd)

    if exact_grid:
        idx_k_f = _snap_grid(idx_k_f)
        idx_q_f = _snap_grid(idx_q_f)
    idx_k_f[total:] = 0.0
    w = _head_weights(chunk, gd, device, exact_grid)
    q, k, v = _core_tensors(chunk, [total], l_cap, gd, device)
    return QSABatch(
        seq_len=torch.tensor([total], dtype=torch.int32, device=device),
        cu_q=torch.tensor([0, chunk], dtype=torch.int32, device=device),
        idx_q=idx_q_f.to(torch.bfloat16).contiguous(), w=w,
        idx_k=idx_k_f.to(torch.bfloat16)[None].contiguous(),
        q=q, k=k, v=v, budget=budget, planted=planted,
        meta=dict(kind="prefill", prefix=prefix, chunk=chunk, seg=seg, n_plant=n_plant,
                  seed=seed, distance=distance, exact_grid=exact_grid))


def make_decode(*, seq_lens, budget: int, n_plant: int, seed: int, device="cpu",
                near_tie=None, tie_count: int = 512, exact_grid: bool = False) -> QSABatch:
    """One query per sequence, at the last position of each sequence.

    near_tie: optional list of bools; a marked sequence gets `tie_count` blocks
    with identical noise-free keys sqrt(128) u plus one block at 0.99 sqrt(128) u
    placed below some of them, instead of the noisy planting.
    """
    device = torch.device(device)
    gh = torch.Generator(device="cpu")
    gh.manual_seed(seed)
    gd = torch.Generator(device=device)
    gd.manual_seed(seed + 7919)
    lens = [int(x) for x in seq_lens]
    n_seq = len(lens)
    l_cap = _cap(max(lens))
    near_tie = list(near_tie) if near_tie is not None else [False] * n_seq

    idx_q_f = torch.randn((n_seq, H_I, D_I), generator=gd, device=device, dtype=torch.float32)
    if exact_grid:
        idx_q_f = _snap_grid(idx_q_f)
    w = _head_weights(n_seq, gd, device, exact_grid)
    idx_q_bf = idx_q_f.to(torch.bfloat16)
    idx_k = torch.empty((n_seq, l_cap, D_I), dtype=torch.bfloat16, device=device)
    planted = []
    for s in range(n_seq):
        kf = torch.zeros((l_cap, D_I), dtype=torch.float32, device=device)
        for t0 in range(0, lens[s], _KV_CHUNK):
            t1 = min(lens[s], t0 + _KV_CHUNK)
            kf[t0:t1] = torch.randn((t1 - t0, D_I), generator=gd, device=device,
                                    dtype=torch.float32)
        u = _unit((w[s].double()[:, None] * idx_q_bf[s].double()).sum(0).cpu())
        n_c = lens[s] // R
        if near_tie[s] and n_c > 0:
            n_t = min(tie_count + 1, n_c)
            blocks = sorted(torch.randperm(n_c, generator=gh)[:n_t].tolist())
            low = int(torch.randint(0, max(1, n_t - 1), (), generator=gh))
            low_block = blocks[low]
            top = [b for b in blocks if b != low_block]
            _plant_tokens(kf, top, u, math.sqrt(D_I), 0.0, gd)
            _plant_tokens(kf, [low_block], u, 0.99 * math.sqrt(D_I), 0.0, gd)
            planted.append(sorted(top))
        else:
            n_p = min(n_plant, n_c)
            blocks = sorted(torch.randperm(n_c, generator=gh)[:n_p].tolist())
            _plant_tokens(kf, blocks, u, math.sqrt(D_I), 0.1, gd)
            planted.append(blocks)
        if exact_grid:
            kf = _snap_grid(kf)
        kf[lens[s]:] = 0.0
        idx_k[s] = kf.to(torch.bfloat16)
    q, k, v = _core_tensors(n_seq, lens, l_cap, gd, device)
    return QSABatch(
        seq_len=torch.tensor(lens, dtype=torch.int32, device=device),
        cu_q=torch.arange(n_seq + 1, dtype=torch.int32, device=device),
        idx_q=idx_q_bf.contiguous(), w=w, idx_k=idx_k.contiguous(), q=q, k=k, v=v,
        budget=budget, planted=planted,
        meta=dict(kind="decode", n_plant=n_plant, seed=seed, near_tie=near_tie,
                  exact_grid=exact_grid))


def make_mtp_decode(*, seq_lens, q_len: int, budget: int, n_plant: int, seed: int,
                    device="cpu", exact_grid: bool = False) -> QSABatch:
    """Multi-token decode: q_len query tokens per sequence at its last positions
    (a new token plus speculative ones).  The tokens of sequence s share a
    random unit direction u_s: their indexer queries are N(0,1) + 8 u_s, and
    n_plant blocks completed before the first of them get token keys
    sqrt(128) u_s + 0.1 N(0,1)."""
    device = torch.device(device)
    gh = torch.Generator(device="cpu")
    gh.manual_seed(seed)
    gd = torch.Generator(device=device)
    gd.manual_seed(seed + 7919)
    lens = [int(x) for x in seq_lens]
    assert all(L >= q_len for L in lens)
    n_seq = len(lens)
    n_q = n_seq * q_len
    l_cap = _cap(max(lens))
    idx_q_f = torch.randn((n_q, H_I, D_I), generator=gd, device=device, dtype=torch.float32)
    idx_k = torch.empty((n_seq, l_cap, D_I), dtype=torch.bfloat16, device=device)
    planted = []
    for s in range(n_seq):
        u = _unit(torch.randn((D_I,), generator=gh, dtype=torch.float64))
        idx_q_f[s * q_len:(s + 1) * q_len] += 8.0 * u.to(device)[None, None, :]
        kf = torch.zeros((l_cap, D_I), dtype=torch.float32, device=device)
        for t0 in range(0, lens[s], _KV_CHUNK):
            t1 = min(lens[s], t0 + _KV_CHUNK)
            kf[t0:t1] = torch.randn((t1 - t0, D_I), generator=gd, device=device,
                                    dtype=torch.float32)
        n_avail = (lens[s] - q_len + 1) // R
        n_p = min(n_plant, n_avail)
        blocks = sorted(torch.randperm(n_avail, generator=gh)[:n_p].tolist()) if n_avail else []
        _plant_tokens(kf, blocks, u, math.sqrt(D_I), 0.1, gd)
        planted.append(blocks)
        if exact_grid:
            kf = _snap_grid(kf)
        kf[lens[s]:] = 0.0
        idx_k[s] = kf.to(torch.bfloat16)
    if exact_grid:
        idx_q_f = _snap_grid(idx_q_f)
    w = _head_weights(n_q, gd, device, exact_grid)
    q, k, v = _core_tensors(n_q, lens, l_cap, gd, device)
    return QSABatch(
        seq_len=torch.tensor(lens, dtype=torch.int32, device=device),
        cu_q=torch.arange(0, n_q + 1, q_len, dtype=torch.int32, device=device),
        idx_q=idx_q_f.to(torch.bfloat16).contiguous(), w=w, idx_k=idx_k.contiguous(), q=q, k=k,
        v=v, budget=budget, planted=planted,
        meta=dict(kind="mtp_decode", q_len=q_len, n_plant=n_plant, seed=seed,
                  exact_grid=exact_grid))


def ragged_lengths(n_seq: int, lo: int, hi: int, seed: int) -> list[int]:
    """Lengths 4*floor(X/4) + d, X log-uniform in [lo, hi], d in {1,2,3}."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = []
    for _ in range(n_seq):
        x = math.exp(math.log(lo) + (math.log(hi) - math.log(lo)) * float(torch.rand((), generator=g)))
        d = 1 + int(torch.randint(0, 3, (), generator=g))
        out.append(R * int(x // R) + d)
    return out


# The five workloads, at full size.  Tests call the same builders at reduced
# sizes with the same structure.

def tiny_prefill(device="cpu", seed=1000, exact_grid=False, T=512):
    """Causal prefill, T=512, budget 16 blocks, 8 planted blocks per 64-query segment."""
    return make_prefill(prefix=0, chunk=T, budget=16, seg=64, n_plant=8, seed=seed,
                        device=device, exact_grid=exact_grid)


def prefill_8k(device="cpu", seed=1001, T=8192, exact_grid=False):
    """Causal prefill, T=8192 (or T<=2048 for the dense case), budget 512, 64 planted."""
    return make_prefill(prefix=0, chunk=T, budget=512, seg=1024, n_plant=64, seed=seed,
                        device=device, exact_grid=exact_grid)


def decode_128k(device="cpu", seed=1002, n_seq=32, ctx=131072, exact_grid=False):
    """Decode: n_seq sequences of ctx cached tokens plus the new one, 32 planted."""
    return make_decode(seq_lens=[ctx + 1] * n_seq, budget=512, n_plant=32, seed=seed,
                       device=device, exact_grid=exact_grid)


def chunked_prefill_1m(device="cpu", seed=1003, prefix=1015808, chunk=32768, exact_grid=False):
    """Chunked prefill: a 32768-token chunk on a 1,015,808-token cached prefix."""
    return make_prefill(prefix=prefix, chunk=chunk, budget=512, seg=1024, n_plant=64,
                        seed=seed, device=device, distance="loguniform", exact_grid=exact_grid)


def mtp_decode_128k(device="cpu", seed=1005, n_seq=32, ctx=131072, q_len=4, exact_grid=False):
    """Multi-token decode: n_seq sequences of ctx cached tokens plus q_len new ones
    (a new token and q_len - 1 speculative tokens), 32 planted blocks each."""
    return make_mtp_decode(seq_lens=[ctx + q_len] * n_seq, q_len=q_len, budget=512, n_plant=32,
                           seed=seed, device=device, exact_grid=exact_grid)


def ragged_decode(device="cpu", seed=1004, n_seq=8, lo=4096, hi=1048572, exact_grid=False):
    """Ragged decode: log-uniform lengths, partial tails, near ties in half the sequences."""
    lens = ragged_lengths(n_seq, lo, hi, seed)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 1)
    ties = [bool(x) for x in torch.randperm(n_seq, generator=g).lt(n_seq // 2).tolist()]
    return make_decode(seq_lens=lens, budget=512, n_plant=32, seed=seed, device=device,
                       near_tie=ties, exact_grid=exact_grid)


def v_cache_layout(v: torch.Tensor) -> torch.Tensor:
    """[n_seq][2][cap][256] token-major values -> [n_seq][2][cap/4][256][4]
    (micro-block-major, dim-major inside a block), the layout libqsa reads."""
    n_seq, h, cap, d = v.shape
    assert cap % R == 0
    return v.reshape(n_seq, h, cap // R, R, d).transpose(-1, -2).contiguous()
