"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Selections: bit-exact for exact-grid inputs and whenever the oracle's
boundary gap exceeds the float32 rounding allowance, otherwise within it.
Attention: max-abs 1e-2 and relative L2 5e-3 per query row (bf16 in/out,
float32 accumulation).  Pooling: bit-exact.  RoPE helper: within one bf16 ulp.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_long_02_amd import qsa
from block_sparse_long_02_amd import workloads as W
from block_sparse_long_02_amd.runner import QSARunner
from oracle import qsa_oracle as O
from tests._harness import OracleView, check_attention, check_selection, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()   # the native library must load


def _sync():
    torch.cuda.synchronize()


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


# ------------------------------------------------------------------ pooling

def test_pool_bit_exact_and_bounded():
    g = torch.Generator().manual_seed(0)
    n_seq, cap = 3, 1024
    idx_k = torch.randn(n_seq, cap, 128, generator=g).to(torch.bfloat16)
    idx_k[1, :8] = torch.tensor([16777216.0, 1.0, -16777216.0, 1.0] * 2).to(torch.bfloat16)[:, None]
    # token order and a pairwise tree round this block differently (0 against 0.25)
    idx_k[1, 8:12] = torch.tensor([1.0, 16777216.0, 1.0, -16777216.0]).to(torch.bfloat16)[:, None]
    begin, end = [0, 0, 100], [256, 77, 101]
    sentinel = torch.full((n_seq, cap // 4, 128), 0x1234, dtype=torch.int16)
    for max_span in (256, 16):            # 16: fewer workgroups than blocks
        bk = sentinel.clone().cuda().view(torch.bfloat16)
        qsa.pool_block_keys(idx_k.cuda(), bk, torch.tensor(begin, dtype=torch.int32).cuda(),
                            torch.tensor(end, dtype=torch.int32).cuda(), max_span)
        _sync()
        got = _bits(bk)
        for s in range(n_seq):
            ref = torch.tensor(O.pool_block_keys(np64(idx_k[s]), end[s]), dtype=torch.float32)
            ref_bits = ref.to(torch.bfloat16).view(torch.int16).numpy()
            assert np.array_equal(got[s, begin[s]:end[s]], ref_bits[begin[s]:end[s]]), (s, max_span)
            assert np.all(got[s, :begin[s]] == 0x1234) and np.all(got[s, end[s]:] == 0x1234)
    # the order-of-addition cases: 2^24 + 1 - 2^24 + 1 pools to 0.25, and
    # 1 + 2^24 + 1 - 2^24 to 0 (a pairwise tree would give 0.25)
    assert float(bk[1, 0, 0].float()) == 0.25
    assert float(bk[1, 2, 0].float()) == 0.0


# --------------------------------------------------------------------- RoPE

def _ordered(bits):
    """bf16 bit patterns (int16) -> integers in the order of the values (+0 == -0)."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b < 0, -mag, mag)


def _ulps(got_bf16, ref_f64):
    ref_bits = torch.tensor(ref_f64, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
    return np.abs(_ordered(_bits(got_bf16)) - _ordered(ref_bits))


def test_rope_helper_within_one_ulp():
    g = torch.Generator().manual_seed(1)
    n = 300
    x = torch.randn(n, 2, 256, generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 1 << 20, (n,), generator=g, dtype=torch.int32)
    pos[:4] = torch.tensor([0, 1, 4095, (1 << 20) - 1], dtype=torch.int32)
    xd = x.cuda().clone()
    qsa.rope_apply(xd, row_stride=512, head_stride=256, n_heads=2, n_rows=n, pos=pos.cuda())
    _sync()
    ref = O.rope(np64(x), pos.numpy().astype(np.float64)[:, None])
    assert np.array_equal(_bits(xd)[..., 64:], _bits(x)[..., 64:])     # untouched dims
    assert _ulps(xd, ref).max() <= 1
    # pos = NULL: consecutive positions from pos0
    xe = x.cuda().clone()
    qsa.rope_apply(xe, row_stride=512, head_stride=256, n_heads=2, n_rows=n, pos0=1000)
    _sync()
    ref2 = O.rope(np64(x), (1000 + np.arange(n, dtype=np.float64))[:, None])
    assert _ulps(xe, ref2).max() <= 1


def test_rope_helper_yarn_table_within_one_ulp():
    # the library's YaRN table against the oracle's (each from the YaRN paper)
    g = torch.Generator().manual_seed(2)
    n = 300
    x = torch.randn(n, 2, 256, generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 1 << 20, (n,), generator=g, dtype=torch.int32)
    pos[:3] = torch.tensor([0, 262143, (1 << 20) - 1], dtype=torch.int32)
    f, _ = qsa.yarn_rope()
    xd = x.cuda().clone()
    qsa.rope_apply(xd, row_stride=512, head_stride=256, n_heads=2, n_rows=n, pos=pos.cuda(),
                   inv_freq=f)
    _sync()
    ref = O.rope(np64(x), pos.numpy().astype(np.float64)[:, None], inv_freq=O.yarn_inv_freq())
    assert np.array_equal(_bits(xd)[..., 64:], _bits(x)[..., 64:])
    assert _ulps(xd, ref).max() <= 1
    # the table is used: it differs from the native rotation at long positions
    xn = x.cuda().clone()
    qsa.rope_apply(xn, row_stride=512, head_stride=256, n_heads=2, n_rows=n, pos=pos.cuda())
    _sync()
    assert not np.array_equal(_bits(xn), _bits(xd))


# ----------------------------------------------- attention on oracle choices

def _load_oracle_selection(r, view, rows):
    sel = torch.full((r.n_q, r.budget), -1, dtype=torch.int32)
    cnt = torch.zeros((r.n_q,), dtype=torch.int32)
    chosen = {}
    for row in range(r.n_q):
        ids = view.select(row)
        sel[row, :len(ids)] = torch.as_tensor(ids, dtype=torch.int32)
        cnt[row] = len(ids)
        chosen[row] = ids
    r.sel.copy_(sel.cuda())
    r.sel_count.copy_(cnt.cuda())
    return chosen


def test_attend_prefill_on_oracle_selection_tiny():
    b = W.tiny_prefill(T=512)
    view = OracleView(b)
    r = QSARunner(b.to("cuda"))
    chosen = _load_oracle_selection(r, view, range(b.n_q))
    r.attend()
    _sync()
    worst = 0.0
    for row in range(b.n_q):
        # the attention's stated input is the stored (bf16, rotated) K cache
        e, rel, _ = check_attention(r.out[row], r.lse[row],
                                    view.attend(row, chosen[row], k_stored=True), f"row {row}")
        worst = max(worst, rel)
    print(f"tiny prefill attention: worst rel-L2 {worst:.2e}")


def test_attend_decode_on_oracle_selection():
    b = W.make_decode(seq_lens=[2051, 9003, 40002, 16384, 5], budget=512, n_plant=32, seed=11)
    view = OracleView(b)
    r = QSARunner(b.to("cuda"))
    chosen = _load_oracle_selection(r, view, range(b.n_q))
    r.attend()
    _sync()
    for row in range(b.n_q):
        check_attention(r.out[row], r.lse[row], view.attend(row, chosen[row], k_stored=True),
                        f"decode row {row}")
    # calls of different sizes on one workspace: the first 2 sequences, then
    # all 5 again
    out_all = r.out.clone()
    qsa.attend_decode(r.b.q[:2], r.b.seq_len[:2], r.k_cache, r.v_cache, r.sel[:2],
                      r.sel_count[:2], r.budget, r.out[:2], r.lse[:2], r.ws_decode)
    r.attend()
    _sync()
    assert torch.equal(r.out, out_all)
    # split-K decode equals the prefill kernel on the same choices up to the
    # order of the float32 sums: one bf16 ulp of the output's magnitude at
    # most, plus float32 rounding near zero
    out_d, lse_d = r.out.clone(), r.lse.clone()
    qsa.attend_prefill(r.b.q, r.b.cu_q, r.b.seq_len, 1, r.k_cache, r.v_cache, r.sel, r.sel_count,
                       r.budget, r.out, r.lse)
    _sync()
    x, y = r.out.float(), out_d.float()
    assert ((x - y).abs() <= torch.maximum(x.abs(), y.abs()) * 2.0 ** -7 + 1e-5).all()
    assert (r.lse - lse_d).abs().max().item() <= 1e-4


# ------------------------------------------------------------- selection

def _select_and_check(b, exact=False, rows=None):
    view = OracleView(b)
    r = QSARunner(b.to("cuda"))
    r.pool()
    r.select()
    _sync()
    sel, cnt = r.sel.cpu().numpy(), r.sel_count.cpu().numpy()
    rows = range(b.n_q) if rows is None else rows
    kinds = {"exact": 0, "near": 0}
    for row in rows:
        kinds[check_selection(view, row, sel[row], int(cnt[row]), exact=exact)] += 1
    return r, view, kinds


def test_index_select_tiny_prefill():
    _, _, kinds = _select_and_check(W.tiny_prefill(T=512))
    print("tiny prefill selection:", kinds)


def test_index_select_exact_grid_prefill():
    b = W.make_prefill(prefix=0, chunk=3001, budget=100, seg=256, n_plant=16, seed=21,
                       exact_grid=True)
    _select_and_check(b, exact=True)


def test_index_select_exact_grid_sampled_path():
    # more than 4096 candidates per row: sample, threshold, filter, select
    b = W.make_prefill(prefix=40000, chunk=77, budget=512, seg=32, n_plant=32, seed=22,
                       exact_grid=True)
    _select_and_check(b, exact=True)


def test_index_select_exact_grid_mid_rows():
    # rows from 3,750 to 6,250 candidates: a tile that mixes rows keeping
    # every candidate with filtered rows, and filtered rows where a fifth to
    # a third of the blocks pass the pre-filter (pending lists drain often)
    b = W.make_prefill(prefix=15000, chunk=10000, budget=512, seg=64, n_plant=32, seed=27,
                       exact_grid=True)
    rows = sorted(set(range(0, 10000, 53)) | set(range(1340, 1420)) | set(range(9968, 10000)))
    _select_and_check(b, exact=True, rows=rows)


def test_index_select_exact_grid_decode():
    b = W.make_decode(seq_lens=[20001, 37002, 70003, 5000, 3], budget=512, n_plant=32, seed=23,
                      exact_grid=True)
    _select_and_check(b, exact=True)


def test_index_select_exact_grid_decode_long_rows():
    # n_c = 32768 (one compaction pass), 35000 and 65536 (passes of 32,768
    # scores, threshold from samples in global memory), and a 1M-token row
    # (262,143 blocks, near ties) beside a short one and one with no candidate
    b = W.make_decode(seq_lens=[131075], budget=512, n_plant=32, seed=29, exact_grid=True)
    _select_and_check(b, exact=True)
    b = W.make_decode(seq_lens=[140001, 262147], budget=512, n_plant=32, seed=29, exact_grid=True)
    _select_and_check(b, exact=True)
    b = W.make_decode(seq_lens=[1048575, 9001, 3], budget=512, n_plant=32, seed=30,
                      exact_grid=True, near_tie=[True, False, False])
    _select_and_check(b, exact=True)


def test_index_select_exact_grid_decode_many_sequences():
    # more than 64 sequences: the dense score pass keeps 1024-column chunks
    # without counting the launch's chunks (up to 64 sequences choose the
    # chunk size from their lengths: 256 columns in the smaller decode tests
    # and the ragged batch, 1024 in the full-size 32 x 128K batches)
    g = np.random.default_rng(95)
    lens = [int(x) for x in g.integers(3, 6000, size=70)]
    b = W.make_decode(seq_lens=lens, budget=512, n_plant=16, seed=95, exact_grid=True)
    r, _, _ = _select_and_check(b, exact=True)
    # the same batch over 256-token pages in a random order: same selections
    rp = QSARunner(r.b, paged=256, page_seed=5)
    rp.pool()
    rp.select()
    _sync()
    assert torch.equal(rp.sel_count, r.sel_count) and torch.equal(rp.sel, r.sel)


def test_index_select_exact_grid_multi_token_tiles():
    # 4 and 3 query rows per sequence (multi-token decode shapes): dense scores
    for prefix, chunk in ((150000, 4), (20001, 3), (9, 4)):
        b = W.make_prefill(prefix=prefix, chunk=chunk, budget=512, seg=4, n_plant=32,
                           seed=30 + chunk, exact_grid=True)
        assert b.max_q_len() <= 4
        _select_and_check(b, exact=True)


def test_index_select_long_row_fallbacks():
    # all ties on a long row: the list overflows, the ordered select over
    # global scores keeps the lowest 512 ids
    b = W.make_decode(seq_lens=[200003], budget=512, n_plant=0, seed=31)
    b.idx_k[:] = b.idx_k[0, 0].clone()
    r, _, _ = _select_and_check(b, exact=True)
    assert np.array_equal(r.sel.cpu().numpy()[0], np.arange(512))
    # only sampled blocks (every 16th, below 8192) score high: the list is short
    b = W.make_decode(seq_lens=[160001], budget=512, n_plant=0, seed=32)
    u = b.idx_q[0].float().sum(0)
    u = u / u.norm()
    for blk in range(0, 8192, 16):
        b.idx_k[0, 4 * blk:4 * blk + 4] = (math.sqrt(128) * (1 + blk / 1e4) * u).to(torch.bfloat16)
    r, _, _ = _select_and_check(b, exact=True)
    assert np.array_equal(r.sel.cpu().numpy()[0], np.arange(0, 8192, 16))


def test_index_select_split_row_fallbacks():
    # rows above 65,536 blocks are compacted in pieces of 32,768 scores.
    # All ties: every piece overflows its segment, and the ordered select
    # over the row's scores keeps the lowest 512 ids; beside it a short row
    # of the same launch takes the unsplit path
    b = W.make_decode(seq_lens=[300003, 5001], budget=512, n_plant=0, seed=33)
    b.idx_k[0] = b.idx_k[0, 0].clone()
    r, _, _ = _select_and_check(b, exact=True)
    assert np.array_equal(r.sel.cpu().numpy()[0], np.arange(512))
    # only sampled blocks below 8192 score high: piece 0 lists 80 of them,
    # the others none, so the list is short of K and the row falls back
    b = W.make_decode(seq_lens=[300001], budget=512, n_plant=0, seed=34)
    u = b.idx_q[0].float().sum(0)
    u = u / u.norm()
    for blk in range(0, 8192, 16):
        b.idx_k[0, 4 * blk:4 * blk + 4] = (math.sqrt(128) * (1 + blk / 1e4) * u).to(torch.bfloat16)
    r, _, _ = _select_and_check(b, exact=True)
    assert np.array_equal(r.sel.cpu().numpy()[0], np.arange(0, 8192, 16))
    # high scores in all three pieces, one piece holding most: the
    # segments concatenate in block order
    b = W.make_decode(seq_lens=[300005], budget=512, n_plant=0, seed=35)
    u = b.idx_q[0].float().sum(0)
    u = u / u.norm()
    hot = sorted(set(list(range(40000, 40000 + 400)) + list(range(1000, 60000, 600)) +
                     list(range(70000, 75000, 500))))
    for blk in hot:
        b.idx_k[0, 4 * blk:4 * blk + 4] = (math.sqrt(128) * (1 + blk / 1e5) * u).to(torch.bfloat16)
    r, _, _ = _select_and_check(b, exact=True)
    assert set(hot) <= set(r.sel.cpu().numpy()[0].tolist())


def test_index_select_decode_rule():
    b = W.make_decode(seq_lens=[131073, 20001, 4100, 99999], budget=512, n_plant=32, seed=24)
    _, _, kinds = _select_and_check(b)
    print("decode selection:", kinds)


def test_index_select_near_ties():
    b = W.make_decode(seq_lens=[9001, 30002, 70003, 4099], budget=512, n_plant=32, seed=25,
                      near_tie=[True, True, False, True])
    r, view, _ = _select_and_check(b)
    sel = r.sel.cpu().numpy()
    for s in (0, 1, 3):
        assert set(b.planted[s]) == set(sel[s].tolist())   # the 512 tied blocks, not the 0.99 one


def test_index_select_budget_sweep_and_tiny_rows():
    for budget in (1, 7, 64, 511, 512):
        b = W.make_prefill(prefix=0, chunk=700, budget=budget, seg=64, n_plant=8, seed=26 + budget,
                           exact_grid=True)
        _select_and_check(b, exact=True)


def test_index_select_fallback_all_ties():
    # identical block keys: every score ties, the list overflows, the exact
    # fallback must keep the lowest 512 block ids
    b = W.make_decode(seq_lens=[40001, 20002], budget=512, n_plant=0, seed=27)
    b.idx_k[:] = b.idx_k[0, 0].clone()
    r, view, _ = _select_and_check(b, exact=True)
    sel = r.sel.cpu().numpy()
    assert np.array_equal(sel[0], np.arange(512)) and np.array_equal(sel[1], np.arange(512))


def test_index_select_fallback_short_list():
    # only the sampled blocks (every 16th) score high, so the threshold lets
    # through fewer than K entries and the exact fallback must take over
    b = W.make_decode(seq_lens=[4 * 8192 + 1], budget=512, n_plant=0, seed=28)
    u = b.idx_q[0].float().sum(0)
    u = u / u.norm()
    for blk in range(0, 8192, 16):
        b.idx_k[0, 4 * blk:4 * blk + 4] = (math.sqrt(128) * (1 + blk / 1e4) * u).to(torch.bfloat16)
    r, view, _ = _select_and_check(b, exact=True)
    assert np.array_equal(r.sel.cpu().numpy()[0], np.arange(0, 8192, 16))


def test_index_select_prefill_fallback_all_ties():
    # the prefill path (more than 4 rows per sequence, more than 4096
    # candidates): identical block keys make every score tie, the filtered
    # list overflows, and the exact fallback that recomputes the scores must
    # keep the lowest 512 block ids of every row
    b = W.make_prefill(prefix=20000, chunk=40, budget=512, seg=64, n_plant=0, seed=33,
                       exact_grid=True)
    b.idx_k[:] = b.idx_k[0, 0].clone()
    r, _, _ = _select_and_check(b, exact=True)
    sel = r.sel.cpu().numpy()
    assert all(np.array_equal(sel[row], np.arange(512)) for row in range(b.n_q))


def test_index_select_prefill_list_ties_at_threshold():
    # the prefill path with rows that keep every candidate (about 2,000 each,
    # under the 4,096-entry list): every 7th block scores one value and all
    # the others tie at a lower one, so the exact select takes the high
    # blocks and then, among the ties at the threshold, the lowest block ids
    # (equal scores keep the lower index).  Exact-grid keys 2u and u/2 with
    # u = sign(sum of the queries).
    b = W.make_prefill(prefix=8000, chunk=40, budget=512, seg=64, n_plant=0, seed=35,
                       exact_grid=True)
    u = torch.sign(b.idx_q.float().sum((0, 1)))
    n_c = 8000 // 4
    for blk in range(n_c + 10):
        b.idx_k[0, 4 * blk:4 * blk + 4] = ((2.0 if blk % 7 == 0 else 0.5) * u).to(torch.bfloat16)
    r, view, _ = _select_and_check(b, exact=True)
    sel = r.sel.cpu().numpy()
    for row in range(b.n_q):
        nc = (8000 + row + 1) // 4
        high = [x for x in range(nc) if x % 7 == 0]
        low = [x for x in range(nc) if x % 7 != 0][:512 - len(high)]
        sc = view.scores(row)
        if sc[0] > sc[1]:   # the high class really scores higher for this row
            assert sel[row].tolist() == sorted(high + low), row
    # every score equal: the lowest 512 ids
    b.idx_k[:] = (0.5 * u).to(torch.bfloat16)
    r, _, _ = _select_and_check(b, exact=True)
    sel = r.sel.cpu().numpy()
    assert all(np.array_equal(sel[row], np.arange(512)) for row in range(b.n_q))


def test_index_select_prefill_fallback_short_list():
    # the prefill path: only the blocks the sample pass scores (every 32nd)
    # score high, so the sampled threshold lets fewer than K blocks through
    # and the exact fallback takes over.  Exact-grid inputs: the fallback's
    # float32 dot products (dims in order) then equal the oracle's scores,
    # and the rest of the selection is decided among the low blocks
    b = W.make_prefill(prefix=20000, chunk=40, budget=512, seg=64, n_plant=0, seed=34,
                       exact_grid=True)
    u = torch.sign(b.idx_q.float().sum((0, 1)))
    n_c = 20000 // 4
    for blk in range(0, n_c, 32):
        b.idx_k[0, 4 * blk:4 * blk + 4] = (2.0 * u).to(torch.bfloat16)
    r, _, _ = _select_and_check(b, exact=True)
    sel = r.sel.cpu().numpy()
    high = set(range(0, n_c, 32))
    assert all(high <= set(sel[row].tolist()) for row in range(b.n_q))


# ------------------------------------------------- indexer transforms (pages)

def _rand_bf16(g, shape):
    # N(0,1) rows, each scaled by 10^u, u uniform in [-3, 3]
    x = torch.randn(*shape, generator=g, dtype=torch.float64)
    sc = 10.0 ** (torch.rand(*shape[:-1], 1, generator=g, dtype=torch.float64) * 6 - 3)
    return (x * sc).to(torch.bfloat16)


_FREQ_1E4 = [1.0e4 ** (-j / 32.0) for j in range(32)]    # a caller-given frequency table


def _transform_cases(g):
    gamma = (torch.rand(128, generator=g) + 0.5).float()
    return [(None, None), (gamma, None), (None, _FREQ_1E4), (gamma, _FREQ_1E4)]


def test_index_key_transform_bit_exact():
    g = torch.Generator().manual_seed(60)
    cap = 1 << 20
    # sequence 0: blocks 0..516 (block 10 all zero); sequence 1: the last
    # 1,144 blocks of a 1M-token cache (positions up to 1,048,572)
    ranges = [(0, 517), (261000, 262144)]
    idx_k = torch.zeros(2, cap, 128, dtype=torch.bfloat16)
    for s, (b0, b1) in enumerate(ranges):
        idx_k[s, 4 * b0:4 * b1] = _rand_bf16(g, (4 * (b1 - b0), 128))
    idx_k[0, 40:44] = 0
    ik = idx_k.cuda()
    begin = torch.tensor([r[0] for r in ranges], dtype=torch.int32).cuda()
    end = torch.tensor([r[1] for r in ranges], dtype=torch.int32).cuda()
    sentinel = torch.full((2, cap // 4, 128), 0x1234, dtype=torch.int16).cuda()
    for ci, (gamma, freq) in enumerate(_transform_cases(g)):
        for max_span in (1144, 16):
            bk = sentinel.clone().view(torch.bfloat16)
            print(f"key transform case {ci} max_span {max_span}", flush=True)
            qsa.pool_block_keys_normed(ik, bk, begin, end, max_span,
                                       gamma=None if gamma is None else gamma.cuda(),
                                       eps=1e-6, inv_freq=freq)
            _sync()
            got = _bits(bk)
            for s, (b0, b1) in enumerate(ranges):
                ref = O.transform_block_keys(np64(idx_k[s, 4 * b0:4 * b1]), b1 - b0,
                                             None if gamma is None else gamma.double().numpy(),
                                             1e-6, freq, first_block=b0)
                ref_bits = torch.tensor(ref, dtype=torch.float32).to(torch.bfloat16)
                ref_bits = ref_bits.view(torch.int16).numpy()
                assert np.array_equal(got[s, b0:b1], ref_bits), (ci, s, max_span)
                assert np.all(got[s, :b0] == 0x1234) and np.all(got[s, b1:] == 0x1234)
            assert np.all(got[0, 10] & 0x7FFF == 0)   # the all-zero block stays (+-)0


def test_index_query_transform_bit_exact():
    g = torch.Generator().manual_seed(61)
    lens, nq = [1 << 20, 5000, 37, 3], [40, 7, 37, 5]   # the last: 2 rows before position 0
    cu = np.concatenate([[0], np.cumsum(nq)]).tolist()
    n_rows = cu[-1] + 6                                 # 6 rows no sequence covers
    q_raw = _rand_bf16(g, (n_rows, 4, 128))
    q_raw[3] = 0
    cu_q = torch.tensor(cu, dtype=torch.int32).cuda()
    seq_len = torch.tensor(lens, dtype=torch.int32).cuda()
    pos = np.concatenate([np.arange(L - n, L) for L, n in zip(lens, nq)])
    valid = pos >= 0
    for ci, (gamma, freq) in enumerate(_transform_cases(g)):
        print(f"query transform case {ci}", flush=True)
        gd = None if gamma is None else gamma.cuda()
        out = torch.full((n_rows, 4, 128), 0x1234, dtype=torch.int16).cuda().view(torch.bfloat16)
        qsa.index_query_transform(q_raw.cuda(), out, cu_q, seq_len, max(nq), gamma=gd, eps=1e-6,
                                  inv_freq=freq)
        inplace = q_raw.cuda()
        qsa.index_query_transform(inplace, inplace, cu_q, seq_len, max(nq), gamma=gd, eps=1e-6,
                                  inv_freq=freq)
        _sync()
        got = _bits(out)
        ref = O.transform_queries(np64(q_raw[:cu[-1]][valid]), pos[valid],
                                  None if gamma is None else gamma.double().numpy(), 1e-6, freq)
        ref_bits = torch.tensor(ref, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
        assert np.array_equal(got[:cu[-1]][valid], ref_bits.numpy()), ci
        assert np.all(got[:cu[-1]][~valid] == 0x1234) and np.all(got[cu[-1]:] == 0x1234)
        assert np.array_equal(_bits(inplace)[:cu[-1]][valid], got[:cu[-1]][valid])
        assert np.all(got[3] & 0x7FFF == 0)


def test_index_select_with_transforms():
    # the select on the pages' transformed keys and queries, both methods:
    # the sampled prefill path (n_c > 4096) and the dense decode path
    g = torch.Generator().manual_seed(62)
    gk, gq = (torch.rand(128, generator=g) + 0.5).float(), (torch.rand(128, generator=g) + 0.5).float()
    batches = [W.make_prefill(prefix=40000, chunk=77, budget=512, seg=32, n_plant=32, seed=63),
               W.make_decode(seq_lens=[20001, 131073, 70003, 5], budget=512, n_plant=32, seed=64),
               W.tiny_prefill(T=512)]
    for bi, b in enumerate(batches):
        print(f"transformed select batch {bi}", flush=True)
        view = OracleView(b, transforms=True, gamma_k=gk.double().numpy(),
                          gamma_q=gq.double().numpy())
        r = QSARunner(b.to("cuda"), transforms=True, gamma_k=gk.cuda(), gamma_q=gq.cuda())
        r.pool()
        r.select()
        _sync()
        for s in range(b.n_seq):                 # the keys the select saw, bit-exact
            n = view.lens[s] // 4
            ref = torch.tensor(view.kbar(s), dtype=torch.float32).to(torch.bfloat16)
            assert torch.equal(r.block_keys[s, :n].cpu().view(torch.int16), ref.view(torch.int16))
        sel, cnt = r.sel.cpu().numpy(), r.sel_count.cpu().numpy()
        kinds = {"exact": 0, "near": 0}
        for row in range(b.n_q):
            kinds[check_selection(view, row, sel[row], int(cnt[row]))] += 1
        print("transformed select:", bi, kinds)


# ------------------------------------------------------------- end to end

def _end_to_end(b, rows, dense=False, yarn=False, transforms=False):
    view = OracleView(b, yarn=yarn, transforms=transforms)
    r = QSARunner(b if b.idx_q.is_cuda else b.to("cuda"), yarn=yarn, transforms=transforms)
    r.step()
    _sync()
    sel, cnt = r.sel.cpu().numpy(), r.sel_count.cpu().numpy()
    kinds = {"exact": 0, "near": 0, "rows_over_1e-2": 0}
    worst = 0.0
    for row in rows:
        kinds[check_selection(view, row, sel[row], int(cnt[row]))] += 1
        ref = view.dense(row) if dense else view.attend(row, sel[row][:cnt[row]])
        _, rel, n_over = check_attention(r.out[row], r.lse[row], ref, f"row {row}")
        kinds["rows_over_1e-2"] += n_over > 0
        worst = max(worst, rel)
    return kinds, worst


def test_end_to_end_tiny_prefill():
    b = W.tiny_prefill(T=512)
    kinds, worst = _end_to_end(b, range(b.n_q))
    print("tiny prefill:", kinds, f"worst rel-L2 {worst:.2e}")


def test_end_to_end_dense_equivalence():
    # T <= 2048 with budget 512: every row keeps every completed block, so the
    # output is plain causal GQA attention over 0..i
    b = W.prefill_8k(T=2048)
    rows = [0, 1, 2, 3, 4, 5, 63, 64, 1000, 2045, 2046, 2047]
    kinds, worst = _end_to_end(b, rows[:6], dense=True)   # naive loops: keep short rows
    kinds, worst = _end_to_end(b, rows)
    print("dense case:", kinds, f"worst rel-L2 {worst:.2e}")


def test_end_to_end_prefill_8k_sampled():
    b = W.prefill_8k(T=8192)
    rng = np.random.default_rng(3)
    rows = sorted(set(rng.choice(8192, 40, replace=False).tolist()) | {2047, 2048, 2051, 8190, 8191})
    kinds, worst = _end_to_end(b, rows)
    print("prefill 8k:", kinds, f"worst rel-L2 {worst:.2e}")


def test_prefill_attention_rows_of_one_workgroup_are_independent():
    # the prefill attention runs one row per wave, 4 rows of one KV head per
    # workgroup: a row whose selection is unusable (count < 0) gets NaN and
    # the rows beside it in its workgroup come out bit for bit as before; a
    # chunk of 510 rows leaves the last workgroup half empty
    b = W.tiny_prefill(T=510)
    r = QSARunner(b.to("cuda"))
    r.step()
    _sync()
    ref_out, ref_lse = r.out.clone(), r.lse.clone()
    cnt = r.sel_count.clone()
    bad = 201                      # the second row of the workgroup of rows 200..203
    r.sel_count[bad] = -1
    r.attend()
    _sync()
    assert torch.isnan(r.out[bad].float()).all() and torch.isnan(r.lse[bad]).all()
    keep = torch.ones(b.n_q, dtype=torch.bool, device="cuda")
    keep[bad] = False
    assert torch.equal(ref_out[keep].view(torch.int16), r.out[keep].view(torch.int16))
    assert torch.equal(ref_lse[keep].view(torch.int32), r.lse[keep].view(torch.int32))
    r.sel_count.copy_(cnt)
    r.attend()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b), [0, 200, 201, 202, 203, 507, 508, 509])
    print("rows of one workgroup:", kinds, f"worst rel-L2 {worst:.2e}", flush=True)


def test_end_to_end_decode_reduced():
    b = W.decode_128k(n_seq=6, ctx=32768)
    kinds, worst = _end_to_end(b, range(6))
    print("decode:", kinds, f"worst rel-L2 {worst:.2e}")


def test_end_to_end_ragged_decode_reduced():
    b = W.ragged_decode(n_seq=6, lo=4096, hi=200000)
    kinds, worst = _end_to_end(b, range(6))
    print("ragged decode:", kinds, f"worst rel-L2 {worst:.2e}")


def test_end_to_end_yarn_decode_and_prefill():
    # YaRN-extended rotations (K cache, queries) and softmax scale, checked
    # against the oracle's own YaRN table and scale; positions past the
    # native 262,144 tokens included
    b = W.make_decode(seq_lens=[270001, 131075, 5000], budget=512, n_plant=32, seed=66)
    kinds, worst = _end_to_end(b, range(3), yarn=True)
    print("yarn decode:", kinds, f"worst rel-L2 {worst:.2e}")
    b = W.prefill_8k(T=2048)
    kinds, worst = _end_to_end(b, [0, 5, 1000, 2047], dense=False, yarn=True)
    print("yarn prefill:", kinds, f"worst rel-L2 {worst:.2e}")


def test_end_to_end_yarn_with_indexer_transforms():
    # the whole path with the pages' indexer transforms and YaRN together
    b = W.make_decode(seq_lens=[300001, 70003], budget=512, n_plant=32, seed=65)
    kinds, worst = _end_to_end(b, range(2), yarn=True, transforms=True)
    print("yarn + transforms decode:", kinds, f"worst rel-L2 {worst:.2e}")
    b = W.tiny_prefill(T=512)
    kinds, worst = _end_to_end(b, range(0, 512, 7), yarn=True, transforms=True)
    print("yarn + transforms tiny prefill:", kinds, f"worst rel-L2 {worst:.2e}")


# ------------------------------------------------------------ paged caches

def _same_results(a, b):
    """Two runners of one batch gave the same selections and outputs, bit for bit."""
    assert torch.equal(a.sel_count, b.sel_count) and torch.equal(a.sel, b.sel)
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(a.lse.view(torch.int32), b.lse.view(torch.int32))


def _check_rows(r, view, rows):
    sel, cnt = r.sel.cpu().numpy(), r.sel_count.cpu().numpy()
    kinds, worst = {"exact": 0, "near": 0, "rows_over_1e-2": 0}, 0.0
    for row in rows:
        kinds[check_selection(view, row, sel[row], int(cnt[row]))] += 1
        _, rel, n_over = check_attention(r.out[row], r.lse[row],
                                         view.attend(row, sel[row][:cnt[row]]), f"row {row}")
        kinds["rows_over_1e-2"] += n_over > 0
        worst = max(worst, rel)
    return kinds, worst


def test_paged_prefill_unaligned_chunk_start():
    # a chunk that starts inside a micro-block (prefix 40001 = 4*10000 + 1) and
    # more than 4096 candidates per row (sampled path); pages of 256 and 1024
    # tokens in a random physical order against the contiguous caches
    b = W.make_prefill(prefix=40001, chunk=333, budget=512, seg=64, n_plant=32, seed=70).to("cuda")
    r0 = QSARunner(b)
    r0.step()
    for P in (256, 1024):
        print(f"paged prefill, {P}-token pages", flush=True)
        r1 = QSARunner(b, paged=P, page_seed=P)
        r1.step()
        _sync()
        _same_results(r0, r1)
    view = OracleView(b)
    kinds, worst = _check_rows(r1, view, list(range(0, 333, 11)) + [332])
    print("paged prefill:", kinds, f"worst rel-L2 {worst:.2e}")


def test_pipelined_prefill_matches_sequential():
    # the step with the chunk's rows in pieces, each piece's attention on a
    # second stream while the next piece is selected, gives the sequential
    # step's results bit for bit (plain; and with the indexer transforms, YaRN
    # and paged caches, where every piece also transforms its own queries)
    b = W.make_prefill(prefix=40001, chunk=333, budget=512, seg=64, n_plant=32, seed=71).to("cuda")
    r0 = QSARunner(b)
    r0.step()
    for parts in (2, 3, 7):
        print(f"pipelined prefill, {parts} pieces", flush=True)
        r1 = QSARunner(b)
        r1.step_pipelined(parts)
        _sync()
        _same_results(r0, r1)
    cfg = dict(transforms=True, yarn=True, paged=256, page_seed=5)
    r2 = QSARunner(b, **cfg)
    r2.step()
    r3 = QSARunner(b, **cfg)
    r3.step_pipelined(4)
    _sync()
    _same_results(r2, r3)


def test_paged_decode_shared_prefix():
    # sequence 1 starts with sequence 0's first 16,384 tokens and maps them to
    # the same 64 physical pages (a prefix-cache hit); ragged lengths
    b = W.make_decode(seq_lens=[70001, 70005, 20003, 3], budget=512, n_plant=32, seed=71)
    n = 16384
    for t in (b.idx_k, b.k, b.v):
        t[1, ..., :n, :] = t[0, ..., :n, :]
    b = b.to("cuda")
    r0 = QSARunner(b)
    r0.step()
    r1 = QSARunner(b, paged=256, page_seed=3, shared_pages={1: (0, n // 256)})
    assert torch.equal(r1.block_table[1, :64], r1.block_table[0, :64])
    r1.step()
    _sync()
    _same_results(r0, r1)
    kinds, worst = _check_rows(r1, OracleView(b), range(4))
    print("paged decode, shared prefix:", kinds, f"worst rel-L2 {worst:.2e}")


def test_paged_mtp_with_transforms_and_yarn():
    # multi-token decode over paged caches with the indexer transforms and YaRN
    b = W.make_mtp_decode(seq_lens=[4 * 20000 + 2, 300005], q_len=4, budget=512, n_plant=32,
                          seed=72).to("cuda")
    r0 = QSARunner(b, transforms=True, yarn=True)
    r0.step()
    r1 = QSARunner(b, transforms=True, yarn=True, paged=512, page_seed=5)
    r1.step()
    _sync()
    _same_results(r0, r1)
    kinds, worst = _check_rows(r1, OracleView(b, transforms=True, yarn=True), range(b.n_q))
    print("paged mtp + transforms + yarn:", kinds, f"worst rel-L2 {worst:.2e}")


# ------------------------------------------------------- multi-token decode

def test_mtp_decode_selection_exact_grid():
    # 4 query tokens per sequence; the last one completes a new block for the
    # first sequence (position 4k+3) and not for the others
    b = W.make_mtp_decode(seq_lens=[4 * 10000 + 4, 70003, 130005], q_len=4, budget=512,
                          n_plant=32, seed=51, exact_grid=True)
    _select_and_check(b, exact=True)


def test_end_to_end_mtp_decode_reduced():
    b = W.mtp_decode_128k(n_seq=5, ctx=20000)
    kinds, worst = _end_to_end(b, range(b.n_q))
    print("mtp decode:", kinds, f"worst rel-L2 {worst:.2e}")


def test_attend_decode_multi_matches_prefill_kernel():
    # split-K over a varlen batch equals the one-row-per-wave prefill kernel
    # on the same selections (also 1 and 3 tokens per sequence), up to the
    # order of the float32 sums: an output may cross one bf16 rounding
    # boundary (one ulp of its magnitude), plus float32 rounding where the sum
    # cancels to near zero
    b = W.make_mtp_decode(seq_lens=[9001, 40003, 7], q_len=3, budget=512, n_plant=16, seed=52)
    r = QSARunner(b.to("cuda"))
    r.step()
    _sync()
    out_m, lse_m = r.out.clone(), r.lse.clone()
    qsa.attend_prefill(r.b.q, r.b.cu_q, r.b.seq_len, r.max_q_len, r.k_cache, r.v_cache, r.sel,
                       r.sel_count, r.budget, r.out, r.lse)
    _sync()
    x, y = r.out.float(), out_m.float()
    bound = torch.maximum(x.abs(), y.abs()) * 2.0 ** -7 + 1e-5
    assert ((x - y).abs() <= bound).all(), (x - y).abs().max().item()
    assert (r.lse - lse_m).abs().max().item() <= 1e-4


# ------------------------------------------------------------- HIP graphs

def test_graph_replays_match_eager():
    # decode (dense select path) and a small prefill (list path): the captured
    # step, replayed several times with eager work in between, must give the
    # eager results exactly (the kernels are deterministic)
    for b in (W.make_decode(seq_lens=[40001, 150003, 9002], budget=512, n_plant=32, seed=41),
              W.tiny_prefill(T=512)):
        r = QSARunner(b.to("cuda"))
        r.step()
        _sync()
        want = (r.sel.clone(), r.sel_count.clone(), r.out.clone(), r.lse.clone())
        g = r.capture()
        junk = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
        for rep in range(4):
            for t in (r.sel, r.out, r.lse):
                t.fill_(0)
            junk.fill_(rep)            # eager work between replays
            _sync()
            g.replay()
            _sync()
            got = (r.sel, r.sel_count, r.out, r.lse)
            for a, e in zip(got, want):
                assert torch.equal(a, e), f"replay {rep} differs"


# ------------------------------------------------ full sizes, sampled rows

def _sampled(n, k, seed, always=()):
    rng = np.random.default_rng(seed)
    return sorted(set(rng.choice(n, k, replace=False).tolist()) | set(always))


def test_full_size_chunked_prefill_1m_sampled_rows():
    # the benchmark's prefill workload and launch configuration: a 32,768-row
    # chunk on a 1,015,808-token prefix; the oracle checks sampled rows
    b = W.chunked_prefill_1m(device="cuda")
    rows = _sampled(b.n_q, 10, 80, always=(0, 1, 4095, b.n_q - 1))
    r = QSARunner(b)
    r.step()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b), rows)
    print("1M prefill, plain:", kinds, f"worst rel-L2 {worst:.2e}", flush=True)
    # the benchmark also times the step as 4 overlapped row pieces
    seq = (r.sel.clone(), r.sel_count.clone(), r.out.clone(), r.lse.clone())
    r.sel.zero_(); r.out.zero_()
    r.step_pipelined(4)
    _sync()
    assert torch.equal(seq[0], r.sel) and torch.equal(seq[1], r.sel_count)
    assert torch.equal(seq[2].view(torch.int16), r.out.view(torch.int16))
    assert torch.equal(seq[3].view(torch.int32), r.lse.view(torch.int32))
    del seq
    del r
    torch.cuda.empty_cache()
    # the pages' configuration: indexer transforms and YaRN, over paged caches
    r = QSARunner(b, transforms=True, yarn=True, paged=256, page_seed=9)
    r.step()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b, transforms=True, yarn=True), rows[:8])
    print("1M prefill, transforms + YaRN, paged:", kinds, f"worst rel-L2 {worst:.2e}")


def test_full_size_chunked_prefill_1m_exact_grid():
    # the benchmark's 1M chunk in its launch configuration, on exact-grid
    # indexer inputs: every float32 score is exact in any summation order, so
    # the sampled-threshold selection must equal the oracle's bit for bit on
    # every checked row (no allowance branch)
    b = W.chunked_prefill_1m(device="cuda", exact_grid=True)
    rows = _sampled(b.n_q, 12, 83, always=(0, 1, 1023, 1024, b.n_q - 1))
    r = QSARunner(b)
    r.step()
    _sync()
    view = OracleView(b)
    sel, cnt = r.sel.cpu().numpy(), r.sel_count.cpu().numpy()
    for row in rows:
        assert check_selection(view, row, sel[row], int(cnt[row]), exact=True) == "exact"
    for row in rows[:4]:
        check_attention(r.out[row], r.lse[row], view.attend(row, sel[row][:cnt[row]]), f"row {row}")
    print("1M prefill, exact grid:", len(rows), "rows bit-exact", flush=True)


def test_max_context_4m_tokens():
    # the ABI's longest sequence (2^22 tokens; 2^20 candidate blocks): a
    # 1,024-row prefill chunk ending one token short of it (log-uniform
    # planting, sampled rows), then decode rows at 2^22 - 1 tokens (one with
    # near ties) beside a 3-token sequence
    L = (1 << 22) - 1
    b = W.make_prefill(prefix=L - 1024, chunk=1024, budget=512, seg=512, n_plant=64, seed=90,
                       device="cuda", distance="loguniform")
    r = QSARunner(b)
    r.step()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b), [0, 1, 511, 512, 1022, 1023])
    print("4M-token prefill chunk:", kinds, f"worst rel-L2 {worst:.2e}", flush=True)
    del r, b
    torch.cuda.empty_cache()
    b = W.make_decode(seq_lens=[L, 3, L - 2], budget=512, n_plant=32, seed=91,
                      near_tie=[False, False, True], device="cuda")
    r = QSARunner(b)
    r.step()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b), [0, 1, 2])
    print("4M-token decode:", kinds, f"worst rel-L2 {worst:.2e}")


def test_full_size_decode_128k_sampled_rows():
    # 32 sequences x (131,072 + 1) tokens, as benchmarked (also replayed from
    # a graph there; the graph test covers replays)
    b = W.decode_128k(device="cuda")
    r = QSARunner(b)
    r.step()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b), _sampled(b.n_q, 6, 81, always=(0, 31)))
    print("decode 32 x 128K:", kinds, f"worst rel-L2 {worst:.2e}")


def test_full_size_decode_selections_exact_grid():
    # the benchmarked decode shapes on exact-grid inputs, selections bit-exact:
    # 32 x 128K (1,024 active 1,024-block chunks, so the dense score pass
    # keeps that size) on sampled rows, the ragged batch to 1M (few active
    # chunks: 256-block chunks; its long row compacted in pieces) on every
    # row, and the 32 x 4-token multi-token decode on sampled rows
    b = W.decode_128k(device="cuda", exact_grid=True)
    _, _, kinds = _select_and_check(b, exact=True, rows=_sampled(b.n_q, 5, 83, always=(0, 31)))
    print("decode 32 x 128K exact grid:", kinds)
    del b
    torch.cuda.empty_cache()
    b = W.ragged_decode(device="cuda", exact_grid=True)
    _, _, kinds = _select_and_check(b, exact=True)
    print("ragged decode exact grid:", kinds)
    del b
    torch.cuda.empty_cache()
    b = W.mtp_decode_128k(device="cuda", exact_grid=True)
    _, _, kinds = _select_and_check(b, exact=True,
                                    rows=_sampled(b.n_q, 6, 84, always=(0, 3, b.n_q - 1)))
    print("mtp decode 32 x 4 at 128K exact grid:", kinds)


def test_full_size_mtp_decode_128k_sampled_rows():
    b = W.mtp_decode_128k(device="cuda")
    r = QSARunner(b)
    r.step()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b), _sampled(b.n_q, 8, 82, always=(0, 3, b.n_q - 1)))
    print("mtp decode 32 x 4 at 128K:", kinds, f"worst rel-L2 {worst:.2e}")


def test_full_size_ragged_decode_all_rows():
    # 8 sequences, log-uniform lengths up to 1M tokens, partial tail blocks,
    # near ties in half of them: every row against the oracle
    b = W.ragged_decode(device="cuda")
    print("lengths", b.seq_lens_host(), flush=True)
    r = QSARunner(b)
    r.step()
    _sync()
    kinds, worst = _check_rows(r, OracleView(b), range(b.n_q))
    print("ragged decode (full size):", kinds, f"worst rel-L2 {worst:.2e}")


# ------------------------------------------------------- mixed and small batches

def _concat(a, b):
    """One batch holding a's sequences then b's (caches padded to one length)."""
    cap = max(a.l_cap, b.l_cap)

    def pad(t):   # [n_seq][..., L][d] -> length cap on the token axis (dim -2)
        out = torch.zeros(*t.shape[:-2], cap, t.shape[-1], dtype=t.dtype)
        out[..., :t.shape[-2], :] = t
        return out
    cu = torch.cat([a.cu_q, b.cu_q[1:] + a.cu_q[-1]])
    return W.QSABatch(seq_len=torch.cat([a.seq_len, b.seq_len]), cu_q=cu,
                      idx_q=torch.cat([a.idx_q, b.idx_q]), w=torch.cat([a.w, b.w]),
                      idx_k=torch.cat([pad(a.idx_k), pad(b.idx_k)]),
                      q=torch.cat([a.q, b.q]), k=torch.cat([pad(a.k), pad(b.k)]),
                      v=torch.cat([pad(a.v), pad(b.v)]), budget=a.budget,
                      meta={"kind": "prefill"})


def test_mixed_prefill_and_decode_rows_in_one_call():
    # a 700-row prefill chunk (past 4096 candidates, sampled path) and three
    # one-row sequences in one call: max_q_len 700 takes the tiled path for all
    pre = W.make_prefill(prefix=20001, chunk=700, budget=512, seg=64, n_plant=16, seed=90)
    dec = W.make_decode(seq_lens=[40001, 9, 70002], budget=512, n_plant=16, seed=91)
    b = _concat(pre, dec)
    assert b.max_q_len() == 700 and b.n_q == 703
    r = QSARunner(b.to("cuda"))
    r.step()
    _sync()
    rows = list(range(0, 700, 37)) + [699, 700, 701, 702]
    kinds, worst = _check_rows(r, OracleView(b), rows)
    print("mixed batch:", kinds, f"worst rel-L2 {worst:.2e}")


def test_small_budget_decode():
    # budget 16 on the decode path (every score kept, one workgroup per row)
    b = W.make_decode(seq_lens=[131073, 20001, 4099, 17], budget=16, n_plant=8, seed=92)
    kinds, worst = _end_to_end(b, range(4))
    print("decode, budget 16:", kinds, f"worst rel-L2 {worst:.2e}")


def test_randomized_parity_sweep():
    # 40 seeded random batches: one-sequence prefill chunks (prefix 0 to 300K,
    # 1 to 3,000 rows), decode (1 to 6 sequences of 1 to 400K tokens, some
    # with near ties) and multi-token decode (1 to 4 rows per sequence), with
    # budgets from 1 to 512, contiguous or paged caches, with and without the
    # indexer transforms and YaRN; sampled rows against the oracle, and the
    # overlapped-pieces prefill against the sequential one
    import random
    for c in range(40):
        rng = random.Random(7100 + c)
        kind = rng.choice(["prefill", "prefill", "decode", "mtp"])
        budget = rng.choice([1, 7, 16, 100, 512, 512])
        paged = rng.choice([None, None, 256, 1024])
        transforms = rng.random() < 0.3
        yarn = rng.random() < 0.2
        if kind == "prefill":
            prefix = rng.choice([0, rng.randint(1, 5000), rng.randint(5000, 300000)])
            chunk = rng.randint(1, 3000)
            b = W.make_prefill(prefix=prefix, chunk=chunk, budget=budget,
                               seg=rng.choice([64, 512]), n_plant=rng.choice([8, 32]),
                               seed=7100 + c, device="cuda",
                               distance=rng.choice(["uniform", "loguniform"]))
            desc = f"prefill prefix={prefix} chunk={chunk}"
        elif kind == "decode":
            lens = [rng.choice([rng.randint(1, 64), rng.randint(64, 20000), rng.randint(20000, 400000)])
                    for _ in range(rng.randint(1, 6))]
            b = W.make_decode(seq_lens=lens, budget=budget, n_plant=16, seed=7100 + c,
                              device="cuda", near_tie=[rng.random() < 0.3 for _ in lens])
            desc = f"decode {lens}"
        else:
            q_len = rng.randint(1, 4)
            lens = [rng.choice([rng.randint(q_len, 64), rng.randint(64, 20000),
                                rng.randint(20000, 300000)]) for _ in range(rng.randint(1, 5))]
            b = W.make_mtp_decode(seq_lens=lens, q_len=q_len, budget=budget, n_plant=16,
                                  seed=7100 + c, device="cuda")
            desc = f"mtp q_len={q_len} {lens}"
        print(f"case {c}: {desc} budget={budget} paged={paged} transforms={transforms} yarn={yarn}",
              flush=True)
        r = QSARunner(b, transforms=transforms, yarn=yarn, paged=paged, page_seed=c)
        r.step()
        _sync()
        rows = sorted({0, b.n_q - 1} | {rng.randrange(b.n_q) for _ in range(4)})
        _check_rows(r, OracleView(b, transforms=transforms, yarn=yarn), rows)
        if kind == "prefill" and b.n_q >= 2:
            seq = (r.sel.clone(), r.sel_count.clone(), r.out.clone(), r.lse.clone())
            r.step_pipelined(rng.randint(2, 5))
            _sync()
            assert torch.equal(seq[0], r.sel) and torch.equal(seq[1], r.sel_count)
            assert torch.equal(seq[2].view(torch.int16), r.out.view(torch.int16))
            assert torch.equal(seq[3].view(torch.int32), r.lse.view(torch.int32))
        del r, b
        torch.cuda.empty_cache()
