"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call
(so no GPU is needed).  Pointer arguments here are never dereferenced."""
import ctypes
import os
import re

import pytest

from block_sparse_long_02_amd import qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

ALIGNED = 0x100000       # fake, 16-byte aligned device addresses (never touched)
MISALIGNED = 0x100002


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qsa.LIB_PATH):
        pytest.fail("libqsa.so is not built (run __graft_entry__.build())")
    return qsa.lib()


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 15, names
    for n in names:
        assert hasattr(L, n), n
        assert n in qsa.SIGNATURES, n


def test_status_strings_and_version(L):
    for code, name in qsa.STATUS.items():
        assert qsa.status_string(code) == name
    assert qsa.status_string(99) == "QSA_ERR_UNKNOWN"
    assert qsa.abi_version() == 4


def test_workspace_queries(L):
    assert L.qsa_index_select_workspace(0, 64, 100) == 0
    assert L.qsa_index_select_workspace(10, 0, 100) == 0
    assert L.qsa_index_select_workspace(10, 64, -1) == 0
    small = L.qsa_index_select_workspace(10, 64, 1000)
    big = L.qsa_index_select_workspace(10, 64, 1 << 18)
    assert small > 10 * 4096 * 8 and big > small       # candidate lists, then samples
    # 32768 query rows at 1M context: 1 GiB of lists plus 0.5 GiB of 16-bit
    # samples of every 32nd block; twice the rows pass 2^31 bytes, which must not wrap
    assert L.qsa_index_select_workspace(32768, 32768, 1 << 18) >= 32768 * 4096 * 8 + 32768 * 8192 * 2
    assert L.qsa_index_select_workspace(65536, 65536, 1 << 18) >= 65536 * 4096 * 8 + 65536 * 8192 * 2
    # up to 4 queries per sequence: every score is kept, one row per query
    dense = L.qsa_index_select_workspace(32, 1, 1 << 15)
    assert dense >= 32 * (1 << 15) * 4
    assert L.qsa_attend_decode_workspace(0) == 0
    assert L.qsa_attend_decode_workspace(32) >= 32 * 2 * 12 * 256 * 4
    assert L.qsa_attend_decode_multi_workspace(0) == 0
    assert L.qsa_attend_decode_multi_workspace(128) >= 128 * 2 * 12 * 256 * 4


def _select(L, **kw):
    a = dict(idx_q=ALIGNED, w=ALIGNED, cu_q=ALIGNED, seq_len=ALIGNED, n_seq=1, n_q=4, max_q_len=4,
             max_blocks=100, bk=ALIGNED, bk_stride=128 * 100, budget=16, sel=ALIGNED,
             cnt=ALIGNED, ws=ALIGNED, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.qsa_index_select(a["idx_q"], a["w"], a["cu_q"], a["seq_len"], a["n_seq"], a["n_q"],
                              a["max_q_len"], a["max_blocks"], a["bk"], a["bk_stride"],
                              a["budget"], a["sel"], a["cnt"], a["ws"], a["ws_bytes"],
                              a.get("table"), a.get("tstride", 0), a.get("ptok", 0), a["stream"])


def test_index_select_rejects_bad_arguments(L):
    assert _select(L, budget=0) == 1
    assert _select(L, budget=513) == 1
    assert _select(L, idx_q=None) == 1
    assert _select(L, w=MISALIGNED) == 1
    assert _select(L, bk_stride=12) == 1
    assert _select(L, n_q=-1) == 1
    assert _select(L, max_q_len=0) == 1
    assert _select(L, max_blocks=(1 << 20) + 1) == 2
    assert _select(L, ws_bytes=1024) == 3
    assert _select(L, n_q=0) == 0          # nothing to do: no HIP call either


def test_attention_and_pool_reject_bad_arguments(L):
    A = ALIGNED
    # prefill: budget, alignment, null
    assert L.qsa_attend_prefill(A, A, A, 1, 4, 4, A, A, 1024, 512, A, A, 0, A, None, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_prefill(A, A, A, 1, 4, 4, A, MISALIGNED, 1024, 512, A, A, 16, A, None, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_prefill(A, None, A, 1, 4, 4, A, A, 1024, 512, A, A, 16, A, None, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_prefill(A, A, A, 1, 4, 4, A, A, 1020, 512, A, A, 16, A, None, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_prefill(A, A, A, 1, 0, 4, A, A, 1024, 512, A, A, 16, A, None, None, 0.0625, None, 0, 0, None) == 0
    assert L.qsa_attend_prefill(A, A, A, 1, 4, 4, A, A, 1024, 512, A, A, 16, A, None, None, -1.0, None, 0, 0, None) == 1
    # decode: workspace too small, bad budget
    assert L.qsa_attend_decode(A, A, 4, A, A, 1024, 512, A, A, 16, A, A, A, 100, None, 0.0625, None, 0, 0, None) == 3
    assert L.qsa_attend_decode(A, A, 4, A, A, 1024, 512, A, A, 600, A, A, A, 1 << 30, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_decode(A, A, 4, A, A, 1024, 512, A, A, 16, A, A, MISALIGNED, 1 << 30, None, 0.0625, None, 0, 0, None) == 1
    # allocation-free decode: more than QSA_NOALLOC_MAX_SEQ (128) sequences is
    # refused on the host, as are the arguments qsa_attend_decode refuses
    assert L.qsa_attend_decode_noalloc(A, A, 129, A, A, 1024, 512, A, A, 16, A, A, None, 0.0625, None, 0, 0, None) == 2
    assert L.qsa_attend_decode_noalloc(A, A, 4, A, A, 1024, 512, A, A, 600, A, A, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_decode_noalloc(A, A, 4, A, A, 1024, 512, A, A, 16, MISALIGNED, A, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_decode_noalloc(A, A, 0, A, A, 1024, 512, A, A, 16, A, A, None, 0.0625, None, 0, 0, None) == 0
    # multi-token decode: cu_q required, workspace sized by n_q
    assert L.qsa_attend_decode_multi(A, None, A, 2, 8, A, A, 1024, 512, A, A, 16, A, A, A, 1 << 30, None, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_decode_multi(A, A, A, 2, 8, A, A, 1024, 512, A, A, 16, A, A, A, 100, None, 0.0625, None, 0, 0, None) == 3
    assert L.qsa_attend_decode_multi(A, A, A, 2, 0, A, A, 1024, 512, A, A, 16, A, A, A, 0, None, 0.0625, None, 0, 0, None) == 0
    # pooling and rope
    assert L.qsa_pool_block_keys(None, 128, A, 128, A, A, 1, 4, None, 0, 0, None) == 1
    assert L.qsa_pool_block_keys(A, 129, A, 128, A, A, 1, 4, None, 0, 0, None) == 1
    assert L.qsa_pool_block_keys(A, 128, A, 128, A, A, 0, 4, None, 0, 0, None) == 0
    assert L.qsa_pool_block_keys(A, 128, A, 128, A, A, -1, 4, None, 0, 0, None) == 1
    assert L.qsa_rope_apply(MISALIGNED, 256, 256, 2, None, 0, 10, None, None) == 1
    assert L.qsa_rope_apply(A, 256, 256, 2, None, 0, 0, None, None) == 0
    assert L.qsa_rope_apply(A, 256, 256, 2, None, (1 << 22), 10, None, None) == 2


def test_indexer_transforms_reject_bad_arguments(L):
    freq = (ctypes.c_double * 32)(*[1.0] * 32)
    bad = (ctypes.c_double * 32)(*([1.0] * 31 + [float("inf")]))
    pool = lambda **kw: L.qsa_pool_block_keys_normed(
        kw.get("ik", ALIGNED), 128 * 64, kw.get("bk", ALIGNED), 128 * 16, ALIGNED, ALIGNED,
        kw.get("n_seq", 1), kw.get("span", 16), None, kw.get("eps", 1e-6),
        kw.get("freq", None), None, 0, 0, None)
    query = lambda **kw: L.qsa_index_query_transform(
        kw.get("q", ALIGNED), kw.get("o", ALIGNED), ALIGNED, ALIGNED, kw.get("n_seq", 1),
        kw.get("n_q", 4), kw.get("mq", 4), None, kw.get("eps", 1e-6), kw.get("freq", None), None)
    for f in (pool, query):
        assert f(eps=-1.0) == 1
        assert f(eps=float("nan")) == 1
        assert f(eps=float("inf")) == 1
        assert f(freq=ctypes.cast(bad, ctypes.c_void_p)) == 1
        assert f(n_seq=-1) == 1
        assert f(n_seq=0) == 0                     # nothing to do, nothing enqueued
        assert f(n_seq=0, freq=ctypes.cast(freq, ctypes.c_void_p)) == 0
    assert pool(ik=None) == 1 and pool(bk=MISALIGNED) == 1
    assert pool(span=0) == 0 and pool(span=-1) == 1
    assert query(q=None) == 1 and query(o=MISALIGNED) == 1
    assert query(n_q=0) == 0 and query(mq=0) == 0 and query(n_q=-1) == 1


def test_rope_tables_and_softmax_scale_are_validated(L):
    A = ALIGNED
    bad = (ctypes.c_double * 32)(*([1.0] * 31 + [float("nan")]))
    badp = ctypes.cast(bad, ctypes.c_void_p)
    for sc in (0.0, -0.0625, float("nan"), float("inf")):
        assert L.qsa_attend_prefill(A, A, A, 1, 4, 4, A, A, 1024, 512, A, A, 16, A, None, None, sc, None, 0, 0, None) == 1
        assert L.qsa_attend_decode(A, A, 4, A, A, 1024, 512, A, A, 16, A, A, A, 1 << 30, None, sc, None, 0, 0, None) == 1
        assert L.qsa_attend_decode_multi(A, A, A, 2, 8, A, A, 1024, 512, A, A, 16, A, A, A, 1 << 30, None, sc, None, 0, 0, None) == 1
    assert L.qsa_attend_prefill(A, A, A, 1, 4, 4, A, A, 1024, 512, A, A, 16, A, None, badp, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_attend_decode(A, A, 4, A, A, 1024, 512, A, A, 16, A, A, A, 1 << 30, badp, 0.0625, None, 0, 0, None) == 1
    assert L.qsa_rope_apply(A, 256, 256, 2, None, 0, 10, badp, None) == 1


def test_yarn_helper_matches_the_oracle(L):
    """Host logic: the library's YaRN table and scale against the oracle's,
    each written separately from the YaRN paper's formula."""
    from oracle import qsa_oracle as O
    import numpy as np
    f, sc = qsa.yarn_rope()
    ref = O.yarn_inv_freq()
    # same float64 steps; numpy's vectorised pow and the C library's pow may
    # differ in the last bit of a frequency
    assert np.allclose(np.asarray(f), ref, rtol=2.5e-16, atol=0)
    assert abs(sc - O.yarn_softmax_scale()) <= 2 ** -24 * O.yarn_softmax_scale()
    f1, sc1 = qsa.yarn_rope(factor=1.0)
    assert np.allclose(f1, O.yarn_inv_freq(factor=1.0), rtol=5e-16, atol=0) and sc1 == 0.0625
    for fac, ctx in ((2.0, 2 * np.pi * 24.25), (8.0, 32768.0)):
        g, _ = qsa.yarn_rope(factor=fac, orig_ctx=ctx)
        assert np.allclose(np.asarray(g), O.yarn_inv_freq(factor=fac, orig_ctx=ctx), rtol=5e-16, atol=0)
    buf = (ctypes.c_double * 32)()
    bp = ctypes.cast(buf, ctypes.c_void_p)
    for args in ((1.0, 4.0, 262144.0, 1.0, 32.0), (1e7, 0.5, 262144.0, 1.0, 32.0),
                 (1e7, 4.0, 0.0, 1.0, 32.0), (1e7, 4.0, 262144.0, 32.0, 32.0),
                 (1e7, 4.0, 262144.0, -1.0, 32.0), (1e7, float("nan"), 262144.0, 1.0, 32.0)):
        assert L.qsa_yarn_rope(*args, bp, None) == 1, args
    assert L.qsa_yarn_rope(1e7, 4.0, 262144.0, 1.0, 32.0, None, None) == 1
    assert L.qsa_yarn_rope(1e7, 4.0, 262144.0, 1.0, 32.0, bp, None) == 0


def test_page_arguments_are_validated(L):
    A = ALIGNED
    # (table_stride, page_tokens): page_tokens must be a power of two in [256, 2^22]
    bad = [(1, 0), (1, 128), (1, 384), (1, 1 << 23), (0, 256), (-4, 256)]
    for ts, pt in bad:
        assert _select(L, table=A, tstride=ts, ptok=pt) == 1, (ts, pt)
        assert L.qsa_pool_block_keys(A, 128, A, 128, A, A, 1, 4, A, ts, pt, None) == 1
        assert L.qsa_pool_block_keys_normed(A, 128, A, 128, A, A, 1, 4, None, 1e-6, None, A, ts, pt,
                                            None) == 1
        assert L.qsa_attend_prefill(A, A, A, 1, 4, 4, A, A, 0, 512, A, A, 16, A, None, None, 0.0625,
                                    A, ts, pt, None) == 1
        assert L.qsa_attend_decode(A, A, 4, A, A, 0, 512, A, A, 16, A, A, A, 1 << 30, None, 0.0625,
                                   A, ts, pt, None) == 1
        assert L.qsa_attend_decode_multi(A, A, A, 2, 8, A, A, 0, 512, A, A, 16, A, A, A, 1 << 30,
                                         None, 0.0625, A, ts, pt, None) == 1
    # a NULL table ignores the page arguments; valid pages with nothing to do enqueue nothing
    assert L.qsa_pool_block_keys(A, 128, A, 128, A, A, 0, 4, None, -1, 3, None) == 0
    assert L.qsa_pool_block_keys(A, 128, A, 128, A, A, 0, 4, A, 16, 256, None) == 0
    assert L.qsa_attend_prefill(A, A, A, 1, 0, 4, A, A, 0, 512, A, A, 16, A, None, None, 0.0625,
                                A, 4, 1 << 22, None) == 0


def test_probe_library_exports_and_validates():
    """The measurement probes (include/qsa_probe.h; not part of the path's
    library) load and reject bad arguments on the host."""
    from block_sparse_long_02_amd import build as B
    path = B.PROBE_LIB
    if not os.path.exists(path):
        B.build_probe()
    P = ctypes.CDLL(path)
    src = open(os.path.join(ROOT, "include", "qsa_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", src)))
    assert names == ["qsa_probe_copy", "qsa_probe_gather", "qsa_probe_mfma_bf16",
                     "qsa_probe_read"], names
    for n in names:
        assert hasattr(P, n), n
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    P.qsa_probe_mfma_bf16.argtypes = [i32, i32, i32, vp, vp]
    P.qsa_probe_read.argtypes = [vp, i64, i32, vp, vp]
    P.qsa_probe_copy.argtypes = [vp, vp, i64, i32, vp]
    P.qsa_probe_gather.argtypes = [vp, i64, vp, i64, i32, i32, vp, vp]
    assert P.qsa_probe_mfma_bf16(0, 10, 8, ALIGNED, None) == 1
    assert P.qsa_probe_mfma_bf16(8, 0, 8, ALIGNED, None) == 1
    assert P.qsa_probe_mfma_bf16(8, 10, 8, None, None) == 1
    assert P.qsa_probe_mfma_bf16(8, 10, 12, ALIGNED, None) == 1
    assert P.qsa_probe_read(ALIGNED, 100, 8, ALIGNED, None) == 1        # not a multiple of 64
    assert P.qsa_probe_read(MISALIGNED, 128, 8, ALIGNED, None) == 1
    assert P.qsa_probe_copy(ALIGNED, ALIGNED, 0, 8, None) == 1
    assert P.qsa_probe_gather(ALIGNED, 1 << 20, ALIGNED, 16, 3000, 8, ALIGNED, None) == 1  # not 2^k
    assert P.qsa_probe_gather(ALIGNED, 1 << 20, None, 16, 2048, 8, ALIGNED, None) == 1
    assert P.qsa_probe_gather(ALIGNED, 1 << 20, ALIGNED, 0, 2048, 8, ALIGNED, None) == 1
    assert P.qsa_probe_gather(ALIGNED, 1 << 40, ALIGNED, 16, 16, 8, ALIGNED, None) == 2


def test_pipeline_piece_bounds():
    """The overlapped prefill schedule covers every row once, in order, with
    a short first piece and, from three pieces on, a short last one."""
    from block_sparse_long_02_amd.runner import piece_bounds
    for n in (1, 3, 7, 8, 333, 32768):
        for parts in (1, 2, 3, 4, 7):
            b = piece_bounds(n, parts)
            assert b[0] == 0 and b[-1] == n and len(b) == max(parts, 1) + 1
            assert all(x <= y for x, y in zip(b, b[1:]))
    assert piece_bounds(32768, 4) == [0, 4096, 16384, 28672, 32768]
    assert piece_bounds(32768, 5) == [0, 4096, 12288, 20480, 28672, 32768]
    assert piece_bounds(32768, 2) == [0, 4096, 32768]


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus above 1 exits with a message before touching a GPU."""
    import subprocess
    import sys
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_attention_allowed_error():
    # 1e-2 wherever the allowance plus half a bf16 ulp stays below it;
    # otherwise the allowance plus half an ulp of the output at that magnitude
    import numpy as np
    from tests._harness import allowed_error
    x = np.array([0.0, 1e-30, 0.5, 1.999, 2.0, 3.99, 4.0, -5.5, 7.99, 8.0, -100.0])
    want = np.array([1e-2] * 6 + [2.0 ** -6, 2.0 ** -6, 2.0 ** -6, 2.0 ** -5, 2.0 ** -2])
    assert np.array_equal(allowed_error(x, np.zeros_like(x)), want)
    b = np.array([0.004, 0.004, 0.02, 0.02])
    x = np.array([1.0, 3.995, 1.0, 3.99])
    # 1.004 lies in [1, 2): 0.004 + 2^-8 < 1e-2.  3.999 lies in [2, 4): 0.004 +
    # 2^-7 > 1e-2.  4.01 lies in [4, 8), so 3.99 with allowance 0.02 takes 2^-6.
    want = np.array([1e-2, 0.004 + 2.0 ** -7, 0.02 + 2.0 ** -8, 0.02 + 2.0 ** -6])
    assert np.allclose(allowed_error(x, b), want, rtol=0, atol=1e-15)
