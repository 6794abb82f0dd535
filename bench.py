"""QSA hot-path benchmark on one MI355X.

Headline (`value`): chunked prefill at 1M context -- a 32,768-token query
chunk on a 1,015,808-token cached prefix (batch 1, budget 512 blocks + tail):
query tokens per second for one step = pool the chunk's new blocks, select
blocks for every query, sparse attention, call after call.  `pipelined`
times the same step with the chunk's rows in 4 pieces, each piece's
attention overlapping the next piece's selection (two streams, same calls and
results).  Alongside it (`decode`): a decode
step for 32 sequences of 131,072 cached tokens + the new one; and
(`mtp_decode`) a multi-token decode step with 4 query tokens per sequence.

Inputs are seeded synthetic tensors generated directly in HBM; the timed
region starts with everything resident.  Timing uses HIP events on the stream
the kernels run on.  `roofline` is for the dominant kernel (the attention
kernel of the prefill step): its algorithmic flops per launch / its mean
duration against the bf16 MFMA peak, the bound it cannot exceed (its
zero-reuse gather bytes already exceed the HBM rate, through cache reuse);
`memory_side` gives the counted bytes beyond L2 (`traffic`, from
profiles/traffic.json while the kernel source is unchanged) against the
HBM peak and the measured achievable read rate.  `rows` gives each hot-path
row against its own roofline.  `prefill_8k` times an 8,192-token prefill
(and the 2,048-token dense case); `ragged_decode` a decode step of 8
sequences of log-uniform lengths up to 1M tokens, against that draw's own
HBM floor.  `index_transforms`
repeats the prefill step with the pages' indexer transforms (RMSNorm and
partial RoPE of block keys and queries) and times each transform kernel;
`yarn` repeats it with the transforms and the YaRN-extended rotations and
softmax scale (the pages' configuration past the native 262,144 tokens).
`paged` repeats the prefill and decode steps over caches kept in 256-token
pages in a random physical order (block tables).
`cpu_baseline` times the CPU oracle on a bounded, stratified sample of the same
workload, with all host threads and with one.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--only prefill|prefill8k|decode|ragged|mtp]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA tokens/s (prefill, decode) at 128K–1M ctx; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0
TOKEN_GATHER_BYTES = 2 * 2 * 256 * 2      # 2 KV heads x (K + V) x 256 dims x bf16
Q_ROW_BYTES = 24 * 256 * 2
BLOCK_KEY_BYTES = 128 * 2
PAGE_TOKENS = 256                         # paged-cache runs: 256-token pages
PIPE_PARTS = 4                            # prefill rows in 4 pieces, select / attend overlapped


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def set_sizes(runner):
    """Sum over query rows of |S_i| = 4*K_i + tail_i, and of n_c."""
    import numpy as np
    cnt = runner.sel_count.cpu().numpy().astype(np.int64)
    pos = np.asarray(runner.b.q_pos_host(), dtype=np.int64)
    tails = (pos + 1) % 4
    return int((4 * cnt + tails).sum()), int(((pos + 1) // 4).sum())


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profiles(kernel_file, key):
    """HBM-side bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated against a
    copy of known size) from the committed counter runs, if they were taken on
    the current source of the kernel's file; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))[key]
    except (KeyError, ValueError):
        return None
    if d.get("source_sha") != src_hash(kernel_file):
        return None
    return d.get("bytes_per_launch")


def achievable_peaks():
    """Measured achievable rates (profiles/achievable_peaks.json, micro-benchmarks
    of the MFMA pipe and of HBM reads), or an empty dict."""
    p = os.path.join(ROOT, "profiles", "achievable_peaks.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return {}
    out = {}
    reads = [v["gbs"] for k, v in d.items() if k.startswith("hbm_read_")]
    mfma = [v["tflops"] for k, v in d.items() if k.startswith("mfma_bf16_")]
    if reads:
        out["hbm_read_gbs"] = max(reads)
    if mfma:
        out["mfma_bf16_tflops"] = max(mfma)
    return out


def decode_traffic():
    """HBM-side bytes of one decode step (sum over its kernels), or None."""
    csrc = os.path.join(ROOT, "block_sparse_long_02_amd", "csrc")
    # (131,073 tokens complete no new block: the step launches no pooling)
    parts = [("qsa_index.hip", "score_dense_decode_128k"),
             ("qsa_index.hip", "select_dense_decode_128k"),
             ("qsa_attend.hip", "attend_decode_128k"),
             ("qsa_attend.hip", "combine_decode_128k")]
    vals = [traffic_from_profiles(os.path.join(csrc, f), k) for f, k in parts]
    return None if any(v is None for v in vals) else int(sum(vals))


def time_steps(r, args):
    """Warm up, then time args.steps sequential steps (pool, select, attend)
    with HIP events: (total ms, mean ms per stage, sorted per-step ms)."""
    import torch
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        ev[k][0].record()
        r.pool()
        ev[k][1].record()
        r.select()
        ev[k][2].record()
        r.attend()
        ev[k][3].record()
    stop.record()
    torch.cuda.synchronize()
    stage = {n: sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)) / args.steps
             for i, n in enumerate(["pool", "select", "attend"])}
    per_step = sorted(ev[k][0].elapsed_time(ev[k][3]) for k in range(args.steps))
    return start.elapsed_time(stop), stage, per_step


def time_prefill(args, transforms=False, batch=None, yarn=False, paged=None, pipelined=True):
    """The chunked-prefill step (or the prefill of `batch`); transforms=True
    runs it with the pages' indexer transforms (normalised, rotated block keys
    and queries), yarn=True with the YaRN-extended rotations and softmax
    scale; pipelined=False skips the overlapped-pieces timing."""
    import torch
    from block_sparse_long_02_amd import workloads as W
    from block_sparse_long_02_amd.runner import QSARunner

    t0 = time.time()
    b = W.chunked_prefill_1m(device="cuda") if batch is None else batch
    r = QSARunner(b, transforms=transforms, yarn=yarn, paged=paged)
    torch.cuda.synchronize()
    log(f"prefill workload ready in {time.time() - t0:.1f}s")
    total_ms, stage, per_step = time_steps(r, args)
    # For comparison: the chunk's rows in PIPE_PARTS pieces, each piece's
    # attention (memory-bound) on a second stream while the next piece is
    # selected (MFMA-bound).  Same calls, same results.  Its gain depends on
    # how the hardware interleaves the two kernels, and some steps come out
    # much slower, so the headline is the sequential step.
    pipe = None
    if pipelined:
        for _ in range(max(1, args.warmup)):
            r.step_pipelined(PIPE_PARTS)
        torch.cuda.synchronize()
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        p_start, p_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p_start.record()
        for k in range(args.steps):
            pev[k][0].record()
            r.step_pipelined(PIPE_PARTS)
            pev[k][1].record()
        p_stop.record()
        torch.cuda.synchronize()
        pipe_steps = sorted(e[0].elapsed_time(e[1]) for e in pev)
        pipe = dict(parts=PIPE_PARTS, ms_per_step=p_start.elapsed_time(p_stop) / args.steps,
                    step_ms_median=pipe_steps[len(pipe_steps) // 2], step_ms_min=pipe_steps[0],
                    step_ms_max=pipe_steps[-1])
    sum_s, sum_nc = set_sizes(r)
    n_q = r.n_q
    attend_bytes = sum_s * TOKEN_GATHER_BYTES + n_q * (2 * Q_ROW_BYTES + 24 * 4 + r.budget * 4)
    attend_gbs = attend_bytes / (stage["attend"] * 1e-3) / 1e9
    # core flops: per token of S and head, q.k and p.v over 256 dims
    attend_flops = sum_s * 24 * 256 * 4
    # the method scores each candidate once (sampling is overhead, not work)
    index_flops = sum_nc * 1024
    res = dict(
        n_q=n_q, ms_per_step=total_ms / args.steps, stages_ms=stage,
        step_ms_median=per_step[len(per_step) // 2], step_ms_min=per_step[0],
        value=n_q / (total_ms / args.steps * 1e-3),
        pipelined=pipe,
        sum_set=sum_s, sum_candidates=sum_nc,
        attend=dict(bytes=attend_bytes, gbs=attend_gbs, flops=attend_flops),
        index=dict(flops=index_flops, tflops=index_flops / (stage["select"] * 1e-3) / 1e12),
        runner=r, batch=b)
    return res


def time_calls(fn, steps):
    """Mean duration (ms) of fn() over `steps` calls, HIP events on the current stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_transforms(args, pre):
    """The prefill workload in the pages' fuller configurations.  Returns
    (yarn, transforms): the step with the indexer transforms and YaRN; the
    step with the transforms alone, plus each transform kernel on its own
    against HBM."""
    from block_sparse_long_02_amd import qsa
    b = pre["batch"]
    tr = time_prefill(args, transforms=True, batch=b)
    r = tr["runner"]
    steps = max(args.steps, 10)
    q_ms = time_calls(lambda: qsa.index_query_transform(b.idx_q, r.idx_q_t, b.cu_q, b.seq_len,
                                                        r.max_q_len), steps)
    k_ms = time_calls(lambda: r.pool(), steps)
    q_bytes = 2 * b.idx_q.numel() * 2                       # read raw, write transformed
    n_new = int((r.pool_end - r.pool_begin).sum().item())
    k_bytes = n_new * (4 * BLOCK_KEY_BYTES + BLOCK_KEY_BYTES)
    del tr["runner"], r
    import torch
    torch.cuda.empty_cache()
    # the pages' configuration at 1M: the transforms and YaRN together
    ya = time_prefill(args, transforms=True, batch=b, yarn=True)
    yarn = {"ms_per_step": round(ya["ms_per_step"], 4), "value": round(ya["value"], 1),
            "unit": "tokens/s", "stages_ms": {k: round(v, 4) for k, v in ya["stages_ms"].items()},
            "attend_gbs_zero_reuse": round(ya["attend"]["gbs"], 1)}
    del ya
    torch.cuda.empty_cache()
    return yarn, {
        "ms_per_step": round(tr["ms_per_step"], 4), "value": round(tr["value"], 1),
        "unit": "tokens/s", "stages_ms": {k: round(v, 4) for k, v in tr["stages_ms"].items()},
        "index_tflops": round(tr["index"]["tflops"], 1),
        "query_transform": {"kernel": "index_query_transform_kernel", "ms": round(q_ms, 4),
                            "bound": "hbm", "algorithmic_bytes": q_bytes,
                            "frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "key_transform": {"kernel": "pool_block_keys_normed_kernel", "ms": round(k_ms, 4),
                          "blocks": n_new, "bound": "hbm", "algorithmic_bytes": k_bytes,
                          "frac": round(k_bytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def time_decode(args, mtp=False, paged=None, ragged=False):
    """Decode step (one query per sequence), or with mtp=True a multi-token
    decode step (4 query tokens per sequence), with ragged=True the ragged
    decode (8 sequences, log-uniform lengths up to 1M tokens); paged=P over
    P-token pages."""
    import torch
    from block_sparse_long_02_amd import workloads as W
    from block_sparse_long_02_amd.runner import QSARunner

    t0 = time.time()
    b = (W.mtp_decode_128k(device="cuda") if mtp else
         W.ragged_decode(device="cuda") if ragged else W.decode_128k(device="cuda"))
    r = QSARunner(b, paged=paged)
    # 512 MB > MALL, swept by a read before each step so that the step starts
    # with none of its data cached and no dirty lines to write back
    flush = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"{'mtp ' if mtp else ''}decode workload ready in {time.time() - t0:.1f}s")
    for _ in range(args.warmup):
        r.step()
    # a decode step is replayed from a HIP graph, as a serving loop would;
    # the stage split comes from two partial graphs timed the same way
    g_step = r.capture()
    g_sel = r.capture(("pool", "select"))
    g_att = r.capture(("attend",))
    torch.cuda.synchronize()

    def timed(graphs, stats=False):
        evs = []
        for _ in range(args.steps):
            flush.sum()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)]
            e[0].record()
            for i, g in enumerate(graphs):
                g.replay()
                e[i + 1].record()
            evs.append(e)
        torch.cuda.synchronize()
        if stats:   # one graph: mean, median, minimum
            d = sorted(e[0].elapsed_time(e[1]) for e in evs)
            return sum(d) / len(d), d[len(d) // 2], d[0]
        return [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / len(evs) for i in range(len(graphs))]

    for g in (g_step, g_sel, g_att):
        g.replay()
    ms, med, mn = timed([g_step], stats=True)
    sel_ms, att_ms = timed([g_sel, g_att])
    sum_s, sum_nc = set_sizes(r)
    n_seq, n_q = r.n_seq, r.n_q
    # block keys once per sequence (its queries are scored together), each
    # query row's own gather, queries in and out
    blocks_read = sum(L // 4 for L in b.seq_lens_host())
    step_bytes = blocks_read * BLOCK_KEY_BYTES + sum_s * TOKEN_GATHER_BYTES + n_q * (
        2 * Q_ROW_BYTES + 4 * 128 * 2 + 16)
    return dict(value=n_q / (ms * 1e-3), ms_per_step=ms, step_ms_median=med, step_ms_min=mn,
                stages_ms=dict(select=sel_ms, attend=att_ms),
                hbm=dict(bytes=step_bytes, gbs=step_bytes / (ms * 1e-3) / 1e9),
                runner=r, batch=b)


def host_cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(pre, budget_s):
    """Time the CPU oracle on a bounded, stratified sample of the prefill
    workload: rows at evenly spaced positions through the chunk, each through
    the oracle's whole per-row pipeline.  Runs once with every host thread
    available to numpy's BLAS and once with one thread."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import qsa_oracle as O
    b = pre["batch"]

    def f64(t):
        return t.detach().float().cpu().double().numpy()

    prefix = b.meta["prefix"]
    chunk = b.meta["chunk"]
    # pooled prefix blocks are cache state (not timed); the chunk's new blocks are step work
    idx_k = f64(b.idx_k[0])
    kb_prefix = O.pool_block_keys(idx_k[:prefix], prefix // 4)
    t0 = time.time()
    kb_new = O.pool_block_keys(idx_k[prefix:prefix + chunk], chunk // 4)
    t_pool = time.time() - t0
    kbar = np.concatenate([kb_prefix, kb_new])
    host_threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    def run(threads, seconds, n_strata):
        # stratified: one row from each of n_strata equal slices of the chunk,
        # slices visited in a shuffled order until the time budget is spent
        rng = np.random.default_rng(threads)
        starts = np.arange(n_strata) * chunk // n_strata
        offs = rng.integers(0, max(1, chunk // n_strata), n_strata)
        order = rng.permutation(n_strata)
        done, t_rows = [], 0.0
        with threadpool_limits(limits=threads):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            for st in order:
                if t_rows > seconds:
                    break
                row = int(min(chunk - 1, starts[st] + offs[st]))
                p = prefix + row
                t1 = time.time()
                n_c = O.completed_blocks(p)
                sc = O.block_scores(f64(b.idx_q[row]), b.w[row].cpu().numpy(), kbar[:n_c])
                blocks = O.select_blocks(sc, b.budget)
                tokens = O.sparse_token_set(blocks, p)
                t = torch.as_tensor(tokens, device=b.k.device)
                k_rows = f64(b.k[0][:, t, :]).transpose(1, 0, 2)
                v_rows = f64(b.v[0][:, t, :]).transpose(1, 0, 2)
                O.attend(f64(b.q[row]), k_rows, v_rows, tokens, p)
                t_rows += time.time() - t1
                done.append(row)
        est = t_pool + t_rows / len(done) * chunk
        return dict(value=chunk / est, threads=int(used), rows=len(done),
                    seconds=round(t_pool + t_rows, 2))

    multi = run(host_threads, budget_s, 1024)
    single = run(1, budget_s, 1024)
    return dict(value=round(multi["value"], 2), unit="tokens/s", cores=multi["threads"],
                kind="oracle", cpu=host_cpu_model(), host_cpus=host_threads,
                sample=(f"{multi['rows']} of {chunk} query rows, stratified (one row from each of "
                        f"{multi['rows']} of 1024 equal slices of the chunk), full per-row pipeline "
                        f"(score {prefix // 4}+ blocks, select, expand, attend) plus pooling of the "
                        f"chunk's {chunk // 4} new blocks; time scaled to the whole chunk"),
                seconds=multi["seconds"],
                single_thread=dict(value=round(single["value"], 2), unit="tokens/s", cores=1,
                                   rows=single["rows"], seconds=single["seconds"]))


def attend_roofline(pre, attend_file):
    """Roofline of the dominant kernel, the prefill attention.  Its zero-reuse
    gather bytes (every selected token once per query row) already exceed the
    HBM rate -- rows that select the same blocks share them through L2 and the
    Infinity Cache -- so the bound it cannot exceed is the MFMA rate of its
    algorithmic flops.  memory_side gives the counted bytes beyond L2 per
    launch (FETCH_SIZE + WRITE_SIZE, calibrated; L2 misses served by HBM or
    the Infinity Cache) against the HBM peak and the measured achievable
    streaming read."""
    ms = pre["stages_ms"]["attend"]
    tflops = pre["attend"]["flops"] / (ms * 1e-3) / 1e12
    traffic = traffic_from_profiles(attend_file, "attend_prefill_1m")
    ach = achievable_peaks()
    mem = {"counted_bytes_per_launch": traffic}
    if traffic:
        gbs = traffic / (ms * 1e-3) / 1e9
        mem.update(counted_gbs=round(gbs, 1), hbm_peak_gbs=HBM_PEAK_GBS,
                   frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
        if "hbm_read_gbs" in ach:
            mem.update(achievable_read_gbs=ach["hbm_read_gbs"],
                       frac_of_achievable_read=round(gbs / ach["hbm_read_gbs"], 4))
    mem["binds"] = ("the memory side: the kernel waits on its gathers (zero-reuse "
                    f"{pre['attend']['gbs'] / 1e3:.1f} TB/s; the counted beyond-L2 bytes include "
                    "Infinity Cache hits, so they can exceed the HBM read rate)")
    return {"kernel": "attend_rows_kernel (sparse prefill attention)", "bound": "mfma",
            "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4), "traffic": traffic,
            "algorithmic_flop_per_launch": pre["attend"]["flops"],
            "mean_launch_ms": round(ms, 4),
            "zero_reuse_gather_bytes_per_launch": pre["attend"]["bytes"],
            "zero_reuse_gbs": round(pre["attend"]["gbs"], 1),
            "memory_side": mem}


def prefill_8k(args):
    """The 8,192-token prefill from an empty cache (budget 512, 64 planted
    blocks per 1,024-row segment) and its 2,048-token dense case: tokens/s,
    and the index select and attention against the bf16 MFMA peak (the KV
    cache, 17 MB, stays in L2 and the Infinity Cache)."""
    import torch
    from block_sparse_long_02_amd import workloads as W
    res = {}
    for T in (8192, 2048):
        pr = time_prefill(args, batch=W.prefill_8k(device="cuda", T=T), pipelined=False)
        st = pr["stages_ms"]
        res[f"T{T}"] = {
            "ms_per_step": round(pr["ms_per_step"], 4), "value": round(pr["value"], 1),
            "unit": "tokens/s", "stages_ms": {k: round(v, 4) for k, v in st.items()},
            "index_select_tflops": round(pr["index"]["tflops"], 1),
            "index_select_frac_mfma": round(pr["index"]["tflops"] / MFMA_BF16_PEAK_TFS, 4),
            "attend_tflops": round(pr["attend"]["flops"] / (st["attend"] * 1e-3) / 1e12, 1),
            "attend_frac_mfma": round(pr["attend"]["flops"] / (st["attend"] * 1e-3) / 1e12
                                      / MFMA_BF16_PEAK_TFS, 4),
            "step_mfma_floor_ms": round((pr["index"]["flops"] + pr["attend"]["flops"])
                                        / (MFMA_BF16_PEAK_TFS * 1e12) * 1e3, 4)}
        log(f"prefill T={T}: {res[f'T{T}']}")
        del pr
        torch.cuda.empty_cache()
    res["workload"] = ("prefill from an empty cache, batch 1, T=8192 (and T=2048, where every row "
                       "keeps every completed block: dense causal attention), budget 512 blocks + tail")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "prefill8k", "decode", "ragged", "mtp"],
                    default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the QSA path here is "
              "single-GPU and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_long_02_amd import qsa
    qsa.lib()
    assert torch.cuda.is_available()

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    if args.only in (None, "prefill"):
        pre = time_prefill(args)
        log(f"prefill: {pre['ms_per_step']:.3f} ms/step, stages {pre['stages_ms']}; "
            f"{PIPE_PARTS} overlapped pieces {pre['pipelined']['ms_per_step']:.3f} ms/step")
        attend_file = os.path.join(ROOT, "block_sparse_long_02_amd", "csrc", "qsa_attend.hip")
        out.update(value=round(pre["value"], 1), unit="tokens/s",
                   ms_per_step=round(pre["ms_per_step"], 4),
                   step_ms_median=round(pre["step_ms_median"], 4),
                   step_ms_min=round(pre["step_ms_min"], 4))
        out["pipelined"] = {k: round(v, 4) for k, v in pre["pipelined"].items()}
        out["config"] = {
            "workload": "chunked prefill: 32768-token chunk on a 1015808-token cached prefix "
                        "(1048576 total), batch 1, budget 512 blocks + tail",
            "global_batch": 1, "seq_len": 1048576, "query_tokens": pre["n_q"], "budget": 512}
        out["roofline"] = attend_roofline(pre, attend_file)
        out["stages_ms"] = {k: round(v, 4) for k, v in pre["stages_ms"].items()}
        pool_bytes = (pre["n_q"] // 4) * (4 * BLOCK_KEY_BYTES + BLOCK_KEY_BYTES)
        out["rows"] = {
            "a1_pool": {"ms": round(pre["stages_ms"]["pool"], 4), "bound": "hbm",
                        "algorithmic_bytes": pool_bytes,
                        "frac": round(pool_bytes / (pre["stages_ms"]["pool"] * 1e-3) / 1e9
                                      / HBM_PEAK_GBS, 4)},
            "a2_a3_index_select": {"ms": round(pre["stages_ms"]["select"], 4), "bound": "mfma",
                                   "algorithmic_tflop": round(pre["index"]["flops"] / 1e12, 3),
                                   "tflops": round(pre["index"]["tflops"], 1),
                                   "frac": round(pre["index"]["tflops"] / MFMA_BF16_PEAK_TFS, 4)},
            "a4_a5_a6_attend_prefill": {"ms": round(pre["stages_ms"]["attend"], 4),
                                        "bound": "gather", "algorithmic_bytes": pre["attend"]["bytes"],
                                        "frac_hbm_zero_reuse": round(pre["attend"]["gbs"] / HBM_PEAK_GBS, 4),
                                        "core_tflops": round(pre["attend"]["flops"] / (pre["stages_ms"]["attend"] * 1e-3) / 1e12, 1),
                                        "frac_mfma": round(pre["attend"]["flops"] / (pre["stages_ms"]["attend"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)}}
        out["index_select"] = {"algorithmic_tflop": round(pre["index"]["flops"] / 1e12, 3),
                               "tflops": round(pre["index"]["tflops"], 1),
                               "frac_of_bf16_mfma_peak": round(pre["index"]["tflops"] / MFMA_BF16_PEAK_TFS, 4)}
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(pre, args.cpu_seconds)
        del pre["runner"]
        torch.cuda.empty_cache()
        out["yarn"], out["index_transforms"] = time_transforms(args, pre)
        log(f"prefill with indexer transforms: {out['index_transforms']}")
        log(f"prefill with indexer transforms and YaRN: {out['yarn']}")
        pg = time_prefill(args, batch=pre["batch"], paged=PAGE_TOKENS)
        out["paged"] = {"page_tokens": PAGE_TOKENS, "order": "random physical pages",
                        "prefill": {"ms_per_step": round(pg["ms_per_step"], 4),
                                    "value": round(pg["value"], 1), "unit": "tokens/s",
                                    "stages_ms": {k: round(v, 4) for k, v in pg["stages_ms"].items()}}}
        log(f"paged prefill: {out['paged']['prefill']}")
        del pg
        torch.cuda.empty_cache()
        del pre
        torch.cuda.empty_cache()
    if args.only in (None, "prefill8k"):
        out["prefill_8k"] = prefill_8k(args)
    if args.only in (None, "decode"):
        dec = time_decode(args)
        log(f"decode: {dec['ms_per_step']:.4f} ms/step, stages {dec['stages_ms']}")
        d = {"value": round(dec["value"], 1), "unit": "tokens/s",
             "ms_per_step": round(dec["ms_per_step"], 4),
             "step_ms_median": round(dec["step_ms_median"], 4),
             "step_ms_min": round(dec["step_ms_min"], 4),
             "config": {"workload": "decode: 32 sequences x (131072 cached + 1 new) tokens, "
                                    "budget 512 blocks + tail, MALL flushed before each step"},
             "roofline": {"bound": "hbm", "scope": "whole step",
                          "achieved": round(dec["hbm"]["gbs"], 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(dec["hbm"]["gbs"] / HBM_PEAK_GBS, 4),
                          "traffic": decode_traffic(),
                          "algorithmic_bytes": dec["hbm"]["bytes"]},
             "stages_ms": {k: round(v, 4) for k, v in dec["stages_ms"].items()}}
        if args.only == "decode":
            out.update(value=d["value"], unit="tokens/s", ms_per_step=d["ms_per_step"],
                       config=d["config"], roofline=d["roofline"])
        else:
            out["decode"] = d
        dec = None
        torch.cuda.empty_cache()
        dp = time_decode(args, paged=PAGE_TOKENS)
        log(f"paged decode: {dp['ms_per_step']:.4f} ms/step, stages {dp['stages_ms']}")
        out.setdefault("paged", {"page_tokens": PAGE_TOKENS, "order": "random physical pages"})
        out["paged"]["decode"] = {"ms_per_step": round(dp["ms_per_step"], 4),
                                  "value": round(dp["value"], 1), "unit": "tokens/s",
                                  "stages_ms": {k: round(v, 4) for k, v in dp["stages_ms"].items()},
                                  "hbm_frac": round(dp["hbm"]["gbs"] / HBM_PEAK_GBS, 4)}
        dp = None
        torch.cuda.empty_cache()
    if args.only in (None, "ragged"):
        rg = time_decode(args, ragged=True)
        lens = rg["batch"].seq_lens_host()
        log(f"ragged decode {lens}: {rg['ms_per_step']:.4f} ms/step, stages {rg['stages_ms']}")
        ach = achievable_peaks()
        out["ragged_decode"] = {
            "value": round(rg["value"], 1), "unit": "tokens/s",
            "ms_per_step": round(rg["ms_per_step"], 4),
            "step_ms_median": round(rg["step_ms_median"], 4),
            "step_ms_min": round(rg["step_ms_min"], 4),
            "config": {"workload": "ragged decode: 8 sequences, lengths log-uniform in "
                                   "[4096, 1048572] plus 1-3 tokens past a block boundary, "
                                   "near ties in half, budget 512 blocks + tail, MALL flushed "
                                   "before each step", "seq_lens": lens},
            # this draw's floor: its block keys and its rows' gathers at the HBM peak
            "floor_ms_at_hbm_peak": round(rg["hbm"]["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
            "floor_ms_at_achievable_read": (round(rg["hbm"]["bytes"] / (ach["hbm_read_gbs"] * 1e9)
                                                  * 1e3, 4) if "hbm_read_gbs" in ach else None),
            "roofline": {"bound": "hbm", "scope": "whole step",
                         "achieved": round(rg["hbm"]["gbs"], 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(rg["hbm"]["gbs"] / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": rg["hbm"]["bytes"]},
            "stages_ms": {k: round(v, 4) for k, v in rg["stages_ms"].items()}}
        rg = None
    dec = None
    torch.cuda.empty_cache()
    if args.only in (None, "mtp"):
        mt = time_decode(args, mtp=True)
        log(f"mtp decode: {mt['ms_per_step']:.4f} ms/step, stages {mt['stages_ms']}")
        m = {"value": round(mt["value"], 1), "unit": "tokens/s",
             "ms_per_step": round(mt["ms_per_step"], 4),
             "step_ms_median": round(mt["step_ms_median"], 4),
             "step_ms_min": round(mt["step_ms_min"], 4),
             "config": {"workload": "multi-token decode: 32 sequences x (131072 cached + 4 new) "
                                    "tokens, 4 query tokens each (a new token and 3 speculative), "
                                    "budget 512 blocks + tail, MALL flushed before each step"},
             "roofline": {"bound": "hbm", "scope": "whole step",
                          "achieved": round(mt["hbm"]["gbs"], 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(mt["hbm"]["gbs"] / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes": mt["hbm"]["bytes"]},
             "stages_ms": {k: round(v, 4) for k, v in mt["stages_ms"].items()}}
        if args.only == "mtp":
            out.update(value=m["value"], unit="tokens/s", ms_per_step=m["ms_per_step"],
                       config=m["config"], roofline=m["roofline"])
        else:
            out["mtp_decode"] = m
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
