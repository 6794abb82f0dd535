"""HBM traffic of the hot-path kernels from rocprofv3 counters.

Two counter runs of the same program give per-dispatch FETCH_SIZE and
WRITE_SIZE (KiB moved between L2 and memory).  The program first runs a plain
copy of known size (read 1 GiB, write 1 GiB) whose counters calibrate both:
factor = known bytes / counted bytes.  Then one step of each workload:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D1 -o run -- \\
        python3 -m block_sparse_long_02_amd.measure probe
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D2 -o run -- \\
        python3 -m block_sparse_long_02_amd.measure probe
    python3 -m block_sparse_long_02_amd.measure summarize D1/run_counter_collection.csv \\
        D2/run_counter_collection.csv profiles/traffic.json

`summarize` writes, per kernel, the calibrated bytes per launch and the hash
of the source file the kernel was built from, so that a reader (bench.py)
uses the figures only while that source is unchanged.

    python3 -m block_sparse_long_02_amd.measure peaks OUT_JSON

times the micro-benchmarks of libqsa_probe.so (built on request with
`python3 -m block_sparse_long_02_amd.build probe`): the sustained rate of the
16x16x32 bf16 MFMA and the sustained HBM read and copy bandwidth, beside the
published peaks the roofline fractions use.

    python3 -m block_sparse_long_02_amd.measure stats TRACE_CSV OUT_MD STEPS WARMUP

summarizes a `rocprofv3 --kernel-trace` run of bench.py: for the hot kernels
of the headline prefill step, the mean duration over the timed steps (the
first WARMUP + STEPS dispatches of the kernel at its first grid size, the
last STEPS of them), and every kernel of this path by (name, grid size).

    python3 -m block_sparse_long_02_amd.measure pmc OUT_MD CSV [CSV ...]

turns counter runs of the same program (any SQ counters, e.g. the MFMA
pipe's busy cycles) into a per-kernel table: each counter's value per
dispatch and the utilisation ratios derived from them.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30

# key -> (substring of the kernel name, source file, which dispatch of that
# kernel: an index in dispatch order, or None for the mean of all).  Pooling
# runs three times: the prefill runner pools its cached prefix, the prefill
# step pools the chunk's new blocks, the decode runner pools its prefix (a
# decode step of 131,073 tokens completes no new block).  The transformed
# pooling runs twice (prefix, then the step's new blocks).  The prefill
# kernels run twice, in the plain step (dispatch 0) and in the step with the
# indexer transforms (dispatch 1), which selects other blocks.
KERNELS = {
    "pool_block_keys_prefill_1m": ("pool_block_keys_kernel", "qsa_pool.hip", 1),
    "score_sample_prefill_1m": ("score_gemm_kernel<2, 4, true, false>", "qsa_index.hip", 0),
    "threshold_prefill_1m": ("threshold_kernel", "qsa_index.hip", 0),
    "score_filter_prefill_1m": ("score_gemm_kernel<2, 8, false, false>", "qsa_index.hip", 0),
    "final_select_prefill_1m": ("final_select_kernel", "qsa_index.hip", 0),
    "attend_prefill_1m": ("attend_rows_kernel", "qsa_attend.hip", 0),
    "attend_prefill_1m_transformed": ("attend_rows_kernel", "qsa_attend.hip", 1),
    "score_dense_decode_128k": ("score_dense_kernel<false>", "qsa_index.hip", None),
    "select_dense_decode_128k": ("select_dense_kernel", "qsa_index.hip", None),
    "key_transform_prefill_1m": ("pool_block_keys_normed_kernel", "qsa_index_transform.hip", 1),
    "query_transform_prefill_1m": ("index_query_transform_kernel", "qsa_index_transform.hip", None),
    "attend_decode_128k": ("attend_split_kernel", "qsa_attend.hip", None),
    "combine_decode_128k": ("combine_kernel", "qsa_attend.hip", None),
}


def src_hash(name: str) -> str:
    path = os.path.join(_PKG, "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def probe():
    """The program the counter runs profile: copy, one prefill step (plain, then
    with the indexer transforms), one decode step."""
    import torch
    from . import workloads as W
    from .runner import QSARunner

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)          # the calibration copy: 1 GiB read, 1 GiB written
    torch.cuda.synchronize()
    del src, dst
    print("MARK copy done", flush=True)

    b = W.chunked_prefill_1m(device="cuda")
    r = QSARunner(b)
    torch.cuda.synchronize()
    print("MARK prefill step", flush=True)
    r.step()
    torch.cuda.synchronize()
    del r
    torch.cuda.empty_cache()
    r = QSARunner(b, transforms=True)
    torch.cuda.synchronize()
    print("MARK prefill step with indexer transforms", flush=True)
    r.step()
    torch.cuda.synchronize()
    del r, b
    torch.cuda.empty_cache()

    b = W.decode_128k(device="cuda")
    r = QSARunner(b)
    torch.cuda.synchronize()
    print("MARK decode step", flush=True)
    r.step()
    torch.cuda.synchronize()
    print("MARK done", flush=True)


def _dispatches(path: str, counter: str):
    """[(dispatch id, kernel name, value in KiB)] in dispatch order."""
    vals = {}
    for row in csv.DictReader(open(path)):
        if row.get("Counter_Name") != counter:
            continue
        key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
        vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return [(d, k, v) for (d, k), v in sorted(vals.items())]


def summarize(fetch_csv: str, write_csv: str, out_json: str):
    fetch = _dispatches(fetch_csv, "FETCH_SIZE")
    write = _dispatches(write_csv, "WRITE_SIZE")

    def find(d, sub, index=None):
        vs = [v for _, k, v in d if sub in k]
        return vs if index is None else vs[index:index + 1]

    copy_f = max(find(fetch, "neg_kernel"))       # the 1 GiB copy is the largest neg dispatch
    copy_w = max(find(write, "neg_kernel"))
    f_fac = COPY_BYTES / 1024.0 / copy_f
    w_fac = COPY_BYTES / 1024.0 / copy_w
    out = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_kib_counted": copy_f,
                           "write_kib_counted": copy_w, "fetch_factor": f_fac,
                           "write_factor": w_fac}}
    for key, (sub, src, index) in KERNELS.items():
        fv, wv = find(fetch, sub, index), find(write, sub, index)
        if not fv or not wv:
            continue
        fb = sum(fv) / len(fv) * 1024.0 * f_fac
        wb = sum(wv) / len(wv) * 1024.0 * w_fac
        out[key] = {"kernel": sub, "source": src, "source_sha": src_hash(src),
                    "launches": len(fv), "fetch_bytes_per_launch": round(fb),
                    "write_bytes_per_launch": round(wb), "bytes_per_launch": round(fb + wb)}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    for k, v in out.items():
        print(k, v)


def peaks(out_json: str):
    """Sustained MFMA and HBM rates from libqsa_probe.so, timed with HIP events."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(_PKG, "libqsa_probe.so"))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.qsa_probe_mfma_bf16.argtypes = [i32, i32, i32, vp, vp]
    lib.qsa_probe_read.argtypes = [vp, i64, i32, vp, vp]
    lib.qsa_probe_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.qsa_probe_gather.argtypes = [vp, i64, vp, i64, i32, i32, vp, vp]
    st = vp(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    props = torch.cuda.get_device_properties(0)
    n_cu = props.multi_processor_count

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return best

    res = {"device": props.name, "compute_units": n_cu}
    iters = 20000
    # 16 chains per wave: with fewer, the compiler rotates the loop-carried
    # accumulators through register moves and the loop measures those
    for chains in (16,):
        for wg_per_cu in (2, 8):
            n_wg = wg_per_cu * n_cu
            t = timed(lambda: lib.qsa_probe_mfma_bf16(n_wg, iters, chains, vp(sink.data_ptr()), st))
            flops = n_wg * 4 * iters * chains * 16384
            u = sink[:4].view(torch.int32).cpu().numpy().astype("int64") & 0xFFFFFFFF
            cyc, ticks = int(u[0] | (u[1] << 32)), int(u[2] | (u[3] << 32))
            ghz = cyc / (ticks / 100e6) / 1e9 if ticks else None
            res[f"mfma_bf16_16x16x32_{chains}chains_{wg_per_cu}wg"] = {
                "tflops": round(flops / t / 1e12, 1), "published_tflops": 2500.0,
                "shader_clock_ghz": round(ghz, 3) if ghz else None,
                "workgroups": n_wg, "seconds": t}
    nbytes = 4 << 30
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for wg_per_cu in (8, 32):
        n = wg_per_cu * n_cu
        t = timed(lambda: lib.qsa_probe_read(vp(a.data_ptr()), nbytes, n, vp(sink.data_ptr()), st))
        res[f"hbm_read_{wg_per_cu}wg"] = {"gbs": round(nbytes / t / 1e9, 1), "bytes": nbytes}
        t = timed(lambda: lib.qsa_probe_copy(vp(a.data_ptr()), vp(b.data_ptr()), nbytes, n, st))
        res[f"hbm_copy_{wg_per_cu}wg"] = {"gbs": round(2 * nbytes / t / 1e9, 1),
                                          "bytes_moved": 2 * nbytes}
    del a, b
    # gathers of fixed-size runs at random places in 8 GiB (32x the MALL),
    # 1 GiB per launch: the access pattern of the attention kernels (2 KB runs)
    gbytes = 8 << 30
    g = torch.ones(gbytes // 4, dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(7)
    for run in (256, 512, 1024, 2048, 4096, 8192, 16384):
        n_runs = (1 << 30) // run
        idx = torch.randperm(gbytes // run, generator=gen, device="cuda")[:n_runs].to(torch.int32)
        n = 8 * n_cu
        t = timed(lambda: lib.qsa_probe_gather(vp(g.data_ptr()), gbytes, vp(idx.data_ptr()), n_runs,
                                               run, n, vp(sink.data_ptr()), st))
        res[f"hbm_gather_{run}B_8wg"] = {"gbs": round((1 << 30) / t / 1e9, 1), "bytes": 1 << 30,
                                         "run_bytes": run}
        del idx
    res["published_hbm_gbs"] = 8000.0
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


HEADLINE = ["pool_block_keys_kernel", "score_gemm_kernel<2, 4, true, false>", "threshold_kernel",
            "score_gemm_kernel<2, 8, false, false>", "final_select_kernel", "attend_rows_kernel"]


def stats(trace_csv: str, out_md: str, steps: str, warmup: str):
    """Kernel durations of a bench.py kernel trace (see the module docstring)."""
    steps, warmup = int(steps), int(warmup)
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))

    def dur(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3   # us

    def grid(r):
        return (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]))

    # the headline step's boundaries: its first WARMUP + STEPS attention
    # launches at the chunk's full grid; step i runs from the end of
    # attention launch i - 1 to the end of attention launch i
    att = [r for r in rows if "attend_rows_kernel" in r["Kernel_Name"]]
    g0 = grid(att[0])
    ends = [int(r["End_Timestamp"]) for r in att if grid(r) == g0][:warmup + steps]
    windows = list(zip([0] + ends[:-1], ends))[warmup:]
    lines = ["| kernel | timed steps | mean us | min us | max us |", "|---|---|---|---|---|"]
    for sub in HEADLINE:
        d = []
        for lo, hi in windows:
            d += [dur(r) for r in rows if sub in r["Kernel_Name"]
                  and lo < int(r["Start_Timestamp"]) and int(r["End_Timestamp"]) <= hi]
        if d:
            lines.append(f"| `{sub}` | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    step = [(hi - lo) / 1e3 for lo, hi in windows[1:]]
    if step:
        lines.append(f"| (step, attention end to attention end) | {len(step)} | "
                     f"{sum(step) / len(step):.1f} | {min(step):.1f} | {max(step):.1f} |")
    lines += ["", "| kernel | grid (x, y) | dispatches | mean us | min us | max us |",
              "|---|---|---|---|---|---|"]
    groups = {}
    for r in rows:
        if "qsa::" not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        groups.setdefault((name, grid(r)), []).append(dur(r))
    for (name, g), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {g[0]}, {g[1]} | {len(d)} | {sum(d) / len(d):.1f} | "
                     f"{min(d):.1f} | {max(d):.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# utilisation ratios from SQ counters (all summed over the GPU's SIMDs or
# CUs): MFMA pipe busy cycles per SIMD-cycle, VALU issue (4 cycles per wave64
# instruction) per SIMD-cycle, and the shares of wave cycles spent waiting
# (on anything, on instruction dependencies) or issuing
SIMDS = 1024


def pmc(out_md: str, *csvs: str):
    """Per-kernel averages of every counter in the given counter runs, and
    the derived ratios, as a markdown table for the kernels of this path."""
    vals = {}
    for path in csvs:
        per = {}
        for row in csv.DictReader(open(path)):
            key = (int(row["Dispatch_Id"]), row["Kernel_Name"], row["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
        for (d, k, c), v in per.items():
            vals.setdefault(k, {}).setdefault(c, []).append(v)
    lines = []
    for k in sorted(vals):
        if "qsa::" not in k:
            continue
        name = k.split("(")[0].replace("void ", "")
        c = {n: sum(v) / len(v) for n, v in vals[k].items()}
        lines.append(f"### `{name}` ({max(len(v) for v in vals[k].values())} dispatches)")
        lines.append("")
        lines.append("| counter | per dispatch |")
        lines.append("|---|---|")
        for n in sorted(c):
            lines.append(f"| {n} | {c[n]:.4g} |")
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs: per-XCD cycles of the dispatch
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        derived = []
        if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            derived.append(("MFMA pipe busy (of SIMD cycles)", c["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / cyc))
        if cyc and "SQ_INSTS_VALU" in c:
            derived.append(("VALU issue (4 cycles per instruction, of SIMD cycles)",
                            4.0 * c["SQ_INSTS_VALU"] / SIMDS / cyc))
        if "SQ_INSTS_MFMA" in c and "SQ_INSTS_VALU" in c and c["SQ_INSTS_MFMA"]:
            derived.append(("VALU instructions per MFMA (MFMA included)", c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]))
        if "SQ_INSTS_MFMA" in c and "SQ_INSTS_LDS" in c and c["SQ_INSTS_MFMA"]:
            derived.append(("LDS instructions per MFMA", c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"]))
        # L2 (TCC counters summed over every channel of the 8 XCDs)
        hit, miss = c.get("TCC_HIT_sum"), c.get("TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss > 0:
            derived.append(("L2 hit rate (of L2 requests)", hit / (hit + miss)))
        lvl, rd = c.get("TCC_EA0_RDREQ_LEVEL_sum"), c.get("TCC_EA0_RDREQ_sum")
        if lvl is not None and rd:
            derived.append(("cycles a read beyond L2 waits, average", lvl / rd))
            if cyc:
                derived.append(("reads beyond L2 in flight, average over the dispatch", lvl / cyc))
        w = c.get("SQ_WAVE_CYCLES")
        if w:
            for n, label in (("SQ_WAIT_ANY", "wave cycles waiting on anything"),
                             ("SQ_WAIT_INST_ANY", "wave cycles waiting on dependencies"),
                             ("SQ_ACTIVE_INST_ANY", "wave cycles issuing")):
                if n in c:
                    derived.append((label, c[n] / w))
        if derived:
            lines.append("")
            lines.append("| derived | value |")
            lines.append("|---|---|")
            for label, v in derived:
                lines.append(f"| {label} | {v:.3f} |")
        lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if sys.argv[1:2] == ["probe"]:
        probe()
    elif sys.argv[1:2] == ["peaks"] and len(sys.argv) == 3:
        peaks(sys.argv[2])
    elif sys.argv[1:2] == ["summarize"] and len(sys.argv) == 5:
        summarize(*sys.argv[2:5])
    elif sys.argv[1:2] == ["pmc"] and len(sys.argv) >= 4:
        pmc(*sys.argv[2:])
    elif sys.argv[1:2] == ["stats"] and len(sys.argv) == 6:
        stats(*sys.argv[2:6])
    else:
        sys.exit("usage: measure.py probe | summarize FETCH_CSV WRITE_CSV OUT_JSON | peaks OUT_JSON"
                 " | pmc OUT_MD CSV [CSV ...] | stats TRACE_CSV OUT_MD STEPS WARMUP")
