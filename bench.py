"""Benchmark of the DSA sparse-attention path on one MI355X.

One step = the whole path over one batch: indexer scores -> top-k (fused into
one call without a score matrix for rows up to 65,536) -> sparse MLA partial
-> combine, with inputs resident in HBM.  Default workload: the
speculative-verify decode batch, 128 requests x 8 query tokens, 64K context
each, FP8 E4M3 latent KV (per-64 power-of-two scales) in 64-token pages, top-2048,
64 heads.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
  python bench.py --summarize-stats KERNEL_STATS_CSV COMMAND...      (rocprofv3 summary text)
  python bench.py --summarize-pmc FETCH_CSV WRITE_CSV WORKLOAD CMD... (traffic JSON)
  python bench.py --summarize-mfma COUNTER_CSV WORKLOAD CMD...        (MFMA-use JSON)
  python bench.py --summarize-lds COUNTER_CSV WORKLOAD CMD...         (LDS-use JSON)

With no flags the line also carries the 32K-token prefill chunk (Partial
against the bf16 MFMA peak, and the Q8 variant: FP8 query quantizer + Q8
attention on the same rows), the shared-prefix batch at KV tiles 32 / 64 /
128, and the box's measured copy bandwidth and bf16 GEMM rate.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

METRIC = "sparse-MLA query tokens/s + HBM GB/s % peak, 64K ctx top-2048, 64 heads"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, vendor figure
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA, vendor figure


def algorithmic_bytes(spec, plan, kv_row_bytes, fused=False):
    """Bytes each kernel must move at minimum, per launch (one step).  With one
    split (fused) Partial writes the bf16 output and lse itself; no Combine.
    The fused selection (index_topk) must read the keys and queries and write
    the indices; its samples and candidates are overhead, not counted."""
    T = spec.num_tokens
    k = spec.k
    S = plan.splits
    out_bytes = T * 64 * (512 * 2 + 4)
    keys = 0
    for L, q in zip(spec.ctx_lens, spec.q_per_req):
        # a request's visible keys are read once for all its query tokens
        keys += L * 256
    vis = sum(min(L, p + 1) for L, q in zip(spec.ctx_lens, spec.q_per_req)
              for p in range(L - q, L))
    d = {
        # keys + indexer queries/weights + visible score writes
        "index_scores": keys + T * (16 * 128 * 2 + 16 * 4) + vis * 4,
        # visible score reads + index writes
        "topk": vis * 4 + T * k * 4,
        # keys + indexer queries/weights + index writes
        "index_topk": keys + T * (16 * 128 * 2 + 16 * 4) + T * k * 4,
    }
    attend_in = T * k * 4 + T * k * kv_row_bytes + T * 64 * 576 * 2   # index, selected rows, q
    if fused:
        d["partial"] = attend_in + out_bytes
    else:
        d["partial"] = attend_in + T * S * 64 * (512 + 1) * 4          # split partials out
        d["combine"] = T * S * 64 * (512 + 1) * 4 + out_bytes          # split partials in
    return d


def time_kv_append(dsa, kv_dtype, dev, rows=32768, reps=20):
    """Writing `rows` new tokens (latent + indexer key) into a scratch pool of
    the workload's KV format: event time per call and algorithmic bytes."""
    pages = (rows + 63) // 64
    lay = dsa.pool_layout(kv_dtype, pages)
    buf = torch.zeros(lay.total_bytes, dtype=torch.uint8, device=dev)
    pool = dsa.Pool(buf, pages, kv_dtype)
    pt = torch.arange(pages, dtype=torch.int32, device=dev).view(1, pages)
    req = torch.zeros(rows, dtype=torch.int32, device=dev)
    pos = torch.arange(rows, dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev).manual_seed(5)
    lat = torch.randn((rows, 576), generator=g, device=dev).to(torch.bfloat16)
    keys = torch.randint(-8, 9, (rows, 128), generator=g, device=dev).to(torch.bfloat16)
    dsa.kv_append(pool, pt, req, pos, lat, keys)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dsa.kv_append(pool, pt, req, pos, lat, keys)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    out_row = (lay.latent_row_bytes if kv_dtype == dsa.KV_FP8 else 2 * 576) + 256
    alg = rows * (576 * 2 + 128 * 2 + 8 + out_row)
    pool.close()
    return {"rows": rows, "avg_us": round(us, 3), "alg_bytes": alg,
            "gbps": round(alg / (us * 1e-6) / 1e9, 1)}


def time_dcp(dsa, synth, wl, spec, dev, G=8, reps=10):
    """The DCP shard layout on one GPU: the batch as G round-robin KV shards.
    Times one rank's share at its real shape (its indexer + top-k over L/G
    positions, its partial over its share of the rows), the merge, the LSE
    combine, and the whole G-shard step run on this one GPU."""
    shards = synth.shard_round_robin(wl, G)
    views = [(dsa.Pool(sh.pool, sh.num_pages, spec.kv_dtype), sh.page_table, sh.tok_pos,
              sh.max_ctx) for sh in shards]
    path = dsa.DcpPath(views, wl.q_offsets, wl.max_q, spec.k, kv_tile=64, sm_scale=spec.sm_scale)
    stream = torch.cuda.current_stream(dev)
    path.step(wl.q_idx, wl.w, wl.q)
    torch.cuda.synchronize()
    calls = {"rank0_select": lambda: path.local_select(0, wl.q_idx, wl.w),
             "merge": path.merge,
             "rank0_attend": lambda: path.local_attend(0, wl.q),
             "combine": lambda: dsa.combine_shards(path.o_part, path.lse_part, path.out, path.lse),
             "all_shards_step": lambda: path.step(wl.q_idx, wl.w, wl.q)}
    res = {}
    for name, fn in calls.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_us"] = round(e0.elapsed_time(e1) * 1000.0 / reps, 2)
    for v in views:
        v[0].close()
    return {"shards": G, **res,
            "note": "one GPU holds all shards; a rank's share is rank0_select + rank0_attend, "
                    "the exchanges (all-gather of local top-k, reduce of partials) are not run"}


def flops(spec):
    T, k = spec.num_tokens, spec.k
    vis = sum(min(L, p + 1) for L, q in zip(spec.ctx_lens, spec.q_per_req)
              for p in range(L - q, L))
    return {"index_scores": vis * 16 * 128 * 2, "index_topk": vis * 16 * 128 * 2,
            "partial": T * 64 * k * (576 + 512) * 2}


def cpu_baseline(wl, budget_s=15.0, max_tokens=512):
    """The oracle, as written, on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dsa_oracle as O
    from tests._harness import HostView

    s = wl.spec
    tok_req = wl.tok_req.cpu().numpy()
    order = list(range(s.num_tokens))
    # sample whole requests from the front of the batch
    reqs = sorted(set(int(tok_req[t]) for t in order[:max_tokens]))
    hv = HostView(wl, reqs=reqs)
    done = 0
    t0 = time.perf_counter()
    for t in order[:max_tokens]:
        hv.token(t, 64, 1)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = 1
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 1)))
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": done / dt, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
            "parallelism": f"one process, tokens one after another; numpy's BLAS uses {threads} "
                           f"thread(s) inside each matrix product",
            "sample": f"{done} query tokens of {s.name} (requests {reqs[0]}..{reqs[-1]}), "
                      f"full per-token path (indexer over the whole context, top-k, attention, "
                      f"combine) in float64 numpy; {dt:.1f} s",
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model}


# rocprofv3 kernel names (mangled or demangled) -> path step.  The fused
# selection (index_topk) is five launches: sample pass, threshold, emit pass,
# select, fallback.
KERNEL_PATTERNS = [
    ("dcp_merge", r"dcp_merge_kernel"),
    ("index_scores", r"index_kernel(ILi0E|<0[,>])"), ("index_sample", r"index_kernel(ILi1E|<1[,>])"),
    ("index_emit", r"index_kernel(ILi2E|<2[,>])"), ("threshold", r"threshold_kernel"),
    ("select", r"select_kernel"), ("fallback", r"fallback_kernel"), ("topk", r"topk_kernel"),
    ("partial_q8", r"partial_q8_kernel"), ("quantize_q8", r"quantize_q8_kernel"),
    ("partial", r"partial"), ("combine", r"combine_kernel")]
FUSED_SELECT = ("index_sample", "threshold", "index_emit", "select", "fallback")
KERNEL_SOURCES = {"index_scores": ("dsa_index.hip",), "topk": ("dsa_topk.hip",),
                  "index_topk": ("dsa_index.hip", "dsa_topk.hip"),
                  "partial": ("dsa_partial.hip",), "combine": ("dsa_partial.hip",),
                  "partial_q8": ("dsa_partial.hip",), "quantize_q8": ("dsa_append.hip",),
                  "dcp_merge": ("dsa_topk.hip",)}
for _k in FUSED_SELECT:
    KERNEL_SOURCES[_k] = KERNEL_SOURCES["index_topk"]
CALIB_BYTES = 1 << 30          # the calibration copy reads and writes 1 GiB


def source_sha(kernel: str) -> str:
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ("dsa_device.h",):
        with open(os.path.join(root, "sparse_attention_09_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _kernel_of(name: str):
    import re
    for k, pat in KERNEL_PATTERNS:
        if re.search(pat, name):
            return k
    return None


def summarize_stats(csv_path: str, command: str) -> str:
    """Text summary of a rocprofv3 --stats kernel table."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", "#",
             f"{'kernel':14s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}  name"]
    fused = {}
    for r in rows:
        k = _kernel_of(r["Name"])
        if k is None:
            continue
        lines.append(f"{k:14s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}  {r['Name'][:90]}")
        if k in FUSED_SELECT:
            fused[k] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3)
    if fused:
        # one fused selection call = one launch of each of its kernels
        calls = max(c for c, _ in fused.values())
        lines.append(f"{'index_topk':14s} {calls:6d} {sum(a for _, a in fused.values()):10.2f} "
                     f"{'':>10s} {'':>10s}  sum of the averages of: {', '.join(sorted(fused))}")
    return "\n".join(lines) + "\n"


def summarize_pmc(fetch_csv: str, write_csv: str, workload: str, commands: list) -> dict:
    """Per-launch HBM traffic of each path kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), scaled by what the same counters read for a copy of
    known size (1 GiB read + 1 GiB written by an elementwise negation)."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals, calib = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "neg" in r["Kernel_Name"].lower():
                calib.append(v)
                continue
            k = _kernel_of(r["Kernel_Name"])
            if k is not None:
                vals.setdefault(k, []).append(v)
        return {k: statistics.median(v) for k, v in vals.items()}, statistics.median(calib)

    fetch, cf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, cw = per_kernel(write_csv, "WRITE_SIZE")
    f_fetch = CALIB_BYTES / (cf * 1024.0)
    f_write = CALIB_BYTES / (cw * 1024.0)
    out = {"workload": workload, "commands": commands,
           "calibration": {"bytes_read": CALIB_BYTES, "bytes_written": CALIB_BYTES,
                           "fetch_kib": cf, "write_kib": cw, "factor_fetch": f_fetch,
                           "factor_write": f_write},
           "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        fb = fetch.get(k, 0.0) * 1024.0 * f_fetch
        wb = write.get(k, 0.0) * 1024.0 * f_write
        out["kernels"][k] = {"fetch_kib": fetch.get(k), "write_kib": write.get(k),
                             "read_bytes": int(fb), "write_bytes": int(wb),
                             "traffic_bytes": int(fb + wb), "source_sha": source_sha(k)}
    parts = [k for k in FUSED_SELECT if k in out["kernels"]]
    if parts:
        # one fused selection call = one launch of each of its kernels
        rb = sum(out["kernels"][k]["read_bytes"] for k in parts)
        wb = sum(out["kernels"][k]["write_bytes"] for k in parts)
        out["kernels"]["index_topk"] = {"parts": parts, "read_bytes": rb, "write_bytes": wb,
                                        "traffic_bytes": rb + wb,
                                        "source_sha": source_sha("index_topk")}
    return out


MOPS_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4")


def summarize_mfma(csv_path: str, workload: str, commands: list) -> dict:
    """Matrix-core use of each path kernel from a rocprofv3 counter run with
    SQ_INSTS_VALU_MFMA_MOPS_{BF16,F8,F6F4} (units of 512 FLOPs; those the run
    collected), SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs), GRBM_GUI_ACTIVE
    (summed over the 8 XCDs) and, optionally, the derived MfmaUtil (per cent).
    Per launch: the counted MFMA TFLOP/s over the dispatch's own duration (per
    type and in total), and the share of SIMD cycles the matrix pipe was busy."""
    import csv
    import statistics
    per = {}
    for r in csv.DictReader(open(csv_path)):
        k = _kernel_of(r["Kernel_Name"])
        if k is None:
            continue
        d = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    simds = 256 * 4
    out = {"workload": workload, "commands": commands,
           "counters": "SQ_INSTS_VALU_MFMA_MOPS_{BF16,F8,F6F4} x 512 FLOPs; SQ_VALU_MFMA_BUSY_CYCLES / "
                       "(GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); MfmaUtil as rocprofv3 derives it",
           "kernels": {}}
    for k, ds in per.items():
        rows = list(ds.values())
        e = {"dispatches": len(rows), "source_sha": source_sha(k)}
        have = [c for c in MOPS_COUNTERS if any(c in r for r in rows)]
        if have:
            mops = [sum(r.get(c, 0.0) for c in have) for r in rows]
            ns = [r["_ns"] for r in rows]
            e["mfma_tflops_counted"] = round(statistics.median(
                m * 512 / (t * 1e-9) / 1e12 for m, t in zip(mops, ns)), 1)
            e["mfma_flops_counted"] = int(statistics.median(m * 512 for m in mops))
            if len(have) > 1:
                e["mfma_flops_by_type"] = {c.rsplit("_", 1)[1]: int(statistics.median(
                    r.get(c, 0.0) * 512 for r in rows)) for c in have}
        busy = [r["SQ_VALU_MFMA_BUSY_CYCLES"] / (r["GRBM_GUI_ACTIVE"] / 8 * simds)
                for r in rows if "SQ_VALU_MFMA_BUSY_CYCLES" in r and r.get("GRBM_GUI_ACTIVE")]
        if busy:
            e["busy_cycles_frac"] = round(statistics.median(busy), 4)
        util = [r["MfmaUtil"] for r in rows if "MfmaUtil" in r]
        if util:
            e["mfma_util"] = round(statistics.median(util) / 100.0, 4)
        elif busy:
            e["mfma_util"] = e["busy_cycles_frac"]
        out["kernels"][k] = e
    parts = [k for k in FUSED_SELECT if k in out["kernels"]]
    if parts:
        # the fused selection: its five launches together
        fl = sum(out["kernels"][k].get("mfma_flops_counted", 0) for k in parts)
        out["kernels"]["index_topk"] = {"parts": parts, "mfma_flops_counted": fl,
                                        "mfma_util": out["kernels"].get("index_emit", {}).get("mfma_util"),
                                        "note": "mfma_util of the emit pass, which does all but 1/32 of the MFMA work",
                                        "source_sha": source_sha("index_topk")}
    return out


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    import json as _json
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    d = _json.load(open(path)).get("kernels", {}).get(kernel)
    if not d or d.get("source_sha") != source_sha(kernel):
        return None
    return d["traffic_bytes"]


FLUSH_BYTES = 1 << 30           # read between timed steps: evicts L2 and the 256 MB MALL


def make_flush(dev):
    """A read of 1 GiB (a sum): it replaces the caches' contents with clean
    lines, so the next step starts cold without paying for write-backs (a
    1 GiB fill measured ~60 us of dirty-line write-back in the next kernel)."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    acc = torch.empty((), dtype=torch.float32, device=dev)

    def flush(i):
        torch.sum(buf, dim=0, out=acc)
    return flush


def time_steps(calls, names, steps, stream, flush=None):
    """`steps` steps of the calls in order on `stream`.  Before each step the
    cache-flush write runs, outside the events; each call is bracketed by
    events.  Returns the per-step times (ms) and each call's mean duration
    (us) over the same steps."""
    import statistics
    n = len(calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush(i)
        ev[i][0].record(stream)
        for j, c in enumerate(calls):
            c()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [ev[i][0].elapsed_time(ev[i][n]) for i in range(steps)]
    per_us = {nm: 1000.0 * statistics.mean(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps))
              for j, nm in enumerate(names)}
    return step_ms, per_us


def measure_peaks(dsa, dev, reps=10):
    """The box's own denominators: a 1 GiB device copy (GB/s, read + write),
    a 2 GiB read (the library's read probe: the bound of a kernel that mostly
    reads) and an 8192^3 bf16 GEMM through torch (TFLOP/s, dense MFMA)."""
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * 4 * a.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    r = torch.ones(1 << 29, dtype=torch.int32, device=dev)
    words = torch.empty(2048, dtype=torch.int32, device=dev)
    dsa.read_probe(r, words)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dsa.read_probe(r, words)
    e1.record()
    torch.cuda.synchronize()
    read_gbps = 4 * r.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del r, words
    n = 8192
    g = torch.Generator(device=dev).manual_seed(1)
    x = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    y = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    z = x @ y
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        z = torch.matmul(x, y, out=z)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return {"copy_gbps": round(copy_gbps, 1), "read_gbps": round(read_gbps, 1),
            "bf16_gemm_tflops": round(gemm_tflops, 1),
            "copy": "1 GiB device-to-device copy (bytes read + written)",
            "read": "2 GiB read once by dsa_read_probe (2048 workgroups, 16-byte loads)",
            "gemm": "8192 x 8192 x 8192 bf16 torch.matmul"}


def setup_path(dsa, synth, name, dev, cus, tile=0, splits=0, select="auto", seed=0):
    spec = synth.spec(name)
    print(f"[bench] generating {spec.name} seed={seed}", file=sys.stderr, flush=True)
    wl = synth.generate(spec, seed=seed, device=dev)
    torch.cuda.synchronize()
    pool = dsa.Pool(wl.pool, wl.num_pages, spec.kv_dtype)
    path = dsa.DsaPath(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.max_q, wl.max_ctx, spec.k,
                       kv_tile=tile, num_splits=splits, sm_scale=spec.sm_scale, cu_count=cus,
                       select=select)
    # one step = these calls in order (what DsaPath.step runs)
    if path.fused_topk:
        names = ["index_topk"]
        calls = [lambda: path.index_topk(wl.q_idx, wl.w)]
    else:
        names = ["index_scores", "topk"]
        calls = [lambda: path.index_scores(wl.q_idx, wl.w), path.topk]
    if path.fused:
        names += ["partial"]
        calls += [lambda: path.attend(wl.q)]
    else:
        names += ["partial", "combine"]
        calls += [lambda: path.partial(wl.q), path.combine]
    return spec, wl, pool, path, names, calls


def mfma_counters(workload: str, kernel: str):
    """MFMA utilisation of a kernel from the committed rocprofv3 counter
    summary (profiles/<workload>_mfma.json), or None when absent or taken on
    other kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"{workload}_mfma.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path)).get("kernels", {}).get(kernel)
    if not d or d.get("source_sha") != source_sha(kernel):
        return None
    return {k: d[k] for k in ("mfma_util", "mfma_tflops_counted", "busy_cycles_frac",
                              "mfma_flops_by_type") if k in d}


def bench_prefill(dsa, synth, dev, cus, flush, peaks, steps=5, warmup=2):
    """The 32K-token prefill chunk: Partial against the bf16 MFMA peak."""
    import statistics
    spec, wl, pool, path, names, calls = setup_path(dsa, synth, "prefill_fp8_32k", dev, cus)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        path.step(wl.q_idx, wl.w, wl.q)
    step_ms, per_us = time_steps(calls, names, steps, stream, flush)
    fl = flops(spec)
    kern = {}
    for n in names:
        d = {"avg_us": round(per_us[n], 1)}
        if n in fl:
            tf = fl[n] / (per_us[n] * 1e-6) / 1e12
            d.update({"tflops": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        kern[n] = d
    med = statistics.median(step_ms)
    tf = kern["partial"]["tflops"]
    out = {"workload": spec.name, "query_tokens": spec.num_tokens, "steps": steps,
           "ms_per_step": round(med, 3), "query_tokens_per_s": round(spec.num_tokens / (med * 1e-3), 1),
           "kv_tile": path.plan.tile, "kernels": kern,
           "roofline": {"kernel": "partial", "bound": "mfma", "achieved": tf,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                        "measured_peak": peaks["bf16_gemm_tflops"],
                        "frac_of_measured": round(tf / peaks["bf16_gemm_tflops"], 4),
                        "flops_per_launch": int(fl["partial"]),
                        "counters": mfma_counters(spec.name, "partial")},
           "fallback_tokens": path.fallback_count()}
    out["q8"] = bench_q8(dsa, spec, wl, pool, path, stream, flush, steps, fl["partial"])
    pool.close()
    del wl, path, pool
    torch.cuda.empty_cache()
    return out


def bench_q8(dsa, spec, wl, pool, path, stream, flush, steps, flops_partial):
    """Q8 on the same chunk and the same selected rows: the query quantizer and
    the Q8 attention (FP8 query x FP8 rows on the f8f6f4 MFMA, bf16 PV).  The
    roof of the attention is its mixed peak: the score's FLOPs at the FP8
    peak plus the value product's at the bf16 peak."""
    import statistics
    T = spec.num_tokens
    codes = torch.empty((T, 64, 576), dtype=torch.uint8, device=wl.q.device)
    scales = torch.empty((T, 64), dtype=torch.float32, device=wl.q.device)
    out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device=wl.q.device)
    lse = torch.empty((T, 64), dtype=torch.float32, device=wl.q.device)
    calls = [lambda: dsa.quantize_q8(wl.q, codes, scales),
             lambda: dsa.sparse_mla_q8(pool, wl.page_table, wl.q_offsets, wl.tok_pos, codes, scales,
                                       path.idx, spec.sm_scale, out, lse)]
    names = ["quantize_q8", "partial_q8"]
    for _ in range(2):
        for c in calls:
            c()
    step_ms, per_us = time_steps(calls, names, steps, stream, flush)
    qk = T * 64 * spec.k * 576 * 2
    pv = T * 64 * spec.k * 512 * 2
    mixed_peak = (qk + pv) / (qk / FP8_PEAK_TFLOPS + pv / BF16_PEAK_TFLOPS)
    tf = flops_partial / (per_us["partial_q8"] * 1e-6) / 1e12
    qbytes = T * 64 * (576 * 2 + 576 + 4)
    return {"ms_per_step": round(statistics.median(step_ms), 3),
            "quantize_q8": {"avg_us": round(per_us["quantize_q8"], 1),
                            "gbps": round(qbytes / (per_us["quantize_q8"] * 1e-6) / 1e9, 1)},
            "partial_q8": {"avg_us": round(per_us["partial_q8"], 1), "tflops": round(tf, 1),
                           "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                           "mixed_peak_tflops": round(mixed_peak, 1),
                           "frac_of_mixed_peak": round(tf / mixed_peak, 4),
                           "counters": mfma_counters(spec.name, "partial_q8")},
            "note": "same selected rows as the bf16 Partial above; FLOPs counted as for it"}


def bench_shared_prefix(dsa, synth, dev, cus, flush, steps=7, warmup=10, rounds=5,
                        tiles=(32, 64, 128)):
    """132 requests sharing a 63,488-token prefix: Partial at KV tiles 32, 64
    and 128 (one split each) on the same selected indices, timed in
    interleaved rounds (each tile's figure is the median of its round
    medians).  Logical bytes are the rows as gathered; unique bytes count each
    physical row once (the shared rows come from the caches, so HBM sees
    about the unique bytes)."""
    import statistics
    spec, wl, pool, path, _, _ = setup_path(dsa, synth, "shared_prefix_fp8", dev, cus)
    stream = torch.cuda.current_stream(dev)
    path.select(wl.q_idx, wl.w)
    torch.cuda.synchronize()
    T, k = spec.num_tokens, spec.k
    idx = path.idx.to(torch.int64)
    req = wl.tok_req.to(torch.int64)[:, None].expand_as(idx)
    phys = wl.page_table.to(torch.int64)[req, torch.clamp(idx, min=0) // 64] * 64 + idx % 64
    uniq_rows = int(torch.unique(phys[idx >= 0]).numel())
    lay = dsa.pool_layout(spec.kv_dtype, 1)
    fixed = T * k * 4 + T * 64 * 576 * 2 + T * 64 * (512 * 2 + 4)     # idx, q, output
    logical = fixed + T * k * lay.latent_row_bytes
    unique = fixed + uniq_rows * lay.latent_row_bytes
    calls = {}
    for tile in tiles:
        out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, 64), dtype=torch.float32, device=dev)

        def call(tile=tile, out=out, lse=lse):
            dsa.sparse_mla(pool, wl.page_table, wl.q_offsets, wl.tok_pos, wl.q, path.idx,
                           spec.sm_scale, tile, out, lse)
        calls[tile] = call
        for _ in range(warmup):
            call()
    # the tiles take turns, round after round, so that drift over the run
    # (a fresh process runs its first kernels slower) reaches every tile alike
    per_round = {tile: [] for tile in tiles}
    for _ in range(rounds):
        for tile in tiles:
            step_ms, _ = time_steps([calls[tile]], ["partial"], steps, stream, flush)
            per_round[tile].append(statistics.median(step_ms))
    res = {}
    for tile in tiles:
        us = 1000.0 * statistics.median(per_round[tile])
        res[str(tile)] = {"avg_us": round(us, 1),
                          "logical_gbps": round(logical / (us * 1e-6) / 1e9, 1),
                          "unique_gbps": round(unique / (us * 1e-6) / 1e9, 1),
                          "rounds_us": [round(1000.0 * x, 1) for x in per_round[tile]]}
    out = {"workload": spec.name, "query_tokens": T, "splits": 1, "partial_by_tile": res,
           "logical_bytes": int(logical), "unique_bytes": int(unique), "unique_rows": uniq_rows,
           "tile128_speedup_over_tile32": round(res["32"]["avg_us"] / res["128"]["avg_us"], 3),
           "timing": f"{rounds} interleaved rounds of {steps} cache-flushed steps per tile; median "
                     f"of the round medians",
           "note": "one split per token; tiles 32 and 128 run the same kernel (a 128-column tile "
                   "streams through LDS as four 32-row steps); the pages report Partial + Combine at KV tile 128 about "
                   "1.12x faster than at tile 32 on H200 (context, other hardware)"}
    pool.close()
    del wl, path, pool
    torch.cuda.empty_cache()
    return out


def summarize_lds(csv_path: str, workload: str, commands: list) -> dict:
    """LDS use of each path kernel from a rocprofv3 counter run with
    SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE (cycles, summed over the CUs),
    SQ_INSTS_LDS and SQ_WAIT_INST_LDS (wave quad-cycles waiting to issue an LDS
    instruction): per launch (median over dispatches), and the share of
    LDS-active cycles lost to bank conflicts."""
    import csv
    import statistics
    per = {}
    for r in csv.DictReader(open(csv_path)):
        k = _kernel_of(r["Kernel_Name"])
        if k is None:
            continue
        d = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    out = {"workload": workload, "commands": commands,
           "counters": "SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_INSTS_LDS, SQ_WAIT_INST_LDS "
                       "per launch (median over dispatches); conflict_frac = conflict / active cycles",
           "kernels": {}}
    for k, ds in per.items():
        rows = list(ds.values())
        e = {"dispatches": len(rows), "source_sha": source_sha(k)}
        for c in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS"):
            vals = [r[c] for r in rows if c in r]
            if vals:
                e[c] = int(statistics.median(vals))
        if e.get("SQ_LDS_IDX_ACTIVE"):
            e["conflict_frac"] = round(e.get("SQ_LDS_BANK_CONFLICT", 0) / e["SQ_LDS_IDX_ACTIVE"], 4)
        out["kernels"][k] = e
    return out


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-lds":
        csv_path, workload = sys.argv[2:4]
        print(json.dumps(summarize_lds(csv_path, workload, sys.argv[4:]), indent=1))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-stats":
        print(summarize_stats(sys.argv[2], " ".join(sys.argv[3:])), end="")
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        fetch_csv, write_csv, workload = sys.argv[2:5]
        print(json.dumps(summarize_pmc(fetch_csv, write_csv, workload, sys.argv[5:]), indent=1))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-mfma":
        csv_path, workload = sys.argv[2:4]
        print(json.dumps(summarize_mfma(csv_path, workload, sys.argv[4:]), indent=1))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="verify_fp8_64k")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--select", default="auto", choices=["auto", "fused", "scores"],
                    help="top-k selection: fused indexer + top-k (auto: rows up to 65,536) "
                         "or the score matrix + top-k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dcp", action="store_true", help="skip the DCP shard-layout timing")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing a HIP graph replay of the step")
    ap.add_argument("--no-flush", action="store_true",
                    help="time back-to-back steps without the cache flush between them")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the prefill and shared-prefix entries and the measured peaks")
    ap.add_argument("--q8", action="store_true",
                    help="also time the Q8 variant (query quantizer + Q8 attention) on the "
                         "workload's selected rows (FP8 pools)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a 1 GiB read + 1 GiB write elementwise copy "
                         "(reference dispatch for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from sparse_attention_09_amd import dsa, synth
    import statistics

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    spec, wl, pool, path, names, calls = setup_path(dsa, synth, args.workload, dev, cus, args.tile,
                                                    args.splits, args.select, args.seed)
    plan = path.plan
    print(f"[bench] plan tile={plan.tile} splits={plan.splits} cus={cus} "
          f"selection={'fused' if path.fused_topk else 'scores+topk'}", file=sys.stderr, flush=True)
    flush = None if args.no_flush else make_flush(dev)

    def step():
        path.step(wl.q_idx, wl.w, wl.q)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps, each preceded by the cache flush (outside the
    # events), with an event on the working stream before the first call and
    # after every call: the step time and each kernel's average launch
    # duration come from the same K steps.
    stream = torch.cuda.current_stream(dev)
    step_ms, per_us = time_steps(calls, names, args.steps, stream, flush)
    ms_step = statistics.median(step_ms)
    print(f"[bench] {args.steps} steps, median {ms_step:.4f} ms/step", file=sys.stderr, flush=True)

    # the same K steps back to back, no flush and no markers between calls
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_plain = e0.elapsed_time(e1) / args.steps
    ms_graph = None
    if not args.no_graph:
        # the same step recorded once on a HIP graph and replayed (no host
        # launch per kernel); every buffer is preallocated
        replay = path.capture(wl.q_idx, wl.w, wl.q)
        for _ in range(max(1, args.warmup // 4)):
            replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_graph = e0.elapsed_time(e1) / args.steps

    fallback_tokens = path.fallback_count()
    unfused = None
    if path.fused_topk:
        # the same selection through the score matrix, for comparison (not in the step)
        path.index_scores(wl.q_idx, wl.w)
        path.topk()
        torch.cuda.synchronize()
        _, u = time_steps([lambda: path.index_scores(wl.q_idx, wl.w), path.topk],
                          ["index_scores", "topk"], args.steps, stream, flush)
        unfused = {n: round(v, 3) for n, v in u.items()}
        path.scores = path.workspace = None
        torch.cuda.empty_cache()

    lay = dsa.pool_layout(spec.kv_dtype, 1)
    byts = algorithmic_bytes(spec, plan, lay.latent_row_bytes, path.fused)
    fl = flops(spec)
    kernels = {}
    for n in names:
        d = {"avg_us": round(per_us[n], 3), "alg_bytes": int(byts[n]),
             "gbps": round(byts[n] / (per_us[n] * 1e-6) / 1e9, 1)}
        if n in fl:
            d["tflops"] = round(fl[n] / (per_us[n] * 1e-6) / 1e12, 2)
        kernels[n] = d
    dom = max(names, key=lambda n: per_us[n])
    path_bytes = sum(byts[n] for n in names)     # the calls the step makes
    path_gbps = path_bytes / (ms_step * 1e-3) / 1e9
    T = spec.num_tokens
    value = T / (ms_step * 1e-3)
    peaks = None if args.no_extra else measure_peaks(dsa, dev)
    # the decode batches are bound by HBM: the roof of the dominant kernel is
    # its algorithmic bytes over the HBM peak (also given against the box's
    # measured copy bandwidth)
    roof = {"kernel": dom, "bound": "hbm", "achieved": kernels[dom]["gbps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(kernels[dom]["gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(spec.name, dom),
            "alg_bytes_per_launch": int(byts[dom]), "avg_us": kernels[dom]["avg_us"]}
    if peaks:
        # the selection and the attention mostly read: the box's read rate is
        # their measured ceiling (its copy rate is lower and also reported)
        roof["measured_peak"] = peaks["read_gbps"]
        roof["frac_of_measured"] = round(kernels[dom]["gbps"] / peaks["read_gbps"], 4)
        roof["frac_of_measured_copy"] = round(kernels[dom]["gbps"] / peaks["copy_gbps"], 4)
    for n in names:
        kernels[n]["traffic_bytes"] = measured_traffic(spec.name, n)
        if n in ("partial", "index_topk"):
            kernels[n]["mfma_counters"] = mfma_counters(spec.name, n)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "requests": spec.num_reqs, "query_tokens": T,
                   "context": int(max(spec.ctx_lens)), "top_k": spec.k, "heads": 64,
                   "kv": "fp8_e4m3_s64" if spec.kv_dtype == dsa.KV_FP8 else "bf16",
                   "kv_tile": plan.tile, "splits": plan.splits,
                   "combine": "in partial (one split)" if path.fused else "separate kernel",
                   "selection": "fused indexer + top-k" if path.fused_topk
                   else "score matrix + top-k",
                   "launch": "eager calls on one stream"},
        "timing": {"statistic": "median over the timed steps",
                   "cache_flush": None if flush is None else "1 GiB read before each step, outside the events",
                   "ms_min": round(min(step_ms), 4), "ms_mean": round(statistics.mean(step_ms), 4),
                   "kernel_avg": "mean launch duration over the same steps"},
        "ms_per_step_back_to_back": round(ms_plain, 4),
        "ms_per_step_graph_replay": None if ms_graph is None else round(ms_graph, 4),
        "hbm": {"path_alg_bytes": int(path_bytes), "gbps": round(path_gbps, 1),
                "frac": round(path_gbps / HBM_PEAK_GBPS, 4)},
        "kernels": kernels,
        "roofline": roof,
        "measured_peaks": peaks,
    }
    if path.fused_topk:
        result["fused_select"] = {"fallback_tokens": fallback_tokens, "cap": path.cap,
                                  "unfused_us": unfused}
    if args.q8 and spec.kv_dtype == dsa.KV_FP8:
        result["q8"] = bench_q8(dsa, spec, wl, pool, path, stream, flush, args.steps, fl["partial"])
    result["kv_append"] = time_kv_append(dsa, spec.kv_dtype, dev)
    if not args.no_dcp and spec.num_tokens * spec.k <= (1 << 22):
        print("[bench] DCP shard layout", file=sys.stderr, flush=True)
        result["dcp"] = time_dcp(dsa, synth, wl, spec, dev)
    if args.calibrate_copy:
        a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)
    result["cpu_baseline"] = cpu
    if not args.no_extra and spec.name == "verify_fp8_64k":
        pool.close()
        del wl, path, pool, calls
        torch.cuda.empty_cache()
        print("[bench] prefill chunk", file=sys.stderr, flush=True)
        result["prefill"] = bench_prefill(dsa, synth, dev, cus, flush, peaks)
        print("[bench] shared-prefix tiles", file=sys.stderr, flush=True)
        result["shared_prefix"] = bench_shared_prefix(dsa, synth, dev, cus, flush)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
