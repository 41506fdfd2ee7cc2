"""Benchmark of the ragged-dot Group-GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME|all] [--no-cpu-baseline]

A step is one ragged-dot call over one batch of synthetic routed-token input already
resident in HBM (the whole hot path: group_sizes scan, tile schedule, MFMA main loop,
masked tails, epilogue -- one kernel launch).  The headline workload is the Mixtral-8x7B-
like FFN up-projection: 4096 tokens, top-2 of 8 experts (m = 8192 rows), k = 4096,
n = 14336, bf16 in / fp32 accumulate / bf16 out.  The timing protocol follows the pages'
micro-benchmark (10 warm-up runs, then timed runs; per-launch median and mean from HIP
events on the launch stream).

Prints one JSON line: useful TFLOP/s of the headline workload (2 * sum(group_sizes) * k * n
per step), the roofline of its kernel, the speedup over the capacity-padded baseline on the
same inputs, and the CPU oracle timed on a bounded sample of the same workload.  With the
default ``--workload all`` the line also carries ``per_config``: the same figures for each of
the five workloads (the 64-row fp32 one, the Mixtral-like bf16 forward, the DeepSeek-like
skewed forward, the Mixtral-like MXFP8 forward and the Llama-4-Scout-like weight gradient).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

# MI355X published peaks (dense, no sparsity)
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0

METRIC = "ragged-dot useful TFLOP/s + % MFMA/HBM roofline; speedup vs padded dot"
DEFAULT_WORKLOAD = "mixtral8x7b_up_bf16"
# the five workloads the benchmark reports together (the headline is the second)
PER_CONFIG = ["tiny_fp32", "mixtral8x7b_up_bf16", "deepseekv3_routed_bf16", "mixtral8x7b_up_mxfp8",
              "llama4scout_wgrad_bf16"]
PROFILE_TRAFFIC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    help="a workload name, or 'all' (the headline plus every entry of PER_CONFIG)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-padded", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 3 times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="no GPU work: read rocprofv3 --pmc outputs under DIR (fetch_<workload>, "
                         "write_<workload>, copy_fetch, copy_write) and record the HBM bytes per launch "
                         "of each workload's dominant kernel in profiles/traffic.json")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30, help="byte count the copy probe was run with")
    ap.add_argument("--library-context", action="store_true",
                    help="only time torch's own GEMMs (hipBLASLt) on the same inputs, for context: the "
                         "bf16 workloads as one matmul per group and as one dense matmul of the same flops")
    return ap.parse_args()


def algorithmic_bytes(w, gs):
    """Inputs read once (weights only of non-empty groups) plus the output written once."""
    esz = {"bf16": 2, "f32": 4, "mxfp8": 1}[w.in_dtype]
    osz = 4 if w.out_dtype == "f32" else 2
    if w.op == "permute":   # token rows and ids read once; sorted rows, both index maps, sizes written
        return w.tokens * w.k * esz + w.m * 4 + w.m * w.k * esz + 2 * w.m * 4 + w.g * 4
    if w.op == "unpermute":   # sorted rows, inverse order and weights read once; token rows written
        return w.m * w.n * esz + w.m * 4 + w.m * 4 + w.tokens * w.n * osz
    S = int(np.sum(gs))
    nonempty = int(np.sum(np.asarray(gs) > 0))
    if w.op in ("m", "m_nk", "m_gated"):
        b = w.m * w.k * esz + nonempty * w.k * w.n * esz * (2 if w.op == "m_gated" else 1) + w.m * w.n * osz
        if w.in_dtype == "mxfp8":
            b += w.m * (w.k // 32) + nonempty * (w.k // 32) * w.n
        return b
    return S * w.k * esz + S * w.n * esz + w.g * w.k * w.n * osz


def useful_flops(w, gs):
    if w.op == "permute":
        return 0.0
    if w.op == "unpermute":   # one multiply-add per element of every routed row
        return 2.0 * w.m * w.n
    return 2.0 * float(np.sum(gs)) * w.k * w.n * (2 if w.op == "m_gated" else 1)


def time_calls(fn, steps, warmup, torch):
    """Wall time of `steps` calls (after `warmup`), synchronised on both sides, and the
    per-launch times from a HIP event pair around every call, recorded on the launch
    stream (the library enqueues on torch's current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([e0.elapsed_time(e1) / 1e3 for e0, e1 in evs])
    return wall, per


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, d, gs, target_s, W, torch):
    """The oracle as it stands, on host cores, over a bounded sample of the workload's
    output rows (m-ragged) or (group, k-index) rows (k-ragged); rate in TFLOP/s."""
    import oracle
    raw = W.to_numpy_raw
    if w.op in ("permute", "unpermute"):
        return cpu_baseline_routing(w, d, target_s, raw, oracle)
    lhs = raw(d["lhs"])
    gsn = raw(d["group_sizes"])
    S = int(gsn.sum())
    rng = np.random.default_rng(0)
    if w.op == "m":
        rhs = raw(d["rhs"])
        ls = raw(d["lhs_scale"]) if "lhs_scale" in d else None
        rs = raw(d["rhs_scale"]) if "rhs_scale" in d else None
        per_unit = 2.0 * w.k * w.n
        run = lambda cnt: oracle.ragged_dot_m(lhs, rhs, gsn, ls, rs, rows=rng.integers(0, S, cnt))
        unit = "rows"
    elif w.op == "m_gated":
        w0, w1 = raw(d["w0"]), raw(d["w1"])
        per_unit = 4.0 * w.k * w.n
        run = lambda cnt: oracle.ragged_dot_m_gated(lhs, w0, w1, gsn, rows=rng.integers(0, S, cnt))
        unit = "rows"
    elif w.op == "m_nk":
        rhs_kn = np.ascontiguousarray(np.swapaxes(raw(d["rhs"]), 1, 2))   # once, outside the timed sample
        per_unit = 2.0 * w.k * w.n
        run = lambda cnt: oracle.ragged_dot_m(lhs, rhs_kn, gsn, rows=rng.integers(0, S, cnt))
        unit = "rows"
    else:
        dout = raw(d["dout"])
        nonempty = np.nonzero(gsn)[0]
        per_unit = 2.0 * float(np.mean(gsn[nonempty])) * w.n
        def run(cnt):
            pairs = np.stack([rng.choice(nonempty, cnt), rng.integers(0, w.k, cnt)], axis=1)
            return oracle.ragged_dot_k(lhs, dout, gsn, pairs=pairs)
        unit = "(group, k-index) output rows"
    cnt, spent, done, flops = 8, 0.0, 0, 0.0
    while spent < target_s:
        t0 = time.perf_counter()
        run(cnt)
        dt = time.perf_counter() - t0
        spent += dt
        done += cnt
        flops += cnt * per_unit
        if dt < target_s / 4:
            cnt *= 2
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(oracle.num_threads()), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} {unit} of the {w.name} workload drawn uniformly, fp64 oracle, {spent:.1f} s"}


def cpu_whole_call(w, d, W, threads):
    """The oracle's whole call on a workload small enough to finish in milliseconds, at a
    given thread count; seconds per call (median of repeated calls over ~1 s)."""
    import oracle
    raw = W.to_numpy_raw
    lhs, rhs, gsn = raw(d["lhs"]), raw(d["rhs"]), raw(d["group_sizes"])
    before = oracle.num_threads()
    oracle.set_num_threads(threads)
    try:
        times, spent = [], 0.0
        while spent < 1.0 or len(times) < 5:
            t0 = time.perf_counter()
            oracle.ragged_dot_m(lhs, rhs, gsn)
            dt = time.perf_counter() - t0
            times.append(dt)
            spent += dt
    finally:
        oracle.set_num_threads(before)
    return float(np.median(times))


def cpu_baseline_routing(w, d, target_s, raw, oracle):
    """The oracle's permute / un-permute over the whole workload, repeated until about
    target_s seconds are spent; rate in GB/s of the same algorithmic bytes."""
    if w.op == "permute":
        x, experts = raw(d["x"]), raw(d["experts"])
        run = lambda: oracle.moe_permute(x, experts, w.g)
    else:
        y, weights = raw(d["y"]), raw(d["weights"])
        c2s = oracle.moe_permute(np.zeros((w.tokens, 1), np.float32), raw(d["experts"]), w.g)[4]
        run = lambda: oracle.moe_unpermute(y, c2s, weights)
    B = algorithmic_bytes(w, None)
    spent, done = 0.0, 0
    while spent < target_s:
        t0 = time.perf_counter()
        run()
        spent += time.perf_counter() - t0
        done += 1
    return {"value": B * done / spent / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} whole {w.name} calls, numpy oracle (single-threaded), {spent:.1f} s"}


def kernels_digest():
    """sha256 of the built library, whose gfx950 code objects hold the kernels; a traffic
    record taken with another build is stale.  (Builds are deterministic, so edits that
    leave the code unchanged, such as comments, keep the record valid.)"""
    import hashlib
    lib = os.path.join(os.path.dirname(os.path.abspath(__file__)), "group_gemm_amd", "libgroupgemm.so")
    try:
        with open(lib, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None


def traffic_for(name):
    """HBM bytes per launch of the workload's dominant kernel, measured with rocprofv3
    counters on the current build; None when there is no such measurement."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    digest = kernels_digest()
    if rec is None or digest is None or rec.get("kernels_sha256") != digest:
        return None
    return rec.get("bytes_per_launch")


def _pmc_rows(path, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    out = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def ingest_traffic(a):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each workload's dominant library kernel,
    scaled by what the same counters read for a plain copy of a known size."""
    d = a.traffic_from
    copy = {}
    for ctr, sub in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        rows = _pmc_rows(os.path.join(d, sub), ctr)
        vals = [v for k, vs in rows.items() if "copyBuffer" in k for v in vs]
        copy[ctr] = a.copy_bytes / (sum(vals) / len(vals) * 1024.0)
    try:
        with open(PROFILE_TRAFFIC) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    digest = kernels_digest()
    for sub in sorted(os.listdir(d)):
        if not sub.startswith("fetch_") or not os.path.isdir(os.path.join(d, sub)):
            continue
        wl = sub[len("fetch_"):]
        per = {}
        for ctr, pre in (("FETCH_SIZE", "fetch_"), ("WRITE_SIZE", "write_")):
            rows = _pmc_rows(os.path.join(d, pre + wl), ctr)
            ours = {k: v for k, v in rows.items() if k.startswith("void gg::") or k.startswith("gg::")}
            kern = max(ours, key=lambda k: sum(ours[k]))
            per[ctr] = (kern, sum(ours[kern]) / len(ours[kern]) * 1024.0 * copy[ctr], len(ours[kern]))
        table[wl] = {"kernel": per["FETCH_SIZE"][0], "dispatches": per["FETCH_SIZE"][2],
                     "fetch_bytes": per["FETCH_SIZE"][1], "write_bytes": per["WRITE_SIZE"][1],
                     "bytes_per_launch": per["FETCH_SIZE"][1] + per["WRITE_SIZE"][1],
                     "fetch_factor": copy["FETCH_SIZE"], "write_factor": copy["WRITE_SIZE"],
                     "kernels_sha256": digest}
        print(wl, json.dumps(table[wl]))
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")


def make_call(w, d, G, torch, dev):
    """The timed call of a workload (outputs and workspace allocated once, outside it)."""
    if w.op == "permute":
        ws = torch.empty(G.workspace_bytes("permute", w.m, w.k, 0, w.g), dtype=torch.uint8, device=dev)
        outs = G.moe_permute(d["x"], d["experts"], w.g, workspace=ws)
        return lambda: G.moe_permute(d["x"], d["experts"], w.g, workspace=ws, out=outs), None
    if w.op == "unpermute":
        # the inverse order the permute of the same routing produces (narrow rows: only the
        # index maps are used)
        narrow = torch.zeros((w.tokens, 8), dtype=torch.bfloat16, device=dev)
        c2s = G.moe_permute(narrow, d["experts"], w.g)[4]
        out = torch.empty((w.tokens, w.n), dtype=torch.bfloat16, device=dev)
        return lambda: G.moe_unpermute(d["y"], c2s, d["weights"], out=out), out
    if w.op == "m_gated":
        out = torch.empty((w.m, w.n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(G.workspace_bytes("ragged_m", w.m, w.k, w.n, w.g), dtype=torch.uint8, device=dev)
        return lambda: G.ragged_dot_m_gated(d["lhs"], d["w0"], d["w1"], d["group_sizes"], act="silu", out=out,
                                            workspace=ws), out
    if w.op in ("m", "m_nk"):
        out_dtype = torch.float32 if w.out_dtype == "f32" else torch.bfloat16
        out = torch.empty((w.m, w.n), dtype=out_dtype, device=dev)
        ws = torch.empty(G.workspace_bytes("ragged_m", w.m, w.k, w.n, w.g), dtype=torch.uint8, device=dev)
        layout = "nk" if w.op == "m_nk" else "kn"
        return lambda: G.ragged_dot_m(d["lhs"], d["rhs"], d["group_sizes"], out=out, lhs_scale=d.get("lhs_scale"),
                                      rhs_scale=d.get("rhs_scale"), workspace=ws, rhs_layout=layout), out
    out = torch.empty((w.g, w.k, w.n), dtype=torch.float32, device=dev)
    ws = torch.empty(G.workspace_bytes("ragged_k", w.m, w.k, w.n, w.g), dtype=torch.uint8, device=dev)
    return lambda: G.ragged_dot_k(d["lhs"], d["dout"], d["group_sizes"], out=out, workspace=ws), out


def run_workload(name, a, torch, G, W, dev, cpu=True):
    """Times one workload; returns its record (the fields of the JSON line's `config`,
    `roofline`, `padded` and `cpu_baseline`, plus the value and step time)."""
    w = W.WORKLOADS[name]
    gs = W.group_sizes(w)
    d = W.make_inputs(w, device=dev, gs=gs)
    torch.cuda.synchronize()
    F = useful_flops(w, gs)
    B = algorithmic_bytes(w, gs)
    fn, out = make_call(w, d, G, torch, dev)
    wall, per = time_calls(fn, a.steps, a.warmup, torch)
    ms_per_step = wall / a.steps * 1e3
    med, mean = float(np.median(per)), float(np.mean(per))
    routing = w.op in ("permute", "unpermute")
    # pure data movement is rated in GB/s of algorithmic bytes, the products in TFLOP/s
    value = B / (wall / a.steps) / 1e9 if routing else F / (wall / a.steps) / 1e12

    # roofline of the (single) kernel: MFMA-bound if the arithmetic intensity exceeds the
    # ridge point of its precision, else HBM-bound; achieved over the median launch
    peak_f = PEAK_TFLOPS[w.in_dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if not routing and F / B >= ridge:
        roof = {"bound": "mfma", "achieved": F / med / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": B / med / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_for(w.name)

    config = {"workload": w.name, "op": f"moe_{w.op}" if routing else f"ragged_dot_{w.op}", "m": w.m, "k": w.k,
              "n": w.n, "g": w.g,
              "group_sizes": {"min": int(gs.min()), "max": int(gs.max()), "sum": int(gs.sum()),
                              "empty": int((gs == 0).sum())},
              "useful_gflop_per_step": F / 1e9, "algorithmic_mb_per_step": B / 1e6,
              "kernel_us_per_launch": {"median": med * 1e6, "mean": mean * 1e6, "min": float(per.min()) * 1e6}}
    if routing:
        config["tokens"], config["top_k"] = w.tokens, w.top_k
        if w.op == "permute":
            config["kernels"] = "histogram, rank, gather (one call; roofline over the whole call)"
    padded = None
    if not a.no_padded and not routing and w.op not in ("m_nk", "m_gated"):
        cap = int(math.ceil(gs.max() / 256.0) * 256)
        pws = torch.empty(G.workspace_bytes(f"padded_{w.op}", w.m, w.k, w.n, w.g, cap, d["lhs"].dtype),
                          dtype=torch.uint8, device=dev)
        if w.op == "m":
            pfn = lambda: G.padded_dot("m", d["lhs"], d["rhs"], d["group_sizes"], cap, out=out,
                                       a_scale=d.get("lhs_scale"), b_scale=d.get("rhs_scale"), workspace=pws)
        else:
            pfn = lambda: G.padded_dot("k", d["lhs"], d["dout"], d["group_sizes"], cap, out=out, workspace=pws)
        psteps = max(5, a.steps // 2)
        pwall, pper = time_calls(pfn, psteps, max(2, a.warmup // 2), torch)
        pmed = float(np.median(pper))
        padded = {"capacity": cap, "capacity_rule": "largest group rounded up to 256 rows",
                  "ms_per_step": pwall / psteps * 1e3, "us_per_call_median": pmed * 1e6,
                  "useful_tflops": F / pmed / 1e12, "speedup_ragged_vs_padded": pmed / med}
        del pws
    elif w.op in ("m_nk", "m_gated"):
        padded = None   # padded_dot is the plain [g,k,n] product only
    rec = {"value": value, "unit": "GB/s" if routing else "TFLOP/s", "ms_per_step": ms_per_step,
           "dtype": {"bf16": "bf16", "f32": "f32", "mxfp8": "e4m3"}[w.in_dtype], "config": config, "roofline": roof,
           "padded": padded}
    if cpu and not a.no_cpu_baseline:
        if w.name == "tiny_fp32":
            # small enough for whole oracle calls: all host threads and one thread
            import oracle
            t_all = cpu_whole_call(w, d, W, oracle.num_threads())
            t_one = cpu_whole_call(w, d, W, 1)
            rec["cpu_baseline"] = {"value": F / t_all / 1e12, "unit": "TFLOP/s", "cores": int(oracle.num_threads()),
                                   "kind": "oracle", "cpu_model": cpu_model(),
                                   "sample": "whole calls, median", "us_per_call": t_all * 1e6,
                                   "us_per_call_1_thread": t_one * 1e6}
        else:
            rec["cpu_baseline"] = cpu_baseline(w, d, gs, a.cpu_seconds, W, torch)
    del d, fn, out
    torch.cuda.empty_cache()
    return rec


def library_context(a, torch, W, dev):
    """torch.matmul (hipBLASLt on ROCm) on the bf16 workloads' own inputs: one call per
    non-empty group (the loop a framework without a grouped kernel runs) and one dense call of
    the same flops.  Context for the roofline fractions only; nothing here is the library."""
    res = {}
    for name in ("mixtral8x7b_up_bf16", "deepseekv3_routed_bf16", "llama4scout_wgrad_bf16"):
        w = W.WORKLOADS[name]
        gs = W.group_sizes(w)
        d = W.make_inputs(w, device=dev, gs=gs)
        offs = np.concatenate([[0], np.cumsum(gs)]).astype(np.int64)
        live = [h for h in range(w.g) if gs[h] > 0]
        flops = useful_flops(w, gs)
        lhs = d["lhs"]
        if w.op == "k":
            dout = d["dout"]
            per_group = lambda: [torch.matmul(lhs[offs[h]:offs[h + 1]].t(), dout[offs[h]:offs[h + 1]]) for h in live]
            rows = int(gs.sum())
            dense = lambda: torch.matmul(lhs[:rows].t(), dout[:rows])
        else:
            rhs = d["rhs"]
            per_group = lambda: [torch.matmul(lhs[offs[h]:offs[h + 1]], rhs[h]) for h in live]
            wide = torch.empty((w.k, w.n), dtype=torch.bfloat16, device=dev).copy_(rhs[0])
            dense = lambda: torch.matmul(lhs[:int(gs.sum())], wide)
        entry = {}
        for kind, fn in (("per_group", per_group), ("dense_same_flops", dense)):
            _, per = time_calls(fn, a.steps, a.warmup, torch)
            med = float(np.median(per))
            entry[kind] = {"median_us": round(med * 1e6, 1), "tflops": round(flops / med / 1e12, 1)}
        res[name] = entry
        del d
    print(json.dumps({"library_context": "torch.matmul (hipBLASLt), bf16 in / bf16 out", "workloads": res}), flush=True)


def main():
    a = parse()
    if a.traffic_from:
        ingest_traffic(a)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the path would shard by "
              "experts or tokens, see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    if a.copy_probe:
        src = torch.ones(a.copy_probe, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": a.copy_probe}), flush=True)
        return
    import group_gemm_amd as G
    from group_gemm_amd import workloads as W

    if a.library_context:
        torch.cuda.set_device(0)
        library_context(a, torch, W, "cuda:0")
        return
    G.lib()   # fail loudly if the HIP library is missing
    dev = "cuda:0"
    torch.cuda.set_device(0)
    headline = DEFAULT_WORKLOAD if a.workload == "all" else a.workload
    if headline not in W.WORKLOADS:
        raise SystemExit(f"unknown workload {headline!r}; known: {sorted(W.WORKLOADS)}")
    per_config = {}
    if a.workload == "all":
        for name in PER_CONFIG:
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            per_config[name] = run_workload(name, a, torch, G, W, dev)
        rec = per_config[headline]
    else:
        rec = run_workload(headline, a, torch, G, W, dev)
    config = dict(rec["config"])
    config["padded"] = rec["padded"]
    line = {"metric": METRIC, "value": rec["value"], "unit": rec["unit"], "n_gpus": 1, "steps": a.steps,
            "warmup": a.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": rec["dtype"],
            "data": "synthetic (seeded routing and N(0,1) / N(0,1/k) operands)", "config": config,
            "roofline": rec["roofline"]}
    if "cpu_baseline" in rec:
        line["cpu_baseline"] = rec["cpu_baseline"]
    if per_config:
        line["per_config"] = {name: {"value": r["value"], "unit": r["unit"], "dtype": r["dtype"],
                                     "us_per_launch": r["config"]["kernel_us_per_launch"],
                                     "config": {k: v for k, v in r["config"].items() if k != "kernel_us_per_launch"},
                                     "roofline": r["roofline"], "padded": r["padded"],
                                     "cpu_baseline": r.get("cpu_baseline")}
                              for name, r in per_config.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
