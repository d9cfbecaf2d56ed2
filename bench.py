"""Benchmark: routed-expert (MoE) quantized decode on one MI355X.

One step = one pass of the whole decode path (moe_route_decode, which is
moe_route + moe_permute in one launch -> moe_ffn_tiered -> moe_combine) over
three layer calls, the decode row counts the metric names:
  * 1 row and 6 rows through the tiered 512-expert top-10 layer (hidden 2048,
    FFN 640; Q6_K/Q8_0 hot, Q4_K/Q4_0 middle, MXFP4 tail; rank prior),
  * 16 bf16 rows through the grouped 256-expert top-8 layer (hidden 7168,
    FFN 2048, Q4_K) with its always-on Q8_0 shared expert.
Weights are synthetic (seeded device normals packed by the library's own
quantizer); every layer keeps several weight copies at distinct addresses and
steps rotate through them, so each call streams its experts from HBM rather
than from the 256 MB last-level cache; activations cycle through 256 distinct
rows so the expert set changes from call to call.

value = weight bytes streamed per step (router + each distinct selected
expert, shared included) / wall time per step, in GB/s.

Timed passes (each over the same steps, inputs and weight rotation):
  1. the step itself, with HIP events only before and after: value,
     ms_per_step (nothing is recorded between kernels, since every event
     record between dependent kernels lengthens the gap between them);
  2. each row count alone: tokens_per_s, ms_per_call;
  3. the library's HIP events around every gate/up launch only: the
     roofline of the dominant kernel (ffn_gate_up);
  4. events around every launch: kernel_ms_per_step and, per row count, the
     summed kernel time of a call (per_config);
  5. each call captured as a HIP graph and replayed (>= 500 replays,
     median / p10 / p90);
  6. with --one-launch, each call as one moe_layer_decode launch:
     one_launch_layer (context only).
Also reported: per row count the weight bytes, GB/s and fraction of the 8 TB/s
HBM peak; the gate/up HBM traffic from stored counter runs; a plain streaming
read (the part's ceiling, and its rate at the workloads' sizes), the floor
of a dependent launch and one wave's dependent-step latencies (with the cost of
the routing's top-k); the CPU oracle timed on a bounded sample of every
workload; and, outside the step, the dense layer GEMV (Llama-3-8B shapes,
Q4_K/Q6_K and the ternary T5 format), the 2048-row prefill chunk (also its
expert GEMMs for the experts of at most 32 rows alone and for the others
alone), the block-scaled MX GEMM and the int8 GEMV and GEMM.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu-baseline]
                    [--decode-only | --prefill-only] [--one-launch]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("weight-stream GB/s (% HBM peak) + MoE-layer tokens/s at 1/6/16 decode rows")
HBM_PEAK_GBS = 8000.0
POOL = 256


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_workload(torch):
    from decode_moe_mul_amd import configs, layers, synth
    t0 = time.time()
    tiered = layers.MoELayer(configs.TIERED, copies=4)
    log(f"tiered layer built ({time.time() - t0:.1f}s)")
    t0 = time.time()
    grouped = layers.MoELayer(configs.GROUPED, copies=2)
    log(f"grouped layer built ({time.time() - t0:.1f}s)")
    xt = torch.from_numpy(synth.normal((POOL, 2048), 1.0, 1, synth.ACT, 0)).cuda()
    xg = torch.from_numpy(synth.bf16_round(synth.normal((POOL, 7168), 1.0, 1, synth.ACT, 1)))
    xg = xg.cuda().to(torch.bfloat16)
    return tiered, grouped, xt, xg


def step_calls(tiered, grouped, xt, xg, s):
    """The three layer calls of step s: (layer, x, copy, rows)."""
    x1 = xt[s % POOL:s % POOL + 1]
    o6 = (6 * s) % (POOL - 6)
    x6 = xt[o6:o6 + 6]
    o16 = (16 * s) % (POOL - 16)
    x16 = xg[o16:o16 + 16]
    return [(tiered, x1, s % 4, 1), (tiered, x6, (s + 2) % 4, 6), (grouped, x16, s % 2, 16)]


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return 1


def _threads(n):
    """Context limiting the BLAS pool to n threads (None: unchanged)."""
    import contextlib
    if n is None:
        return contextlib.nullcontext()
    from threadpoolctl import threadpool_limits
    return threadpool_limits(n)


_ORACLE_EXPERTS = {}   # oracle-quantized experts per layer, shared by the timed runs
_ORACLE_DENSE = []


def _oracle_moe_rate(cfg, T, budget_s, threads=None, seed=2, max_experts=None):
    """The oracle on layer calls of T rows of cfg: route (router GEMV, top-k,
    softmax) then dequantize-then-dot of each selected expert, timed per call
    over distinct row sets until budget_s is spent.  Weights are drawn on the
    host with the same shapes and distributions as the device layers and
    quantized by the oracle (untimed).  With max_experts, each call evaluates
    only that many of its distinct experts and the call time is scaled by
    (distinct experts) / (evaluated), as is the byte count (a bounded sample
    of a call too long to run whole)."""
    from decode_moe_mul_amd import synth
    from oracle import formats as fm
    from oracle import moe
    Wr = synth.normal((cfg.E, cfg.H), cfg.sigma_router, 0, synth.ROUTER, 0)
    b = None if cfg.prior_lambda is None else synth.rank_prior(cfg.E, cfg.prior_lambda)
    cache = _ORACLE_EXPERTS.setdefault(cfg.name, {})

    def expert(e):
        if e not in cache:
            t = cfg.tier_of(e)
            tags = ((synth.GATE, synth.UP, synth.DOWN) if e < cfg.E
                    else (synth.SH_GATE, synth.SH_UP, synth.SH_DOWN))
            idx = e if e < cfg.E else e - cfg.E
            wg = synth.normal((cfg.F, cfg.H), cfg.sigma_w, 0, tags[0], idx)
            wu = synth.normal((cfg.F, cfg.H), cfg.sigma_w, 0, tags[1], idx)
            wd = synth.normal((cfg.H, cfg.F), cfg.sigma_w, 0, tags[2], idx)
            cache[e] = (t.fmt_gate_up, fm.quantize(t.fmt_gate_up, wg),
                        fm.quantize(t.fmt_gate_up, wu), t.fmt_down, fm.quantize(t.fmt_down, wd))
        return cache[e]

    def ebytes(e):
        t = cfg.tier_of(e)
        return (2 * fm.tensor_bytes(t.fmt_gate_up, cfg.F, cfg.H)
                + fm.tensor_bytes(t.fmt_down, cfg.H, cfg.F))

    calls, elapsed, nbytes, tokens = 0, 0.0, 0.0, 0
    with _threads(threads):
        for c in range(1 << 20):
            x = synth.normal((T, cfg.H), 1.0, seed, synth.ACT, c)
            if cfg.x_dtype == "bf16":
                x = synth.bf16_round(x)
            ids, p, _ = moe.route(x, Wr, b, cfg.k, cfg.n_shared)   # untimed: pick experts
            distinct = [int(e) for e in np.unique(ids)]
            use = distinct if max_experts is None else distinct[:max_experts]
            for e in use:
                expert(e)
            t0 = time.perf_counter()
            ids, p, _ = moe.route(x, Wr, b, cfg.k, cfg.n_shared)
            t_route = time.perf_counter() - t0
            t0 = time.perf_counter()
            if max_experts is None:
                moe.moe_layer(x, ids, p, expert, cfg.H, cfg.F, cfg.E_total)
            else:
                for e in use:
                    ts = np.nonzero((ids == e).any(axis=1))[0]
                    moe.expert_ffn(expert(e), cfg.H, cfg.F, x[ts])
            t_exp = (time.perf_counter() - t0) * len(distinct) / len(use)
            elapsed += t_route + t_exp
            nbytes += cfg.E * cfg.H * 4 + sum(ebytes(e) for e in distinct)
            tokens += T
            calls += 1
            if elapsed > budget_s:
                break
    return {"threads": threads or _blas_threads(), "calls": calls,
            "s_per_call": round(elapsed / calls, 4),
            "gbs": round(nbytes / elapsed / 1e9, 4),
            "tokens_per_s": round(tokens / elapsed, 3)}


def _oracle_dense_rate(budget_s, threads=None):
    """The oracle on the Llama-3-8B layer's seven quantized matrices at one
    row (dequantize-then-dot per matrix)."""
    from decode_moe_mul_amd import configs, synth
    from oracle import formats as fm
    from oracle import moe
    if not _ORACLE_DENSE:
        for i, (name, N, K, fmt) in enumerate(configs.LLAMA8B_GEMV.mats):
            _ORACLE_DENSE.append((fmt, fm.quantize(fmt, synth.normal((N, K), 0.02, 0, synth.DENSE, i)),
                                  N, K))
    mats = _ORACLE_DENSE
    nbytes = sum(fm.tensor_bytes(f, N, K) for f, _, N, K in mats)
    calls, elapsed = 0, 0.0
    with _threads(threads):
        while elapsed < budget_s:
            xs = {K: synth.normal((1, K), 1.0, 3, synth.ACT, 100 * calls + K) for K in (4096, 14336)}
            t0 = time.perf_counter()
            for f, buf, N, K in mats:
                moe.gemv(f, buf, N, K, xs[K])
            elapsed += time.perf_counter() - t0
            calls += 1
    return {"threads": threads or _blas_threads(), "calls": calls,
            "s_per_call": round(elapsed / calls, 4),
            "gbs": round(nbytes * calls / elapsed / 1e9, 4),
            "tokens_per_s": round(calls / elapsed, 3)}


def cpu_baseline(budget_s=8.0):
    """The oracle (float64 NumPy, as it stands) timed on this host's cores
    on bounded samples of every workload; the headline `value` is the tiered
    layer at 1 row (the decode config the bench's first call uses), with the
    BLAS pool at its default size.  C1-C3 are also timed on one thread."""
    from decode_moe_mul_amd import configs
    cores = _blas_threads()
    cfgs = {}
    t3 = _oracle_moe_rate(configs.TIERED, 1, budget_s)
    cfgs["tiered_1row"] = t3
    cfgs["tiered_1row"]["single_thread"] = _oracle_moe_rate(configs.TIERED, 1, budget_s / 4, 1)
    cfgs["tiered_6rows"] = _oracle_moe_rate(configs.TIERED, 6, budget_s / 4)
    cfgs["tiered_6rows"]["single_thread"] = _oracle_moe_rate(configs.TIERED, 6, budget_s / 4, 1)
    cfgs["tiny_4rows"] = _oracle_moe_rate(configs.TINY, 4, 1.0)
    cfgs["tiny_4rows"]["single_thread"] = _oracle_moe_rate(configs.TINY, 4, 1.0, 1)
    cfgs["dense_gemv_1row"] = _oracle_dense_rate(budget_s / 4)
    cfgs["dense_gemv_1row"]["single_thread"] = _oracle_dense_rate(budget_s / 4, 1)
    cfgs["grouped_16rows"] = _oracle_moe_rate(configs.GROUPED, 16, budget_s / 4, max_experts=3)
    cfgs["grouped_16rows"]["sample"] = "3 of the distinct experts of each call, scaled"
    cfgs["prefill_2048rows"] = _oracle_moe_rate(configs.PREFILL, 2048, budget_s / 4,
                                                max_experts=12)
    cfgs["prefill_2048rows"]["sample"] = "12 of the distinct experts of the chunk, scaled"
    return {"value": t3["gbs"], "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"tiered 512-expert layer at 1 row, {t3['calls']} calls, float64 NumPy "
                      f"dequantize-then-dot ({t3['s_per_call']} s per call; "
                      f"{t3['tokens_per_s']} tokens/s); every workload in `configs`",
            "configs": cfgs}


# ------------------------------------------------------------------ traffic --
# HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
# this script (FETCH_SIZE, then WRITE_SIZE).  Every run copies CAL_BYTES once
# with a plain device copy before the timed region; the counters that copy
# reports calibrate the KiB units.  The summary is stored with a hash of the
# kernel sources and ignored once they change.
CAL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gate_up_traffic.json")
KERNEL_SOURCES = ("decode_moe_mul_amd/csrc/gemv.hip", "decode_moe_mul_amd/csrc/decode.hpp",
                  "decode_moe_mul_amd/csrc/common.hpp", "decode_moe_mul_amd/csrc/dequant.hpp")


def kernel_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic():
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, counter, pick):
    vals = {}
    for r in rows:
        if r.get("Counter_Name") != counter or not pick(r):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return vals


def summarize_trace(trace_dir):
    """Markdown table of a rocprofv3 --kernel-trace run: per kernel (short
    name, the routed FFN's phases told apart) and grid size in workgroups,
    the launch count and the average / min / max duration; then the routed
    FFN phases' averages over all their launches."""
    import collections
    import csv
    import glob
    import re
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]

    def short(name):
        name = re.sub(r"^void ", "", name).replace("qmoe::", "")
        m = re.match(r"(\w+)(<[^>]*>)?", name)
        base = m.group(1) + (m.group(2) or "")
        if base.startswith("ffn_decode_kernel<0"):
            return "ffn_gate_up " + base
        if base.startswith("ffn_decode_kernel<1"):
            return "ffn_down " + base
        return base

    by = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            blocks = 1
            for ax in "XYZ":
                g = int(r.get(f"Grid_Size_{ax}", "1") or 1)
                w = int(r.get(f"Workgroup_Size_{ax}", "1") or 1)
                blocks *= max(1, g // max(1, w))
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            by[(short(r["Kernel_Name"]), blocks)].append(us)
    keep = ("ffn_", "route", "router", "topk", "permute", "combine", "prefill", "qgemv",
            "layer", "mxfp4", "quantize_act", "q8_0_i8")
    print("| kernel | blocks | launches | avg us | min us | max us |")
    print("|---|---:|---:|---:|---:|---:|")
    phase = collections.defaultdict(list)
    for (k, b), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        if not any(k.startswith(p) or p in k for p in keep):
            continue
        print(f"| {k} | {b} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        phase[k.split()[0]].extend(v)
    print()
    for k in ("ffn_gate_up", "ffn_down"):
        if phase.get(k):
            v = phase[k]
            print(f"{k}: {len(v)} launches, average {sum(v) / len(v):.3f} us")


def summarize_pmc(fetch_dir, write_dir):
    """Write TRAFFIC_FILE from the two counter runs."""
    is_gu = lambda r: "ffn_decode_kernel<0" in r["Kernel_Name"]
    # the calibration copy: the last large runtime copy of the program (the
    # later ones are small reads of routing results)
    is_copy = lambda r: "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536
    out = {"kernel_hash": kernel_hash(), "cal_bytes": CAL_BYTES}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _pmc_rows(d)
        gu = _per_dispatch(rows, counter, is_gu)
        cp = _per_dispatch(rows, counter, is_copy)
        cal = cp[max(cp, key=int)]  # KiB the counter reports for CAL_BYTES
        out[f"{name}_cal_kib"] = cal
        out[f"{name}_kib_per_launch"] = sum(gu.values()) / len(gu)
        out[f"{name}_bytes_per_launch"] = sum(gu.values()) / len(gu) * CAL_BYTES / cal
        out[f"{name}_launches"] = len(gu)
    out["traffic_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def summarize_prefill_pmc(dirs):
    """Markdown table of rocprofv3 --pmc runs of `bench.py --prefill-only`:
    per prefill kernel (pass 1 = gate/up, pass 2 = down; the row-tile class
    in the template arguments) the launches and the average of every counter
    per dispatch; FETCH_SIZE / WRITE_SIZE scaled to bytes by the run's 256 MiB
    calibration copy; the MFMA busy fraction as SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE x CUs x 4 SIMDs) when both were collected."""
    import collections
    import re
    rows = []
    for d in dirs:
        rows += _pmc_rows(d)

    def group(name):
        n = re.sub(r"^void ", "", name).replace("qmoe::", "")
        m = re.match(r"(\w+)(<[^>]*>)?", n)
        return m.group(1) + (m.group(2) or "")

    keep = ("prefill", "router_gemm", "topk", "permute", "combine")
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for r in rows:
        k = group(r["Kernel_Name"])
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        c = r["Counter_Name"]
        per[k][c][key] = per[k][c].get(key, 0.0) + float(r["Counter_Value"])
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = {}
        for k, cs in per.items():
            if "copyBuffer" in k and c in cs:
                cp.update(cs[c])
        if cp:
            # the calibration copy is the largest plain copy of the run
            cal[c] = CAL_BYTES / (max(cp.values()) * 1024)   # bytes per counted byte
    counters = sorted({c for k, cs in per.items() for c in cs})
    print("| kernel | launches | " + " | ".join(counters) + " |")
    print("|---|---:|" + "---:|" * len(counters))
    for k in sorted(per):
        if not any(p in k for p in keep):
            continue
        cs = per[k]
        n = max(len(v) for v in cs.values())
        vals = []
        for c in counters:
            v = cs.get(c)
            vals.append("" if not v else f"{sum(v.values()) / len(v):.4g}")
        print(f"| {k} | {n} | " + " | ".join(vals) + " |")
    print()
    cus = 256
    for k in sorted(per):
        if not k.startswith("prefill_kernel"):
            continue
        cs = per[k]
        line = [k]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in cs and c in cal:
                b = sum(cs[c].values()) / len(cs[c]) * 1024 * cal[c]
                line.append(f"{c} {b / 1e6:.1f} MB per launch")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in cs and "GRBM_GUI_ACTIVE" in cs:
            busy = sum(cs["SQ_VALU_MFMA_BUSY_CYCLES"].values())
            act = sum(cs["GRBM_GUI_ACTIVE"].values())
            line.append(f"MFMA busy {busy / (act * cus * 4):.4f} of GRBM_GUI_ACTIVE x {cus} CUs x 4")
        print("- " + "; ".join(line))


def _events_ms(torch, fn, n):
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(n):
        fn(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


def dense_gemv(torch, steps):
    """One dense decoder layer's quantized matrices at one fp32 row (Q, K, V,
    O, gate, up in Q4_K; down in Q6_K; Llama-3-8B shapes), 8 weight copies
    rotated so the last-level cache cannot serve them: one qgemv launch per
    matrix, and all seven in one qgemv_batch launch."""
    from decode_moe_mul_amd import configs, layers, synth
    from decode_moe_mul_amd import qmoe
    layer = layers.DenseLayer(configs.LLAMA8B_GEMV, copies=8)
    x = torch.from_numpy(synth.normal((1, 4096), 1.0, 3, synth.ACT, 0)).cuda()
    xd = torch.from_numpy(synth.normal((1, 14336), 1.0, 3, synth.ACT, 1)).cuda()
    xs = {n: (xd if n == "down" else x) for (n, _, _, _) in configs.LLAMA8B_GEMV.mats}
    nbytes = layer.weight_bytes()
    res = {"workload": "llama3_8b_layer_gemv Q4_K x6 + Q6_K down, 1 fp32 row",
           "weight_bytes": int(nbytes)}
    for mode, batched in (("per_matrix", False), ("batched", True)):
        fwd = lambda i: layer.forward(xs, i % 8, batched=batched)
        for i in range(16):
            fwd(i)
        ms = _events_ms(torch, fwd, steps)
        qmoe.profile_reset()
        qmoe.profile_enable(True)
        _events_ms(torch, fwd, steps)
        qmoe.profile_enable(False)
        n, kms = qmoe.profile_read("qgemv")
        kernel_ms = kms / steps
        log(f"dense layer gemv ({mode}): {ms * 1e3:.1f} us per token "
            f"({kernel_ms * 1e3:.1f} us in kernels)")
        res[mode] = {"us_per_token": round(ms * 1e3, 2),
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel_us": round(kernel_ms * 1e3, 2),
                     "kernel_gbs": round(nbytes / (kernel_ms * 1e-3) / 1e9, 1)}
    del layer
    torch.cuda.empty_cache()
    return res


def ternary_gemv(torch, steps):
    """The same layer's seven matrices in the ternary T5 format (1.75 bits per
    weight), one fp32 row, 8 weight copies rotated: one qgemv_t5 launch per
    matrix, and all seven in one qgemv_batch launch."""
    from decode_moe_mul_amd import configs, layers, synth
    from decode_moe_mul_amd import qmoe
    cfg = configs.LLAMA8B_GEMV_T5
    layer = layers.DenseLayer(cfg, copies=8)
    x = torch.from_numpy(synth.normal((1, 4096), 1.0, 3, synth.ACT, 0)).cuda()
    xd = torch.from_numpy(synth.normal((1, 14336), 1.0, 3, synth.ACT, 1)).cuda()
    xs = {n: (xd if n == "down" else x) for (n, _, _, _) in cfg.mats}
    nbytes = layer.weight_bytes()
    nweights = sum(N * K for (_, N, K, _) in cfg.mats)
    res = {"workload": "llama3_8b_layer_gemv T5 ternary x7 (1.75 bits/weight), 1 fp32 row",
           "weight_bytes": int(nbytes)}
    for mode, batched in (("per_matrix", False), ("batched", True)):
        fwd = lambda i: layer.forward(xs, i % 8, batched=batched)
        for i in range(16):
            fwd(i)
        ms = _events_ms(torch, fwd, steps)
        qmoe.profile_reset()
        qmoe.profile_enable(True)
        _events_ms(torch, fwd, steps)
        qmoe.profile_enable(False)
        kernel_ms = qmoe.profile_read("qgemv_t5")[1] / steps
        log(f"ternary layer gemv ({mode}): {ms * 1e3:.1f} us per token "
            f"({kernel_ms * 1e3:.1f} us in kernels)")
        res[mode] = {"us_per_token": round(ms * 1e3, 2),
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel_us": round(kernel_ms * 1e3, 2),
                     "kernel_gbs": round(nbytes / (kernel_ms * 1e-3) / 1e9, 1),
                     "gweights_per_s": round(nweights / (ms * 1e-3) / 1e9, 1)}
    del layer
    torch.cuda.empty_cache()
    return res


def int8_gemv(torch, calls=50):
    """The Llama-3-8B layer's seven matrices in Q8_0 at 1 and 16 decode rows:
    qgemv_q8_0 on fp32 activations against qquantize_act_q8 + qgemv_q8_0_i8
    (int8 activations, v_dot4 integer dot products), 4 weight copies
    rotated."""
    from decode_moe_mul_amd import configs, qmoe, synth
    mats = [(n, N, K) for (n, N, K, _) in configs.LLAMA8B_GEMV.mats]
    copies = 4
    bufs = []
    for c in range(copies):
        row = []
        for i, (n, N, K) in enumerate(mats):
            W = synth.normal_device((N, K), 0.02, 9, synth.GATE, 100 * c + i, "cuda")
            row.append(qmoe.quantize("q8_0", W))
            del W
        bufs.append(row)
    nbytes = sum(qmoe.tensor_bytes("q8_0", N, K) for _, N, K in mats)
    out = {"workload": "llama3_8b_layer_gemv in Q8_0 x7", "weight_bytes": int(nbytes)}
    for R in (1, 16):
        xs = {K: torch.from_numpy(synth.normal((R, K), 1.0, 4, synth.ACT, K)).cuda()
              for K in {K for _, _, K in mats}}
        ys = [torch.empty((R, N), dtype=torch.float32, device="cuda") for _, N, _ in mats]

        def fp_call(i):
            for j, (n, N, K) in enumerate(mats):
                qmoe.gemv("q8_0", bufs[i % copies][j], N, K, xs[K], out=ys[j])

        def i8_call(i):
            qs = {K: qmoe.quantize_act_q8(x) for K, x in xs.items()}
            for j, (n, N, K) in enumerate(mats):
                q, d = qs[K]
                qmoe.gemv_q8_0_i8(bufs[i % copies][j], N, K, q, d, out=ys[j])

        fp_call(0), i8_call(0)
        fms = _events_ms(torch, fp_call, calls)
        ims = _events_ms(torch, i8_call, calls)
        out[f"rows_{R}"] = {"fp_act_us": round(fms * 1e3, 2),
                            "fp_act_gbs": round(nbytes / (fms * 1e-3) / 1e9, 1),
                            "int8_act_us": round(ims * 1e3, 2),
                            "int8_act_gbs": round(nbytes / (ims * 1e-3) / 1e9, 1)}
    del bufs
    torch.cuda.empty_cache()
    log(f"int8 gemv: {out}")
    return out


def int8_prefill(torch, calls=10):
    """Prefill of the Llama-3-8B layer's seven matrices in Q8_0 at 2048 rows
    on the int8 matrix cores (qquantize_act_q8 once per input, then
    qgemm_q8_0_i8 per matrix), beside the 16-bit path a BF16/FP16 prefill
    takes: the same weights dequantized to fp16 and torch.matmul (the
    library GEMM)."""
    from decode_moe_mul_amd import configs, qmoe, synth
    R = 2048
    mats = [(n, N, K) for (n, N, K, _) in configs.LLAMA8B_GEMV.mats]
    bufs, w16 = [], []
    for i, (n, N, K) in enumerate(mats):
        W = synth.normal_device((N, K), 0.02, 9, synth.GATE, i, "cuda")
        bufs.append(qmoe.quantize("q8_0", W))
        w16.append(qmoe.dequantize("q8_0", bufs[-1], N, K).half())
        del W
    xs = {K: torch.from_numpy(synth.normal((R, K), 1.0, 4, synth.ACT, K)).cuda()
          for K in {K for _, _, K in mats}}
    x16 = {K: x.half() for K, x in xs.items()}
    ys = [torch.empty((R, N), dtype=torch.float32, device="cuda") for _, N, _ in mats]
    flops = sum(2.0 * R * N * K for _, N, K in mats)

    def i8_call(i):
        qs = {K: qmoe.quantize_act_q8(x) for K, x in xs.items()}
        for j, (n, N, K) in enumerate(mats):
            q, d = qs[K]
            qmoe.gemm_q8_0_i8(bufs[j], N, K, q, d, out=ys[j])

    def f16_call(i):
        for j, (n, N, K) in enumerate(mats):
            torch.matmul(x16[K], w16[j].t())

    i8_call(0), f16_call(0)
    ims = _events_ms(torch, i8_call, calls)
    fms = _events_ms(torch, f16_call, calls)
    qmoe.profile_reset()
    qmoe.profile_enable(True)
    _events_ms(torch, i8_call, calls)
    qmoe.profile_enable(False)
    gemm_ms = qmoe.profile_read("q8_0_i8_gemm")[1] / calls
    quant_ms = qmoe.profile_read("quantize_act_q8")[1] / calls
    out = {"workload": "llama3_8b_layer in Q8_0, 2048 rows (7 matrices)",
           "rows": R, "gflop": round(flops / 1e9, 1),
           "int8_ms": round(ims, 4), "int8_tokens_per_s": round(R / (ims * 1e-3), 1),
           "int8_gemm_kernel_ms": round(gemm_ms, 4), "int8_quantize_ms": round(quant_ms, 4),
           "int8_tops": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
           "int8_frac_of_int8_peak": round(flops / (gemm_ms * 1e-3) / 5.0e15, 4),
           "fp16_library_ms": round(fms, 4),
           "fp16_tflops": round(flops / (fms * 1e-3) / 1e12, 1),
           "fp16_frac_of_fp16_peak": round(flops / (fms * 1e-3) / 2.5e15, 4),
           "speedup_int8_over_fp16": round(fms / ims, 3)}
    del bufs, w16
    torch.cuda.empty_cache()
    log(f"int8 prefill: {out}")
    return out


def mx_gemm(torch, calls=20):
    """MXFP4 weights x MXFP8 activations on the block-scaled matrix cores
    (qgemm_mxfp4_mxfp8) for 2048 activation rows: the tail tier's expert
    shapes (gate/up [640, 2048], down [2048, 640]) and a Llama-3-8B MLP shape
    ([14336, 4096]).  Reported beside it: the activation quantizer, and
    dequantize-to-fp16 + torch.matmul (the library GEMM) on the same matrix
    as context."""
    from decode_moe_mul_amd import qmoe, synth
    R = 2048
    out = {"rows": R, "peak_tflops": 5000.0, "peak_note": "dense fp8 MFMA", "shapes": {}}
    for name, N, K in (("tail_gate_up", 640, 2048), ("tail_down", 2048, 640),
                       ("llama_up", 14336, 4096)):
        W = synth.normal_device((N, K), 0.02, 5, synth.UP, 0, "cuda")
        buf = qmoe.quantize("mxfp4", W)
        x = torch.from_numpy(synth.normal((R, K), 1.0, 6, synth.ACT, 0)).cuda()
        codes, scales = qmoe.quantize_act_mxfp8(x)
        y = torch.empty((R, N), dtype=torch.float32, device="cuda")
        qmoe.gemm_mxfp4_mxfp8(buf, N, K, codes, scales, out=y)
        ms = _events_ms(torch, lambda i: qmoe.gemm_mxfp4_mxfp8(buf, N, K, codes, scales, out=y),
                        calls)
        qms = _events_ms(torch, lambda i: qmoe.quantize_act_mxfp8(x), calls)
        w16 = qmoe.dequantize("mxfp4", buf, N, K).half()
        x16 = x.half()
        torch.matmul(x16, w16.t())
        dms = _events_ms(torch, lambda i: torch.matmul(x16, w16.t()), calls)
        flops = 2.0 * R * N * K
        out["shapes"][name] = {
            "N": N, "K": K, "us": round(ms * 1e3, 2),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac": round(flops / (ms * 1e-3) / 5.0e15, 4),
            "quantize_us": round(qms * 1e3, 2),
            "fp16_library_gemm_us": round(dms * 1e3, 2)}
        del W, buf, w16
    torch.cuda.empty_cache()
    log(f"mx gemm: {out['shapes']}")
    return out


def prefill_chunk(torch, calls=10):
    """The tiered 512-expert layer on a 2048-row prefill chunk: router GEMM,
    top-k, permutation, grouped gate/up and down on the matrix cores, combine.
    Reports the HBM rate on the weight bytes of the experts touched and the
    matrix-core utilisation (useful flops of the expert GEMMs / time / dense
    bf16 peak)."""
    from decode_moe_mul_amd import configs, layers, synth
    from decode_moe_mul_amd import qmoe
    cfg = configs.PREFILL
    layer = layers.MoELayer(cfg, copies=2)
    T = 2048
    x = torch.from_numpy(synth.normal((T, cfg.H), 1.0, 4, synth.ACT, 0)).cuda()
    _, ws = layer.forward(x, 0, prefill=True)
    ids = ws["ids"].cpu().numpy()
    nbytes = layer.weight_bytes(ids)
    A = T * (cfg.k + cfg.n_shared)
    flops = 2.0 * A * 3 * cfg.F * cfg.H
    for i in range(3):
        layer.forward(x, i % 2, prefill=True)
    ms = _events_ms(torch, lambda i: layer.forward(x, i % 2, prefill=True), calls)
    qmoe.profile_reset()
    qmoe.profile_enable(True)
    _events_ms(torch, lambda i: layer.forward(x, i % 2, prefill=True), calls)
    qmoe.profile_enable(False)
    kern = {k: qmoe.profile_read(k)[1] / calls for k in
            ("router_gemm", "topk", "permute", "prefill_prep", "prefill_gate_up",
             "prefill_down", "combine")}
    gemm_ms = kern["prefill_gate_up"] + kern["prefill_down"]
    # the same chunk with the MXFP4 tier on the block-scaled matrix cores
    for i in range(3):
        layer.forward(x, i % 2, prefill=True, mx=True)
    mx_ms = _events_ms(torch, lambda i: layer.forward(x, i % 2, prefill=True, mx=True), calls)
    qmoe.profile_reset()
    qmoe.profile_enable(True)
    _events_ms(torch, lambda i: layer.forward(x, i % 2, prefill=True, mx=True), calls)
    qmoe.profile_enable(False)
    mx_kern = {k: qmoe.profile_read(k)[1] / calls for k in
               ("prefill_mx_prep", "prefill_gate_up", "prefill_down")}
    split = _prefill_split(torch, layer, x, ws, calls)
    del layer
    torch.cuda.empty_cache()
    log(f"prefill 2048 rows: {ms:.3f} ms per call (expert GEMMs {gemm_ms:.3f} ms)")
    return {"workload": "prefill2048_tiered_e512_top10 H=2048 F=640, fp32 rows",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "weight_bytes": int(nbytes), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "expert_gemm_ms": round(gemm_ms, 4),
            "useful_gflop": round(flops / 1e9, 2),
            "mfma_util": round(flops / (gemm_ms * 1e-3) / 2.5e15, 4),
            "mfma_util_whole_call": round(flops / (ms * 1e-3) / 2.5e15, 4),
            "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
            "mx_tail_tier": {"ms_per_call": round(mx_ms, 4),
                             "kernel_ms": {k: round(v, 4) for k, v in mx_kern.items()}},
            "by_expert_rows": split}


def _prefill_split(torch, layer, x, ws, calls):
    """The chunk's expert GEMMs (qgemm_grouped_prefill) for two halves of its
    routing alone: the experts with at most 32 rows (one small tile each,
    bound by their weight stream) and the others (128-row tiles on the
    matrix cores).  Each half is the same call with offsets and perm that
    keep only those experts' rows, so the two times show where the mixed
    launches' time goes."""
    from decode_moe_mul_amd import qmoe
    c = layer.cfg
    T = x.shape[0]
    kt = c.k + c.n_shared
    offs = ws["offsets"].cpu().numpy().astype(np.int64)
    perm = ws["perm"].cpu().numpy()
    cnt = np.diff(offs)
    L = qmoe.lib()
    s = qmoe._stream()
    arr = layer.tier_arrays[0]
    o = torch.empty_like(ws["o"])
    out = {}
    for name, keep in (("up_to_32_rows", (cnt > 0) & (cnt <= 32)), ("over_32_rows", cnt > 32)):
        off2 = np.zeros(c.E_total + 1, np.int32)
        off2[1:] = np.cumsum(np.where(keep, cnt, 0))
        rows = np.concatenate([perm[offs[e]:offs[e + 1]] for e in np.nonzero(keep)[0]])
        p2 = np.zeros(T * kt, np.int32)
        p2[:len(rows)] = rows
        off_t = torch.from_numpy(off2).cuda()
        perm_t = torch.from_numpy(p2).cuda()

        def call(i):
            qmoe._check(L.qgemm_grouped_prefill(
                arr, len(arr), c.E_total, c.H, c.F, qmoe._p(x), qmoe._dtype_code(x), T, kt,
                qmoe._p(off_t), qmoe._p(perm_t), qmoe._p(o), qmoe._p(ws["ffn"]),
                ws["ffn"].numel(), s), "qgemm_grouped_prefill")
        for i in range(3):
            call(i)
        qmoe.profile_reset()
        qmoe.profile_enable(True)
        _events_ms(torch, call, calls)
        qmoe.profile_enable(False)
        gu, dn = (qmoe.profile_read(k)[1] / calls for k in ("prefill_gate_up", "prefill_down"))
        nbytes = sum(layer.expert_bytes(int(e)) for e in np.nonzero(keep)[0])
        flops = 2.0 * len(rows) * 3 * c.F * c.H
        out[name] = {"experts": int(keep.sum()), "rows": int(len(rows)),
                     "weight_bytes": int(nbytes), "gate_up_ms": round(gu, 4),
                     "down_ms": round(dn, 4),
                     "weight_gbs": round(nbytes / ((gu + dn) * 1e-3) / 1e9, 1),
                     "tflops": round(flops / ((gu + dn) * 1e-3) / 1e12, 1)}
    log(f"prefill split by expert rows: {out}")
    return out


# names of the kernels the library records for one decode layer call
DECODE_KERNELS = ("route_decode", "router_gemv", "topk", "permute", "ffn_gate_up", "ffn_down",
                  "ffn_down_combine", "combine")


def stream_ceiling(torch, reps=20):
    """The HBM read rate of a plain streaming read (qmoe_stream_read: 16-byte
    nontemporal loads, a contiguous chunk per block, eight loads in flight
    per lane) over a 2 GiB buffer, best of 2 / 4 / 8 / 16 blocks per CU: the
    practical ceiling of a weight stream."""
    from decode_moe_mul_amd import qmoe
    nbytes = 2 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {"bytes": nbytes, "per_blocks_per_cu": {}}
    for bpc in (2, 4, 8, 16):
        qmoe.stream_read(buf, bpc, sink)
        ms = _events_ms(torch, lambda i: qmoe.stream_read(buf, bpc, sink), reps)
        out["per_blocks_per_cu"][str(bpc)] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    best = max(out["per_blocks_per_cu"].values())
    out["gbs"] = best
    out["frac_of_peak"] = round(best / HBM_PEAK_GBS, 4)
    # the same read at the sizes of the decode workloads (one launch per
    # read, rotating over 8 disjoint slices so that the last-level cache does
    # not serve them): what a single weight stream of that size can reach
    out["at_size"] = {}
    for name, nb in (("tiered_1row", 37564108), ("tiered_6rows", 143694950),
                     ("dense_layer", 137822208)):
        n16 = nb // 16 * 16
        slices = [buf.view(torch.uint8)[i * (nbytes // 8):i * (nbytes // 8) + n16].view(torch.int32)
                  for i in range(8)]
        for sl in slices:
            qmoe.stream_read(sl, 8, sink)
        best_us = None
        for bpc in (2, 4, 8, 16):
            ms = _events_ms(torch, lambda i: qmoe.stream_read(slices[i % 8], bpc, sink), 40)
            best_us = ms * 1e3 if best_us is None else min(best_us, ms * 1e3)
        out["at_size"][name] = {"bytes": n16, "us": round(best_us, 2),
                                "gbs": round(n16 / (best_us * 1e-6) / 1e9, 1),
                                "frac_of_peak": round(n16 / (best_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"streaming read at workload sizes: {out['at_size']}")
    del buf
    torch.cuda.empty_cache()
    log(f"streaming-read ceiling: {best} GB/s")
    # the floor of a chain of dependent launches: reads of 4 KiB (one block
    # per CU) back to back on one stream, each waiting for the last; captured
    # as one graph of 200 launches so that the host's enqueue rate is out of
    # the measurement (eager: the host's rate bounds it)
    tiny = torch.zeros(1024, dtype=torch.int32, device="cuda")
    n = 200
    qmoe.stream_read(tiny, 1, sink)
    out["launch_chain_eager_us"] = round(
        _events_ms(torch, lambda i: qmoe.stream_read(tiny, 1, sink), n) * 1e3, 2)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            qmoe.stream_read(tiny, 1, sink)
    g.replay()
    out["launch_chain_graph_us"] = round(_events_ms(torch, lambda i: g.replay(), 10) * 1e3 / n, 2)
    del g
    log(f"dependent launches: {out['launch_chain_graph_us']} us each in a graph, "
        f"{out['launch_chain_eager_us']} us eager")
    # one wave's dependent-step latencies and the routing top-k (median of 5)
    runs = [qmoe.wave_latency() for _ in range(6)][1:]
    lat = {k: sorted(r[k] for r in runs)[len(runs) // 2] for k in runs[0]}
    mhz = lat["shader_clock_mhz"] or 2400
    lat["wave_topk_512_k10_us"] = round(lat["wave_topk_512_k10_cycles"] / mhz, 3)
    out["wave_latency"] = lat
    log(f"wave latency: {lat}")
    return out


def graph_replay(torch, calls, iters=500, warm=50):
    """Each decode call captured as a HIP graph (torch.cuda.CUDAGraph around
    the library calls) and replayed on one stream: `warm` untimed replays,
    then `iters` timed ones with an event before each, rotating through the
    captured calls (distinct weight copies and input rows).  Returns the
    per-replay times in us (median, p10, p90)."""
    graphs = []
    for layer, x, copy, rows in calls:
        layer.forward(x, copy)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(x, copy)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warm):
        graphs[i % len(graphs)].replay()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    for i in range(iters):
        ev[i].record(stream)
        graphs[i % len(graphs)].replay()
    ev[iters].record(stream)
    torch.cuda.synchronize()
    us = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(iters)])
    del graphs
    return {"iters": iters, "median_us": round(float(np.median(us)), 2),
            "p10_us": round(float(np.percentile(us, 10)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="skip the dense-GEMV, prefill, MX and int8 sections (counter runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the 2048-row prefill section (prefill counter runs)")
    ap.add_argument("--one-launch", action="store_true",
                    help="also time the one-launch layer (moe_layer_decode) at 1, 6 and 16 rows")
    ap.add_argument("--graph-iters", type=int, default=500)
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-prefill-pmc", nargs="+", metavar="PMC_DIR",
                    help="print the prefill kernels' counter table of rocprofv3 --pmc runs and exit")
    a = ap.parse_args()
    if a.summarize_pmc:
        summarize_pmc(*a.summarize_pmc)
        return
    if a.summarize_trace:
        summarize_trace(a.summarize_trace)
        return
    if a.summarize_prefill_pmc:
        summarize_prefill_pmc(a.summarize_prefill_pmc)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode path has "
                                   "no multi-GPU mode (run with --gpus 1)"}))
        sys.exit(2)

    import torch
    from decode_moe_mul_amd import qmoe

    torch.cuda.set_device(0)
    qmoe.lib()
    if a.prefill_only:
        cal_src = torch.empty(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
        torch.empty_like(cal_src).copy_(cal_src)
        torch.cuda.synchronize()
        del cal_src
        print(json.dumps({"prefill": prefill_chunk(torch)}), flush=True)
        return
    tiered, grouped, xt, xg = build_workload(torch)
    stream = torch.cuda.current_stream()
    ROWS = (1, 6, 16)

    # algorithmic bytes per call (routing is deterministic: take it from one pass)
    call_bytes = np.zeros((a.steps, 3))
    gate_up_bytes = []
    for s in range(a.steps):
        g_step = 0
        for i, (layer, x, copy, rows) in enumerate(step_calls(tiered, grouped, xt, xg, s)):
            _, ws = layer.forward(x, copy)
            ids = ws["ids"].cpu().numpy()
            call_bytes[s, i] = layer.weight_bytes(ids)
            flat = np.unique(ids)
            g_step += sum(2 * qmoe.tensor_bytes(layer.cfg.tier_of(int(e)).fmt_gate_up,
                                                layer.cfg.F, layer.cfg.H) for e in flat)
        gate_up_bytes.append(g_step)

    # calibration copy for the traffic counters (outside the timed region)
    cal_src = torch.empty(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    for s in range(a.warmup):
        for layer, x, copy, rows in step_calls(tiered, grouped, xt, xg, s):
            layer.forward(x, copy)
    torch.cuda.synchronize()

    def timed(calls_of_step, tag, one_launch=False):
        """ms for a.steps steps of the given calls, events only at the ends."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        if one_launch:
            for s in range(3):
                for layer, x, copy, rows in calls_of_step(s):
                    layer.forward(x, copy, one_launch=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(a.steps):
            for layer, x, copy, rows in calls_of_step(s):
                layer.forward(x, copy, one_launch=one_launch, check=False)
        t1.record(stream)
        torch.cuda.synchronize()
        log(f"timed {tag}: {t0.elapsed_time(t1) / a.steps:.4f} ms per step")
        return t0.elapsed_time(t1)

    def kernel_ms(calls_of_step, names):
        """Summed duration of the library's launches (HIP events around every
        launch, on its stream) over a.steps steps, per kernel name."""
        qmoe.profile_reset()
        qmoe.profile_enable(True)
        timed(calls_of_step, "all-kernel events")
        qmoe.profile_enable(False)
        return {k: qmoe.profile_read(k) for k in names}

    one_call = lambda i: (lambda s: [step_calls(tiered, grouped, xt, xg, s)[i]])
    whole_step = lambda s: step_calls(tiered, grouped, xt, xg, s)

    # 1. the step (value, ms_per_step): the three calls, nothing recorded
    #    between kernels
    total_ms = timed(whole_step, "step")
    ms_step = total_ms / a.steps
    # 2. each row count on its own, same inputs and weight rotation
    call_ms = np.array([timed(one_call(i), f"rows={r}") for i, r in enumerate(ROWS)])
    # 3. the dominant kernel: library HIP events around every gate/up launch
    #    (recorded on the launch stream) over the same steps
    qmoe.profile_reset()
    qmoe.profile_only("ffn_gate_up")
    qmoe.profile_enable(True)
    timed(whole_step, "gate/up events")
    qmoe.profile_enable(False)
    qmoe.profile_only(None)
    n_gu, gu_ms = qmoe.profile_read("ffn_gate_up")
    # 4. every kernel's time over the step, and per row count the layer's
    #    summed kernel time (the 70 % bar is judged on it)
    step_kernels = kernel_ms(whole_step, DECODE_KERNELS)
    call_kernel_ms = []
    for i in range(3):
        ks = kernel_ms(one_call(i), DECODE_KERNELS)
        call_kernel_ms.append(sum(v[1] for v in ks.values()) / a.steps)
    # 5. graph replay of each call (>= 500 replays, median / p10 / p90)
    graphs = {}
    for i, r in enumerate(ROWS):
        copies = 4 if i < 2 else 2
        calls = [step_calls(tiered, grouped, xt, xg, s)[i] for s in range(copies)]
        graphs[str(r)] = graph_replay(torch, calls, a.graph_iters)
        log(f"graph replay rows={r}: {graphs[str(r)]}")
    # 6. the retired one-launch layer (opt-in)
    one_launch = None
    if a.one_launch:
        one_ms = np.array([timed(one_call(i), f"one launch rows={r}", one_launch=True)
                           for i, r in enumerate(ROWS)])
        for r in (1, 6):
            tiered.check_one_launch(r)
        grouped.check_one_launch(16)
        one_launch = {"ms_per_call": {str(r): round(one_ms[i] / a.steps, 5)
                                      for i, r in enumerate(ROWS)},
                      "tokens_per_s": {str(r): round(r * a.steps / (one_ms[i] * 1e-3), 1)
                                       for i, r in enumerate(ROWS)}}

    per_config = {}
    mean_bytes = call_bytes.mean(axis=0)
    for i, r in enumerate(ROWS):
        wall = call_ms[i] / a.steps
        kern = call_kernel_ms[i]
        g = graphs[str(r)]
        per_config[str(r)] = {
            "layer": "tiered" if i < 2 else "grouped",
            "weight_bytes_per_call": int(mean_bytes[i]),
            "ms_per_call": round(wall, 5),
            "tokens_per_s": round(r / (wall * 1e-3), 1),
            "gbs": round(mean_bytes[i] / (wall * 1e-3) / 1e9, 1),
            "hbm_frac": round(mean_bytes[i] / (wall * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_us_per_call": round(kern * 1e3, 2),
            "kernel_gbs": round(mean_bytes[i] / (kern * 1e-3) / 1e9, 1),
            "kernel_hbm_frac": round(mean_bytes[i] / (kern * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "meets_70pct_bar": bool(mean_bytes[i] / (kern * 1e-3) / 1e9 >= 0.7 * HBM_PEAK_GBS),
            "graph_replay": dict(g, gbs_median=round(mean_bytes[i] / (g["median_us"] * 1e-6) / 1e9,
                                                     1)),
        }

    ceiling = stream_ceiling(torch)
    dense = None if a.decode_only else dense_gemv(torch, a.steps)
    ternary = None if a.decode_only else ternary_gemv(torch, a.steps)
    prefill = None if a.decode_only else prefill_chunk(torch)
    mx = None if a.decode_only else mx_gemm(torch)
    i8 = None if a.decode_only else int8_gemv(torch)
    i8p = None if a.decode_only else int8_prefill(torch)

    t = stored_traffic()
    traffic = None if t is None else int(t["traffic_bytes_per_launch"])
    total_bytes = float(call_bytes.sum())
    gbs = total_bytes / (total_ms * 1e-3) / 1e9
    gu_gbs = float(np.sum(gate_up_bytes)) / (gu_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "moe_decode_rows_1_6_16",
                   "layers": {"rows_1_and_6": "tiered E=512 top-10 H=2048 F=640 "
                                              "Q6_K/Q8_0 | Q4_K/Q4_0 | MXFP4, rank prior",
                              "rows_16": "grouped E=256 top-8 H=7168 F=2048 Q4_K "
                                         "+ Q8_0 shared, bf16 rows"},
                   "weight_copies": {"tiered": 4, "grouped": 2}},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": {str(r): round(r * a.steps / (call_ms[i] * 1e-3), 1)
                         for i, r in enumerate(ROWS)},
        "ms_per_call": {str(r): round(call_ms[i] / a.steps, 5) for i, r in enumerate(ROWS)},
        "per_config": per_config,
        "weight_bytes_per_step": int(total_bytes / a.steps),
        "kernel_ms_per_step": {k: round(v[1] / a.steps, 5) for k, v in step_kernels.items()
                               if v[0]},
        "roofline": {"bound": "hbm", "kernel": "ffn_gate_up",
                     "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "launches": n_gu,
                     "avg_launch_us": round(gu_ms * 1e3 / max(n_gu, 1), 3),
                     "algorithmic_bytes_per_launch": int(np.sum(gate_up_bytes) / max(n_gu, 1))},
        "stream_read_ceiling": ceiling,
    }
    if dense is not None:
        out["dense_gemv"] = dense
    if ternary is not None:
        out["ternary_gemv"] = ternary
    if one_launch is not None:
        out["one_launch_layer"] = one_launch
    if prefill is not None:
        out["prefill"] = prefill
    if mx is not None:
        out["mx_gemm"] = mx
    if i8 is not None:
        out["int8_gemv"] = i8
    if i8p is not None:
        out["int8_prefill"] = i8p
    if not a.no_cpu_baseline:
        log("timing the CPU oracle on bounded samples ...")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
