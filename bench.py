#!/usr/bin/env python3
"""Benchmark of the ReTopK decode-step attention path on one MI355X.

A step is one retopk_decode_step call on one attention layer (recall, path
decision, candidate union, candidate scores, rerank, the exact path for heads
that fall back or refresh, softmax-V and the cache update). Layers are
rotated, as a decoder visits them token by token, over enough distinct KV
buffers (each with its own handle and query-support caches) that no layer's
keys stay in the 256 MB Infinity Cache between its steps. Inputs are
resident in HBM before the timed region; nothing is allocated inside it.

Prints one JSON line: the metric is microseconds per decode step per layer
(lower is better) on the 128K-context, K = 512 GQA layer, with the exact
Top-K baseline, a forced-reuse run, dense softmax attention over every key
(the paper's "Full Attention" comparison column), the path mix, the roofline
of the step kernel (a decode step is one launch of it) over the timed steps,
the same on exact calls and on dense calls, whole-step rooflines of the exact
and the forced-reuse steps, event-bracketed per-launch times, and the CPU
oracle baseline.

Counter support: --copy-calibration runs plain copies of known size,
--summarize-traffic turns rocprofv3 FETCH_SIZE / WRITE_SIZE runs into the
per-call HBM bytes that the roofline objects report as "traffic", and
--summarize-kernels turns rocprofv3 kernel traces into the committed
duration tables.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ReTopK decode attn µs/step/layer @128K K=512 (HBM GB/s %peak; vs exact Top-K)"
HBM_PEAK_GBS = 8000.0
ROW_BYTES = 256  # one bf16 key or value row of 128 dims


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048, help="timed layer-steps")
    ap.add_argument("--warmup", type=int, default=64, help="untimed layer-steps before timing")
    ap.add_argument("--workload", default="headline128k")
    ap.add_argument("--layers", type=int, default=0, help="rotated layers (0: enough to exceed 1 GiB of KV)")
    ap.add_argument("--from-start", action="store_true",
                    help="every rotated layer starts at the first decode step (no spread of the layers' "
                         "positions over the workload's steps): times the steps right after the cache "
                         "initialisation, where candidate sets are largest")
    for flag, typ in (("top-k", int), ("top-r", int), ("window", int), ("cache-cap", int), ("tau", float),
                      ("refresh-every", int)):
        ap.add_argument(f"--{flag}", type=typ, default=None,
                        help=f"override the workload's {flag.replace('-', '_')} (sensitivity runs)")
    ap.add_argument("--retrieval", choices=("similarity", "recent"), default=None,
                    help="retrieval of the natural leg: similarity-guided (the method) or recent-R (ablation)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--token-layers", type=int, default=28,
                    help="layers of the graph-replayed decode token leg (0 skips it)")
    ap.add_argument("--only", choices=list(LEGS) + ["fidelity", "stream", "scoreab", "ablation", "token"],
                    default=None,
                    help="run one timed leg only (for profiler runs)")
    ap.add_argument("--fidelity-steps", type=int, default=32,
                    help="decode steps of the support-fidelity leg (0 skips it)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel event-timed pass (counter runs: the last --steps "
                         "dispatches of each kernel are then the timed steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 8 plain device-to-device copies of 256 MiB each, the known-size "
                         "reference for the HBM byte counters")
    ap.add_argument("--summarize-traffic", metavar="DIR", default=None,
                    help="turn rocprofv3 counter runs under DIR (<leg>_<COUNTER>/ and "
                         "copy_<COUNTER>/) into profiles/traffic.json and exit")
    ap.add_argument("--summarize-kernels", metavar="DIR", default=None,
                    help="turn rocprofv3 --kernel-trace --stats runs (DIR/prof_<leg>/) into "
                         "profiles/kernels_<workload>.md and exit")
    ap.add_argument("--json-out", metavar="FILE", default=None,
                    help="also write the result line to FILE (counter runs keep it beside their counters)")
    ap.add_argument("--profile-tag", default="",
                    help="with --summarize-kernels: suffix of the summary's file name (e.g. _20steps)")
    ap.add_argument("--last", type=int, default=64,
                    help="with --summarize-traffic / --summarize-kernels: dispatches per kernel to "
                         "average (the last ones, i.e. the timed steps)")
    return ap.parse_args()


LEGS = ("natural", "exact", "reuse", "dense")
RHO_BINS = (0.85, 0.875, 0.9, 0.925, 0.95)
COPY_BYTES = 256 << 20
COPY_REPS = 8
TRAFFIC_COUNTERS = ("FETCH_SIZE", "WRITE_SIZE")


def copy_calibration():
    """Eight plain device copies of COPY_BYTES: each reads and writes exactly that
    many bytes of HBM, which scales the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "copies": COPY_REPS}), flush=True)


def _counter_rows(path):
    import csv
    rows = []
    for dirpath, _, files in os.walk(path):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(dirpath, fn)) as f:
                    rows.extend(csv.DictReader(f))
    return rows


def _short_name(full):
    """Kernel name without namespaces, template arguments or arguments:
    "ns::(anonymous namespace)::k<true>(int, ...)" -> "k"."""
    return full.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0].split("::")[-1].strip()


def _per_dispatch(rows, counter, last=None):
    """{(kernel short name, grid size): [counter value per dispatch, in dispatch
    order]} (KiB). A call that launches one kernel more than once with
    different grids shows up as several keys. With `last`, only each kernel's
    timed window is kept: its last `last` calls, i.e. its last
    last * (grids among its last `last` dispatches) dispatches."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name = _short_name(r["Kernel_Name"])
        per.setdefault(name, {}).setdefault(int(r["Dispatch_Id"]), [int(r.get("Grid_Size") or 0), 0.0])
        per[name][int(r["Dispatch_Id"])][1] += float(r["Counter_Value"])
    out = {}
    for name, dd in per.items():
        ds = [dd[i] for i in sorted(dd)]
        if last is not None:
            ngrid = len({g for g, _ in ds[-last:]})
            ds = ds[-last * ngrid:]
        for g, v in ds:
            out.setdefault((name, g), []).append(v)
    return out


def summarize_traffic(root, last, workload):
    """Average FETCH_SIZE / WRITE_SIZE over the last `last` dispatches of each
    library kernel per leg, scaled so that a plain copy of known size reads
    (and writes) exactly its size; written to profiles/traffic.json."""
    scale = {}
    for c in TRAFFIC_COUNTERS:
        per = _per_dispatch(_counter_rows(os.path.join(root, f"copy_{c}")), c)
        vals = [v for k, vs in per.items() if "copy" in k[0].lower() for v in vs
                if v * 1024 > COPY_BYTES / 4]  # the copies, not small copy dispatches
        if not vals:
            raise SystemExit(f"no copy dispatch with {c} under {root}/copy_{c}")
        scale[c] = COPY_BYTES / (1024.0 * float(np.median(vals)))
    out = []
    for leg in LEGS:
        got = {}
        for c in TRAFFIC_COUNTERS:
            d = os.path.join(root, f"{leg}_{c}")
            if os.path.isdir(d):
                got[c] = _per_dispatch(_counter_rows(d), c, last)
        if len(got) != len(TRAFFIC_COUNTERS):
            continue
        # per kernel: the launches of one call (one per grid size) summed
        names = sorted({k[0] for k in got["FETCH_SIZE"] if k[0].startswith("k_")})
        for kern in names:
            parts, fb, wb, nd = [], 0.0, 0.0, 0
            for key in sorted(k for k in got["FETCH_SIZE"] if k[0] == kern):
                if key not in got["WRITE_SIZE"]:
                    continue
                f = got["FETCH_SIZE"][key]
                w = got["WRITE_SIZE"][key]
                pf = float(np.mean(f)) * 1024 * scale["FETCH_SIZE"]
                pw = float(np.mean(w)) * 1024 * scale["WRITE_SIZE"]
                parts.append({"grid_threads": key[1], "dispatches": len(f), "fetch_bytes": int(pf),
                              "write_bytes": int(pw)})
                fb, wb, nd = fb + pf, wb + pw, nd + len(f)
            if not parts:
                continue
            # the counter run's own result line (--json-out): its timed window and
            # the algorithmic bytes of the same launches
            win, alg = None, None
            jpath = os.path.join(root, f"{leg}_FETCH_SIZE.json")
            if os.path.exists(jpath):
                with open(jpath) as fh:
                    res = json.loads(fh.read())
                cfg = res.get("config", {})
                win = {"steps": res.get("steps"), "warmup": res.get("warmup"), "layers": cfg.get("rotated_layers")}
                roof = res.get({"natural": "roofline", "exact": "roofline_exact", "dense": "roofline_dense"}.get(leg, ""))
                if roof:
                    alg = roof.get("algorithmic_bytes_per_launch", roof.get("algorithmic_bytes_per_call"))
                elif leg == "reuse" and res.get("reuse_step_roofline"):
                    alg = res["reuse_step_roofline"]["algorithmic_bytes_per_step"]
            if kern != "k_step" and kern != {"dense": "k_dense"}.get(leg, "k_step"):
                alg = None
            out.append({"kernel": kern, "workload": workload, "leg": leg, "window": win,
                        "algorithmic_bytes_per_launch": alg, "dispatches": nd,
                        "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
                        "hbm_bytes_per_launch": int(fb + wb), "launches_per_call": parts,
                        "copy_scale": {c: round(scale[c], 4) for c in TRAFFIC_COUNTERS},
                        "kernel_source_sha": kernel_source_hash()})
    doc = {"commands": [
        "(on one MI355X, from the repository root after `cd /tmp && export TMPDIR=/tmp`, absolute paths)",
        "(<DIR>: any output directory)",
        "rocprofv3 --pmc <C> --output-format csv -d <DIR>/copy_<C> -o pmc -- python3 bench.py "
        "--copy-calibration",
        "rocprofv3 --pmc <C> --output-format csv -d <DIR>/<LEG>_<C> -o pmc -- python3 bench.py "
        "[--workload <W>] --only <LEG> --steps <S> --warmup <WU> --no-cpu-baseline --no-breakdown "
        "--json-out <DIR>/<LEG>_<C>.json",
        "for C in FETCH_SIZE WRITE_SIZE, LEG in natural exact reuse dense; then",
        "python3 bench.py [--workload <W>] --summarize-traffic <DIR> --last <S>",
        "(each row records its run's window: steps S, warm-up WU and rotated layers)"],
        "rows": out}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    # rows of other workloads or windows are kept; this run's replace their namesakes
    keep = []
    if os.path.exists(path):
        with open(path) as fh:
            old = json.load(fh)
        new_keys = {(n["kernel"], n["workload"], n["leg"], json.dumps(n["window"])) for n in out}
        for r in (old["rows"] if isinstance(old, dict) else old):
            key = (r.get("kernel"), r.get("workload"), r.get("leg"), json.dumps(r.get("window")))
            if r.get("window") is not None and key not in new_keys:
                keep.append(r)
    doc["rows"] = keep + out
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
    for r in out:
        print(f"{r['leg']:8s} {r['kernel']:12s} fetch {r['fetch_bytes_per_launch'] / 1e6:9.3f} MB "
              f"write {r['write_bytes_per_launch'] / 1e6:8.3f} MB per launch")
    print(f"copy scale {scale}; wrote {path}")


PROFILE_CMD = ("rocprofv3 --kernel-trace --stats -d {root}/prof_{leg} -o {leg} --output-format csv -- "
               "python3 bench.py{wl} --only {leg} --steps {steps} --warmup {warmup} --no-cpu-baseline "
               "--no-breakdown")
LEG_TITLES = {"natural": "natural ReTopK decode steps (the metric's step)",
              "exact": "Exact Top-K baseline (retopk_exact_topk_attn, every head exact)",
              "reuse": "forced reuse (tau = -2, T_r = 0)",
              "dense": "dense softmax attention over every key (retopk_dense_attn)"}


def summarize_kernels(root, last, workload, warmup=64, tag=""):
    """Per-kernel durations of the timed dispatches (the last `last` of each
    library kernel) from rocprofv3 kernel traces, plus the whole-run --stats
    rows; written to profiles/kernels_<workload>.md."""
    import csv
    lines = [f"# Kernel durations, {workload}: rocprofv3 --kernel-trace --stats", "",
             "Each leg is one run of the command below on one MI355X (from the repository root, after "
             "`cd /tmp && export TMPDIR=/tmp`, with absolute paths). The first table of a leg averages "
             f"the last {last} dispatches of each library kernel, which are the timed decode steps; "
             "the second is rocprofv3's own --stats summary of the whole run (it also counts the cache "
             "initialisation and warm-up dispatches). Summarised by "
             f"`python3 bench.py --summarize-kernels <DIR> --last {last}`, <DIR> being the "
             "directory the commands wrote to.", ""]
    for leg in LEGS:
        d = os.path.join(root, f"prof_{leg}")
        trace = os.path.join(d, f"{leg}_kernel_trace.csv")
        stats = os.path.join(d, f"{leg}_kernel_stats.csv")
        if not os.path.exists(trace):
            continue
        with open(trace) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
        # the timed window: the last `last` calls of each kernel (a call may launch
        # it more than once, with different grids), then one row per grid
        by_name = {}
        for r in rows:
            name = _short_name(r["Kernel_Name"])
            by_name.setdefault(name, []).append(
                (int(r.get("Grid_Size_X") or 0), int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        per = {}
        for name, ds in by_name.items():
            grids = {g for g, _, _ in ds[-last:]}
            for g, a, e in ds[-last * len(grids):]:
                per.setdefault((name, g), []).append((a, e))
        lines += [f"## {leg}: {LEG_TITLES[leg]}", "", "```", PROFILE_CMD.format(
                      leg=leg, steps=last, root="<DIR>", warmup=warmup,
                      wl="" if workload == "headline128k" else f" --workload {workload}"), "```", "",
                  f"Timed dispatches (last {last} of each kernel and grid; a call that launches the kernel "
                  "twice, with different grids, has one row per launch):", "",
                  "| kernel | grid (threads) | dispatches | avg µs | median µs | min µs | max µs |",
                  "|---|---|---|---|---|---|---|"]
        for key in sorted(k for k in per if k[0].startswith("k_") and k[0] != "k_reset"):
            dur = np.array([(e - s) / 1000.0 for s, e in per[key][-last:]])
            lines.append(f"| {key[0]} | {key[1]} | {len(dur)} | {dur.mean():.2f} | {np.median(dur):.2f} | "
                         f"{dur.min():.2f} | {dur.max():.2f} |")
        steps = [k for k in per if k[0] == "k_step"]
        if steps:
            step_key = min(steps, key=lambda k: min(s for s, _ in per[k][-last:]))  # a call's first launch
            st = np.array([s for s, _ in per[step_key][-last:]], dtype=np.float64)
            gap = np.diff(st) / 1000.0
            lines += ["", f"Step period under the tracer (k_step start to the next k_step start): median "
                          f"{np.median(gap):.2f} µs, mean {gap.mean():.2f} µs (under the tracer; the untraced "
                          "step time is the bench line's value)."]
        if os.path.exists(stats):
            with open(stats) as f:
                srows = list(csv.DictReader(f))
            lines += ["", "rocprofv3 --stats (whole run):", "",
                      "| kernel | calls | avg µs | min µs | max µs | total % |", "|---|---|---|---|---|---|"]
            for r in srows:
                name = _short_name(r["Name"])
                lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1000:.2f} | "
                             f"{float(r['MinNs']) / 1000:.2f} | {float(r['MaxNs']) / 1000:.2f} | "
                             f"{float(r['Percentage']):.1f} |")
        lines.append("")
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}{tag}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {path}")


def kernel_source_hash():
    """Hash of the kernels' code (the kernel source and the internal header),
    with comments and whitespace removed: counters taken on one version stay
    valid across comment-only edits."""
    h = hashlib.sha256()
    for name in ("retopk_kernels.hip", "retopk_dense.hip", "retopk_internal.h"):
        with open(os.path.join(ROOT, "sparse_long_context_head_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, leg, window):
    """HBM bytes per launch from committed rocprofv3 counter runs taken on the
    current kernel code over the same timed window (steps, warm-up, rotated
    layers) as this run; else None. Second value: a counter row of the current
    code over another window (its window, HBM bytes and that run's own
    algorithmic bytes), or None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        doc = json.load(f)
    rows = doc["rows"] if isinstance(doc, dict) else doc
    other = None
    for r in rows:
        if r.get("kernel") == kernel and r.get("workload") == workload and \
                r.get("leg") == leg and r.get("kernel_source_sha") == kernel_source_hash():
            if r.get("window") == window:
                return r.get("hbm_bytes_per_launch"), None
            if r.get("window") is not None:
                other = {"window": r["window"], "hbm_bytes_per_launch": r.get("hbm_bytes_per_launch"),
                         "algorithmic_bytes_per_launch": r.get("algorithmic_bytes_per_launch")}
    return None, other


def layer_offsets(counts, total):
    """Decode steps by which each rotated layer is advanced (untimed, right after
    its cache initialisation), layer l then running counts[l] consecutive decode
    positions, so that the layers' windows spread evenly over the workload's
    `total` decode steps: the first starts at step 1 and the last ends at step
    `total` (a multiple of T_r in every configuration, so a refresh step is
    timed). With one layer, or windows as long as the run, no layer is
    advanced."""
    nl = len(counts)
    if nl <= 1 or max(counts) >= total:
        return [0] * nl
    return [round(l * (total - counts[l]) / (nl - 1)) for l in range(nl)]


def check_device_error(B, layers, leg):
    """Every call of the leg completed its work: no work group of any call gave
    up a bounded wait (the handle's sticky device error word is 0)."""
    for i, layer in enumerate(layers):
        word = B.retopk_read_device_error(layer.handle)
        if word != 0:
            raise SystemExit(f"{leg}: layer {i} reports device error word {word}: a call gave up a wait, "
                             "its results are not valid")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.last, args.workload)
        return
    if args.summarize_kernels:
        summarize_kernels(args.summarize_kernels, args.last, args.workload, args.warmup, args.profile_tag)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path has no "
              f"multi-GPU leg", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    from sparse_long_context_head_amd import binding as B
    from sparse_long_context_head_amd.workload import WORKLOADS, generate

    wl = WORKLOADS[args.workload]
    over = {k: getattr(args, k) for k in ("top_k", "top_r", "window", "cache_cap", "tau", "refresh_every")
            if getattr(args, k) is not None}
    if over:
        wl = wl.replace(**over)
    retrieval = args.retrieval or "similarity"
    kv_bytes = 2 * wl.batch * wl.n_kv_heads * wl.max_len * ROW_BYTES
    nl = args.layers or max(1, math.ceil((1 << 30) / kv_bytes))
    n_pos = math.ceil((args.warmup + args.steps) / nl)
    if n_pos > wl.decode_steps:
        wl = wl.replace(decode_steps=n_pos)
    counts = [len(range(l, args.warmup + args.steps, nl)) for l in range(nl)]
    offsets = [0] * nl if args.from_start else layer_offsets(counts, wl.decode_steps)
    L0, G = wl.prompt_len, wl.n_q_heads // wl.n_kv_heads
    log(f"workload {wl.name}: B={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} L0={L0} "
        f"K={wl.top_k}; {nl} rotated layers; {n_pos} decode positions per layer from offsets {offsets}")
    t0 = time.time()
    data = generate(wl)
    log(f"generated inputs in {time.time() - t0:.1f}s")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    k0 = B.bf16_tensor(data["k"], dev)
    v0 = B.bf16_tensor(data["v"], dev)
    q_tail = B.bf16_tensor(data["q_tail"], dev)
    q_dec = B.bf16_tensor(data["q_dec"], dev)
    ks = [k0] + [k0.clone() for _ in range(nl - 1)]
    vs = [v0] + [v0.clone() for _ in range(nl - 1)]
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def make_layers(init=True, **override):
        """Handles with initialised caches, each advanced through its offset's
        decode steps (untimed setup: the cache state a layer has at that point
        of the decode)."""
        override = {"retrieval": retrieval, **override}
        layers = [B.ReTopKLayer.from_workload(wl, **override) for _ in range(nl)]
        for l in range(nl):
            if init:
                layers[l].init_from_prefill(q_tail, ks[l], L0, stream)
                for pos in range(1, offsets[l] + 1):
                    layers[l].decode_step(q_dec[pos - 1], ks[l], vs[l], L0 + pos, pos, out, stream)
        torch.cuda.synchronize()
        return layers

    def schedule(s):
        """layer-step s -> (layer, decode position)"""
        return s % nl, offsets[s % nl] + s // nl + 1

    # the timed (layer, position) pairs: per layer a contiguous run of positions
    timed_pos = {}
    for s_ in range(args.warmup, args.warmup + args.steps):
        l_, p_ = schedule(s_)
        timed_pos.setdefault(l_, []).append(p_)
    mean_len = float(np.mean([L0 + p_ for ps in timed_pos.values() for p_ in ps]))
    window = {"steps": args.steps, "warmup": args.warmup, "layers": nl}

    def run(layers, s0, n, exact=False):
        for s in range(s0, s0 + n):
            l, pos = schedule(s)
            if exact == "dense":
                layers[l].dense_attn(q_dec[pos - 1], ks[l], vs[l], L0 + pos, out, stream)
            elif exact:
                layers[l].exact_topk_attn(q_dec[pos - 1], ks[l], vs[l], L0 + pos, out, None, stream)
            else:
                layers[l].decode_step(q_dec[pos - 1], ks[l], vs[l], L0 + pos, pos, out, stream)

    def timed(layers, exact=False):
        run(layers, 0, args.warmup, exact)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run(layers, args.warmup, args.steps, exact)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps * 1000.0  # us per layer-step

    def step_percentiles(layers, exact=False):
        """Per-step times from an event pair around every timed step (each pair
        adds a dispatch gap, so these run a little longer than the timed mean).
        A GPU sleep queued first keeps the device busy while the host enqueues
        the steps, so that host submission time does not enter the pairs."""
        run(layers, 0, args.warmup, exact)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda._sleep(int(2.4e9 * 60e-6 * args.steps))  # about 60 us of host time per step
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            run(layers, args.warmup + i, 1, exact)
            b.record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) * 1000.0 for a, b in ev])
        return {"p50": round(float(np.percentile(t, 50)), 3), "p90": round(float(np.percentile(t, 90)), 3),
                "p99": round(float(np.percentile(t, 99)), 3), "max": round(float(t.max()), 3),
                "mean": round(float(t.mean()), 3)}

    def kernel_breakdown(layers, exact=False):
        run(layers, 0, args.warmup, exact)
        torch.cuda.synchronize()
        for layer in layers:
            B.retopk_set_timing(layer.handle, True)
            B.retopk_read_kernel_times(layer.handle)
        run(layers, args.warmup, args.steps, exact)
        tot = {}
        for layer in layers:
            for name, (ms, n) in B.retopk_read_kernel_times(layer.handle).items():
                t = tot.setdefault(name, [0.0, 0])
                t[0] += ms
                t[1] += n
            B.retopk_set_timing(layer.handle, False)
        return {k: {"us_per_step": round(v[0] * 1000 / args.steps, 3),
                    "us_per_launch": round(v[0] * 1000 / max(v[1], 1), 3), "launches": v[1]}
                for k, v in tot.items() if v[1]}

    result = {"metric": METRIC, "unit": "us/step/layer", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": wl.name, "batch": wl.batch, "n_q_heads": wl.n_q_heads,
                         "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                         "prompt_len": L0, "top_k": wl.top_k, "cache_cap": wl.cache_cap,
                         "window": wl.window, "top_r": wl.top_r, "tau": wl.tau, "retrieval": retrieval,
                         "refresh_every": wl.refresh_every, "rotated_layers": nl,
                         "decode_positions": n_pos, "layer_offsets": offsets,
                         "timed_positions": {str(l_): [min(ps), max(ps)] for l_, ps in sorted(timed_pos.items())},
                         "parallelism": "single GPU"}}

    def timed_paths(layers):
        """Path bits and M_t of every head over exactly the timed layer-steps."""
        paths, ms, lens = [], [], []
        for l_, ps in sorted(timed_pos.items()):
            assert ps == list(range(min(ps), max(ps) + 1))
            path, _, m = layers[l_].stats(min(ps), len(ps))
            paths.append(path)
            ms.append(m)
            lens.extend(L0 + p_ for p_ in ps)
        return np.concatenate(paths), np.concatenate(ms), np.array(lens, dtype=np.float64)

    def kernel_bytes(path, m, lens):
        """Algorithmic HBM bytes per launch of each decode-step kernel,
        averaged over the timed steps (path bits and M_t per head-step from
        the statistics ring). Only what the method must move is counted:
        queries, the q_bar cache, the retrieved supports, key and value rows,
        outputs and cache entries; candidate, score and histogram workspaces
        are not. k_step (the whole step): every head's query and C cached
        normalised queries; a reusing head's R supports, M_t key rows,
        min(K, M_t) value rows, its output and cache entry; every key row of
        a KV group holding an exact head; an exact head's K value rows, output
        and cache entry."""
        d, K, C, R = wl.head_dim, wl.top_k, wl.cache_cap, wl.top_r
        T = path.shape[0]
        exact = (path & 1) == 1
        reuse = ~exact
        gex = exact.reshape(T, wl.batch, wl.n_kv_heads, G).any(-1)
        n = np.minimum(K, m)
        entry = 4 * d + 4 * K
        ln = lens.reshape(T, 1, 1)
        per = {
            "k_step": (2 * d + 4 * C * d
                       + reuse * (4 * R * K + ROW_BYTES * (m + n) + 4 * d + entry)
                       + exact * (ROW_BYTES * np.minimum(K, ln) + 4 * d + entry)).sum()
                      + (gex * ROW_BYTES * lens.reshape(T, 1, 1)).sum(),
        }
        return {k: float(v) / T for k, v in per.items()}

    def roofline(kernel, alg, us, leg, per="launch"):
        gbs = alg / (us * 1e-6) / 1e9
        traffic, other = load_traffic(kernel, wl.name, leg, window)
        r = {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
             f"algorithmic_bytes_per_{per}": int(alg), f"us_per_{per}": round(us, 3)}
        if traffic is None and other is not None:
            # counters of the same kernel code, taken over another timed window
            r["traffic_other_window"] = other
        return r

    def path_mix(path, m):
        exact = (path & 1) == 1
        refresh = (path & 2) == 2
        gexact = exact.reshape(exact.shape[0], wl.batch, wl.n_kv_heads, G).any(-1)
        mr = m[~exact]
        return {
            "head_steps": int(exact.size), "reuse": round(float((~exact).mean()), 5),
            "exact_fallback": round(float((exact & ~refresh).mean()), 5),
            "exact_refresh": round(float(refresh.mean()), 5),
            "kv_group_steps_with_exact": round(float(gexact.mean()), 5),
            "M_t": {"mean": round(float(mr.mean()), 1) if mr.size else None,
                    "p50": int(np.percentile(mr, 50)) if mr.size else None,
                    "p90": int(np.percentile(mr, 90)) if mr.size else None,
                    "max": int(mr.max()) if mr.size else None}}

    # --- natural ReTopK step (the headline value) ---------------------------
    if args.only in (None, "natural"):
        nat = make_layers()
        init_state = nat[0].read_state()
        us = timed(nat)
        result["value"] = round(us, 3)
        result["ms_per_step"] = round(us / 1000.0, 6)
        log(f"natural ReTopK: {us:.2f} us/step/layer")
        path, m, lens = timed_paths(nat)
        result["path_mix"] = path_mix(path, m)
        # A decode step is one launch of k_step, so the timed region's per-step
        # time (HIP events on the launch stream) is its average launch duration;
        # the algorithmic bytes are averaged over the same timed steps.
        result["roofline"] = roofline("k_step", kernel_bytes(path, m, lens)["k_step"], us, "natural")
        check_device_error(B, nat, "natural")
        for layer in nat:
            layer.close()
        if not args.no_breakdown:
            # per-launch times with an event pair around every launch (each pair
            # adds a dispatch gap, so these run longer than the timed step)
            nat = make_layers()
            result["kernels_natural"] = kernel_breakdown(nat)
            check_device_error(B, nat, "natural (per-launch events)")
            for layer in nat:
                layer.close()
            nat = make_layers()
            result["natural_step_us_percentiles"] = step_percentiles(nat)
            check_device_error(B, nat, "natural (percentiles)")
            for layer in nat:
                layer.close()

    # --- exact Top-K baseline -----------------------------------------------
    if args.only in (None, "exact"):
        ex = make_layers()
        us_ex = timed(ex, exact=True)
        result["exact_topk_us_per_step"] = round(us_ex, 3)
        log(f"exact Top-K: {us_ex:.2f} us/step/layer")
        check_device_error(B, ex, "exact")
        # the whole exact step: every KV group's key rows once, the union of the
        # selected value rows per group (measured), q in and out
        pos = round(mean_len) - L0
        sel = torch.empty((wl.batch, wl.n_q_heads, wl.top_k), dtype=torch.int32, device=dev)
        ex[0].exact_topk_attn(q_dec[pos - 1], ks[0], vs[0], L0 + pos, out, sel, stream)
        torch.cuda.synchronize()
        s_ = sel.cpu().numpy().reshape(wl.batch, wl.n_kv_heads, G * wl.top_k)
        v_rows = sum(len(np.unique(r[r >= 0])) for r in s_.reshape(-1, G * wl.top_k))
        step_alg = ROW_BYTES * (mean_len * wl.batch * wl.n_kv_heads + v_rows) \
            + wl.batch * wl.n_q_heads * wl.head_dim * (2 + 4)
        gbs = step_alg / (us_ex * 1e-6) / 1e9
        result["exact_step_roofline"] = {"bound": "hbm", "achieved": round(gbs, 1),
                                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                                         "algorithmic_bytes_per_step": int(step_alg),
                                         "unique_v_rows": int(v_rows)}
        # an exact call is one launch of k_step, timed per call
        result["roofline_exact"] = roofline("k_step", step_alg, us_ex, "exact", per="call")
        for layer in ex:
            layer.close()
        if not args.no_breakdown:
            ex = make_layers()
            result["kernels_exact"] = kernel_breakdown(ex, exact=True)
            check_device_error(B, ex, "exact (per-launch events)")
            for layer in ex:
                layer.close()
        if "value" in result:
            result["speedup_vs_exact"] = round(us_ex / result["value"], 3)

    # --- forced reuse (every head reuses every step) ------------------------
    if args.only in (None, "reuse"):
        ru = make_layers(tau=-2.0, refresh_every=0)
        us_ru = timed(ru)
        result["forced_reuse_us_per_step"] = round(us_ru, 3)
        log(f"forced reuse: {us_ru:.2f} us/step/layer")
        check_device_error(B, ru, "reuse")
        path_r, m_r, lens_r = timed_paths(ru)
        alg = sum(kernel_bytes(path_r, m_r, lens_r).values())
        gbs = alg / (us_ru * 1e-6) / 1e9
        result["reuse_step_roofline"] = {"bound": "hbm", "achieved": round(gbs, 1),
                                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                                         "algorithmic_bytes_per_step": int(alg),
                                         "M_t_mean": round(float(m_r.mean()), 1)}
        for layer in ru:
            layer.close()
        if not args.no_breakdown:
            ru = make_layers(tau=-2.0, refresh_every=0)
            result["kernels_forced_reuse"] = kernel_breakdown(ru)
            check_device_error(B, ru, "reuse (per-launch events)")
            for layer in ru:
                layer.close()
        if "exact_topk_us_per_step" in result:
            result["speedup_reuse_vs_exact"] = round(result["exact_topk_us_per_step"] / us_ru, 3)

    # --- dense attention over every key (comparison column) -----------------
    if args.only in (None, "dense"):
        de = make_layers(init=False)
        us_de = timed(de, exact="dense")
        result["dense_attn_us_per_step"] = round(us_de, 3)
        log(f"dense attention: {us_de:.2f} us/step/layer")
        # every key and value row of every KV group once, q in and out
        dense_alg = 2 * ROW_BYTES * mean_len * wl.batch * wl.n_kv_heads \
            + wl.batch * wl.n_q_heads * wl.head_dim * (2 + 4)
        # a dense call is k_dense (the row slices) then k_dense_merge, timed per call
        result["roofline_dense"] = roofline("k_dense", dense_alg, us_de, "dense", per="call")
        for layer in de:
            layer.close()
        if not args.no_breakdown:
            de = make_layers(init=False)
            result["kernels_dense"] = kernel_breakdown(de, exact="dense")
            for layer in de:
                layer.close()
        if "value" in result:
            result["speedup_vs_dense"] = round(us_de / result["value"], 3)
        if "exact_topk_us_per_step" in result:
            result["dense_vs_exact"] = round(result["exact_topk_us_per_step"] / us_de, 3)

    # --- retrieval ablation: similarity-guided against recent-R --------------
    # (Experiments, component ablation, Table 3: the exact-path rate and the
    # mean candidate count of each, here over the natural leg's timed window)
    if args.only in (None, "ablation"):
        abl = {}
        for mode in ("similarity", "recent"):
            lay = make_layers(retrieval=mode)
            us_m = timed(lay)
            pth, mm, _ = timed_paths(lay)
            check_device_error(B, lay, f"ablation ({mode})")
            for layer in lay:
                layer.close()
            pm = path_mix(pth, mm)
            abl[mode] = {"us_per_step": round(us_m, 3), "exact_path_rate": round(1.0 - pm["reuse"], 5),
                         "exact_fallback": pm["exact_fallback"], "M_t_mean": pm["M_t"]["mean"]}
            log(f"retrieval {mode}: {us_m:.2f} us/step, exact-path rate {1.0 - pm['reuse']:.4f}, "
                f"M_t mean {pm['M_t']['mean']}")
        result["retrieval_ablation"] = abl

    # --- one decode token over many layers: eager calls against a graph replay
    # (Experiments, Kernel efficiency analysis, Table 4: ms/token over the 28
    # layers, workspaces reused across layers)
    if args.only in (None, "token") and args.token_layers > 0:
        result["token"] = token_leg(B, torch, wl, data, k0, v0, q_tail, q_dec, dev, args, L0)

    # --- support fidelity against Exact Top-K (quality, not timed) ----------
    if args.only in (None, "fidelity") and args.fidelity_steps > 0:
        result["fidelity"] = support_fidelity(wl, data, q_tail, q_dec, ks[0], vs[0], out, stream,
                                              min(args.fidelity_steps, wl.decode_steps))

    # --- the measured streaming-read ceiling (the library's plain read kernel) --
    if args.only in (None, "stream"):
        result["stream_read"] = stream_read(B, torch, dev, stream)
        gbs = result["stream_read"]["gbs"]
        for key in ("roofline", "roofline_exact", "roofline_dense"):
            if key in result:
                result[key]["frac_of_stream_read"] = round(result[key]["achieved"] / gbs, 4)

    # --- the score pass on matrix cores against the vector ALUs --------------
    if args.only in (None, "scoreab"):
        result["score_unit_ab"] = score_unit_ab(B, torch, ks[0], q_dec, stream)

    # --- CPU oracle baseline ------------------------------------------------
    if not args.no_cpu_baseline and args.only in (None, "natural"):
        result["cpu_baseline"] = cpu_baseline(wl, data, init_state, args.cpu_seconds)
    if "value" not in result:
        result["value"] = None
    line = json.dumps(result)
    if args.json_out:
        with open(args.json_out, "w") as fh:
            fh.write(line + "\n")
    print(line, flush=True)


def token_leg(B, torch, wl, data, k0, v0, q_tail, q_dec, dev, args, L0):
    """Decode tokens over n layers that share one set of workspaces (a
    retopk_group): each layer has its own KV buffers (copies of the
    workload's) and caches. Eager: retopk_decode_step of every layer per token.
    Graph: one retopk_group_replay per token (the captured position update
    and all layers' steps), after copying the token's query into the captured
    query buffer (timed with it). Both from the initialised caches, over the
    same decode positions (warm-up tokens first); HIP events on the stream and
    the host's enqueue time per token."""
    n = args.token_layers
    tokens = max(8, min(args.steps, 64))
    warm = 2
    if warm + tokens > wl.decode_steps:
        tokens = wl.decode_steps - warm
    stream = torch.cuda.Stream(device=dev)
    ks = [k0] + [k0.clone() for _ in range(n - 1)]
    vs = [v0] + [v0.clone() for _ in range(n - 1)]
    shape = (wl.batch, wl.n_q_heads, wl.head_dim)
    outs = [torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(n)]
    qbuf = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    grp = B.ReTopKGroup.from_workload(wl, n)

    def init():
        with torch.cuda.stream(stream):
            for l in range(n):
                grp.layers[l].init_from_prefill(q_tail, ks[l], L0, stream)
        stream.synchronize()

    def timed(step_fn):
        for t in range(1, warm + 1):
            step_fn(t)
        stream.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        h0 = time.perf_counter()
        for t in range(warm + 1, warm + tokens + 1):
            step_fn(t)
        host = (time.perf_counter() - h0) / tokens * 1e6
        b.record(stream)
        stream.synchronize()
        return a.elapsed_time(b) / tokens, host

    def eager_token(t):
        for l in range(n):
            grp.layers[l].decode_step(q_dec[t - 1], ks[l], vs[l], L0 + t, t, outs[l], stream)

    init()
    ms_e, host_e = timed(eager_token)
    check_device_error(B, grp.layers[:1], "token (eager)")
    init()
    grp.capture([qbuf] * n, ks, vs, outs, stream)
    grp.set_position(L0 + 1, 1)

    def graph_token(t):
        with torch.cuda.stream(stream):
            qbuf.copy_(q_dec[t - 1])
        grp.replay(stream)

    ms_g, host_g = timed(graph_token)
    check_device_error(B, grp.layers[:1], "token (graph)")
    ws_bytes = grp.device_bytes()
    grp.close()
    del ks, vs
    log(f"token over {n} layers: eager {ms_e:.3f} ms, graph {ms_g:.3f} ms (host {host_e:.0f} / {host_g:.0f} us)")
    return {"layers": n, "tokens": tokens, "warmup_tokens": warm,
            "eager_ms_per_token": round(ms_e, 4), "graph_ms_per_token": round(ms_g, 4),
            "eager_us_per_layer_step": round(ms_e * 1000 / n, 3),
            "graph_us_per_layer_step": round(ms_g * 1000 / n, 3),
            "eager_host_us_per_token": round(host_e, 1), "graph_host_us_per_token": round(host_g, 1),
            "group_device_bytes": ws_bytes}


def stream_read(B, torch, dev, stream):
    """Best of three timed batches of ten plain streaming reads of 1 GiB (one
    retopk_stream_read launch each), HIP events on the launch stream."""
    buf = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        B.retopk_stream_read(buf, sink, stream)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            B.retopk_stream_read(buf, sink, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 10
        best = ms if best is None else min(best, ms)
    gbs = (1 << 30) / (best * 1e-3) / 1e9
    log(f"streaming read: {gbs:.0f} GB/s")
    del buf
    return {"kernel": "k_stream_read", "bytes": 1 << 30, "us_per_launch": round(best * 1000, 2),
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def score_unit_ab(B, torch, k, q_dec, stream):
    """The full-history score pass of one call (7 query heads per KV head,
    every key row of batch entry 0) as the library's score probe runs it on
    MFMA and on the vector ALUs: best of three batches of ten launches each,
    alternating, HIP events on the launch stream."""
    rows = k[0].reshape(-1, 128)
    q = q_dec[0, 0, :7].contiguous()
    sink = torch.zeros(1, dtype=torch.float32, device=k.device)
    best = {1: None, 0: None}
    for _ in range(3):
        B.retopk_score_probe(1, rows, q, sink, stream)
        B.retopk_score_probe(0, rows, q, sink, stream)
    torch.cuda.synchronize()
    for _ in range(3):
        for mode in (1, 0):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(10):
                B.retopk_score_probe(mode, rows, q, sink, stream)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 10
            best[mode] = ms if best[mode] is None else min(best[mode], ms)
    nbytes = rows.shape[0] * 256
    res = {"rows": int(rows.shape[0]), "bytes": nbytes, "query_heads": 7}
    for mode, name in ((1, "mfma"), (0, "valu")):
        res[f"{name}_us"] = round(best[mode] * 1000, 2)
        res[f"{name}_gbs"] = round(nbytes / (best[mode] * 1e-3) / 1e9, 1)
    log(f"score pass A/B: MFMA {res['mfma_us']} us, VALU {res['valu_us']} us over {res['rows']} rows")
    return res


def _cos(a, b):
    na, nb = float(np.linalg.norm(a)), float(np.linalg.norm(b))
    return float(a @ b) / (na * nb) if na > 0 and nb > 0 else 1.0


def support_fidelity(wl, data, q_tail, q_dec, k, v, out, stream, n_steps):
    """Attention-support fidelity of the natural ReTopK path against Exact
    Top-K on one layer (Experimental Results, Attention-support fidelity,
    Figures 5-6): for every head-step, the Exact Top-K support recall
    |S_hat & S| / |S|, the retained attention mass (full-attention softmax mass
    on S_hat over that on S), the cosine of the two renormalised attention
    distributions over positions, and the cosine of the two head outputs. S_hat
    and both outputs come from the library (a decode step, then the stateless
    Exact Top-K call on the same query); the full-attention weights are
    computed here in float64 from the bf16 keys. Summarised over all
    head-steps, over reuse-path ones, and by rho_max."""
    import torch

    from sparse_long_context_head_amd import binding as B
    G, d, L0 = wl.n_q_heads // wl.n_kv_heads, wl.head_dim, wl.prompt_len
    dev = out.device
    layer = B.ReTopKLayer.from_workload(wl)
    layer.init_from_prefill(q_tail, k, L0, stream)
    out_x = torch.empty_like(out)
    sel = torch.empty((wl.batch, wl.n_q_heads, wl.top_k), dtype=torch.int32, device=dev)
    dec = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kf_all = {(b, g): dec(data["k"][b, g, :L0 + n_steps])
              for b in range(wl.batch) for g in range(wl.n_kv_heads)}
    rows = []
    for t in range(1, n_steps + 1):
        L = L0 + t
        layer.decode_step(q_dec[t - 1], k, v, L, t, out, stream)
        info = layer.step_info()
        o_r = out.cpu().numpy().astype(np.float64)
        layer.exact_topk_attn(q_dec[t - 1], k, v, L, out_x, sel, stream)
        o_x = out_x.cpu().numpy().astype(np.float64)
        s_x = sel.cpu().numpy()
        for b in range(wl.batch):
            for g in range(wl.n_kv_heads):
                kf = kf_all[b, g][:L]
                for h in range(g * G, (g + 1) * G):
                    e = kf @ dec(data["q_dec"][t - 1, b, h]) / math.sqrt(d)
                    a = np.exp(e - e.max())
                    S = s_x[b, h, :min(wl.top_k, L)]
                    Sh = info["sel"][b, h, :info["sel_len"][b, h]]
                    pS = np.zeros(L)
                    pS[S] = a[S] / a[S].sum()
                    pH = np.zeros(L)
                    pH[Sh] = a[Sh] / a[Sh].sum()
                    rows.append((int(info["path"][b, h]), float(info["rho_max"][b, h]),
                                 t,
                                 len(np.intersect1d(S, Sh)) / len(S), float(a[Sh].sum() / a[S].sum()),
                                 _cos(pS, pH), _cos(o_r[b, h], o_x[b, h])))
    # columns: path, rho_max, step, recall, retained mass, attention cosine, output cosine
    layer.close()
    r = np.array(rows)

    def summary(m):
        if not m.any():
            return None
        return {"head_steps": int(m.sum()), "support_recall": round(float(r[m, 3].mean()), 4),
                "retained_mass": round(float(r[m, 4].mean()), 5),
                "attention_cosine": round(float(r[m, 5].mean()), 5),
                "output_cosine": round(float(r[m, 6].mean()), 6)}

    reuse = r[:, 0] == 0
    edges = (-np.inf,) + RHO_BINS + (np.inf,)
    by = []
    for lo, hi in zip(edges[:-1], edges[1:]):
        m = reuse & (r[:, 1] >= lo) & (r[:, 1] < hi)
        if m.any():
            by.append({"rho_max": [None if np.isinf(lo) else lo, None if np.isinf(hi) else hi], **summary(m)})
    # the cache starts from exact supports; reuse steps only re-rank earlier
    # supports and the recent window, so recall against the current query's
    # Exact Top-K support is shown per decode step as well
    by_step = {str(t): summary(r[:, 2] == t) for t in (1, 2, 4, 8, 16, 32, 64, 128, 256) if t <= n_steps}
    log(f"fidelity over {len(rows)} head-steps: recall {r[:, 3].mean():.3f}, mass {r[:, 4].mean():.4f}, "
        f"output cosine {r[:, 6].mean():.5f}")
    return {"decode_steps": n_steps, "all": summary(np.ones(len(r), bool)), "reuse": summary(reuse),
            "reuse_by_rho_max": by, "by_decode_step": by_step}


def cpu_baseline(wl, data, init_state, budget_s):
    """The CPU oracle, as written, on a bounded sample of the same workload,
    from the GPU's post-initialisation cache of layer 0 and decode step 1 on:
    natural steps (the metric's step, its path mix included), then steps with
    every head on the exact path (tau above 1) and steps with every head
    reusing (tau = -2, no refresh), each timed per step with perf_counter
    within its share of the budget (at least 2 exact and 32 reuse steps)."""
    import oracle.retopk_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    L0 = wl.prompt_len

    def run(share, min_steps, **override):
        orc = O.ReTopKOracle.from_workload(wl, **override)
        orc.set_state(*init_state)
        spent, steps, exact = 0.0, 0, 0
        while (spent < share or steps < min_steps) and steps < wl.decode_steps:
            t = steps + 1
            a = time.perf_counter()
            rec = orc.step(data["q_dec"][t - 1], data["k"], data["v"], L0 + t, t)
            spent += time.perf_counter() - a
            steps += 1
            exact += int(rec.path.sum())
        return spent / steps * 1e6, steps, exact

    us, steps, exact_hs = run(0.4 * budget_s, 1)
    us_x, steps_x, _ = run(0.3 * budget_s, 2, tau=2.0)
    us_r, steps_r, _ = run(0.3 * budget_s, 32, tau=-2.0, refresh_every=0)
    heads = wl.batch * wl.n_q_heads
    log(f"cpu oracle: natural {us:.0f} us/step/layer over {steps} steps; exact {us_x:.0f} ({steps_x}); "
        f"reuse {us_r:.0f} ({steps_r})")
    return {"value": round(us, 1), "unit": "us/step/layer", "cores": cores, "kind": "oracle",
            "sample": f"{steps} natural ReTopK decode steps (t_dec 1..{steps}) of one {wl.name} layer from "
                      f"the post-initialisation cache ({exact_hs} exact head-steps of {steps * heads}); "
                      f"{steps_x} steps with every head exact and {steps_r} with every head reusing, "
                      "from the same cache; float64 NumPy, per-step perf_counter",
            "exact_us_per_step": round(us_x, 1), "exact_steps": steps_x,
            "reuse_us_per_step": round(us_r, 1), "reuse_steps": steps_r,
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
