#!/usr/bin/env python3
"""Throughput of the quantized gated delta-rule decode step on one MI355X.

One "step" is one decode step of the whole batch: every (sequence, value head)
state is dequantized, updated, read out, requantized and written back once.
Metric: quantized state-updates/s (sequence x head x step) and the algorithmic
HBM bytes/s of the decode kernel as a fraction of MI355X peak (8 TB/s).

Default workload: B = 1024 sequences, 32 value heads sharing 16 key heads,
128 x 128 states at the 6-bit mix (64 rows 8-bit, 64 rows 4-bit per head,
fp32 row factors, calibrated column factors), bf16 q/k/v, synthetic seeded
inputs.  The timed loop rotates over --pools independent state pools so the
working set (pools x 419 MB) exceeds the 256 MB Infinity Cache.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
COUNTERS_FILE = ROOT / "profiles" / "decode_counters.json"
# what the measured kernel is built from: its source and the build flags
DECODE_SRC = [ROOT / "linear_attention_recurrent_rule_amd" / "csrc" / "decode128.hip",
              ROOT / "linear_attention_recurrent_rule_amd" / "csrc" / "tile128.h",
              ROOT / "linear_attention_recurrent_rule_amd" / "csrc" / "stq_internal.h",
              ROOT / "linear_attention_recurrent_rule_amd" / "build.py"]


def _code_only(text: str, suffix: str) -> str:
    """The source without comments and blank lines: edits to comments leave
    the compiled kernel, and so the recorded counters, unchanged."""
    import re

    if suffix == ".py":
        text = re.sub(r'(?m)^\s*#.*$', "", text)
        text = re.sub(r'(?s)""".*?"""', "", text)
    else:
        text = re.sub(r"(?s)/\*.*?\*/", "", text)
        text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def decode_source_sha256() -> str:
    h = hashlib.sha256()
    for f in DECODE_SRC:
        h.update(_code_only(f.read_text(), f.suffix).encode())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200, help="launches per timed block")
    p.add_argument("--warmup", type=int, default=400, help="untimed launches first")
    p.add_argument("--warmup-floor-ms", type=float, default=100.0,
                   help="after the --warmup launches, keep launching (untimed, counted and "
                        "reported as warmup_launches) until this much wall time has passed: "
                        "the clocks need about 30 ms of load to leave their idle state")
    p.add_argument("--blocks", type=int, default=3,
                   help="timed blocks of --steps launches; ms_per_step is their median")
    p.add_argument("--workload", default="highconc_6bit")
    p.add_argument("--batch", type=int, default=None,
                   help="override the workload's number of sequences B (a batch-size sweep; "
                        "the workload is then named <workload>_B<B>)")
    p.add_argument("--pools", type=int, default=4, help="state pools rotated in the timed loop")
    p.add_argument("--mode", choices=("in_place", "double_buffered"), default="in_place",
                   help="in_place: each step rewrites the pool it reads; double_buffered: "
                        "step t reads pool t and writes pool t+1 (stq_decode_step_into)")
    p.add_argument("--window", type=int, default=16, help="distinct input steps cycled")
    p.add_argument("--no-variants", action="store_true", help="skip the comparison formats")
    p.add_argument("--variants", default=None,
                   help="comma-separated subset of the comparison variants to run")
    p.add_argument("--graph", action="store_true",
                   help="time replays of a HIP graph of the launches instead of eager "
                        "launches (for the launch-bound small workloads)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only-decode", action="store_true",
                   help="time the main workload only (for profiler runs)")
    p.add_argument("--trace-summary", default=None, metavar="KERNEL_TRACE_CSV",
                   help="no GPU work: summarise a rocprofv3 kernel trace (calls, avg, min, max "
                        "per kernel, and the average over each kernel's last --timed-launches "
                        "dispatches) and exit")
    p.add_argument("--timed-launches", type=int, default=None,
                   help="with --trace-summary: dispatches of each kernel that were timed "
                        "(default: --blocks x --steps)")
    p.add_argument("--pmc-summary", default=None, metavar="COUNTER_COLLECTION_CSV",
                   help="no GPU work: average each counter of a rocprofv3 --pmc CSV per "
                        "dispatch, per kernel, and exit")
    p.add_argument("--skip", type=int, default=None,
                   help="with --trace-summary: average the timed launches over dispatches "
                        "skip .. skip + timed - 1 of each kernel (the line's warmup_launches for "
                        "the main measurement) instead of its last ones")
    p.add_argument("--with-copy", action="store_true",
                   help="also run the 1 GiB reference copy (with --only-decode)")
    p.add_argument("--drift", action="store_true",
                   help="instead of timing: run the workload's T steps on the packed state and "
                        "on an FP32 state from the same S0 and print the drift as one JSON line")
    p.add_argument("--layers", type=int, default=None, help="layers for --drift (default: all)")
    p.add_argument("--refit", action="store_true",
                   help="--drift with the refit format (per-state column factors refit every "
                        "step, row-impact weights from the calibration steps)")
    p.add_argument("--drift-steps", type=int, default=None, help="T for --drift (default: the "
                   "workload's)")
    p.add_argument("--alloc", action="store_true",
                   help="--drift with the ragged format: FP16 pivot rows and 8/6/4/2-bit rows "
                        "chosen by the lifetime-aware assignment (with --refit: the refit variant)")
    p.add_argument("--gate", action="store_true",
                   help="--drift with a per-key-row gate of the KDA form in place of alpha, "
                        "d_i = sigmoid(N(2.5, 1.5)) per (sequence, value head, key row, step)")
    return p.parse_args()


def unit_state_bytes(fmt: str, d: int, n8: int) -> int:
    if fmt == "fp32":
        return 4 * d * d
    if fmt == "int8row":
        return d * d + 4 * d
    if fmt == "refit":  # plus the state's own column factors
        return n8 * d + (d - n8) * d // 2 + 8 * d
    return n8 * d + (d - n8) * d // 2 + 4 * d


def algorithmic_bytes(fmt: str, B: int, hv: int, hk: int, d: int, n8: int, in_el: int,
                      gated: bool = False, out_el: int = 4) -> int:
    """Bytes one decode launch must move: read + write of every state, q and k
    once per key head, v, alpha (or the fp32 row gate), beta once per value
    head, o written once (out_el bytes per element)."""
    state = 2 * unit_state_bytes(fmt, d, n8) * B * hv
    gate = 4 * d if gated else 4
    vecs = B * hk * 2 * d * in_el + B * hv * (d * in_el + gate + 4 + out_el * d)
    return state + vecs


def measure_copy(torch, stq, nbytes: int = 1 << 30, iters: int = 10) -> float:
    """Practical HBM ceiling: read + write bytes/s of the library's plain
    streaming copy over buffers far larger than the Infinity Cache."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        stq.stream_copy(src, dst)
    torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record()
    for _ in range(iters):
        stq.stream_copy(src, dst)
    e_ev.record()
    torch.cuda.synchronize()
    return 2 * nbytes * iters / (s_ev.elapsed_time(e_ev) / 1e3) / 1e9


def alloc_pivots(hv: int, d: int) -> int:
    """FP16 pivot rows per slot: the paper's KDA share, 512 of 81,920 key rows
    (App. C.2 Table C1), of this layer's Hv * d rows."""
    return int(round(hv * d * 512 / 81920))


def alloc_nominal(w) -> int:
    """Nominal integer width of the ragged format for a workload: 6 bits for
    the 6-bit mix (half the rows 8-bit), 4 bits below it (Table C1 budgets)."""
    return 6 if 2 * w.n8 >= w.d else 4


def calibrate_alloc(torch, stq, S0, step_inputs, *, B, hv, hk, d, steps, nominal, n_pivot,
                    horizon=2048, gated=False, refit=False):
    """Offline calibration of the ragged format on unquantized FP32-state steps
    from S0: pass 1 folds the column maxima and the log retention (and the row
    impact for the refit format), FINALIZE sets c; pass 2 replays the same
    steps and folds the candidate distortions against that c; then the
    lifetime-aware assignment.  step_inputs(t) gives (q, k, v, alpha or gate,
    beta).  Returns (counts [Hv][5] numpy, c, perm, w2 or None)."""
    fmt = stq.FMT_ALLOC_REFIT if refit else stq.FMT_ALLOC
    cal = stq.State(stq.Geometry(1, hv, hk, d, 0, fmt, nominal_bits=nominal, n_pivot=n_pivot))
    fp = stq.State(stq.Geometry(B, hv, hk, d, 0, stq.FMT_FP32))
    cal.calibrate(None, stq.CAL_RESET)
    cal.calibrate_retention(flags=stq.CAL_RESET)
    if refit:
        cal.calibrate_impact(None, None, None, None, stq.CAL_RESET)
    for pass_ in (0, 1):
        fp.pack(S0)
        for t in range(steps):
            q, k, v, g, b = step_inputs(t)
            if gated:
                fp.decode_step_gated(q, k, v, g, b)
            else:
                fp.decode_step(q, k, v, g, b)
            if pass_ == 0:
                cal.calibrate(fp.s32, stq.CAL_COLS)
                if gated:
                    cal.calibrate_retention(gate=g)
                else:
                    cal.calibrate_retention(alpha=g)
                if refit and gated:
                    cal.calibrate_impact(q, k, None, b, 0, gate=g)
                elif refit:
                    cal.calibrate_impact(q, k, g, b, 0)
            else:
                cal.calibrate(fp.s32, stq.CAL_DIST)
        if pass_ == 0:
            cal.calibrate(None, stq.CAL_FINALIZE)
    cal.allocate(horizon)
    if refit:
        cal.calibrate_impact(None, None, None, None, stq.CAL_FINALIZE)
    counts = cal.layout[:, :5].cpu().numpy().copy()
    out = (counts, cal.c.clone(), cal.perm.clone(), cal.w2.clone() if refit else None)
    del fp, cal
    torch.cuda.synchronize()
    return out


def alloc_unit_bytes(counts, d: int) -> float:
    """Average bytes per (slot, head) of a ragged layout: the used segment
    bytes plus the fp32 row factors."""
    import numpy as np
    rb = np.array([2 * d, d, 3 * d // 4, d // 2, d // 4])
    seg = (counts * rb).sum(axis=1)
    seg = (seg + 15) // 16 * 16
    return float(seg.mean() + 4 * d)


def _time_oracle_steps(oracle, wl, w, ps, n_max, budget_s, threads):
    """Successive oracle decode steps of workload w from packed state ps (each
    from the previous step's result) until n_max steps or budget_s seconds;
    returns (steps, seconds)."""
    p8, p4, r = ps.pool8, ps.pool4, ps.r
    n, dt = 0, 0.0
    while n < n_max and dt < budget_s:
        x = wl.workload_inputs(w, n)
        t1 = time.perf_counter()
        res = oracle.step(p8, p4, r, ps.c, ps.perm, x.q, x.k, x.v, x.alpha, x.beta, n8=w.n8,
                          nthreads=threads)
        dt += time.perf_counter() - t1
        p8, p4, r = res["pool8"], res["pool4"], res["r"]
        n += 1
    return n, dt


def cpu_baseline(np, wl, w, B, hv, d) -> dict:
    """The oracle timed on the host cores: the benchmarked workload over about
    10 s, the small mixed workload over its whole T = 256 steps, one full step
    of the serving workload and of the 4.5-bit high-concurrency workload, and
    a single-thread sample."""
    import oracle

    threads = oracle.default_threads()
    ps = wl.random_packed_state(B, hv, d, w.n8, seed=w.seed + 700)
    n_steps, dt = _time_oracle_steps(oracle, wl, w, ps, 32, 10.0, threads)
    cpu = dict(value=B * hv * n_steps / dt, unit="state-updates/s", cores=threads, kind="oracle",
               sample=f"{n_steps} successive full decode steps of the workload ({B * hv} "
                      f"units each, d={d}, n8={w.n8}) from a seeded random packed state, "
                      f"{dt:.1f}s wall on {threads} threads")
    configs = {}
    for name, n_max in (("small_mixed", None), ("serving_6bit", 1), ("highconc_4p5bit", 1)):
        wc = wl.WORKLOADS[name]
        n_max = wc.T if n_max is None else n_max
        psc = wl.random_packed_state(wc.B, wc.hv, wc.d, wc.n8, seed=wc.seed + 700)
        n, t_ = _time_oracle_steps(oracle, wl, wc, psc, n_max, 60.0, threads)
        configs[name] = dict(value=wc.B * wc.hv * n / t_, unit="state-updates/s", cores=threads,
                             sample=f"{n} decode step(s) of {wc.B * wc.hv} units (d={wc.d}, "
                                    f"n8={wc.n8}), {t_:.2f}s wall")
    cpu["configs"] = configs
    # the same oracle on one thread, over the first 64 sequences of one step
    nb = min(B, 64)
    x = wl.workload_inputs(w, 0)
    t1 = time.perf_counter()
    oracle.step(ps.pool8[:nb], ps.pool4[:nb], ps.r[:nb], ps.c, ps.perm, x.q[:nb], x.k[:nb],
                x.v[:nb], x.alpha[:nb], x.beta[:nb], n8=w.n8, nthreads=1)
    dt1 = time.perf_counter() - t1
    cpu["single_thread"] = dict(value=nb * hv / dt1, unit="state-updates/s", cores=1,
                                sample=f"one decode step of {nb * hv} units, {dt1:.2f}s")
    log(f"[bench] oracle: {cpu['value']:.0f} updates/s on {threads} threads, "
        f"{cpu['single_thread']['value']:.0f} on one; "
        + ", ".join(f"{k}: {v['value']:.0f}" for k, v in configs.items()))
    return cpu


def trace_summary(path: str, timed: int, skip: int | None = None) -> str:
    """Per-kernel calls / avg / min / max (us) of a rocprofv3 kernel-trace CSV,
    and each kernel's average over `timed` of its dispatches: the last ones,
    or those after the first `skip`."""
    import csv

    durs: dict[str, list[float]] = {}
    with open(path, newline="") as f:
        rows = sorted(csv.DictReader(f), key=lambda r_: int(r_["Start_Timestamp"]))
    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("void ", "").strip()
        depth = 0
        for i, ch in enumerate(name):  # cut the argument list after the template
            depth += (ch == "<") - (ch == ">")
            if ch == "(" and depth == 0:
                return name[:i]
        return name

    for r_ in rows:
        name = short(r_["Kernel_Name"])
        durs.setdefault(name, []).append(
            (int(r_["End_Timestamp"]) - int(r_["Start_Timestamp"])) / 1e3)
    label = f"last_{timed}_avg_us" if skip is None else f"{skip}+{timed}_avg_us"
    out = [f"{'kernel':<58} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {label:>16}"]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        if skip is None:
            tail = v[-timed:] if len(v) >= timed else v
        else:
            tail = v[skip:skip + timed] or v
        out.append(f"{name[:58]:<58} {len(v):>6} {sum(v) / len(v):>9.1f} {min(v):>9.1f} "
                   f"{max(v):>9.1f} {sum(tail) / len(tail):>16.1f}")
    return "\n".join(out)


def pmc_summary(path: str) -> str:
    """Per kernel: dispatches and the average of each counter per dispatch
    (summed over the per-agent/per-block rows of a dispatch) of a rocprofv3
    --pmc counter-collection CSV."""
    import csv
    from collections import defaultdict

    per = defaultdict(float)
    kern = {}
    with open(path, newline="") as f:
        for r_ in csv.DictReader(f):
            key = (r_["Dispatch_Id"], r_["Counter_Name"])
            per[key] += float(r_["Counter_Value"])
            kern[r_["Dispatch_Id"]] = r_["Kernel_Name"]
    by = defaultdict(lambda: defaultdict(list))
    for (disp, ctr), v in per.items():
        name = kern[disp].replace("(anonymous namespace)::", "").replace("void ", "")
        by[name.split("(")[0] if "<" not in name else name[:name.index(">") + 1]][ctr].append(v)
    out = []
    for name, ctrs in sorted(by.items()):
        n = max(len(v) for v in ctrs.values())
        out.append(f"{name}  ({n} dispatches)")
        for ctr, v in sorted(ctrs.items()):
            out.append(f"    {ctr:28s} {sum(v) / len(v):20.1f}")
    return "\n".join(out)


def main():
    args = parse()
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.timed_launches or args.blocks * args.steps,
                            args.skip))
        return
    if args.gpus != 1:
        log("bench.py measures one GPU only: the decode step has no exchange between units, "
            "so a multi-GPU run would shard sequence slots and run this same kernel on each "
            "GPU's share; that path is not built. Run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_recurrent_rule_amd import stq
    from linear_attention_recurrent_rule_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stq.lib()  # fails loudly if libstq.so is missing
    w = wl.WORKLOADS[args.workload]
    if args.batch is not None:
        if args.batch < 1:
            raise SystemExit("--batch must be at least 1")
        w = dataclasses.replace(w, B=args.batch, name=f"{w.name}_B{args.batch}")
    B, hv, hk, d = w.B, w.hv, w.hk, w.d
    in_el = 2 if w.dtype == "bf16" else 4
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731

    def to_dev_inputs(x):
        if x.dtype == "bf16":
            cv = lambda bits: dev(bits.view(np.int16)).view(torch.bfloat16)  # noqa: E731
            return cv(x.q_bits), cv(x.k_bits), cv(x.v_bits), dev(x.alpha), dev(x.beta)
        return dev(x.q), dev(x.k), dev(x.v), dev(x.alpha), dev(x.beta)

    if args.drift:
        print(json.dumps(run_drift(args, np, torch, stq, wl, w)), flush=True)
        return

    # ---------------------------------------------------------------- setup --
    t0 = time.time()
    log(f"[bench] workload {w.name}: B={B} Hv={hv} Hk={hk} d={d} n8={w.n8} {w.dtype}")
    S0 = dev(wl.initial_state(w))
    log(f"[bench] S0 generated ({S0.numel() * 4 / 2**30:.2f} GiB) in {time.time() - t0:.1f}s")

    if w.calib_seed is None:
        # no calibration stream (the tiny workload): c = 1, rows in order
        c = torch.ones((hv, d), dtype=torch.float32, device="cuda")
        perm = torch.arange(d, dtype=torch.int32, device="cuda").repeat(hv, 1).contiguous()
    else:
        # offline calibration: 32 unquantized steps on the calibration stream
        fp_cal = stq.State(stq.Geometry(B, hv, hk, d, 0, stq.FMT_FP32))
        fp_cal.pack(S0)
        cal = stq.State(stq.Geometry(1, hv, hk, d, w.n8, stq.FMT_MIXED48))
        cal.calibrate(None, stq.CAL_RESET)
        for t in range(w.calib_steps):
            q, k, v, a, b = to_dev_inputs(wl.workload_inputs(w, t, calibration=True))
            fp_cal.decode_step(q, k, v, a, b)
            last = t == w.calib_steps - 1
            cal.calibrate(fp_cal.s32, stq.CAL_COLS | (stq.CAL_ROWS if last else 0))
        cal.calibrate(None, stq.CAL_FINALIZE)
        c, perm = cal.c.clone(), cal.perm.clone()
        del fp_cal
        torch.cuda.synchronize()
    log(f"[bench] calibrated in {time.time() - t0:.1f}s")

    window = [to_dev_inputs(wl.workload_inputs(w, t)) for t in range(args.window)]

    def alloc_cal_inputs(t, gated_):
        q, k, v, a, b = to_dev_inputs(wl.workload_inputs(w, t, calibration=True))
        if gated_:
            a = dev(wl.draw_gate(B, hv, d, seed=w.calib_seed, step=t))
        return q, k, v, a, b
    o_f32 = torch.empty((B, hv, d), dtype=torch.float32, device="cuda")
    o = o_f32

    alloc_cal = {}  # (gated, refit) -> (counts, c, perm, w2) of the ragged format
    gate_cache = []

    def gate_window():
        if not gate_cache:
            gate_cache.extend(dev(wl.draw_gate(B, hv, d, seed=w.seed, step=t))
                              for t in range(len(window)))
        return gate_cache

    def make_pools(fmt: int, n8: int, n: int, gated: bool = False):
        pools = []
        for _ in range(n):
            if fmt in (stq.FMT_ALLOC, stq.FMT_ALLOC_REFIT):
                refit_ = fmt == stq.FMT_ALLOC_REFIT
                counts, ca, pa, w2a = alloc_cal[(gated, refit_)]
                st = stq.State(stq.Geometry(B, hv, hk, d, 0, fmt, nominal_bits=alloc_nominal(w),
                                            n_pivot=alloc_pivots(hv, d)))
                st.set_alloc_layout(counts, ca, pa)
                if refit_:
                    st.w2.copy_(w2a)
            else:
                st = stq.State(stq.Geometry(B, hv, hk, d, n8, fmt))
            if fmt in (stq.FMT_MIXED48, stq.FMT_REFIT):
                st.set_calibration(c, perm)
            st.pack(S0)
            pools.append(st)
        torch.cuda.synchronize()
        return pools

    gates = None

    def launch(pools, t, into):
        q, k, v, a, b = window[t % len(window)]
        src = pools[t % len(pools)]
        if gates is not None:
            dst = pools[(t + 1) % len(pools)] if into else None
            src.decode_step_gated(q, k, v, gates[t % len(gates)], b, o=o, dst=dst)
        elif into:
            src.decode_step_into(pools[(t + 1) % len(pools)], q, k, v, a, b, o=o)
        else:
            src.decode_step(q, k, v, a, b, o=o)

    def warm_up(pools, warmup, into, run):
        """The --warmup launches, then more until --warmup-floor-ms of wall
        time has passed since the first; returns the launches made (all of
        them reported).  `run(t)` issues launch t and returns how many it
        issued."""
        t0 = time.perf_counter()
        n = 0
        while n < warmup:
            n += run(n)
        torch.cuda.synchronize()
        while (time.perf_counter() - t0) * 1e3 < args.warmup_floor_ms:
            for _ in range(16):
                n += run(n)
            torch.cuda.synchronize()
        return n

    def time_decode(pools, steps, warmup, into=False):
        """Warm-up, then --blocks timed blocks of `steps` back-to-back
        launches, each bracketed by HIP events on the launch stream (no event
        between launches); the blocks follow each other without a host
        synchronisation.  Returns per-block ms per launch and the warm-up
        launch count."""
        if args.graph:
            return time_decode_graph(pools, steps, warmup, into)
        stream = torch.cuda.current_stream()

        def run(t):
            launch(pools, t, into)
            return 1
        n_warm = warm_up(pools, warmup, into, run)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.blocks)]
        t = n_warm
        for start, end in ev:
            start.record(stream)
            for _ in range(steps):
                launch(pools, t, into)
                t += 1
            end.record(stream)
        torch.cuda.synchronize()
        return [start.elapsed_time(end) / steps for start, end in ev], n_warm

    def time_decode_graph(pools, steps, warmup, into=False):
        """The same launches captured once in a HIP graph (one pass over the
        input window and the pools) and replayed: the launch cost of the
        host binding leaves the timed region, which matters for the small
        workloads whose kernels last a few microseconds."""
        period = len(window) * len(pools) // math.gcd(len(window), len(pools))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # eager pass on the capture stream first
            for t in range(period):
                launch(pools, t, into)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for t in range(period):
                launch(pools, t, into)
        reps = max(1, -(-steps // period))

        def run(_t):
            graph.replay()
            return period
        n_warm = warm_up(pools, warmup, into, run) + period  # + the eager pass
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.blocks)]
        for start, end in ev:
            start.record(stream)
            for _ in range(reps):
                graph.replay()
            end.record(stream)
        torch.cuda.synchronize()
        del graph
        return [start.elapsed_time(end) / (reps * period) for start, end in ev], n_warm

    def measure(fmt_name: str, fmt: int, n8: int, npools: int, steps: int, warmup: int,
                into: bool = False, gated: bool = False, out_bf16: bool = False):
        nonlocal gates, o
        o = torch.empty((B, hv, d), dtype=torch.bfloat16, device="cuda") if out_bf16 else o_f32
        if gated:  # per-key-row gates of the KDA form, one per window step (drawn first,
            gates = gate_window()  # so that no host work separates set-up and warm-up)
        pools = make_pools(fmt, n8, npools, gated)
        blocks, n_warm = time_decode(pools, steps, warmup, into)
        gates = None
        o = o_f32
        mean_ms = sorted(blocks)[len(blocks) // 2]  # the median block
        nbytes = algorithmic_bytes(fmt_name, B, hv, hk, d, n8, in_el, gated, 2 if out_bf16 else 4)
        if fmt in (stq.FMT_ALLOC, stq.FMT_ALLOC_REFIT):
            refit_ = fmt == stq.FMT_ALLOC_REFIT
            # segment + row factors, plus the state's own column factors when refit
            unit = alloc_unit_bytes(alloc_cal[(gated, refit_)][0], d) + (4 * d if refit_ else 0)
            nbytes = int(2 * unit * B * hv) + algorithmic_bytes("fp32", B, hv, hk, d, 0, in_el,
                                                                 gated) - 2 * 4 * d * d * B * hv
        res = dict(updates_per_s=B * hv / (mean_ms / 1e3), ms_per_step=mean_ms,
                   kernel_ms_mean=mean_ms, blocks_ms_per_step=blocks, warmup_launches=n_warm,
                   algorithmic_bytes_per_launch=nbytes,
                   hbm_gbps=nbytes / (mean_ms / 1e3) / 1e9,
                   frac_of_peak=nbytes / (mean_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                   pools=npools, pool_bytes=int(pools[0].buffer.numel()),
                   mode="double_buffered" if into else "in_place")
        del pools
        torch.cuda.empty_cache()
        return res

    # ------------------------------------------------------------ main run --
    into = args.mode == "double_buffered"
    main_res = measure("mixed", stq.FMT_MIXED48, w.n8, args.pools, args.steps, args.warmup, into)
    log(f"[bench] main: {main_res['updates_per_s'] / 1e6:.1f} M updates/s, "
        f"{main_res['hbm_gbps']:.0f} GB/s ({100 * main_res['frac_of_peak']:.1f}% of peak)")

    variants = {}
    copy_gbps = None
    if not args.only_decode and not args.no_variants:
        chosen = None if args.variants is None else set(args.variants.split(","))
        want = lambda name: chosen is None or name in chosen  # noqa: E731
        other = "in_place" if into else "double_buffered"
        if want(other):
            variants[other] = measure("mixed", stq.FMT_MIXED48, w.n8, args.pools, args.steps,
                                      args.warmup, not into)
        if not into and want("single_pool_as_stated"):
            variants["single_pool_as_stated"] = measure("mixed", stq.FMT_MIXED48, w.n8, 1,
                                                        args.steps, args.warmup)
        if w.n8 != 16 and want("mix_4p5bit_n8_16"):
            variants["mix_4p5bit_n8_16"] = measure("mixed", stq.FMT_MIXED48, 16, args.pools,
                                                   args.steps, args.warmup)
        if want("int8row"):
            variants["int8row"] = measure("int8row", stq.FMT_INT8ROW, d, args.pools, args.steps,
                                          args.warmup)
        if d == 128 and w.n8 % 16 == 0 and want("refit_column_factors"):
            variants["refit_column_factors"] = measure("refit", stq.FMT_REFIT, w.n8, args.pools,
                                                       args.steps, args.warmup)
        if want("bf16_readout"):
            variants["bf16_readout"] = measure("mixed", stq.FMT_MIXED48, w.n8, args.pools,
                                               args.steps, args.warmup, out_bf16=True)
        if want("row_gate_kda"):
            variants["row_gate_kda"] = measure("mixed", stq.FMT_MIXED48, w.n8, args.pools,
                                               args.steps, args.warmup, gated=True)
        # ragged rows (FP16 pivots + 8/6/4/2 bits from the lifetime-aware
        # assignment): scalar gate, KDA row gate, and the scalar gate with the
        # column refit, each with its own calibration
        for name, gated_, refit_ in (("alloc_pivots", False, False),
                                     ("alloc_pivots_kda_gate", True, False),
                                     ("alloc_pivots_refit", False, True)):
            if not want(name):
                continue
            t1 = time.time()
            alloc_cal[(gated_, refit_)] = calibrate_alloc(
                torch, stq, S0, lambda t: alloc_cal_inputs(t, gated_), B=B, hv=hv, hk=hk, d=d,
                steps=w.calib_steps, nominal=alloc_nominal(w), n_pivot=alloc_pivots(hv, d),
                gated=gated_, refit=refit_)
            cnt = alloc_cal[(gated_, refit_)][0]
            res = measure("mixed", stq.FMT_ALLOC_REFIT if refit_ else stq.FMT_ALLOC, w.n8,
                          args.pools, args.steps, args.warmup, gated=gated_)
            res["rows_by_width"] = {str(b): int(cnt[:, k].sum())
                                    for k, b in enumerate((16, 8, 6, 4, 2))}
            res["bits_per_value"] = 8 * alloc_unit_bytes(cnt, d) / (d * d)
            res["calibration_s"] = time.time() - t1
            variants[name] = res
        if want("fp32_state"):
            variants["fp32_state"] = measure("fp32", stq.FMT_FP32, 0, 2, args.steps, args.warmup)
        for k_, v_ in variants.items():
            log(f"[bench] {k_}: {v_['updates_per_s'] / 1e6:.1f} M updates/s, "
                f"{v_['hbm_gbps']:.0f} GB/s")
    if args.with_copy or (not args.only_decode and not args.no_variants):
        copy_gbps = measure_copy(torch, stq)
        log(f"[bench] streaming copy ceiling (1 GiB -> 1 GiB): {copy_gbps:.0f} GB/s")

    # ------------------------------------------------------- CPU baseline --
    cpu = None
    if not args.no_cpu_baseline and not args.only_decode:
        cpu = cpu_baseline(np, wl, w, B, hv, d)

    # -------------------------------------------------------- roofline etc --
    traffic = None
    if COUNTERS_FILE.exists():
        try:
            cnt = json.loads(COUNTERS_FILE.read_text())
            sha = decode_source_sha256()
            if cnt.get("decode_source_sha256") == sha and cnt.get("workload") == w.name:
                traffic = cnt.get("hbm_bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    achieved = main_res["hbm_gbps"]
    line = {
        "metric": "quantized state-updates/s (seq*head*step) + % of MI355X peak HBM GB/s",
        "value": main_res["updates_per_s"],
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "timing": {"blocks": args.blocks, "steps_per_block": args.steps,
                   "blocks_ms_per_step": main_res["blocks_ms_per_step"],
                   "statistic": "median block",
                   "warmup_launches": main_res["warmup_launches"],
                   "warmup_floor_ms": args.warmup_floor_ms},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={B}, Hv={hv} value heads over Hk={hk} key heads, "
                        f"d_k=d_v={d}, n8={w.n8} 8-bit rows + {d - w.n8} 4-bit rows per head "
                        f"({8 * unit_state_bytes('mixed', d, w.n8) / (d * d):.2f} bits/value), "
                        f"{w.dtype} q/k/v, {args.pools} rotated pools (MALL-cold), "
                        f"{main_res['mode'].replace('_', '-')} state update",
            "mode": main_res["mode"], "launch": "hip_graph" if args.graph else "eager",
            "global_batch": B, "heads_v": hv, "heads_k": hk, "d": d, "n8": w.n8,
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "cpu_baseline": cpu,
        "hbm_gbps": achieved,
        "kernel_ms_mean": main_res["kernel_ms_mean"],
        "algorithmic_bytes_per_launch": main_res["algorithmic_bytes_per_launch"],
        "copy_ceiling_gbps": copy_gbps,
        "variants": variants,
    }
    print(json.dumps(line), flush=True)


def device_inputs(torch, w, layer: int, t: int, calibration: bool = False):
    """One step of inputs drawn on the device (same laws as the host generator:
    q, k ~ N(0, 1) L2-normalised, v ~ N(0, 1), alpha ~ U(lo, 1),
    beta = sigmoid(N(0, 1)); bf16 by round-to-nearest-even), for workloads too
    large to draw on the host every step."""
    seed = (w.calib_seed if calibration else w.seed) * 1_000_003 + layer * 10_007 + t
    g = torch.Generator(device="cuda").manual_seed(seed)
    B, hk, hv, d = w.B, w.hk, w.hv, w.d
    q = torch.randn(B, hk, d, device="cuda", generator=g)
    k = torch.randn(B, hk, d, device="cuda", generator=g)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(B, hv, d, device="cuda", generator=g)
    a = torch.rand(B, hv, device="cuda", generator=g) * (1.0 - w.alpha_lo) + w.alpha_lo
    b = torch.sigmoid(torch.randn(B, hv, device="cuda", generator=g))
    if w.dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q.contiguous(), k.contiguous(), v.contiguous(), a.contiguous(), b.contiguous()


def device_initial_state(torch, w, layer: int):
    """S0 [B][Hv][d][d] on the device with the workload's law (outlier rows and
    columns from per-head log-normal factors)."""
    g = torch.Generator(device="cuda").manual_seed(w.seed * 1_000_003 + layer * 10_007 + 999_983)
    S = torch.randn(w.B, w.hv, w.d, w.d, device="cuda", generator=g)
    if w.s0 == "zero":
        return S.zero_()
    if w.s0 == "normal":
        return S.mul_(w.s0_scale)
    ra = torch.exp(torch.randn(1, w.hv, w.d, 1, device="cuda", generator=g) * w.outlier_sigma)
    ce = torch.exp(torch.randn(1, w.hv, 1, w.d, device="cuda", generator=g) * w.outlier_sigma)
    return S.mul_(ra).mul_(ce)


def run_drift(args, np, torch, stq, wl, w) -> dict:
    """Drift of the packed (quantized) trajectory against the FP32-state
    trajectory from the same S0 with the same inputs: relative Frobenius error
    of the dequantized state and relative L2 error of the readout, per layer
    at checkpoints, aggregated over layers.  Small workloads draw inputs on
    the host (the generator the tests use); the stacked one on the device."""
    layers = args.layers or w.layers
    T = args.drift_steps or w.T
    if T >= 512:
        checkpoints = sorted(set(list(range(256, T + 1, 256)) + [T]))
    else:
        checkpoints = sorted(set([1, 2, max(1, T // 4), max(1, T // 2), T]))
    # one layer small enough to draw on the host every step
    host = layers == 1 and w.units * w.d <= 1 << 22
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731

    def gate_for(layer, t, calibration):
        seed = w.calib_seed if calibration else w.seed
        if host:
            return dev(wl.draw_gate(w.B, w.hv, w.d, seed=seed, step=t, layer=layer))
        g = torch.Generator(device="cuda").manual_seed(seed * 1_000_003 + layer * 10_007 + t
                                                       + 500_009)
        return torch.sigmoid(torch.randn(w.B, w.hv, w.d, device="cuda", generator=g) * 1.5
                             + 2.5).contiguous()

    def inputs(layer, t, calibration=False):
        if not host:
            x = device_inputs(torch, w, layer, t, calibration)
        else:
            h = wl.workload_inputs(w, t, calibration=calibration, layer=layer)
            if h.dtype == "bf16":
                cv = lambda bits: dev(bits.view(np.int16)).view(torch.bfloat16)  # noqa: E731
                x = cv(h.q_bits), cv(h.k_bits), cv(h.v_bits), dev(h.alpha), dev(h.beta)
            else:
                x = dev(h.q), dev(h.k), dev(h.v), dev(h.alpha), dev(h.beta)
        # with --gate, the fourth entry is the row gate [B][Hv][d] instead of alpha
        if args.gate:
            x = (x[0], x[1], x[2], gate_for(layer, t, calibration), x[4])
        return x

    def step(st, x, o=None):
        if args.gate:
            return st.decode_step_gated(*x, o=o)
        return st.decode_step(*x, o=o)

    t0 = time.time()
    quant, ref = [], []
    alloc_counts = []
    for layer in range(layers):
        S0 = dev(wl.initial_state(w, layer=layer)) if host else device_initial_state(torch, w, layer)
        fp = stq.State(stq.Geometry(w.B, w.hv, w.hk, w.d, 0, stq.FMT_FP32))
        fp.pack(S0)
        n8 = w.n8
        if w.calib_seed is None:  # all rows 8-bit, c = 1 (uniform rowwise INT8)
            qs = stq.State(stq.Geometry(w.B, w.hv, w.hk, w.d, w.d, stq.FMT_INT8ROW))
        elif args.alloc:
            counts, ca, pa, w2a = calibrate_alloc(
                torch, stq, S0, lambda t: inputs(layer, t, calibration=True), B=w.B, hv=w.hv,
                hk=w.hk, d=w.d, steps=w.calib_steps, nominal=alloc_nominal(w),
                n_pivot=alloc_pivots(w.hv, w.d), gated=args.gate, refit=args.refit)
            fmt = stq.FMT_ALLOC_REFIT if args.refit else stq.FMT_ALLOC
            qs = stq.State(stq.Geometry(w.B, w.hv, w.hk, w.d, 0, fmt,
                                        nominal_bits=alloc_nominal(w),
                                        n_pivot=alloc_pivots(w.hv, w.d)))
            qs.set_alloc_layout(counts, ca, pa)
            if args.refit:
                qs.w2.copy_(w2a)
            alloc_counts.append(counts)
        else:
            fmt = stq.FMT_REFIT if args.refit else stq.FMT_MIXED48
            cal = stq.State(stq.Geometry(1, w.hv, w.hk, w.d, n8, fmt))
            cal.calibrate(None, stq.CAL_RESET)
            if args.refit:
                cal.calibrate_impact(None, None, None, None, stq.CAL_RESET)
            fpc = stq.State(stq.Geometry(w.B, w.hv, w.hk, w.d, 0, stq.FMT_FP32))
            fpc.pack(S0)
            for t in range(w.calib_steps):
                x = inputs(layer, t, calibration=True)
                step(fpc, x)
                if args.refit and args.gate:
                    cal.calibrate_impact(x[0], x[1], None, x[4], 0, gate=x[3])
                elif args.refit:
                    cal.calibrate_impact(x[0], x[1], x[3], x[4], 0)
                last = t == w.calib_steps - 1
                cal.calibrate(fpc.s32, stq.CAL_COLS | (stq.CAL_ROWS if last else 0))
            cal.calibrate(None, stq.CAL_FINALIZE)
            qs = stq.State(stq.Geometry(w.B, w.hv, w.hk, w.d, n8, fmt))
            qs.set_calibration(cal.c.clone(), cal.perm.clone())
            if args.refit:
                cal.calibrate_impact(None, None, None, None, stq.CAL_FINALIZE)
                qs.w2.copy_(cal.w2)
            del fpc, cal
        qs.pack(S0)
        del S0
        quant.append(qs)
        ref.append(fp)
        if layer % 8 == 7:
            torch.cuda.synchronize()
            log(f"[drift] {layer + 1} of {layers} layers set up ({time.time() - t0:.0f}s)")
    torch.cuda.synchronize()
    log(f"[drift] {w.name}: {layers} layer(s) packed and calibrated in {time.time() - t0:.1f}s")

    oq = torch.empty(w.B, w.hv, w.d, device="cuda")
    of = torch.empty_like(oq)
    points = []
    o_err_sum = torch.zeros(layers, device="cuda", dtype=torch.float64)
    o_ref_sum = torch.zeros_like(o_err_sum)
    for t in range(1, T + 1):
        check = t in checkpoints
        o_rel = []
        for layer in range(layers):
            x = inputs(layer, t - 1)
            step(quant[layer], x, o=oq)
            step(ref[layer], x, o=of)
            err = (oq - of).double().pow(2).sum()
            nrm = of.double().pow(2).sum()
            o_err_sum[layer] += err
            o_ref_sum[layer] += nrm
            if check:
                o_rel.append(float((err / nrm).sqrt()))
        if t % 64 == 0 and not check:
            log(f"[drift] step {t} of {T} ({time.time() - t0:.0f}s)")
        if check:
            s_rel = []
            for layer in range(layers):
                Sq = quant[layer].dequant()
                Sf = ref[layer].s32
                s_rel.append(float((Sq - Sf).double().norm() / Sf.double().norm()))
                del Sq
            points.append(dict(step=t, state_rel_fro_mean=float(np.mean(s_rel)),
                               state_rel_fro_max=float(np.max(s_rel)),
                               readout_rel_l2_mean=float(np.mean(o_rel)),
                               readout_rel_l2_max=float(np.max(o_rel))))
            log(f"[drift] step {t}: state rel Frobenius mean {points[-1]['state_rel_fro_mean']:.3e}"
                f" max {points[-1]['state_rel_fro_max']:.3e}, readout rel L2 mean "
                f"{points[-1]['readout_rel_l2_mean']:.3e} ({time.time() - t0:.0f}s)")
    o_all = (o_err_sum / o_ref_sum).sqrt().cpu().numpy()
    return {"drift": {"workload": w.name, "layers": layers, "steps": T,
                      "inputs": "host generator" if host else "device generator",
                      "state": ("int8row" if w.calib_seed is None
                                else ("ragged rows (FP16 pivots, 8/6/4/2 bits)" if args.alloc
                                      else "packed") + (", refit column factors" if args.refit
                                                        else "")),
                      "rows_by_width": ({str(b): int(sum(cn[:, k].sum() for cn in alloc_counts))
                                         for k, b in enumerate((16, 8, 6, 4, 2))}
                                        if alloc_counts else None),
                      "bits_per_value": (8 * float(np.mean([alloc_unit_bytes(cn, w.d)
                                                            for cn in alloc_counts])) / w.d ** 2
                                         if alloc_counts else None),
                      "n8": w.n8 if w.calib_seed is not None else w.d,
                      "gate": "per key row (KDA form)" if args.gate else "scalar",
                      "checkpoints": points,
                      "readout_rel_l2_over_all_steps_mean": float(np.mean(o_all)),
                      "readout_rel_l2_over_all_steps_max": float(np.max(o_all))}}


if __name__ == "__main__":
    main()
