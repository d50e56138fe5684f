"""Throughput of the fixed-cost drafting path on one MI355X.

    python bench.py [--gpus 1] [--steps 256] [--warmup 16] [--workload q3_8b_128k]

A step is one drafting round for all C sequences: greedy verification of the
drafted block, append of the accepted rows + incremental summary update, and
the drafter's block attention (LongSpark paper page, Fig. 2).  The headline
workload is the Qwen3-8B-shaped tapped layer at concurrency 16 with a 128K
prefix per sequence; the same state is also swept over 4K..128K prefixes
(first L0 rows of the same allocation) to show the round cost is flat in the
prefix while the one-shot summary init grows linearly.

Inputs are synthetic and seeded (fixed_cost_drafter_amd.workload) and are
resident in HBM before timing starts.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
HIDDEN = 4096                  # target hidden size of the Qwen3-8B-shaped layer (boundary state)
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
_CS = "fixed_cost_drafter_amd/csrc/"
KERNEL_SOURCES = {
    "verify": _CS + "verify.hip",
    "append": (_CS + "append.hip", _CS + "merge_ops.hpp"),
    "draft": (_CS + "draft.hip", _CS + "draft_ops.hpp"),
    "init": _CS + "init.hip",
    "verify_attention": _CS + "verify_attn.hip",
    "verify_sampling": _CS + "sampling.hip",
    "verify_append": (_CS + "verify.hip", _CS + "append.hip", _CS + "merge_ops.hpp"),
    "update_draft": (_CS + "round.hip", _CS + "draft_ops.hpp", _CS + "merge_ops.hpp"),
    "round": (_CS + "verify.hip", _CS + "round.hip", _CS + "draft_ops.hpp", _CS + "merge_ops.hpp"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed, so
    that a comment or layout edit leaves a kernel's hash unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(rel) -> str:
    """Hash of the code (not the comments) of a kernel's sources and the
    shared headers: recorded with each profile, compared before a profile's
    figures are reported for the kernel as it now is."""
    h = hashlib.sha256()
    rels = rel if isinstance(rel, tuple) else (rel,)
    for p in (*rels, "fixed_cost_drafter_amd/csrc/common.hpp", "fixed_cost_drafter_amd/csrc/accept.hpp"):
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic work per launch (what the method must move / compute)
# ---------------------------------------------------------------------------
def algorithmic(wl, mean_tau: float, L0: int) -> dict:
    e = 2 if wl.dtype == "bf16" else 4
    units = wl.C * wl.Hkv
    G = wl.G
    verify = wl.C * (wl.B + 1) * wl.V * e + wl.C * wl.B * 4 + wl.C * (wl.B + 2) * 4
    rows = wl.C * mean_tau * wl.Hkv * wl.d * e * 2            # new k, v rows read
    append = (rows * 2                                          # read + ring write
              + units * wl.S * (2 * wl.d + 2) * 4 * 2           # fp32 state read + write
              + units * wl.S * wl.d * e * 2                     # slot k, v write
              + wl.Hkv * wl.S * wl.d * e)                       # slot queries
    nkeys = wl.W + wl.S + wl.B
    draft = (units * nkeys * wl.d * e * 2                       # keys + values
             + 2 * wl.C * wl.B * wl.Hq * wl.d * e               # q in, out
             + wl.C * wl.W * 4)                                 # ring positions
    draft_flop = units * 4 * wl.B * G * nkeys * wl.d
    init = units * L0 * wl.d * e * 2                            # the prefix, once
    init_flop = units * L0 * 6 * wl.S * wl.d
    # update and draft in one launch: the merged slots never leave the chip
    update_draft = append + draft - units * wl.S * wl.d * e * 2
    return dict(verify=verify, append=append, draft=draft, draft_flop=draft_flop,
                update_draft=update_draft, init=init, init_flop=init_flop,
                round=verify + update_draft)


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
# kernels that make up one call of each entry point: substrings of their
# names (a tuple: all of its substrings)
ENTRY_KERNELS = {
    "verify": ("verify_partial", "verify_finalize"),
    "verify_append": ("verify_partial", ("append_units", "true>")),
    "round": ("verify_partial", "update_draft"),
    "update_draft": ("update_draft",),
    "verify_sampling": ("samp_stats", "samp_decide_sums", "samp_draw"),
    "append": (("append_units", "false>"), "len_snapshot", "append_kernel"),
    "draft": ("draft_direct", "draft_combine", "draft_generic"),
    "verify_attention": ("attn_mfma_partial", "attn_combine", "attn_generic"),
    "init": ("init_mfma32_partial", "init_generic_partial", "init_finalize"),
}
CALIB_BYTES = 512 << 20        # the streaming copy used to scale the counters
CALIB_KERNEL = "neg_kernel"


def copy_calibration(dev):
    """One plain streaming copy of known size (reads and writes CALIB_BYTES).

    Run before timing so that a rocprofv3 --pmc pass over this program sees it
    and can scale FETCH_SIZE / WRITE_SIZE to bytes.
    """
    import torch
    src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def stream_reference(dev, reps=20) -> dict:
    """What a plain library streaming kernel (torch.neg: read n bytes, write n)
    reaches on this GPU at the round's scale (64 MiB each way, inputs resident
    in the last-level cache after the first rep) and at 512 MiB (HBM): the
    practical ceiling beside the 8 TB/s peak.  Events over reps back-to-back
    launches."""
    import torch
    out = {}
    for mib in (64, 512):
        src = torch.ones((mib << 20) // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            torch.neg(src, out=dst)
        z.record()
        z.synchronize()
        t = a.elapsed_time(z) * 1e-3 / reps
        out[f"copy_{mib}MiB_gb_per_s"] = round(2 * (mib << 20) / t / 1e9, 1)
        del src, dst
    return out


def mfma_reference(dev, n=8192, reps=10) -> dict:
    """What a tuned library bf16 GEMM (torch.mm, n x n x n, contiguous
    operands) reaches on this GPU: the practical dense-MFMA ceiling beside the
    2.5 PFLOP/s datasheet peak.  Events over reps back-to-back products.  Run
    after every other timing: its power draw lowers the clock of what follows."""
    import torch
    a = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    b = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.mm(a, b, out=c)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    tf = 2.0 * n ** 3 / t / 1e12
    del a, b, c
    return dict(gemm=f"{n}x{n}x{n} bf16 torch.mm", tflop_per_s=round(tf, 1),
                frac_of_peak=round(tf / MFMA_BF16_PEAK_TFS, 4))


def load_traffic(kernel: str):
    """HBM bytes per call of an entry point from the committed PMC summary, if current."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
        ent = t.get("entry_points", {}).get(kernel)
        if not ent or ent.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
            return None
        return int(ent["fetch_bytes"] + ent["write_bytes"])
    except (OSError, ValueError, KeyError, TypeError):
        return None


def summarize_traffic(fetch_dir: str, write_dir: str, command: str) -> dict:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; csv) into bytes per call.

    Both counters are KiB per dispatch.  They are scaled by what the same
    counter reads for the calibration copy (CALIB_BYTES read and written), so
    the figures are bytes as a plain copy would count them.
    """
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = {}
        for fn in files:
            with open(fn, newline="") as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]) * 1024)
        return vals

    out = {"command": command, "entry_points": {}, "kernels": {}}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        vals = per_kernel(d, counter)
        calib = [v for n, vs in vals.items() if CALIB_KERNEL in n for v in vs]
        if not calib:
            raise SystemExit(f"calibration copy not found in the {counter} run")
        factor = CALIB_BYTES / max(calib)
        out[f"{key}_scale"] = round(factor, 4)
        out[f"{key}_calibration_raw_bytes"] = max(calib)
        # a second point: the 64 MiB copies of the streaming reference (each
        # reads and writes 64 MiB), if the run made them; their scale should
        # match the 512 MiB copy's
        small = sorted(v for v in calib if v < 0.5 * max(calib))
        if small:
            out[f"{key}_scale_64MiB"] = round((64 << 20) / small[len(small) // 2], 4)
            out[f"{key}_calibration_64MiB_dispatches"] = len(small)
        for name, vs in vals.items():
            short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            ent = out["kernels"].setdefault(short, {})
            ent["dispatches"] = len(vs)
            ent[f"{key}_bytes"] = statistics.mean(vs) * factor
    for entry, parts in ENTRY_KERNELS.items():
        f = w = 0.0
        seen = []
        for short, ent in out["kernels"].items():
            if any(all(q in short for q in (p if isinstance(p, tuple) else (p,))) for p in parts):
                f += ent.get("fetch_bytes", 0.0)
                w += ent.get("write_bytes", 0.0)
                seen.append(short)
        if seen:
            out["entry_points"][entry] = dict(fetch_bytes=round(f), write_bytes=round(w), kernels=seen,
                                              source_hash=source_hash(KERNEL_SOURCES[entry]))
    return out


COUNTERS_JSON = os.path.join(ROOT, "profiles", "counters.json")
MFMA_COUNTERS = ("MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE", "SQ_WAIT_INST_ANY", "SQ_WAVES")


def summarize_counters(dirs, command: str) -> dict:
    """rocprofv3 --pmc runs (csv) -> mean value per dispatch of each counter, per kernel."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for fn in files:
            with open(fn, newline="") as f:
                for row in csv.DictReader(f):
                    short = row["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                    vals.setdefault(short, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    out = {"command": command, "kernels": {}, "entry_points": {}}
    for short, cs in vals.items():
        out["kernels"][short] = {k: statistics.mean(v) for k, v in cs.items()}
        out["kernels"][short]["dispatches"] = max(len(v) for v in cs.values())
    for entry, parts in ENTRY_KERNELS.items():
        # the entry point's main kernel: the first of its list, and of the
        # kernels that match it (instances of one template) the one whose
        # dispatches are longest (GRBM_GUI_ACTIVE)
        first = parts[0]
        hits = [(short, ent) for short, ent in out["kernels"].items()
                if all(q in short for q in (first if isinstance(first, tuple) else (first,)))]
        if hits:
            short, ent = max(hits, key=lambda se: se[1].get("GRBM_GUI_ACTIVE", 0.0))
            out["entry_points"][entry] = dict(kernel=short, source_hash=source_hash(KERNEL_SOURCES[entry]),
                                              **{k: v for k, v in ent.items() if k != "dispatches"})
    return out


def executed_flop(entry: str):
    """bf16 MFMA flops one call of the entry point issues, from the committed
    counters (SQ_INSTS_VALU_MFMA_MOPS_BF16, units of 512 flops, summed over the
    call's kernels, one dispatch each), if they are current; else None."""
    if not os.path.exists(COUNTERS_JSON):
        return None
    try:
        with open(COUNTERS_JSON) as f:
            c = json.load(f)
        ent = c.get("entry_points", {}).get(entry)
        if not ent or ent.get("source_hash") != source_hash(KERNEL_SOURCES[entry]):
            return None
        parts = ENTRY_KERNELS[entry]
        mops = [k.get("SQ_INSTS_VALU_MFMA_MOPS_BF16") for short, k in c["kernels"].items()
                if any(all(q in short for q in (p if isinstance(p, tuple) else (p,))) for p in parts)]
        if not mops or any(m is None for m in mops):
            return None
        return 512.0 * sum(mops)
    except (OSError, ValueError, KeyError, TypeError):
        return None


def load_counters(entry: str):
    """Counter means of an entry point's main kernel from the committed summary, if current."""
    if not os.path.exists(COUNTERS_JSON):
        return None
    try:
        with open(COUNTERS_JSON) as f:
            ent = json.load(f).get("entry_points", {}).get(entry)
        if not ent or ent.get("source_hash") != source_hash(KERNEL_SOURCES[entry]):
            return None
        return ent
    except (OSError, ValueError, KeyError, TypeError):
        return None


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------
def run_gpu(args, wl):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd import workload as WLM
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round

    dev = "cuda"
    torch.cuda.set_device(0)
    copy_calibration(dev)
    stream_ref = stream_reference(dev)
    log(f"streaming copy reference: {stream_ref}")
    rows = max(WLM.SWEEP_L0) if args.sweep else wl.L0
    rows = max(rows, wl.L0)
    t0 = time.time()
    K_host, V_host = WLM.prefix(wl, L0=rows, threads=args.threads, log=log)
    log(f"prefix {K_host.shape} drawn in {time.time() - t0:.1f}s")
    runner = PathRunner(wl, K_host, V_host, max_L0=rows, device=dev)
    del K_host, V_host
    n_rounds = args.warmup + args.steps
    pool = []
    for k in range(min(WLM.pool_size(wl), n_rounds)):
        logits, planted = WLM.logits_entry(wl, k)
        pool.append((LB.to_device(logits, dev), planted))
    rounds = [upload_round(WLM.round_inputs(wl, r, pool[r % len(pool)][1]), dev)
              for r in range(n_rounds)]
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.time() - t0:.1f}s)")
    stream = torch.cuda.current_stream()

    def time_init(L0, reps=5):
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            runner.init(L0)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return statistics.median(ts)

    def bind_all(rn):
        """every round's calls marshalled once, so the timed loop only issues them"""
        return [rn.bind_round(pool[r % len(pool)][0], rounds[r], stream) for r in range(n_rounds)]

    def run_rounds(L0, rn=None, passes=args.passes):
        """``passes`` timed passes of args.steps rounds each (after args.warmup
        untimed rounds), every pass bracketed by a device synchronisation on
        both sides; the median pass by wall clock is reported.  Between the
        summary init and the warmup, args.heat untimed rounds (the inputs
        cycled) let the clock leave the init's power-limited level: a serving
        loop runs rounds back to back, not right after a prefill."""
        runner_ = rn if rn is not None else runner
        runner_.init(L0)
        calls = bind_all(runner_)
        for r in range(args.heat):
            calls[r % n_rounds]()
        for r in range(args.warmup):
            calls[r]()
        torch.cuda.synchronize()
        res = []
        for _ in range(passes):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            e0.record(stream)
            for r in range(args.warmup, n_rounds):
                calls[r]()
            t_issue = time.perf_counter()
            e1.record(stream)
            torch.cuda.synchronize()
            t_end = time.perf_counter()
            res.append(dict(wall_s=t_end - t_start, issue_s=t_issue - t_start,
                            gpu_s=e0.elapsed_time(e1) * 1e-3))
        res_sorted = sorted(res, key=lambda x: x["wall_s"])
        med = dict(res_sorted[len(res_sorted) // 2])
        med["passes_wall_s"] = [x["wall_s"] for x in res]
        med["passes_gpu_s"] = [x["gpu_s"] for x in res]
        return med

    def run_graph(L0):
        """K rounds captured once in a HIP graph, replayed; the same inputs as run_rounds."""
        runner.init(L0)
        calls = bind_all(runner)
        for r in range(args.warmup):
            calls[r]()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            cap = bind_all_on(runner, side)
            g.capture_begin()
            for r in range(args.warmup, n_rounds):
                cap[r]()
            g.capture_end()
        torch.cuda.current_stream().wait_stream(side)
        runner.init(L0)  # capture does not execute: replay from the same state
        for r in range(args.warmup):
            calls[r]()
        torch.cuda.synchronize()
        walls = []
        for _ in range(args.passes):
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t_start)
        return dict(wall_s=statistics.median(walls))

    def bind_all_on(rn, strm):
        return [rn.bind_round(pool[r % len(pool)][0], rounds[r], strm) for r in range(n_rounds)]

    out = {}
    out["stream_reference"] = stream_ref
    # headline: the workload's own prefix
    out["steps"] = args.steps
    main = run_rounds(wl.L0)
    taus = LB.to_host(runner.buf.tau)

    def back_to_back(fn, n):
        """average launch duration: n consecutive launches between two events"""
        for i in range(4):
            fn(i)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        z.record(stream)
        z.synchronize()
        return a.elapsed_time(z) * 1e-3 / n

    # each entry point of the round timed over its own region of back-to-back
    # launches on the round's inputs (the state after the timed rounds)
    s_, b_ = runner.state, runner.buf
    P = len(pool)
    kern = dict(
        verify_s=back_to_back(lambda i: s_.verify_greedy(pool[i % P][0], rounds[i % n_rounds]["draft"],
                                                         b_.target_tok, b_.tau), args.steps),
        draft_s=back_to_back(lambda i: s_.draft_attention(rounds[i % n_rounds]["q"], rounds[i % n_rounds]["k_blk"],
                                                          rounds[i % n_rounds]["v_blk"], b_.out), args.steps),
        append_s=back_to_back(lambda i: s_.append_accepted(rounds[i % n_rounds]["k_new"],
                                                           rounds[i % n_rounds]["v_new"], b_.tau), args.steps),
    )
    # where the draft's bytes come from: the back-to-back calls above may find
    # its 80.8 MB working set in the 256 MB last-level cache (MALL); here each
    # call follows a 512 MiB copy that evicts L2 and MALL (events around the
    # draft call only)
    scrub_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    scrub_dst = torch.empty_like(scrub_src)
    cold = []
    for i in range(max(8, min(args.steps, 32))):
        scrub_dst.copy_(scrub_src)
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        s_.draft_attention(rounds[i % n_rounds]["q"], rounds[i % n_rounds]["k_blk"],
                           rounds[i % n_rounds]["v_blk"], b_.out)
        z.record(stream)
        cold.append((a, z))
    warm = []
    for i in range(max(8, min(args.steps, 32))):
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        s_.draft_attention(rounds[i % n_rounds]["q"], rounds[i % n_rounds]["k_blk"],
                           rounds[i % n_rounds]["v_blk"], b_.out)
        z.record(stream)
        warm.append((a, z))
    torch.cuda.synchronize()
    kern["draft_cold_s"] = statistics.median(a.elapsed_time(z) for a, z in cold) * 1e-3
    kern["draft_warm_single_s"] = statistics.median(a.elapsed_time(z) for a, z in warm) * 1e-3
    del scrub_src, scrub_dst
    # the fused call the rounds use (verification keys + update deriving tau);
    # the state keeps advancing, which the per-call cost does not depend on
    kern["verify_append_s"] = back_to_back(
        lambda i: s_.verify_append(pool[i % P][0], rounds[i % n_rounds]["draft"], b_.target_tok, b_.tau,
                                   rounds[i % n_rounds]["k_new"], rounds[i % n_rounds]["v_new"]),
        args.steps)
    # the round's two launches inside a run of rounds (ls_verify_keys, then
    # ls_update_draft: the launches of ls_verify_append_draft), events around
    # each on the launch stream, so each sees the caches as the round leaves
    # them (the key pass streams the logits through the MALL)
    split = [runner.bind_round_split(pool[r % P][0], rounds[r % n_rounds], stream)
             for r in range(args.steps)]
    for i in range(4):
        split[i][0]()
        split[i][1]()
    torch.cuda.synchronize()
    ev = []
    for i in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        split[i][0]()
        e[1].record(stream)
        split[i][1]()
        e[2].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    kern["verify_keys_event_s"] = statistics.mean(e[0].elapsed_time(e[1]) for e in ev) * 1e-3
    kern["update_draft_event_s"] = statistics.mean(e[1].elapsed_time(e[2]) for e in ev) * 1e-3
    def split_round(i):
        keys, upd = split[i % len(split)]
        keys()
        upd()
    kern["round_split_s"] = back_to_back(split_round, args.steps)
    # an event recorded between two launches lengthens the round by ~1.5 us
    # (the kernel trace has update_draft shorter than the per-launch events
    # say), so its time per launch is also taken as the difference of two
    # event-bracketed runs of back-to-back launches: whole rounds, and the
    # key passes alone
    kern["verify_keys_s"] = back_to_back(lambda i: split[i % len(split)][0](), args.steps)
    kern["update_draft_s"] = kern["round_split_s"] - kern["verify_keys_s"]
    out.update(main=main, kern=kern)
    if args.graph:
        out["graph"] = run_graph(wl.L0)
        log(f"graph replay: {args.steps / out['graph']['wall_s']:.0f} rounds/s")
    # the init is timed after the round passes, as in the sweep: right after
    # the streaming-copy reference (about 20 GB moved) the same init reads
    # 20-25% slower, at the clock those copies leave behind
    out["init_s"] = time_init(wl.L0)
    sweep = {}
    if args.sweep:
        for L0 in WLM.SWEEP_L0:
            it = time_init(L0)
            rr = run_rounds(L0)
            sweep[str(L0)] = dict(init_ms=round(it * 1e3, 4),
                                  rounds_per_s=round(args.steps / rr["wall_s"], 1),
                                  ms_per_round=round(rr["wall_s"] / args.steps * 1e3, 5))
            log(f"sweep L0={L0}: init {it*1e3:.3f} ms, {args.steps / rr['wall_s']:.0f} rounds/s")
    out["sweep"] = sweep
    out["state_bytes_per_seq"] = runner.state.state_bytes() // wl.C

    def per_call(fn, n):
        """mean duration of fn(i) over n calls, events on the launch stream"""
        for i in range(4):
            fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i in range(n):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(z) for a, z in ev) * 1e-3

    if not args.next:
        return out
    # the drafter's proposal at T = 0 over [C, B, V] logits
    drafter_logits = [t[:, :wl.B].contiguous() for t, _ in pool[:2]]
    draft_tok = torch.empty((wl.C, wl.B), dtype=torch.int32, device=dev)
    out["argmax_s"] = per_call(
        lambda i: runner.state.draft_argmax(drafter_logits[i % 2], draft_tok), args.steps)
    # the boundary state view: row tau-1 of [C, B+1, H] target states (H = 4096)
    hidden = torch.randn((wl.C, wl.B + 1, HIDDEN), device=dev).to(LB.torch_dtype(wl.dtype))
    hrow = torch.empty((wl.C, HIDDEN), dtype=hidden.dtype, device=dev)
    out["boundary_s"] = per_call(
        lambda i: runner.state.gather_boundary(hidden, runner.buf.tau, hrow), args.steps)
    # the target's verification attention over the whole context (the O(L)
    # cost per round that the drafter avoids): context L0 - B - 1 rows so that
    # the verified block is the last B + 1 rows of the resident prefix
    L_ctx = wl.L0 - wl.B - 1
    Lt = torch.full((wl.C,), L_ctx, dtype=torch.int32, device=dev)
    qv = LB.to_device(WLM.verify_queries(wl, 0), dev)
    ov = torch.empty_like(qv)
    out["vattn_L"] = L_ctx
    out["vattn_s"] = per_call(
        lambda i: runner.state.verify_attention(runner.k_prefix, runner.v_prefix, Lt, wl.L0, qv, ov),
        8)
    # sampled verification at T = 1 (speculative sampling): both logit tensors once
    tl_host, _ = WLM.logits_entry(wl, 0)
    samp = WLM.sampling_inputs(wl, 0, tl_host, temperature=1.0)
    dls = LB.to_device(samp["draft_logits"], dev)
    sd = {k: LB.to_device(samp[k], dev) for k in ("draft", "u_accept", "u_sample")}
    stoks = torch.empty((wl.C, wl.B + 1), dtype=torch.int32, device=dev)
    staus = torch.empty((wl.C,), dtype=torch.int32, device=dev)
    out["sampling_s"] = per_call(
        lambda i: runner.state.verify_sampling(pool[0][0], dls, sd["draft"], 1.0, sd["u_accept"],
                                               sd["u_sample"], stoks, staus), args.steps)
    out["sampling_tau"] = float(LB.to_host(staus).mean())
    del tl_host, samp, dls
    # one view switched off (cost side of the view ablations)
    abl = {}
    for name, kw in (("no_summary", dict(S=0, lambdas=())), ("no_window", dict(W=0))):
        wl2 = wl.with_(name=f"{wl.name}_{name}", **kw)
        rn2 = PathRunner(wl2, runner.k_prefix, runner.v_prefix, max_L0=rows, device=dev)
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rn2.init(wl.L0)
        z.record(stream)
        z.synchronize()
        rr = run_rounds(wl.L0, rn=rn2)
        abl[name] = dict(W=wl2.W, S=wl2.S, rounds_per_s=round(args.steps / rr["wall_s"], 1),
                         init_ms=round(a.elapsed_time(z), 4),
                         state_bytes_per_seq=rn2.state.state_bytes() // wl.C)
        log(f"ablation {name}: {abl[name]}")
        del rn2
    out["ablations"] = abl
    out["last_tau"] = taus.tolist()
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ---------------------------------------------------------------------------
_CPU = {}          # inputs of the sample, set before the worker processes fork
CPU_L_INIT = 1024  # prefix rows the oracle's state starts from (round cost does not depend on it)
CPU_POOL = 2       # logits tensors cycled by the sample
CPU_INPUTS = 32    # distinct round inputs cycled by the sample


def host_cpus() -> int:
    """CPUs this process may run on (the box's share, whatever nproc shows), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_rounds(seqs, n_rounds):
    """n_rounds full rounds (verify, append, draft attention) of sequences ``seqs``
    with the oracle; returns the seconds they took."""
    from oracle import longspark_oracle as O
    c0, c1 = seqs
    wl, u, logl = _CPU["wl"], _CPU["u"], _CPU["logl"]
    st = O.summary_init(u, logl, _CPU["Kp"][c0:c1], _CPU["Vp"][c0:c1], wl.W)
    t0 = time.perf_counter()
    for r in range(n_rounds):
        logits = _CPU["pool"][r % len(_CPU["pool"])][c0:c1]
        inp = _CPU["inputs"][r % len(_CPU["inputs"])]
        _, tau = O.verify_greedy(logits, inp["draft"][c0:c1])
        O.append_accepted(st, inp["k_new"][c0:c1], inp["v_new"][c0:c1], tau)
        O.draft_attention(st, inp["q"][c0:c1], inp["k_blk"][c0:c1], inp["v_blk"][c0:c1])
    return time.perf_counter() - t0


def _cpu_worker(job):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        return _cpu_rounds(*job)


def cpu_baseline(wl, budget_s: float):
    """The oracle timed on the host, before anything touches the GPU.

    Single thread: the whole batch in this process with one BLAS thread.
    All cores: the C sequences are independent, so host_cpus() worker processes
    (forked now, with no GPU context to inherit) each run the oracle's rounds
    on their share of the sequences with one BLAS thread; the rate is the
    rounds of the whole batch over the wall time of the slowest worker.
    """
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from fixed_cost_drafter_amd import workload as WLM
    t_setup = time.perf_counter()
    Kp, Vp = WLM.prefix(wl, L0=CPU_L_INIT, threads=4)
    pool, planted = [], []
    for k in range(CPU_POOL):
        lg, pl = WLM.logits_entry(wl, k)
        pool.append(lg)
        planted.append(pl)
    _CPU.update(wl=wl, u=WLM.slot_queries(wl), logl=WLM.log_lambda(wl), Kp=Kp, Vp=Vp, pool=pool,
                inputs=[WLM.round_inputs(wl, r, planted[r % CPU_POOL]) for r in range(CPU_INPUTS)])
    log(f"cpu_baseline: inputs ready ({time.perf_counter() - t_setup:.1f}s)")
    # one thread: rounds until about a third of the budget is spent
    with threadpool_limits(1):
        n1 = 2
        t1 = _cpu_rounds((0, wl.C), n1)
        while t1 < budget_s / 3 and n1 < 64:
            n1 *= 2
            t1 = _cpu_rounds((0, wl.C), n1)
    rate1 = n1 / t1
    log(f"cpu_baseline: 1 thread {rate1:.3f} rounds/s ({n1} rounds)")
    workers = min(host_cpus(), wl.C)
    per = -(-wl.C // workers)
    jobs_seqs = [(c, min(wl.C, c + per)) for c in range(0, wl.C, per)]
    workers = len(jobs_seqs)
    n_par = int(min(wl.rounds, max(8, budget_s * 2 / 3 * rate1 * workers)))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as p:
        t0 = time.perf_counter()
        secs = p.map(_cpu_worker, [(js, n_par) for js in jobs_seqs])
        wall = time.perf_counter() - t0
    rate_all = n_par / max(secs)
    log(f"cpu_baseline: {workers} processes {rate_all:.3f} rounds/s ({n_par} rounds, wall {wall:.1f}s)")
    _CPU.clear()
    return dict(value=round(rate_all, 3), unit="rounds/s", cores=workers, kind="oracle",
                sample=(f"{n_par} full rounds (verify + append + draft attention, all {wl.C} sequences "
                        f"and heads, V={wl.V}) of the {wl.name} shapes on {workers} worker processes "
                        f"(one BLAS thread each, {per} sequence(s) each; rate = rounds / slowest "
                        f"worker); the oracle's summary initialised over the first {CPU_L_INIT} prefix "
                        f"rows (round cost does not depend on the prefix); {CPU_POOL} logits tensors "
                        f"and {CPU_INPUTS} round inputs cycled; fp64 numpy"),
                single_thread=dict(value=round(rate1, 3), rounds=n1),
                host=dict(cpu_model=cpu_model(), cpus_usable=host_cpus(),
                          nproc=os.cpu_count(), thread_source="worker processes x 1 BLAS thread"))


def next_steps(wl, g) -> dict:
    """The steps beside the headline round: proposal argmax, boundary gather, view ablations."""
    e = 2 if wl.dtype == "bf16" else 4
    arg_bytes = wl.C * wl.B * wl.V * e + wl.C * wl.B * 4
    bnd_bytes = 2 * wl.C * HIDDEN * e + wl.C * 4
    res = {}
    for name, t, nbytes in (("draft_argmax", g["argmax_s"], arg_bytes),
                            ("gather_boundary", g["boundary_s"], bnd_bytes)):
        bw = nbytes / t / 1e9
        res[name] = dict(avg_us=round(t * 1e6, 3), alg_bytes=int(nbytes), gb_per_s=round(bw, 1),
                         hbm_frac=round(bw / HBM_PEAK_GBS, 4))
    res["gather_boundary"]["hidden"] = HIDDEN
    sbytes = wl.C * (2 * wl.B + 1) * wl.V * e + 2 * wl.C * wl.V * e
    bw = sbytes / g["sampling_s"] / 1e9
    res["verify_sampling"] = dict(avg_us=round(g["sampling_s"] * 1e6, 3), alg_bytes=int(sbytes),
                                  gb_per_s=round(bw, 1), hbm_frac=round(bw / HBM_PEAK_GBS, 4),
                                  temperature=1.0, mean_tau=round(g["sampling_tau"], 3))
    # verification attention: every context row's K and V, plus q and out
    vat = g["vattn_s"]
    vbytes = wl.C * (g["vattn_L"] + wl.B + 1) * wl.Hkv * wl.d * e * 2 + 2 * wl.C * (wl.B + 1) * wl.Hq * wl.d * e
    vflop = 4 * wl.C * wl.Hq * (wl.B + 1) * (g["vattn_L"] + wl.B + 1) * wl.d
    bw = vbytes / vat / 1e9
    res["verify_attention"] = dict(avg_us=round(vat * 1e6, 2), context_rows=g["vattn_L"],
                                   alg_bytes=int(vbytes), gb_per_s=round(bw, 1),
                                   hbm_frac=round(bw / HBM_PEAK_GBS, 4),
                                   tflop_per_s=round(vflop / vat / 1e12, 1),
                                   vs_draft_round=round(vat / (g["main"]["wall_s"] / g["steps"]), 1))
    res["ablations"] = g["ablations"]
    return res


def result_line(args, wl, g: dict, cpu) -> dict:
    """The one JSON line from the GPU measurements ``g`` (run_gpu's result plus
    the MFMA reference) and the oracle's CPU rate: the metric, the roofline of
    the round's longest kernel and every entry point's own figures."""
    from fixed_cost_drafter_amd import workload as WLM
    main_r = g["main"]
    value = args.steps / main_r["wall_s"]
    mean_tau = WLM.expected_tau(wl)
    alg = algorithmic(wl, mean_tau, wl.L0)
    k = g["kern"]
    kt = dict(verify=k["verify_s"], append=k["append_s"], draft=k["draft_s"],
              update_draft=k["update_draft_s"])
    # the roofline line is the round's longest kernel: the round is
    # ls_verify_append_draft = verify_partial (the key pass) + update_draft,
    # and update_draft is the longer of the two (timed inside the rounds);
    # the separate entry points' kernels are listed beside it
    dominant = "update_draft"
    kernels = {}
    for name, t in kt.items():
        bw = alg[name] / t / 1e9
        ent = dict(avg_us=round(t * 1e6, 3), alg_bytes=int(alg[name]),
                   gb_per_s=round(bw, 1), hbm_frac=round(bw / HBM_PEAK_GBS, 4))
        if name in ("draft", "update_draft"):
            tf = alg["draft_flop"] / t / 1e12
            ent.update(alg_flop=int(alg["draft_flop"]), tflop_per_s=round(tf, 2),
                       mfma_frac=round(tf / MFMA_BF16_PEAK_TFS, 4))
        if name == "draft":
            # single calls with events around each: after a 512 MiB copy (L2
            # and MALL cold) and back to back (warm)
            ent.update(single_call_us_cold=round(k["draft_cold_s"] * 1e6, 3),
                       single_call_us_warm=round(k["draft_warm_single_s"] * 1e6, 3))
        kernels[name] = ent
    kernels["update_draft"]["avg_us_events_around_each_launch"] = round(k["update_draft_event_s"] * 1e6, 3)
    t_keys = k["verify_keys_s"]
    kernels["verify_keys"] = dict(avg_us=round(t_keys * 1e6, 3), alg_bytes=int(alg["verify"]),
                                  gb_per_s=round(alg["verify"] / t_keys / 1e9, 1),
                                  hbm_frac=round(alg["verify"] / t_keys / 1e9 / HBM_PEAK_GBS, 4))
    t_rs = k["round_split_s"]
    kernels["round_call"] = dict(avg_us=round(t_rs * 1e6, 3), alg_bytes=int(alg["round"]),
                                 gb_per_s=round(alg["round"] / t_rs / 1e9, 1),
                                 hbm_frac=round(alg["round"] / t_rs / 1e9 / HBM_PEAK_GBS, 4))
    t_va = k["verify_append_s"]
    bw_va = (alg["verify"] + alg["append"]) / t_va / 1e9
    kernels["verify_append"] = dict(avg_us=round(t_va * 1e6, 3), alg_bytes=int(alg["verify"] + alg["append"]),
                                    gb_per_s=round(bw_va, 1), hbm_frac=round(bw_va / HBM_PEAK_GBS, 4))
    init_s = g["init_s"]
    init_bw = alg["init"] / init_s / 1e9
    # the definition's flops (6 S d per prefix row and KV head) over the time;
    # the far splits leave out the faster half of the slots on old rows, so
    # the MFMA work issued is less: executed_* count it (the counters)
    ex = executed_flop("init")
    kernels["init"] = dict(avg_us=round(init_s * 1e6, 2), alg_bytes=int(alg["init"]),
                           gb_per_s=round(init_bw, 1), hbm_frac=round(init_bw / HBM_PEAK_GBS, 4),
                           tflop_per_s=round(alg["init_flop"] / init_s / 1e12, 1),
                           mfma_frac=round(alg["init_flop"] / init_s / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                           executed_flop=ex,
                           executed_tflop_per_s=round(ex / init_s / 1e12, 1) if ex else None,
                           mfma_frac_executed=round(ex / init_s / 1e12 / MFMA_BF16_PEAK_TFS, 4) if ex else None,
                           # the executed rate over what a library bf16 GEMM reaches here
                           frac_of_mfma_reference=round(ex / init_s / 1e12 / g["mfma_reference"]["tflop_per_s"], 4)
                           if ex else None)
    for name in ("draft", "init", "update_draft"):
        cnt = load_counters(name)
        if cnt and "MfmaUtil" in cnt:
            # MFMA busy share from the counters (MfmaUtil: busy cycles / (active
            # cycles x SIMDs)) beside the algorithmic flops / time above
            kernels[name]["mfma_util_counter"] = round(cnt["MfmaUtil"] / 100.0, 4)
    d = kernels[dominant]
    traffic = load_traffic(dominant)
    ref = g["stream_reference"].get("copy_64MiB_gb_per_s")
    roof = dict(kernel=dominant, bound="hbm", achieved=d["gb_per_s"], peak=HBM_PEAK_GBS,
                unit="GB/s", frac=d["hbm_frac"], traffic=traffic,
                mfma_frac_algorithmic=d.get("mfma_frac"), mfma_util_counter=d.get("mfma_util_counter"),
                # beside the datasheet peak: the same rate over what a plain library copy
                # of the round's scale reaches on this GPU (stream_reference)
                frac_of_stream_reference=round(d["gb_per_s"] / ref, 4) if ref else None)
    line = {
        "metric": "draft rounds/s at concurrency 16, prefix 32K–128K; % HBM/MFMA peak",
        "value": round(value, 1),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["wall_s"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": dict(WLM.describe(wl), step="verify+append+draft_attention round (ls_verify_append_draft)",
                       mean_tau_expected=round(mean_tau, 3)),
        "roofline": roof,
        "kernels": kernels,
        "round_alg_bytes": int(alg["round"]),
        "round_gb_per_s": round(alg["round"] * value / 1e9, 1),
        "gpu_event_ms_per_step": round(main_r["gpu_s"] / args.steps * 1e3, 5),
        "passes": args.passes,
        "pass_ms_per_step": [round(w / args.steps * 1e3, 5) for w in main_r["passes_wall_s"]],
        "pass_gpu_ms_per_step": [round(w / args.steps * 1e3, 5) for w in main_r["passes_gpu_s"]],
        "heat_rounds": args.heat,
        "stream_reference": g["stream_reference"],
        "mfma_reference": g["mfma_reference"],
        "host_issue_us_per_round": round(main_r["issue_s"] / args.steps * 1e6, 2),
        "sweep": g["sweep"],
        "graph_rounds_per_s": (round(args.steps / g["graph"]["wall_s"], 1) if "graph" in g else None),
        "state_bytes_per_seq": g["state_bytes_per_seq"],
        "next": next_steps(wl, g) if args.next else None,
    }
    line["cpu_baseline"] = cpu
    return line


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="q3_8b_128k",
                    help="a named workload (fixed_cost_drafter_amd/configs/<name>.json) or a JSON file")
    ap.add_argument("--passes", type=int, default=5,
                    help="timed passes of --steps rounds; the median pass is reported")
    ap.add_argument("--heat", type=int, default=400,
                    help="untimed rounds between the summary init and the warmup rounds")
    ap.add_argument("--no-sweep", dest="sweep", action="store_false")
    ap.add_argument("--no-cpu", dest="cpu", action="store_false")
    ap.add_argument("--cpu-budget", type=float, default=18.0)
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--no-next", dest="next", action="store_false",
                    help="skip the steps beside the round (argmax, boundary, view ablations)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the K rounds captured in one HIP graph")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc csv runs into the traffic table and exit")
    ap.add_argument("--traffic-command", default="",
                    help="the command the counter runs were made with (recorded in the table)")
    ap.add_argument("--counters", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc csv runs (e.g. MfmaUtil) into profiles/counters.json and exit")
    args = ap.parse_args(argv)
    if args.counters:
        t = summarize_counters(args.counters, args.traffic_command)
        os.makedirs(os.path.dirname(COUNTERS_JSON), exist_ok=True)
        with open(COUNTERS_JSON, "w") as f:
            json.dump(t, f, indent=1, sort_keys=True)
        print(json.dumps(t["entry_points"]))
        return 0
    if args.traffic:
        t = summarize_traffic(args.traffic[0], args.traffic[1], args.traffic_command)
        os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
        with open(TRAFFIC_JSON, "w") as f:
            json.dump(t, f, indent=1, sort_keys=True)
        print(json.dumps(t["entry_points"]))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the drafting "
              "state shards by sequence or KV head with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    from fixed_cost_drafter_amd import workload as WLM
    wl = WLM.resolve_workload(args.workload)
    cpu = None
    if args.cpu:
        # first, while no process has touched the GPU: the workers fork from here
        log("timing the oracle on the host (cpu_baseline)")
        cpu = cpu_baseline(wl, args.cpu_budget)
    g = run_gpu(args, wl)
    g["mfma_reference"] = mfma_reference("cuda")
    log(f"MFMA reference: {g['mfma_reference']}")
    line = result_line(args, wl, g, cpu)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
