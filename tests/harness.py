"""Lockstep runs of the HIP path and the CPU oracle on the same seeded inputs.

Test infrastructure.  Both sides read the arrays from
fixed_cost_drafter_amd.workload; the oracle never sees a value produced by the
GPU.  Comparisons:
  * bit-exact: tau, target_tok, ring_k/ring_v contents, ring_pos, seq_len;
  * f32 workloads: normwise relative error max|x-y| / max|y| <= 1e-5;
  * bf16 workloads: max|x-y| <= 2e-2 on unit-scale outputs (slots, out,
    the pooled means n/l), relative 2e-2 on l, absolute 2e-2 on m.
"""
from __future__ import annotations

import sys
import time

import numpy as np

from fixed_cost_drafter_amd import workload as WLM
from oracle import longspark_oracle as O

F32_REL = 1e-5
BF16_ABS = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def as_f64(a):
    return O.decode(a)


def close(name, got, ref, dtype, mask=None, scaled=False):
    """Assert the stated tolerance; return the error figure.

    ``scaled`` (bf16): outputs that are not unit-scale are held to the same
    bound relative to their size, |x - y| <= 2e-2 max(1, |y|) per element.
    """
    g = as_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        g, r = g[mask], r[mask]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    if scaled and dtype != "f32":
        rel = np.max(np.abs(g - r) / np.maximum(1.0, np.abs(r))) if g.size else 0.0
        assert rel <= BF16_ABS, f"{name}: max scaled err {rel:.3e} > {BF16_ABS}"
        return rel
    err = np.max(np.abs(g - r)) if g.size else 0.0
    if dtype == "f32":
        scale = max(np.max(np.abs(r)) if r.size else 0.0, 1e-30)
        rel = err / scale
        assert rel <= F32_REL, f"{name}: normwise rel err {rel:.3e} > {F32_REL}"
        return rel
    assert err <= BF16_ABS, f"{name}: max abs err {err:.3e} > {BF16_ABS}"
    return err


def exact(name, got, ref):
    got = np.asarray(got)
    ref = np.asarray(ref)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}: "
                             f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}")


def compare_state(runner, ost: O.OracleState, dtype, heads=None, scaled=False):
    """GPU state vs oracle state; ``heads`` restricts the float checks;
    ``scaled``: see close()."""
    snap = runner.snapshot()
    # the library keeps window and slot values in key tiles [rows/tw][d][tw],
    # at d = 128 keys in 32-key tiles in MFMA operand order, and bf16
    # numerators in 32-slot accumulator tiles
    from fixed_cost_drafter_amd.binding import keys_to_rows, n_to_rows, values_to_rows
    snap["sum_n"] = n_to_rows(snap["sum_n"], dtype)
    snap["ring_v"] = values_to_rows(snap["ring_v"])
    snap["slot_v"] = values_to_rows(snap["slot_v"])
    snap["ring_k"] = keys_to_rows(snap["ring_k"])
    snap["slot_k"] = keys_to_rows(snap["slot_k"])
    exact("seq_len", snap["seq_len"].astype(np.int64), ost.seq_len)
    exact("ring_pos", snap["ring_pos"], ost.ring_pos)
    exact("ring_k", snap["ring_k"], ost.ring_k)
    exact("ring_v", snap["ring_v"], ost.ring_v)
    d = ost.d
    if ost.m.shape[2] == 0:  # no summary view (S = 0): only the window to compare
        return {}
    todo = heads if heads is not None else [(c, h) for c in range(ost.m.shape[0])
                                            for h in range(ost.m.shape[1])]
    errs = {}
    for c, h in todo:
        if dtype == "f32":
            errs["m"] = close("sum_m", snap["sum_m"][c, h], ost.m[c, h], dtype)
            errs["l"] = close("sum_l", snap["sum_l"][c, h], ost.l[c, h], dtype)
            errs["n"] = close("sum_n", snap["sum_n"][c, h], ost.n[c, h], dtype)
        else:
            em = np.max(np.abs(snap["sum_m"][c, h].astype(np.float64) - ost.m[c, h]))
            assert em <= BF16_ABS, f"sum_m ({c},{h}) err {em}"
            rl = np.max(np.abs(snap["sum_l"][c, h] / ost.l[c, h] - 1.0))
            assert rl <= BF16_ABS, f"sum_l ({c},{h}) rel err {rl}"
            mean = snap["sum_n"][c, h].astype(np.float64) / snap["sum_l"][c, h][:, None].astype(np.float64)
            close("n/l", mean, ost.n[c, h] / ost.l[c, h][:, None], dtype, scaled=scaled)
        errs["slot_k"] = close("slot_k", snap["slot_k"][c, h], ost.slot_k[c, h], dtype, scaled=scaled)
        errs["slot_v"] = close("slot_v", snap["slot_v"][c, h], ost.slot_v[c, h], dtype, scaled=scaled)
    return errs


def lockstep(wl: WLM.Workload, rounds: int, k_prefix=None, v_prefix=None, heads=None,
             check_state_every=1, runner=None, tau_override=None, device="cuda", fused=False,
             logits_fn=None, draft_fn=None, calls=None):
    """Run ``rounds`` rounds on both sides and compare after each.

    ``heads`` samples (c, h) pairs for the float checks of large workloads
    (the oracle's summary and attention are computed only there).
    ``tau_override`` (round -> tau array) replaces the verified tau on both
    sides before the append (device-side clamping and the error flag).
    ``calls`` picks the entry points of a round: "separate" (default:
    ls_verify_greedy, ls_append_accepted, ls_draft_attention), "two"
    (ls_verify_append, then ls_draft_attention), "round" (the bench's call,
    ls_verify_append_draft) or "mixed" (round, two, separate in turn on the
    same state); ``fused=True`` means "round".  For "two" and "round"
    target_tok and tau are checked after the round.
    ``logits_fn(r)`` -> (logits, planted or None) replaces the pooled logits;
    ``draft_fn(r, target)`` -> draft [C, B] replaces the round's drafts, built
    from the oracle's target tokens ``target`` (never from GPU output).
    Returns (runner, oracle_state, stats).
    """
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round

    calls = calls or ("round" if fused else "separate")
    assert calls in ("separate", "two", "round", "mixed"), calls
    assert not (calls != "separate" and tau_override), "the fused calls derive tau themselves"
    t0 = time.time()
    if k_prefix is None:
        k_prefix, v_prefix = WLM.prefix(wl, threads=16)
    if runner is None:
        runner = PathRunner(wl, k_prefix, v_prefix, device=device)
        runner.init()
    log(f"[{wl.name}] init launched ({time.time() - t0:.1f}s)")
    u = WLM.slot_queries(wl)
    logl = WLM.log_lambda(wl)
    L0 = k_prefix.shape[1]
    ost = O.summary_init(u, logl, np.ascontiguousarray(k_prefix[:, :L0]),
                         np.ascontiguousarray(v_prefix[:, :L0]), wl.W, heads=heads)
    torch.cuda.synchronize()
    compare_state(runner, ost, wl.dtype, heads)
    log(f"[{wl.name}] init parity ok ({time.time() - t0:.1f}s)")
    stats = dict(tau=[])
    pool = {}
    G = wl.G
    pairs = None
    if heads is not None:
        pairs = [(c, h * G + g) for c, h in heads for g in range(G)]
    for r in range(rounds):
        if logits_fn is None:
            # a pooled logits tensor: its oracle argmax is a pure function of
            # it, computed once per pool entry
            k = r % WLM.pool_size(wl)
            if k not in pool:
                logits, planted = WLM.logits_entry(wl, k)
                pool[k] = (logits, planted, LB.to_device(logits, device), O.target_argmax(logits))
            logits, planted, logits_dev, tgt_ref = pool[k]
        else:
            logits, planted = logits_fn(r)
            logits_dev = LB.to_device(logits, device)
            tgt_ref = O.target_argmax(logits)
        inp = WLM.round_inputs(wl, r, planted if planted is not None else tgt_ref)
        if draft_fn is not None:
            inp["draft"] = np.ascontiguousarray(draft_fn(r, tgt_ref), dtype=np.int32)
        tau_ref = O.accepted_length(tgt_ref, inp["draft"])
        if planted is not None:
            exact("target_tok==planted", tgt_ref, planted)
        dev = upload_round(inp, device)
        b = runner.buf
        s = runner.state
        tau_use = tau_ref
        # "mixed": the three call sequences in turn on one state
        mode = ("round", "two", "separate")[r % 3] if calls == "mixed" else calls
        fused = mode != "separate"
        if mode == "round":
            runner.round(logits_dev, dev)
        elif mode == "two":
            runner.round_two_calls(logits_dev, dev)
        else:
            s.verify_greedy(logits_dev, dev["draft"], b.target_tok, b.tau)
            torch.cuda.synchronize()
            exact("target_tok", LB.to_host(b.target_tok), tgt_ref)
            exact("tau", LB.to_host(b.tau), tau_ref)
            if tau_override is not None and r in tau_override:
                forced = np.asarray(tau_override[r], dtype=np.int32)
                b.tau.copy_(LB.to_device(forced, device))
                tau_use = np.clip(forced, 1, wl.B + 1)
            s.append_accepted(dev["k_new"], dev["v_new"], b.tau)
            s.draft_attention(dev["q"], dev["k_blk"], dev["v_blk"], b.out)
        O.append_accepted(ost, inp["k_new"], inp["v_new"], tau_use, heads=heads)
        out_ref = O.draft_attention(ost, inp["q"], inp["k_blk"], inp["v_blk"], pairs=pairs)
        torch.cuda.synchronize()
        if fused:
            exact(f"round {r} target_tok", LB.to_host(b.target_tok), tgt_ref)
            exact(f"round {r} tau", LB.to_host(b.tau), tau_ref)
        stats["tau"].append(tau_ref.copy())
        if check_state_every and (r % check_state_every == 0 or r == rounds - 1):
            compare_state(runner, ost, wl.dtype, heads)
            if rounds > 32:
                log(f"[{wl.name}] round {r}: state parity ok ({time.time() - t0:.1f}s)")
        out = LB.to_host(b.out)
        if pairs is None:
            close("out", out, out_ref, wl.dtype)
        else:
            for c, hq in pairs:
                close("out", out[c, :, hq], out_ref[c, :, hq], wl.dtype)
    log(f"[{wl.name}] {rounds} rounds parity ok ({time.time() - t0:.1f}s)")
    return runner, ost, stats
