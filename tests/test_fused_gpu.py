"""Greedy verification + update in one call (ls_verify_append) against the
separate entry points (ls_verify_greedy, then ls_append_accepted).

The fused call derives tau from the verification's partial keys inside the
update; it must give the same target tokens, tau and state, bit for bit, as
the two calls, over rounds that accept every draft, none, and a random mix.
The fused path against the oracle is tests/test_parity_gpu.py's
full-size and edge-logits cases (lockstep with fused=True)."""
import numpy as np
import pytest

from fixed_cost_drafter_amd import workload as WLM
from tests import harness as H
from tests.test_parity_gpu import SMALL, _announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["bf16_wrap", "bf16_b40", "bf16_b47", "bf16_s128_b40", "bf16_s128_short",
                                  "f32_d32_wrap"])
def test_verify_append_matches_separate_calls(name):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round
    wl = SMALL[name]
    rounds = 6
    _announce(wl, f"fused verify+append vs separate calls x {rounds}")
    Kp, Vp = WLM.prefix(wl, threads=4)
    fused, sep = PathRunner(wl, Kp, Vp), PathRunner(wl, Kp, Vp)
    fused.init()
    sep.init()
    for r in range(rounds):
        logits, planted = WLM.logits_entry(wl, r)
        inp = WLM.round_inputs(wl, r, planted)
        if r == 1:    # every draft accepted: tau = B + 1
            inp["draft"] = np.ascontiguousarray(planted[:, :wl.B]).astype(np.int32)
        elif r == 2:  # the first draft rejected: tau = 1
            inp["draft"] = ((planted[:, :wl.B] + 1) % wl.V).astype(np.int32)
        dev = upload_round(inp)
        lg = LB.to_device(logits)
        fused.round(lg, dev)
        sep.round_separate(lg, dev)
        torch.cuda.synchronize()
        tau = LB.to_host(fused.buf.tau)
        H.exact(f"round {r} tau", tau, LB.to_host(sep.buf.tau))
        H.exact(f"round {r} target_tok", LB.to_host(fused.buf.target_tok), LB.to_host(sep.buf.target_tok))
        if r == 1:
            assert np.all(tau == wl.B + 1)
        elif r == 2:
            assert np.all(tau == 1)
        a, b = fused.snapshot(), sep.snapshot()
        for k in a:
            H.exact(f"round {r} {k}", a[k], b[k])
        H.exact(f"round {r} out", LB.to_host(fused.buf.out), LB.to_host(sep.buf.out))
