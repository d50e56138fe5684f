"""One drafting round captured in a HIP graph and replayed.

A caller may capture the round (ls_verify_append_draft: the key pass, then
the update and the draft attention) once and replay it every round.  The
round's kernels take all sizes from their arguments and tau from device
memory, and no call records a memset (the key pass zeroes the arrival
counters with its own stores), so a replay must do exactly what the eager
calls do.  bf16_s128_short has two workgroups per KV head, so its replays
also exercise the arrival counters.  The replays here run with the program's own eager work
and synchronisations between them, and every replay is compared bit for bit
with an eager run of the same rounds.
"""
import numpy as np
import pytest

from fixed_cost_drafter_amd import workload as WLM
from tests import harness as H
from tests.test_parity_gpu import SMALL, _announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["bf16_halves", "bf16_wrap", "bf16_s128_short", "f32_d32_wrap"])
def test_graph_replay_matches_eager(name):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round
    wl = SMALL[name]
    rounds = 4
    _announce(wl, f"graph replay of one round x {rounds}")
    Kp, Vp = WLM.prefix(wl, threads=4)
    inputs = []
    for r in range(rounds):
        logits, planted = WLM.logits_entry(wl, r)
        inputs.append((LB.to_device(logits), upload_round(WLM.round_inputs(wl, r, planted))))

    def observe(rn):
        snap = rn.snapshot()
        snap["out"] = LB.to_host(rn.buf.out)
        snap["tau"] = LB.to_host(rn.buf.tau)
        snap["target_tok"] = LB.to_host(rn.buf.target_tok)
        return snap

    eager = PathRunner(wl, Kp, Vp)
    eager.init()
    want = []
    for r in range(rounds):
        eager.round(*inputs[r])
        torch.cuda.synchronize()
        want.append(observe(eager))

    rn = PathRunner(wl, Kp, Vp)
    logits_buf = inputs[0][0].clone()
    dev_buf = {k: v.clone() for k, v in inputs[0][1].items()}
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        rn.round(logits_buf, dev_buf)
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    rn.init()  # capture runs nothing: the state starts from the same init as eager
    torch.cuda.synchronize()
    for r in range(rounds):
        logits_buf.copy_(inputs[r][0])
        for k, v in inputs[r][1].items():
            dev_buf[k].copy_(v)
        noise = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        got = observe(rn)
        for k in want[r]:
            H.exact(f"replay {r} {k}", got[k], want[r][k])
    del graph
