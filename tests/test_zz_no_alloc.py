"""ls_verify_greedy_noalloc (no workspace, static device scratch) against
ls_verify_greedy (caller's workspace) and the oracle, bit for bit.

Three calls in a row on one GPU share the static scratch: the full
verification shape (C = 16, B = 16, V = 151936), then a smaller bf16 call
on edge-case logits, then a small f32 call, so that each later call runs on
what the one before it left in the array.
"""
import numpy as np
import pytest

from fixed_cost_drafter_amd import workload as WLM
from oracle import longspark_oracle as O
from tests import harness as H

pytestmark = pytest.mark.gpu


def _call(wl, logits):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    tgt_ref = O.target_argmax(logits)
    inp = WLM.round_inputs(wl, 0, tgt_ref)
    draft = inp["draft"]
    draft[0, : wl.B // 2] = tgt_ref[0, : wl.B // 2]   # one long accepted prefix
    tau_ref = O.accepted_length(tgt_ref, draft)
    dims = LB.make_dims(wl.C, wl.Hq, wl.Hkv, wl.d, wl.W, wl.S, wl.B, wl.V, wl.dtype)
    lg, dr = LB.to_device(logits), LB.to_device(draft)
    ws = torch.empty(LB.ls_workspace_bytes(dims, 1), dtype=torch.uint8, device="cuda")
    tt_a = torch.full((wl.C, wl.B + 1), -7, dtype=torch.int32, device="cuda")
    tt_b = torch.full((wl.C, wl.B + 1), -9, dtype=torch.int32, device="cuda")
    tau_a = torch.full((wl.C,), -7, dtype=torch.int32, device="cuda")
    tau_b = torch.full((wl.C,), -9, dtype=torch.int32, device="cuda")
    LB.ls_verify_greedy(dims, lg, dr, tt_a, tau_a, ws, ws.numel())
    LB.ls_verify_greedy_noalloc(dims, lg, dr, tt_b, tau_b)
    torch.cuda.synchronize()
    H.exact("noalloc target_tok vs workspace call", LB.to_host(tt_b), LB.to_host(tt_a))
    H.exact("noalloc tau vs workspace call", LB.to_host(tau_b), LB.to_host(tau_a))
    H.exact("noalloc target_tok vs oracle", LB.to_host(tt_b), tgt_ref)
    H.exact("noalloc tau vs oracle", LB.to_host(tau_b), tau_ref)
    return LB.to_host(tau_b)


def test_noalloc_verify_matches_the_workspace_entry_point():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    big = WLM.WORKLOADS["q3_8b_128k"]
    H.log(f"CASE noalloc verify 1/3: C={big.C} B={big.B} V={big.V} bf16 pooled logits")
    logits, _ = WLM.logits_entry(big, 0)
    tau = _call(big, logits)
    assert tau[0] >= big.B // 2 + 1
    small = big.with_(name="noalloc_small", C=3, B=5, V=20001)
    H.log(f"CASE noalloc verify 2/3: C={small.C} B={small.B} V={small.V} bf16 edge logits")
    _call(small, WLM.edge_logits(small, 1))
    tiny = WLM.WORKLOADS["tiny_f32"].with_(name="noalloc_f32", C=2, V=9000)
    H.log(f"CASE noalloc verify 3/3: C={tiny.C} B={tiny.B} V={tiny.V} f32 edge logits")
    _call(tiny, WLM.edge_logits(tiny, 2))
