"""GPU parity of the next-step entry points against the CPU oracle (C ABI).

ls_draft_argmax (the drafter's proposal at T = 0) and ls_gather_boundary (the
boundary state view): integer and copy results, so the bar is bit-exact.
Every case prints its name and shape before it touches the GPU.
"""
import numpy as np
import pytest

from fixed_cost_drafter_amd import workload as WLM
from oracle import longspark_oracle as O
from tests import harness as H
from tests.test_parity_gpu import SMALL

pytestmark = pytest.mark.gpu


def _state(wl):
    from fixed_cost_drafter_amd import binding as LB
    return LB.DrafterState.for_workload(wl, WLM.slot_queries(wl), WLM.log_lambda(wl), max_L0=1)


ARGMAX_CASES = {
    "tiny_f32": WLM.WORKLOADS["tiny_f32"],
    "bf16_l1": SMALL["bf16_l1"],                 # V = 1001: scalar path and a ragged chunk
    "bf16_s64_ragged": SMALL["bf16_s64_ragged"],  # V = 20001: two chunks + tail
    "q3_8b": WLM.WORKLOADS["q3_8b_128k"],        # C = 16, B = 16, V = 151936
}


@pytest.mark.parametrize("name", list(ARGMAX_CASES))
def test_draft_argmax_parity(name):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    wl = ARGMAX_CASES[name]
    H.log(f"CASE draft_argmax {name} dtype={wl.dtype} C={wl.C} B={wl.B} V={wl.V}")
    st = _state(wl)
    out = torch.empty((wl.C, wl.B), dtype=torch.int32, device="cuda")
    for k in range(2):
        logits, _ = WLM.logits_entry(wl, k)
        drafter = np.ascontiguousarray(logits[:, :wl.B])    # [C, B, V], ~25% rows with a tie
        st.draft_argmax(LB.to_device(drafter), out)
        torch.cuda.synchronize()
        H.exact(f"draft_tok {name} #{k}", LB.to_host(out), O.draft_argmax(drafter))


def test_draft_argmax_edge_rows():
    """All-equal rows, -0 against +0, the maximum at the last index or in the tail."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    wl = SMALL["bf16_s64_ragged"].with_(name="argmax_edges", C=1, B=6, V=20001)
    H.log(f"CASE draft_argmax edges V={wl.V}")
    x = np.zeros((1, 6, wl.V), dtype=np.float32)
    x[0, 1, :] = -0.0
    x[0, 1, 7] = 0.0                       # +0 after -0s: index 0 still wins
    x[0, 2, :] = -1.0
    x[0, 2, wl.V - 1] = 2.0                # maximum in the ragged tail
    x[0, 3, 16384] = 3.0                   # first element of the second chunk
    x[0, 3, 16383] = 3.0                   # ... tied with the last of the first
    x[0, 4, ::2] = 1.5                     # every even index ties
    x[0, 5, 12345] = 1e-30                 # a tiny positive against zeros
    bits = WLM.f32_to_bf16_bits(x)
    st = _state(wl)
    out = torch.empty((1, 6), dtype=torch.int32, device="cuda")
    st.draft_argmax(LB.to_device(bits), out)
    torch.cuda.synchronize()
    got = LB.to_host(out)
    H.exact("edge rows", got, O.draft_argmax(bits))
    assert got.tolist() == [[0, 0, wl.V - 1, 16383, 0, 12345]]


@pytest.mark.parametrize("dtype,H_", [("bf16", 4096), ("f32", 37), ("bf16", 7)])
def test_gather_boundary_parity(dtype, H_):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    wl = (SMALL["bf16_s64_ragged"] if dtype == "bf16" else WLM.WORKLOADS["tiny_f32"]).with_(
        name=f"boundary_{dtype}_{H_}", C=5, B=6)
    H.log(f"CASE gather_boundary dtype={dtype} C={wl.C} B={wl.B} H={H_}")
    rng = np.random.default_rng(31 + H_)
    hidden = rng.standard_normal((wl.C, wl.B + 1, H_)).astype(np.float32)
    if dtype == "bf16":
        hidden = WLM.f32_to_bf16_bits(hidden)
    st = _state(wl)
    out = torch.empty((wl.C, H_), dtype=LB.torch_dtype(dtype), device="cuda")
    for taus in ([1, 7, 3, 2, 5], [7, 7, 1, 1, 4]):
        tau = LB.to_device(np.asarray(taus, dtype=np.int32))
        st.gather_boundary(LB.to_device(hidden), tau, out)
        torch.cuda.synchronize()
        H.exact(f"boundary {taus}", LB.to_host(out), O.boundary_row(hidden, taus))
    assert int(LB.to_host(st.err_flag)[0]) == 0
    # out of range: clamped to [1, B+1] and flagged
    tau = LB.to_device(np.asarray([0, 9, 3, 2, 5], dtype=np.int32))
    st.gather_boundary(LB.to_device(hidden), tau, out)
    torch.cuda.synchronize()
    H.exact("boundary clamped", LB.to_host(out), O.boundary_row(hidden, [1, 7, 3, 2, 5]))
    assert int(LB.to_host(st.err_flag)[0]) & 1


# one view switched off (Table 5's ablations, cost side): S = 0 or W = 0
ABLATIONS = {
    "bf16_no_summary": SMALL["bf16_s64_ragged"].with_(name="bf16_no_summary", S=0, rounds=5),
    "bf16_no_window": SMALL["bf16_s64_ragged"].with_(name="bf16_no_window", W=0, rounds=5),
    "bf16_block_only": SMALL["bf16_wrap"].with_(name="bf16_block_only", W=0, S=0, rounds=4),
    "f32_no_summary": WLM.WORKLOADS["tiny_f32"].with_(name="f32_no_summary", S=0, lambdas=(),
                                                      rounds=6),
    "f32_no_window": WLM.WORKLOADS["tiny_f32"].with_(name="f32_no_window", W=0, rounds=6),
}


@pytest.mark.parametrize("name", list(ABLATIONS))
def test_view_ablation_parity(name):
    wl = ABLATIONS[name]
    H.log(f"CASE ablation {name} dtype={wl.dtype} C={wl.C} W={wl.W} S={wl.S} B={wl.B} "
          f"L0={wl.L0} seed={wl.seed}")
    _, ost, stats = H.lockstep(wl, wl.rounds)
    assert int(ost.seq_len.min()) > wl.L0
