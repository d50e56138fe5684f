"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Every case prints its name, seed and shape before it touches the GPU.
"""
import numpy as np
import pytest

from fixed_cost_drafter_amd import workload as WLM
from oracle import longspark_oracle as O
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from fixed_cost_drafter_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    yield


def _announce(wl, extra=""):
    H.log(f"CASE {wl.name} dtype={wl.dtype} C={wl.C} Hq={wl.Hq} Hkv={wl.Hkv} d={wl.d} "
          f"L0={wl.L0} W={wl.W} S={wl.S} B={wl.B} V={wl.V} seed={wl.seed} {extra}")


# small shapes: several tiles, ragged tails, every round checked in full
SMALL = {
    "tiny_f32": WLM.WORKLOADS["tiny_f32"],
    # f32, d=32, ring wraps many times, L0 not a multiple of any tile
    "f32_d32_wrap": WLM.WORKLOADS["tiny_f32"].with_(
        name="f32_d32_wrap", C=3, Hq=6, Hkv=3, d=32, L0=77, W=9, S=5, B=6, V=300, rounds=12,
        lambdas=(1.0, 0.999, 0.9, 0.5, 0.0), seed=11),
    # bf16, S=64, ragged prefix (300 rows: tiles of 64 + tail), V spans 2 chunks + tail
    "bf16_s64_ragged": WLM.Workload(
        "bf16_s64_ragged", "bf16", C=2, Hq=8, Hkv=2, d=128, L0=300, W=64, S=64, B=5, V=20001,
        rounds=6, p_match=0.8, seed=12),
    # bf16, S=128, prefix shorter than the window (empty ring slots are masked),
    # B*G = 48 (a 16-row tail in the second 32-row slice)
    "bf16_s128_short": WLM.Workload(
        "bf16_s128_short", "bf16", C=3, Hq=16, Hkv=4, d=128, L0=37, W=128, S=128, B=12,
        V=4096, rounds=10, p_match=0.85, seed=13),
    # bf16, single-row prefix, B*G = 32, odd vocabulary (scalar verify path)
    "bf16_l1": WLM.Workload(
        "bf16_l1", "bf16", C=2, Hq=32, Hkv=8, d=128, L0=1, W=64, S=128, B=8, V=1001,
        rounds=5, p_match=0.9, seed=14),
    # bf16, B = 40: two block chunks (one ragged), B*G = 40 (ragged 32-row slice)
    "bf16_b40": WLM.Workload(
        "bf16_b40", "bf16", C=2, Hq=8, Hkv=8, d=128, L0=500, W=96, S=64, B=40, V=3000,
        rounds=6, p_match=0.9, seed=16),
    # bf16, keys split over two workgroups per KV head + combine (W = 512,
    # 32 query rows per KV head), prefix shorter than the window
    "bf16_halves": WLM.Workload(
        "bf16_halves", "bf16", C=2, Hq=8, Hkv=2, d=128, L0=300, W=512, S=64, B=8, V=2000,
        rounds=5, p_match=0.8, seed=17),
    # bf16, ring wraps inside the round loop, G=1, B=16 at C=5
    "bf16_wrap": WLM.Workload(
        "bf16_wrap", "bf16", C=5, Hq=4, Hkv=4, d=128, L0=130, W=32, S=64, B=16, V=9000,
        rounds=14, p_match=0.75, seed=15),
    # the largest block (B = 47): 48 verified rows, a ragged second block chunk
    # (15 keys), B*G = 47 query rows (a full and a ragged 32-row slice)
    "bf16_b47": WLM.Workload(
        "bf16_b47", "bf16", C=2, Hq=4, Hkv=4, d=128, L0=333, W=64, S=128, B=47, V=5000,
        rounds=5, p_match=0.95, seed=21),
    # the summary merge with two 32-row score blocks (B + 1 > 32) over 128 slots
    "bf16_s128_b40": WLM.Workload(
        "bf16_s128_b40", "bf16", C=2, Hq=2, Hkv=2, d=128, L0=90, W=128, S=128, B=40, V=1504,
        rounds=5, p_match=0.92, seed=20),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(name):
    wl = SMALL[name]
    _announce(wl, f"rounds={wl.rounds}")
    _, _, stats = H.lockstep(wl, wl.rounds)
    taus = np.concatenate(stats["tau"])
    assert taus.min() >= 1 and taus.max() <= wl.B + 1


def test_parity_q3_4b_8k_all_heads():
    wl = WLM.WORKLOADS["q3_4b_8k"]
    _announce(wl, "rounds=64 (state checked every 8)")
    _, _, stats = H.lockstep(wl, wl.rounds, check_state_every=8)
    taus = np.concatenate(stats["tau"]).astype(float)
    H.log(f"mean tau {taus.mean():.2f} (expected {WLM.expected_tau(wl):.2f})")


@pytest.mark.parametrize("name", ["q3_8b_32k", "q3_8b_128k"])
def test_parity_full_size_sampled(name):
    """Full shape, full prefix, bench launch configuration; sampled heads."""
    wl = WLM.WORKLOADS[name]
    heads = [(0, 0), (7, 3), (15, 7)]
    _announce(wl, f"rounds=6 sampled heads={heads}")
    H.lockstep(wl, 6, heads=heads, check_state_every=2)


def test_tau_out_of_range_is_clamped_and_flagged():
    from fixed_cost_drafter_amd import binding as LB
    wl = SMALL["bf16_wrap"]
    _announce(wl, "forced tau = [0, 99, 3, 17, 1]")
    runner, _, _ = H.lockstep(wl, 3, tau_override={1: [0, 99, 3, 17, 1]})
    assert int(LB.to_host(runner.state.err_flag)[0]) & 1
    # init resets the flag
    runner.init()
    import torch
    torch.cuda.synchronize()
    assert int(LB.to_host(runner.state.err_flag)[0]) == 0


def test_runs_are_deterministic():
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round
    wl = SMALL["bf16_s128_short"]
    _announce(wl, "determinism x2")
    Kp, Vp = WLM.prefix(wl, threads=4)
    outs = []
    for _ in range(2):
        rn = PathRunner(wl, Kp, Vp)
        rn.init()
        for r in range(4):
            logits, planted = WLM.logits_entry(wl, r)
            dev = upload_round(WLM.round_inputs(wl, r, planted))
            rn.round(LB.to_device(logits), dev)
        torch.cuda.synchronize()
        snap = rn.snapshot()
        snap["out"] = LB.to_host(rn.buf.out)
        outs.append(snap)
    for k in outs[0]:
        H.exact(f"rerun {k}", outs[1][k], outs[0][k])


def test_checkpoint_restore_replays_identically():
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round
    wl = SMALL["bf16_wrap"]
    _announce(wl, "checkpoint after round 3")
    Kp, Vp = WLM.prefix(wl, threads=4)
    rn = PathRunner(wl, Kp, Vp)
    rn.init()

    def step(r):
        logits, planted = WLM.logits_entry(wl, r)
        rn.round(LB.to_device(logits), upload_round(WLM.round_inputs(wl, r, planted)))

    for r in range(4):
        step(r)
    torch.cuda.synchronize()
    snap = rn.snapshot()
    for r in range(4, 8):
        step(r)
    torch.cuda.synchronize()
    first = rn.snapshot()
    first["out"] = LB.to_host(rn.buf.out)
    rn.restore(snap)
    for r in range(4, 8):
        step(r)
    torch.cuda.synchronize()
    second = rn.snapshot()
    second["out"] = LB.to_host(rn.buf.out)
    for k in first:
        H.exact(f"replay {k}", second[k], first[k])


def test_prefix_stride_and_sub_prefix():
    """A prefix read from a longer allocation (rows stride > L0) equals a tight one."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner
    wl = SMALL["bf16_s64_ragged"]
    _announce(wl, "L0=200 inside a 300-row allocation")
    Kp, Vp = WLM.prefix(wl, threads=4)
    a = PathRunner(wl, Kp, Vp)
    a.init(L0=200)
    b = PathRunner(wl, np.ascontiguousarray(Kp[:, :200]), np.ascontiguousarray(Vp[:, :200]))
    b.init()
    torch.cuda.synchronize()
    sa, sb = a.snapshot(), b.snapshot()
    for k in sa:
        H.exact(f"stride {k}", sa[k], sb[k])
    ost = O.summary_init(WLM.slot_queries(wl), WLM.log_lambda(wl), Kp[:, :200], Vp[:, :200],
                         wl.W)
    H.compare_state(a, ost, wl.dtype)
    del LB
