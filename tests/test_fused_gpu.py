"""The fused entry points against the separate ones.

ls_verify_append (greedy verification + update in one call) derives tau from
the verification's partial keys inside the update; it must give the same
target tokens, tau, state and draft output, bit for bit, as ls_verify_greedy
then ls_append_accepted.  ls_verify_append_draft (the whole round in one call)
must match ls_verify_append + ls_draft_attention bit for bit in everything but
the attention output, which differs only in the order the softmax visits the
keys; its halves (ls_verify_keys, ls_update_draft) must match it bit for bit.
Each runs over rounds that accept every draft, none, and a random mix.  The
one-call round also meets the oracle here on seeded random shapes; the fused
paths against the oracle are otherwise tests/test_parity_gpu.py's small
round-mode, random-shape, full-size and edge-logits cases."""
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
        fused.round_two_calls(lg, dev)
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


@pytest.mark.parametrize("name", ["bf16_wrap", "bf16_s128_short", "bf16_halves", "bf16_l1", "bf16_s64_r2",
                                  "bf16_w32_full", "q3_8b_32k"])
def test_round_matches_two_calls(name):
    """ls_verify_append_draft (update and draft in one launch) against
    ls_verify_append + ls_draft_attention: target tokens, tau and the whole
    state bit for bit, the attention output within the oracle's bf16 bound
    with a small mean difference (the fused kernel visits the new window rows
    and the slots as chunks of their own, so only the order in which the
    softmax sees the keys differs), over rounds that accept every draft,
    none, and a random mix."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round
    wl = SMALL[name] if name in SMALL else WLM.WORKLOADS[name].with_(L0=3000)
    rounds = 6
    _announce(wl, f"one-call round vs two calls x {rounds}")
    Kp, Vp = WLM.prefix(wl, threads=8)
    one, two = PathRunner(wl, Kp, Vp), PathRunner(wl, Kp, Vp)
    one.init()
    two.init()
    for r in range(rounds):
        logits, planted = WLM.logits_entry(wl, r % WLM.pool_size(wl))
        inp = WLM.round_inputs(wl, r, planted)
        if r == 1:    # every draft accepted: tau = B + 1
            inp["draft"] = np.ascontiguousarray(planted[:, :wl.B]).astype(np.int32)
        elif r == 2:  # the first draft rejected: tau = 1
            inp["draft"] = ((planted[:, :wl.B] + 1) % wl.V).astype(np.int32)
        dev = upload_round(inp)
        lg = LB.to_device(logits)
        one.round(lg, dev)
        two.round_two_calls(lg, dev)
        torch.cuda.synchronize()
        H.exact(f"round {r} tau", LB.to_host(one.buf.tau), LB.to_host(two.buf.tau))
        H.exact(f"round {r} target_tok", LB.to_host(one.buf.target_tok), LB.to_host(two.buf.target_tok))
        a, b = one.snapshot(), two.snapshot()
        for k in a:
            H.exact(f"round {r} {k}", a[k], b[k])
        got = H.as_f64(LB.to_host(one.buf.out))
        ref = H.as_f64(LB.to_host(two.buf.out))
        # the probabilities enter P.V as bf16 relative to the running maximum,
        # so a different chunk order rounds them differently (up to 2^-9 of
        # the values' size, the same error each path has against the exact
        # result): the two are held to the bound each meets against the
        # oracle, and their mean difference must stay far below it
        diff = np.abs(got - ref)
        H.log(f"round {r}: max diff {float(diff.max()):.3e} mean {float(diff.mean()):.3e} "
              f"unequal {float(np.mean(diff > 0)):.4f}")
        assert float(diff.max()) <= H.BF16_ABS, f"round {r}: max diff {float(diff.max()):.3e}"
        assert float(diff.mean()) <= 1e-3, f"round {r}: mean diff {float(diff.mean()):.3e}"


@pytest.mark.parametrize("name", ["bf16_wrap", "bf16_s128_short", "bf16_halves", "f32_d32_wrap", "q3_8b_32k"])
def test_split_round_matches_one_call(name):
    """ls_verify_keys then ls_update_draft against ls_verify_append_draft:
    the same launches, so everything matches bit for bit, the output too
    (f32_d32_wrap: the shapes the fused kernel does not take, where both run
    the separate kernels)."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round
    wl = SMALL[name] if name in SMALL else WLM.WORKLOADS[name].with_(L0=3000)
    rounds = 5
    _announce(wl, f"split round vs one call x {rounds}")
    Kp, Vp = WLM.prefix(wl, threads=8)
    one, two = PathRunner(wl, Kp, Vp), PathRunner(wl, Kp, Vp)
    one.init()
    two.init()
    for r in range(rounds):
        logits, planted = WLM.logits_entry(wl, r % WLM.pool_size(wl))
        dev = upload_round(WLM.round_inputs(wl, r, planted))
        lg = LB.to_device(logits)
        one.round(lg, dev)
        two.round_split(lg, dev)
        torch.cuda.synchronize()
        for k in ("tau", "target_tok", "out"):
            H.exact(f"round {r} {k}", LB.to_host(getattr(one.buf, k)), LB.to_host(getattr(two.buf, k)))
        a, b = one.snapshot(), two.snapshot()
        for k in a:
            H.exact(f"round {r} {k}", a[k], b[k])


@pytest.mark.parametrize("name", ["bf16_s128_short", "q3_8b_32k"])
def test_update_draft_repeats_without_a_key_pass(name):
    """Two ls_update_draft calls after one key pass: the second merges the
    same accepted rows into the summary once more at the same lengths.  The
    reference replays that second update from a restored state: the state
    after the first update, with the lengths put back, and a fresh key pass
    (the same logits give the same keys).  The shapes have two workgroups
    per KV head, so the second call's state writes need the arrival counters
    that the first call left at zero."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    from fixed_cost_drafter_amd.runner import PathRunner, upload_round
    wl = SMALL[name] if name in SMALL else WLM.WORKLOADS[name].with_(L0=3000)
    assert wl.B * wl.Hq // wl.Hkv > 32, "two workgroups per KV head"
    _announce(wl, "update_draft twice after one key pass")
    Kp, Vp = WLM.prefix(wl, threads=8)
    twice, ref = PathRunner(wl, Kp, Vp), PathRunner(wl, Kp, Vp)
    twice.init()
    ref.init()
    logits, planted = WLM.logits_entry(wl, 0)
    dev = upload_round(WLM.round_inputs(wl, 0, planted))
    lg = LB.to_device(logits)
    s, b = twice.state, twice.buf
    s.verify_keys(lg)
    upd = lambda st, bf: st.update_draft(dev["draft"], bf.target_tok, bf.tau, dev["k_new"], dev["v_new"],
                                         dev["q"], dev["k_blk"], dev["v_blk"], bf.out)
    upd(s, b)
    torch.cuda.synchronize()
    first = twice.snapshot()
    seq0 = LB.to_host(ref.state.seq_len)
    upd(s, b)
    torch.cuda.synchronize()
    after = twice.snapshot()
    assert not np.array_equal(first["sum_n"], after["sum_n"]), "the second update wrote no summary"
    back = dict(first)
    back["seq_len"] = seq0
    ref.restore(back)
    ref.round_split(lg, dev)
    torch.cuda.synchronize()
    want = ref.snapshot()
    for k in after:
        H.exact(k, after[k], want[k])
    H.exact("out", LB.to_host(twice.buf.out), LB.to_host(ref.buf.out))


def _random_round_shapes(n, seed=2024):
    """Seeded bf16 shapes that the one-call round's fused kernel takes: W a
    multiple of 32 from 32 to 256, S in {64, 128}, 1 <= B <= min(31, W - 1),
    B * G <= 64 query rows per KV head (one or two workgroups), C and the
    prefix length (shorter than the window, or wrapping it) varied."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        W = 32 * int(rng.integers(1, 9))
        S = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, min(31, W - 1) + 1))
        if B * G > 64 or (len(shapes) % 2 == 1 and B * G <= 32):
            continue  # every other shape has two workgroups per KV head
        C = int(rng.integers(1, 5))
        L0 = int(rng.integers(1, 3 * W))
        V = int(rng.choice([1000, 4096, 9001]))
        shapes.append(WLM.Workload(
            f"rand{len(shapes)}", "bf16", C=C, Hq=Hkv * G, Hkv=Hkv, d=128, L0=L0, W=W, S=S, B=B, V=V,
            rounds=4, p_match=float(rng.choice([0.5, 0.85, 0.97])), seed=100 + len(shapes)))
    return shapes


RANDOM_ROUND = _random_round_shapes(20)


@pytest.mark.parametrize("wl", RANDOM_ROUND, ids=[w.name for w in RANDOM_ROUND])
def test_round_random_shapes_against_the_oracle(wl):
    """The one-call round against the oracle, every round and the whole state,
    over seeded random shapes that its fused kernel takes."""
    _announce(wl, f"G={wl.Hq // wl.Hkv} rows/head={wl.B * wl.Hq // wl.Hkv} rounds={wl.rounds} one-call round")
    H.lockstep(wl, wl.rounds, calls="round")


MINIMAL_ROUND = {
    # one drafted token, one query row per KV head, a one-row prefix
    "min_b1_g1": WLM.Workload("min_b1_g1", "bf16", C=1, Hq=1, Hkv=1, d=128, L0=1, W=32, S=64, B=1,
                              V=1000, rounds=6, p_match=0.5, seed=41),
    # one drafted token, eight query heads per KV head, a prefix that wraps the window
    "min_b1_g8": WLM.Workload("min_b1_g8", "bf16", C=2, Hq=16, Hkv=2, d=128, L0=1000, W=32, S=128, B=1,
                              V=1000, rounds=6, p_match=0.5, seed=42),
}


@pytest.mark.parametrize("name", list(MINIMAL_ROUND))
def test_round_minimal_shapes_against_the_oracle(name):
    """The one-call round at the smallest shapes its fused kernel takes."""
    wl = MINIMAL_ROUND[name]
    _announce(wl, f"rounds={wl.rounds} one-call round")
    H.lockstep(wl, wl.rounds, calls="round")


MAXIMAL_ROUND = {
    # the largest block the fused kernel takes (B + 1 = 32 verified rows, a
    # 31-row block chunk), every draft accepted: tau = 32 every round, so the
    # chunk of new rows is full and the 64-row window wraps every other round;
    # 62 query rows per KV head (two workgroups)
    "max_b31_g2_all": WLM.Workload("max_b31_g2_all", "bf16", C=2, Hq=8, Hkv=4, d=128, L0=100, W=64,
                                   S=128, B=31, V=3000, rounds=6, p_match=1.0, seed=43),
    # the same block at one query row per draft and KV head (one workgroup),
    # a long window and mostly accepted drafts
    "max_b31_g1": WLM.Workload("max_b31_g1", "bf16", C=3, Hq=2, Hkv=2, d=128, L0=700, W=256, S=64,
                               B=31, V=3000, rounds=6, p_match=0.97, seed=44),
}


@pytest.mark.parametrize("name", list(MAXIMAL_ROUND))
def test_round_largest_block_against_the_oracle(name):
    """The one-call round at the largest block its fused kernel takes."""
    wl = MAXIMAL_ROUND[name]
    _announce(wl, f"rounds={wl.rounds} one-call round")
    _, _, stats = H.lockstep(wl, wl.rounds, calls="round")
    if wl.p_match == 1.0:
        assert all((t == wl.B + 1).all() for t in stats["tau"]), "every draft accepted"


def test_round_when_sibling_workgroups_run_apart():
    """C = 48 units of 64 query rows: 768 workgroups for 256 CUs, so the two
    workgroups of a (sequence, KV head) run in different waves of the
    dispatch and the second starts after the first has finished.  The state
    must still be merged exactly once (the arrival counters pick the writer);
    checked against the oracle on sampled heads, every round."""
    wl = WLM.Workload("siblings_apart", "bf16", C=48, Hq=32, Hkv=8, d=128, L0=600, W=256, S=128, B=16,
                      V=4096, rounds=4, p_match=0.8, seed=43)
    assert wl.B * wl.Hq // wl.Hkv == 64 and wl.C * wl.Hkv * 2 >= 3 * 256
    _announce(wl, "one-call round, sibling workgroups in different dispatch waves")
    H.lockstep(wl, wl.rounds, calls="round", heads=[(0, 0), (17, 3), (47, 7)])
