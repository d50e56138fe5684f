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
    "bf16_vmax": SMALL["bf16_vmax"],              # V = 2^20: 128 chunks per row
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


@pytest.mark.parametrize("V", [20001, 20000])
def test_draft_argmax_edge_rows(V):
    """All-equal rows, -0 against +0, negative rows, the maximum at the last
    index or across a chunk boundary.  V = 20000 keeps rows 16-byte aligned
    (the packed 16-bit key path); V = 20001 does not (the scalar path)."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    wl = SMALL["bf16_s64_ragged"].with_(name="argmax_edges", C=1, B=12, V=V)
    H.log(f"CASE draft_argmax edges V={wl.V}")
    x = np.zeros((1, 12, wl.V), dtype=np.float32)
    x[0, 1, :] = -0.0
    x[0, 1, 7] = 0.0                       # +0 after -0s: index 0 still wins
    x[0, 2, :] = -1.0
    x[0, 2, wl.V - 1] = 2.0                # maximum at the last index
    x[0, 3, 16384] = 3.0                   # first element of a later chunk ...
    x[0, 3, 16383] = 3.0                   # ... tied with the last of the one before
    x[0, 4, ::2] = 1.5                     # every even index ties
    x[0, 5, 12345] = 1e-30                 # a tiny positive against zeros
    x[0, 6, :] = -1.0
    x[0, 6, 100] = -0.0
    x[0, 6, 50] = 0.0                      # +0 before -0, the rest negative: 50
    x[0, 7, :] = -1.0
    x[0, 7, 200] = 0.0
    x[0, 7, 150] = -0.0                    # -0 before +0: 150
    x[0, 8, :] = -2.0 - np.arange(wl.V) % 97   # all negative: the -2s tie, index 0
    x[0, 9, :] = -np.inf
    x[0, 9, wl.V - 2] = -3.0               # everything -inf but one
    x[0, 10, :] = -np.inf                  # all -inf: index 0
    x[0, 11, 8191] = 5.0
    x[0, 11, 8192] = 5.0                   # tie across the 8192-logit chunk boundary
    bits = WLM.f32_to_bf16_bits(x)
    st = _state(wl)
    out = torch.empty((1, 12), dtype=torch.int32, device="cuda")
    st.draft_argmax(LB.to_device(bits), out)
    torch.cuda.synchronize()
    got = LB.to_host(out)
    H.exact("edge rows", got, O.draft_argmax(bits))
    assert got.tolist() == [[0, 0, wl.V - 1, 16383, 0, 12345, 50, 150, 0, wl.V - 2, 0, 8191]]


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


# target-side verification attention (the prefix-dependent cost the drafter avoids)
ATTN_CASES = {
    # M = (B+1)*G = 24 query rows (2 waves); ragged contexts incl. L = 0, tiles + tails
    "bf16_m24": (SMALL["bf16_s64_ragged"].with_(name="vattn_m24", C=3, Hq=8, Hkv=2, B=5),
                 [0, 37, 300]),
    # M = 68 (5 waves, a 4-row tail group); contexts span several splits
    "bf16_m68": (SMALL["bf16_s64_ragged"].with_(name="vattn_m68", C=2, Hq=16, Hkv=4, B=16),
                 [5000, 777]),
    # f32 generic path
    "f32": (WLM.WORKLOADS["tiny_f32"].with_(name="vattn_f32", C=2, B=4), [60, 5]),
}


def _attn_run(wl, L, clamp_to=None):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    max_rows = max(L if clamp_to is None else clamp_to) + wl.B + 1
    rows = max_rows + 7                                   # rows_stride > max_rows
    Kc, Vc = WLM.prefix(wl, L0=rows, threads=4)
    q = WLM.verify_queries(wl, 0)
    st = LB.DrafterState.for_workload(wl, WLM.slot_queries(wl), WLM.log_lambda(wl),
                                      max_L0=max_rows - wl.B - 1)
    out = torch.empty((wl.C, wl.B + 1, wl.Hq, wl.d), dtype=LB.torch_dtype(wl.dtype), device="cuda")
    st.verify_attention(LB.to_device(Kc), LB.to_device(Vc),
                        LB.to_device(np.asarray(L, dtype=np.int32)), max_rows, LB.to_device(q), out)
    torch.cuda.synchronize()
    return Kc, Vc, q, LB.to_host(out), int(LB.to_host(st.err_flag)[0])


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_verify_attention_parity(name):
    wl, L = ATTN_CASES[name]
    H.log(f"CASE verify_attention {name} dtype={wl.dtype} C={wl.C} Hq={wl.Hq} Hkv={wl.Hkv} "
          f"B={wl.B} L={L} seed={wl.seed}")
    Kc, Vc, q, got, err = _attn_run(wl, L)
    assert err == 0
    H.close(f"verify_attention {name}", got, O.verify_attention(Kc, Vc, q, L), wl.dtype)


def test_verify_attention_full_size_sampled():
    """Qwen3-8B-shaped layer, 32K context, C = 16: sampled (sequence, head) pairs."""
    wl = WLM.WORKLOADS["q3_8b_32k"]
    L = [wl.L0 - 97 * c for c in range(wl.C)]             # ragged contexts near 32K
    H.log(f"CASE verify_attention full C={wl.C} L={L[0]}..{L[-1]} B={wl.B} V={wl.V}")
    Kc, Vc, q, got, err = _attn_run(wl, L)
    assert err == 0
    pairs = [(0, 0), (7, 13), (15, 31)]
    ref = O.verify_attention(Kc, Vc, q, L, pairs=pairs)
    for c, hq in pairs:
        H.close(f"verify_attention ({c},{hq})", got[c, :, hq], ref[c, :, hq], wl.dtype)


def test_verify_attention_clamps_and_flags_bad_context():
    wl, _ = ATTN_CASES["bf16_m24"]
    H.log("CASE verify_attention clamp L=[-4, 50, 10**6] max context 60")
    L = [-4, 50, 10 ** 6]
    Kc, Vc, q, got, err = _attn_run(wl, L, clamp_to=[0, 50, 60])
    assert err & 1
    H.close("verify_attention clamped", got, O.verify_attention(Kc, Vc, q, [0, 50, 60]), wl.dtype)


# sampled verification (textbook speculative sampling), fp32 decisions on the GPU.
# The GPU forms p and q in fp32 and sums the drawn row in fp32 (64-element
# segments, 256 segments, <= 64 chunks): relative error below 5e-5 for the
# acceptance test and below 2e-5 of the total for the running sums.  A decision
# inside that band may go either way: an acceptance inside it makes the rest of
# the sequence ambiguous (skipped, and counted); a draw accepts every token whose
# fp64 CDF interval comes within the band of the threshold (and has weight).
ACCEPT_EPS, DRAW_EPS = 5e-5, 2e-5


def _sampling_expectation(tl, dl, draft, T, ua, us, c):
    """(tau, accepted drafts, allowed drawn tokens) from the fp64 rule, or None when an
    acceptance decision of sequence c lies within ACCEPT_EPS of its threshold."""
    p = O.softmax_t(tl[c:c + 1], T)[0]
    q = O.softmax_t(dl[c:c + 1], T)[0]
    B = q.shape[0]
    j = 0
    while j < B:
        d = int(draft[c, j])
        a, b = float(ua[c, j]) * q[j, d], p[j, d]
        if max(a, b) > 0.0 and abs(a - b) <= ACCEPT_EPS * max(a, b):
            return None     # (0 < 0 is false in any precision: no ambiguity)
        if not a < b:
            break
        j += 1
    w = np.maximum(p[j] - q[j], 0.0) if j < B else p[B]
    if not np.any(w > 0.0):   # an empty residual: the oracle's rule draws from p_j
        w = p[j]
    cs = np.cumsum(w)
    thr = float(us[c]) * cs[-1]
    band = DRAW_EPS * cs[-1]
    lo = np.concatenate([[0.0], cs[:-1]])
    allowed = np.nonzero((w > 0) & (lo <= thr + band) & (cs >= thr - band))[0]
    return j + 1, [int(x) for x in draft[c, :j]], set(int(x) for x in allowed)


SAMPLING_CASES = {
    "bf16_small_T1": (SMALL["bf16_s64_ragged"].with_(name="samp_bf16", C=6, B=5, V=3000), 1.0),
    "bf16_small_T07": (SMALL["bf16_s64_ragged"].with_(name="samp_bf16_t07", C=6, B=5, V=20001), 0.7),
    "f32_tiny": (WLM.WORKLOADS["tiny_f32"].with_(name="samp_f32", C=4, B=4), 1.0),
    "q3_8b_full": (WLM.WORKLOADS["q3_8b_128k"], 1.0),
    # V = 2^20: 128 chunks per row, more than one lane's share (64) in the
    # decision's statistics merge
    "bf16_vmax_T1": (SMALL["bf16_vmax"], 1.0),
    "f32_vmax_T1": (SMALL["f32_vmax"], 1.0),
}


@pytest.mark.parametrize("name", list(SAMPLING_CASES))
def test_verify_sampling_parity(name):
    import torch
    from fixed_cost_drafter_amd import binding as LB
    wl, T = SAMPLING_CASES[name]
    H.log(f"CASE verify_sampling {name} dtype={wl.dtype} C={wl.C} B={wl.B} V={wl.V} T={T}")
    st = _state(wl)
    tokens = torch.empty((wl.C, wl.B + 1), dtype=torch.int32, device="cuda")
    tau = torch.empty((wl.C,), dtype=torch.int32, device="cuda")
    checked = skipped = 0
    for r in range(2):
        tl, _ = WLM.logits_entry(wl, r)
        inp = WLM.sampling_inputs(wl, r, tl, temperature=T)
        dl = inp["draft_logits"]
        st.verify_sampling(LB.to_device(tl), LB.to_device(dl), LB.to_device(inp["draft"]), T,
                           LB.to_device(inp["u_accept"]), LB.to_device(inp["u_sample"]), tokens, tau)
        torch.cuda.synchronize()
        got_tok, got_tau = LB.to_host(tokens), LB.to_host(tau)
        for c in range(wl.C):
            exp = _sampling_expectation(tl, dl, inp["draft"], T, inp["u_accept"], inp["u_sample"], c)
            if exp is None:
                skipped += 1
                continue
            checked += 1
            t_ref, acc, allowed = exp
            assert got_tau[c] == t_ref, (name, r, c, got_tau[c], t_ref)
            assert got_tok[c, :t_ref - 1].tolist() == acc, (name, r, c)
            assert int(got_tok[c, t_ref - 1]) in allowed, (name, r, c, got_tok[c, t_ref - 1], sorted(allowed)[:8])
            assert (got_tok[c, t_ref:] == -1).all()
    H.log(f"{name}: {checked} sequences compared, {skipped} with an acceptance within {ACCEPT_EPS}")
    assert skipped <= max(1, (checked + skipped) // 10)


def test_verify_sampling_equal_distributions_accept_all():
    """Drafter == target: every draft is accepted and the bonus comes from p_B."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    wl = SMALL["bf16_s64_ragged"].with_(name="samp_equal", C=4, B=6, V=5000)
    H.log(f"CASE verify_sampling equal distributions C={wl.C} B={wl.B} V={wl.V}")
    tl, _ = WLM.logits_entry(wl, 0)
    inp = WLM.sampling_inputs(wl, 0, tl, noise=0.0)
    st = _state(wl)
    tokens = torch.empty((wl.C, wl.B + 1), dtype=torch.int32, device="cuda")
    tau = torch.empty((wl.C,), dtype=torch.int32, device="cuda")
    st.verify_sampling(LB.to_device(tl), LB.to_device(inp["draft_logits"]), LB.to_device(inp["draft"]),
                       1.0, LB.to_device(inp["u_accept"]), LB.to_device(inp["u_sample"]), tokens, tau)
    torch.cuda.synchronize()
    assert LB.to_host(tau).tolist() == [wl.B + 1] * wl.C
    assert np.array_equal(LB.to_host(tokens)[:, :wl.B], inp["draft"])


def test_verify_sampling_empty_residual_draws_from_the_target():
    """Drafter == target except that row 1's drafted token has logit -inf in both:
    draft 0 is accepted, draft 1 rejected with p = q = 0, the residual
    max(0, p_1 - q_1) is zero everywhere and the token comes from p_1."""
    import torch
    from fixed_cost_drafter_amd import binding as LB
    wl = SMALL["bf16_s64_ragged"].with_(name="samp_empty_residual", C=5, B=4, V=20001)
    H.log(f"CASE verify_sampling empty residual C={wl.C} B={wl.B} V={wl.V}")
    tl, _ = WLM.logits_entry(wl, 3)
    inp = WLM.sampling_inputs(wl, 3, tl, noise=0.0)
    x = WLM.bf16_bits_to_f32(tl)
    draft = inp["draft"].copy()
    for c in range(wl.C):
        x[c, 1, draft[c, 1]] = -np.inf
    tl2 = WLM.f32_to_bf16_bits(x)
    dl2 = np.ascontiguousarray(tl2[:, :wl.B])
    ua = np.full((wl.C, wl.B), 0.5, dtype=np.float32)
    us = np.array([0.0, 0.25, 0.5, 0.75, 0.999], dtype=np.float32)
    st = _state(wl)
    tokens = torch.empty((wl.C, wl.B + 1), dtype=torch.int32, device="cuda")
    tau = torch.empty((wl.C,), dtype=torch.int32, device="cuda")
    st.verify_sampling(LB.to_device(tl2), LB.to_device(dl2), LB.to_device(draft), 1.0,
                       LB.to_device(ua), LB.to_device(us), tokens, tau)
    torch.cuda.synchronize()
    got_tok, got_tau = LB.to_host(tokens), LB.to_host(tau)
    ref_tok, ref_tau = O.verify_sampling(tl2, dl2, draft, 1.0, ua, us)
    assert got_tau.tolist() == ref_tau.tolist() == [2] * wl.C
    for c in range(wl.C):
        exp = _sampling_expectation(tl2, dl2, draft, 1.0, ua, us, c)
        assert exp is not None and exp[0] == 2
        assert int(got_tok[c, 0]) == int(draft[c, 0])
        assert int(got_tok[c, 1]) in exp[2], (c, got_tok[c, 1], sorted(exp[2])[:8], ref_tok[c, 1])
        assert (got_tok[c, 2:] == -1).all()
