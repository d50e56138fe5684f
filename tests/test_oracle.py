"""Pins of the CPU oracle against facts the definitions fix (no GPU).

Each pin is independent of the oracle's own code: hand-worked examples
(tests/golden/, each citing the page passage), brute force in plain Python,
textbook special cases through torch's scaled_dot_product_attention, and
invariants (incremental update == full recompute, ring closed form,
permutation invariance).  ``test_pins_catch_planted_mistakes`` plants
plausible mistakes in the oracle and checks that some pin fails.
"""
import collections
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import longspark_oracle as O
from fixed_cost_drafter_amd import workload as WLM
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# decoding
# --------------------------------------------------------------------------
def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC040, 0x4090, 0x0000, 0x8000, 0x3E80], dtype=np.uint16)
    assert O.decode(bits).tolist() == [1.0, -3.0, 4.5, 0.0, -0.0, 0.25]


# --------------------------------------------------------------------------
# summary pins
# --------------------------------------------------------------------------
def _summary_case_arrays(case):
    lam = np.asarray(case["lambda"], dtype=np.float64)
    with np.errstate(divide="ignore"):
        logl = np.log(lam)
    return (np.asarray(case["u"]), logl, np.asarray(case["K"]), np.asarray(case["V"]))


@pytest.mark.parametrize("idx", [0, 1])
def test_summary_worked_example(idx):
    case = _load("summary_worked_example.json")["cases"][idx]
    u, logl, K, V = _summary_case_arrays(case)
    m, l, n = O.summary_reference(u, logl, K, V)
    d = case["d"]
    np.testing.assert_allclose(m, case["m"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, case["l"], rtol=1e-13)
    np.testing.assert_allclose(n[:, :d] / l[:, None], case["slot_k"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(n[:, d:] / l[:, None], case["slot_v"], rtol=1e-13, atol=1e-14)


def _rand_summary(seed, L=37, d=8, S=6, lam=(1.0, 0.9, 0.5, 0.1, 0.0, 0.999)):
    r = _rng(seed)
    u = r.standard_normal((S, d))
    K = r.standard_normal((L, d))
    V = r.standard_normal((L, d))
    with np.errstate(divide="ignore"):
        logl = np.log(np.asarray(lam[:S], dtype=np.float64))
    return u, logl, K, V


def test_summary_lambda_one_is_softmax_pooling_sdpa():
    """lambda = 1: the slot is plain softmax attention of u_j over the rows (values [k; v])."""
    u, _, K, V = _rand_summary(1, S=5)
    logl = np.zeros(5)
    m, l, n = O.summary_reference(u, logl, K, V)
    d = K.shape[1]
    q = torch.tensor(u)[None, None]
    k = torch.tensor(K)[None, None]
    v = torch.tensor(np.concatenate([K, V], 1))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1 / math.sqrt(d))[0, 0]
    np.testing.assert_allclose(n / l[:, None], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_summary_decay_is_alibi_bias_sdpa():
    """Any lambda: SDPA with the additive bias (t-p) ln(lambda_j) (-inf for lambda = 0, p < t)."""
    u, logl, K, V = _rand_summary(2)
    L, d = K.shape
    t = L - 1
    bias = np.empty((u.shape[0], L))
    for j in range(u.shape[0]):
        for p in range(L):
            if p == t:
                bias[j, p] = 0.0
            elif logl[j] == -np.inf:
                bias[j, p] = -np.inf
            else:
                bias[j, p] = (t - p) * logl[j]
    q = torch.tensor(u)[None, None]
    k = torch.tensor(K)[None, None]
    v = torch.tensor(np.concatenate([K, V], 1))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.tensor(bias)[None, None], scale=1 / math.sqrt(d))[0, 0]
    m, l, n = O.summary_reference(u, logl, K, V)
    np.testing.assert_allclose(n / l[:, None], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_summary_naive_weights_tiny():
    """Direct weights exp(s) * lambda**(t-p) with Python's pow (0**0 = 1), no max-subtraction."""
    lam = [1.0, 0.9, 0.5, 0.0]
    u, logl, K, V = _rand_summary(3, L=6, d=4, S=4, lam=lam)
    m, l, n = O.summary_reference(u, logl, K, V)
    L, d = K.shape
    t = L - 1
    for j in range(4):
        wsum = 0.0
        acc = [0.0] * (2 * d)
        for p in range(L):
            s = sum(u[j][e] * K[p][e] for e in range(d)) / math.sqrt(d)
            w = math.exp(s) * lam[j] ** (t - p)
            wsum += w
            for e in range(d):
                acc[e] += w * K[p][e]
                acc[d + e] += w * V[p][e]
        assert math.isclose(l[j] * math.exp(m[j]), wsum, rel_tol=1e-12)
        np.testing.assert_allclose(n[j] / l[j], np.array(acc) / wsum, rtol=1e-12, atol=1e-13)


def test_summary_lambda_zero_is_newest_row_and_single_row():
    u, logl, K, V = _rand_summary(4)
    m, l, n = O.summary_reference(u, logl, K, V)
    j0 = int(np.where(np.isneginf(logl))[0][0])
    d = K.shape[1]
    assert l[j0] == 1.0
    np.testing.assert_array_equal(n[j0], np.concatenate([K[-1], V[-1]]))
    # a single retained row: every slot is that row, m = u.k/sqrt(d), l = 1
    m1, l1, n1 = O.summary_reference(u, logl, K[:1], V[:1])
    np.testing.assert_array_equal(l1, np.ones_like(l1))
    np.testing.assert_allclose(m1, u @ K[0] / math.sqrt(d), rtol=1e-15)
    np.testing.assert_allclose(n1, np.tile(np.concatenate([K[0], V[0]]), (u.shape[0], 1)))


def test_summary_init_and_bf16_inputs_decode_exactly():
    """bf16 inputs: the oracle sees the exact decoded values (compare with f64 inputs)."""
    wl = WLM.WORKLOADS["tiny_f32"].with_(dtype="bf16", C=2, Hkv=2, Hq=4, L0=20, S=4)
    u = WLM.slot_queries(wl)
    logl = WLM.log_lambda(wl)
    K, V = WLM.prefix(wl, threads=1)
    st = O.summary_init(u, logl, K, V, wl.W)
    for c in range(2):
        for h in range(2):
            m, l, n = O.summary_reference(WLM.bf16_bits_to_f32(u[h]).astype(np.float64), logl,
                                          WLM.bf16_bits_to_f32(K[c, :, h]).astype(np.float64),
                                          WLM.bf16_bits_to_f32(V[c, :, h]).astype(np.float64))
            np.testing.assert_array_equal(st.m[c, h], m)
            np.testing.assert_array_equal(st.n[c, h], n)


# --------------------------------------------------------------------------
# ring window pins
# --------------------------------------------------------------------------
def _ring_closed_form(L, W):
    pos = np.full(W, -1)
    for s in range(W):
        p = L - 1 - ((L - 1 - s) % W)
        pos[s] = p if p >= 0 else -1
    return pos


def _tiny_state(C=2, Hkv=2, d=4, W=8, S=3, L0=5, dtype=np.float32, seed=5):
    r = _rng(seed)
    u = r.standard_normal((Hkv, S, d)).astype(dtype)
    logl = np.log(np.array([1.0, 0.5, 0.9][:S]))
    K = r.standard_normal((C, L0, Hkv, d)).astype(dtype)
    V = r.standard_normal((C, L0, Hkv, d)).astype(dtype)
    return O.summary_init(u, logl, K, V, W), K, V


def test_ring_worked_example():
    g = _load("ring_worked_example.json")
    W, L0 = g["W"], g["L0"]
    st, _, _ = _tiny_state(C=1, Hkv=1, W=W, L0=L0)
    assert st.ring_pos[0].tolist() == g["ring_pos_after_init"]
    r = _rng(0)
    for T, pos, sl in zip(g["appends"], g["ring_pos_after"], g["seq_len_after"]):
        kn = r.standard_normal((1, 4, 1, 4)).astype(np.float32)
        O.append_accepted(st, kn, kn, np.array([T]))
        assert st.ring_pos[0].tolist() == pos
        assert int(st.seq_len[0]) == sl


def test_ring_matches_closed_form_and_deque():
    C, Hkv, d, W, B = 2, 2, 4, 8, 5
    st, K, V = _tiny_state(C=C, Hkv=Hkv, d=d, W=W, L0=3)
    dq = [collections.deque(maxlen=W) for _ in range(C)]
    for c in range(C):
        for p in range(3):
            dq[c].append((p, K[c, p].copy()))
    r = _rng(11)
    for _ in range(12):
        kn = r.standard_normal((C, B + 1, Hkv, d)).astype(np.float32)
        vn = r.standard_normal((C, B + 1, Hkv, d)).astype(np.float32)
        tau = r.integers(1, B + 2, size=C)
        for c in range(C):
            for i in range(tau[c]):
                dq[c].append((int(st.seq_len[c]) + i, kn[c, i].copy()))
        O.append_accepted(st, kn, vn, tau)
        for c in range(C):
            L = int(st.seq_len[c])
            np.testing.assert_array_equal(st.ring_pos[c], _ring_closed_form(L, W))
            for p, row in dq[c]:
                np.testing.assert_array_equal(st.ring_k[c, :, p % W, :], row)
                assert st.ring_pos[c, p % W] == p


# --------------------------------------------------------------------------
# incremental summary == full recompute (Fig. 3)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L0", [1, 5, 40])
def test_incremental_equals_full_recompute(L0):
    C, Hkv, d, W, S, B = 2, 2, 6, 8, 6, 4
    r = _rng(100 + L0)
    u = r.standard_normal((Hkv, S, d)).astype(np.float32)
    with np.errstate(divide="ignore"):
        logl = np.log(np.array([1.0, 0.999, 0.9, 0.5, 0.1, 0.0])).astype(np.float32)
    K = r.standard_normal((C, L0, Hkv, d)).astype(np.float32)
    V = r.standard_normal((C, L0, Hkv, d)).astype(np.float32)
    st = O.summary_init(u, logl, K, V, W)
    hist_k = [[K[c, :, h, :] for h in range(Hkv)] for c in range(C)]
    hist_v = [[V[c, :, h, :] for h in range(Hkv)] for c in range(C)]
    for _ in range(15):
        kn = r.standard_normal((C, B + 1, Hkv, d)).astype(np.float32)
        vn = r.standard_normal((C, B + 1, Hkv, d)).astype(np.float32)
        tau = r.integers(1, B + 2, size=C)
        O.append_accepted(st, kn, vn, tau)
        for c in range(C):
            for h in range(Hkv):
                hist_k[c][h] = np.concatenate([hist_k[c][h], kn[c, :tau[c], h, :]])
                hist_v[c][h] = np.concatenate([hist_v[c][h], vn[c, :tau[c], h, :]])
    for c in range(C):
        for h in range(Hkv):
            m, l, n = O.full_recompute(u[h], logl, hist_k[c][h], hist_v[c][h])
            np.testing.assert_allclose(st.m[c, h], m, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(st.l[c, h], l, rtol=1e-12)
            np.testing.assert_allclose(st.n[c, h], n, rtol=1e-11, atol=1e-12)


def test_append_rejects_out_of_range_tau():
    st, _, _ = _tiny_state()
    kn = np.zeros((2, 4, 2, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        O.append_accepted(st, kn, kn, np.array([0, 1]))
    with pytest.raises(ValueError):
        O.append_accepted(st, kn, kn, np.array([1, 5]))


# --------------------------------------------------------------------------
# greedy verification pins
# --------------------------------------------------------------------------
def test_verify_worked_example():
    g = _load("verify_worked_example.json")
    logits = np.asarray(g["logits"], dtype=np.float32)
    target, tau = O.verify_greedy(logits, np.asarray(g["draft"], dtype=np.int32))
    assert target.tolist() == g["target_tok"]
    assert tau.tolist() == g["tau"]
    # the same logits as bf16 bit patterns (all values are exact in bf16)
    target2, tau2 = O.verify_greedy(WLM.f32_to_bf16_bits(logits), np.asarray(g["draft"]))
    assert target2.tolist() == g["target_tok"] and tau2.tolist() == g["tau"]


def _brute_verify(x, draft):
    C, B1, V = len(x), len(x[0]), len(x[0][0])
    tgt, tau = [], []
    for c in range(C):
        row_t = []
        for i in range(B1):
            best, arg = None, None
            for v in range(V):
                if best is None or x[c][i][v] > best:
                    best, arg = x[c][i][v], v
            row_t.append(arg)
        M = 0
        while M < B1 - 1 and draft[c][M] == row_t[M]:
            M += 1
        tgt.append(row_t)
        tau.append(M + 1)
    return tgt, tau


def test_verify_brute_force_with_many_ties():
    r = _rng(7)
    C, B, V = 6, 5, 9
    for trial in range(20):
        x = r.integers(-2, 3, size=(C, B + 1, V)).astype(np.float32)   # heavy ties
        bt, _ = _brute_verify(x.tolist(), [[0] * B] * C)
        draft = np.array([[bt[c][i] if r.random() < 0.7 else (bt[c][i] + 1) % V
                           for i in range(B)] for c in range(C)], dtype=np.int32)
        tgt, tau = O.verify_greedy(x, draft)
        bt, btau = _brute_verify(x.tolist(), draft.tolist())
        assert tgt.tolist() == bt and tau.tolist() == btau


def test_verify_recovers_planted_tokens_and_mean_tau():
    wl = WLM.WORKLOADS["tiny_f32"].with_(C=64, V=40, B=6, p_match=0.75)
    taus = []
    for k in range(12):
        logits, g = WLM.logits_entry(wl, k)
        rnd = WLM.round_inputs(wl, k, g)
        tgt, tau = O.verify_greedy(logits, rnd["draft"])
        np.testing.assert_array_equal(tgt, g)
        assert np.all((tau >= 1) & (tau <= wl.B + 1))
        taus.append(tau)
    taus = np.concatenate(taus).astype(np.float64)
    se = taus.std() / math.sqrt(taus.size)
    assert abs(taus.mean() - WLM.expected_tau(wl)) < 4 * se


# --------------------------------------------------------------------------
# draft attention pins
# --------------------------------------------------------------------------
def test_draft_attention_worked_example():
    g = _load("draft_attention_worked_example.json")
    d = g["d"]
    nr = len(g["ring_pos"])
    st = O.OracleState(
        u=np.zeros((1, 1, d)), log_lambda=np.zeros(1),
        m=np.zeros((1, 1, 1)), l=np.ones((1, 1, 1)),
        n=np.concatenate([np.asarray(g["slot_k"]), np.asarray(g["slot_v"])], 1)[None, None],
        ring_k=np.asarray(g["ring_k"])[None, None], ring_v=np.asarray(g["ring_v"])[None, None],
        ring_pos=np.asarray(g["ring_pos"], dtype=np.int32)[None], seq_len=np.array([8]))
    assert st.ring_k.shape == (1, 1, nr, d)
    q = np.asarray(g["q"])[None, None, None]
    kb = np.asarray(g["block_k"])[None, :, None]
    vb = np.asarray(g["block_v"])[None, :, None]
    out = O.draft_attention(st, q, kb, vb)
    np.testing.assert_allclose(out[0, 0, 0], g["out"], rtol=1e-14)


def _rand_round_state(seed, C=2, Hq=4, Hkv=2, d=8, W=8, S=3, B=3, L0=5):
    st, _, _ = _tiny_state(C=C, Hkv=Hkv, d=d, W=W, S=S, L0=L0, seed=seed)
    r = _rng(seed + 1)
    q = r.standard_normal((C, B, Hq, d))
    kb = r.standard_normal((C, B, Hkv, d))
    vb = r.standard_normal((C, B, Hkv, d))
    return st, q, kb, vb


def test_draft_attention_brute_force_loops():
    st, q, kb, vb = _rand_round_state(21)
    out = O.draft_attention(st, q, kb, vb)
    C, B, Hq, d = q.shape
    G = Hq // kb.shape[2]
    for c in range(C):
        for hq in range(Hq):
            h = hq // G
            keys, vals = [], []
            for s in range(st.ring_k.shape[2]):
                if st.ring_pos[c, s] >= 0:
                    keys.append(st.ring_k[c, h, s].astype(float).tolist())
                    vals.append(st.ring_v[c, h, s].astype(float).tolist())
            for j in range(st.n.shape[2]):
                keys.append((st.n[c, h, j, :d] / st.l[c, h, j]).tolist())
                vals.append((st.n[c, h, j, d:] / st.l[c, h, j]).tolist())
            for b2 in range(B):
                keys.append(kb[c, b2, h].tolist())
                vals.append(vb[c, b2, h].tolist())
            for b in range(B):
                sc = [sum(q[c, b, hq, e] * k[e] for e in range(d)) / math.sqrt(d) for k in keys]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                z = sum(w)
                ref = [sum(w[i] * vals[i][e] for i in range(len(w))) / z for e in range(d)]
                np.testing.assert_allclose(out[c, b, hq], ref, rtol=1e-12, atol=1e-13)


def test_draft_attention_sdpa_gqa():
    st, q, kb, vb = _rand_round_state(31, C=2, Hq=6, Hkv=2, L0=20)
    out = O.draft_attention(st, q, kb, vb)
    C, B, Hq, d = q.shape
    Hkv = kb.shape[2]
    for c in range(C):
        valid = st.ring_pos[c] >= 0
        K = np.concatenate([st.ring_k[c][:, valid].astype(float), st.slot_k[c],
                            kb[c].transpose(1, 0, 2)], axis=1)           # [Hkv, nk, d]
        Vv = np.concatenate([st.ring_v[c][:, valid].astype(float), st.slot_v[c],
                             vb[c].transpose(1, 0, 2)], axis=1)
        Kt = torch.tensor(K).repeat_interleave(Hq // Hkv, dim=0)
        Vt = torch.tensor(Vv).repeat_interleave(Hq // Hkv, dim=0)
        Qt = torch.tensor(q[c].transpose(1, 0, 2))                       # [Hq, B, d]
        ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=False)
        np.testing.assert_allclose(out[c], ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def test_draft_attention_ring_order_invariance_and_constant_values():
    st, q, kb, vb = _rand_round_state(41, L0=30)
    out = O.draft_attention(st, q, kb, vb)
    perm = _rng(3).permutation(st.ring_k.shape[2])
    st2 = st.copy()
    st2.ring_k = st.ring_k[:, :, perm]
    st2.ring_v = st.ring_v[:, :, perm]
    st2.ring_pos = st.ring_pos[:, perm]
    np.testing.assert_allclose(O.draft_attention(st2, q, kb, vb), out, rtol=1e-12, atol=1e-13)
    # every value equal to one vector -> output equals it
    st3 = st.copy()
    cvec = np.arange(st.d, dtype=np.float64) - 2.5
    st3.ring_v = np.broadcast_to(cvec, st.ring_v.shape).astype(np.float32)
    st3.n = st.n.copy()
    st3.n[..., st.d:] = st.l[..., None] * cvec
    out3 = O.draft_attention(st3, q, kb, np.broadcast_to(cvec, vb.shape))
    np.testing.assert_allclose(out3, np.broadcast_to(cvec, out3.shape), rtol=1e-12, atol=1e-12)


def test_draft_round_touches_fixed_number_of_rows():
    """Fixed cost: after any prefix length the round reads W + S + B rows per KV head."""
    for L0 in (3, 50, 400):
        st, q, kb, vb = _rand_round_state(51, W=8, L0=L0)
        n_keys = int((st.ring_pos[0] >= 0).sum()) + st.n.shape[2] + kb.shape[1]
        assert n_keys == min(L0, 8) + 3 + 3


# --------------------------------------------------------------------------
# the pins catch planted mistakes in the oracle
# --------------------------------------------------------------------------
def _run_pins():
    """Run a set of pins; return the number that failed."""
    pins = [
        lambda: test_summary_worked_example(0),
        lambda: test_summary_worked_example(1),
        test_summary_decay_is_alibi_bias_sdpa,
        test_summary_lambda_one_is_softmax_pooling_sdpa,
        lambda: test_incremental_equals_full_recompute(5),
        test_verify_worked_example,
        test_draft_attention_worked_example,
        test_draft_attention_sdpa_gqa,
        test_ring_worked_example,
    ]
    failed = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            failed += 1
    return failed


_real_decay_bias = O.decay_bias
_real_reference = O.summary_reference
_real_draft = O.draft_attention


def _bias_sign_flip(dist, log_lambda):
    return -_real_decay_bias(dist, log_lambda)


def _bias_off_by_one(dist, log_lambda):
    return _real_decay_bias(np.asarray(dist) + 1, log_lambda)


def _reference_no_scale(u, log_lambda, K, V, t=None):
    d = np.asarray(K).shape[1]
    return _real_reference(np.asarray(O.decode(u)) * math.sqrt(d), log_lambda, K, V, t)


def _draft_swapped_kv(state, q, k_blk, v_blk, pairs=None):
    return _real_draft(state, q, v_blk, k_blk, pairs)


@pytest.mark.parametrize("name,target,mutant", [
    ("decay sign", "decay_bias", _bias_sign_flip),
    ("decay off by one", "decay_bias", _bias_off_by_one),
    ("missing 1/sqrt(d)", "summary_reference", _reference_no_scale),
    ("block k/v swapped", "draft_attention", _draft_swapped_kv),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, target, mutant):
    assert _run_pins() == 0
    monkeypatch.setattr(O, target, mutant)
    assert _run_pins() > 0, f"no pin caught: {name}"
