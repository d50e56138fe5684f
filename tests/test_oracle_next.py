"""Pins of the oracle's next-step functions (no GPU).

draft_argmax (the drafter's proposal at T = 0), boundary_row (the boundary
state view), verify_attention (the target's causal attention of the verified
block over the whole context) and the drafting path with one view switched
off (S = 0 or W = 0).  As in test_oracle.py, every pin is independent of the
oracle's code: hand-worked examples under tests/golden/, brute force in plain
Python, torch's scaled_dot_product_attention with an explicit mask, and
special cases; the last test plants mistakes in the oracle and checks that a
pin fails.
"""
import json
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
# drafter proposal at T = 0
# --------------------------------------------------------------------------
def test_draft_argmax_worked_example():
    case = _load("draft_argmax_worked_example.json")
    got = O.draft_argmax(np.asarray(case["logits"], dtype=np.float32))
    assert got.dtype == np.int32
    assert got.tolist() == case["draft"]


def _first_max_index(row):
    best, at = None, None
    for i, x in enumerate(row):
        if best is None or x > best:   # strict: the first occurrence wins
            best, at = x, i
    return at


def test_draft_argmax_brute_force_with_ties():
    rng = _rng(7)
    x = WLM.f32_to_bf16_bits(rng.standard_normal((3, 4, 97)).astype(np.float32))
    # plant ties: copy each row's max to a later and an earlier index
    x = x.copy()
    for c in range(3):
        for b in range(4):
            vals = WLM.bf16_bits_to_f32(x[c, b])
            j = int(np.argmax(vals))
            x[c, b, (j + 11) % 97] = x[c, b, j]
            if b % 2:
                x[c, b, max(0, j - 5)] = x[c, b, j]
    got = O.draft_argmax(x)
    f = WLM.bf16_bits_to_f32(x)
    for c in range(3):
        for b in range(4):
            assert got[c, b] == _first_max_index(f[c, b].tolist())


def test_draft_argmax_is_verify_target_of_the_same_rows():
    """The drafter's argmax and the target's greedy token are the same reduction."""
    rng = _rng(8)
    logits = WLM.f32_to_bf16_bits(rng.standard_normal((2, 6, 50)).astype(np.float32))
    target, _ = O.verify_greedy(logits, np.zeros((2, 5), dtype=np.int32))
    assert np.array_equal(O.draft_argmax(logits[:, :5]), target[:, :5])


# --------------------------------------------------------------------------
# boundary state view
# --------------------------------------------------------------------------
def test_boundary_worked_example():
    case = _load("boundary_worked_example.json")
    got = O.boundary_row(np.asarray(case["hidden"], dtype=np.float32), case["tau"])
    assert got.tolist() == case["boundary"]


def test_boundary_extremes_and_bits():
    rng = _rng(9)
    hidden = WLM.f32_to_bf16_bits(rng.standard_normal((4, 5, 16)).astype(np.float32))
    # tau = 1: only the last committed token x0 (row 0); tau = B+1: every row
    got = O.boundary_row(hidden, [1, 5, 1, 5])
    assert got.dtype == np.uint16
    assert np.array_equal(got[0], hidden[0, 0]) and np.array_equal(got[2], hidden[2, 0])
    assert np.array_equal(got[1], hidden[1, 4]) and np.array_equal(got[3], hidden[3, 4])
    with pytest.raises(ValueError):
        O.boundary_row(hidden, [0, 1, 1, 1])
    with pytest.raises(ValueError):
        O.boundary_row(hidden, [6, 1, 1, 1])


# --------------------------------------------------------------------------
# target-side verification attention
# --------------------------------------------------------------------------
def test_verify_attention_worked_example():
    case = _load("verify_attention_worked_example.json")
    k = np.asarray(case["k"], dtype=np.float32)[None]   # [1, R, Hkv, d]
    v = np.asarray(case["v"], dtype=np.float32)[None]
    q = np.asarray(case["q"], dtype=np.float32)[None]   # [1, B+1, Hq, d]
    got = O.verify_attention(k, v, q, [case["L"]])
    np.testing.assert_allclose(got[0], np.asarray(case["out"]), rtol=0, atol=1e-7)


def _sdpa_verify(k, v, q, L, G):
    """torch SDPA with an explicit boolean mask, GQA by repeating KV heads."""
    C, B1, Hq, d = q.shape
    out = np.zeros(q.shape)
    for c in range(C):
        n = L[c] + B1
        kk = torch.tensor(k[c, :n], dtype=torch.float64).permute(1, 0, 2)   # [Hkv, n, d]
        vv = torch.tensor(v[c, :n], dtype=torch.float64).permute(1, 0, 2)
        qq = torch.tensor(q[c], dtype=torch.float64).permute(1, 0, 2)       # [Hq, B1, d]
        kk = kk.repeat_interleave(G, dim=0)
        vv = vv.repeat_interleave(G, dim=0)
        mask = torch.arange(n)[None, :] <= (L[c] + torch.arange(B1))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        out[c] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("Hq,Hkv,B1", [(4, 2, 5), (6, 3, 1), (2, 2, 3)])
def test_verify_attention_sdpa(Hq, Hkv, B1):
    rng = _rng(10 + Hq + B1)
    C, d = 3, 16
    L = [0, 7, 20]
    R = max(L) + B1
    k = rng.standard_normal((C, R, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((C, R, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((C, B1, Hq, d)).astype(np.float32)
    got = O.verify_attention(k, v, q, L)
    np.testing.assert_allclose(got, _sdpa_verify(k, v, q, L, Hq // Hkv), rtol=1e-12, atol=1e-12)


def test_verify_attention_special_cases():
    rng = _rng(11)
    d = 8
    k = rng.standard_normal((1, 6, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, 6, 1, d)).astype(np.float32)
    # L = 0: causal self-attention among the block
    q = rng.standard_normal((1, 6, 1, d)).astype(np.float32)
    got = O.verify_attention(k, v, q, [0])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q[0, :, 0], dtype=torch.float64)[None], torch.tensor(k[0, :, 0], dtype=torch.float64)[None],
        torch.tensor(v[0, :, 0], dtype=torch.float64)[None], is_causal=True)[0]
    np.testing.assert_allclose(got[0, :, 0], ref.numpy(), rtol=1e-12, atol=1e-12)
    # one verified position (B = 0): plain decode attention over all L + 1 rows
    q1 = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    got1 = O.verify_attention(k, v, q1, [5])
    s = (q1[0, 0, 0].astype(np.float64) @ k[0, :, 0].T.astype(np.float64)) / np.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    np.testing.assert_allclose(got1[0, 0, 0], p @ v[0, :, 0].astype(np.float64), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# one view switched off (S = 0 or W = 0)
# --------------------------------------------------------------------------
def _views_case(seed, W, S, L0=30, B=3, C=2, Hkv=2, G=2, d=8):
    rng = _rng(seed)
    kp = rng.standard_normal((C, L0, Hkv, d)).astype(np.float32)
    vp = rng.standard_normal((C, L0, Hkv, d)).astype(np.float32)
    u = rng.standard_normal((Hkv, S, d)).astype(np.float32)
    logl = np.log(np.linspace(0.5, 0.99, S)) if S else np.zeros((0,))
    st = O.summary_init(u, logl, kp, vp, W)
    q = rng.standard_normal((C, B, Hkv * G, d)).astype(np.float32)
    kb = rng.standard_normal((C, B, Hkv, d)).astype(np.float32)
    vb = rng.standard_normal((C, B, Hkv, d)).astype(np.float32)
    return st, kp, vp, q, kb, vb


def _sdpa_over(keys, vals, qrows):
    s = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(qrows, dtype=torch.float64)[None], torch.tensor(keys, dtype=torch.float64)[None],
        torch.tensor(vals, dtype=torch.float64)[None])[0]
    return s.numpy()


def test_draft_attention_without_summary_slots():
    """S = 0: the drafter attends to the window and the block only."""
    st, kp, vp, q, kb, vb = _views_case(12, W=8, S=0)
    out = O.draft_attention(st, q, kb, vb)
    G = q.shape[2] // kb.shape[2]
    for c in range(q.shape[0]):
        for hq in range(q.shape[2]):
            h = hq // G
            keys = np.concatenate([kp[c, -8:, h], kb[c, :, h]])
            vals = np.concatenate([vp[c, -8:, h], vb[c, :, h]])
            np.testing.assert_allclose(out[c, :, hq], _sdpa_over(keys, vals, q[c, :, hq]),
                                       rtol=1e-12, atol=1e-12)


def test_draft_attention_without_window():
    """W = 0: the drafter attends to the summary slots and the block only."""
    st, kp, vp, q, kb, vb = _views_case(13, W=0, S=4)
    out = O.draft_attention(st, q, kb, vb)
    G = q.shape[2] // kb.shape[2]
    for c in range(q.shape[0]):
        for hq in range(q.shape[2]):
            h = hq // G
            m, l, n = O.summary_reference(st.u[h], st.log_lambda, kp[c, :, h], vp[c, :, h])
            d = kp.shape[-1]
            keys = np.concatenate([n[:, :d] / l[:, None], kb[c, :, h]])
            vals = np.concatenate([n[:, d:] / l[:, None], vb[c, :, h]])
            np.testing.assert_allclose(out[c, :, hq], _sdpa_over(keys, vals, q[c, :, hq]),
                                       rtol=1e-12, atol=1e-12)


def test_append_without_window_keeps_counting_and_summary():
    """W = 0: no ring rows, seq_len still advances, the summary still covers every row."""
    st, kp, vp, _, _, _ = _views_case(14, W=0, S=4, L0=10, C=1, Hkv=1)
    rng = _rng(15)
    rows_k, rows_v = [kp[0, :, 0]], [vp[0, :, 0]]
    for tau in (2, 1, 4):
        kn = rng.standard_normal((1, 4, 1, 8)).astype(np.float32)
        vn = rng.standard_normal((1, 4, 1, 8)).astype(np.float32)
        O.append_accepted(st, kn, vn, [tau])
        rows_k.append(kn[0, :tau, 0])
        rows_v.append(vn[0, :tau, 0])
    assert st.ring_k.shape[2] == 0 and int(st.seq_len[0]) == 10 + 7
    m, l, n = O.summary_reference(st.u[0], st.log_lambda, np.concatenate(rows_k), np.concatenate(rows_v))
    np.testing.assert_allclose(st.m[0, 0], m, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st.n[0, 0] / st.l[0, 0][:, None], n / l[:, None], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# the pins catch planted mistakes
# --------------------------------------------------------------------------
def _run_pins():
    pins = [
        test_draft_argmax_worked_example,
        test_draft_argmax_brute_force_with_ties,
        test_boundary_worked_example,
        test_boundary_extremes_and_bits,
        test_verify_attention_worked_example,
        lambda: test_verify_attention_sdpa(4, 2, 5),
        test_verify_attention_special_cases,
    ]
    failed = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            failed += 1
    return failed


_real_verify_attention = O.verify_attention


def _argmax_last_on_ties(logits):
    x = O.decode(logits)
    return (x.shape[-1] - 1 - np.argmax(x[..., ::-1], axis=-1)).astype(np.int32)


def _boundary_off_by_one(hidden, tau):
    hidden = np.asarray(hidden)
    tau = np.minimum(np.asarray(tau), hidden.shape[1] - 1)
    return np.stack([hidden[c, t] for c, t in enumerate(tau)])


def _verify_full(k_cache, v_cache, q, L):
    """every verified query sees all L + B + 1 rows (the causal mask dropped)"""
    C, B1, Hq, d = q.shape
    G = Hq // k_cache.shape[2]
    out = np.zeros(q.shape)
    for c in range(C):
        n = int(L[c]) + B1
        for hq in range(Hq):
            kk = O.decode(k_cache[c, :n, hq // G])
            vv = O.decode(v_cache[c, :n, hq // G])
            s = O.decode(q[c, :, hq]) @ kk.T / np.sqrt(d)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[c, :, hq] = (p / p.sum(axis=1, keepdims=True)) @ vv
    return out


def _verify_shifted_mask(k_cache, v_cache, q, L, pairs=None):
    """query i sees rows 0..L+i-1 (its own row dropped)"""
    C, B1, Hq, d = q.shape
    G = Hq // k_cache.shape[2]
    out = np.zeros(q.shape)
    for c in range(C):
        n = int(L[c]) + B1
        for hq in range(Hq):
            kk = O.decode(k_cache[c, :n, hq // G])
            vv = O.decode(v_cache[c, :n, hq // G])
            s = O.decode(q[c, :, hq]) @ kk.T / np.sqrt(d)
            vis = np.arange(n)[None, :] < (int(L[c]) + np.arange(B1))[:, None]
            vis[:, 0] = True
            s = np.where(vis, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[c, :, hq] = (p / p.sum(axis=1, keepdims=True)) @ vv
    return out


@pytest.mark.parametrize("name,target,mutant", [
    ("argmax keeps the last tie", "draft_argmax", _argmax_last_on_ties),
    ("boundary one row late", "boundary_row", _boundary_off_by_one),
    ("causal mask dropped", "verify_attention", lambda k, v, q, L, pairs=None: _verify_full(k, v, q, L)),
    ("causal mask shifted", "verify_attention", _verify_shifted_mask),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, target, mutant):
    assert _run_pins() == 0
    monkeypatch.setattr(O, target, mutant)
    assert _run_pins() > 0, f"no pin caught: {name}"
