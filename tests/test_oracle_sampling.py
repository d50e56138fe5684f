"""Pins of the oracle's sampled verification (no GPU).

softmax_t, inverse_cdf and verify_sampling (the textbook speculative-sampling
rule).  Independent of the oracle's code: a hand-worked example, brute force
in plain Python, torch's softmax, and the property that makes the rule
lossless -- the first emitted token is distributed as the target's own
distribution whatever the drafter's.  The last test plants mistakes in the
oracle and checks that a pin fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import longspark_oracle as O
from tests.conftest import GOLDEN


def test_sampling_worked_example():
    with open(os.path.join(GOLDEN, "sampling_worked_example.json")) as f:
        case = json.load(f)
    tokens, tau = O.verify_sampling(np.asarray(case["target_logits"], dtype=np.float32),
                                    np.asarray(case["draft_logits"], dtype=np.float32),
                                    np.asarray(case["draft"]), case["T"],
                                    np.asarray(case["u_accept"]), np.asarray(case["u_sample"]))
    assert tokens.tolist() == case["tokens"]
    assert tau.tolist() == case["tau"]


def _brute_inverse_cdf(w, u):
    total = 0.0
    for x in w:
        total += x
    run = 0.0
    for k, x in enumerate(w):
        run += x
        if run > u * total:
            return k
    return len(w) - 1


def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(40)
    for _ in range(200):
        w = rng.random(9) * (rng.random(9) < 0.6)       # many exact zeros
        if w.sum() == 0:
            w[3] = 1.0
        u = float(rng.choice([0.0, rng.random()]))
        k = O.inverse_cdf(w, u)
        assert k == _brute_inverse_cdf(w.tolist(), u)
        assert w[k] > 0                                  # never a zero-weight token


def test_softmax_t_matches_torch():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 50)).astype(np.float32)
    for T in (0.3, 1.0, 2.5):
        ref = torch.softmax(torch.tensor(x, dtype=torch.float64) / T, dim=-1).numpy()
        np.testing.assert_allclose(O.softmax_t(x, T), ref, rtol=1e-13, atol=1e-15)


def _first_token_histogram(p_logits, q_logits, T, trials, seed):
    """Empirical law of the first emitted token: drafts drawn from q, fresh uniforms."""
    rng = np.random.default_rng(seed)
    q = O.softmax_t(q_logits, T)
    V = q.shape[-1]
    counts = np.zeros(V)
    target = np.stack([p_logits, p_logits])[None]        # [1, 2, V]: row 0 and a bonus row
    for _ in range(trials):
        d = rng.choice(V, p=q[0])
        tokens, _ = O.verify_sampling(target, q_logits[None], np.array([[d]]), T,
                                      rng.random((1, 1)), rng.random(1))
        counts[tokens[0, 0]] += 1
    return counts / trials


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_first_token_is_distributed_as_the_target(T):
    """Speculative sampling is lossless: token 1 follows p_0 whatever q is."""
    rng = np.random.default_rng(42)
    p_logits = rng.standard_normal(6).astype(np.float32) * 1.5
    q_logits = (p_logits + rng.standard_normal(6).astype(np.float32) * 1.5)[None]
    trials = 20000
    freq = _first_token_histogram(p_logits, q_logits, T, trials, 43)
    p0 = O.softmax_t(p_logits, T)
    sigma = np.sqrt(p0 * (1 - p0) / trials)
    assert np.all(np.abs(freq - p0) < 5 * sigma + 1e-9), (freq, p0)


def test_equal_distributions_accept_every_draft():
    """p == q: every draft is accepted (u < 1 = p/q) and the bonus comes from p_B."""
    rng = np.random.default_rng(44)
    logits = rng.standard_normal((2, 4, 30)).astype(np.float32)
    draft = rng.integers(0, 30, size=(2, 3))
    u_s = np.array([0.3, 0.8])
    tokens, tau = O.verify_sampling(logits, logits[:, :3], draft, 1.0, rng.random((2, 3)), u_s)
    assert tau.tolist() == [4, 4]
    assert tokens[:, :3].tolist() == draft.tolist()
    for c in range(2):
        p_b = O.softmax_t(logits[c, 3], 1.0)
        assert tokens[c, 3] == _brute_inverse_cdf(p_b.tolist(), u_s[c])


def test_empty_residual_draws_from_the_target():
    """p_j == q_j with p_j(d) = q_j(d) = 0 (a drafted token with logit -inf):
    u * 0 < 0 fails, so d is rejected, max(0, p - q) is zero everywhere and the
    token comes from p_j itself (an inverse-CDF draw over the target row)."""
    rng = np.random.default_rng(45)
    logits = rng.standard_normal((3, 4, 25)).astype(np.float32)
    draft = rng.integers(0, 25, size=(3, 3))
    for c in range(3):                      # row 1: its draft has p = q = 0
        logits[c, 1, draft[c, 1]] = -np.inf
    draft[:, 0] = np.argmax(logits[:, 0], axis=-1)   # accepted: p/q = 1 > u
    u_s = np.array([0.05, 0.5, 0.95])
    tokens, tau = O.verify_sampling(logits, logits[:, :3], draft, 1.0, rng.random((3, 3)) * 0.9, u_s)
    assert tau.tolist() == [2, 2, 2]
    for c in range(3):
        p1 = O.softmax_t(logits[c, 1], 1.0)
        assert tokens[c, 0] == draft[c, 0]
        assert tokens[c, 1] == _brute_inverse_cdf(p1.tolist(), u_s[c])
        assert 0 <= tokens[c, 1] < 25 and tokens[c, 1] != draft[c, 1]


# --------------------------------------------------------------------------
# the pins catch planted mistakes
# --------------------------------------------------------------------------
def _run_pins():
    pins = [test_sampling_worked_example, test_inverse_cdf_brute_force,
            lambda: test_first_token_is_distributed_as_the_target(1.0),
            test_equal_distributions_accept_every_draft, test_empty_residual_draws_from_the_target]
    failed = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            failed += 1
    return failed


_real_inverse_cdf = O.inverse_cdf
_real_softmax_t = O.softmax_t


def _cdf_left(w, u):
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return int(np.searchsorted(c, u * c[-1], side="left"))


def _sampling_inverted_ratio(tl, dl, draft, T, ua, us):
    # accept when u * p < q: the ratio upside down
    return _generic_sampling(tl, dl, draft, T, ua, us, accept=lambda u, p, q: u * p < q)


def _sampling_unclipped_residual(tl, dl, draft, T, ua, us):
    return _generic_sampling(tl, dl, draft, T, ua, us, residual=lambda p, q: np.abs(p - q))


def _sampling_bonus_from_previous_row(tl, dl, draft, T, ua, us):
    return _generic_sampling(tl, dl, draft, T, ua, us, bonus_row=-2)


def _generic_sampling(tl, dl, draft, T, ua, us, accept=lambda u, p, q: u * q < p,
                      residual=lambda p, q: np.maximum(p - q, 0.0), bonus_row=-1):
    p = _real_softmax_t(tl, T)
    q = _real_softmax_t(dl, T)
    C, B1, _ = p.shape
    B = B1 - 1
    tokens = np.full((C, B1), -1, dtype=np.int32)
    tau = np.zeros((C,), dtype=np.int32)
    for c in range(C):
        j = 0
        while j < B and accept(ua[c, j], p[c, j, draft[c, j]], q[c, j, draft[c, j]]):
            tokens[c, j] = draft[c, j]
            j += 1
        w = residual(p[c, j], q[c, j]) if j < B else p[c, B1 + bonus_row]
        tokens[c, j] = _real_inverse_cdf(w, us[c])
        tau[c] = j + 1
    return tokens, tau


@pytest.mark.parametrize("name,target,mutant", [
    ("inverse CDF takes the boundary", "inverse_cdf", _cdf_left),
    ("acceptance ratio inverted", "verify_sampling", _sampling_inverted_ratio),
    ("residual not clipped at 0", "verify_sampling", _sampling_unclipped_residual),
    ("bonus from the wrong row", "verify_sampling", _sampling_bonus_from_previous_row),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, target, mutant):
    assert _run_pins() == 0
    monkeypatch.setattr(O, target, mutant)
    assert _run_pins() > 0, f"no pin caught: {name}"
