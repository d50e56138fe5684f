"""Plain CPU oracle for LongSpark's per-round fixed-cost drafting path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table
or helper with the HIP library; the two meet only through the seeded inputs.

Source: the paper page "LongSpark: Efficient speculative decoding with a
fixed-cost parallel drafter" (arXiv 2609.37029), in particular

* Fig. 2 caption -- one decoding round: (a) the target verifies the proposed
  tokens, (b) three fixed-size views are taken from the target's state (a
  boundary state, a recent KV window and a global context summary), (c) the
  drafter proposes the next block from those views at a cost that does not
  depend on the prefix length;
* Fig. 3 caption -- the summary is initialised over the whole prefix during
  target prefill and afterwards updated with only the newly retained KV rows
  N, with |N| <= B+1;
* Table 3 caption -- greedy decoding (T=0);
* Table 1 caption -- the accepted length tau.

The pages print no formula for the summary.  The reading used throughout is:
S slots per KV head; slot j pools the retained rows p = 0..t (t = newest
retained row) with weights

    w_jp = exp(u_j . k_p / sqrt(d)) * lambda_j ** (t - p)

(0 ** 0 = 1), holding key sum_p w_jp k_p / sum_p w_jp and value
sum_p w_jp v_p / sum_p w_jp.  It is stored as an online-softmax state
(m, l, n): a_jp = u_j . k_p / sqrt(d) + (t - p) ln(lambda_j), m_j = max_p a_jp,
l_j = sum_p exp(a_jp - m_j), n_j = sum_p exp(a_jp - m_j) [k_p ; v_p].

Everything is computed in float64 from inputs decoded exactly (bf16 -> f32
-> f64).  numpy's matmul/argmax serve as library steps; there is no blocking,
fusion or reordering beyond what the definitions state.

Parity status of each function (what pins it is in tests/test_oracle.py):
  summary_reference, summary_init, append_accepted, full_recompute,
  target_argmax, accepted_length, verify_greedy, draft_attention: pinned
  (closed forms, brute force, SDPA special cases, worked examples under
  tests/golden/).
  draft_argmax, boundary_row, verify_attention, and the S = 0 / W = 0 views:
  pinned in tests/test_oracle_next.py (brute force, SDPA with an explicit
  mask, worked examples).
  softmax_t, inverse_cdf, verify_sampling: pinned in tests/test_oracle_sampling.py
  (worked example, brute force, the sampled token distributed as the target's,
  p == q acceptance).
  Parity with the pages' own LongSpark numbers: unpinned -- the pages print
  no formula and no per-step output for this path.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "decode",
    "decay_bias",
    "summary_reference",
    "OracleState",
    "summary_init",
    "target_argmax",
    "accepted_length",
    "verify_greedy",
    "append_accepted",
    "full_recompute",
    "draft_attention",
    "draft_argmax",
    "boundary_row",
    "verify_attention",
    "softmax_t",
    "inverse_cdf",
    "verify_sampling",
]


# --------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------
def decode(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of an input array.

    ``uint16`` arrays hold bfloat16 bit patterns (the upper half of an IEEE
    binary32); ``float32``/``float64`` arrays are taken as they are.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


# --------------------------------------------------------------------------
# the summary (Fig. 3) -- plain definition
# --------------------------------------------------------------------------
def decay_bias(dist: np.ndarray, log_lambda: np.ndarray) -> np.ndarray:
    """(t - p) * ln(lambda_j), with the distance-0 term fixed at 0.

    ``dist`` [L] holds t - p >= 0, ``log_lambda`` [S].  Returns [L, S].
    lambda_j = 0 is passed as ln = -inf: its rows at distance >= 1 get -inf
    (weight 0) and the newest row gets 0 (weight lambda**0 = 1).
    """
    dist = np.asarray(dist, dtype=np.float64)[:, None]
    logl = np.asarray(log_lambda, dtype=np.float64)[None, :]
    with np.errstate(invalid="ignore"):
        prod = dist * logl
    return np.where(dist == 0.0, 0.0, prod)


def summary_reference(u, log_lambda, K, V, t=None):
    """Summary state of one (sequence, KV head) over retained rows 0..L-1.

    u [S, d], log_lambda [S], K and V [L, d] (any decodable dtype).  ``t`` is
    the position of the newest row (default L-1).  Returns m [S], l [S],
    n [S, 2d] (first d columns pool keys, last d pool values), in float64.
    """
    u = decode(u)
    K = decode(K)
    V = decode(V)
    L, d = K.shape
    if t is None:
        t = L - 1
    s = K @ u.T / np.sqrt(d)                      # [L, S]  u_j . k_p / sqrt(d)
    a = s + decay_bias(t - np.arange(L), decode(np.asarray(log_lambda)))
    m = a.max(axis=0)                             # [S]
    w = np.exp(a - m[None, :])                    # [L, S]
    l = w.sum(axis=0)
    n = w.T @ np.concatenate([K, V], axis=1)      # [S, 2d]
    return m, l, n


# --------------------------------------------------------------------------
# state
# --------------------------------------------------------------------------
@dataclass
class OracleState:
    """Drafter context state of all C sequences (Fig. 2 (b): window + summary).

    m, l [C, Hkv, S] and n [C, Hkv, S, 2d] are float64.  The ring holds raw
    input rows (bf16 bit patterns or float32) [C, Hkv, W, d]; ring_pos [C, W]
    is the absolute position held by each ring slot (-1 = empty); seq_len [C]
    counts retained rows.
    """

    u: np.ndarray
    log_lambda: np.ndarray
    m: np.ndarray
    l: np.ndarray
    n: np.ndarray
    ring_k: np.ndarray
    ring_v: np.ndarray
    ring_pos: np.ndarray
    seq_len: np.ndarray
    extra: dict = field(default_factory=dict)

    @property
    def d(self) -> int:
        return self.ring_k.shape[-1]

    @property
    def slot_k(self) -> np.ndarray:
        return self.n[..., : self.d] / self.l[..., None]

    @property
    def slot_v(self) -> np.ndarray:
        return self.n[..., self.d:] / self.l[..., None]

    def copy(self) -> "OracleState":
        return OracleState(
            self.u, self.log_lambda, self.m.copy(), self.l.copy(), self.n.copy(),
            self.ring_k.copy(), self.ring_v.copy(), self.ring_pos.copy(),
            self.seq_len.copy(), dict(self.extra))


def summary_init(u, log_lambda, k_prefix, v_prefix, W, heads=None):
    """Prefill view (Fig. 3: the summary is initialised over the full prefix).

    u [Hkv, S, d]; log_lambda [S]; k_prefix, v_prefix [C, L0, Hkv, d];
    W = ring rows.  Returns an ``OracleState`` whose summary covers every
    prefix row, whose ring holds the last min(W, L0) rows at slot p mod W, and
    whose other ring slots are empty (position -1, zero rows).

    ``heads`` optionally restricts the summary to a list of (c, h) pairs (the
    other entries stay NaN) so that large prefixes can be sampled.
    """
    C, L0, Hkv, d = k_prefix.shape
    S = u.shape[1]
    m = np.full((C, Hkv, S), np.nan)
    l = np.full((C, Hkv, S), np.nan)
    n = np.full((C, Hkv, S, 2 * d), np.nan)
    todo = heads if heads is not None else [(c, h) for c in range(C) for h in range(Hkv)]
    for c, h in todo:
        m[c, h], l[c, h], n[c, h] = summary_reference(
            u[h], log_lambda, k_prefix[c, :, h, :], v_prefix[c, :, h, :])

    ring_k = np.zeros((C, Hkv, W, d), dtype=k_prefix.dtype)
    ring_v = np.zeros((C, Hkv, W, d), dtype=v_prefix.dtype)
    ring_pos = np.full((C, W), -1, dtype=np.int32)
    for p in range(max(0, L0 - W), L0):
        ring_k[:, :, p % W, :] = k_prefix[:, p, :, :]
        ring_v[:, :, p % W, :] = v_prefix[:, p, :, :]
        ring_pos[:, p % W] = p
    seq_len = np.full((C,), L0, dtype=np.int64)
    return OracleState(np.asarray(u), np.asarray(log_lambda), m, l, n,
                       ring_k, ring_v, ring_pos, seq_len)


# --------------------------------------------------------------------------
# greedy verification (Fig. 2 (a); Table 3, T = 0)
# --------------------------------------------------------------------------
def target_argmax(logits):
    """The target's greedy token at each verified position.

    logits [C, B+1, V] (any decodable dtype).  Returns int32 [C, B+1]:
    g_i = argmax_v logits[c, i, v], the lowest index on ties (+0 and -0 are
    equal as decoded float64 values).
    """
    x = decode(logits)
    C, B1, _ = x.shape
    target = np.zeros((C, B1), dtype=np.int32)
    for c in range(C):
        for i in range(B1):
            target[c, i] = int(np.argmax(x[c, i]))   # first occurrence of the max
    return target


def accepted_length(target, draft):
    """tau = M + 1, where M is the longest prefix with draft[c, i] == g_i.

    target [C, B+1] (the g_i), draft [C, B].  Returns tau [C] int32: the M
    accepted drafts plus the target's own token g_M are committed.
    """
    target = np.asarray(target)
    draft = np.asarray(draft)
    C, B1 = target.shape
    B = B1 - 1
    tau = np.zeros((C,), dtype=np.int32)
    for c in range(C):
        M = 0
        while M < B and int(draft[c, M]) == int(target[c, M]):
            M += 1
        tau[c] = M + 1
    return tau


def verify_greedy(logits, draft):
    """Greedy acceptance of a drafted block.

    logits [C, B+1, V]: the target's scores at the B+1 verified positions
    (the last committed token, then drafts 1..B).  draft [C, B]: the drafted
    tokens.  g_i = argmax_v logits[c, i, v] (lowest index on ties); M is the
    longest prefix with draft[c, i] == g_i; tau = M + 1 tokens are committed
    (the M accepted drafts plus the target's own token g_M).

    Returns target_tok [C, B+1] int32 (all g_i) and tau [C] int32.
    """
    target = target_argmax(logits)
    return target, accepted_length(target, draft)


# --------------------------------------------------------------------------
# per-round update: ring window + incremental summary (Fig. 2 (b), Fig. 3)
# --------------------------------------------------------------------------
def append_accepted(state: OracleState, k_new, v_new, tau, heads=None) -> OracleState:
    """Append the tau[c] newly retained rows of each sequence, in place.

    k_new, v_new [C, B+1, Hkv, d]: KV rows of the verified positions; the
    first tau[c] of them are retained (Fig. 3: |N| <= B+1).  The summary is
    updated from those rows only: relative to the new newest position
    t' = t + tau, every old a_jp grows by tau * ln(lambda_j), which moves m
    and leaves l, n unchanged; the new rows are then merged by the online
    softmax rule.  ``heads`` restricts the summary update to (c, h) pairs.
    """
    C, B1, Hkv, d = k_new.shape
    W = state.ring_k.shape[2]
    u = decode(state.u)
    logl = decode(np.asarray(state.log_lambda))
    tau = np.asarray(tau).astype(np.int64)
    if np.any(tau < 1) or np.any(tau > B1):
        raise ValueError("tau must lie in [1, B+1]")
    todo = heads if heads is not None else [(c, h) for c in range(C) for h in range(Hkv)]
    for c, h in todo:
        T = int(tau[c])
        L = int(state.seq_len[c])
        kk = decode(k_new[c, :T, h, :])            # [T, d]
        vv = decode(v_new[c, :T, h, :])
        with np.errstate(invalid="ignore"):
            m_shift = state.m[c, h] + T * logl     # -inf where lambda = 0
        dist = (L + T - 1) - (L + np.arange(T))    # t' - p for the new rows
        a = kk @ u[h].T / np.sqrt(d) + decay_bias(dist, logl)       # [T, S]
        m_star = np.maximum(m_shift, a.max(axis=0))
        old_scale = np.where(np.isneginf(m_shift), 0.0,
                             np.exp(np.where(np.isneginf(m_shift), 0.0, m_shift - m_star)))
        w = np.exp(a - m_star[None, :])            # [T, S]
        state.l[c, h] = state.l[c, h] * old_scale + w.sum(axis=0)
        state.n[c, h] = (state.n[c, h] * old_scale[:, None]
                         + w.T @ np.concatenate([kk, vv], axis=1))
        state.m[c, h] = m_star
    for c in range(C):
        T = int(tau[c])
        L = int(state.seq_len[c])
        for i in range(T if W > 0 else 0):         # W = 0: no window view
            state.ring_k[c, :, (L + i) % W, :] = k_new[c, i, :, :]
            state.ring_v[c, :, (L + i) % W, :] = v_new[c, i, :, :]
            state.ring_pos[c, (L + i) % W] = L + i
        state.seq_len[c] = L + T
    return state


def full_recompute(u, log_lambda, K_rows, V_rows):
    """Summary over every retained row, recomputed from scratch (test aid).

    K_rows, V_rows [L, d] for one (c, h).  Equal to summary_reference; kept as
    its own name so tests read as 'incremental == full recompute'.
    """
    return summary_reference(u, log_lambda, K_rows, V_rows)


# --------------------------------------------------------------------------
# drafter block attention (Fig. 2 (c))
# --------------------------------------------------------------------------
def draft_attention(state: OracleState, q, k_blk, v_blk, pairs=None):
    """Bidirectional GQA attention of the drafted block over the three views.

    q [C, B, Hq, d]; k_blk, v_blk [C, B, Hkv, d].  Query head hq reads KV head
    hq // (Hq / Hkv).  Its keys/values are the occupied ring rows, the S
    summary slots (pooled key, pooled value) and the B block rows; softmax
    scale 1/sqrt(d); no mask inside the block.  Returns out [C, B, Hq, d]
    float64.  ``pairs`` restricts the work to (c, hq) pairs (others NaN).
    """
    C, B, Hq, d = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    qq = decode(q)
    kb = decode(k_blk)
    vb = decode(v_blk)
    out = np.full((C, B, Hq, d), np.nan)
    slot_k = state.slot_k
    slot_v = state.slot_v
    todo = pairs if pairs is not None else [(c, hq) for c in range(C) for hq in range(Hq)]
    for c, hq in todo:
        h = hq // G
        valid = state.ring_pos[c] >= 0
        keys = np.concatenate([decode(state.ring_k[c, h][valid]), slot_k[c, h], kb[c, :, h, :]])
        vals = np.concatenate([decode(state.ring_v[c, h][valid]), slot_v[c, h], vb[c, :, h, :]])
        s = qq[c, :, hq, :] @ keys.T / np.sqrt(d)  # [B, nkeys]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[c, :, hq, :] = p @ vals
    return out


# --------------------------------------------------------------------------
# drafter proposal at T = 0 (Fig. 1 caption: drafting time counts the
# proposal and sampling of the drafted tokens; Table 3: greedy decoding)
# --------------------------------------------------------------------------
def draft_argmax(logits):
    """Greedy proposal of the drafted block.

    logits [C, B, V]: the drafter's scores at the B block positions.  Returns
    int32 [C, B]: the argmax over V of each row, lowest index on ties (+0 and
    -0 compare equal, as the decoded float64 values do).
    """
    x = decode(logits)
    return np.argmax(x, axis=-1).astype(np.int32)   # first occurrence of the max


# --------------------------------------------------------------------------
# boundary state view (Fig. 2 (b))
# --------------------------------------------------------------------------
def boundary_row(hidden, tau):
    """The target state at the accepted boundary.

    hidden [C, B+1, H]: the target's states at the B+1 verified positions.
    After verification tau[c] of them are committed; the boundary is the
    newest committed position, row tau[c] - 1 of the block.  Returns the raw
    rows [C, H] (a copy: same dtype, same bits).
    """
    hidden = np.asarray(hidden)
    tau = np.asarray(tau).astype(np.int64)
    C, B1 = hidden.shape[:2]
    if np.any(tau < 1) or np.any(tau > B1):
        raise ValueError("tau must lie in [1, B+1]")
    out = np.empty((C,) + hidden.shape[2:], dtype=hidden.dtype)
    for c in range(C):
        out[c] = hidden[c, tau[c] - 1]
    return out


# --------------------------------------------------------------------------
# target-side verification attention (Fig. 2 (a)): the prefix-dependent cost
# the drafter avoids
# --------------------------------------------------------------------------
def verify_attention(k_cache, v_cache, q, L, pairs=None):
    """Causal GQA attention of the B+1 verified positions over the whole context.

    k_cache, v_cache [C, R, Hkv, d]: the target's KV rows of one layer; rows
    0..L[c]-1 are the context before the block and rows L[c]..L[c]+B hold the
    B+1 verified positions.  q [C, B+1, Hq, d]: their queries.  Query i (at
    position L[c] + i) attends to rows 0..L[c]+i; query head hq reads KV head
    hq // (Hq / Hkv); scale 1/sqrt(d).  Returns float64 [C, B+1, Hq, d].
    ``pairs`` restricts the work to (c, hq) pairs (others NaN).
    """
    C, B1, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    L = np.asarray(L).astype(np.int64)
    qq = decode(q)
    out = np.full((C, B1, Hq, d), np.nan)
    todo = pairs if pairs is not None else [(c, hq) for c in range(C) for hq in range(Hq)]
    for c, hq in todo:
        h = hq // G
        n = int(L[c]) + B1
        keys = decode(k_cache[c, :n, h, :])          # [n, d]
        vals = decode(v_cache[c, :n, h, :])
        s = qq[c, :, hq, :] @ keys.T / np.sqrt(d)    # [B+1, n]
        visible = np.arange(n)[None, :] <= (int(L[c]) + np.arange(B1))[:, None]
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[c, :, hq, :] = p @ vals
    return out


# --------------------------------------------------------------------------
# sampled verification (Table 1 reports accepted lengths at temperature 1,
# Table 3 separately for greedy decoding; the rule itself is not printed on
# the pages: this is the textbook speculative-sampling rule)
# --------------------------------------------------------------------------
def softmax_t(logits, temperature):
    """Row-wise softmax of decoded logits / temperature (float64), temperature > 0."""
    x = decode(logits) / float(temperature)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def inverse_cdf(w, u):
    """Draw from unnormalised weights w >= 0 with a uniform u in [0, 1): the
    smallest index k whose running sum w_0 + ... + w_k exceeds u * sum(w)."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return int(np.searchsorted(c, u * c[-1], side="right"))


def verify_sampling(target_logits, draft_logits, draft, temperature, u_accept, u_sample):
    """Speculative-sampling verification of a drafted block.

    target_logits [C, B+1, V]: the target's scores at the B+1 verified
    positions; row j predicts the token after position j.  draft_logits
    [C, B, V]: the drafter's scores for the same B predictions; draft [C, B]
    its sampled tokens.  p_j = softmax(target row j / T), q_j = softmax(draft
    row j / T).  Draft j is accepted when u_accept[c, j] * q_j(d) < p_j(d),
    i.e. with probability min(1, p/q); at the first rejection the emitted
    token is drawn from max(0, p_j - q_j) with u_sample[c] (inverse_cdf), or
    from p_j when that residual is zero everywhere (p_j == q_j, reachable only
    when the drafted token has p = q = 0); if all B drafts are accepted the
    extra token is drawn from p_B.

    Returns tokens [C, B+1] int32 (the first tau[c] are emitted, the rest -1)
    and tau [C] int32 in [1, B+1].
    """
    p = softmax_t(target_logits, temperature)
    q = softmax_t(draft_logits, temperature)
    draft = np.asarray(draft)
    u_accept = np.asarray(u_accept, dtype=np.float64)
    u_sample = np.asarray(u_sample, dtype=np.float64)
    C, B1, _ = p.shape
    B = B1 - 1
    tokens = np.full((C, B1), -1, dtype=np.int32)
    tau = np.zeros((C,), dtype=np.int32)
    for c in range(C):
        j = 0
        while j < B:
            d = int(draft[c, j])
            if u_accept[c, j] * q[c, j, d] < p[c, j, d]:
                tokens[c, j] = d
                j += 1
            else:
                break
        w = np.maximum(p[c, j] - q[c, j], 0.0) if j < B else p[c, B]
        if not np.any(w > 0.0):
            # a rejection with p_j == q_j (the drafted token has p = q = 0):
            # the residual is empty, so the token is drawn from p_j itself
            w = p[c, j]
        tokens[c, j] = inverse_cdf(w, u_sample[c])
        tau[c] = j + 1
    return tokens, tau
