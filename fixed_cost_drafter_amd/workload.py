"""Seeded synthetic workloads for the drafting path.

This module only draws inputs.  It holds none of the path's arithmetic: it
never pools, attends, takes an argmax or merges anything.  The target's
greedy token at each verified position is *planted* (a value above every
other logit of the row), so draft tokens with a given match probability can
be drawn without looking at the logits.  Both the HIP path and the CPU
oracle read the arrays made here.

Storage dtypes: bf16 values are numpy ``uint16`` bit patterns, rounded from
float32 normals with round-to-nearest-even; f32 values are ``float32``.

Workload shapes follow the paper's settings: Qwen3-4B / Qwen3-8B shaped
attention layers (32 query heads, 8 KV heads, head dim 128), concurrency 16,
block B = 16, vocabulary 151936, prefixes of 8K / 32K / 64K / 128K rows
(LongSpark paper page, Fig. 1 and Table 2: Qwen3-8B at concurrency 16 on
32K / 64K / 128K contexts).  Values are N(0, 1): the real post-RoPE KV rows,
queries and logits of those runs are not available, and the path's cost
depends only on the shapes.
"""
from __future__ import annotations

import dataclasses
import json
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# stream identifiers inside a workload's seed tree
_U, _PREFIX, _ROUND, _LOGITS, _VQ, _SAMP, _EDGE = 0, 1, 2, 3, 4, 5, 6
LOGIT_CLIP = 4.0        # ordinary logits are clipped to [-4, 4]
LOGIT_TOP = 4.5         # the planted greedy token's logit (exact in bf16 and f32)
TIE_PROB = 0.25         # share of rows with a second, higher-index copy of the top value


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    C: int              # concurrent sequences
    Hq: int
    Hkv: int
    d: int
    L0: int             # prefix rows per sequence
    W: int              # recent-window rows
    S: int              # summary slots
    B: int              # drafted block length
    V: int              # vocabulary
    rounds: int
    p_match: float      # per-position probability that a draft token equals the target's
    seed: int
    lambdas: tuple = () # explicit decays; empty -> 1 - 2**-(j mod 16)
    logits_pool: int = 0  # 0 -> one logits tensor per round; else cycle this many

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIG_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "configs")
CONFIG_NAMES = ("tiny_f32", "q3_4b_8k", "q3_8b_32k", "q3_8b_64k", "q3_8b_128k")


def load_workload(path: str) -> Workload:
    """A workload from its JSON file: the Workload fields by name (lambdas a
    list, empty for the default decays); an "about" text is allowed."""
    with open(path) as f:
        cfg = json.load(f)
    cfg.pop("about", None)
    fields = {f.name for f in dataclasses.fields(Workload)}
    unknown = set(cfg) - fields
    if unknown:
        raise ValueError(f"{path}: unknown workload fields {sorted(unknown)}")
    cfg["lambdas"] = tuple(float(x) for x in cfg.get("lambdas", ()))
    return Workload(**cfg)


def resolve_workload(name_or_path: str) -> Workload:
    """A named workload (configs/<name>.json) or the JSON file at a path."""
    if name_or_path in WORKLOADS:
        return WORKLOADS[name_or_path]
    if os.path.isfile(name_or_path):
        return load_workload(name_or_path)
    raise KeyError(f"no workload {name_or_path!r}: not one of {sorted(WORKLOADS)} and not a file")


# the five workloads: tiny fp32; Qwen3-4B-shaped, one sequence, 8K prefix;
# Qwen3-8B-shaped at concurrency 16 with 32K, 64K and 128K prefixes
WORKLOADS = {n: load_workload(os.path.join(CONFIG_DIR, n + ".json")) for n in CONFIG_NAMES}
SWEEP_L0 = (4096, 16384, 32768, 65536, 131072)


# --------------------------------------------------------------------------
# primitives
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) -> uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) float32 draws in storage dtype."""
    return to_storage(rng.standard_normal(size=shape, dtype=np.float32), dtype)


# --------------------------------------------------------------------------
# model-side parameters
# --------------------------------------------------------------------------
def lambdas(wl: Workload) -> np.ndarray:
    """Per-slot decays: explicit, or 1 - 2**-(j mod 16) (16 scales, lambda=0 at j%16==0)."""
    if wl.lambdas:
        assert len(wl.lambdas) == wl.S
        return np.asarray(wl.lambdas, dtype=np.float64)
    j = np.arange(wl.S)
    return 1.0 - np.exp2(-(j % 16).astype(np.float64))


def log_lambda(wl: Workload) -> np.ndarray:
    """ln(lambda_j) as float32, -inf where lambda_j = 0."""
    lam = lambdas(wl)
    with np.errstate(divide="ignore"):
        return np.log(lam).astype(np.float32)


def slot_queries(wl: Workload) -> np.ndarray:
    """u [Hkv, S, d]: seeded N(0, 1) slot queries, shared by all sequences."""
    return normal(_rng(wl.seed, _U), (wl.Hkv, wl.S, wl.d), wl.dtype)


# --------------------------------------------------------------------------
# prefix
# --------------------------------------------------------------------------
def _fill_rows(out: np.ndarray, rng: np.random.Generator, dtype: str, chunk_rows: int):
    rows = out.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = normal(rng, out[r0:r1].shape, dtype)


def prefix(wl: Workload, L0: int | None = None, threads: int = 8, rows_alloc: int | None = None,
           log=None):
    """k_prefix, v_prefix [C, rows_alloc, Hkv, d] with rows 0..L0-1 drawn.

    Each (sequence, K|V) has its own stream and rows are drawn in order, so the
    first L rows of a longer prefix equal a prefix drawn with L0 = L.
    ``rows_alloc`` (>= L0) leaves room at the end of each sequence (unfilled).
    """
    L0 = wl.L0 if L0 is None else L0
    rows_alloc = L0 if rows_alloc is None else rows_alloc
    assert rows_alloc >= L0
    sd = storage_dtype(wl.dtype)
    K = np.empty((wl.C, rows_alloc, wl.Hkv, wl.d), dtype=sd)
    V = np.empty((wl.C, rows_alloc, wl.Hkv, wl.d), dtype=sd)
    jobs = []
    for c in range(wl.C):
        jobs.append((K[c, :L0], _rng(wl.seed, _PREFIX, c, 0)))
        jobs.append((V[c, :L0], _rng(wl.seed, _PREFIX, c, 1)))
    chunk = max(1, (1 << 22) // (wl.Hkv * wl.d))
    done = [0]

    def run(job):
        _fill_rows(job[0], job[1], wl.dtype, chunk)
        done[0] += 1
        if log is not None and (done[0] % max(1, len(jobs) // 4) == 0):
            log(f"prefix: {done[0]}/{len(jobs)} streams drawn")

    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, jobs))
    return K, V


# --------------------------------------------------------------------------
# per-round inputs
# --------------------------------------------------------------------------
def logits_entry(wl: Workload, k: int):
    """One logits tensor [C, B+1, V] and its planted greedy tokens [C, B+1].

    Ordinary logits are N(0, 1) clipped to [-4, 4]; the planted token of each
    row gets 4.5, so it is the row's maximum.  In about a quarter of the rows
    a second token with a higher index also gets 4.5, a tie that only the
    lowest-index rule resolves to the planted token.
    """
    rng = _rng(wl.seed, _LOGITS, k)
    shape = (wl.C, wl.B + 1, wl.V)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    np.clip(x, -LOGIT_CLIP, LOGIT_CLIP, out=x)
    g = rng.integers(0, wl.V, size=shape[:2])
    tie = rng.random(size=shape[:2]) < TIE_PROB
    off = rng.integers(0, np.iinfo(np.int64).max, size=shape[:2])
    for c in range(wl.C):
        for i in range(wl.B + 1):
            x[c, i, g[c, i]] = LOGIT_TOP
            room = wl.V - 1 - g[c, i]
            if tie[c, i] and room > 0:
                x[c, i, g[c, i] + 1 + off[c, i] % room] = LOGIT_TOP
    return to_storage(x, wl.dtype), g.astype(np.int32)


EDGE_KINDS = 8
EDGE_CHUNK = 8192       # a boundary the rows put ties across (any reduction that splits rows)


def edge_logits(wl: Workload, k: int) -> np.ndarray:
    """Logits [C, B+1, V] made of the rows on which an argmax reduction slips most easily.

    Row (c, i) is of kind (c (B+1) + i + k) mod 8:
      0  every value negative; the maximum -0.125 sits at two positions on
         either side of a multiple of 8192 (a tie across a chunk boundary);
      1  +0 and -0 only, signs drawn at random (all equal: the first wins);
      2  -inf everywhere;
      3  -inf everywhere except a -0 and a +0 at two random positions;
      4  N(0, 1) with 3.0 at 8192 m - 1, 8192 m and V - 1 (positive ties);
      5  N(0, 1) with 3.0 at V - 1 only (the ragged last chunk);
      6  N(0, 1) with 3.0 at 0 and at V - 1;
      7  the smallest positive subnormal of the storage type at a random
         position, +0 / -0 elsewhere in the first half and negative values
         in the second.
    No value is compared here: each kind is built from its description.
    """
    rng = _rng(wl.seed, _EDGE, k)
    C, B1, V = wl.C, wl.B + 1, wl.V
    x = rng.standard_normal(size=(C, B1, V), dtype=np.float32)
    np.clip(x, -LOGIT_CLIP, LOGIT_CLIP, out=x)
    tiny = np.float32(np.uint32(0x00010000).view(np.float32) if wl.dtype == "bf16"
                      else np.uint32(1).view(np.float32))
    nb = max(1, (V - 1) // EDGE_CHUNK)           # chunk boundaries inside the row
    for c in range(C):
        for i in range(B1):
            kind = (c * B1 + i + k) % EDGE_KINDS
            row = x[c, i]
            m = 1 + int(rng.integers(0, nb))
            lo, hi = min(EDGE_CHUNK * m - 1, V - 2), min(EDGE_CHUNK * m, V - 1)
            if kind == 0:
                np.negative(np.abs(row), out=row)
                row -= np.float32(0.25)
                row[lo] = row[hi] = np.float32(-0.125)
            elif kind == 1:
                row[:] = np.where(rng.random(V) < 0.5, np.float32(-0.0), np.float32(0.0))
            elif kind == 2:
                row[:] = -np.inf
            elif kind == 3:
                row[:] = -np.inf
                a, b = rng.choice(V, size=2, replace=False)
                row[a], row[b] = np.float32(-0.0), np.float32(0.0)
            elif kind == 4:
                row[lo] = row[hi] = row[V - 1] = np.float32(3.0)
            elif kind == 5:
                row[V - 1] = np.float32(3.0)
            elif kind == 6:
                row[0] = row[V - 1] = np.float32(3.0)
            else:
                half = V // 2
                row[:half] = np.where(rng.random(half) < 0.5, np.float32(-0.0), np.float32(0.0))
                np.negative(np.abs(row[half:]), out=row[half:])
                row[half:] -= np.float32(0.25)
                row[int(rng.integers(0, V))] = tiny
    return to_storage(x, wl.dtype)


def pool_size(wl: Workload) -> int:
    return wl.logits_pool if wl.logits_pool > 0 else wl.rounds


def round_inputs(wl: Workload, r: int, planted: np.ndarray):
    """Inputs of round r (except the logits, which come from the pool).

    ``planted`` [C, B+1] are the greedy tokens of the logits this round uses.
    Draft token i equals planted[:, i] with probability p_match, otherwise it
    is uniform over the other V-1 tokens.
    """
    rng = _rng(wl.seed, _ROUND, r)
    C, B, Hq, Hkv, d, V = wl.C, wl.B, wl.Hq, wl.Hkv, wl.d, wl.V
    k_new = normal(rng, (C, B + 1, Hkv, d), wl.dtype)
    v_new = normal(rng, (C, B + 1, Hkv, d), wl.dtype)
    match = rng.random(size=(C, B)) < wl.p_match
    other = rng.integers(0, V - 1, size=(C, B))
    g = planted[:, :B].astype(np.int64)
    other = other + (other >= g)
    draft = np.where(match, g, other).astype(np.int32)
    q = normal(rng, (C, B, Hq, d), wl.dtype)
    k_blk = normal(rng, (C, B, Hkv, d), wl.dtype)
    v_blk = normal(rng, (C, B, Hkv, d), wl.dtype)
    return dict(k_new=k_new, v_new=v_new, draft=draft, q=q, k_blk=k_blk, v_blk=v_blk)


def verify_queries(wl: Workload, r: int) -> np.ndarray:
    """q [C, B+1, Hq, d]: the target's queries at the B+1 verified positions of round r
    (seeded N(0, 1); the matching K/V rows are prefix rows L..L+B)."""
    return normal(_rng(wl.seed, _VQ, r), (wl.C, wl.B + 1, wl.Hq, wl.d), wl.dtype)


def sampling_inputs(wl: Workload, r: int, target_logits: np.ndarray, temperature: float = 1.0,
                    noise: float = 0.5) -> dict:
    """Inputs of sampled verification for round r, beside the target's logits [C, B+1, V].

    draft_logits [C, B, V]: target rows 0..B-1 plus N(0, noise), rounded to the
    storage dtype (a drafter close to the target); draft [C, B]: tokens drawn
    from softmax(draft_logits / T) row by row on the host (float64 inverse
    CDF); u_accept [C, B] and u_sample [C]: float32 uniforms in [0, 1).
    """
    rng = _rng(wl.seed, _SAMP, r)
    C, B = wl.C, wl.B
    base = bf16_bits_to_f32(target_logits) if wl.dtype == "bf16" else np.asarray(target_logits, np.float32)
    dl32 = base[:, :B].astype(np.float32) + (noise * rng.standard_normal((C, B, wl.V))).astype(np.float32)
    draft_logits = f32_to_bf16_bits(dl32) if wl.dtype == "bf16" else dl32
    dq = (bf16_bits_to_f32(draft_logits) if wl.dtype == "bf16" else draft_logits).astype(np.float64)
    dq = dq / temperature
    dq -= dq.max(axis=-1, keepdims=True)
    w = np.exp(dq)
    cdf = np.cumsum(w, axis=-1)
    u = rng.random((C, B))
    draft = np.empty((C, B), dtype=np.int32)
    for c in range(C):
        for j in range(B):
            draft[c, j] = min(int(np.searchsorted(cdf[c, j], u[c, j] * cdf[c, j, -1], side="right")),
                              wl.V - 1)
    u_accept = rng.random((C, B)).astype(np.float32)
    u_sample = rng.random((C,)).astype(np.float32)
    return dict(draft_logits=draft_logits, draft=draft, u_accept=u_accept, u_sample=u_sample)


def expected_tau(wl: Workload) -> float:
    """E[tau] = 1 + sum_{k=1..B} p^k for independent per-position matches."""
    return 1.0 + sum(wl.p_match ** k for k in range(1, wl.B + 1))


def state_bytes(wl: Workload) -> int:
    """Bytes of one sequence's drafter context state (ring + fp32 summary + slots)."""
    e = 2 if wl.dtype == "bf16" else 4
    ring = 2 * wl.Hkv * wl.W * wl.d * e + 4 * wl.W
    summ = wl.Hkv * wl.S * (2 * wl.d + 2) * 4
    slots = 2 * wl.Hkv * wl.S * wl.d * e
    return ring + summ + slots + 4


def describe(wl: Workload) -> dict:
    return dict(workload=wl.name, dtype=wl.dtype, C=wl.C, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d,
                L0=wl.L0, W=wl.W, S=wl.S, B=wl.B, V=wl.V, p_match=wl.p_match, seed=wl.seed)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

