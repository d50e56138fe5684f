"""Device-side driver of one drafting round (plumbing around the C ABI).

A round follows the paper page's Fig. 2: (a) greedy verification of the
drafted block, (b) append of the accepted rows to the window + incremental
summary update, (c) the drafter's block attention.  All three run on one
stream with no host synchronisation: tau goes from the verify kernel to the
append kernel in device memory.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as LB
from . import workload as WLM


class RoundBuffers:
    """Per-round device inputs and outputs of one workload."""

    def __init__(self, wl: WLM.Workload, device="cuda"):
        td = LB.torch_dtype(wl.dtype)
        self.target_tok = torch.zeros((wl.C, wl.B + 1), dtype=torch.int32, device=device)
        self.tau = torch.zeros((wl.C,), dtype=torch.int32, device=device)
        self.out = torch.zeros((wl.C, wl.B, wl.Hq, wl.d), dtype=td, device=device)


def upload_round(inputs: dict, device="cuda") -> dict:
    return {k: LB.to_device(v, device) for k, v in inputs.items()}


class PathRunner:
    """Holds the device state of one workload and runs rounds on it."""

    def __init__(self, wl: WLM.Workload, k_prefix: np.ndarray | torch.Tensor,
                 v_prefix: np.ndarray | torch.Tensor, max_L0: int | None = None,
                 device="cuda"):
        self.wl = wl
        self.device = device
        self.u = WLM.slot_queries(wl)
        self.log_lambda = WLM.log_lambda(wl)
        self.k_prefix = k_prefix if isinstance(k_prefix, torch.Tensor) else LB.to_device(k_prefix, device)
        self.v_prefix = v_prefix if isinstance(v_prefix, torch.Tensor) else LB.to_device(v_prefix, device)
        rows = self.k_prefix.shape[1]
        self.state = LB.DrafterState.for_workload(
            wl, self.u, self.log_lambda, max_L0=max_L0 or rows, device=device)
        self.buf = RoundBuffers(wl, device)

    def init(self, L0: int | None = None, stream=None):
        rows = self.k_prefix.shape[1]
        self.state.summary_init(self.k_prefix, self.v_prefix, L0 or rows, rows, stream)

    def round(self, logits: torch.Tensor, dev: dict, stream=None):
        """One drafting round in one call (ls_verify_append_draft): verification,
        update and draft attention, the update and the draft in one launch."""
        s, b = self.state, self.buf
        s.verify_append_draft(logits, dev["draft"], b.target_tok, b.tau, dev["k_new"], dev["v_new"],
                              dev["q"], dev["k_blk"], dev["v_blk"], b.out, stream)

    def round_two_calls(self, logits: torch.Tensor, dev: dict, stream=None):
        """The same round as verification + update in one call (the update derives
        tau from the verification's keys), then the draft attention."""
        s, b = self.state, self.buf
        s.verify_append(logits, dev["draft"], b.target_tok, b.tau, dev["k_new"], dev["v_new"], stream)
        s.draft_attention(dev["q"], dev["k_blk"], dev["v_blk"], b.out, stream)

    def bind_round(self, logits: torch.Tensor, dev: dict, stream=None):
        """round() with its arguments marshalled once; calling the result issues
        the round.  The tensors must stay alive while it is used."""
        s, b = self.state, self.buf
        return s.bind_verify_append_draft(logits, dev["draft"], b.target_tok, b.tau, dev["k_new"],
                                          dev["v_new"], dev["q"], dev["k_blk"], dev["v_blk"], b.out,
                                          stream)

    def round_split(self, logits: torch.Tensor, dev: dict, stream=None):
        """round() as its two launches called one by one: ls_verify_keys (the
        pass over the logits), then ls_update_draft."""
        s, b = self.state, self.buf
        s.verify_keys(logits, stream)
        s.update_draft(dev["draft"], b.target_tok, b.tau, dev["k_new"], dev["v_new"], dev["q"],
                       dev["k_blk"], dev["v_blk"], b.out, stream)

    def bind_round_split(self, logits: torch.Tensor, dev: dict, stream=None):
        """round_split() marshalled once: (key pass, update + draft) callables."""
        s, b = self.state, self.buf
        return (s.bind_verify_keys(logits, stream),
                s.bind_update_draft(dev["draft"], b.target_tok, b.tau, dev["k_new"], dev["v_new"],
                                    dev["q"], dev["k_blk"], dev["v_blk"], b.out, stream))

    def round_separate(self, logits: torch.Tensor, dev: dict, stream=None):
        """The same round through the three separate entry points."""
        s, b = self.state, self.buf
        s.verify_greedy(logits, dev["draft"], b.target_tok, b.tau, stream)
        s.append_accepted(dev["k_new"], dev["v_new"], b.tau, stream)
        s.draft_attention(dev["q"], dev["k_blk"], dev["v_blk"], b.out, stream)

    def snapshot(self) -> dict:
        """Host copy of the whole drafter state (checkpoint)."""
        s = self.state
        names = ("ring_k", "ring_v", "ring_pos", "seq_len", "sum_m", "sum_l", "sum_n",
                 "slot_k", "slot_v", "err_flag")
        return {n: LB.to_host(getattr(s, n)) for n in names}

    def restore(self, snap: dict):
        s = self.state
        for n, a in snap.items():
            getattr(s, n).copy_(LB.to_device(a, self.device))
