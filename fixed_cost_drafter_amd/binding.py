"""ctypes binding of liblongspark.so (argument marshalling only).

The functions here carry the C ABI's names and do nothing but turn torch
tensors (device memory owned by the caller) and streams into pointers, call
the library and raise on a non-zero status.  Every step of the drafting path
runs in the library's HIP kernels; there is no fallback.  Importing this
module fails loudly when the library has not been built.

``DrafterState`` allocates the fixed-size context state with torch (device
memory and streams are torch's job here) and hands the library its pointers.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LONGSPARK_LIB selects another build of the same library (e.g. the host-side
# sanitizer build of fixed_cost_drafter_amd.sanitize)
LIB_PATH = os.environ.get("LONGSPARK_LIB") or os.path.join(_HERE, "liblongspark.so")

LS_F32, LS_BF16 = 0, 1
STATUS = {0: "LS_OK", 1: "LS_ERR_NULL", 2: "LS_ERR_SHAPE", 3: "LS_ERR_DTYPE",
          4: "LS_ERR_WORKSPACE", 5: "LS_ERR_ALIGN", 6: "LS_ERR_HIP", 7: "LS_ERR_SCRATCH"}
EXPORTS = ("ls_workspace_bytes", "ls_summary_init", "ls_verify_greedy", "ls_append_accepted",
           "ls_draft_attention", "ls_draft_argmax", "ls_gather_boundary", "ls_verify_attention",
           "ls_verify_sampling", "ls_verify_append", "ls_verify_append_draft",
           "ls_verify_keys", "ls_update_draft", "ls_verify_greedy_noalloc", "ls_status_string",
           "ls_version")


class LsDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("C", "Hq", "Hkv", "d", "W", "S", "B", "V", "dtype")]


class LsState(ctypes.Structure):
    _fields_ = [("ring_k", ctypes.c_void_p), ("ring_v", ctypes.c_void_p),
                ("ring_pos", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("sum_m", ctypes.c_void_p), ("sum_l", ctypes.c_void_p),
                ("sum_n", ctypes.c_void_p), ("slot_k", ctypes.c_void_p),
                ("slot_v", ctypes.c_void_p), ("u", ctypes.c_void_p),
                ("log_lambda", ctypes.c_void_p), ("err_flag", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class LsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} "
                         f"({_lib.ls_status_string(status).decode()})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m fixed_cost_drafter_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D, S = ctypes.POINTER(LsDims), ctypes.POINTER(LsState)
    lib.ls_workspace_bytes.argtypes = [D, I32]
    lib.ls_workspace_bytes.restype = SZ
    lib.ls_summary_init.argtypes = [D, S, P, P, I32, I64, P]
    lib.ls_verify_greedy.argtypes = [D, P, P, P, P, P, SZ, P]
    lib.ls_append_accepted.argtypes = [D, S, P, P, P, P]
    lib.ls_draft_attention.argtypes = [D, S, P, P, P, P, P]
    lib.ls_draft_argmax.argtypes = [D, P, P, P, SZ, P]
    lib.ls_gather_boundary.argtypes = [D, P, I32, P, P, P, P]
    lib.ls_verify_attention.argtypes = [D, P, P, I64, P, I32, P, P, P, SZ, P, P]
    lib.ls_verify_sampling.argtypes = [D, P, P, P, ctypes.c_float, P, P, P, P, P, SZ, P]
    lib.ls_verify_append.argtypes = [D, S, P, P, P, P, P, P, P]
    lib.ls_verify_greedy_noalloc.argtypes = [D, P, P, P, P, P]
    lib.ls_verify_append_draft.argtypes = [D, S, P, P, P, P, P, P, P, P, P, P, P]
    lib.ls_verify_keys.argtypes = [D, S, P, P]
    lib.ls_update_draft.argtypes = [D, S, P, P, P, P, P, P, P, P, P, P]
    for f in ("ls_summary_init", "ls_verify_greedy", "ls_append_accepted", "ls_draft_attention",
              "ls_draft_argmax", "ls_gather_boundary", "ls_verify_attention", "ls_verify_sampling",
              "ls_verify_append", "ls_verify_greedy_noalloc", "ls_verify_append_draft",
              "ls_verify_keys", "ls_update_draft"):
        getattr(lib, f).restype = ctypes.c_int
    lib.ls_status_string.argtypes = [ctypes.c_int]
    lib.ls_status_string.restype = ctypes.c_char_p
    lib.ls_version.argtypes = []
    lib.ls_version.restype = I32
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if not x.is_contiguous():
            raise ValueError("tensors passed to liblongspark must be contiguous")
        return x.data_ptr()
    raise TypeError(f"expected a torch tensor or a raw pointer, got {type(x)}")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise LsError(fn, status)


class BoundCall:
    """One C-ABI call with every argument already marshalled (raw pointers,
    ctypes references, the stream handle): calling it only crosses into the
    library and checks the status.  For loops that issue the same calls
    many times, e.g. a round's calls prepared before a timed region."""

    __slots__ = ("name", "fn", "args")

    def __init__(self, name: str, *args):
        self.name = name
        self.fn = getattr(_lib, name)
        self.args = args

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            raise LsError(self.name, rc)


def make_dims(C, Hq, Hkv, d, W, S, B, V, dtype) -> LsDims:
    dt = {"f32": LS_F32, "bf16": LS_BF16}.get(dtype, dtype)
    return LsDims(C, Hq, Hkv, d, W, S, B, V, dt)


def value_tile(rows: int) -> int:
    """Key-tile width of the window / slot value layout [rows/tw][d][tw]."""
    return 32 if rows % 32 == 0 else rows


def values_to_rows(a: np.ndarray) -> np.ndarray:
    """Host copy of key-tiled values [..., rows/tw, d, tw] -> [..., rows, d]."""
    *lead, nt, d, tw = a.shape
    return np.ascontiguousarray(np.swapaxes(a, -1, -2).reshape(*lead, nt * tw, d))


def key_tiled(rows: int, d: int) -> bool:
    """Window / slot keys are stored in 32-key tiles in MFMA operand order when d = 128."""
    return d == 128 and rows % 32 == 0


def key_tile_order() -> np.ndarray:
    """[32, 128]: element offset of (key, dimension) inside one stored key tile.

    Key k = 8a + 4b + r, dimension e = 32s + 8g + i go to element
    ((((b*4 + s)*4 + g)*16 + 4a + r)*8 + i.
    """
    k = np.arange(32)[:, None]
    e = np.arange(128)[None, :]
    piece = ((((k >> 2) & 1) * 4 + (e >> 5)) * 4 + ((e >> 3) & 3)) * 16 + 4 * (k >> 3) + (k & 3)
    return piece * 8 + (e & 7)


def keys_to_rows(a: np.ndarray) -> np.ndarray:
    """Host copy of stored window / slot keys [..., rows, d] -> row-major keys."""
    *lead, rows, d = a.shape
    if not key_tiled(rows, d):
        return a
    t = a.reshape(*lead, rows // 32, 32 * d)
    return np.ascontiguousarray(t[..., key_tile_order()].reshape(*lead, rows, d))


def n_tiled(dtype: str, d: int, S: int) -> bool:
    """bf16 states at d = 128 keep the summary numerators n in MFMA accumulator tiles."""
    return dtype == "bf16" and d == 128 and S % 32 == 0


def n_tile_order() -> np.ndarray:
    """[32, 256]: float offset of (slot, entry) inside one stored 32-slot tile of n.

    Entry e = 32t + 8g + 4b + r of slot s goes to float ((t*4 + g)*64 + 32b + s)*4 + r.
    """
    s = np.arange(32)[:, None]
    e = np.arange(256)[None, :]
    lane = s + 32 * ((e >> 2) & 1)
    return (((e >> 5) * 4 + ((e >> 3) & 3)) * 64 + lane) * 4 + (e & 3)


def n_to_rows(a: np.ndarray, dtype: str) -> np.ndarray:
    """Host copy of stored numerators [..., S, 2d] -> [slot][entry] order."""
    *lead, S, e2 = a.shape
    if not n_tiled(dtype, e2 // 2, S):
        return a
    t = a.reshape(*lead, S // 32, 32 * e2)
    return np.ascontiguousarray(t[..., n_tile_order()].reshape(*lead, S, e2))


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a storage array (uint16 bf16 bits or float32 / int32) to the device."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# --------------------------------------------------------------------------
# the C ABI, one wrapper per entry point
# --------------------------------------------------------------------------
def ls_workspace_bytes(dims: LsDims, max_L0: int) -> int:
    return int(_lib.ls_workspace_bytes(ctypes.byref(dims), int(max_L0)))


def ls_summary_init(dims: LsDims, state: LsState, k_prefix, v_prefix, L0: int,
                    prefix_rows_stride: int, stream=None):
    _check("ls_summary_init", _lib.ls_summary_init(
        ctypes.byref(dims), ctypes.byref(state), _ptr(k_prefix), _ptr(v_prefix), int(L0),
        int(prefix_rows_stride), _stream(stream)))


def ls_verify_greedy(dims: LsDims, logits, draft, target_tok, tau, workspace, workspace_bytes,
                     stream=None):
    _check("ls_verify_greedy", _lib.ls_verify_greedy(
        ctypes.byref(dims), _ptr(logits), _ptr(draft), _ptr(target_tok), _ptr(tau),
        _ptr(workspace), int(workspace_bytes), _stream(stream)))


def ls_verify_greedy_noalloc(dims: LsDims, logits, draft, target_tok, tau, stream=None):
    _check("ls_verify_greedy_noalloc", _lib.ls_verify_greedy_noalloc(
        ctypes.byref(dims), _ptr(logits), _ptr(draft), _ptr(target_tok), _ptr(tau),
        _stream(stream)))


def ls_append_accepted(dims: LsDims, state: LsState, k_new, v_new, tau, stream=None):
    _check("ls_append_accepted", _lib.ls_append_accepted(
        ctypes.byref(dims), ctypes.byref(state), _ptr(k_new), _ptr(v_new), _ptr(tau),
        _stream(stream)))


def ls_verify_append(dims: LsDims, state: LsState, logits, draft, target_tok, tau, k_new, v_new,
                     stream=None):
    _check("ls_verify_append", _lib.ls_verify_append(
        ctypes.byref(dims), ctypes.byref(state), _ptr(logits), _ptr(draft), _ptr(target_tok),
        _ptr(tau), _ptr(k_new), _ptr(v_new), _stream(stream)))


def ls_verify_append_draft(dims: LsDims, state: LsState, logits, draft, target_tok, tau, k_new,
                           v_new, q, k_blk, v_blk, out, stream=None):
    _check("ls_verify_append_draft", _lib.ls_verify_append_draft(
        ctypes.byref(dims), ctypes.byref(state), _ptr(logits), _ptr(draft), _ptr(target_tok),
        _ptr(tau), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(out),
        _stream(stream)))


def ls_verify_keys(dims: LsDims, state: LsState, logits, stream=None):
    _check("ls_verify_keys", _lib.ls_verify_keys(
        ctypes.byref(dims), ctypes.byref(state), _ptr(logits), _stream(stream)))


def ls_update_draft(dims: LsDims, state: LsState, draft, target_tok, tau, k_new, v_new, q, k_blk,
                    v_blk, out, stream=None):
    _check("ls_update_draft", _lib.ls_update_draft(
        ctypes.byref(dims), ctypes.byref(state), _ptr(draft), _ptr(target_tok), _ptr(tau),
        _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(out), _stream(stream)))


def ls_draft_attention(dims: LsDims, state: LsState, q, k_blk, v_blk, out, stream=None):
    _check("ls_draft_attention", _lib.ls_draft_attention(
        ctypes.byref(dims), ctypes.byref(state), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(out),
        _stream(stream)))


def ls_draft_argmax(dims: LsDims, logits, draft_tok, workspace, workspace_bytes, stream=None):
    _check("ls_draft_argmax", _lib.ls_draft_argmax(
        ctypes.byref(dims), _ptr(logits), _ptr(draft_tok), _ptr(workspace), int(workspace_bytes),
        _stream(stream)))


def ls_gather_boundary(dims: LsDims, hidden, H: int, tau, out, err_flag=None, stream=None):
    _check("ls_gather_boundary", _lib.ls_gather_boundary(
        ctypes.byref(dims), _ptr(hidden), int(H), _ptr(tau), _ptr(out), _ptr(err_flag),
        _stream(stream)))


def ls_verify_attention(dims: LsDims, k_cache, v_cache, rows_stride: int, L, max_rows: int, q, out,
                        workspace, workspace_bytes, err_flag=None, stream=None):
    _check("ls_verify_attention", _lib.ls_verify_attention(
        ctypes.byref(dims), _ptr(k_cache), _ptr(v_cache), int(rows_stride), _ptr(L), int(max_rows),
        _ptr(q), _ptr(out), _ptr(workspace), int(workspace_bytes), _ptr(err_flag), _stream(stream)))


def ls_verify_sampling(dims: LsDims, target_logits, draft_logits, draft, temperature: float,
                       u_accept, u_sample, tokens, tau, workspace, workspace_bytes, stream=None):
    _check("ls_verify_sampling", _lib.ls_verify_sampling(
        ctypes.byref(dims), _ptr(target_logits), _ptr(draft_logits), _ptr(draft),
        float(temperature), _ptr(u_accept), _ptr(u_sample), _ptr(tokens), _ptr(tau),
        _ptr(workspace), int(workspace_bytes), _stream(stream)))


def ls_status_string(status: int) -> str:
    return _lib.ls_status_string(int(status)).decode()


def ls_version() -> int:
    return int(_lib.ls_version())


# --------------------------------------------------------------------------
# device state (torch-allocated)
# --------------------------------------------------------------------------
class DrafterState:
    """The drafter's fixed-size context state plus workspace, on one device.

    ``u`` [Hkv, S, d] and ``log_lambda`` [S] are the slot parameters (storage
    arrays from numpy or tensors).  ``max_L0`` sizes the workspace for the
    longest prefix that ``summary_init`` will be called with.
    """

    def __init__(self, C, Hq, Hkv, d, W, S, B, V, dtype, u, log_lambda, max_L0,
                 device="cuda"):
        self.dtype = dtype
        self.dims = make_dims(C, Hq, Hkv, d, W, S, B, V, dtype)
        td = torch_dtype(dtype)
        z = lambda *shape, dt=td: torch.zeros(shape, dtype=dt, device=device)
        self.ring_k = z(C, Hkv, W, d)
        tw, ts = value_tile(W), value_tile(S)
        self.ring_v = z(C, Hkv, W // tw, d, tw)  # key-tiled values
        self.ring_pos = torch.full((C, W), -1, dtype=torch.int32, device=device)
        self.seq_len = z(C, dt=torch.int32)
        self.sum_m = z(C, Hkv, S, dt=torch.float32)
        self.sum_l = z(C, Hkv, S, dt=torch.float32)
        self.sum_n = z(C, Hkv, S, 2 * d, dt=torch.float32)
        self.slot_k = z(C, Hkv, S, d)
        self.slot_v = z(C, Hkv, S // ts, d, ts)  # key-tiled values
        self.u = u if isinstance(u, torch.Tensor) else to_device(u, device)
        lg = log_lambda if isinstance(log_lambda, torch.Tensor) else to_device(
            np.asarray(log_lambda, dtype=np.float32), device)
        self.log_lambda = lg.to(torch.float32).contiguous()
        self.err_flag = z(1, dt=torch.int32)
        nbytes = ls_workspace_bytes(self.dims, max_L0)
        if nbytes == 0:
            raise LsError("ls_workspace_bytes", 2)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c_state = LsState(
            _ptr(self.ring_k), _ptr(self.ring_v), _ptr(self.ring_pos), _ptr(self.seq_len),
            _ptr(self.sum_m), _ptr(self.sum_l), _ptr(self.sum_n), _ptr(self.slot_k),
            _ptr(self.slot_v), _ptr(self.u), _ptr(self.log_lambda), _ptr(self.err_flag),
            _ptr(self.workspace), nbytes)

    @classmethod
    def for_workload(cls, wl, u, log_lambda, max_L0=None, device="cuda"):
        return cls(wl.C, wl.Hq, wl.Hkv, wl.d, wl.W, wl.S, wl.B, wl.V, wl.dtype, u, log_lambda,
                   wl.L0 if max_L0 is None else max_L0, device)

    # the four calls of the path, on this state
    def summary_init(self, k_prefix, v_prefix, L0=None, prefix_rows_stride=None, stream=None):
        rows = k_prefix.shape[1]
        L0 = rows if L0 is None else L0
        ls_summary_init(self.dims, self.c_state, k_prefix, v_prefix, L0,
                        rows if prefix_rows_stride is None else prefix_rows_stride, stream)

    def verify_greedy(self, logits, draft, target_tok, tau, stream=None):
        ls_verify_greedy(self.dims, logits, draft, target_tok, tau, self.workspace,
                         self.workspace.numel(), stream)

    def append_accepted(self, k_new, v_new, tau, stream=None):
        ls_append_accepted(self.dims, self.c_state, k_new, v_new, tau, stream)

    def verify_append(self, logits, draft, target_tok, tau, k_new, v_new, stream=None):
        ls_verify_append(self.dims, self.c_state, logits, draft, target_tok, tau, k_new, v_new,
                         stream)

    def draft_attention(self, q, k_blk, v_blk, out, stream=None):
        ls_draft_attention(self.dims, self.c_state, q, k_blk, v_blk, out, stream)

    def verify_append_draft(self, logits, draft, target_tok, tau, k_new, v_new, q, k_blk, v_blk, out,
                            stream=None):
        ls_verify_append_draft(self.dims, self.c_state, logits, draft, target_tok, tau, k_new, v_new,
                               q, k_blk, v_blk, out, stream)

    def verify_keys(self, logits, stream=None):
        ls_verify_keys(self.dims, self.c_state, logits, stream)

    def update_draft(self, draft, target_tok, tau, k_new, v_new, q, k_blk, v_blk, out, stream=None):
        ls_update_draft(self.dims, self.c_state, draft, target_tok, tau, k_new, v_new, q, k_blk, v_blk,
                        out, stream)

    # the round's calls with their arguments fixed (see BoundCall)
    def bind_verify_keys(self, logits, stream=None):
        return BoundCall("ls_verify_keys", ctypes.byref(self.dims), ctypes.byref(self.c_state),
                         _ptr(logits), _stream(stream))

    def bind_update_draft(self, draft, target_tok, tau, k_new, v_new, q, k_blk, v_blk, out,
                          stream=None):
        return BoundCall("ls_update_draft", ctypes.byref(self.dims), ctypes.byref(self.c_state),
                         _ptr(draft), _ptr(target_tok), _ptr(tau), _ptr(k_new), _ptr(v_new), _ptr(q),
                         _ptr(k_blk), _ptr(v_blk), _ptr(out), _stream(stream))

    def bind_verify_append(self, logits, draft, target_tok, tau, k_new, v_new, stream=None):
        return BoundCall("ls_verify_append", ctypes.byref(self.dims), ctypes.byref(self.c_state),
                         _ptr(logits), _ptr(draft), _ptr(target_tok), _ptr(tau), _ptr(k_new),
                         _ptr(v_new), _stream(stream))

    def bind_verify_append_draft(self, logits, draft, target_tok, tau, k_new, v_new, q, k_blk, v_blk,
                                 out, stream=None):
        return BoundCall("ls_verify_append_draft", ctypes.byref(self.dims), ctypes.byref(self.c_state),
                         _ptr(logits), _ptr(draft), _ptr(target_tok), _ptr(tau), _ptr(k_new),
                         _ptr(v_new), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(out), _stream(stream))

    def bind_draft_attention(self, q, k_blk, v_blk, out, stream=None):
        return BoundCall("ls_draft_attention", ctypes.byref(self.dims), ctypes.byref(self.c_state),
                         _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(out), _stream(stream))

    def draft_argmax(self, logits, draft_tok, stream=None):
        ls_draft_argmax(self.dims, logits, draft_tok, self.workspace, self.workspace.numel(), stream)

    def gather_boundary(self, hidden, tau, out, stream=None):
        ls_gather_boundary(self.dims, hidden, hidden.shape[-1], tau, out, self.err_flag, stream)

    def verify_attention(self, k_cache, v_cache, L, max_rows, q, out, stream=None):
        """k_cache, v_cache [C, rows, Hkv, d]; L [C] int32 device; the workspace must have been
        sized for max_L0 >= max_rows - B - 1."""
        ls_verify_attention(self.dims, k_cache, v_cache, k_cache.shape[1], L, max_rows, q, out,
                            self.workspace, self.workspace.numel(), self.err_flag, stream)

    def verify_sampling(self, target_logits, draft_logits, draft, temperature, u_accept, u_sample,
                        tokens, tau, stream=None):
        ls_verify_sampling(self.dims, target_logits, draft_logits, draft, temperature, u_accept,
                           u_sample, tokens, tau, self.workspace, self.workspace.numel(), stream)

    def state_bytes(self) -> int:
        ts = (self.ring_k, self.ring_v, self.ring_pos, self.seq_len, self.sum_m, self.sum_l,
              self.sum_n, self.slot_k, self.slot_v)
        return sum(t.numel() * t.element_size() for t in ts)
