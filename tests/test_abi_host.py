"""Host-side checks of the C ABI (no GPU: nothing here launches a kernel).

The library must load, export every function that include/longspark.h
declares, size workspaces, and reject bad arguments with the documented
status codes before touching the device.
"""
import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "longspark.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Tests that pass never-dereferenced fake addresses run only where no GPU is
# visible: validation must reject them before any launch, and on a machine
# without a device a validation bug shows up as LS_ERR_HIP instead of a fault.
no_device = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation tests run without a GPU")


@pytest.fixture(scope="module")
def LB():
    from fixed_cost_drafter_amd import binding
    return binding


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ls_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_path_calls():
    names = _declared_functions()
    for n in ("ls_summary_init", "ls_append_accepted", "ls_draft_attention", "ls_verify_greedy"):
        assert n in names


def test_library_exports_every_declared_function(LB):
    names = _declared_functions()
    for n in names:
        assert hasattr(LB.lib(), n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LB.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ls_\w+)", out))
    assert set(names) <= exported
    assert set(LB.EXPORTS) == set(names)


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "longspark.h"\nint main(void){ls_dims d={0};(void)d;return 0;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-c", str(src), "-o", str(tmp_path / "t.o")], check=True)


def test_version_and_status_strings(LB):
    assert LB.ls_version() == 107
    assert LB.ls_status_string(0) == "ok"
    for s in range(1, 8):
        assert LB.ls_status_string(s) and LB.ls_status_string(s) != "unknown status"
    assert LB.ls_status_string(99) == "unknown status"


def _dims(LB, **kw):
    base = dict(C=16, Hq=32, Hkv=8, d=128, W=1024, S=128, B=16, V=151936, dtype="bf16")
    base.update(kw)
    return LB.make_dims(**base)


def test_workspace_bytes(LB):
    d = _dims(LB)
    small = LB.ls_workspace_bytes(d, 1024)
    big = LB.ls_workspace_bytes(d, 131072)
    assert 0 < small <= big
    # init partials dominate: splits * C*Hkv*S*(2d+2) floats
    assert big >= 4 * 16 * 8 * 128 * 258
    # monotone in the prefix bound (a call with a shorter prefix always fits)
    prev = 0
    for L in (1, 63, 64, 65, 255, 256, 257, 4096, 5000, 131072):
        w = LB.ls_workspace_bytes(d, L)
        assert w >= prev
        prev = w
    # invalid dims -> 0
    assert LB.ls_workspace_bytes(_dims(LB, Hq=30), 100) == 0


@no_device
@pytest.mark.parametrize("bad,status", [
    (dict(dtype=7), 3),
    (dict(C=0), 2), (dict(Hq=0), 2), (dict(V=0), 2), (dict(S=-1), 2), (dict(W=-32), 2),
    (dict(Hq=30), 2),                 # Hq % Hkv != 0
    (dict(B=48), 2),                  # B > 47
    (dict(W=16, B=16), 2),            # B+1 > W
    (dict(d=64), 2),                  # bf16 needs d = 128
    (dict(S=96), 2),                  # bf16 needs S in {0, 64, 128}
    (dict(W=1000), 2),                # bf16 needs W % 32 == 0
    (dict(Hq=64, Hkv=8, B=16), 2),    # B*G = 128 > 64
    (dict(dtype="f32", d=48), 2),     # f32 d not supported
    (dict(dtype="f32", d=16, S=300), 2),
    (dict(V=(1 << 20) + 1), 2),       # vocabulary above 2^20
])
def test_bad_dims_are_rejected_before_any_launch(LB, bad, status):
    d = _dims(LB, **bad)
    rc = LB.lib().ls_verify_greedy(ctypes.byref(d), 16, 16, 16, 16, 256, 1 << 30, None)
    assert rc == status
    st = LB.LsState()
    rc = LB.lib().ls_draft_attention(ctypes.byref(d), ctypes.byref(st), 16, 16, 16, 16, None)
    assert rc == status
    rc = LB.lib().ls_verify_append(ctypes.byref(d), ctypes.byref(st), 16, 16, 16, 16, 16, 16, None)
    assert rc == status


@no_device
def test_null_state_and_pointers(LB):
    d = _dims(LB)
    L = LB.lib()
    assert L.ls_summary_init(ctypes.byref(d), None, 16, 16, 100, 100, None) == 1
    assert L.ls_append_accepted(None, None, 16, 16, 16, None) == 1
    st = LB.LsState()  # all NULL
    assert L.ls_append_accepted(ctypes.byref(d), ctypes.byref(st), 16, 16, 16, None) == 1
    assert L.ls_verify_greedy(ctypes.byref(d), None, 16, 16, 16, 256, 1 << 30, None) == 1
    assert L.ls_verify_append(ctypes.byref(d), ctypes.byref(st), 16, 16, 16, 16, 16, 16, None) == 1


def _fake_state(LB, d, ws_bytes, align=16):
    # distinct, never-dereferenced addresses: validation must reject or accept
    # without touching them (no call below reaches a launch)
    p = [0x10000 * (i + 1) for i in range(13)]
    st = LB.LsState(*p, ws_bytes)
    if align != 16:
        st.ring_k = p[0] + align
    return st


@no_device
def test_shape_workspace_and_alignment_errors(LB):
    d = _dims(LB)
    L = LB.lib()
    need = LB.ls_workspace_bytes(d, 32768)
    st = _fake_state(LB, d, need)
    # L0 < 1 and stride < L0
    assert L.ls_summary_init(ctypes.byref(d), ctypes.byref(st), 16, 16, 0, 10, None) == 2
    assert L.ls_summary_init(ctypes.byref(d), ctypes.byref(st), 16, 16, 100, 99, None) == 2
    # workspace one byte short
    small = _fake_state(LB, d, need - 1)
    assert L.ls_summary_init(ctypes.byref(d), ctypes.byref(small), 16, 16, 32768, 32768,
                             None) == 4
    # misaligned ring
    bad = _fake_state(LB, d, need, align=8)
    assert L.ls_append_accepted(ctypes.byref(d), ctypes.byref(bad), 16, 16, 16, None) == 5
    # misaligned round inputs
    assert L.ls_append_accepted(ctypes.byref(d), ctypes.byref(st), 18, 16, 16, None) == 5
    assert L.ls_draft_attention(ctypes.byref(d), ctypes.byref(st), 16, 16, 16, 24, None) == 5
    # verify: workspace too small
    assert L.ls_verify_greedy(ctypes.byref(d), 16, 16, 16, 16, 256, 8, None) == 4


@no_device
def test_argmax_and_boundary_validation(LB):
    d = _dims(LB)
    L = LB.lib()
    # the drafter argmax: null pointers, workspace too small, misaligned workspace
    assert L.ls_draft_argmax(ctypes.byref(d), None, 16, 256, 1 << 30, None) == 1
    assert L.ls_draft_argmax(ctypes.byref(d), 16, None, 256, 1 << 30, None) == 1
    assert L.ls_draft_argmax(ctypes.byref(d), 16, 16, 256, 8, None) == 4
    assert L.ls_draft_argmax(ctypes.byref(d), 16, 16, 264, 1 << 30, None) == 5
    bad = LB.make_dims(1, 2, 1, 16, 16, 4, 4, 0, "f32")  # V = 0
    assert L.ls_draft_argmax(ctypes.byref(bad), 16, 16, 256, 1 << 30, None) == 2
    # the boundary gather: null pointers, H < 1
    assert L.ls_gather_boundary(ctypes.byref(d), None, 8, 16, 16, None, None) == 1
    assert L.ls_gather_boundary(ctypes.byref(d), 16, 8, None, 16, None, None) == 1
    assert L.ls_gather_boundary(ctypes.byref(d), 16, 8, 16, None, None, None) == 1
    assert L.ls_gather_boundary(ctypes.byref(d), 16, 0, 16, 16, None, None) == 2


@no_device
def test_view_ablations_accept_null_view_arrays(LB):
    """W = 0 / S = 0: the switched-off view's arrays may be NULL; the others may not."""
    L = LB.lib()
    d = _dims(LB, W=0)
    need = LB.ls_workspace_bytes(d, 1)
    p = [0x10000 * (i + 1) for i in range(13)]
    st = LB.LsState(*p, need)
    st.ring_k = st.ring_v = st.ring_pos = None
    st.u = None            # a summary array: still required with S > 0
    assert L.ls_append_accepted(ctypes.byref(d), ctypes.byref(st), 16, 16, 16, None) == 1
    d2 = _dims(LB, S=0)
    st2 = LB.LsState(*p, LB.ls_workspace_bytes(d2, 1))
    st2.sum_m = st2.sum_l = st2.sum_n = st2.slot_k = st2.slot_v = st2.u = st2.log_lambda = None
    st2.ring_pos = None    # a window array: still required with W > 0
    assert L.ls_append_accepted(ctypes.byref(d2), ctypes.byref(st2), 16, 16, 16, None) == 1


@no_device
def test_verify_attention_validation(LB):
    d = _dims(LB)
    L = LB.lib()
    ws = LB.ls_workspace_bytes(d, 1 << 17)
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("kc", 16), ("vc", 16), ("stride", 1 << 17), ("L", 16), ("max_rows", 1 << 17), ("q", 16),
        ("out", 16), ("ws", 256), ("wsb", ws), ("err", None), ("stream", None))]
    call = lambda **kw: L.ls_verify_attention(ctypes.byref(d), *args(**kw))
    assert call(kc=None) == 1 and call(L=None) == 1 and call(out=None) == 1
    assert call(max_rows=16) == 2                        # max_rows < B + 1
    assert call(stride=1000, max_rows=2000) == 2         # rows_stride < max_rows
    assert call(q=24) == 5                               # misaligned
    assert call(wsb=ws - 1) == 4 or ws == 0              # workspace too small
    wide = _dims(LB, Hq=64, Hkv=8, B=16)                 # (B+1)*G = 136 > 128 rows
    assert L.ls_verify_attention(ctypes.byref(wide), *args()) == 2


def test_key_tile_order(LB):
    """The stored key tile is a permutation that keeps 8 dimensions of a key
    together and puts each 16x16x32 A-operand load in 1 KB of consecutive
    16-byte pieces (instruction mb*4 + ks, lane kg*16 + m reads key
    8*(m//4) + 4*mb + m%4, dimensions 32*ks + 8*kg ..)."""
    import numpy as np
    o = LB.key_tile_order()
    assert sorted(o.ravel().tolist()) == list(range(32 * 128))
    assert np.all(np.diff(o.reshape(32, 16, 8), axis=-1) == 1)
    for mb in range(2):
        for ks in range(4):
            for kg in range(4):
                for m in range(16):
                    key = 8 * (m // 4) + 4 * mb + m % 4
                    assert o[key, 32 * ks + 8 * kg] == ((mb * 4 + ks) * 64 + kg * 16 + m) * 8
    # host de-tiling inverts the layout; other shapes pass through
    rng = np.random.default_rng(5)
    rows = rng.integers(0, 1 << 16, size=(2, 3, 64, 128), dtype=np.uint16)
    stored = np.empty_like(rows)
    t = stored.reshape(2, 3, 2, 32 * 128)
    t[..., o] = rows.reshape(2, 3, 2, 32, 128)
    assert np.array_equal(LB.keys_to_rows(stored), rows)
    small = rng.random((1, 2, 48, 128)).astype(np.float32)
    assert LB.keys_to_rows(small) is small
    assert not LB.key_tiled(64, 64) and LB.key_tiled(1024, 128)


def test_n_tile_order(LB):
    """The stored numerator tile is a permutation in which the summary update's
    accumulator load (entry block t, group g, lanes 32b + s: slot s, entries
    32t + 8g + 4b .. + 3) is 1 KB of consecutive 16-byte pieces."""
    import numpy as np
    o = LB.n_tile_order()
    assert sorted(o.ravel().tolist()) == list(range(32 * 256))
    assert np.all(np.diff(o.reshape(32, 64, 4), axis=-1) == 1)
    for t in range(8):
        for g in range(4):
            for lane in range(64):
                s, b = lane % 32, lane // 32
                assert o[s, 32 * t + 8 * g + 4 * b] == ((t * 4 + g) * 64 + lane) * 4
    rng = np.random.default_rng(6)
    rows = rng.random((2, 3, 64, 256)).astype(np.float32)
    stored = np.empty_like(rows)
    stored.reshape(2, 3, 2, 32 * 256)[..., o] = rows.reshape(2, 3, 2, 32, 256)
    assert np.array_equal(LB.n_to_rows(stored, "bf16"), rows)
    assert LB.n_to_rows(rows, "f32") is rows


@no_device
def test_verify_append_validation(LB):
    """The fused verification + update checks the state like ls_append_accepted and
    every per-round pointer like both calls, before any launch."""
    d = _dims(LB)
    L = LB.lib()
    st = _fake_state(LB, d, LB.ls_workspace_bytes(d, 1))
    call = lambda *a: L.ls_verify_append(ctypes.byref(d), ctypes.byref(st), *a, None)
    assert call(None, 16, 16, 16, 16, 16) == 1       # logits
    assert call(16, None, 16, 16, 16, 16) == 1       # draft
    assert call(16, 16, None, 16, 16, 16) == 1       # target_tok
    assert call(16, 16, 16, None, 16, 16) == 1       # tau
    assert call(16, 16, 16, 16, None, 16) == 1       # k_new
    assert call(16, 16, 16, 16, 16, 24) == 5         # v_new not 16-byte aligned
    small = _fake_state(LB, d, 256)
    assert L.ls_verify_append(ctypes.byref(d), ctypes.byref(small), 16, 16, 16, 16, 16, 16,
                              None) == 4             # workspace too small



@no_device
def test_round_entry_validation(LB):
    """The one-call round and its two halves check dims, state and every
    pointer they take, before any launch."""
    d = _dims(LB)
    L = LB.lib()
    st = _fake_state(LB, d, LB.ls_workspace_bytes(d, 1))
    one = lambda *a: L.ls_verify_append_draft(ctypes.byref(d), ctypes.byref(st), *a, None)
    upd = lambda *a: L.ls_update_draft(ctypes.byref(d), ctypes.byref(st), *a, None)
    ok = [16] * 10
    for i in range(10):  # logits, draft, target_tok, tau, k_new, v_new, q, k_blk, v_blk, out
        args = list(ok)
        args[i] = None
        assert one(*args) == 1, i
        if i > 0:
            assert upd(*args[1:]) == 1, i
    for i in (4, 5, 6, 7, 8, 9):  # the 16-byte rows: k_new, v_new, q, k_blk, v_blk, out
        args = list(ok)
        args[i] = 24
        assert one(*args) == 5, i
        assert upd(*args[1:]) == 5, i
    assert L.ls_verify_keys(ctypes.byref(d), ctypes.byref(st), None, None) == 1
    assert L.ls_verify_keys(None, ctypes.byref(st), 16, None) == 1
    empty = LB.LsState()
    assert L.ls_verify_keys(ctypes.byref(d), ctypes.byref(empty), 16, None) == 1
    small = _fake_state(LB, d, 256)
    assert L.ls_verify_keys(ctypes.byref(d), ctypes.byref(small), 16, None) == 4
    assert L.ls_update_draft(ctypes.byref(d), ctypes.byref(small), *ok[1:], None) == 4
    assert L.ls_verify_append_draft(ctypes.byref(d), ctypes.byref(small), *ok, None) == 4
    bad = _dims(LB, B=48)
    assert L.ls_verify_keys(ctypes.byref(bad), ctypes.byref(st), 16, None) == 2
    assert L.ls_update_draft(ctypes.byref(bad), ctypes.byref(st), *ok[1:], None) == 2


@no_device
def test_noalloc_verify_rejects_what_its_static_scratch_cannot_hold(LB):
    """ls_verify_greedy_noalloc: 65536 partial keys at most (C (B+1) ceil(V/8192));
    larger calls return LS_ERR_SCRATCH before any HIP call, bad sizes and NULL
    pointers the usual codes."""
    L = LB.lib()
    fake = 1 << 30
    big = _dims(LB, C=3500)            # 3500 * 17 rows * 19 chunks = 1.13M keys
    assert L.ls_verify_greedy_noalloc(ctypes.byref(big), fake, fake, fake, fake, None) == 7
    edge = _dims(LB, C=203)            # 203 * 17 * 19 = 65569 > 65536
    assert L.ls_verify_greedy_noalloc(ctypes.byref(edge), fake, fake, fake, fake, None) == 7
    ok = _dims(LB, C=202)              # 202 * 17 * 19 = 65246 keys: fits
    assert L.ls_verify_greedy_noalloc(ctypes.byref(ok), None, fake, fake, fake, None) == 1
    assert L.ls_verify_greedy_noalloc(ctypes.byref(_dims(LB, B=0)), fake, fake, fake, fake, None) == 2
    assert L.ls_verify_greedy_noalloc(None, fake, fake, fake, fake, None) == 1
    # in range, valid pointers, but no device here: the symbol lookup fails with LS_ERR_HIP
    assert L.ls_verify_greedy_noalloc(ctypes.byref(ok), fake, fake, fake, fake, None) == 6
