"""C ABI checks that need no GPU: symbols, version, sizes, validation errors.

No call here reaches a kernel launch: every case fails validation or is an
empty problem, which returns before touching the device.
"""

import ctypes
import os
import re

import pytest

import rwkv_wkv7_delta_amd as wk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wk.LIB_PATH):
        pytest.skip("libwkv7.so not built")
    return wk.lib()


def _declared():
    with open(os.path.join(ROOT, "include", "wkv7.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wkv7_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(wk.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.wkv7_abi_version() == 1
    for s in range(6):
        assert len(L.wkv7_status_string(s)) > 0
    assert L.wkv7_status_string(99) == b"unknown status"


def test_tape_and_workspace_sizes(L):
    d = wk.make_desc(8, 4096, 40, 64, wk.WKV7_BF16, 16)
    tape = 8 * 4096 * 40 * 64 * 2 + 8 * 40 * 128 * 64 * 64 * 2   # states every 32 tokens
    assert wk.tape_bytes(d) == tape
    assert wk.workspace_bytes(d, True) == tape + 256      # + the per-key pass's work queues
    assert wk.workspace_bytes(d, False) == 2 * tape + 256
    d = wk.make_desc(1, 65, 2, 64, wk.WKV7_F32, 0)   # 3 blocks of 32 tokens, the last ragged
    assert wk.tape_bytes(d) == 65 * 2 * 64 * 2 + 2 * 3 * 64 * 64 * 2
    assert wk.tape_bytes(wk.make_desc(3, 0, 2, 64, wk.WKV7_BF16, 16)) == 0
    assert wk.tape_bytes(wk.make_desc(1, 64, 1, 48, wk.WKV7_F32, 0)) == 0   # invalid N
    # N = 32: the scan writes a tape of the same layout; the sequential reverse
    # pass's workspace holds fp32 states every 16 tokens; the chunked form
    # (N = 64 only) has no size.
    assert wk.tape_bytes(wk.make_desc(1, 64, 1, 32, wk.WKV7_F32, 0)) == 64 * 32 * 2 + 2 * 32 * 32 * 2
    assert wk.workspace_bytes(wk.make_desc(1, 64, 1, 32, wk.WKV7_F32, 0), False) == 4 * 32 * 32 * 4
    assert wk.workspace_bytes(wk.make_desc(1, 64, 1, 32, wk.WKV7_F32, 0), True) == 4 * 32 * 32 * 4
    # the chunked backward at N = 32: its own scratch (dX, block adjoints) and the queues
    assert wk.workspace_bytes(wk.make_desc(1, 64, 1, 32, wk.WKV7_BF16, 16), True) == \
        64 * 32 * 2 + 2 * 32 * 32 * 2 + 256
    assert wk.workspace_bytes(wk.make_desc(1, 64, 1, 128, wk.WKV7_BF16, 16), True) == 0


def test_ckpt_and_one_argument_workspace_sizes(L):
    """wkv7_ckpt_bytes: the fp32 state entering every 16 tokens, [B][H][ceil(T/16)][N][N],
    for either form; wkv7_workspace_bytes(desc): the backward's scratch when the
    caller passes nothing the forward wrote (= wkv7_backward_workspace_bytes(desc, 0))."""
    for B, T, H, N, dt, cl in ((8, 4096, 40, 64, wk.WKV7_BF16, 16), (2, 33, 3, 32, wk.WKV7_F32, 0),
                               (1, 1, 1, 128, wk.WKV7_BF16, 0), (3, 0, 2, 64, wk.WKV7_BF16, 16)):
        d = wk.make_desc(B, T, H, N, dt, cl)
        assert L.wkv7_ckpt_bytes(ctypes.byref(d)) == B * H * ((T + 15) // 16) * N * N * 4
        assert wk.ckpt_bytes(d) == L.wkv7_ckpt_bytes(ctypes.byref(d))
        assert L.wkv7_workspace_bytes(ctypes.byref(d)) == \
            L.wkv7_backward_workspace_bytes(ctypes.byref(d), 0)
    d = wk.make_desc(8, 4096, 40, 64, wk.WKV7_BF16, 16)
    assert L.wkv7_workspace_bytes(ctypes.byref(d)) == 2 * wk.tape_bytes(d) + 256
    d = wk.make_desc(2, 33, 3, 32, wk.WKV7_F32, 0)
    assert L.wkv7_workspace_bytes(ctypes.byref(d)) == wk.ckpt_bytes(d)
    for bad in (wk.make_desc(1, 8, 1, 48, wk.WKV7_BF16, 0), wk.make_desc(-1, 8, 1, 64, wk.WKV7_BF16, 0)):
        assert L.wkv7_ckpt_bytes(ctypes.byref(bad)) == 0
        assert L.wkv7_workspace_bytes(ctypes.byref(bad)) == 0
    assert L.wkv7_ckpt_bytes(None) == 0 and L.wkv7_workspace_bytes(None) == 0


def test_backward_ckpt_validation(L):
    """wkv7_backward_ckpt: the sequential reverse pass (chunk_len 0) from the
    caller's fp32 checkpoints, which are required; no workspace."""
    f = L.wkv7_backward_ckpt
    d = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 0)
    args = [FAKE] * 6 + [None, FAKE, None]
    assert f(None, *args, FAKE, *[FAKE] * 6, None, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *args, None, *[FAKE] * 6, None, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *args, FAKE + 8, *[FAKE] * 6, None, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *args, FAKE, *[FAKE] * 5, None, None, None) == wk.WKV7_ERR_INVALID_ARG
    d16 = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 16)
    assert f(ctypes.byref(d16), *args, FAKE, *[FAKE] * 6, None, None) == wk.WKV7_ERR_UNSUPPORTED
    d0 = wk.make_desc(0, 8, 1, 64, wk.WKV7_BF16, 0)
    assert f(ctypes.byref(d0), *args, None, *[FAKE] * 6, None, None) == wk.WKV7_OK


def test_forward_ckpt_validation(L):
    f = L.wkv7_forward_ckpt
    d = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 16)
    assert f(None, *[FAKE] * 6, None, FAKE, None, FAKE, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *[FAKE] * 6, None, FAKE, None, FAKE + 8, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *[FAKE] * 6, None, None, None, FAKE, None) == wk.WKV7_ERR_INVALID_ARG
    # the chunked form at N = 128 writes checkpoints too: validated like the others
    assert f(ctypes.byref(wk.make_desc(1, 8, 1, 128, wk.WKV7_BF16, 16)), *[FAKE] * 6, None, None,
             None, FAKE, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(wk.make_desc(0, 8, 1, 64, wk.WKV7_BF16, 16)), *[FAKE] * 6, None, FAKE,
             None, FAKE, None) == wk.WKV7_OK


FAKE = 1 << 20   # aligned, never dereferenced (validation fails first or nothing runs)


def _fwd(L, d, ptrs=None, y=FAKE):
    p = ptrs if ptrs is not None else [FAKE] * 6
    return L.wkv7_forward(ctypes.byref(d), *p, None, y, None, None, None)


def test_forward_validation(L):
    assert L.wkv7_forward(None, *[FAKE] * 6, None, FAKE, None, None, None) == wk.WKV7_ERR_INVALID_ARG
    assert _fwd(L, wk.make_desc(1, 8, 1, 48, wk.WKV7_BF16, 0)) == wk.WKV7_ERR_UNSUPPORTED
    # N = 128, chunked: no tape (the chunked backward runs N = 32 and 64), checked
    # before anything is launched; y is required as everywhere.
    d128 = wk.make_desc(1, 8, 1, 128, wk.WKV7_BF16, 16)
    assert L.wkv7_forward(ctypes.byref(d128), *[FAKE] * 6, None, FAKE, None, FAKE, None) == \
        wk.WKV7_ERR_UNSUPPORTED
    assert _fwd(L, d128, y=None) == wk.WKV7_ERR_INVALID_ARG
    assert wk.tape_bytes(d128) == 0
    assert _fwd(L, wk.make_desc(1, 8, 1, 32, wk.WKV7_F32, 16)) == wk.WKV7_ERR_UNSUPPORTED
    assert _fwd(L, wk.make_desc(1, 8, 1, 128, wk.WKV7_BF16, 0), y=None) == wk.WKV7_ERR_INVALID_ARG
    assert _fwd(L, wk.make_desc(0, 8, 1, 32, wk.WKV7_BF16, 0)) == wk.WKV7_OK
    assert _fwd(L, wk.make_desc(-1, 8, 1, 64, wk.WKV7_BF16, 0)) == wk.WKV7_ERR_INVALID_ARG
    assert _fwd(L, wk.make_desc(1, 8, 1, 64, 7, 0)) == wk.WKV7_ERR_UNSUPPORTED
    assert _fwd(L, wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 8)) == wk.WKV7_ERR_UNSUPPORTED
    assert _fwd(L, wk.make_desc(1, 8, 1, 64, wk.WKV7_F32, 16)) == wk.WKV7_ERR_UNSUPPORTED
    d = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 0)
    assert _fwd(L, d, ptrs=[FAKE] * 5 + [None]) == wk.WKV7_ERR_INVALID_ARG
    assert _fwd(L, d, ptrs=[FAKE] * 5 + [FAKE + 8]) == wk.WKV7_ERR_INVALID_ARG
    assert _fwd(L, d, y=None) == wk.WKV7_ERR_INVALID_ARG
    # Empty problems return OK without launching anything.
    assert _fwd(L, wk.make_desc(0, 8, 4, 64, wk.WKV7_BF16, 0)) == wk.WKV7_OK
    assert _fwd(L, wk.make_desc(2, 8, 0, 64, wk.WKV7_BF16, 16)) == wk.WKV7_OK


def test_split_workspace_sizes(L):
    """Explicit segment counts need no device: 3 states (entry, and the two map
    runs) of 64 x 64 fp32 per segment of every split head."""
    st = 64 * 64 * 4
    d = wk.make_desc(4, 1024, 12, 64, wk.WKV7_BF16, 16)
    assert wk.split_workspace_bytes(d, 4) == 48 * 3 * 4 * st
    assert wk.split_workspace_bytes(d, 1) == 0
    assert wk.split_workspace_bytes(d, 40) == 48 * 3 * 16 * st      # at most 16 segments
    assert wk.split_workspace_bytes(d, -1) == 0
    assert wk.split_workspace_bytes(d, -17) == 0
    # Sequential segments: one fp32 state per head and one int flag per head
    # (rounded up to 256 bytes), whatever the number of segments.
    assert wk.split_workspace_bytes(d, -4) == 48 * st + 256
    assert wk.split_workspace_bytes(wk.make_desc(8, 4096, 40, 64, wk.WKV7_BF16, 16), -4) == \
        320 * st + 1280
    # T = 64: four segments would start at 0, 32, 64, 96; two fit.
    assert wk.split_workspace_bytes(wk.make_desc(1, 64, 2, 64, wk.WKV7_BF16, 16), 4) == 2 * 3 * 2 * st
    assert wk.split_workspace_bytes(wk.make_desc(1, 32, 2, 64, wk.WKV7_BF16, 16), 4) == 0
    # The scan splits by maps only, at every head size.
    assert wk.split_workspace_bytes(wk.make_desc(1, 1024, 2, 64, wk.WKV7_BF16, 0), 4) == 2 * 3 * 4 * st
    assert wk.split_workspace_bytes(wk.make_desc(1, 1024, 2, 64, wk.WKV7_F32, 0), 4) == 2 * 3 * 4 * st
    assert wk.split_workspace_bytes(wk.make_desc(1, 1024, 2, 64, wk.WKV7_BF16, 0), -4) == 0
    assert wk.split_workspace_bytes(wk.make_desc(1, 1024, 2, 32, wk.WKV7_BF16, 0), 4) == 2 * 3 * 4 * st // 4
    assert wk.split_workspace_bytes(wk.make_desc(1, 1024, 2, 128, wk.WKV7_F32, 0), 4) == 2 * 3 * 4 * st * 4


def test_split_plan_query(L):
    """The plan query for explicit segment counts (no device needed) and its
    errors, which are those of wkv7_forward_split."""
    d = wk.make_desc(4, 1024, 12, 64, wk.WKV7_BF16, 16)
    p = wk.split_plan(d, 4)
    assert (p.kind, p.split_from, p.nseg, p.seg_len) == (wk.WKV7_SPLIT_MAPS, 0, 4, 256)
    p = wk.split_plan(d, 1)
    assert (p.kind, p.split_from, p.nseg, p.seg_len) == (wk.WKV7_SPLIT_NONE, 48, 1, 1024)
    p = wk.split_plan(d, -3)   # 1024 / 3 rounded up to whole 32-token blocks
    assert (p.kind, p.split_from, p.nseg, p.seg_len) == (wk.WKV7_SPLIT_SEQUENTIAL, 0, 3, 352)
    p = wk.split_plan(wk.make_desc(1, 32, 2, 64, wk.WKV7_BF16, 16), 4)   # one block: no split
    assert (p.kind, p.split_from, p.nseg) == (wk.WKV7_SPLIT_NONE, 2, 1)
    plan = wk.SplitPlan()
    assert L.wkv7_forward_split_plan(ctypes.byref(d), 4, None) == wk.WKV7_ERR_INVALID_ARG
    assert L.wkv7_forward_split_plan(ctypes.byref(d), -17, ctypes.byref(plan)) == wk.WKV7_ERR_INVALID_ARG
    assert L.wkv7_forward_split_plan(None, 4, ctypes.byref(plan)) == wk.WKV7_ERR_INVALID_ARG
    scan = wk.make_desc(1, 1024, 2, 64, wk.WKV7_BF16, 0)
    assert L.wkv7_forward_split_plan(ctypes.byref(scan), -4, ctypes.byref(plan)) == wk.WKV7_ERR_UNSUPPORTED
    bad = wk.make_desc(1, 64, 1, 48, wk.WKV7_BF16, 16)
    assert L.wkv7_forward_split_plan(ctypes.byref(bad), 4, ctypes.byref(plan)) == wk.WKV7_ERR_UNSUPPORTED


def test_split_forward_validation(L):
    d = wk.make_desc(1, 256, 1, 64, wk.WKV7_BF16, 16)
    f = L.wkv7_forward_split
    args = [FAKE] * 6 + [None, FAKE, None, None]
    assert f(ctypes.byref(d), *args, -17, None, 0, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *args, -4, None, 0, None) == wk.WKV7_ERR_WORKSPACE
    assert f(ctypes.byref(d), *args, 4, None, 0, None) == wk.WKV7_ERR_WORKSPACE
    need = wk.split_workspace_bytes(d, 4)
    assert f(ctypes.byref(d), *args, 4, FAKE, need - 16, None) == wk.WKV7_ERR_WORKSPACE
    assert f(ctypes.byref(d), *args, 4, FAKE + 8, need, None) == wk.WKV7_ERR_INVALID_ARG
    d0 = wk.make_desc(1, 256, 1, 64, wk.WKV7_BF16, 0)
    assert f(ctypes.byref(d0), *args, 4, FAKE, need - 16, None) == wk.WKV7_ERR_WORKSPACE
    assert f(ctypes.byref(d0), *args, -4, FAKE, need, None) == wk.WKV7_ERR_UNSUPPORTED
    d32 = wk.make_desc(1, 256, 1, 32, wk.WKV7_BF16, 0)
    assert f(ctypes.byref(d32), *args, 4, None, 0, None) == wk.WKV7_ERR_WORKSPACE
    assert f(ctypes.byref(d32), *args, -4, None, 0, None) == wk.WKV7_ERR_UNSUPPORTED
    assert f(None, *args, 4, FAKE, need, None) == wk.WKV7_ERR_INVALID_ARG
    de = wk.make_desc(0, 256, 1, 64, wk.WKV7_BF16, 16)
    assert f(ctypes.byref(de), *args, 4, None, 0, None) == wk.WKV7_OK


def test_split_static_validation(L):
    """wkv7_forward_split_static validates like wkv7_forward_split and refuses a
    plan that needs more than the static scratch before touching the device."""
    f = L.wkv7_forward_split_static
    args = [FAKE] * 6 + [None, FAKE, None, None]
    d = wk.make_desc(1, 256, 1, 64, wk.WKV7_BF16, 16)
    assert f(None, *args, 4, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *args, -17, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *[FAKE] * 5, FAKE + 8, None, FAKE, None, None, 4, None) == \
        wk.WKV7_ERR_INVALID_ARG
    # the chunked form at N = 128 splits by maps only
    assert f(ctypes.byref(wk.make_desc(1, 256, 1, 128, wk.WKV7_BF16, 16)), *args, -2, None) == \
        wk.WKV7_ERR_UNSUPPORTED
    big = wk.make_desc(4, 4096, 32, 64, wk.WKV7_BF16, 16)   # 128 heads x 16 segments x 3 maps
    assert wk.split_workspace_bytes(big, 16) > wk.STATIC_SCRATCH_BYTES
    assert f(ctypes.byref(big), *args, 16, None) == wk.WKV7_ERR_STATIC_SCRATCH
    assert b"static" in L.wkv7_status_string(wk.WKV7_ERR_STATIC_SCRATCH)
    assert f(ctypes.byref(wk.make_desc(0, 256, 1, 64, wk.WKV7_BF16, 16)), *args, 4, None) == wk.WKV7_OK


def test_backward_validation(L):
    d = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 16)
    args = [FAKE] * 6 + [None, FAKE, None]
    grads = [FAKE] * 6
    assert L.wkv7_backward(ctypes.byref(d), *args, None, *grads, None, None, 0, None) == \
        wk.WKV7_ERR_WORKSPACE
    assert L.wkv7_backward(ctypes.byref(d), *args, None, *grads, None, FAKE, 100, None) == \
        wk.WKV7_ERR_WORKSPACE
    assert L.wkv7_backward(ctypes.byref(d), *args, None, *[FAKE] * 5, None, None, FAKE,
                           1 << 30, None) == wk.WKV7_ERR_INVALID_ARG
    # With a tape the workspace still has to hold the backward's own scratch.
    need = wk.workspace_bytes(d, True)
    assert L.wkv7_backward(ctypes.byref(d), *args, FAKE, *grads, None, FAKE, need - 16, None) == \
        wk.WKV7_ERR_WORKSPACE
    # B*H*ceil(T/16) workgroups must fit a 32-bit grid.
    big = wk.make_desc(1 << 14, 256, 1 << 14, 64, wk.WKV7_BF16, 16)
    assert L.wkv7_backward(ctypes.byref(big), *args, FAKE, *grads, None, FAKE, 1 << 40, None) == \
        wk.WKV7_ERR_UNSUPPORTED
    # The chunked backward is bf16 at N = 32 and 64 (fp32 and N = 128 take
    # chunk_len = 0, the sequential reverse pass).
    d32 = wk.make_desc(1, 8, 1, 64, wk.WKV7_F32, 16)
    assert L.wkv7_backward(ctypes.byref(d32), *args, FAKE, *grads, None, None, 0, None) == \
        wk.WKV7_ERR_UNSUPPORTED
    for n in (48, 128):
        dn = wk.make_desc(1, 8, 1, n, wk.WKV7_BF16, 16)
        assert L.wkv7_backward(ctypes.byref(dn), *args, FAKE, *grads, None, FAKE, 1 << 30, None) == \
            wk.WKV7_ERR_UNSUPPORTED
    d0 = wk.make_desc(0, 8, 1, 64, wk.WKV7_BF16, 16)
    assert L.wkv7_backward(ctypes.byref(d0), *args, FAKE, *grads, None, None, 0, None) == wk.WKV7_OK


def test_sequential_backward_validation(L):
    """chunk_len = 0 selects the sequential reverse pass: either dtype, N = 32, 64,
    128, a workspace of fp32 states every 16 tokens, no separate stages."""
    for n, dt in ((32, wk.WKV7_F32), (64, wk.WKV7_BF16), (128, wk.WKV7_F32)):
        d = wk.make_desc(2, 33, 3, n, dt, 0)
        need = 2 * 3 * 3 * n * n * 4          # ceil(33 / 16) = 3 states per head
        assert wk.workspace_bytes(d, True) == need   # the tape is not used
        assert wk.workspace_bytes(d, False) == need
        args = [FAKE] * 6 + [None, FAKE, None]
        assert L.wkv7_backward(ctypes.byref(d), *args, None, *[FAKE] * 6, None, FAKE, need - 16,
                               None) == wk.WKV7_ERR_WORKSPACE
        for name in ("wkv7_backward_adjoint", "wkv7_backward_gradients"):
            assert getattr(L, name)(ctypes.byref(d), *args, FAKE, *[FAKE] * 6, None, FAKE, need,
                                    None) == wk.WKV7_ERR_UNSUPPORTED, name
    # The chunked backward stays bf16 at N = 64.
    assert wk.workspace_bytes(wk.make_desc(1, 64, 1, 64, wk.WKV7_F32, 16), True) == 0


def test_backward_stage_validation(L):
    """The two stage entry points validate like wkv7_backward and need a tape."""
    d = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 16)
    args = [FAKE] * 6 + [None, FAKE, None]
    grads = [FAKE] * 6
    need = wk.workspace_bytes(d, True)
    for name in ("wkv7_backward_adjoint", "wkv7_backward_gradients"):
        f = getattr(L, name)
        assert f(ctypes.byref(d), *args, None, *grads, None, FAKE, 1 << 30, None) == \
            wk.WKV7_ERR_INVALID_ARG, name
        assert f(ctypes.byref(d), *args, FAKE, *grads, None, FAKE, need - 16, None) == \
            wk.WKV7_ERR_WORKSPACE, name
        assert f(ctypes.byref(d), *args, FAKE, *[FAKE] * 5, None, None, FAKE, need, None) == \
            wk.WKV7_ERR_INVALID_ARG, name
        d32 = wk.make_desc(1, 8, 1, 64, wk.WKV7_F32, 0)   # sequential: no stages
        assert f(ctypes.byref(d32), *args, FAKE, *grads, None, FAKE, need, None) == \
            wk.WKV7_ERR_UNSUPPORTED, name
        d0 = wk.make_desc(0, 8, 1, 64, wk.WKV7_BF16, 16)
        assert f(ctypes.byref(d0), *args, None, *grads, None, None, 0, None) == wk.WKV7_OK, name


def test_backward_overlapped_validation(L):
    """wkv7_backward_overlapped validates exactly like wkv7_backward (aux stream or not)."""
    d = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 16)
    args = [FAKE] * 6 + [None, FAKE, None]
    grads = [FAKE] * 6
    f = L.wkv7_backward_overlapped
    for aux in (None, FAKE):
        assert f(ctypes.byref(d), *args, None, *grads, None, None, 0, None, aux) == wk.WKV7_ERR_WORKSPACE
        assert f(ctypes.byref(d), *args, None, *[FAKE] * 5, None, None, FAKE, 1 << 30, None, aux) == \
            wk.WKV7_ERR_INVALID_ARG
        d32 = wk.make_desc(1, 8, 1, 64, wk.WKV7_F32, 16)
        assert f(ctypes.byref(d32), *args, FAKE, *grads, None, None, 0, None, aux) == wk.WKV7_ERR_UNSUPPORTED
        # (the sequential pass without checkpoints: it needs scratch for its own)
        dseq = wk.make_desc(1, 8, 1, 64, wk.WKV7_F32, 0)
        assert f(ctypes.byref(dseq), *args, None, *grads, None, None, 0, None, aux) == wk.WKV7_ERR_WORKSPACE
        d0 = wk.make_desc(0, 8, 1, 64, wk.WKV7_BF16, 16)
        assert f(ctypes.byref(d0), *args, FAKE, *grads, None, None, 0, None, aux) == wk.WKV7_OK


def test_decode_validation(L):
    f = L.wkv7_decode_step
    assert f(1, 1, 48, wk.WKV7_BF16, *[FAKE] * 8, None) == wk.WKV7_ERR_UNSUPPORTED
    assert f(0, 1, 32, wk.WKV7_BF16, *[FAKE] * 8, None) == wk.WKV7_OK
    assert f(0, 1, 128, wk.WKV7_F32, *[FAKE] * 8, None) == wk.WKV7_OK
    assert f(1, 1, 128, wk.WKV7_BF16, *[FAKE] * 6, None, FAKE, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(-1, 1, 64, wk.WKV7_BF16, *[FAKE] * 8, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(1, 1, 64, 5, *[FAKE] * 8, None) == wk.WKV7_ERR_UNSUPPORTED
    assert f(1, 1, 64, wk.WKV7_BF16, *[FAKE] * 6, None, FAKE, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(1, 1, 64, wk.WKV7_BF16, *[FAKE] * 6, FAKE + 4, FAKE, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(0, 3, 64, wk.WKV7_BF16, *[FAKE] * 8, None) == wk.WKV7_OK


def test_removal_pair_validation(L):
    """a and b are both given or both NULL (a = b = 0); one alone is an invalid
    argument.  With both NULL the backward accepts NULL da and db; with both
    given it still requires them."""
    d = wk.make_desc(1, 8, 1, 64, wk.WKV7_BF16, 16)
    for ab in ([FAKE, None], [None, FAKE]):
        assert _fwd(L, d, ptrs=[FAKE] * 4 + ab) == wk.WKV7_ERR_INVALID_ARG
        assert L.wkv7_forward_split(ctypes.byref(d), *[FAKE] * 4, *ab, None, FAKE, None, None,
                                    1, None, 0, None) == wk.WKV7_ERR_INVALID_ARG
        assert L.wkv7_decode_step(1, 1, 64, wk.WKV7_BF16, *[FAKE] * 4, *ab, FAKE, FAKE, None) == \
            wk.WKV7_ERR_INVALID_ARG
        assert L.wkv7_backward(ctypes.byref(d), *[FAKE] * 4, *ab, None, FAKE, None, None,
                               *[FAKE] * 6, None, FAKE, 1 << 30, None) == wk.WKV7_ERR_INVALID_ARG
    # Both NULL: validation passes up to the workspace check (nothing is launched).
    assert L.wkv7_backward(ctypes.byref(d), *[FAKE] * 4, None, None, None, FAKE, None, None,
                           *[FAKE] * 4, None, None, None, None, 0, None) == wk.WKV7_ERR_WORKSPACE
    assert L.wkv7_backward(ctypes.byref(d), *[FAKE] * 4, None, None, None, FAKE, None, None,
                           *[FAKE] * 4, FAKE + 8, None, None, None, 0, None) == wk.WKV7_ERR_INVALID_ARG
    # Both given: da and db are required.
    assert L.wkv7_backward(ctypes.byref(d), *[FAKE] * 6, None, FAKE, None, None,
                           *[FAKE] * 4, None, None, None, FAKE, 1 << 30, None) == wk.WKV7_ERR_INVALID_ARG
    # Empty problems stay valid with a = b = NULL.
    assert _fwd(L, wk.make_desc(0, 8, 4, 64, wk.WKV7_BF16, 16), ptrs=[FAKE] * 4 + [None, None]) == wk.WKV7_OK


def test_epilogue_validation(L):
    """wkv7_epilogue: settings, pointers and shapes are checked before any launch."""
    f = L.wkv7_epilogue
    P = wk.EpilogueParams
    ok = P(None, None, None, 1e-5, wk.EPI_NORM_TERM)
    d = wk.make_desc(2, 8, 3, 64, wk.WKV7_BF16, 16)
    toks = [FAKE] * 4   # y, r, k, v
    assert f(ctypes.byref(d), *toks, None, None, FAKE, None) == wk.WKV7_ERR_INVALID_ARG  # params
    for bad in (P(None, None, None, 1e-5, 3), P(None, None, None, 1e-5, -1),
                P(None, None, None, -1e-5, 1), P(None, None, None, float("nan"), 1),
                P(None, None, None, float("inf"), 1), P(FAKE + 4, None, None, 1e-5, 1),
                P(None, FAKE + 8, None, 1e-5, 1), P(None, None, FAKE + 2, 1e-5, 1)):
        assert f(ctypes.byref(d), *toks, None, ctypes.byref(bad), FAKE, None) == \
            wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), None, *toks[1:], None, ctypes.byref(ok), FAKE, None) == \
        wk.WKV7_ERR_INVALID_ARG   # y
    assert f(ctypes.byref(d), *toks, None, ctypes.byref(ok), None, None) == \
        wk.WKV7_ERR_INVALID_ARG   # out
    assert f(ctypes.byref(d), *toks, FAKE + 8, ctypes.byref(ok), FAKE, None) == \
        wk.WKV7_ERR_INVALID_ARG   # misaligned gate
    with_u = P(FAKE, None, None, 1e-5, 1)
    for i in range(1, 4):   # the term reads r, k and v
        args = list(toks)
        args[i] = None
        assert f(ctypes.byref(d), *args, None, ctypes.byref(with_u), FAKE, None) == \
            wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(wk.make_desc(2, 8, 3, 48, wk.WKV7_BF16, 0)), *toks, None,
             ctypes.byref(ok), FAKE, None) == wk.WKV7_ERR_UNSUPPORTED
    assert f(ctypes.byref(wk.make_desc(2, 8, 3, 64, 7, 0)), *toks, None, ctypes.byref(ok), FAKE,
             None) == wk.WKV7_ERR_UNSUPPORTED
    assert f(None, *toks, None, ctypes.byref(ok), FAKE, None) == wk.WKV7_ERR_INVALID_ARG
    # empty problems: nothing to do, no pointer needed
    for e in (wk.make_desc(0, 8, 3, 64, wk.WKV7_F32, 0), wk.make_desc(2, 0, 3, 128, wk.WKV7_BF16, 0)):
        assert f(ctypes.byref(e), None, None, None, None, None, ctypes.byref(ok), None, None) == \
            wk.WKV7_OK


def test_forward_epilogue_validation(L):
    f = L.wkv7_forward_epilogue
    ok = wk.EpilogueParams(None, None, None, 1e-5, wk.EPI_NORM_TERM)
    ins = [FAKE] * 6 + [None]   # r, w, k, v, a, b, s0
    d = wk.make_desc(1, 32, 2, 64, wk.WKV7_BF16, 16)
    assert f(ctypes.byref(d), *ins, None, None, FAKE, None, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(d), *ins, None, ctypes.byref(ok), None, None, None) == \
        wk.WKV7_ERR_INVALID_ARG   # out
    assert f(ctypes.byref(d), *[FAKE] * 4, FAKE, None, None, None, ctypes.byref(ok), FAKE, None,
             None) == wk.WKV7_ERR_INVALID_ARG   # a without b
    assert f(ctypes.byref(d), *ins, None, ctypes.byref(wk.EpilogueParams(None, None, None, 0.0, 9)),
             FAKE, None, None) == wk.WKV7_ERR_INVALID_ARG
    assert f(ctypes.byref(wk.make_desc(1, 32, 2, 64, wk.WKV7_F32, 16)), *ins, None,
             ctypes.byref(ok), FAKE, None, None) == wk.WKV7_ERR_UNSUPPORTED
    assert f(ctypes.byref(wk.make_desc(1, 32, 2, 128, wk.WKV7_BF16, 16)), *ins, None,
             ctypes.byref(ok), None, None, None) == wk.WKV7_ERR_INVALID_ARG   # out, at N = 128 too
    assert f(ctypes.byref(d), *ins[:6], FAKE + 4, None, ctypes.byref(ok), FAKE, None, None) == \
        wk.WKV7_ERR_INVALID_ARG   # misaligned s0
    assert f(ctypes.byref(wk.make_desc(0, 32, 2, 64, wk.WKV7_BF16, 16)), *[None] * 8,
             ctypes.byref(ok), None, None, None) == wk.WKV7_OK


def test_binding_has_no_cpu_fallback():
    """The binding routes every call through libwkv7.so and never imports the oracle."""
    import inspect
    src = inspect.getsource(wk)
    assert "oracle" not in src.replace("no CPU fallback", "")
