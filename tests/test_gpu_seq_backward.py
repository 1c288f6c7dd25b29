"""GPU parity of the sequential reverse pass (wkv7_backward with chunk_len = 0).

The adjoint recurrence runs token by token in fp32 on the vector ALU, one
workgroup per head, from fp32 states the sequential forward writes every 16
tokens; it takes fp32 and bf16 inputs and head sizes 32, 64 and 128.  Each test
calls the HIP library through the C ABI and compares every gradient with the
fp64 oracle's reverse-mode gradients (pinned to finite differences and closed
forms on the CPU).  Tolerances: fp32 inputs max relative error <= 1e-4; bf16
inputs <= 2e-2 and cosine >= 0.9999.
"""

import numpy as np
import pytest

import oracle
from rwkv_wkv7_delta_amd import synth
from tests._util import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

NAMES = ("dr", "dw", "dk", "dv", "da", "db", "ds0")


@pytest.fixture(scope="module")
def wk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rwkv_wkv7_delta_amd as wk
    wk.lib()
    return wk


def _grads(wk, inp, dsT=None, ab=True):
    import torch
    dt = inp.dtype
    dev = [to_dev(x, dt) for x in (inp.r, inp.w, inp.k, inp.v)]
    dev += [to_dev(x, dt) for x in (inp.a, inp.b)] if ab else [None, None]
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    dsT_d = to_dev(dsT, "fp32") if dsT is not None else None
    g = wk.backward(*dev, to_dev(inp.dy, dt), s0, dsT_d, None, chunk_len=0)
    torch.cuda.synchronize()
    return [to_np(x) if x is not None else None for x in g]


def _check(wk, inp, what, dsT=None, ab=True):
    if not ab:
        inp.a = np.zeros_like(inp.a)
        inp.b = np.zeros_like(inp.b)
    got = _grads(wk, inp, dsT, ab)
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy, dsT)
    for name, x, rr in zip(NAMES, got, ref):
        if x is None:
            assert not ab and name in ("da", "db")
            continue
        assert_close(x, rr, inp.dtype, f"{what} {name}")


@pytest.mark.parametrize("N", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 16, 17, 70])
def test_seq_bwd(wk, N, dtype, T):
    inp = synth.generate(2, T, 3, N, dtype=dtype, seed=500 + T + N, random_s0=True, backward=True)
    dsT = (0.1 * np.random.default_rng(T + N).standard_normal(inp.s0.shape)).astype(np.float32)
    _check(wk, inp, f"seq bwd N={N} {dtype} T={T}", dsT)


@pytest.mark.parametrize("N", [32, 64, 128])
def test_seq_bwd_decay_only(wk, N):
    inp = synth.generate(2, 50, 3, N, dtype="fp32", seed=520 + N, random_s0=True, backward=True)
    _check(wk, inp, f"seq bwd a=b=0 N={N}", ab=False)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_seq_bwd_n128_both_layouts(wk, dtype):
    """N = 128: with at most half as many heads as compute units each head's rows
    run over two workgroups (each adds its rows' share of the per-key sums to
    outputs cleared first: fp32 atomics, or packed bf16 ones); with more heads,
    over one.  Sampled heads of both against the oracle."""
    ncu = __import__("torch").cuda.get_device_properties(0).multi_processor_count
    H = ncu // 2
    inp = synth.generate(1, 45, H, 128, dtype=dtype, seed=560, random_s0=True, backward=True)
    dsT = (0.1 * np.random.default_rng(561).standard_normal(inp.s0.shape)).astype(np.float32)
    g = _grads(wk, inp, dsT)
    pairs = [(0, 0), (0, 1), (0, H // 2), (0, H - 1)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    ref = oracle.backward(*sel, oracle.select_heads(inp.s0, pairs, state=True),
                          oracle.select_heads(inp.dy, pairs), oracle.select_heads(dsT, pairs, state=True))
    for name, x, rr in zip(NAMES, g, ref):
        assert_close(oracle.select_heads(x, pairs, state=name == "ds0"), rr, dtype, f"two workgroups {name}")
    H = ncu // 2 + 1
    inp = synth.generate(1, 40, H, 128, dtype=dtype, seed=562, random_s0=True, backward=True)
    g = _grads(wk, inp)
    pairs = [(0, 0), (0, H // 3), (0, H - 1)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    ref = oracle.backward(*sel, oracle.select_heads(inp.s0, pairs, state=True),
                          oracle.select_heads(inp.dy, pairs))
    for name, x, rr in zip(NAMES, g, ref):
        assert_close(oracle.select_heads(x, pairs, state=name == "ds0"), rr, dtype, f"one workgroup {name}")


def test_seq_bwd_fp32_small_workload(wk):
    """B=1, T=64, H=2, fp32, zero initial state, no dsT: the small fp32 workload."""
    inp = synth.generate(1, 64, 2, 64, dtype="fp32", seed=0, backward=True)
    _check(wk, inp, "seq bwd fp32 small")


def test_seq_bwd_0_19b_shape(wk):
    """B=4, T=1024, H=12, bf16, zero state: all 48 heads against the oracle."""
    inp = synth.generate(4, 1024, 12, 64, dtype="bf16", seed=0, backward=True)
    _check(wk, inp, "seq bwd 0.19b")


def test_seq_and_chunked_backward_agree(wk):
    """bf16 at N = 64: the sequential and the chunked backward, both against the oracle."""
    import torch
    inp = synth.generate(2, 100, 3, 64, dtype="bf16", seed=530, random_s0=True, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, "bf16")
    gs = wk.backward(*dev, dy, s0, None, None, chunk_len=0)
    gc = wk.backward(*dev, dy, s0, None, None, chunk_len=16)
    torch.cuda.synchronize()
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy)
    for name, xs, xc, rr in zip(NAMES, gs, gc, ref):
        assert_close(to_np(xs), rr, "bf16", f"sequential {name}")
        assert_close(to_np(xc), rr, "bf16", f"chunked {name}")


def test_seq_bwd_without_ds0(wk):
    import torch
    inp = synth.generate(1, 40, 2, 32, dtype="fp32", seed=540, random_s0=True, backward=True)
    dev = [to_dev(x, "fp32") for x in inp.tensors()]
    g = wk.backward(*dev, to_dev(inp.dy, "fp32"), to_dev(inp.s0, "fp32"), None, None,
                    chunk_len=0, want_ds0=False)
    torch.cuda.synchronize()
    assert g[6] is None
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy)
    for name, x, rr in zip(NAMES[:6], g[:6], ref[:6]):
        assert_close(to_np(x), rr, "fp32", f"no ds0 {name}")


def test_seq_bwd_2_9b_shape_sampled(wk):
    """B=8, T=4096, H=40, bf16, dy ~ N(0,1): the sequential reverse pass over the
    whole 2.9B-model shape on the GPU, the oracle on sampled heads."""
    import torch
    inp = synth.generate(8, 4096, 40, 64, dtype="bf16", seed=0, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    g = wk.backward(*dev, to_dev(inp.dy, "bf16"), None, None, None, chunk_len=0)
    torch.cuda.synchronize()
    pairs = [(0, 0), (7, 39), (3, 21)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    ref = oracle.backward(*sel, None, oracle.select_heads(inp.dy, pairs))
    for name, x, rr in zip(NAMES[:6], g[:6], ref[:6]):
        assert_close(oracle.select_heads(to_np(x), pairs), rr, "bf16", f"2.9b seq bwd {name}")
    assert_close(oracle.select_heads(to_np(g[6]), pairs, state=True), ref[6], "bf16", "2.9b seq bwd ds0")


def test_many_heads_scan_tape_and_checkpoints(wk):
    """640 heads (the scan's 4-lanes-per-row layout): the chunked backward from a tape
    the scan wrote, and the sequential reverse pass (whose scan writes the fp32
    checkpoints in that layout), both against the oracle."""
    import torch
    inp = synth.generate(16, 40, 40, 64, dtype="bf16", seed=550, random_s0=True, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, "bf16")
    _, _, tape = wk.forward(*dev, s0, chunk_len=0, want_state=False, want_tape=True)
    gc = wk.backward(*dev, dy, s0, None, tape, chunk_len=16)
    gs = wk.backward(*dev, dy, s0, None, None, chunk_len=0)
    torch.cuda.synchronize()
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy)
    for name, xc, xs, rr in zip(NAMES, gc, gs, ref):
        assert_close(to_np(xc), rr, "bf16", f"640 heads, chunked from scan tape {name}")
        assert_close(to_np(xs), rr, "bf16", f"640 heads, sequential {name}")
