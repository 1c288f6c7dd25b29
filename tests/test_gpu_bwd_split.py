"""GPU parity of the chunked backward with its adjoint chain in time segments.

With few heads the automatic plan of wkv7_forward_split splits every head,
and the chunked backward then runs its adjoint chain the same way: the last
segment and the affine maps (P from the identity with dy = 0, H from zero) of
the middle ones, the entry adjoints composed in fp32, then the other segments.
Every gradient is compared with the fp64 oracle's on the same seeded inputs,
to the bf16 tolerance (max relative error <= 2e-2, cosine >= 0.9999).
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


def _plan(wk, B, T, H, N):
    p = wk.split_plan(wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16), 0)
    assert p.kind == wk.WKV7_SPLIT_MAPS and p.split_from == 0 and p.nseg >= 2
    return p


def _check(got, inp, dsT, what, ab=True):
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy, dsT)
    for name, x, rr in zip(NAMES, got, ref):
        if x is None:
            assert not ab and name in ("da", "db")
            continue
        assert_close(to_np(x), rr, "bf16", f"{what} {name}")


@pytest.mark.parametrize("N", [32, 64])
@pytest.mark.parametrize("T", [600, 1024])
@pytest.mark.parametrize("with_tape", [True, False])
def test_bwd_split_matches_oracle(wk, N, T, with_tape):
    import torch
    B, H = 1, 3
    p = _plan(wk, B, T, H, N)
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=900 + T + N, random_s0=True, backward=True)
    dsT = (0.1 * np.random.default_rng(T + N).standard_normal(inp.s0.shape)).astype(np.float32)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    tape = wk.forward(*dev, s0, chunk_len=16, want_tape=True)[2] if with_tape else None
    g = wk.backward(*dev, to_dev(inp.dy, "bf16"), s0, to_dev(dsT, "fp32"), tape, chunk_len=16)
    torch.cuda.synchronize()
    _check(g, inp, dsT, f"split bwd N={N} T={T} nseg={p.nseg} tape={with_tape}")


def test_bwd_split_workspace_holds_the_states(wk):
    B, T, H, N = 1, 1024, 3, 64
    p = _plan(wk, B, T, H, N)
    d = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16)
    tb = wk.tape_bytes(d)
    states = B * H * 3 * p.nseg * N * N * 4
    assert wk.workspace_bytes(d, True) == (tb + 256 + 255) // 256 * 256 + states
    assert wk.workspace_bytes(d, False) == (2 * tb + 256 + 255) // 256 * 256 + states


def test_bwd_split_decay_only_and_stages(wk):
    """a = b = 0 under the split, and the two stages called one after the other
    (the adjoint chain, then the per-key pass from its workspace)."""
    import torch
    B, T, H, N = 2, 700, 2, 64
    _plan(wk, B, T, H, N)
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=950, random_s0=True, backward=True)
    inp.a = np.zeros_like(inp.a)
    inp.b = np.zeros_like(inp.b)
    dev = [to_dev(x, "bf16") for x in (inp.r, inp.w, inp.k, inp.v)]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, "bf16")
    g = wk.backward(*dev, None, None, dy, s0, None, None, chunk_len=16)
    torch.cuda.synchronize()
    _check(g, inp, None, "split bwd a=b=0", ab=False)

    inp = synth.generate(B, T, H, N, dtype="bf16", seed=951, random_s0=True, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, "bf16")
    tape = wk.forward(*dev, s0, chunk_len=16, want_tape=True)[2]
    d = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16)
    ws = torch.empty(wk.workspace_bytes(d, True) // 4 + 64, device="cuda")
    grads = [torch.empty_like(dev[0]) for _ in range(6)]
    ds0 = torch.empty(B, H, N, N, device="cuda")
    wk.backward(*dev, dy, s0, None, tape, chunk_len=16, workspace=ws, grads=grads, ds0=ds0, stage="adjoint")
    wk.backward(*dev, dy, s0, None, tape, chunk_len=16, workspace=ws, grads=grads, ds0=ds0, stage="gradients")
    torch.cuda.synchronize()
    _check(grads + [ds0], inp, None, "split bwd stages")
