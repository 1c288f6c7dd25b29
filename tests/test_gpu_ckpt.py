"""fp32 checkpoints (wkv7_forward_ckpt) and the sequential reverse pass that
reads them (wkv7_backward_ckpt).

The checkpoints are the state entering every 16 tokens, compared with the
oracle's prefix states; the forward's y and S_T are unchanged by writing them;
the reverse pass from the scan's checkpoints equals the pass that re-runs the
scan itself bit for bit (the same kernels compute the same values), and from
the chunked form's checkpoints it meets the oracle's gradients.
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


def _prefix_states(inp, T):
    xs = inp.tensors()
    out = [inp.s0.astype(np.float64)]
    for t in range(16, T, 16):
        out.append(oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1])
    return np.stack(out, axis=2)   # [B, H, nst, N, N]


@pytest.mark.parametrize("dtype,N,chunk_len", [("fp32", 64, 0), ("bf16", 64, 0), ("fp32", 32, 0),
                                              ("bf16", 128, 0), ("bf16", 64, 16)])
def test_forward_ckpt_holds_entry_states(wk, dtype, N, chunk_len):
    import torch
    B, T, H = 2, 75, 3
    inp = synth.generate(B, T, H, N, dtype=dtype, seed=40 + N, random_s0=True)
    dev = [to_dev(x, dtype) for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    y, sT, ck = wk.forward(*dev, s0, chunk_len=chunk_len, want_ckpt=True)
    y2, sT2, _ = wk.forward(*dev, s0, chunk_len=chunk_len)
    torch.cuda.synchronize()
    assert ck.shape == (B, H, (T + 15) // 16, N, N)
    assert torch.equal(y, y2) and torch.equal(sT, sT2)
    ref = _prefix_states(inp, T)
    tol = "fp32" if dtype == "fp32" else "bf16"
    for m in range(ref.shape[2]):
        assert_close(to_np(ck[:, :, m]), ref[:, :, m], tol, f"ckpt {m}")
    if chunk_len == 0:
        # the scan hands its fp32 registers over unrounded: chunk 0 is s0 itself
        assert torch.equal(ck[:, :, 0], s0)


@pytest.mark.parametrize("dtype,N", [("fp32", 64), ("bf16", 32), ("fp32", 128)])
def test_reverse_pass_from_scan_ckpt_is_the_same_computation(wk, dtype, N):
    import torch
    inp = synth.generate(2, 70, 2, N, dtype=dtype, seed=50 + N, random_s0=True, backward=True)
    dev = [to_dev(x, dtype) for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, dtype)
    _, _, ck = wk.forward(*dev, s0, chunk_len=0, want_ckpt=True)
    g_ck = wk.backward(*dev, dy, s0, None, None, chunk_len=0, ckpt=ck)
    g_own = wk.backward(*dev, dy, s0, None, None, chunk_len=0)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, g_ck, g_own):
        assert torch.equal(a, b), name
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy)
    for name, x, rr in zip(NAMES, g_ck, ref):
        assert_close(to_np(x), rr, dtype, f"from scan ckpt {name}")


def test_reverse_pass_from_chunked_ckpt(wk):
    """The chunked form's fp32 checkpoints feed the fp32 reverse pass."""
    import torch
    inp = synth.generate(2, 200, 3, 64, dtype="bf16", seed=60, random_s0=True, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, "bf16")
    y, _, ck = wk.forward(*dev, s0, chunk_len=16, want_ckpt=True)
    g = wk.backward(*dev, dy, s0, None, None, chunk_len=0, ckpt=ck)
    torch.cuda.synchronize()
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy)
    for name, x, rr in zip(NAMES, g, ref):
        assert_close(to_np(x), rr, "bf16", f"from chunked ckpt {name}")


def test_ckpt_decay_only_and_empty(wk):
    import torch
    inp = synth.generate(1, 40, 2, 64, dtype="bf16", seed=61, random_s0=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    for cl in (0, 16):
        _, _, ck = wk.forward(dev[0], dev[1], dev[2], dev[3], None, None, s0, chunk_len=cl,
                              want_ckpt=True)
        torch.cuda.synchronize()
        z = np.zeros_like(inp.a)
        xs = (inp.r, inp.w, inp.k, inp.v, z, z)
        for m, t in enumerate((0, 16, 32)):
            ref = oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1]
            assert_close(to_np(ck[:, :, m]), ref, "bf16", f"a=b=0 L={cl} ckpt {m}")
    e = torch.zeros(1, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    _, sT, ck = wk.forward(e, e, e, e, e, e, s0, chunk_len=16, want_ckpt=True)
    torch.cuda.synchronize()
    assert ck.numel() == 0 and torch.equal(sT, s0)
