"""GPU parity of the sequential scan and the decode step at head sizes 32 and 128.

The head size N is a template parameter of both kernels (the state expansion
of "Millions of States: Designing a Scalable MoE Architecture with RWKV-7
Meta-learner", Abstract, grows it); the chunked form and the backward run
N = 64 only and return WKV7_ERR_UNSUPPORTED otherwise.  Each test calls the
HIP library through the C ABI and compares with the fp64 oracle (whose code
takes any N and whose pins run at N = 4 .. 7).  Tolerances: fp32 inputs max
relative error <= 1e-4; bf16 inputs <= 2e-2 and cosine >= 0.9999.
"""

import numpy as np
import pytest

import oracle
from rwkv_wkv7_delta_amd import synth
from tests._util import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rwkv_wkv7_delta_amd as wk
    wk.lib()
    return wk


def _check_fwd(wk, inp, what, ab=True):
    import torch
    dev = [to_dev(x, inp.dtype) for x in (inp.r, inp.w, inp.k, inp.v)]
    ab_dev = [to_dev(x, inp.dtype) for x in (inp.a, inp.b)] if ab else [None, None]
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    y, sT, _ = wk.forward(*dev, *ab_dev, s0, chunk_len=0)
    torch.cuda.synchronize()
    a, b = (inp.a, inp.b) if ab else (np.zeros_like(inp.a), np.zeros_like(inp.b))
    yr, sr = oracle.forward(inp.r, inp.w, inp.k, inp.v, a, b, inp.s0)
    assert_close(to_np(y), yr, inp.dtype, f"{what} y")
    assert_close(to_np(sT), sr, inp.dtype, f"{what} sT")


@pytest.mark.parametrize("N", [32, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 17, 70])
def test_seq_fwd(wk, N, dtype, T):
    inp = synth.generate(2, T, 3, N, dtype=dtype, seed=400 + T + N, random_s0=True)
    _check_fwd(wk, inp, f"seq N={N} {dtype} T={T}")


@pytest.mark.parametrize("N", [32, 128])
def test_seq_fwd_many_heads_launch(wk, N):
    """B*H >= 512: the many-heads launch (4 lanes per row; N = 128: 16 lanes, two workgroups of 16 waves per head)."""
    inp = synth.generate(16, 40, 40, N, dtype="bf16", seed=410 + N, random_s0=True)
    _check_fwd(wk, inp, f"seq N={N} 640 heads")


@pytest.mark.parametrize("N", [32, 128])
def test_seq_fwd_decay_only(wk, N):
    inp = synth.generate(2, 50, 3, N, dtype="bf16", seed=420 + N, random_s0=True)
    _check_fwd(wk, inp, f"seq N={N} a=b=0", ab=False)


@pytest.mark.parametrize("N", [32, 128])
def test_empty_sequence_copies_state(wk, N):
    import torch
    s0 = torch.randn(2, 3, N, N, device="cuda")
    z = torch.empty(2, 0, 3, N, device="cuda", dtype=torch.bfloat16)
    _, sT, _ = wk.forward(z, z, z, z, z, z, s0, chunk_len=0, out=z)
    torch.cuda.synchronize()
    assert torch.equal(sT, s0)


@pytest.mark.parametrize("N", [32, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ab", [True, False])
def test_decode_steps(wk, N, dtype, ab):
    """Six decode steps on resident states against the oracle's decode."""
    import torch
    inp = synth.generate(3, 6, 5, N, dtype=dtype, seed=430 + N, random_s0=True)
    if not ab:
        inp.a = np.zeros_like(inp.a)
        inp.b = np.zeros_like(inp.b)
    state = to_dev(inp.s0, "fp32")
    ref = inp.s0.astype(np.float64)
    for t in range(6):
        sl = [np.ascontiguousarray(x[:, t]) for x in inp.tensors()]
        dev = [to_dev(x, dtype) for x in sl[:4]]
        dev += [to_dev(x, dtype) for x in sl[4:]] if ab else [None, None]
        y = wk.decode_step(*dev, state)
        torch.cuda.synchronize()
        yr, ref = oracle.decode_step(*sl, ref)
        assert_close(to_np(y), yr, dtype, f"decode N={N} {dtype} step {t} y")
    assert_close(to_np(state), ref, dtype, f"decode N={N} {dtype} state")


def test_decode_n128_many_heads(wk):
    """B=64, H=40 at N=128 (2560 heads, 167.8 MB of state): one step vs the oracle."""
    import torch
    inp = synth.generate(64, 1, 40, 128, dtype="bf16", seed=440, random_s0=True)
    sl = [np.ascontiguousarray(x[:, 0]) for x in inp.tensors()]
    state = to_dev(inp.s0, "fp32")
    y = wk.decode_step(*[to_dev(x, "bf16") for x in sl], state)
    torch.cuda.synchronize()
    yr, sr = oracle.decode_step(*sl, inp.s0)
    assert_close(to_np(y), yr, "bf16", "decode N=128 B=64 y")
    assert_close(to_np(state), sr, "bf16", "decode N=128 B=64 state")
