"""wkv7_forward_split_static (the entry point that allocates nothing) against
wkv7_forward_split with a workspace, through the C ABI.

Two calls in a row, the second on a smaller input (the static scratch keeps
the first call's contents), in both split modes and both forms: the results
must equal the workspace entry point's bit for bit (same kernels, same plan)
and meet the oracle at the bf16 tolerance.  A plan beyond the static scratch
is refused with WKV7_ERR_STATIC_SCRATCH, its outputs untouched.
"""

import ctypes

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


def _both(wk, inp, chunk_len, segments):
    import torch
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    ys, sTs, tapes = wk.forward(*dev, s0, chunk_len=chunk_len, want_tape=True, segments=segments,
                                static_scratch=True)
    yw, sTw, tapew = wk.forward(*dev, s0, chunk_len=chunk_len, want_tape=True, segments=segments)
    torch.cuda.synchronize()
    assert torch.equal(ys, yw) and torch.equal(sTs, sTw) and torch.equal(tapes, tapew)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(to_np(ys), yr, inp.dtype, f"static L={chunk_len} seg={segments} y")
    assert_close(to_np(sTs), sr, inp.dtype, f"static L={chunk_len} seg={segments} sT")


@pytest.mark.parametrize("chunk_len,segments", [(16, 4), (16, -3), (0, 4)])
def test_static_scratch_matches_workspace_entry(wk, chunk_len, segments):
    big = synth.generate(4, 1024, 12, 64, dtype="bf16", seed=90, random_s0=True)
    small = synth.generate(1, 300, 3, 64, dtype="bf16", seed=91, random_s0=True)
    _both(wk, big, chunk_len, segments)
    _both(wk, small, chunk_len, segments)


def test_static_scratch_limit(wk):
    import torch
    B, T, H = 4, 4096, 32
    desc = wk.make_desc(B, T, H, 64, wk.WKV7_BF16, 16)
    assert wk.split_workspace_bytes(desc, 16) > wk.STATIC_SCRATCH_BYTES
    x = [torch.zeros(B, T, H, 64, device="cuda", dtype=torch.bfloat16) for _ in range(6)]
    y = torch.full_like(x[0], 7.0)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = wk.lib().wkv7_forward_split_static(ctypes.byref(desc), *[p(t) for t in x], None, p(y), None,
                                            None, 16, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == wk.WKV7_ERR_STATIC_SCRATCH
    assert bool((y == 7.0).all())
