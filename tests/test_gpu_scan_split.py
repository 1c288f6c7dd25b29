"""GPU parity of the sequential scan split in time (wkv7_forward_split with
chunk_len = 0, by maps; N = 32, 64 and 128).

The state update is affine in the state, S <- S M_t + v_t k_t^T with
M_t = diag(w_t) + a_t b_t^T ("Paper Review: RWKV-7 Goose", The approach), so a
segment maps its entry state as S_out = S_in P + Hm.  The scan runs segment 0
and the two map runs of the middle segments first, composes the entry states
in fp32, then re-runs segments 1 .. n-1 with their outputs.  Every result (y,
the final state, the tape) is compared with the fp64 oracle on the same seeded
inputs, or with the unsplit scan.  Tolerances: fp32 inputs max relative error
<= 1e-4; bf16 inputs <= 2e-2 and cosine >= 0.9999.
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


def _run(wk, inp, segments, ab=True, want_tape=False):
    import torch
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    if not ab:
        dev[4] = dev[5] = None
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    y, sT, tape = wk.forward(*dev, s0, chunk_len=0, want_tape=want_tape, segments=segments)
    torch.cuda.synchronize()
    return to_np(y), to_np(sT), tape


def _plan_bytes(wk, inp, segments):
    B, T, H, N = inp.r.shape
    dt = wk.WKV7_BF16 if inp.dtype == "bf16" else wk.WKV7_F32
    return wk.split_workspace_bytes(wk.make_desc(B, T, H, N, dt, 0), segments)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("segments", [2, 3, 5])
@pytest.mark.parametrize("T", [100, 257])
def test_scan_split_matches_oracle(wk, dtype, segments, T):
    inp = synth.generate(2, T, 3, 64, dtype=dtype, seed=500 + T + segments, random_s0=True)
    assert _plan_bytes(wk, inp, segments) > 0
    y, sT, _ = _run(wk, inp, segments)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, dtype, f"scan split{segments} {dtype} T={T} y")
    assert_close(sT, sr, dtype, f"scan split{segments} {dtype} T={T} sT")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("N", [32, 128])
@pytest.mark.parametrize("T", [100, 257])
def test_scan_split_head_sizes(wk, dtype, N, T):
    """N = 32 and 128 (four segments: two compositions by the any-N kernel)."""
    inp = synth.generate(2, T, 3, N, dtype=dtype, seed=580 + T + N, random_s0=True)
    assert _plan_bytes(wk, inp, 4) > 0
    y, sT, _ = _run(wk, inp, 4)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, dtype, f"scan split N={N} {dtype} T={T} y")
    assert_close(sT, sr, dtype, f"scan split N={N} {dtype} T={T} sT")


@pytest.mark.parametrize("N", [32, 128])
def test_scan_split_head_sizes_auto(wk, N):
    """The library's plan at few heads: B=1, T=2048, H=4."""
    inp = synth.generate(1, 2048, 4, N, dtype="bf16", seed=590 + N, random_s0=True)
    assert _plan_bytes(wk, inp, 0) > 0
    y, sT, _ = _run(wk, inp, 0)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", f"scan split auto N={N} y")
    assert_close(sT, sr, "bf16", f"scan split auto N={N} sT")


@pytest.mark.parametrize("segments", [2, 4])
def test_scan_split_decay_only(wk, segments):
    """a = b = NULL: the specialised scan under the segment plan."""
    inp = synth.generate(2, 200, 3, 64, dtype="bf16", seed=520 + segments, random_s0=True)
    inp.a = np.zeros_like(inp.a)
    inp.b = np.zeros_like(inp.b)
    y, sT, _ = _run(wk, inp, segments, ab=False)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", f"scan split{segments} a=b=0 y")
    assert_close(sT, sr, "bf16", f"scan split{segments} a=b=0 sT")


def test_scan_split_mixed_layouts(wk):
    """192 heads in 3 segments: the first launch holds 576 runs (the many-heads
    layout, one workgroup per run), the second 384 (four per run)."""
    inp = synth.generate(16, 100, 12, 64, dtype="bf16", seed=530, random_s0=True)
    y, sT, _ = _run(wk, inp, 3)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", "scan split 192 heads y")
    assert_close(sT, sr, "bf16", "scan split 192 heads sT")


def test_scan_split_auto_few_heads(wk):
    """B=1, T=4096, H=12 with the library's own plan for the scan (12 heads
    fill a fifth of the device: every head is split); 320 heads are not."""
    inp = synth.generate(1, 4096, 12, 64, dtype="bf16", seed=540, random_s0=False)
    assert _plan_bytes(wk, inp, 0) > 0
    assert wk.split_workspace_bytes(wk.make_desc(8, 4096, 40, 64, wk.WKV7_BF16, 0), 0) == 0
    y, sT, _ = _run(wk, inp, 0)
    yr, sr = oracle.forward(*inp.tensors(), None)
    assert_close(y, yr, "bf16", "scan split auto y")
    assert_close(sT, sr, "bf16", "scan split auto sT")


@pytest.mark.parametrize("ab", [True, False])
def test_scan_split_tape_matches_unsplit(wk, ab):
    """The split scan's y, sT and tape (removal read-outs and block states)
    agree with the unsplit scan's; the tape then feeds the chunked backward,
    checked against the oracle's gradients."""
    import torch
    inp = synth.generate(2, 300, 3, 64, dtype="bf16", seed=550 + ab, random_s0=True,
                         backward=True)
    if not ab:
        inp.a = np.zeros_like(inp.a)
        inp.b = np.zeros_like(inp.b)
    B, T, H, N = inp.r.shape
    outs = []
    for seg in (None, 4):
        y, sT, tape = _run(wk, inp, seg, ab=ab, want_tape=True)
        z, st = wk.split_tape(tape, B, T, H, N)
        outs.append((y, sT, to_np(z), to_np(st), tape))
    for i, name in enumerate(("y", "sT", "tape Z", "tape states")):
        if name == "tape Z" and not ab:
            continue   # no removal read-outs are written for a = b = 0
        assert_close(outs[1][i], outs[0][i], "bf16", f"scan split vs unsplit {name}")
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    if not ab:
        dev[4] = dev[5] = None
    s0 = to_dev(inp.s0, "fp32")
    g = wk.backward(*dev, to_dev(inp.dy, "bf16"), s0, None, outs[1][4])
    torch.cuda.synchronize()
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy)
    for j, name in enumerate(("dr", "dw", "dk", "dv", "da", "db", "ds0")):
        if g[j] is None:
            assert not ab and name in ("da", "db")
            continue
        assert_close(to_np(g[j]), ref[j], "bf16", f"backward from split scan tape {name}")


@pytest.mark.parametrize("T", [1, 32, 33, 64, 65])
def test_scan_split_short_sequences(wk, T):
    """Segments start at multiples of 32 tokens and the last keeps at least one:
    T = 1 and 32 run unsplit, 33 as 32 + 1 tokens, 64 as 32 + 32, 65 as
    32 + 32 + 1 (three segments: one map run)."""
    inp = synth.generate(1, T, 2, 64, dtype="fp32", seed=560 + T, random_s0=True)
    y, sT, _ = _run(wk, inp, 3)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "fp32", f"scan split short T={T} y")
    assert_close(sT, sr, "fp32", f"scan split short T={T} sT")


def test_scan_split_empty_sequence(wk):
    """T = 0: no tokens; the final state is s0."""
    inp = synth.generate(1, 0, 2, 64, dtype="fp32", seed=570, random_s0=True)
    y, sT, _ = _run(wk, inp, 4)
    assert y.shape == (1, 0, 2, 64)
    np.testing.assert_array_equal(sT, inp.s0)


@pytest.mark.parametrize("N", [32, 64, 128])
def test_scan_split_sixteen_segments_fp32(wk, N):
    """The most segments a plan takes (16 of 64 tokens, the last 40): fourteen
    fp32 compositions in a row, held to the fp32 tolerance."""
    inp = synth.generate(1, 1000, 2, N, dtype="fp32", seed=600 + N, random_s0=True)
    B, T, H, _ = inp.r.shape
    st = N * N * 4
    assert _plan_bytes(wk, inp, 16) == B * H * 3 * 16 * st
    y, sT, _ = _run(wk, inp, 16)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "fp32", f"scan split 16 N={N} y")
    assert_close(sT, sr, "fp32", f"scan split 16 N={N} sT")
