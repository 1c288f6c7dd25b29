"""GPU parity of the chunked backward (dr, dw, dk, dv, da, db, ds0).

The HIP gradients are compared with the fp64 oracle's reverse-mode gradients
(themselves pinned to central finite differences on the CPU) and, on the
T = 32 slice of the 2.9B-model shape, checked directly against finite
differences of the oracle forward, element by element.
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


def _gpu_grads(wk, inp, dsT=None, use_tape=True, fwd_chunk=16):
    import torch
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    dy = to_dev(inp.dy, inp.dtype)
    dsT_d = to_dev(dsT, "fp32") if dsT is not None else None
    tape = None
    if use_tape:
        _, _, tape = wk.forward(*dev, s0, chunk_len=fwd_chunk, want_state=False, want_tape=True)
    g = wk.backward(*dev, dy, s0, dsT_d, tape, chunk_len=fwd_chunk)
    torch.cuda.synchronize()
    return [to_np(x) for x in g]


def _check(got, ref, what):
    for name, x, rr in zip(NAMES, got, ref):
        assert_close(x, rr, "bf16", f"{what} {name}")


@pytest.mark.parametrize("T", [1, 16, 33, 64, 100, 200])
def test_bwd_ragged(wk, T):
    inp = synth.generate(2, T, 2, 64, dtype="bf16", seed=200 + T, random_s0=True, backward=True)
    dsT = (0.1 * np.random.default_rng(T).standard_normal(inp.s0.shape)).astype(np.float32)
    got = _gpu_grads(wk, inp, dsT)
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy, dsT)
    _check(got, ref, f"T={T}")


def test_bwd_stages_compose_to_backward(wk):
    """wkv7_backward_adjoint then wkv7_backward_gradients == wkv7_backward, bit for bit
    (same kernels, same inputs), and each stage writes only its own outputs."""
    import torch
    inp = synth.generate(2, 150, 3, 64, dtype="bf16", seed=77, random_s0=True, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, "bf16")
    _, _, tape = wk.forward(*dev, s0, chunk_len=16, want_state=False, want_tape=True)
    whole = wk.backward(*dev, dy, s0, None, tape)
    sentinel = torch.tensor(1234.0, dtype=torch.bfloat16)
    grads = [torch.full_like(dev[0], 1234.0) for _ in range(6)]
    ds0 = torch.full_like(s0, 1234.0)
    desc = wk.make_desc(2, 150, 3, 64, wk.WKV7_BF16, 16)
    ws = torch.empty(wk.workspace_bytes(desc, True) // 4, device=s0.device)
    wk.backward(*dev, dy, s0, None, tape, workspace=ws, stage="adjoint", grads=grads, ds0=ds0)
    torch.cuda.synchronize()
    for i in (0, 1, 2, 4, 5):   # dr, dw, dk, da, db untouched by the first stage
        assert bool((grads[i].cpu() == sentinel).all()), NAMES[i]
    assert torch.equal(grads[3], whole[3]) and torch.equal(ds0, whole[6])
    wk.backward(*dev, dy, s0, None, tape, workspace=ws, stage="gradients", grads=grads, ds0=ds0)
    torch.cuda.synchronize()
    for i in range(6):
        assert torch.equal(grads[i], whole[i]), NAMES[i]
    assert torch.equal(ds0, whole[6])


@pytest.mark.parametrize("use_tape", [True, False])
def test_bwd_overlapped_matches_single_stream(wk, use_tape):
    """wkv7_backward_overlapped (two batch-row groups, the first group's per-key
    pass on a second stream) == wkv7_backward, bit for bit, at 320 heads (more
    than one per compute unit); the per-key pass's block queue resets itself, so
    a second gradients stage on the same workspace repeats the result."""
    import torch
    B, T, H = 8, 96, 40
    inp = synth.generate(B, T, H, 64, dtype="bf16", seed=31, random_s0=True, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    dy = to_dev(inp.dy, "bf16")
    dsT = to_dev((0.1 * np.random.default_rng(5).standard_normal(inp.s0.shape)).astype(np.float32), "fp32")
    tape = None
    if use_tape:
        _, _, tape = wk.forward(*dev, s0, chunk_len=16, want_state=False, want_tape=True)
    ref = wk.backward(*dev, dy, s0, dsT, tape)
    aux = torch.cuda.Stream()
    got = wk.backward(*dev, dy, s0, dsT, tape, aux_stream=aux)
    torch.cuda.synchronize()
    for i, name in enumerate(NAMES):
        assert torch.equal(got[i], ref[i]), name
    if use_tape:
        desc = wk.make_desc(B, T, H, 64, wk.WKV7_BF16, 16)
        ws = torch.empty(wk.workspace_bytes(desc, True) // 4, device=s0.device)
        grads = [torch.empty_like(dev[0]) for _ in range(6)]
        wk.backward(*dev, dy, s0, dsT, tape, workspace=ws, stage="adjoint", grads=grads)
        for rep in range(2):
            for i in (0, 1, 2, 4, 5):
                grads[i].fill_(7.0)
            wk.backward(*dev, dy, s0, dsT, tape, workspace=ws, stage="gradients", grads=grads)
            torch.cuda.synchronize()
            for i in range(6):
                assert torch.equal(grads[i], ref[i]), (rep, NAMES[i])


def test_bwd_overlapped_without_split_is_plain_backward(wk):
    """Few heads (B*H below the compute units) or one batch row: the two-stream
    entry point runs the plain backward on the first stream."""
    import torch
    for (B, H) in [(2, 3), (1, 40)]:
        inp = synth.generate(B, 70, H, 64, dtype="bf16", seed=40 + B, random_s0=True, backward=True)
        dev = [to_dev(x, "bf16") for x in inp.tensors()]
        s0 = to_dev(inp.s0, "fp32")
        dy = to_dev(inp.dy, "bf16")
        _, _, tape = wk.forward(*dev, s0, chunk_len=16, want_state=False, want_tape=True)
        ref = wk.backward(*dev, dy, s0, None, tape)
        got = wk.backward(*dev, dy, s0, None, tape, aux_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        for i, name in enumerate(NAMES):
            assert torch.equal(got[i], ref[i]), (B, H, name)


@pytest.mark.parametrize("fwd_chunk", [0, 16])
def test_bwd_without_tape_matches_tape_path(wk, fwd_chunk):
    """Without a tape the chunked backward re-runs the chunked forward into the
    workspace first; with chunk_len = 0 the sequential reverse pass runs, which
    uses no tape either way."""
    inp = synth.generate(1, 150, 3, 64, dtype="bf16", seed=31, random_s0=True, backward=True)
    a = _gpu_grads(wk, inp, use_tape=True, fwd_chunk=fwd_chunk)
    b = _gpu_grads(wk, inp, use_tape=False, fwd_chunk=fwd_chunk)
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy)
    _check(a, ref, "tape")
    _check(b, ref, "re-run")


def test_bwd_zero_initial_state_no_dsT(wk):
    inp = synth.generate(2, 96, 2, 64, dtype="bf16", seed=32, backward=True)
    got = _gpu_grads(wk, inp)
    ref = oracle.backward(*inp.tensors(), None, inp.dy)
    _check(got, ref, "zero s0")


def test_bwd_empty_sequence(wk):
    import torch
    z = torch.zeros(2, 0, 3, 64, device="cuda", dtype=torch.bfloat16)
    dsT = torch.randn(2, 3, 64, 64, device="cuda")
    g = wk.backward(z, z, z, z, z, z, z, None, dsT, None)
    assert torch.equal(g[-1], dsT)


def test_bwd_2_9b_t32_slice_vs_oracle_and_fd(wk):
    """B=8, H=40, T=32 slice of the 2.9B-model shape, dy ~ N(0,1), dsT = 0."""
    wl = synth.WORKLOADS["fwd_bwd_2.9b"]
    inp = synth.generate_workload(wl, seed=0, T=32)
    got = _gpu_grads(wk, inp)
    ref = oracle.backward(*inp.tensors(), None, inp.dy)
    _check(got[:6], ref[:6], "2.9b T=32")
    # Element-wise central differences of the fp64 oracle forward on a few
    # heads: each sampled GPU gradient element must match d L / d x_e to the
    # bf16 bar (relative to the tensor's largest gradient).
    pairs = [(0, 0), (7, 39), (3, 21)]
    sel = [oracle.select_heads(x, pairs).astype(np.float64) for x in inp.tensors()]
    s0 = np.zeros((len(pairs), 1, 64, 64))
    dy = oracle.select_heads(inp.dy, pairs).astype(np.float64)
    ref_sel = oracle.backward(*sel, s0, dy)
    gpu_sel = [oracle.select_heads(x, pairs) for x in got[:6]]
    gpu_sel.append(oracle.select_heads(got[6], pairs, state=True))

    def loss(xs, st):
        y, _ = oracle.forward(*xs, st)
        return float((y * dy).sum())

    h = 1e-3
    rng = np.random.default_rng(3)
    for q in range(7):
        arr = sel[q] if q < 6 else s0
        scale = np.abs(ref_sel[q]).max()
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(sel, s0)
            arr[idx] = old - h
            lm = loss(sel, s0)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - ref_sel[q][idx]) <= 1e-6 * scale      # oracle vs FD
            assert abs(gpu_sel[q][idx] - fd) <= 2e-2 * scale, (NAMES[q], idx, gpu_sel[q][idx], fd)


def test_bwd_2_9b_full_sampled(wk):
    """B=8, T=4096, H=40, bf16, dy ~ N(0,1), dsT = 0: the full fwd + bwd on the
    GPU in the benchmarked launch configuration; the oracle on sampled heads."""
    wl = synth.WORKLOADS["fwd_bwd_2.9b"]
    inp = synth.generate_workload(wl, seed=0)
    got = _gpu_grads(wk, inp)
    pairs = [(0, 0), (7, 39), (4, 13)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    ref = oracle.backward(*sel, None, oracle.select_heads(inp.dy, pairs))
    for name, x, rr in zip(NAMES, got[:6], ref[:6]):
        assert_close(oracle.select_heads(x, pairs), rr, "bf16", f"2.9b full {name}")
    assert_close(oracle.select_heads(got[6], pairs, state=True), ref[6], "bf16", "2.9b full ds0")
    for x in got:
        assert np.all(np.isfinite(x))
