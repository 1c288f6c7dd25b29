"""GPU parity of the chunked forward at head size N = 32 against the fp64 oracle.

The larger and smaller WKV states of "Millions of States: Designing a Scalable
MoE Architecture with RWKV-7 Meta-learner" (Abstract) read as other head sizes
of the same recurrence; the chunked form at N = 32 runs two producer, two
consumer and two inverse waves per head, two workgroups per compute unit.
bf16 inputs with an fp32 state: max relative error <= 2e-2, cosine >= 0.9999.
"""

import numpy as np
import pytest

import oracle
from rwkv_wkv7_delta_amd import synth
from tests._util import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

N = 32


@pytest.fixture(scope="module")
def wk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rwkv_wkv7_delta_amd as wk
    wk.lib()
    return wk


def _run(wk, inp, chunk_len=16, want_tape=False, segments=None, decay_only=False, want_ckpt=False):
    import torch
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    if decay_only:
        dev[4] = dev[5] = None
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    y, sT, extra = wk.forward(*dev, s0, chunk_len=chunk_len, want_tape=want_tape,
                              segments=segments, want_ckpt=want_ckpt)
    torch.cuda.synchronize()
    return to_np(y), to_np(sT), extra


def _ref(inp, decay_only=False):
    r, w, k, v, a, b = inp.tensors()
    if decay_only:
        a, b = np.zeros_like(a), np.zeros_like(b)
    return oracle.forward(r, w, k, v, a, b, inp.s0)


@pytest.mark.parametrize("T", [1, 16, 33, 70, 130, 257])
def test_chunked_forward_ragged(wk, T):
    inp = synth.generate(2, T, 3, N, dtype="bf16", seed=700 + T, random_s0=True)
    y, sT, _ = _run(wk, inp)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", f"N=32 T={T} y")
    assert_close(sT, sr, "bf16", f"N=32 T={T} sT")


def test_chunked_forward_zero_state_and_decay_only(wk):
    inp = synth.generate(1, 200, 4, N, dtype="bf16", seed=711)
    for decay_only in (False, True):
        y, sT, _ = _run(wk, inp, decay_only=decay_only)
        yr, sr = _ref(inp, decay_only)
        assert_close(y, yr, "bf16", f"N=32 zero s0 decay_only={decay_only} y")
        assert_close(sT, sr, "bf16", f"N=32 zero s0 decay_only={decay_only} sT")


def test_chunked_matches_scan(wk):
    inp = synth.generate(2, 512, 4, N, dtype="bf16", seed=712, random_s0=True)
    yc, sc, _ = _run(wk, inp, chunk_len=16)
    ys, ss, _ = _run(wk, inp, chunk_len=0)
    assert_close(yc, ys, "bf16", "N=32 chunk vs scan y")
    assert_close(sc, ss, "bf16", "N=32 chunk vs scan sT")


def test_many_heads_two_per_compute_unit(wk):
    """B=16, T=1024, H=40 (640 heads: more than one workgroup per compute unit
    everywhere), sampled heads against the oracle."""
    inp = synth.generate(16, 1024, 40, N, dtype="bf16", seed=713, random_s0=True)
    y, sT, _ = _run(wk, inp)
    pairs = [(0, 0), (3, 17), (9, 39), (15, 22), (7, 5)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(y, pairs), yr, "bf16", "N=32 640 heads y")
    assert_close(oracle.select_heads(sT, pairs, state=True), sr, "bf16", "N=32 640 heads sT")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(sT))


def test_tape_holds_entry_states_and_removal_readouts(wk):
    B, T, H = 1, 75, 2
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=714, random_s0=True)
    _, _, tape = _run(wk, inp, want_tape=True)
    z, st = (to_np(x) for x in wk.split_tape(tape, B, T, H, N))
    xs = inp.tensors()
    prefix = [inp.s0.astype(np.float64)]
    for t in range(1, T):
        prefix.append(oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1])
    zr = np.stack([np.einsum("bhij,bhj->bhi", prefix[t], xs[4][:, t].astype(np.float64))
                   for t in range(T)], axis=1)
    assert_close(z, zr, "bf16", "N=32 tape z")
    nblk = (T + 31) // 32
    assert st.shape == (B, H, nblk, N, N)
    for m in range(nblk):
        assert_close(st[:, :, m], np.swapaxes(prefix[32 * m], -1, -2), "bf16", f"N=32 tape state {m}")


def test_checkpoints(wk):
    import torch
    B, T, H = 2, 75, 3
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=715, random_s0=True)
    y, sT, ck = _run(wk, inp, want_ckpt=True)
    xs = inp.tensors()
    assert ck.shape == (B, H, (T + 15) // 16, N, N)
    for m, t in enumerate(range(0, T, 16)):
        ref = inp.s0.astype(np.float64) if t == 0 else oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1]
        assert_close(to_np(ck[:, :, m]), ref, "bf16", f"N=32 ckpt {m}")


@pytest.mark.parametrize("segments", [2, 3, 5, -2, -3])
def test_split_in_time(wk, segments):
    """Maps (2, 3, 5 segments: the composition of the scan's kernel serves
    N = 32) and sequential segments (-2, -3)."""
    inp = synth.generate(2, 257, 3, N, dtype="bf16", seed=720 + segments, random_s0=True)
    B, T, H, _ = inp.r.shape
    assert wk.split_workspace_bytes(wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16), segments) > 0
    y, sT, _ = _run(wk, inp, segments=segments)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", f"N=32 split {segments} y")
    assert_close(sT, sr, "bf16", f"N=32 split {segments} sT")


def test_split_automatic_few_heads(wk):
    """48 heads (B=4, T=1024, H=12): the library's plan splits every head."""
    inp = synth.generate(4, 1024, 12, N, dtype="bf16", seed=730)
    y, sT, _ = _run(wk, inp, segments=0)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", "N=32 automatic split y")
    assert_close(sT, sr, "bf16", "N=32 automatic split sT")


@pytest.mark.parametrize("kind", ["replace", "swap", "steep_decay"])
def test_special_regimes(wk, kind):
    inp = synth.generate_edge(kind, 2, 300, 3, N, dtype="bf16", seed=740)
    y, sT, _ = _run(wk, inp)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", f"N=32 {kind} y")
    assert_close(sT, sr, "bf16", f"N=32 {kind} sT")


def test_forward_epilogue_at_n32(wk):
    """chunk_len = 16 at N = 32 takes the forward and then the step in place."""
    import torch
    B, T, H = 2, 100, 3
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=750, random_s0=True)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=751)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    out, sT = wk.forward_epilogue(*dev, to_dev(inp.s0, "fp32"), to_dev(e.g, "bf16"),
                                  to_dev(e.u, "fp32"), to_dev(e.gamma, "fp32"),
                                  to_dev(e.beta, "fp32"), eps=1e-5, mode=1, chunk_len=16)
    torch.cuda.synchronize()
    yr, sr = _ref(inp)
    ref = oracle.epilogue(yr, inp.r, inp.k, inp.v, e.g, e.u, e.gamma, e.beta, eps=1e-5, mode=1)
    assert_close(to_np(out), ref, "bf16", "N=32 forward + step")
    assert_close(to_np(sT), sr, "bf16", "N=32 forward + step sT")


# ---------------------------------------------------------------------------
# The chunked backward at N = 32
# ---------------------------------------------------------------------------

NAMES = ("dr", "dw", "dk", "dv", "da", "db", "ds0")


def _grads(wk, inp, dsT=None, use_tape=True, decay_only=False, aux=False, chunk_len=16):
    import torch
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    if decay_only:
        dev[4] = dev[5] = None
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    dy = to_dev(inp.dy, "bf16")
    dsT_d = to_dev(dsT, "fp32") if dsT is not None else None
    tape = None
    if use_tape and chunk_len == 16:
        _, _, tape = wk.forward(*dev, s0, chunk_len=16, want_state=False, want_tape=True)
    g = wk.backward(*dev, dy, s0, dsT_d, tape, chunk_len=chunk_len,
                    aux_stream=torch.cuda.Stream() if aux else None)
    torch.cuda.synchronize()
    return [None if x is None else to_np(x) for x in g]


def _ref_grads(inp, dsT=None, decay_only=False):
    r, w, k, v, a, b = inp.tensors()
    if decay_only:
        a, b = np.zeros_like(a), np.zeros_like(b)
    return oracle.backward(r, w, k, v, a, b, inp.s0, inp.dy, dsT)


def _check(got, ref, what, decay_only=False):
    for name, x, rr in zip(NAMES, got, ref):
        if decay_only and name in ("da", "db"):
            assert x is None
            continue
        assert_close(x, rr, "bf16", f"{what} {name}")


@pytest.mark.parametrize("T", [1, 16, 33, 64, 100, 200])
def test_backward_ragged(wk, T):
    inp = synth.generate(2, T, 2, N, dtype="bf16", seed=800 + T, random_s0=True, backward=True)
    dsT = (0.1 * np.random.default_rng(T).standard_normal(inp.s0.shape)).astype(np.float32)
    _check(_grads(wk, inp, dsT), _ref_grads(inp, dsT), f"N=32 T={T}")


def test_backward_without_tape_and_decay_only(wk):
    inp = synth.generate(2, 150, 3, N, dtype="bf16", seed=810, random_s0=True, backward=True)
    _check(_grads(wk, inp, use_tape=False), _ref_grads(inp), "N=32 no tape")
    _check(_grads(wk, inp, decay_only=True), _ref_grads(inp, decay_only=True), "N=32 a=b=0", True)


def test_backward_matches_sequential_reverse_pass(wk):
    inp = synth.generate(2, 200, 3, N, dtype="bf16", seed=811, random_s0=True, backward=True)
    chunked = _grads(wk, inp)
    seq = _grads(wk, inp, chunk_len=0)
    for name, x, y in zip(NAMES, chunked, seq):
        assert_close(x, y, "bf16", f"N=32 chunked vs sequential {name}")


def test_backward_many_heads_two_streams(wk):
    """B=16, T=512, H=40 (640 heads, more than two per compute unit): the
    two-stream backward splits the batch rows; sampled heads against the oracle."""
    import torch
    inp = synth.generate(16, 512, 40, N, dtype="bf16", seed=812, random_s0=True, backward=True)
    got = _grads(wk, inp, aux=True)
    pairs = [(0, 0), (5, 17), (11, 39), (15, 3)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    ref = oracle.backward(*sel, oracle.select_heads(inp.s0, pairs, state=True),
                          oracle.select_heads(inp.dy, pairs))
    for name, x, rr in zip(NAMES, got, ref):
        xs = oracle.select_heads(x, pairs, state=(name == "ds0"))
        assert_close(xs, rr, "bf16", f"N=32 640 heads {name}")
        assert np.all(np.isfinite(x))
