"""GPU parity of the a = b = 0 specialisation (a and b passed as NULL).

With a = b = 0 the transition is diagonal, S <- S diag(w_t) + v_t k_t^T: the
vector-decay recurrence that RWKV-7 extends ("Paper Review: RWKV-7 Goose",
Background information on delta rule).  Every entry point then runs kernels
specialised for it; each test here calls them through the C ABI and compares
with the fp64 oracle run on the same inputs with explicit zero a and b (the
oracle's a = b = 0 case is pinned to closed forms on the CPU).  Tolerances:
fp32 inputs max relative error <= 1e-4; bf16 inputs <= 2e-2 and cosine >= 0.9999.
"""

import numpy as np
import pytest

import oracle
from rwkv_wkv7_delta_amd import synth
from tests._util import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

NAMES = ("dr", "dw", "dk", "dv", "ds0")


@pytest.fixture(scope="module")
def wk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rwkv_wkv7_delta_amd as wk
    wk.lib()
    return wk


def _inputs(B, T, H, dtype, seed, random_s0=True, backward=False):
    inp = synth.generate(B, T, H, 64, dtype=dtype, seed=seed, random_s0=random_s0,
                         backward=backward)
    inp.a = np.zeros_like(inp.a)
    inp.b = np.zeros_like(inp.b)
    return inp


def _dev(inp):
    r, w, k, v = (to_dev(x, inp.dtype) for x in (inp.r, inp.w, inp.k, inp.v))
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    return r, w, k, v, s0


def _fwd(wk, inp, chunk_len, **kw):
    import torch
    r, w, k, v, s0 = _dev(inp)
    y, sT, tape = wk.forward(r, w, k, v, None, None, s0, chunk_len=chunk_len, **kw)
    torch.cuda.synchronize()
    return to_np(y), to_np(sT), tape


def _check_fwd(wk, inp, chunk_len, what, **kw):
    y, sT, _ = _fwd(wk, inp, chunk_len, **kw)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, inp.dtype, f"{what} y")
    assert_close(sT, sr, inp.dtype, f"{what} sT")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 17, 70])
def test_seq_fwd(wk, dtype, T):
    _check_fwd(wk, _inputs(2, T, 3, dtype, 300 + T), 0, f"seq {dtype} T={T}")


def test_seq_fwd_many_heads_launch(wk):
    """B*H >= 512: the one-workgroup-per-head launch of the scan."""
    _check_fwd(wk, _inputs(16, 40, 40, "bf16", 310), 0, "seq 640 heads")


@pytest.mark.parametrize("T", [1, 16, 31, 75, 257])
def test_chunked_fwd(wk, T):
    _check_fwd(wk, _inputs(2, T, 3, "bf16", 320 + T), 16, f"chunked T={T}")


def test_chunked_fwd_zero_state_no_final_state(wk):
    import torch
    inp = _inputs(1, 64, 2, "bf16", 330, random_s0=False)
    r, w, k, v, _ = _dev(inp)
    y, sT, _ = wk.forward(r, w, k, v, None, None, None, chunk_len=16, want_state=False)
    torch.cuda.synchronize()
    assert sT is None
    assert_close(to_np(y), oracle.forward(*inp.tensors(), None)[0], "bf16", "chunked s0=0 y")


@pytest.mark.parametrize("segments", [3, -3])
@pytest.mark.parametrize("T", [100, 257])
def test_split_fwd(wk, segments, T):
    """Maps (segments > 0) and sequential segments (< 0) over the specialised kernel."""
    _check_fwd(wk, _inputs(2, T, 3, "bf16", 340 + T), 16, f"split {segments} T={T}",
               segments=segments)


def test_split_fwd_auto_0_19b(wk):
    """B=4, T=1024, H=12 with the library's own segment plan."""
    _check_fwd(wk, _inputs(4, 1024, 12, "bf16", 350, random_s0=False), 16, "split auto 0.19b",
               segments=0)


def test_unsplit_and_split_agree_with_tape(wk):
    """The split forward's y, sT and tape state blocks match the unsplit ones."""
    import torch
    inp = _inputs(2, 300, 3, "bf16", 355)
    r, w, k, v, s0 = _dev(inp)
    B, T, H, N = inp.r.shape
    outs = []
    for seg in (None, 4, -4):
        y, sT, tape = wk.forward(r, w, k, v, None, None, s0, chunk_len=16, want_tape=True,
                                 segments=seg)
        torch.cuda.synchronize()
        outs.append((to_np(y), to_np(sT), to_np(wk.split_tape(tape, B, T, H, N)[1])))
    for y, sT, st in outs[1:]:
        assert_close(y, outs[0][0], "bf16", "split y vs unsplit")
        assert_close(sT, outs[0][1], "bf16", "split sT vs unsplit")
        assert_close(st, outs[0][2], "bf16", "split tape states vs unsplit")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_steps(wk, dtype):
    """Eight decode steps on resident states against the oracle's decode."""
    import torch
    inp = _inputs(3, 8, 5, dtype, 360)
    state = to_dev(inp.s0, "fp32")
    ref = inp.s0.astype(np.float64)
    for t in range(8):
        r, w, k, v = (to_dev(np.ascontiguousarray(x[:, t]), dtype) for x in (inp.r, inp.w, inp.k, inp.v))
        y = wk.decode_step(r, w, k, v, None, None, state)
        torch.cuda.synchronize()
        sl = [x[:, t] for x in inp.tensors()]
        yr, ref = oracle.decode_step(*sl, ref)
        assert_close(to_np(y), yr, dtype, f"decode {dtype} step {t} y")
    assert_close(to_np(state), ref, dtype, f"decode {dtype} state")


def _grads(wk, inp, dsT=None, use_tape=True, fwd_chunk=16, aux=False):
    import torch
    r, w, k, v, s0 = _dev(inp)
    dy = to_dev(inp.dy, inp.dtype)
    dsT_d = to_dev(dsT, "fp32") if dsT is not None else None
    tape = None
    if use_tape:
        _, _, tape = wk.forward(r, w, k, v, None, None, s0, chunk_len=fwd_chunk,
                                want_state=False, want_tape=True)
    extra = {"aux_stream": torch.cuda.Stream()} if aux else {}
    g = wk.backward(r, w, k, v, None, None, dy, s0, dsT_d, tape, chunk_len=fwd_chunk, **extra)
    torch.cuda.synchronize()
    assert g[4] is None and g[5] is None
    return [to_np(x) for x in g[:4]] + [to_np(g[6])]


def _ref_grads(inp, dsT=None):
    g = oracle.backward(*inp.tensors(), inp.s0, inp.dy, dsT)
    return g[:4] + (g[6],)


@pytest.mark.parametrize("T", [1, 16, 33, 100, 200])
def test_bwd(wk, T):
    inp = _inputs(2, T, 2, "bf16", 370 + T, backward=True)
    dsT = (0.1 * np.random.default_rng(T).standard_normal(inp.s0.shape)).astype(np.float32)
    for name, x, rr in zip(NAMES, _grads(wk, inp, dsT), _ref_grads(inp, dsT)):
        assert_close(x, rr, "bf16", f"T={T} {name}")


@pytest.mark.parametrize("fwd_chunk", [0, 16])
def test_bwd_without_tape(wk, fwd_chunk):
    """No tape: the chunked backward re-runs the specialised chunked forward;
    chunk_len = 0 runs the specialised sequential reverse pass."""
    inp = _inputs(1, 150, 3, "bf16", 380, backward=True)
    for name, x, rr in zip(NAMES, _grads(wk, inp, use_tape=False, fwd_chunk=fwd_chunk),
                           _ref_grads(inp)):
        assert_close(x, rr, "bf16", f"no tape (fwd chunk {fwd_chunk}) {name}")


def test_bwd_overlapped_two_groups(wk):
    """More heads than compute units: the two-stream backward splits the batch rows."""
    import torch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    H = 16
    B = (ncu + H - 1) // H + 2
    inp = _inputs(B, 40, H, "bf16", 390, backward=True)
    for name, x, rr in zip(NAMES, _grads(wk, inp, aux=True), _ref_grads(inp)):
        assert_close(x, rr, "bf16", f"overlapped B={B} {name}")


def test_bwd_leaves_da_db_buffers_untouched(wk):
    """da and db passed as buffers with a = b = None are not written."""
    import torch
    inp = _inputs(1, 48, 2, "bf16", 395, backward=True)
    r, w, k, v, s0 = _dev(inp)
    dy = to_dev(inp.dy, "bf16")
    grads = [torch.empty_like(r) for _ in range(4)] + [torch.full_like(r, 7.0) for _ in range(2)]
    g = wk.backward(r, w, k, v, None, None, dy, s0, None, None, grads=grads)
    torch.cuda.synchronize()
    assert bool((g[4] == 7.0).all()) and bool((g[5] == 7.0).all())
    ref = _ref_grads(inp)
    for name, x, rr in zip(NAMES, [to_np(x) for x in g[:4]] + [to_np(g[6])], ref):
        assert_close(x, rr, "bf16", f"with da/db buffers {name}")


def test_fwd_bwd_2_9b_shape_sampled(wk):
    """B=8, T=4096, H=40 (the 2.9B-model shape), bf16, a = b = 0: the forward
    with the library's own split plan and the overlapped backward on the GPU,
    the oracle on sampled heads."""
    import torch
    inp = _inputs(8, 4096, 40, "bf16", 0, random_s0=False, backward=True)
    r, w, k, v, _ = _dev(inp)
    dy = to_dev(inp.dy, "bf16")
    y, _, tape = wk.forward(r, w, k, v, None, None, None, chunk_len=16, want_state=False,
                            want_tape=True, segments=0)
    g = wk.backward(r, w, k, v, None, None, dy, None, None, tape, aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    pairs = [(0, 0), (7, 39), (4, 13)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, _ = oracle.forward(*sel, None)
    assert_close(oracle.select_heads(to_np(y), pairs), yr, "bf16", "2.9b a=b=0 y")
    ref = oracle.backward(*sel, None, oracle.select_heads(inp.dy, pairs))
    got = [to_np(x) for x in g[:4]]
    for name, x, rr in zip(NAMES, got, ref[:4]):
        assert_close(oracle.select_heads(x, pairs), rr, "bf16", f"2.9b a=b=0 {name}")
    assert g[4] is None and g[5] is None
