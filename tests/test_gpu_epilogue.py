"""GPU parity of the step after the read-out, on its own and fused into the
forward, through the C ABI, against the fp64 oracle.

"Paper Review: RWKV-7 Goose", The approach: the receptance also attends to the
current token, and the result is normalised per head and gated.  The kernels
compute in fp32 and write the token dtype:

* on its own (wkv7_epilogue), on the same inputs as the oracle: fp32 results
  within 1e-5 of max |ref|; bf16 results within their rounding, 2^-8 |ref|
  elementwise plus 1e-5 max |ref|.
* fused after the recurrence (wkv7_forward_epilogue): the oracle runs its
  forward and then the step, all in fp64; bf16 tolerance as for the forward
  (max relative error <= 2e-2, cosine >= 0.9999).
"""

import numpy as np
import pytest

import oracle
from rwkv_wkv7_delta_amd import synth
from tests._util import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

MODES = (0, 1, 2)


@pytest.fixture(scope="module")
def wk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rwkv_wkv7_delta_amd as wk
    wk.lib()
    return wk


def _check_exact_inputs(out, ref, dtype, what):
    out = np.asarray(out, dtype=np.float64)
    assert np.all(np.isfinite(out)), f"{what}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(out - ref)
    if dtype == "fp32":
        assert err.max() <= 1e-5 * scale, f"{what}: {err.max() / scale:.3e} of max |ref|"
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * scale
        worst = np.argmax(err - bound)
        assert np.all(err <= bound), f"{what}: |err| {err.flat[worst]:.3e} > {bound.flat[worst]:.3e}"


def _parts(wk, e, dtype, use):
    """Device tensors of the learned parts; `use` names the ones passed."""
    g = to_dev(e.g, dtype) if "g" in use else None
    u = to_dev(e.u, "fp32") if "u" in use else None
    gamma = to_dev(e.gamma, "fp32") if "gamma" in use else None
    beta = to_dev(e.beta, "fp32") if "beta" in use else None
    return g, u, gamma, beta


def _ref_parts(e, use):
    return tuple(getattr(e, x) if x in use else None for x in ("g", "u", "gamma", "beta"))


ALL = ("g", "u", "gamma", "beta")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("N", [32, 64, 128])
@pytest.mark.parametrize("mode", MODES)
def test_epilogue_alone(wk, dtype, N, mode):
    """B=2, T=37, H=3 (222 rows: a ragged last workgroup), every learned part."""
    import torch
    B, T, H = 2, 37, 3
    inp = synth.generate(B, T, H, N, dtype=dtype, seed=3)
    e = synth.generate_epilogue(B, T, H, N, dtype=dtype, seed=4)
    y = to_dev(e.y, dtype)
    r, k, v = (to_dev(x, dtype) for x in (inp.r, inp.k, inp.v))
    out = wk.epilogue(y, r, k, v, *_parts(wk, e, dtype, ALL), eps=1e-5, mode=mode)
    torch.cuda.synchronize()
    ref = oracle.epilogue(e.y, inp.r, inp.k, inp.v, *_ref_parts(e, ALL), eps=1e-5, mode=mode)
    _check_exact_inputs(to_np(out), ref, dtype, f"epilogue {dtype} N={N} mode={mode}")


@pytest.mark.parametrize("use", [(), ("g",), ("u",), ("gamma", "beta"), ("u", "beta")])
@pytest.mark.parametrize("mode", MODES)
def test_epilogue_optional_parts(wk, use, mode):
    """Absent parts (NULL) stand for g = 1, no term, gamma = 1, beta = 0; r, k
    and v are not read without the term (passed as None then)."""
    import torch
    B, T, H, N = 1, 50, 4, 64
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=5)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=6)
    y = to_dev(e.y, "bf16")
    term = "u" in use
    r, k, v = ((to_dev(x, "bf16") for x in (inp.r, inp.k, inp.v)) if term else (None,) * 3)
    out = wk.epilogue(y, r, k, v, *_parts(wk, e, "bf16", use), eps=1e-3, mode=mode)
    torch.cuda.synchronize()
    ref = oracle.epilogue(e.y, inp.r, inp.k, inp.v, *_ref_parts(e, use), eps=1e-3, mode=mode)
    _check_exact_inputs(to_np(out), ref, "bf16", f"epilogue parts={use} mode={mode}")


def test_epilogue_identity_and_in_place(wk):
    """Mode 0 with no term and no gate copies y bit for bit; out = y works in
    place and matches the separate output."""
    import torch
    B, T, H, N = 2, 33, 5, 64
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=7)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=8)
    y = to_dev(e.y, "bf16")
    same = wk.epilogue(y, None, None, None, mode=0)
    r, k, v = (to_dev(x, "bf16") for x in (inp.r, inp.k, inp.v))
    parts = _parts(wk, e, "bf16", ALL)
    sep = wk.epilogue(y, r, k, v, *parts, mode=1)
    y2 = y.clone()
    inplace = wk.epilogue(y2, r, k, v, *parts, mode=1, out=y2)
    torch.cuda.synchronize()
    assert torch.equal(same, y)
    assert inplace.data_ptr() == y2.data_ptr()
    assert torch.equal(inplace, sep)


def test_epilogue_empty(wk):
    import torch
    y = torch.empty(2, 0, 3, 64, device="cuda", dtype=torch.bfloat16)
    out = wk.epilogue(y, y, y, y, mode=1)
    assert out.shape == y.shape


def test_epilogue_full_size_2_9b_shape(wk):
    """B=8, T=4096, H=40, N=64 bf16 (1.3 M rows, past the grid's stride): every
    row against the oracle on the same inputs."""
    import torch
    B, T, H, N = 8, 4096, 40, 64
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=9)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=10)
    y = to_dev(e.y, "bf16")
    r, k, v = (to_dev(x, "bf16") for x in (inp.r, inp.k, inp.v))
    out = wk.epilogue(y, r, k, v, *_parts(wk, e, "bf16", ALL), eps=1e-5, mode=1)
    torch.cuda.synchronize()
    out = to_np(out)
    ref = oracle.epilogue(e.y, inp.r, inp.k, inp.v, *_ref_parts(e, ALL), eps=1e-5, mode=1)
    _check_exact_inputs(out, ref, "bf16", "epilogue 2.9b shape")


# ---------------------------------------------------------------------------
# Fused after the recurrence
# ---------------------------------------------------------------------------

def _fused_case(wk, inp, e, chunk_len, mode, use=ALL, decay_only=False):
    import torch
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    if decay_only:
        dev[4] = dev[5] = None
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    out, sT = wk.forward_epilogue(*dev, s0, *_parts(wk, e, inp.dtype, use), eps=1e-5, mode=mode,
                                  chunk_len=chunk_len)
    torch.cuda.synchronize()
    a, b = (np.zeros_like(inp.a), np.zeros_like(inp.b)) if decay_only else (inp.a, inp.b)
    yr, sr = oracle.forward(inp.r, inp.w, inp.k, inp.v, a, b, inp.s0)
    ref = oracle.epilogue(yr, inp.r, inp.k, inp.v, *_ref_parts(e, use), eps=1e-5, mode=mode)
    return to_np(out), to_np(sT), ref, sr


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T", [16, 300])
def test_fused_chunked_forward(wk, mode, T):
    """Chunked forward with the step fused (B=2, H=3, s0 ~ 0.1 N(0,1)); T=300
    ends in a partial chunk."""
    B, H, N = 2, 3, 64
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=11, random_s0=True)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=12)
    out, sT, ref, sr = _fused_case(wk, inp, e, 16, mode)
    assert_close(out, ref, "bf16", f"fused mode={mode} T={T}")
    assert_close(sT, sr, "bf16", f"fused sT mode={mode} T={T}")


@pytest.mark.parametrize("use", [(), ("g",), ("u",), ("gamma", "beta")])
def test_fused_chunked_optional_parts_and_decay_only(wk, use):
    B, T, H, N = 1, 200, 4, 64
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=13)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=14)
    for decay_only in (False, True):
        out, sT, ref, sr = _fused_case(wk, inp, e, 16, 1, use=use, decay_only=decay_only)
        assert_close(out, ref, "bf16", f"fused parts={use} decay_only={decay_only}")
        assert_close(sT, sr, "bf16", f"fused sT parts={use} decay_only={decay_only}")


def test_fused_mode0_without_parts_is_the_forward_read_out(wk):
    """With no term, no normalisation and no gate the fused kernel writes y
    itself: the same values wkv7_forward writes (both round the fp32 read-out)."""
    import torch
    B, T, H, N = 2, 160, 3, 64
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=15, random_s0=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    out, sT = wk.forward_epilogue(*dev, s0, mode=0, chunk_len=16)
    y, sT2, _ = wk.forward(*dev, s0, chunk_len=16)
    torch.cuda.synchronize()
    assert torch.equal(out, y)
    assert torch.equal(sT, sT2)


@pytest.mark.parametrize("N,dtype", [(32, "bf16"), (64, "fp32"), (128, "bf16")])
def test_forward_epilogue_sequential(wk, N, dtype):
    """chunk_len = 0: the scan, then the step in place."""
    B, T, H = 2, 45, 3
    inp = synth.generate(B, T, H, N, dtype=dtype, seed=16, random_s0=True)
    e = synth.generate_epilogue(B, T, H, N, dtype=dtype, seed=17)
    out, sT, ref, sr = _fused_case(wk, inp, e, 0, 1)
    assert_close(out, ref, dtype, f"scan + epilogue N={N} {dtype}")
    assert_close(sT, sr, dtype, f"scan sT N={N} {dtype}")


@pytest.mark.timeout(600)
def test_fused_full_size_2_9b_sampled_heads(wk):
    """B=8, T=4096, H=40 in one launch, as timed; 8 heads checked at full T."""
    import torch
    B, T, H, N = 8, 4096, 40, 64
    inp = synth.generate_workload(synth.WORKLOADS["fwd_bwd_2.9b"], seed=0)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=18)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    out, sT = wk.forward_epilogue(*dev, None, *_parts(wk, e, "bf16", ALL), eps=1e-5, mode=1,
                                  chunk_len=16)
    torch.cuda.synchronize()
    out, sT = to_np(out), to_np(sT)
    del dev
    pairs = [(0, 0), (1, 7), (2, 13), (3, 21), (4, 26), (5, 33), (6, 38), (7, 39)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, None)
    for i, (b_, h_) in enumerate(pairs):
        ref = oracle.epilogue(yr[i:i + 1], *(x[i:i + 1] for x in (sel[0], sel[2], sel[3])),
                              e.g[b_:b_ + 1, :, h_:h_ + 1], e.u[h_:h_ + 1], e.gamma[h_:h_ + 1],
                              e.beta[h_:h_ + 1], eps=1e-5, mode=1)
        assert_close(out[b_:b_ + 1, :, h_:h_ + 1], ref, "bf16", f"fused 2.9b head ({b_}, {h_})")
        assert_close(sT[b_, h_], sr[i, 0], "bf16", f"fused 2.9b sT ({b_}, {h_})")
    assert np.all(np.isfinite(out))
