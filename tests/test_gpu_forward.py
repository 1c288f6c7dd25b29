"""GPU parity of the forward scan, the chunked forward and the decode step.

Every test calls the HIP library through the C ABI (via the ctypes binding)
and compares with the fp64 oracle on the same seeded inputs.  Tolerances:
fp32 inputs max relative error <= 1e-4; bf16 inputs <= 2e-2 and cosine >= 0.9999.
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


def _run_fwd(wk, inp, chunk_len, want_tape=False):
    import torch
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    y, sT, tape = wk.forward(*dev, s0, chunk_len=chunk_len, want_tape=want_tape)
    torch.cuda.synchronize()
    if tape is not None:
        B, T, H, N = inp.r.shape
        tape = tuple(to_np(x) for x in wk.split_tape(tape, B, T, H, N))
    return to_np(y), to_np(sT), tape


def _check_fwd(wk, inp, chunk_len, what):
    y, sT, _ = _run_fwd(wk, inp, chunk_len)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, inp.dtype, f"{what} y")
    assert_close(sT, sr, inp.dtype, f"{what} sT")
    return y, sT


# ---------------------------------------------------------------------------
# Sequential scan
# ---------------------------------------------------------------------------

def test_seq_fwd_fp32_small_workload(wk):
    """B=1, T=64, H=2, fp32, zero initial state, seed 0."""
    wl = synth.WORKLOADS["fwd_fp32_small"]
    inp = synth.generate_workload(wl, seed=0)
    _check_fwd(wk, inp, 0, "fwd_fp32_small")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 17, 70, 200])
def test_seq_fwd_ragged(wk, dtype, T):
    inp = synth.generate(2, T, 3, 64, dtype=dtype, seed=T, random_s0=True)
    _check_fwd(wk, inp, 0, f"seq {dtype} T={T}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_seq_fwd_many_heads_launch(wk, dtype):
    """B*H >= 512 takes the one-workgroup-per-head launch with 4 lanes per state row."""
    inp = synth.generate(16, 40, 40, 64, dtype=dtype, seed=5, random_s0=True)
    _check_fwd(wk, inp, 0, f"seq 640 heads {dtype}")


def test_seq_fwd_0_19b_full(wk):
    """B=4, T=1024, H=12 (0.19B-model shape), bf16, zero state: all 48 heads."""
    wl = synth.WORKLOADS["fwd_0.19b"]
    inp = synth.generate_workload(wl, seed=0)
    _check_fwd(wk, inp, 0, "fwd_0.19b")


# ---------------------------------------------------------------------------
# Chunked forward (bf16 MFMA)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 16, 33, 70, 130, 257])
def test_chunk_fwd_ragged(wk, T):
    inp = synth.generate(2, T, 3, 64, dtype="bf16", seed=100 + T, random_s0=True)
    _check_fwd(wk, inp, 16, f"chunk T={T}")


def test_chunk_fwd_0_19b_full(wk):
    """B=4, T=1024, H=12 (0.19B-model shape), bf16, zero state, through the
    chunked form: every head against the oracle."""
    wl = synth.WORKLOADS["fwd_0.19b"]
    inp = synth.generate_workload(wl, seed=0)
    _check_fwd(wk, inp, 16, "chunked fwd_0.19b")


def test_chunk_fwd_zero_state(wk):
    inp = synth.generate(1, 96, 2, 64, dtype="bf16", seed=7)
    _check_fwd(wk, inp, 16, "chunk zero s0")


def test_chunk_matches_sequential_on_gpu(wk):
    inp = synth.generate(2, 512, 4, 64, dtype="bf16", seed=8, random_s0=True)
    yc, sc, _ = _run_fwd(wk, inp, 16)
    ys, ss, _ = _run_fwd(wk, inp, 0)
    assert_close(yc, ys, "bf16", "chunk vs seq y")
    assert_close(sc, ss, "bf16", "chunk vs seq sT")


def test_chunk_fwd_1_5b_full_sampled(wk):
    """B=8, T=4096, H=32 (1.5B-model shape), s0 ~ 0.1 N(0,1): full GPU run, the
    oracle on sampled heads over the whole sequence."""
    wl = synth.WORKLOADS["chunked_fwd_1.5b"]
    inp = synth.generate_workload(wl, seed=0)
    y, sT, _ = _run_fwd(wk, inp, 16)
    pairs = [(0, 0), (3, 17), (7, 31), (5, 9)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(y, pairs), yr, "bf16", "1.5b y")
    assert_close(oracle.select_heads(sT, pairs, state=True), sr, "bf16", "1.5b sT")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(sT))


# ---------------------------------------------------------------------------
# Checkpoints and edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,chunk_len", [("bf16", 0), ("bf16", 16), ("fp32", 0)])
def test_tape_holds_entry_states_and_removal_readouts(wk, dtype, chunk_len):
    """The forward's tape: z_t = S_{t-1} a_t for every token and the state
    entering every 32-token block (stored key-major), against the oracle's
    prefix states."""
    B, T, H = 1, 75, 2
    inp = synth.generate(B, T, H, 64, dtype=dtype, seed=9, random_s0=True)
    _, _, (z, st) = _run_fwd(wk, inp, chunk_len, want_tape=True)
    xs = inp.tensors()
    prefix = [inp.s0.astype(np.float64)]
    for t in range(1, T):
        prefix.append(oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1])
    zr = np.stack([np.einsum("bhij,bhj->bhi", prefix[t], xs[4][:, t].astype(np.float64))
                   for t in range(T)], axis=1)
    assert_close(z, zr, "bf16", "tape z")
    nblk = (T + 31) // 32
    assert st.shape == (B, H, nblk, 64, 64)
    for m in range(nblk):
        assert_close(st[:, :, m], np.swapaxes(prefix[32 * m], -1, -2), "bf16", f"tape state {m}")


def test_empty_sequence_copies_state(wk):
    import torch
    s0 = torch.randn(2, 3, 64, 64, device="cuda")
    z = torch.zeros(2, 0, 3, 64, device="cuda", dtype=torch.bfloat16)
    y, sT, _ = wk.forward(z, z, z, z, z, z, s0, chunk_len=16)
    assert torch.equal(sT, s0)
    y, sT, _ = wk.forward(z, z, z, z, z, z, None, chunk_len=0)
    assert torch.count_nonzero(sT) == 0


# ---------------------------------------------------------------------------
# Decode step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_small(wk, dtype):
    import torch
    steps, B, H = 20, 3, 5
    inp = synth.generate(B, steps, H, 64, dtype=dtype, seed=11, random_s0=True,
                         token_shape=(steps, B, H, 64))
    state = to_dev(inp.s0, "fp32")
    ys = []
    for t in range(steps):
        ys.append(to_np(wk.decode_step(*(to_dev(x[t], dtype) for x in inp.tensors()), state)))
    torch.cuda.synchronize()
    # The oracle's sequence forward equals T decode steps (pinned on the CPU).
    seq = [np.ascontiguousarray(np.moveaxis(x, 0, 1)) for x in inp.tensors()]
    yr, sr = oracle.forward(*seq, inp.s0)
    assert_close(np.stack(ys, 1), yr, dtype, "decode y")
    assert_close(to_np(state), sr, dtype, "decode state")


def test_decode_2_9b_shape_sampled(wk):
    """B=256, H=40 resident fp32 states ~ 0.1 N(0,1), bf16 per-step inputs:
    32 successive in-place steps at the full launch shape, oracle on sampled heads."""
    import torch
    wl = synth.WORKLOADS["decode_2.9b"]
    steps = 32
    inp = synth.generate_workload(wl, seed=0, T=steps)
    state = to_dev(inp.s0, "fp32")
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    ys = [to_np(wk.decode_step(*(x[t] for x in dev), state)) for t in range(steps)]
    torch.cuda.synchronize()
    y = np.stack(ys, 1)   # [B, steps, H, N]
    pairs = [(0, 0), (100, 7), (255, 39), (31, 20)]
    seq = [np.ascontiguousarray(np.moveaxis(x, 0, 1)) for x in inp.tensors()]
    sel = [oracle.select_heads(x, pairs) for x in seq]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(y, pairs), yr, "bf16", "decode 2.9b y")
    assert_close(oracle.select_heads(to_np(state), pairs, state=True), sr, "bf16", "decode 2.9b state")


def test_decode_steps_match_sequential_scan_on_gpu(wk):
    import torch
    inp = synth.generate(2, 50, 3, 64, dtype="bf16", seed=12, random_s0=True)
    y, sT, _ = _run_fwd(wk, inp, 0)
    state = to_dev(inp.s0, "fp32")
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    ys = [to_np(wk.decode_step(*(x[:, t].contiguous() for x in dev), state)) for t in range(50)]
    torch.cuda.synchronize()
    np.testing.assert_allclose(np.stack(ys, 1), y, rtol=0, atol=1e-2 * np.abs(y).max())
    np.testing.assert_allclose(to_np(state), sT, rtol=0, atol=1e-5 * np.abs(sT).max())
