"""GPU parity of the forward split in time (wkv7_forward_split).

Each head's sequence runs as segments, in one of two ways: by maps (segment 0
and the affine maps of the middle segments first, their entry states composed
in fp32, then the remaining segments again with their outputs), or
sequentially (one workgroup per segment, each handing its final state to the
next).  Every result (y, the final state, the tape and gradients computed from
that tape) is compared with the fp64 oracle on the same seeded inputs, to the
bf16 tolerance (max relative error <= 2e-2, cosine >= 0.9999).
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


def _run(wk, inp, segments, want_tape=False):
    import torch
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    y, sT, tape = wk.forward(*dev, s0, chunk_len=16, want_tape=want_tape, segments=segments)
    torch.cuda.synchronize()
    return to_np(y), to_np(sT), tape


def _plan_bytes(wk, inp, segments):
    B, T, H, N = inp.r.shape
    return wk.split_workspace_bytes(wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16), segments)


@pytest.mark.parametrize("segments", [2, 3, 4, 7])
@pytest.mark.parametrize("T", [100, 257, 512])
def test_split_fwd_matches_oracle(wk, segments, T):
    inp = synth.generate(2, T, 3, 64, dtype="bf16", seed=300 + T + segments, random_s0=True)
    assert _plan_bytes(wk, inp, segments) > 0
    y, sT, _ = _run(wk, inp, segments)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", f"split{segments} T={T} y")
    assert_close(sT, sr, "bf16", f"split{segments} T={T} sT")


@pytest.mark.parametrize("segments", [-2, -3, -4, -7])
@pytest.mark.parametrize("T", [100, 257, 512])
def test_sequential_segments_match_oracle(wk, segments, T):
    inp = synth.generate(2, T, 3, 64, dtype="bf16", seed=400 + T - segments, random_s0=True)
    assert _plan_bytes(wk, inp, segments) > 0
    y, sT, _ = _run(wk, inp, segments)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", f"seq{-segments} T={T} y")
    assert_close(sT, sr, "bf16", f"seq{-segments} T={T} sT")


def test_sequential_segments_tape_and_backward(wk):
    """The tape of a sequential split (segments [0, 64), [64, 128), [128, 150))
    against the oracle's prefix states, and gradients computed from it."""
    import torch
    B, T, H = 1, 150, 2
    inp = synth.generate(B, T, H, 64, dtype="bf16", seed=37, random_s0=True, backward=True)
    _, _, tape = _run(wk, inp, -3, want_tape=True)
    z, st = (to_np(x) for x in wk.split_tape(tape, B, T, H, 64))
    xs = inp.tensors()
    prefix = [inp.s0.astype(np.float64)]
    for t in range(1, T):
        prefix.append(oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1])
    zr = np.stack([np.einsum("bhij,bhj->bhi", prefix[t], xs[4][:, t].astype(np.float64))
                   for t in range(T)], axis=1)
    assert_close(z, zr, "bf16", "sequential tape z")
    for m in range((T + 31) // 32):
        assert_close(st[:, :, m], np.swapaxes(prefix[32 * m], -1, -2), "bf16", f"sequential tape state {m}")
    dev = [to_dev(x, "bf16") for x in xs]
    s0 = to_dev(inp.s0, "fp32")
    g = wk.backward(*dev, to_dev(inp.dy, "bf16"), s0, None, tape)
    torch.cuda.synchronize()
    ref = oracle.backward(*xs, inp.s0, inp.dy, None)
    for name, x, rr in zip(("dr", "dw", "dk", "dv", "da", "db", "ds0"), g, ref):
        assert_close(to_np(x), rr, "bf16", f"sequential-tape {name}")


def test_split_fwd_zero_state_and_short_last_segment(wk):
    """T = 193: three segments of 96, 96 and 1 token; zero initial state."""
    inp = synth.generate(1, 193, 2, 64, dtype="bf16", seed=31)
    y, sT, _ = _run(wk, inp, 3)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", "split short last y")
    assert_close(sT, sr, "bf16", "split short last sT")


def test_split_fwd_too_short_to_split(wk):
    """T = 32 cannot take a second segment: the call runs unsplit."""
    inp = synth.generate(1, 32, 2, 64, dtype="bf16", seed=32, random_s0=True)
    assert _plan_bytes(wk, inp, 4) == 0
    y, sT, _ = _run(wk, inp, 4)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", "unsplit y")
    assert_close(sT, sr, "bf16", "unsplit sT")


def test_split_fwd_tape(wk):
    """The tape of a split run: removal read-outs z_t = S_{t-1} a_t and the
    state entering every 32-token block, against the oracle's prefix states
    (segments [0, 32), [32, 64), [64, 75))."""
    B, T, H = 1, 75, 2
    inp = synth.generate(B, T, H, 64, dtype="bf16", seed=33, random_s0=True)
    _, _, tape = _run(wk, inp, 3, want_tape=True)
    z, st = (to_np(x) for x in wk.split_tape(tape, B, T, H, 64))
    xs = inp.tensors()
    prefix = [inp.s0.astype(np.float64)]
    for t in range(1, T):
        prefix.append(oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1])
    zr = np.stack([np.einsum("bhij,bhj->bhi", prefix[t], xs[4][:, t].astype(np.float64))
                   for t in range(T)], axis=1)
    assert_close(z, zr, "bf16", "split tape z")
    for m in range((T + 31) // 32):
        assert_close(st[:, :, m], np.swapaxes(prefix[32 * m], -1, -2), "bf16", f"split tape state {m}")


def test_backward_from_split_tape(wk):
    """Gradients computed from a split forward's tape match the oracle's."""
    import torch
    inp = synth.generate(2, 200, 2, 64, dtype="bf16", seed=34, random_s0=True, backward=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    _, _, tape = wk.forward(*dev, s0, chunk_len=16, want_state=False, want_tape=True, segments=4)
    g = wk.backward(*dev, to_dev(inp.dy, "bf16"), s0, None, tape)
    torch.cuda.synchronize()
    ref = oracle.backward(*inp.tensors(), inp.s0, inp.dy, None)
    for name, x, rr in zip(("dr", "dw", "dk", "dv", "da", "db", "ds0"), g, ref):
        assert_close(to_np(x), rr, "bf16", f"split-tape {name}")


def test_split_fwd_0_19b_automatic(wk):
    """B=4, T=1024, H=12 (0.19B-model shape), zero state, the library's own
    segment count: every head against the oracle."""
    wl = synth.WORKLOADS["fwd_0.19b"]
    inp = synth.generate_workload(wl, seed=0)
    assert _plan_bytes(wk, inp, 0) > 0   # 48 heads fill well under a third of the device
    y, sT, _ = _run(wk, inp, 0)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    assert_close(y, yr, "bf16", "auto split 0.19b y")
    assert_close(sT, sr, "bf16", "auto split 0.19b sT")


def test_split_plan_thresholds(wk):
    """The automatic plan's thresholds on this device (no launch): every head
    split when the heads fill at most a third of the compute units, the last
    partial round split when it fills at most a fifth of them, else none; no
    split when T is too short for two segments of 128 tokens."""
    import torch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count

    def plan(H, T=640):
        d = wk.make_desc(1, T, H, 64, wk.WKV7_BF16, 16)
        p = wk.split_plan(d, 0)
        assert (wk.split_workspace_bytes(d, 0) > 0) == (p.kind == wk.WKV7_SPLIT_MAPS)
        return p.kind, p.split_from

    M, NO = wk.WKV7_SPLIT_MAPS, wk.WKV7_SPLIT_NONE
    assert plan(ncu // 3) == (M, 0)
    assert plan(ncu // 3 + 1) == (NO, ncu // 3 + 1)
    assert plan(ncu) == (NO, ncu)
    assert plan(ncu + ncu // 8) == (M, ncu)
    assert plan(ncu + ncu // 5) == (M, ncu)
    assert plan(ncu + ncu // 4) == (NO, ncu + ncu // 4)
    assert plan(2 * ncu) == (NO, 2 * ncu)
    assert plan(ncu // 4, T=160) == (NO, ncu // 4)
    p = wk.split_plan(wk.make_desc(1, 640, ncu // 8, 64, wk.WKV7_BF16, 16), 0)
    assert p.kind == M and p.nseg >= 2 and p.seg_len % 32 == 0 and (p.nseg - 1) * p.seg_len < 640


def test_split_fwd_partial_last_round(wk):
    """More heads than compute units: the automatic plan splits only the heads
    of the last, partial round.  Sampled heads on both sides of the boundary."""
    import torch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    H = ncu + ncu // 8
    T = 640
    inp = synth.generate(1, T, H, 64, dtype="bf16", seed=35, random_s0=True)
    assert _plan_bytes(wk, inp, 0) > 0
    y, sT, _ = _run(wk, inp, 0)
    pairs = [(0, 0), (0, ncu - 1), (0, ncu), (0, H - 1), (0, ncu + 3)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(y, pairs), yr, "bf16", "tail split y")
    assert_close(oracle.select_heads(sT, pairs, state=True), sr, "bf16", "tail split sT")


def test_sequential_segments_2_9b_shape_sampled(wk):
    """B=8, T=4096, H=40 as 4 sequential segments per head (1280 workgroups,
    each waiting for its head's previous segment): sampled heads against the
    oracle, the whole output against the unsplit forward's."""
    import torch
    B, T, H = 8, 4096, 40
    inp = synth.generate(B, T, H, 64, dtype="bf16", seed=38, random_s0=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    y, sT, _ = wk.forward(*dev, s0, chunk_len=16, segments=-4)
    y1, sT1, _ = wk.forward(*dev, s0, chunk_len=16)
    torch.cuda.synchronize()
    pairs = [(0, 0), (3, 21), (7, 39)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    yn, sn = to_np(y), to_np(sT)
    assert_close(oracle.select_heads(yn, pairs), yr, "bf16", "2.9b sequential y")
    assert_close(oracle.select_heads(sn, pairs, state=True), sr, "bf16", "2.9b sequential sT")
    assert_close(yn, to_np(y1), "bf16", "2.9b sequential vs unsplit y")
    assert_close(sn, to_np(sT1), "bf16", "2.9b sequential vs unsplit sT")


@pytest.mark.parametrize("H", [36, 40])
def test_split_fwd_2_9b_shape_sampled(wk, H):
    """B=8, T=4096 with the automatic plan and the tape: H=40 (the 2.9B-model
    shape, 320 heads, left whole on 256 compute units) and H=36 (288 heads, whose
    32 past the first full round are split there).  Sampled heads against the
    oracle, the whole output and tape against the unsplit forward's."""
    import torch
    B, T = 8, 4096
    inp = synth.generate(B, T, H, 64, dtype="bf16", seed=36)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    y, sT, tape = wk.forward(*dev, None, chunk_len=16, want_tape=True, segments=0)
    y1, sT1, tape1 = wk.forward(*dev, None, chunk_len=16, want_tape=True)
    torch.cuda.synchronize()
    pairs = [(0, 0), (6, 15), (6, 16), (7, H - 1), (7, 2), (7, 4)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, None)
    yn, sn = to_np(y), to_np(sT)
    assert_close(oracle.select_heads(yn, pairs), yr, "bf16", "2.9b split y")
    assert_close(oracle.select_heads(sn, pairs, state=True), sr, "bf16", "2.9b split sT")
    assert_close(yn, to_np(y1), "bf16", "2.9b split vs unsplit y")
    z, st = wk.split_tape(tape, B, T, H, 64)
    z1, st1 = wk.split_tape(tape1, B, T, H, 64)
    assert_close(to_np(z), to_np(z1), "bf16", "2.9b split tape z")
    assert_close(to_np(st), to_np(st1), "bf16", "2.9b split tape states")


def test_tape_into_caller_buffer(wk):
    """forward(tape_out=...) writes the same tape into a caller's buffer, split or not."""
    import torch
    inp = synth.generate(2, 200, 3, 64, dtype="bf16", seed=610, random_s0=True)
    dev = [to_dev(x, "bf16") for x in inp.tensors()]
    s0 = to_dev(inp.s0, "fp32")
    B, T, H, N = inp.r.shape
    nbytes = wk.tape_bytes(wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16))
    for seg in (None, 0, 3):
        _, _, ref = wk.forward(*dev, s0, chunk_len=16, want_tape=True, segments=seg)
        buf = torch.full((nbytes // 2 + 64,), 3.0, device="cuda", dtype=torch.bfloat16)
        _, _, got = wk.forward(*dev, s0, chunk_len=16, tape_out=buf, segments=seg)
        torch.cuda.synchronize()
        assert got.data_ptr() == buf.data_ptr()
        assert torch.equal(buf[:nbytes // 2], ref[:nbytes // 2]), seg
        assert bool((buf[nbytes // 2:] == 3.0).all())   # nothing written past the tape


def test_expired_segment_wait_shows_as_nan(wk, monkeypatch):
    """Sequential segments with the wait forced to expire from the host
    (WKV7_SEGMENT_SPIN_LIMIT=0: no polling, so a segment whose predecessor has
    not yet published gives up at once).  Every kernel still exits normally,
    and no segment is ever silently wrong: each is either the oracle's result or
    entirely NaN, a NaN segment makes every later segment of its head and the
    final state NaN."""
    monkeypatch.setenv("WKV7_SEGMENT_SPIN_LIMIT", "0")
    B, T, H, nseg = 4, 512, 8, 4
    inp = synth.generate(B, T, H, 64, dtype="bf16", seed=78, random_s0=True)
    y, sT, _ = _run(wk, inp, -nseg)
    yr, sr = oracle.forward(*inp.tensors(), inp.s0)
    seg_len = T // nseg
    lost_heads = 0
    for b in range(B):
        for h in range(H):
            lost = False
            for sg in range(nseg):
                blk = y[b, sg * seg_len:(sg + 1) * seg_len, h]
                if np.isnan(blk).all():
                    lost = True
                    continue
                assert not lost, f"head ({b}, {h}) segment {sg} follows a NaN segment but is not NaN"
                assert not np.isnan(blk).any(), f"head ({b}, {h}) segment {sg} partly NaN"
                ref = yr[b, sg * seg_len:(sg + 1) * seg_len, h]
                assert np.abs(blk - ref).max() <= 2e-2 * np.abs(ref).max(), f"head ({b}, {h}) segment {sg}"
            if lost:
                lost_heads += 1
                assert np.isnan(sT[b, h]).all()
            else:
                assert_close(sT[b, h], sr[b, h], "bf16", f"head ({b}, {h}) sT")
    print(f"{lost_heads} of {B * H} heads had a segment whose wait expired")
