"""GPU parity of the chunked forward at head size N = 128 against the fp64 oracle.

The state expansion of "Millions of States: Designing a Scalable MoE
Architecture with RWKV-7 Meta-learner" (Abstract) read as a larger head of the
same recurrence.  At N = 128 the chunked forward splits each head's value rows
over two workgroups, each of which forms the chunk factors itself, and splits
in time by affine maps.  bf16 inputs with an fp32 state: max relative error
<= 2e-2, cosine >= 0.9999.
"""

import numpy as np
import pytest

import oracle
from rwkv_wkv7_delta_amd import synth
from tests._util import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

N = 128
NAMES = ("dr", "dw", "dk", "dv", "da", "db", "ds0")


@pytest.fixture(scope="module")
def wk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rwkv_wkv7_delta_amd as wk
    wk.lib()
    return wk


def _dev(inp, decay_only=False):
    dev = [to_dev(x, inp.dtype) for x in inp.tensors()]
    if decay_only:
        dev[4] = dev[5] = None
    s0 = to_dev(inp.s0, "fp32") if inp.s0 is not None else None
    return dev, s0


def _run(wk, inp, chunk_len=16, decay_only=False, **kw):
    import torch
    dev, s0 = _dev(inp, decay_only)
    y, sT, extra = wk.forward(*dev, s0, chunk_len=chunk_len, **kw)
    torch.cuda.synchronize()
    return to_np(y), to_np(sT), extra


def _ref(inp, decay_only=False):
    r, w, k, v, a, b = inp.tensors()
    if decay_only:
        a, b = np.zeros_like(a), np.zeros_like(b)
    return oracle.forward(r, w, k, v, a, b, inp.s0)


@pytest.mark.parametrize("T", [1, 15, 16, 33, 70, 130, 257])
def test_chunked_forward_ragged(wk, T):
    inp = synth.generate(2, T, 3, N, dtype="bf16", seed=900 + T, random_s0=True)
    y, sT, _ = _run(wk, inp)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", f"N=128 T={T} y")
    assert_close(sT, sr, "bf16", f"N=128 T={T} sT")


@pytest.mark.parametrize("B,H", [(1, 1), (1, 5), (3, 7), (2, 12)])
def test_head_counts_off_the_xcd_groups(wk, B, H):
    """Head counts that leave the last group of eight heads partial (1, 5, 21)
    or fill it (24): every head's two workgroups find their rows."""
    inp = synth.generate(B, 90, H, N, dtype="bf16", seed=910 + B * H, random_s0=True)
    y, sT, _ = _run(wk, inp)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", f"N=128 B={B} H={H} y")
    assert_close(sT, sr, "bf16", f"N=128 B={B} H={H} sT")


def test_zero_state_and_decay_only(wk):
    inp = synth.generate(1, 200, 4, N, dtype="bf16", seed=920)
    for decay_only in (False, True):
        y, sT, _ = _run(wk, inp, decay_only=decay_only)
        yr, sr = _ref(inp, decay_only)
        assert_close(y, yr, "bf16", f"N=128 zero s0 decay_only={decay_only} y")
        assert_close(sT, sr, "bf16", f"N=128 zero s0 decay_only={decay_only} sT")


def test_chunked_matches_scan(wk):
    inp = synth.generate(2, 512, 4, N, dtype="bf16", seed=921, random_s0=True)
    yc, sc, _ = _run(wk, inp, chunk_len=16)
    ys, ss, _ = _run(wk, inp, chunk_len=0)
    assert_close(yc, ys, "bf16", "N=128 chunk vs scan y")
    assert_close(sc, ss, "bf16", "N=128 chunk vs scan sT")


def test_many_heads_several_rounds(wk):
    """B=8, T=256, H=40 (320 heads, 640 workgroups: more than one round on the
    device), every head against the oracle."""
    inp = synth.generate(8, 256, 40, N, dtype="bf16", seed=922, random_s0=True)
    y, sT, _ = _run(wk, inp)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", "N=128 320 heads y")
    assert_close(sT, sr, "bf16", "N=128 320 heads sT")


def test_many_heads_decay_only(wk):
    inp = synth.generate(8, 96, 40, N, dtype="bf16", seed=923, random_s0=True)
    y, sT, _ = _run(wk, inp, decay_only=True)
    yr, sr = _ref(inp, decay_only=True)
    assert_close(y, yr, "bf16", "N=128 320 heads a=b=0 y")
    assert_close(sT, sr, "bf16", "N=128 320 heads a=b=0 sT")


@pytest.mark.parametrize("kind", ["linear", "replace", "correlated", "swap", "steep_decay"])
def test_special_regimes(wk, kind):
    """The pages' regimes (linear attention, exact replacement with repeated
    keys, correlated removal keys, the alpha = 2 swap, decays at the edge of
    the chunked form's domain), T = 300 with a ragged last chunk."""
    inp = synth.generate_edge(kind, 2, 300, 3, N, dtype="bf16", seed=930)
    y, sT, _ = _run(wk, inp)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", f"N=128 {kind} y")
    assert_close(sT, sr, "bf16", f"N=128 {kind} sT")


def test_checkpoints_and_reverse_pass_from_them(wk):
    """wkv7_forward_ckpt through the chunked form: the fp32 state entering every
    16 tokens equals the oracle's prefix states, and the sequential reverse pass
    from those checkpoints gives the oracle's gradients."""
    import torch
    B, T, H = 2, 75, 3
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=940, random_s0=True, backward=True)
    dev, s0 = _dev(inp)
    y, sT, ck = wk.forward(*dev, s0, chunk_len=16, want_ckpt=True)
    torch.cuda.synchronize()
    xs = inp.tensors()
    assert ck.shape == (B, H, (T + 15) // 16, N, N)
    for m, t in enumerate(range(0, T, 16)):
        ref = inp.s0.astype(np.float64) if t == 0 else oracle.forward(*(x[:, :t] for x in xs), inp.s0)[1]
        assert_close(to_np(ck[:, :, m]), ref, "bf16", f"N=128 ckpt {m}")
    yr, sr = oracle.forward(*xs, inp.s0)
    assert_close(to_np(y), yr, "bf16", "N=128 ckpt y")
    dy = to_dev(inp.dy, "bf16")
    g = wk.backward(*dev, dy, s0, None, None, chunk_len=0, ckpt=ck)
    torch.cuda.synchronize()
    gr = oracle.backward(*xs, inp.s0, inp.dy)
    for name, x, rr in zip(NAMES, g, gr):
        assert_close(to_np(x), rr, "bf16", f"N=128 reverse pass from chunked ckpt {name}")


def test_forward_epilogue(wk):
    """chunk_len = 16 at N = 128: the forward, then the step after the read-out in place."""
    import torch
    B, T, H = 2, 100, 3
    inp = synth.generate(B, T, H, N, dtype="bf16", seed=950, random_s0=True)
    e = synth.generate_epilogue(B, T, H, N, dtype="bf16", seed=951)
    dev, s0 = _dev(inp)
    out, sT = wk.forward_epilogue(*dev, s0, to_dev(e.g, "bf16"), to_dev(e.u, "fp32"),
                                  to_dev(e.gamma, "fp32"), to_dev(e.beta, "fp32"), eps=1e-5,
                                  mode=1, chunk_len=16)
    torch.cuda.synchronize()
    yr, sr = _ref(inp)
    ref = oracle.epilogue(yr, inp.r, inp.k, inp.v, e.g, e.u, e.gamma, e.beta, eps=1e-5, mode=1)
    assert_close(to_np(out), ref, "bf16", "N=128 forward + step")
    assert_close(to_np(sT), sr, "bf16", "N=128 forward + step sT")


def test_what_n128_does_not_take(wk):
    """No tape (the chunked backward takes N = 32 and 64), no sequential
    segments, no chunked backward; too short for segments, the automatic
    split plan runs it unsplit."""
    import torch
    inp = synth.generate(1, 64, 2, N, dtype="bf16", seed=960, random_s0=True)
    dev, s0 = _dev(inp)
    desc = wk.make_desc(1, 64, 2, N, wk.WKV7_BF16, 16)
    assert wk.tape_bytes(desc) == 0
    assert wk.workspace_bytes(desc, True) == 0 and wk.workspace_bytes(desc, False) == 0
    assert wk.split_workspace_bytes(desc, 0) == 0
    plan = wk.split_plan(desc, 0)
    assert plan.nseg == 1 and plan.split_from == 2
    with pytest.raises(wk.WKV7Error):
        wk.forward(*dev, s0, chunk_len=16, want_tape=True)
    with pytest.raises(wk.WKV7Error):
        wk.forward(*dev, s0, chunk_len=16, want_tape=True, segments=2)
    with pytest.raises(wk.WKV7Error):
        wk.forward(*dev, s0, chunk_len=16, segments=-2)
    with pytest.raises(wk.WKV7Error):
        wk.split_plan(desc, -2)
    with pytest.raises(wk.WKV7Error):
        wk.backward(*dev, to_dev(inp.r, "bf16"), s0, None, None, chunk_len=16)
    y, sT, _ = _run(wk, inp, segments=0)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", "N=128 automatic plan y")
    assert_close(sT, sr, "bf16", "N=128 automatic plan sT")


@pytest.mark.parametrize("segments", [2, 3, 5])
def test_split_in_time_by_maps(wk, segments):
    """Every head in 2, 3 or 5 time segments by affine maps (ragged T, random
    s0; the composition is the scan's N = 128 kernel)."""
    inp = synth.generate(2, 290, 3, N, dtype="bf16", seed=980 + segments, random_s0=True)
    B, T, H, _ = inp.r.shape
    desc = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16)
    assert wk.split_plan(desc, segments).nseg == segments
    assert wk.split_workspace_bytes(desc, segments) == B * H * 3 * segments * N * N * 4
    y, sT, _ = _run(wk, inp, segments=segments)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", f"N=128 split {segments} y")
    assert_close(sT, sr, "bf16", f"N=128 split {segments} sT")


def test_split_decay_only_and_static_scratch(wk):
    inp = synth.generate(1, 300, 2, N, dtype="bf16", seed=990, random_s0=True)
    y, sT, _ = _run(wk, inp, decay_only=True, segments=3)
    yr, sr = _ref(inp, decay_only=True)
    assert_close(y, yr, "bf16", "N=128 split a=b=0 y")
    assert_close(sT, sr, "bf16", "N=128 split a=b=0 sT")
    y, sT, _ = _run(wk, inp, segments=4, static_scratch=True)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", "N=128 split in the static scratch y")
    assert_close(sT, sr, "bf16", "N=128 split in the static scratch sT")


def test_split_automatic_few_heads(wk):
    """B=1, T=4096, H=12 (24 workgroups unsplit): the library's plan splits
    every head; sampled heads against the oracle, the rest against the unsplit run."""
    inp = synth.generate(1, 4096, 12, N, dtype="bf16", seed=995, random_s0=True)
    desc = wk.make_desc(1, 4096, 12, N, wk.WKV7_BF16, 16)
    plan = wk.split_plan(desc, 0)
    assert plan.nseg >= 2 and plan.split_from == 0
    y, sT, _ = _run(wk, inp, segments=0)
    yu, su, _ = _run(wk, inp)
    assert_close(y, yu, "bf16", "N=128 automatic split vs unsplit y")
    assert_close(sT, su, "bf16", "N=128 automatic split vs unsplit sT")
    pairs = [(0, 0), (0, 7), (0, 11)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(y, pairs), yr, "bf16", "N=128 automatic split y")
    assert_close(oracle.select_heads(sT, pairs, state=True), sr, "bf16", "N=128 automatic split sT")


def test_1_5b_width_sampled(wk):
    """B=8, T=4096, H=16 (the 1.5B model's channels as 128-wide heads: 128
    heads, two workgroups each, the bench's N = 128 workload),
    random s0: sampled heads at full T against the oracle, every output finite."""
    inp = synth.generate(8, 4096, 16, N, dtype="bf16", seed=970, random_s0=True)
    y, sT, _ = _run(wk, inp)
    pairs = [(0, 0), (3, 9), (7, 15)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(y, pairs), yr, "bf16", "N=128 1.5B width y")
    assert_close(oracle.select_heads(sT, pairs, state=True), sr, "bf16", "N=128 1.5B width sT")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(sT))


def test_many_heads_checkpoints(wk):
    """B=8, T=96, H=40 (one workgroup per head): the chunked form's fp32
    checkpoints against the scan's (same layout) and y against the oracle."""
    import torch
    inp = synth.generate(8, 96, 40, N, dtype="bf16", seed=1001, random_s0=True)
    dev, s0 = _dev(inp)
    yc, _, ckc = wk.forward(*dev, s0, chunk_len=16, want_ckpt=True)
    ys, _, cks = wk.forward(*dev, s0, chunk_len=0, want_ckpt=True)
    torch.cuda.synchronize()
    assert_close(to_np(ckc), to_np(cks), "bf16", "N=128 320 heads ckpt vs scan")
    pairs = [(0, 0), (3, 21), (7, 39)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, _ = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(to_np(yc), pairs), yr, "bf16", "N=128 320 heads ckpt run y")


def test_many_heads_split_explicit(wk):
    """B=8, T=256, H=40 in 3 segments by maps: 960 items in the first launch,
    one workgroup each (map runs from the identity with v = 0 and from zero)."""
    inp = synth.generate(8, 256, 40, N, dtype="bf16", seed=1002, random_s0=True)
    y, sT, _ = _run(wk, inp, segments=3)
    yr, sr = _ref(inp)
    assert_close(y, yr, "bf16", "N=128 320 heads split y")
    assert_close(sT, sr, "bf16", "N=128 320 heads split sT")


def test_split_partial_round_automatic(wk):
    """B=8, T=512, H=36 (288 heads: one workgroup each, a last round of 32 on a
    256-compute-unit device): the automatic plan splits the last round's heads
    by maps; all heads against the unsplit run, sampled ones against the oracle."""
    inp = synth.generate(8, 512, 36, N, dtype="bf16", seed=1003, random_s0=True)
    desc = wk.make_desc(8, 512, 36, N, wk.WKV7_BF16, 16)
    plan = wk.split_plan(desc, 0)
    y, sT, _ = _run(wk, inp, segments=0)
    yu, su, _ = _run(wk, inp)
    assert_close(y, yu, "bf16", "N=128 partial-round split vs unsplit y")
    assert_close(sT, su, "bf16", "N=128 partial-round split vs unsplit sT")
    pairs = [(0, 0), (7, 35), (7, 20), (7, 10)]   # (7, 20..35): heads of the split last round
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    yr, sr = oracle.forward(*sel, oracle.select_heads(inp.s0, pairs, state=True))
    assert_close(oracle.select_heads(y, pairs), yr, "bf16", "N=128 partial-round split y")
    assert_close(oracle.select_heads(sT, pairs, state=True), sr, "bf16", "N=128 partial-round split sT")
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert plan.split_from == 256 and plan.nseg >= 2
