"""HIP graph capture of the library's calls.

The entry points launch kernels only (no memset, allocation or synchronising
call inside them), so a caller may capture them in a HIP graph.  Each test
runs a call eagerly, captures the same call (same buffers) into a graph, then
replays the graph several times with the program's own eager work between
the replays (every output overwritten with NaN, a synchronisation), and checks
that every replay reproduces the eager outputs bit for bit: the kernels are
deterministic, and a capture that dropped or froze a step (such as clearing an
output the kernels then accumulate into) would leave NaN or stale values.
"""

import pytest

from rwkv_wkv7_delta_amd import synth
from tests._util import to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def wk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rwkv_wkv7_delta_amd as wk
    wk.lib()
    return wk


def _capture(torch, fn):
    """Warm up fn on a side stream, then capture it; returns the graph and the
    outputs of the captured call (tensors the replays write)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, [o for o in outs if o is not None]


def _check_replays(torch, g, outs, ref, what):
    assert len(outs) == len(ref)
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"{what}: replay {i}, output {j} differs from the eager call"


def _inputs(B, T, H, N, dtype, seed):
    inp = synth.generate(B, T, H, N, dtype=dtype, seed=seed, random_s0=True, backward=True)
    dev = [to_dev(x, dtype) for x in inp.tensors()]
    return dev, to_dev(inp.s0, "fp32"), to_dev(inp.dy, dtype)


def test_graph_chunked_forward_with_tape(wk):
    import torch
    ins, s0, _ = _inputs(2, 200, 5, 64, "bf16", 801)
    fn = lambda: wk.forward(*ins, s0, chunk_len=16, want_tape=True)
    ref = [x.clone() for x in fn() if x is not None]
    g, outs = _capture(torch, fn)
    _check_replays(torch, g, outs, ref, "chunked forward")


def test_graph_chunked_forward_n128_with_ckpt(wk):
    """The chunked forward at N = 128 (two workgroups per head, their factor
    slots in LDS) with fp32 checkpoints."""
    import torch
    ins, s0, _ = _inputs(2, 150, 3, 128, "bf16", 809)
    fn = lambda: wk.forward(*ins, s0, chunk_len=16, want_ckpt=True)
    ref = [x.clone() for x in fn() if x is not None]
    g, outs = _capture(torch, fn)
    _check_replays(torch, g, outs, ref, "chunked forward N = 128")


def test_graph_split_forward_static_scratch(wk):
    """The no-allocation entry with the automatic plan on few heads (time
    segments by maps in the library's static scratch, and their composition)."""
    import torch
    ins, s0, _ = _inputs(1, 640, 4, 64, "bf16", 802)
    d = wk.make_desc(1, 640, 4, 64, wk.WKV7_BF16, 16)
    assert wk.split_plan(d, 0).kind == wk.WKV7_SPLIT_MAPS
    fn = lambda: wk.forward(*ins, s0, chunk_len=16, want_tape=True, segments=0, static_scratch=True)
    ref = [x.clone() for x in fn() if x is not None]
    g, outs = _capture(torch, fn)
    _check_replays(torch, g, outs, ref, "split forward, static scratch")


@pytest.mark.parametrize("T", [150, 640])
def test_graph_chunked_backward(wk, T):
    """T = 640 with 8 heads: the adjoint chain in time segments (two launches
    and the composition of the entry adjoints between them)."""
    import torch
    B, H = 2, 4
    ins, s0, dy = _inputs(B, T, H, 64, "bf16", 803)
    _, _, tape = wk.forward(*ins, s0, chunk_len=16, want_tape=True)
    d = wk.make_desc(B, T, H, 64, wk.WKV7_BF16, 16)
    ws = torch.empty(wk.workspace_bytes(d, True) // 4 + 64, device="cuda")
    fn = lambda: wk.backward(*ins, dy, s0, None, tape, chunk_len=16, workspace=ws)
    ref = [x.clone() for x in fn() if x is not None]
    g, outs = _capture(torch, fn)
    _check_replays(torch, g, outs, ref, "chunked backward")


def test_graph_overlapped_backward_two_streams(wk):
    """More heads than compute units: the backward's two batch-row groups on two
    streams (the second stream joins the capture through the library's events)."""
    import torch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    B, T, H = 2, 64, ncu // 2 + 8
    ins, s0, dy = _inputs(B, T, H, 64, "bf16", 804)
    _, _, tape = wk.forward(*ins, s0, chunk_len=16, want_tape=True)
    d = wk.make_desc(B, T, H, 64, wk.WKV7_BF16, 16)
    ws = torch.empty(wk.workspace_bytes(d, True) // 4 + 64, device="cuda")
    aux = torch.cuda.Stream()
    fn = lambda: wk.backward(*ins, dy, s0, None, tape, chunk_len=16, workspace=ws, aux_stream=aux)
    ref = [x.clone() for x in fn() if x is not None]
    torch.cuda.synchronize()
    one = wk.backward(*ins, dy, s0, None, tape, chunk_len=16)
    torch.cuda.synchronize()
    for x, r in zip([x for x in one if x is not None], ref):
        assert torch.equal(x, r), "two streams and one stream differ"
    g, outs = _capture(torch, fn)
    _check_replays(torch, g, outs, ref, "overlapped backward")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_graph_sequential_backward_n128_two_workgroups(wk, dtype):
    """N = 128 with few heads: each head's rows over two workgroups, whose
    per-key sums are added into outputs that a fill kernel clears first."""
    import torch
    B, T, H, N = 1, 50, 3, 128
    ins, s0, dy = _inputs(B, T, H, N, dtype, 805)
    d = wk.make_desc(B, T, H, N, wk.WKV7_F32 if dtype == "fp32" else wk.WKV7_BF16, 0)
    ws = torch.empty(wk.workspace_bytes(d, False) // 4 + 64, device="cuda")
    fn = lambda: wk.backward(*ins, dy, s0, None, None, chunk_len=0, workspace=ws)
    ref = [x.clone() for x in fn() if x is not None]
    g, outs = _capture(torch, fn)
    _check_replays(torch, g, outs, ref, f"sequential backward N=128 {dtype}")


def test_graph_decode_steps_in_place(wk):
    """The decode step updates the states in place: k replays equal k eager steps."""
    import torch
    B, H, N = 8, 4, 64
    g0 = torch.Generator(device="cuda")
    g0.manual_seed(806)
    r, k, v = (torch.randn(B, H, N, device="cuda", generator=g0).bfloat16() for _ in range(3))
    w = torch.exp(-0.6065 * torch.sigmoid(torch.randn(B, H, N, device="cuda", generator=g0))).bfloat16()
    kap = torch.nn.functional.normalize(torch.randn(B, H, N, device="cuda", generator=g0), dim=-1)
    a, b = (-kap).bfloat16(), (0.5 * kap).bfloat16()
    state0 = 0.1 * torch.randn(B, H, N, N, device="cuda", generator=g0)
    eager = state0.clone()
    ys = []
    for _ in range(REPLAYS + 1):
        ys.append(wk.decode_step(r, w, k, v, a, b, eager).clone())
    torch.cuda.synchronize()
    state = state0.clone()
    y = torch.empty_like(r)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        wk.decode_step(r, w, k, v, a, b, state, out=y)   # warm-up: the first step
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(y, ys[0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wk.decode_step(r, w, k, v, a, b, state, out=y)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ys[i + 1]), f"decode replay {i}"
    assert torch.equal(state, eager)
