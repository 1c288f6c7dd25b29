#!/usr/bin/env python3
"""WKV7 benchmark on one MI355X: fwd + bwd tokens/s at H=40, N=64, T=4096.

One step is one pass of the whole training hot path over one batch of the
2.9B-model-shaped workload (B=8, T=4096, H=40, N=64, bf16 inputs, fp32 state):
the chunked forward writing its tape (removal read-outs and chunk entry
states), then the two-pass chunked backward producing dr, dw, dk, dv, da, db
and ds0.  Inputs are seeded synthetic data resident in
HBM before the timed region.  Prints ONE JSON line.

Also measured (reported under "secondary", not the headline): the chunked
forward at the 1.5B-model shape and the single-token decode step at B=256,
H=40, on device-generated inputs of the same distribution.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Algorithmic bytes per token-head (bf16 token tensors, 128 B per vector):
FWD_BYTES_PER_TH = 7 * 128          # r, w, k, v, a, b in + y out
BWD_BYTES_PER_TH = (7 + 6) * 128    # r, w, k, v, a, b, dy in + 6 gradients out
STATE_BYTES = 64 * 64 * 4           # one fp32 state


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--seed", type=int, default=0)
    return p.parse_args()


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "rwkv_wkv7_delta_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file, digest, per_launch_units):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_fwd_bwd_2.9b.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel_file)
    if not k or k.get("source_digest") != digest:
        return None
    return float(k["hbm_bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1",
                          "gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import rwkv_wkv7_delta_amd as wk
    from rwkv_wkv7_delta_amd import synth

    wk.lib()   # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS["fwd_bwd_2.9b"]
    B, T, H, N = wl.B, wl.T, wl.H, wl.N
    t_gen = time.time()
    inp = synth.generate_workload(wl, seed=args.seed)
    ins = [torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in inp.tensors()]
    dy = torch.from_numpy(inp.dy).to(torch.bfloat16).to(dev)
    t_gen = time.time() - t_gen

    desc = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16)
    y = torch.empty_like(ins[0])
    tape = torch.empty(wk.tape_bytes(desc) // 2, device=dev, dtype=torch.bfloat16)
    wsb = wk.workspace_bytes(desc, True)
    work = torch.empty(wsb // 2, device=dev, dtype=torch.bfloat16)
    grads = [torch.empty_like(ins[0]) for _ in range(6)]
    ds0 = torch.empty((B, H, N, N), device=dev, dtype=torch.float32)
    L = wk.lib()
    import ctypes
    ptr = [x.data_ptr() for x in ins]
    stream = torch.cuda.current_stream()

    def fwd():
        st = L.wkv7_forward(ctypes.byref(desc), *ptr, None, y.data_ptr(), None, tape.data_ptr(),
                            stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"wkv7_forward status {st}")

    def bwd():
        st = L.wkv7_backward(ctypes.byref(desc), *ptr, None, dy.data_ptr(), None,
                             tape.data_ptr(), *[g.data_ptr() for g in grads], ds0.data_ptr(),
                             work.data_ptr(), wsb, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"wkv7_backward status {st}")

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        fwd()
        ev[s][1].record(stream)
        bwd()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = wall * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms_per_step / 1e3)

    # Roofline of the dominant kernel (the backward), algorithmic bytes per launch.
    th = B * T * H
    bwd_bytes = th * BWD_BYTES_PER_TH
    fwd_bytes = th * FWD_BYTES_PER_TH
    dominant = "chunk_bwd_kernel" if bwd_ms >= fwd_ms else "chunk_fwd_kernel"
    if dominant == "chunk_bwd_kernel":
        dom_bytes, dom_ms, dom_file = bwd_bytes, bwd_ms, "wkv7_bwd.hip"
    else:
        dom_bytes, dom_ms, dom_file = fwd_bytes, fwd_ms, "wkv7_chunk_fwd.hip"
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = load_traffic(dom_file, src_digest(dom_file), th)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": dominant,
                "kernel_ms": round(dom_ms, 4),
                "fwd_kernel_ms": round(fwd_ms, 4), "bwd_kernel_ms": round(bwd_ms, 4),
                "fwd_achieved_GBs": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1),
                "algorithmic_bytes_per_launch": dom_bytes}

    out = {
        "metric": "WKV7 fwd+bwd tokens/s (H=40,N=64,T=4096) and achieved HBM GB/s / MFMA % peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fwd_bwd_2.9b: B=8 T=4096 H=40 N=64 bf16 inputs, fp32 state, "
                               "dy~N(0,1), dsT=0, chunked L=16, bf16 tape",
                   "global_batch": B, "seq_len": T, "heads": H, "head_size": N,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
    }

    if not args.no_secondary:
        out["secondary"] = secondary(torch, wk, dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, wl, grads, y, ds0)
    out["input_generation_s"] = round(t_gen, 1)
    print(json.dumps(out), flush=True)


def _dev_inputs(torch, shape, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    r, k, v = (torch.randn(shape, device=dev, generator=g).bfloat16() for _ in range(3))
    w = torch.exp(-0.6065 * torch.sigmoid(torch.randn(shape, device=dev, generator=g))).bfloat16()
    kap = torch.nn.functional.normalize(torch.randn(shape, device=dev, generator=g), dim=-1)
    al = torch.sigmoid(torch.randn(shape, device=dev, generator=g))
    return [r, w, k, v, (-kap).bfloat16(), (kap * al).bfloat16()]


def _time(torch, fn, n):
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def secondary(torch, wk, dev):
    res = {}
    B, T, H, N = 8, 4096, 32, 64
    ins = _dev_inputs(torch, (B, T, H, N), dev, 1)
    s0 = 0.1 * torch.randn(B, H, N, N, device=dev)
    y = torch.empty_like(ins[0])
    ms = _time(torch, lambda: wk.forward(*ins, s0, chunk_len=16, out=y), 5)
    nbytes = B * T * H * FWD_BYTES_PER_TH + 2 * B * H * STATE_BYTES
    res["chunked_fwd_1.5b"] = {"workload": "B=8 T=4096 H=32 bf16, s0~0.1N(0,1), L=16, returns sT",
                               "ms": round(ms, 4), "tokens_per_s": round(B * T / ms * 1e3, 1),
                               "alg_GBs": round(nbytes / ms / 1e6, 1),
                               "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del ins, s0, y
    Bd, Hd, steps = 256, 40, 512
    st = 0.1 * torch.randn(Bd, Hd, N, N, device=dev)
    seq = _dev_inputs(torch, (steps, Bd, Hd, N), dev, 2)
    yd = torch.empty(Bd, Hd, N, device=dev, dtype=torch.bfloat16)

    def run_all():
        for t in range(steps):
            wk.decode_step(*(x[t] for x in seq), st, out=yd)

    ms = _time(torch, run_all, 1)
    per_step = ms / steps
    nbytes = Bd * Hd * (2 * STATE_BYTES + FWD_BYTES_PER_TH)
    res["decode_2.9b"] = {"workload": "B=256 H=40, 512 in-place steps, fp32 state, bf16 inputs",
                          "us_per_step": round(per_step * 1e3, 2),
                          "tokens_per_s": round(Bd / per_step * 1e3, 1),
                          "alg_GBs": round(nbytes / per_step / 1e6, 1),
                          "note": "the 168 MB state fits the 256 MB Infinity Cache"}
    return res


def cpu_baseline(inp, wl, grads, y, ds0):
    """fp64 oracle (test infrastructure) on the same workload (all heads, full
    T: a few seconds on 16 host cores); also checks the GPU outputs against it."""
    import oracle
    from tests._util import maxrel, cosine
    threads = min(16, len(os.sched_getaffinity(0)))
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    sel = [oracle.select_heads(x, pairs) for x in inp.tensors()]
    dsel = oracle.select_heads(inp.dy, pairs)
    t0 = time.perf_counter()
    yr, _ = oracle.forward(*sel, nthreads=threads)
    gr = oracle.backward(*sel, None, dsel, nthreads=threads)
    dt = time.perf_counter() - t0
    token_heads = len(pairs) * wl.T
    value = token_heads / wl.H / dt
    worst = {}
    yg = oracle.select_heads(y.float().cpu().numpy(), pairs)
    worst["y"] = maxrel(yg, yr)
    names = ("dr", "dw", "dk", "dv", "da", "db")
    cos_min = cosine(yg, yr)
    for n, g, rr in zip(names, grads, gr[:6]):
        gg = oracle.select_heads(g.float().cpu().numpy(), pairs)
        worst[n] = maxrel(gg, rr)
        cos_min = min(cos_min, cosine(gg, rr))
    dsg = oracle.select_heads(ds0.cpu().numpy(), pairs, state=True)
    worst["ds0"] = maxrel(dsg, gr[6])
    return {"value": round(value, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fwd+bwd of all {len(pairs)} heads of the workload at full T={wl.T}, "
                      f"fp64, {dt:.1f} s wall",
            "parity_on_sample": {"max_rel": {k: float(f"{v:.3e}") for k, v in worst.items()},
                                 "min_cos": round(cos_min, 7),
                                 "pass": bool(max(worst.values()) <= 2e-2 and cos_min >= 0.9999)}}


if __name__ == "__main__":
    main()
