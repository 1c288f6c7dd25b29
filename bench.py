#!/usr/bin/env python3
"""WKV7 benchmark on one MI355X: fwd + bwd tokens/s at H=40, N=64, T=4096.

One step is one pass of the whole training hot path over one batch of the
2.9B-model-shaped workload (B=8, T=4096, H=40, N=64, bf16 inputs, fp32 state):
the chunked forward writing its tape (removal read-outs and block entry
states), then the two-pass chunked backward producing dr, dw, dk, dv, da, db
and ds0 (wkv7_backward_overlapped on two streams).  Inputs are seeded
synthetic data resident in HBM before the timed region.  A second timed loop
runs the same kernels one at a time, with HIP events around each launch, for
the per-kernel roofline.  Prints ONE JSON line.

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
# Algorithmic bytes per token-head of each kernel (bf16 token tensors, 128 B per
# vector): the token tensors of the method that the kernel reads and writes;
# the forward tape and the backward workspace are implementation traffic.
FWD_BYTES_PER_TH = 7 * 128          # forward: r, w, k, v, a, b in, y out
ADJ_BYTES_PER_TH = 7 * 128          # adjoint pass: r, w, k, a, b, dy in, dv out
GRAD_BYTES_PER_TH = 12 * 128        # gradient pass: r, w, k, v, a, b, dy in, dr, dw, dk, da, db out
STATE_BYTES = 64 * 64 * 4           # one fp32 state
# Template arguments of each kernel's instance for the general recurrence in one
# launch (not the time-segmented or the a = b = 0 instances).
PLAIN_INSTANCE = {"chunk_fwd_kernel": "<64, false, true, false, false>", "bwd_chain_kernel": "<64, true>",
                  "bwd_keys_kernel": "<64, true>"}
KERNELS = {   # kernel symbol -> (entry point that launches it alone, source, bytes per token-head)
    "chunk_fwd_kernel": ("wkv7_forward", "wkv7_chunk_fwd.hip", FWD_BYTES_PER_TH),
    "bwd_chain_kernel": ("wkv7_backward_adjoint", "wkv7_bwd.hip", ADJ_BYTES_PER_TH),
    "bwd_keys_kernel": ("wkv7_backward_gradients", "wkv7_bwd.hip", GRAD_BYTES_PER_TH),
}
# Algorithmic bytes per token-head of a whole training step: the forward reads
# r, w, k, v, a, b and writes y (7 vectors); the backward reads r, w, k, v, a,
# b, dy and writes the six token gradients (13 vectors).
STEP_BYTES_PER_TH = 20 * 128
BF16_MFMA_PEAK_TFLOPS = 2500.0      # dense bf16 matrix-core peak
PROFILE_JSON = os.path.join(ROOT, "profiles", "hbm_traffic_fwd_bwd_2.9b.json")
SQ_JSON = os.path.join(ROOT, "profiles", "sq_counters_fwd_bwd_2.9b.json")
SQ_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
               "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT",
               "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE")
MOPS_FLOPS = 512                    # SQ_INSTS_VALU_MFMA_MOPS_*: matrix-core work in units of 512 flops
COPY_BYTES = 1 << 30                # calibration copy: 1 GiB read + 1 GiB written


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # 50 timed steps (about 80 ms of device time): the fixed cost of the first
    # launch and the final synchronisation, about half a millisecond, then adds
    # about 1 % to a step instead of several per cent at 10 steps.
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 1 GiB device copy (for scaling HBM counters)")
    p.add_argument("--workload", choices=("step", "chunked_fwd_1.5b", "chunked_fwd_n128",
                                          "sequential_bwd_2.9b"),
                   default="step",
                   help="chunked_fwd_1.5b: time only the chunked forward at the 1.5B-model shape "
                        "(the line under secondary) and print it; chunked_fwd_n128: the same "
                        "at N = 128 over the 1.5B model's channels (H = 16); sequential_bwd_2.9b: the "
                        "sequential reverse pass (checkpointing scan + adjoint) at the 2.9B-model "
                        "shape in bf16, two calls (for counter runs)")
    p.add_argument("--summarize-sq", nargs=5,
                   metavar=("STEP_PMC_DIR", "STEP_STEPS", "CFG_PMC_DIR", "CFG_REPS", "CMD"),
                   help="turn two rocprofv3 --pmc runs of this script (SQ_COUNTERS; the step, "
                        "then --workload chunked_fwd_1.5b) into "
                        "profiles/sq_counters_fwd_bwd_2.9b.{md,json} and exit")
    p.add_argument("--summarize-sq-n128", nargs=3, metavar=("PMC_DIRS", "REPS", "CMD"),
                   help="turn two rocprofv3 --pmc runs of --workload chunked_fwd_n128 (SQ_COUNTERS) "
                        "into profiles/sq_counters_chunked_fwd_n128.md and exit")
    p.add_argument("--summarize-ktrace", nargs=4, metavar=("KTRACE_DIR", "LAST_N", "CMD", "OUT"),
                   help="per-kernel durations of the last LAST_N launches of each kernel in a "
                        "rocprofv3 kernel trace, as a markdown table in OUT; then exit")
    p.add_argument("--summarize-profile", nargs=6,
                   metavar=("KTRACE_DIR", "KTRACE_STEPS", "FETCH_DIR", "WRITE_DIR", "PMC_STEPS", "CMD"),
                   help="turn rocprofv3 outputs of this script into profiles/ summaries and exit "
                        "(*_STEPS: the --steps of those runs; the last that many launches of "
                        "each kernel are the one-at-a-time ones)")
    return p.parse_args()


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "rwkv_wkv7_delta_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_sq(kernel, digest):
    """Matrix-core and LDS figures of `kernel` from the committed SQ-counter
    summary, or None when absent or when the kernel's source changed since."""
    if not os.path.exists(SQ_JSON):
        return None
    with open(SQ_JSON) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_digest") != digest:
        return None
    return k


def load_traffic(kernel, digest):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when absent or when the kernel's source changed since."""
    if not os.path.exists(PROFILE_JSON):
        return None
    with open(PROFILE_JSON) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_digest") != digest:
        return None
    return float(k["hbm_bytes_per_launch"])


def _csv_rows(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _short(name):
    for k in KERNELS:
        # a plain kernel, or the plain instance of a kernel template
        if f"::{k}(" in name or f"::{k}{PLAIN_INSTANCE.get(k, '')}(" in name:
            return k
    return None


def summarize_profile(ktrace_dir, ktrace_steps, fetch_dir, write_dir, pmc_steps, cmd):
    """Write profiles/ summaries from this script's rocprofv3 runs.  Per kernel:
    the --stats line (every launch in the process) and the average over its last
    `steps` launches in the kernel trace, which are the timed one-at-a-time
    launches whose HIP-event durations the roofline uses; FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, last `pmc_steps` launches) scaled by what the
    same counter reads for the 1 GiB calibration copy."""
    ktrace_steps, pmc_steps = int(ktrace_steps), int(pmc_steps)
    stats = {}
    for r in _csv_rows(ktrace_dir, "kernel_stats.csv"):
        k = _short(r["Name"])
        if k:
            stats[k] = {"calls": int(r["Calls"]), "stats_avg_ns": float(r["AverageNs"])}
    launches = {}
    for r in _csv_rows(ktrace_dir, "kernel_trace.csv"):
        k = _short(r["Kernel_Name"])
        if k:
            launches.setdefault(k, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    for k, ls in launches.items():
        ls.sort()
        last = [e - b for b, e in ls[-ktrace_steps:]]
        stats[k].update({"timed_launches": len(last), "avg_ns": float(np.mean(last)),
                         "min_ns": float(min(last)), "max_ns": float(max(last))})
    counters = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        per, copy = {}, []
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            k = _short(r["Kernel_Name"])
            if k:
                per.setdefault(k, []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
            elif "neg_kernel" in r["Kernel_Name"]:
                copy.append(float(r["Counter_Value"]))
        if len(copy) != 1:
            raise SystemExit(f"{cname}: expected one calibration copy, found {len(copy)}")
        counters[cname] = {"per_kernel_kib": {k: float(np.mean([x for _, x in sorted(v)[-pmc_steps:]]))
                                              for k, v in per.items()},
                           "copy_kib": copy[0],
                           "bytes_per_unit": COPY_BYTES / copy[0]}
    os.makedirs(os.path.dirname(PROFILE_JSON), exist_ok=True)
    rec = {"workload": "fwd_bwd_2.9b: B=8 T=4096 H=40 N=64 bf16, chunked L=16, bf16 tape",
           "command": cmd,
           "calibration": {c: {"copy_bytes": COPY_BYTES, "copy_counter_kib": v["copy_kib"],
                               "bytes_per_counter_unit": round(v["bytes_per_unit"], 4)}
                           for c, v in counters.items()},
           "kernels": {}}
    th = 8 * 4096 * 40
    lines = ["# rocprofv3 summary: WKV7 fwd+bwd, B=8 T=4096 H=40 N=64 bf16 (2.9B-model shape)", "",
             "Command (run from the repository root; kernel trace, then one counter pass each):", "",
             "```", cmd, "```", "",
             "The timed columns average each kernel's last launches in the trace: the "
             "one-at-a-time launches of the bench's second timed loop, whose HIP-event "
             "durations the roofline uses (`--stats` averages every launch in the process, "
             "including the two-stream step where the backward's kernels run side by side on "
             "batch-row groups).", "",
             "HBM bytes = counter (KiB per dispatch) x bytes-per-unit of the 1 GiB calibration copy "
             f"(FETCH {counters['FETCH_SIZE']['bytes_per_unit']:.1f}, "
             f"WRITE {counters['WRITE_SIZE']['bytes_per_unit']:.1f} bytes per KiB counted).", "",
             "| kernel | timed launches | avg us | min us | max us | --stats calls / avg us | "
             "HBM read MB | HBM write MB | algorithmic MB | counted / algorithmic |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for k, (entry, src, per_th) in KERNELS.items():
        st = stats.get(k)
        fk = counters["FETCH_SIZE"]["per_kernel_kib"].get(k)
        wk_ = counters["WRITE_SIZE"]["per_kernel_kib"].get(k)
        if st is None or fk is None or wk_ is None:
            continue
        rd = fk * counters["FETCH_SIZE"]["bytes_per_unit"]
        wr = wk_ * counters["WRITE_SIZE"]["bytes_per_unit"]
        alg = th * per_th
        rec["kernels"][k] = {"entry_point": entry, "source": src, "source_digest": src_digest(src),
                             **st, "fetch_kib": fk, "write_kib": wk_,
                             "hbm_read_bytes": round(rd), "hbm_write_bytes": round(wr),
                             "hbm_bytes_per_launch": round(rd + wr),
                             "algorithmic_bytes_per_launch": alg}
        lines.append(f"| {k} | {st['timed_launches']} | {st['avg_ns'] / 1e3:.1f} | "
                     f"{st['min_ns'] / 1e3:.1f} | {st['max_ns'] / 1e3:.1f} | "
                     f"{st['calls']} / {st['stats_avg_ns'] / 1e3:.1f} | {rd / 1e6:.0f} | "
                     f"{wr / 1e6:.0f} | {alg / 1e6:.0f} | {(rd + wr) / alg:.2f} |")
    with open(PROFILE_JSON, "w") as f:
        json.dump(rec, f, indent=1)
    with open(os.path.join(ROOT, "profiles", "kernels_fwd_bwd_2.9b.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _sq_per_kernel(pmc_dir, steps, select):
    """Average per dispatch of every counter over the last `steps` dispatches of
    each kernel that `select(name)` maps to a key (`pmc_dir`: comma-separated
    directories of counter passes over the same program)."""
    per = {}
    for d in pmc_dir.split(","):   # one directory per counter pass
        for r in _csv_rows(d, "counter_collection.csv"):
            k = select(r["Kernel_Name"])
            if k:
                per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                    (int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    out = {}
    for k, cs in per.items():
        out[k] = {}
        for c, vals in cs.items():
            agg = {}
            for did, v in vals:   # one dispatch may report a counter in several rows
                agg[did] = agg.get(did, 0.0) + v
            last = [agg[d] for d in sorted(agg)[-steps:]]
            out[k][c] = float(np.mean(last))
    return out


def summarize_sq(step_dir, step_steps, cfg_dir, cfg_steps, cmd):
    """profiles/sq_counters_fwd_bwd_2.9b.{md,json} from two rocprofv3 --pmc runs
    of this script with SQ_COUNTERS: the training step's three kernels (their
    one-at-a-time launches) and the chunked forward at the 1.5B-model shape."""
    step = _sq_per_kernel(step_dir, int(step_steps), _short)
    cfg = _sq_per_kernel(cfg_dir, int(cfg_steps),
                         lambda n: "chunk_fwd_kernel (1.5B shape)" if "chunk_fwd_kernel" in n else None)
    rec = {"command": cmd, "counters": list(SQ_COUNTERS), "mops_flops": MOPS_FLOPS, "kernels": {}}
    lines = ["# rocprofv3 SQ counters: the training step's kernels (2.9B-model shape) and the "
             "chunked forward (1.5B-model shape)", "",
             "Command (run from the repository root; one counter pass per workload):", "",
             "```", cmd, "```", "",
             "Per dispatch, averaged over the one-at-a-time launches.  MFMA flops = "
             f"SQ_INSTS_VALU_MFMA_MOPS_BF16 x {MOPS_FLOPS}.  Ratios: MFMA busy / CU busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CU_CYCLES; VALU busy / CU busy = "
             "SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES; LDS wait per LDS instruction = "
             "SQ_WAIT_INST_LDS / SQ_INSTS_LDS; bank-conflict cycles per LDS instruction = "
             "SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS.", "",
             "| kernel | MFMA GFLOP / launch | MFMA busy / CU busy | VALU insts (M) | "
             "VALU busy / CU busy | LDS insts (M) | LDS wait / LDS inst | conflict cycles / LDS inst | "
             "GRBM_GUI_ACTIVE |",
             "|---|---|---|---|---|---|---|---|---|"]
    srcs = {k: v[1] for k, v in KERNELS.items()}
    rows = [(k, v, srcs[k]) for k, v in step.items()] + \
           [(k, v, "wkv7_chunk_fwd.hip") for k, v in cfg.items()]
    for k, c, src in rows:
        g = lambda n: c.get(n, float("nan"))
        busy = g("SQ_BUSY_CU_CYCLES")
        nlds = g("SQ_INSTS_LDS")
        flops = g("SQ_INSTS_VALU_MFMA_MOPS_BF16") * MOPS_FLOPS
        rec["kernels"][k] = {"source": src, "source_digest": src_digest(src), "counters": c,
                             "mfma_flops_per_launch": flops,
                             "mfma_busy_over_cu_busy": g("SQ_VALU_MFMA_BUSY_CYCLES") / busy,
                             "valu_busy_over_cu_busy": g("SQ_ACTIVE_INST_VALU") / busy,
                             "lds_wait_per_lds_inst": g("SQ_WAIT_INST_LDS") / nlds,
                             "bank_conflict_cycles_per_lds_inst": g("SQ_LDS_BANK_CONFLICT") / nlds}
        e = rec["kernels"][k]
        lines.append(f"| {k} | {flops / 1e9:.1f} | {e['mfma_busy_over_cu_busy']:.3f} | "
                     f"{g('SQ_INSTS_VALU') / 1e6:.1f} | {e['valu_busy_over_cu_busy']:.3f} | "
                     f"{nlds / 1e6:.1f} | {e['lds_wait_per_lds_inst']:.2f} | "
                     f"{e['bank_conflict_cycles_per_lds_inst']:.3f} | {g('GRBM_GUI_ACTIVE'):.4g} |")
    lines += ["", "Raw averages per dispatch:", "",
              "| kernel | " + " | ".join(SQ_COUNTERS) + " |",
              "|---|" + "---|" * len(SQ_COUNTERS)]
    for k, c, _ in rows:
        lines.append(f"| {k} | " + " | ".join(f"{c.get(n, float('nan')):.4g}" for n in SQ_COUNTERS) + " |")
    with open(SQ_JSON, "w") as f:
        json.dump(rec, f, indent=1)
    with open(os.path.join(ROOT, "profiles", "sq_counters_fwd_bwd_2.9b.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sq_n128(pmc_dirs, reps, cmd):
    """profiles/sq_counters_chunked_fwd_n128.md from the two SQ_COUNTERS passes of
    --workload chunked_fwd_n128: the N = 128 chunked forward's timed launches."""
    c = _sq_per_kernel(pmc_dirs, int(reps),
                       lambda n: "chunk128_fwd_kernel" if "chunk128_fwd_kernel<2, true, false>" in n else None)
    c = c["chunk128_fwd_kernel"]
    g = lambda n: c.get(n, float("nan"))
    busy, nlds = g("SQ_BUSY_CU_CYCLES"), g("SQ_INSTS_LDS")
    flops = g("SQ_INSTS_VALU_MFMA_MOPS_BF16") * MOPS_FLOPS
    lines = ["# rocprofv3 SQ counters: the chunked forward at N = 128 (B=8, T=4096, H=16)", "",
             "Command (run from the repository root; two counter passes):", "",
             "```", cmd, "```", "",
             "Per dispatch, averaged over the timed launches; the ratios as in "
             "sq_counters_fwd_bwd_2.9b.md (busy ratios summed over a compute unit's four SIMDs).", "",
             "| kernel | MFMA GFLOP / launch | MFMA busy / CU busy | VALU insts (M) | VALU busy / CU busy | "
             "LDS insts (M) | LDS wait / LDS inst | conflict cycles / LDS inst | GRBM_GUI_ACTIVE |",
             "|---|---|---|---|---|---|---|---|---|",
             f"| chunk128_fwd_kernel | {flops / 1e9:.1f} | {g('SQ_VALU_MFMA_BUSY_CYCLES') / busy:.3f} | "
             f"{g('SQ_INSTS_VALU') / 1e6:.1f} | {g('SQ_ACTIVE_INST_VALU') / busy:.3f} | {nlds / 1e6:.1f} | "
             f"{g('SQ_WAIT_INST_LDS') / nlds:.2f} | {g('SQ_LDS_BANK_CONFLICT') / nlds:.3f} | "
             f"{g('GRBM_GUI_ACTIVE'):.4g} |", "",
             "| " + " | ".join(SQ_COUNTERS) + " |", "|" + "---|" * len(SQ_COUNTERS),
             "| " + " | ".join(f"{g(n):.4g}" for n in SQ_COUNTERS) + " |"]
    with open(os.path.join(ROOT, "profiles", "sq_counters_chunked_fwd_n128.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_ktrace(ktrace_dir, last_n, cmd, out):
    """Per-kernel durations of the last `last_n` launches in a kernel trace."""
    last_n = int(last_n)
    stats = {r["Name"]: (int(r["Calls"]), float(r["AverageNs"]))
             for r in _csv_rows(ktrace_dir, "kernel_stats.csv")}
    launches = {}
    for r in _csv_rows(ktrace_dir, "kernel_trace.csv"):
        launches.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    lines = ["# rocprofv3 kernel trace", "", "Command (run from the repository root):", "",
             "```", cmd, "```", "",
             f"Durations of each of the library's kernels over its last {last_n} launches (the "
             "timed ones), and the --stats line (every launch in the process); the input "
             "generator's torch kernels are left out.", "",
             "| kernel | launches used | median us | mean us | min us | max us | --stats calls / avg us |",
             "|---|---|---|---|---|---|---|"]
    for name, ls in sorted(launches.items(), key=lambda kv: -len(kv[1])):
        if "wkv7::" not in name:
            continue
        ls.sort()
        d = np.array([e - b for b, e in ls[-last_n:]], dtype=np.float64) / 1e3
        short = name.replace("void ", "").replace("wkv7::(anonymous namespace)::", "").split("(")[0][:70]
        calls, avg = stats.get(name, (0, float("nan")))
        lines.append(f"| {short} | {len(d)} | {np.median(d):.1f} | {d.mean():.1f} | {d.min():.1f} | "
                     f"{d.max():.1f} | {calls} / {avg / 1e3:.1f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def chunked_fwd_15b(torch, wk, dev, reps=25, calls=4):
    """The chunked forward at the 1.5B-model shape (B=8, T=4096, H=32, s0 ~
    0.1 N(0,1), final state returned): `reps` repetitions of `calls` back-to-back
    calls between HIP events on the launch stream (so that the host's launch
    time between calls stays hidden), after three untimed ones; the median per
    call and its spread."""
    B, T, H, N = 8, 4096, 32, 64
    ins = _dev_inputs(torch, (B, T, H, N), dev, 1)
    s0 = 0.1 * torch.randn(B, H, N, N, device=dev)
    y = torch.empty_like(ins[0])
    fn = lambda: wk.forward(*ins, s0, chunk_len=16, out=y)
    for _ in range(3):
        fn()
    t = np.array([_time(torch, fn, calls) for _ in range(reps)])
    ms = float(np.median(t))
    nbytes = B * T * H * FWD_BYTES_PER_TH + 2 * B * H * STATE_BYTES
    return {"workload": "B=8 T=4096 H=32 bf16, s0~0.1N(0,1), L=16, returns sT",
            "reps": reps, "calls_per_rep": calls, "ms": round(ms, 4),
            "ms_p10_p90": [round(float(np.percentile(t, 10)), 4), round(float(np.percentile(t, 90)), 4)],
            "tokens_per_s": round(B * T / ms * 1e3, 1),
            "alg_GBs": round(nbytes / ms / 1e6, 1),
            "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}


def chunked_fwd_n128(torch, wk, dev, reps=25, calls=4):
    """The chunked forward at head size 128 over the 1.5B model's channels
    (B=8, T=4096, H=16 heads of 128, s0 ~ 0.1 N(0,1), final state returned),
    timed as chunked_fwd_15b times the N = 64 shape."""
    B, T, H, N = 8, 4096, 16, 128
    ins = _dev_inputs(torch, (B, T, H, N), dev, 3)
    s0 = 0.1 * torch.randn(B, H, N, N, device=dev)
    y = torch.empty_like(ins[0])
    fn = lambda: wk.forward(*ins, s0, chunk_len=16, out=y)
    for _ in range(3):
        fn()
    t = np.array([_time(torch, fn, calls) for _ in range(reps)])
    ms = float(np.median(t))
    nbytes = B * T * H * 7 * N * 2 + 2 * B * H * N * N * 4
    return {"workload": "B=8 T=4096 H=16 N=128 bf16, s0~0.1N(0,1), L=16, returns sT",
            "reps": reps, "calls_per_rep": calls, "ms": round(ms, 4),
            "ms_p10_p90": [round(float(np.percentile(t, 10)), 4), round(float(np.percentile(t, 90)), 4)],
            "tokens_per_s": round(B * T / ms * 1e3, 1),
            "alg_GBs": round(nbytes / ms / 1e6, 1),
            "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}


def sequential_bwd_29b(torch, wk, dev, calls=2):
    """The sequential reverse pass (chunk_len = 0: the checkpointing scan, then
    the adjoint) at the 2.9B-model shape in bf16, zero s0, dy ~ N(0,1), no ds0:
    `calls` calls, each between HIP events (few, so that a counter run stays
    short); the last call's time."""
    B, T, H, N = 8, 4096, 40, 64
    ins = _dev_inputs(torch, (B, T, H, N), dev, 12)
    g = torch.Generator(device=dev)
    g.manual_seed(13)
    dy = torch.randn(B, T, H, N, device=dev, generator=g).bfloat16()
    desc = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 0)
    ws = torch.empty(wk.workspace_bytes(desc, False) // 4 + 64, device=dev)
    grads = [torch.empty_like(ins[0]) for _ in range(6)]
    ms = 0.0
    for _ in range(calls):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        wk.backward(*ins, dy, None, None, None, chunk_len=0, workspace=ws, grads=grads, want_ds0=False)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
    return {"shape": "B=8 T=4096 H=40 N=64 bf16, zero s0, dy~N(0,1)", "calls": calls,
            "ms": round(ms, 3), "tokens_per_s": round(B * T / ms * 1e3, 1)}


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile)
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
        return
    if args.summarize_ktrace:
        summarize_ktrace(*args.summarize_ktrace)
        return
    if args.summarize_sq_n128:
        summarize_sq_n128(*args.summarize_sq_n128)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU: the kernels work on one GPU's share (B*H heads); --gpus must be 1",
                          "gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import rwkv_wkv7_delta_amd as wk
    from rwkv_wkv7_delta_amd import synth

    wk.lib()   # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.workload == "chunked_fwd_1.5b":
        print(json.dumps({"workload": "chunked_fwd_1.5b", **chunked_fwd_15b(torch, wk, dev)}),
              flush=True)
        return
    if args.workload == "chunked_fwd_n128":
        print(json.dumps({"workload": "chunked_fwd_n128", **chunked_fwd_n128(torch, wk, dev)}),
              flush=True)
        return
    if args.workload == "sequential_bwd_2.9b":
        print(json.dumps({"workload": "sequential_bwd_2.9b", **sequential_bwd_29b(torch, wk, dev)}),
              flush=True)
        return
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

    def call(name, *args):
        st = getattr(L, name)(*args)
        if st != 0:
            raise RuntimeError(f"{name} status {st}")

    def fwd():
        call("wkv7_forward", ctypes.byref(desc), *ptr, None, y.data_ptr(), None, tape.data_ptr(),
             stream.cuda_stream)

    # The step's forward: wkv7_forward_split with the library's own plan (with
    # more heads than compute units, a small last, partial round of heads runs
    # split in time; 320 heads on 256 compute units run whole).
    sws_bytes = wk.split_workspace_bytes(desc, 0)
    sws = torch.empty(max(sws_bytes // 4, 4), device=dev, dtype=torch.float32)

    def fwd_split():
        call("wkv7_forward_split", ctypes.byref(desc), *ptr, None, y.data_ptr(), None,
             tape.data_ptr(), 0, sws.data_ptr(), sws_bytes, stream.cuda_stream)

    bargs = lambda: (ctypes.byref(desc), *ptr, None, dy.data_ptr(), None, tape.data_ptr(),
                     *[g.data_ptr() for g in grads], ds0.data_ptr(), work.data_ptr(), wsb,
                     stream.cuda_stream)

    # The step: the forward, then the whole backward on two streams
    # (wkv7_backward_overlapped: the per-key pass of the first batch rows runs
    # on `aux` beside the adjoint chain of the rest).
    aux = torch.cuda.Stream()

    def bwd_overlapped():
        call("wkv7_backward_overlapped", *bargs(), aux.cuda_stream)

    # The same kernels one at a time (wkv7_backward = wkv7_backward_adjoint +
    # wkv7_backward_gradients), so that each can be timed on its own.
    def bwd_adjoint():
        call("wkv7_backward_adjoint", *bargs())

    def bwd_gradients():
        call("wkv7_backward_gradients", *bargs())

    stages = [("chunk_fwd_kernel", fwd), ("bwd_chain_kernel", bwd_adjoint),
              ("bwd_keys_kernel", bwd_gradients)]
    for _ in range(args.warmup):
        fwd_split()
        bwd_overlapped()
    torch.cuda.synchronize()
    if args.copy_calibration:
        # A plain copy of known size on the same stream, so that HBM counters
        # of a profiled run can be scaled (bytes per counted unit).
        # torch.neg is a plain streaming elementwise kernel (a same-dtype copy_
        # may go to a DMA engine instead of a kernel).
        csrc = torch.empty(COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
        cdst = torch.empty_like(csrc)
        torch.cuda.synchronize()
        torch.neg(csrc, out=cdst)
        torch.cuda.synchronize()
        del csrc, cdst

    # Timed region 1 (the headline): K whole steps, synchronised on both sides.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd_split()
        bwd_overlapped()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms_per_step / 1e3)

    # The step's two halves on their own (HIP events on the launch stream),
    # before the per-kernel loop so that its launches stay the last ones.
    halves = {}
    for name, fn in (("forward_split_ms", fwd_split), ("forward_unsplit_ms", fwd),
                     ("backward_overlapped_ms", bwd_overlapped)):
        halves[name] = round(_time(torch, fn, args.steps), 4)

    # Timed region 2 (per kernel): K steps of the same kernels one at a time, a
    # HIP event on the launch stream around every launch.  These are the last K
    # launches of each kernel in the process (the profile summaries use them).
    for _, fn in stages:
        fn()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, (_, fn) in enumerate(stages):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    kernel_ms = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev]))
                 for i, (name, _) in enumerate(stages)}

    # Roofline of the dominant kernel: algorithmic bytes per launch (per token-head
    # figure x B*T*H token-heads) over its average launch duration.
    th = B * T * H
    per_kernel = {}
    for name, ms in kernel_ms.items():
        entry, src, per_th = KERNELS[name]
        nbytes = th * per_th
        per_kernel[name] = {"entry_point": entry, "ms": round(ms, 4),
                            "algorithmic_bytes": nbytes,
                            "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                            "hbm_bytes_counted": load_traffic(name, src_digest(src))}
    for name, ms in kernel_ms.items():
        sq = load_sq(name, src_digest(KERNELS[name][1]))
        per_kernel[name]["mfma_pct"] = (None if sq is None else round(
            100.0 * sq["mfma_flops_per_launch"] / (ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12), 2))
    dominant = max(kernel_ms, key=kernel_ms.get)
    dk = per_kernel[dominant]
    achieved = dk["achieved_GBs"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": dk["hbm_bytes_counted"], "kernel": dominant,
                "kernel_ms": dk["ms"], "algorithmic_bytes_per_launch": dk["algorithmic_bytes"],
                "kernels": per_kernel,
                "timed_separately": "kernel times from K further steps with the backward's two "
                                    "stages launched one at a time (one kernel per call, HIP "
                                    "events around each); their sum per step: "
                                    f"{staged_ms:.4f} ms",
                "step_parts": halves,
                "mfma_pct": dk["mfma_pct"],
                "mfma_pct_note": "matrix-core flops per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, "
                                 "committed counter summary, null once the kernel's source "
                                 "changed) over the live launch time, against 2.5 PFLOP/s"}
    step_bytes = th * STEP_BYTES_PER_TH
    step_roofline = {"bound": "hbm", "bytes_per_token_head": STEP_BYTES_PER_TH,
                     "achieved": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "note": "the whole step: 7 token vectors through the forward (r, w, k, v, a, "
                             "b in, y out) and 13 through the backward (r, w, k, v, a, b, dy in, "
                             "6 gradients out), 128 bytes each, over ms_per_step"}

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
                               "dy~N(0,1), dsT=0, chunked L=16, bf16 tape; step = wkv7_forward_split "
                               "(automatic plan) + wkv7_backward_overlapped (two streams)",
                   "global_batch": B, "seq_len": T, "heads": H, "head_size": N,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "step_roofline": step_roofline,
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
    N = 64
    res["chunked_fwd_1.5b"] = chunked_fwd_15b(torch, wk, dev)
    # The chunked forward at head size 32 over the same model width as the
    # 1.5B shape (H=64 heads of 32 channels, 512 heads: two workgroups per
    # compute unit).
    B, T, H, N2 = 8, 4096, 64, 32
    ins = _dev_inputs(torch, (B, T, H, N2), dev, 2)
    s0 = 0.1 * torch.randn(B, H, N2, N2, device=dev)
    y = torch.empty_like(ins[0])
    fn = lambda: wk.forward(*ins, s0, chunk_len=16, out=y)
    for _ in range(3):
        fn()
    ms = float(np.median([_time(torch, fn, 4) for _ in range(10)]))
    nbytes = B * T * H * 7 * N2 * 2 + 2 * B * H * N2 * N2 * 4
    res["chunked_fwd_n32"] = {"workload": "B=8 T=4096 H=64 N=32 bf16, s0~0.1N(0,1), L=16, returns sT "
                                          "(median of 10 repetitions of 4 calls)",
                              "ms": round(ms, 4), "tokens_per_s": round(B * T / ms * 1e3, 1),
                              "alg_GBs": round(nbytes / ms / 1e6, 1),
                              "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del ins, s0, y
    # The chunked forward at head size 128: the 1.5B model's channels as 16
    # heads of 128 (each head's rows over two workgroups), 40 heads of 128
    # (320 heads: one workgroup per head), and the 0.19B token shape (48 heads,
    # beside the scan's line at N = 128).
    n128 = {"1.5b_width": chunked_fwd_n128(torch, wk, dev)}
    for name, (B, T, H) in (("h40", (8, 4096, 40)), ("0.19b_tokens", (4, 1024, 12))):
        ins = _dev_inputs(torch, (B, T, H, 128), dev, 3)
        s0 = 0.1 * torch.randn(B, H, 128, 128, device=dev)
        y = torch.empty_like(ins[0])
        # (wkv7_forward_split, automatic plan: at 320 heads the last round's
        # heads split in time; at 48 heads no split)
        d128 = wk.make_desc(B, T, H, 128, wk.WKV7_BF16, 16)
        ws128 = torch.empty(max(wk.split_workspace_bytes(d128, 0) // 4, 4), device=dev)
        fn = lambda: wk.forward(*ins, s0, chunk_len=16, out=y, segments=0, workspace=ws128)
        for _ in range(3):
            fn()
        ms = float(np.median([_time(torch, fn, 4) for _ in range(10)]))
        nbytes = B * T * H * 7 * 128 * 2 + 2 * B * H * 128 * 128 * 4
        n128[name] = {"B": B, "T": T, "H": H, "ms": round(ms, 4),
                      "tokens_per_s": round(B * T / ms * 1e3, 1),
                      "alg_GBs": round(nbytes / ms / 1e6, 1),
                      "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                      "plan_nseg": int(wk.split_plan(d128, 0).nseg)}
        del ins, s0, y, ws128
    # few heads (B=1, T=4096, H=12: 24 workgroups unsplit), split in time by the
    # automatic plan
    B, T, H = 1, 4096, 12
    ins = _dev_inputs(torch, (B, T, H, 128), dev, 4)
    s0 = 0.1 * torch.randn(B, H, 128, 128, device=dev)
    y = torch.empty_like(ins[0])
    desc = wk.make_desc(B, T, H, 128, wk.WKV7_BF16, 16)
    ws = torch.empty(max(wk.split_workspace_bytes(desc, 0) // 4, 4), device=dev)
    few = {}
    for name, seg in (("unsplit_ms", None), ("split_ms", 0)):
        fn = lambda: wk.forward(*ins, s0, chunk_len=16, out=y, segments=seg, workspace=ws)
        for _ in range(3):
            fn()
        few[name] = round(float(np.median([_time(torch, fn, 4) for _ in range(10)])), 4)
    few["segments"] = int(wk.split_plan(desc, 0).nseg)
    few["tokens_per_s"] = round(B * T / few["split_ms"] * 1e3, 1)
    n128["12_heads_split"] = {"B": B, "T": T, "H": H, **few}
    del ins, s0, y, ws
    # the training step at N = 128 (0.19B token shape): the chunked forward
    # writing fp32 checkpoints, then the sequential reverse pass from them
    B, T, H = 4, 1024, 12
    ins = _dev_inputs(torch, (B, T, H, 128), dev, 5)
    dyn = torch.randn(B, T, H, 128, device=dev).bfloat16()
    grads = [torch.empty_like(ins[0]) for _ in range(6)]
    ds0 = torch.empty(B, H, 128, 128, device=dev)

    def step128():
        yv, _, ck = wk.forward(*ins, None, chunk_len=16, want_state=False, want_ckpt=True)
        wk.backward(*ins, dyn, None, None, None, chunk_len=0, ckpt=ck, grads=grads, ds0=ds0)

    for _ in range(2):
        step128()
    ms = float(np.median([_time(torch, step128, 2) for _ in range(5)]))
    n128["train_step_0.19b_tokens"] = {"B": B, "T": T, "H": H, "ms": round(ms, 4),
                                       "tokens_per_s": round(B * T / ms * 1e3, 1),
                                       "note": "wkv7_forward_ckpt (chunked) + wkv7_backward_ckpt "
                                               "(sequential reverse pass), all 7 gradients"}
    del ins, dyn, grads, ds0
    res["chunked_fwd_n128"] = {"workload": "N=128 bf16, s0~0.1N(0,1), L=16, returns sT (1.5b_width: "
                                           "wkv7_forward, median of 25 repetitions of 4 calls; the others "
                                           "of 10; h40, 0.19b_tokens, 12_heads_split: "
                                           "wkv7_forward_split, automatic plan)",
                               **n128}
    # The step after the read-out (current-token term, per-head normalisation,
    # gate) at the 2.9B-model shape: on its own (HBM-bound: y, r, k, v, g read,
    # the result written, 6 x 128 bytes per token-head), and after the chunked
    # forward, as a second kernel or fused into it.
    B, T, H = 8, 4096, 40
    ins = _dev_inputs(torch, (B, T, H, N), dev, 7)
    g = torch.sigmoid(torch.randn(B, T, H, N, device=dev)).bfloat16()
    u, gamma, beta = (torch.randn(H, N, device=dev) * sc + off
                      for sc, off in ((0.5, 0.0), (0.2, 1.0), (0.2, 0.0)))
    y = torch.empty_like(ins[0])
    out = torch.empty_like(ins[0])
    parts = dict(g=g, u=u, gamma=gamma, beta=beta, eps=1e-5, mode=wk.EPI_NORM_TERM)

    def epi_alone():
        wk.epilogue(y, ins[0], ins[2], ins[3], out=out, **parts)

    def fwd_plain():
        wk.forward(*ins, None, chunk_len=16, want_state=False, out=y)

    def fwd_then_epi():
        fwd_plain()
        epi_alone()

    def fwd_fused():
        wk.forward_epilogue(*ins, None, chunk_len=16, want_state=False, out=out, **parts)

    forms = (("epilogue", epi_alone), ("forward", fwd_plain), ("forward_then_epilogue", fwd_then_epi),
             ("forward_epilogue_fused", fwd_fused))
    reps = {name: [] for name, _ in forms}
    for _ in range(3):
        for name, fn in forms:
            reps[name].append(_time(torch, fn, 10))
    med = {name: float(np.median(v)) for name, v in reps.items()}
    epi_bytes = B * T * H * 6 * N * 2
    res["epilogue_2.9b"] = {
        "workload": "B=8 T=4096 H=40 N=64 bf16, mode norm-then-term with u, gamma, beta, g "
                    "(medians of 3 interleaved repetitions of 10 calls)",
        "epilogue_ms": round(med["epilogue"], 4),
        "epilogue_alg_GBs": round(epi_bytes / med["epilogue"] / 1e6, 1),
        "epilogue_frac_hbm": round(epi_bytes / med["epilogue"] / 1e6 / HBM_PEAK_GBS, 4),
        "forward_ms": round(med["forward"], 4),
        "forward_then_epilogue_ms": round(med["forward_then_epilogue"], 4),
        "forward_epilogue_fused_ms": round(med["forward_epilogue_fused"], 4)}
    del ins, g, u, gamma, beta, y, out, parts
    # a = b = 0 (the decay-only recurrence, a and b passed as NULL) at the
    # 2.9B-model shape: the specialised forward (library's split plan, with its
    # tape) and the overlapped backward (no da, db).
    B, T, H = 8, 4096, 40
    ins = _dev_inputs(torch, (B, T, H, N), dev, 5)[:4]
    dy = torch.randn(B, T, H, N, device=dev).bfloat16()
    aux = torch.cuda.Stream()
    fdesc = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16)
    tape = torch.empty(wk.tape_bytes(fdesc) // 2, device=dev, dtype=torch.bfloat16)
    fws = torch.empty(max(wk.split_workspace_bytes(fdesc, 0) // 4, 4), device=dev)
    bws = torch.empty(wk.workspace_bytes(fdesc, True) // 4, device=dev)
    y = torch.empty_like(ins[0])
    grads = [torch.empty_like(ins[0]) for _ in range(4)] + [None, None]

    def fwd0():
        wk.forward(*ins, None, None, None, chunk_len=16, want_state=False, out=y,
                   segments=0, workspace=fws, tape_out=tape)

    def step0():
        fwd0()
        wk.backward(*ins, None, None, dy, None, None, tape, want_ds0=False, workspace=bws,
                    grads=grads, aux_stream=aux)

    ms_f = _time(torch, fwd0, 10)
    ms = _time(torch, step0, 10)
    res["fwd_bwd_decay_only_2.9b"] = {
        "workload": "B=8 T=4096 H=40 bf16, a = b = 0 (NULL), zero s0, split forward with tape "
                    "+ overlapped backward (dr, dw, dk, dv)",
        "ms": round(ms, 4), "tokens_per_s": round(B * T / ms * 1e3, 1),
        "forward_ms": round(ms_f, 4),
        "forward_alg_GBs": round(B * T * H * 5 * 128 / ms_f / 1e6, 1)}
    del ins, dy, tape, fws, bws, y, grads
    # The 0.19B-model shape: few heads (48), so the T-long serial chain sets the
    # time (latency, not bandwidth); both forms of the forward.
    B, T, H = 4, 1024, 12
    ins = _dev_inputs(torch, (B, T, H, N), dev, 3)
    y = torch.empty_like(ins[0])
    # Calls through the C ABI with prepared arguments: at tens of microseconds
    # per call the binding's own checks would otherwise be part of the time.
    import ctypes
    L = wk.lib()
    ptr = [x.data_ptr() for x in ins]
    stream = torch.cuda.current_stream().cuda_stream
    sdesc = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 16)
    qdesc = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 0)

    def split_call(d):
        nbytes = wk.split_workspace_bytes(d, 0)
        ws = torch.empty(max(nbytes // 4, 4), device=dev)

        def fn():
            if L.wkv7_forward_split(ctypes.byref(d), *ptr, None, y.data_ptr(), None, None, 0,
                                    ws.data_ptr(), nbytes, stream) != 0:
                raise RuntimeError("wkv7_forward_split failed")
        fn.split = True
        return fn

    def plain_call(d):
        def fn():
            if L.wkv7_forward(ctypes.byref(d), *ptr, None, y.data_ptr(), None, None, stream) != 0:
                raise RuntimeError("wkv7_forward failed")
        return fn

    forms = (("chunked_split_fwd_0.19b", 16, split_call(sdesc)),
             ("chunked_fwd_0.19b", 16, plain_call(sdesc)),
             ("sequential_fwd_0.19b", 0, plain_call(qdesc)))
    reps = {name: [] for name, _, _ in forms}
    for _ in range(3):   # interleaved repetitions; the median is reported
        for name, _, fn in forms:
            reps[name].append(_time(torch, fn, 20))
    for name, cl, fn in forms:
        ms = float(np.median(reps[name]))
        form = (f"chunk_len={cl}, wkv7_forward_split, automatic plan (every head in time "
                "segments)" if getattr(fn, "split", False) else f"chunk_len={cl}")
        res[name] = {"workload": f"B=4 T=1024 H=12 bf16, zero s0, {form}",
                     "ms": round(ms, 4), "tokens_per_s": round(B * T / ms * 1e3, 1),
                     "us_per_16_tokens": round(ms * 1e3 / (T / 16), 3)}
    del ins, y
    # One sequence of 4096 tokens, 12 heads: the scan's serial chain alone, and
    # split in time by the library's plan.
    B, T, H = 1, 4096, 12
    ins = _dev_inputs(torch, (B, T, H, N), dev, 5)
    y = torch.empty_like(ins[0])
    ptr = [x.data_ptr() for x in ins]
    qdesc = wk.make_desc(B, T, H, N, wk.WKV7_BF16, 0)
    forms = (("sequential_split_fwd_12_heads", split_call(qdesc)),
             ("sequential_fwd_12_heads", plain_call(qdesc)))
    reps = {name: [] for name, _ in forms}
    for _ in range(3):
        for name, fn in forms:
            reps[name].append(_time(torch, fn, 20))
    for name, fn in forms:
        ms = float(np.median(reps[name]))
        form = ", wkv7_forward_split, automatic plan" if getattr(fn, "split", False) else ""
        res[name] = {"workload": f"B=1 T=4096 H=12 bf16, zero s0, chunk_len=0{form}",
                     "ms": round(ms, 4), "tokens_per_s": round(B * T / ms * 1e3, 1)}
    del ins, y, forms

    # Decode steps through the C ABI with prepared arguments: a step takes tens
    # of microseconds on the device, the binding's own checks about as long.
    def decode_steps(Bn, Hn, Nn, inputs, st, yd, nsteps):
        ptrs = [[x[t].data_ptr() for x in inputs] for t in range(nsteps)]
        sp, yp = st.data_ptr(), yd.data_ptr()

        def fn():
            for t in range(nsteps):
                if L.wkv7_decode_step(Bn, Hn, Nn, wk.WKV7_BF16, *ptrs[t], sp, yp, stream) != 0:
                    raise RuntimeError("wkv7_decode_step failed")
        return fn

    Bd, Hd, steps = 256, 40, 512
    st = 0.1 * torch.randn(Bd, Hd, N, N, device=dev)
    seq = _dev_inputs(torch, (steps, Bd, Hd, N), dev, 2)
    yd = torch.empty(Bd, Hd, N, device=dev, dtype=torch.bfloat16)
    run_all = decode_steps(Bd, Hd, N, seq, st, yd, steps)

    ms = _time(torch, run_all, 1)
    per_step = ms / steps
    nbytes = Bd * Hd * (2 * STATE_BYTES + FWD_BYTES_PER_TH)
    res["decode_2.9b"] = {"workload": "B=256 H=40, 512 in-place steps, fp32 state, bf16 inputs",
                          "us_per_step": round(per_step * 1e3, 2),
                          "tokens_per_s": round(Bd / per_step * 1e3, 1),
                          "alg_GBs": round(nbytes / per_step / 1e6, 1),
                          "note": "the 168 MB state fits the 256 MB Infinity Cache"}
    del st, seq, yd
    # B=512: the 335 MB of state no longer fits the 256 MB cache (HBM-bound).
    Bd2 = 512
    st = 0.1 * torch.randn(Bd2, Hd, N, N, device=dev)
    one = _dev_inputs(torch, (8, Bd2, Hd, N), dev, 4)
    yd = torch.empty(Bd2, Hd, N, device=dev, dtype=torch.bfloat16)

    per_step = _time(torch, decode_steps(Bd2, Hd, N, one, st, yd, 8), 5) / 8
    nbytes = Bd2 * Hd * (2 * STATE_BYTES + FWD_BYTES_PER_TH)
    res["decode_b512"] = {"workload": "B=512 H=40, in-place steps, fp32 state, bf16 inputs",
                          "us_per_step": round(per_step * 1e3, 2),
                          "tokens_per_s": round(Bd2 / per_step * 1e3, 1),
                          "alg_GBs": round(nbytes / per_step / 1e6, 1),
                          "frac_hbm": round(nbytes / per_step / 1e6 / HBM_PEAK_GBS, 4)}
    del st, one, yd
    # Other head sizes at the same 168 MB of state: N = 128 (B = 64) and N = 32 (B = 1024).
    for Nn, Bn in ((128, 64), (32, 1024)):
        st = 0.1 * torch.randn(Bn, Hd, Nn, Nn, device=dev)
        one = _dev_inputs(torch, (8, Bn, Hd, Nn), dev, 6)
        yd = torch.empty(Bn, Hd, Nn, device=dev, dtype=torch.bfloat16)

        per_step = _time(torch, decode_steps(Bn, Hd, Nn, one, st, yd, 8), 5) / 8
        nbytes = Bn * Hd * (2 * Nn * Nn * 4 + 7 * Nn * 2)
        res[f"decode_n{Nn}"] = {"workload": f"B={Bn} H=40 N={Nn}, in-place steps, fp32 state, bf16 inputs",
                                "us_per_step": round(per_step * 1e3, 2),
                                "tokens_per_s": round(Bn / per_step * 1e3, 1),
                                "alg_GBs": round(nbytes / per_step / 1e6, 1)}
        del st, one, yd
    # The sequential reverse pass (chunk_len = 0) on the 0.19B-model shape, fp32 inputs.
    ins = [x.float() for x in _dev_inputs(torch, (4, 1024, 12, N), dev, 8)]
    dyf = torch.randn(4, 1024, 12, N, device=dev)
    sdesc = wk.make_desc(4, 1024, 12, N, wk.WKV7_F32, 0)
    sws = torch.empty(wk.workspace_bytes(sdesc, False) // 4, device=dev)
    sgr = [torch.empty_like(ins[0]) for _ in range(6)]
    ms = _time(torch, lambda: wk.backward(*ins, dyf, None, None, None, chunk_len=0, workspace=sws,
                                          grads=sgr, want_ds0=False), 3)
    res["sequential_bwd_0.19b_fp32"] = {
        "workload": "B=4 T=1024 H=12 N=64 fp32, zero s0, dy~N(0,1): checkpointing scan + reverse pass",
        "ms": round(ms, 4), "tokens_per_s": round(4 * 1024 / ms * 1e3, 1)}
    del ins, dyf, sws, sgr
    # The sequential scan with many heads: the 1.5B-model shape (256 heads, 16 lanes
    # per state row) and 512 heads (4 lanes per state row).
    for name, (Bs, Ts, Hs) in (("sequential_fwd_1.5b", (8, 4096, 32)),
                               ("sequential_fwd_512_heads", (16, 2048, 32))):
        ins = _dev_inputs(torch, (Bs, Ts, Hs, N), dev, 9)
        y = torch.empty_like(ins[0])
        qd = wk.make_desc(Bs, Ts, Hs, N, wk.WKV7_BF16, 0)
        qp = [x.data_ptr() for x in ins]

        def scan():
            if L.wkv7_forward(ctypes.byref(qd), *qp, None, y.data_ptr(), None, None, stream) != 0:
                raise RuntimeError("wkv7_forward failed")

        ms = _time(torch, scan, 5)
        res[name] = {"workload": f"B={Bs} T={Ts} H={Hs} N=64 bf16, zero s0, chunk_len=0",
                     "ms": round(ms, 4), "tokens_per_s": round(Bs * Ts / ms * 1e3, 1)}
        del ins, y
    # The sequential scan at N = 128 and N = 32 on the 0.19B-model token shape.
    for Nn in (128, 32):
        ins = _dev_inputs(torch, (4, 1024, 12, Nn), dev, 7)
        y = torch.empty_like(ins[0])
        ms = _time(torch, lambda: wk.forward(*ins, None, chunk_len=0, want_state=False, out=y), 10)
        res[f"sequential_fwd_n{Nn}"] = {"workload": f"B=4 T=1024 H=12 N={Nn} bf16, zero s0, chunk_len=0",
                                        "ms": round(ms, 4), "tokens_per_s": round(4 * 1024 / ms * 1e3, 1)}
        del ins, y
    # The scan split in time by the library's plan at N = 32 (0.19B token shape:
    # 48 heads, 96 workgroups) and N = 128 (B=1 T=2048 H=4), each beside its
    # unsplit time on the same inputs.
    for Nn, (Bs, Ts, Hs) in ((32, (4, 1024, 12)), (128, (1, 2048, 4))):
        ins = _dev_inputs(torch, (Bs, Ts, Hs, Nn), dev, 8)
        y = torch.empty_like(ins[0])
        ms = {seg: _time(torch, lambda: wk.forward(*ins, None, chunk_len=0, want_state=False, out=y,
                                                   segments=seg), 10) for seg in (1, 0)}
        res[f"sequential_split_fwd_n{Nn}"] = {
            "workload": f"B={Bs} T={Ts} H={Hs} N={Nn} bf16, zero s0, chunk_len=0, "
                        "wkv7_forward_split, automatic plan (both times through the binding)",
            "ms": round(ms[0], 4), "tokens_per_s": round(Bs * Ts / ms[0] * 1e3, 1),
            "unsplit_ms": round(ms[1], 4)}
        del ins, y
    return res


def cpu_baseline(inp, wl, grads, y, ds0):
    """fp64 oracle (test infrastructure) on the same workload (all heads, full
    T: a few seconds on the host's cores); also checks the GPU outputs against it."""
    import oracle
    from tests._util import maxrel, cosine
    threads = len(os.sched_getaffinity(0))   # every core this process may run on
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
