"""Shared test helpers: tolerance metrics and device transfer (no method arithmetic)."""

import numpy as np

# Tolerances: max relative error <= 1e-4 for fp32 inputs; <= 2e-2 with cosine
# similarity >= 0.9999 for bf16 inputs with an fp32 state.
TOL = {"fp32": dict(maxrel=1e-4, cos=None), "bf16": dict(maxrel=2e-2, cos=0.9999)}


def maxrel(x, ref):
    """max |x - ref| / max |ref| over the whole tensor (per-tensor relative error)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / den) if den > 0 else float(np.abs(x).max())


def cosine(x, ref):
    x = np.asarray(x, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    nx, nr = np.linalg.norm(x), np.linalg.norm(ref)
    if nx == 0 and nr == 0:
        return 1.0
    return float(np.dot(x, ref) / (nx * nr))


def assert_close(x, ref, dtype, what=""):
    tol = TOL[dtype]
    mr = maxrel(x, ref)
    assert np.all(np.isfinite(np.asarray(x, dtype=np.float64))), f"{what}: non-finite values"
    assert mr <= tol["maxrel"], f"{what}: maxrel {mr:.3e} > {tol['maxrel']}"
    if tol["cos"] is not None:
        c = cosine(x, ref)
        assert c >= tol["cos"], f"{what}: cosine {c:.8f} < {tol['cos']}"
    return mr


def to_dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def to_np(t):
    import torch
    return t.detach().float().cpu().numpy() if t.dtype != torch.float64 else t.cpu().numpy()


def frac_bits(x):
    """Largest number of fractional binary digits among the non-zero entries of x
    (fp64 values; every finite double is a dyadic rational)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    x = x[x != 0]
    if x.size == 0:
        return 0
    m, e = np.frexp(x)
    mi = np.abs(m * 2.0 ** 53).astype(np.int64)
    tz = np.zeros_like(mi)
    t = mi.copy()
    for _ in range(54):
        z = (t & 1) == 0
        if not z.any():
            break
        tz += z
        t = np.where(z, t >> 1, t)
    return int(np.max(53 - e - tz))
