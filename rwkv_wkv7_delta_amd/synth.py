"""Seeded synthetic inputs shaped like RWKV-7 WKV7 tensors.

This module only draws and rounds inputs; it contains none of the recurrence's
arithmetic, so both the fp64 oracle (test infrastructure) and the HIP path can
consume its arrays bit-for-bit.

Recipe (the five workloads of the WKV7 hot path; RWKV-7 "Goose" pages, P2
Abstract and P5 Architecture describe vector decay, a per-channel in-context
learning rate and separate removal / replacement keys):

* ``r, k, v ~ N(0, 1)``                      (receptance, replacement key, value)
* ``w = exp(-0.6065 * sigmoid(u))``, ``u ~ N(0, 1)``   (decay in (0.5453, 1))
* ``kappa = normalise(N(0, 1)^N)`` per (b, t, h) token-head (removal key)
* ``alpha = sigmoid(N(0, 1))`` per element (in-context learning rate)
* ``a = -kappa``, ``b = kappa * alpha``
* ``s0 ~ 0.1 * N(0, 1)`` where the workload has a random initial state
* ``dy ~ N(0, 1)``, ``dsT = 0`` for the backward workload

Draw order from ``numpy.random.default_rng(seed)`` (PCG64): r, k, v, u, kappa,
alpha_raw, then s0 (if any), then dy (if any).  Everything is drawn in fp64,
rounded to fp32 (round-to-nearest-even) and, for bf16 workloads, rounded again
fp32 -> bf16 (RNE).  The returned arrays are fp32 holding exactly those
rounded values, so upcasting them to fp64 is exact.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

DECAY_SCALE = 0.6065


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round an fp32 array to the nearest bfloat16 value (ties to even).

    Returns fp32 values that are exactly representable in bf16.  Inputs are
    finite here; NaN handling is not needed for synthetic data.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


@dataclass
class Workload:
    """A named shape + dtype + options, one of the WKV7 workloads."""

    name: str
    B: int
    T: int
    H: int
    N: int = 64
    dtype: str = "bf16"          # "fp32" or "bf16": dtype of r,w,k,v,a,b,y and gradients
    random_s0: bool = False      # s0 ~ 0.1 N(0,1) instead of zeros
    backward: bool = False       # also draw dy (dsT = 0)
    chunk_len: int = 0           # 0 = sequential scan, else chunked form
    decode_steps: int = 0        # >0: decode workload, T is the step count
    notes: str = ""


# The five workloads of the WKV7 hot path.  Index 0 is small enough for the
# oracle to finish in well under a second.
WORKLOADS: Dict[str, Workload] = {
    "fwd_fp32_small": Workload("fwd_fp32_small", B=1, T=64, H=2, dtype="fp32"),
    "fwd_0.19b": Workload("fwd_0.19b", B=4, T=1024, H=12, dtype="bf16"),
    "chunked_fwd_1.5b": Workload("chunked_fwd_1.5b", B=8, T=4096, H=32, dtype="bf16",
                                 random_s0=True, chunk_len=16),
    "fwd_bwd_2.9b": Workload("fwd_bwd_2.9b", B=8, T=4096, H=40, dtype="bf16",
                             backward=True, chunk_len=16),
    "decode_2.9b": Workload("decode_2.9b", B=256, T=512, H=40, dtype="bf16",
                            random_s0=True, decode_steps=512),
}


@dataclass
class Inputs:
    r: np.ndarray
    w: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    s0: Optional[np.ndarray] = None
    dy: Optional[np.ndarray] = None
    dsT: Optional[np.ndarray] = None
    dtype: str = "fp32"
    meta: dict = field(default_factory=dict)

    def tensors(self):
        return (self.r, self.w, self.k, self.v, self.a, self.b)


def generate(B: int, T: int, H: int, N: int = 64, *, dtype: str = "fp32", seed: int = 0,
             random_s0: bool = False, backward: bool = False,
             token_shape: Optional[tuple] = None) -> Inputs:
    """Draw one workload's inputs.

    ``token_shape`` overrides the token-tensor shape (default ``(B, T, H, N)``);
    the decode workload uses ``(T, B, H, N)`` = one ``[B, H, N]`` slice per step.
    """
    if dtype not in ("fp32", "bf16"):
        raise ValueError(f"dtype must be fp32 or bf16, got {dtype!r}")
    shape = tuple(token_shape) if token_shape is not None else (B, T, H, N)
    if shape[-1] != N:
        raise ValueError("last dimension of token_shape must be N")
    rng = np.random.default_rng(seed)

    def rnd(x: np.ndarray) -> np.ndarray:
        x32 = x.astype(np.float32)
        return round_to_bf16(x32) if dtype == "bf16" else x32

    r = rnd(rng.standard_normal(shape))
    k = rnd(rng.standard_normal(shape))
    v = rnd(rng.standard_normal(shape))
    u = rng.standard_normal(shape)
    w = rnd(np.exp(-DECAY_SCALE * _sigmoid(u)))
    del u
    kappa = rng.standard_normal(shape)
    kappa /= np.linalg.norm(kappa, axis=-1, keepdims=True)
    alpha = _sigmoid(rng.standard_normal(shape))
    a = rnd(-kappa)
    b = rnd(kappa * alpha)
    del kappa, alpha
    s0 = None
    if random_s0:
        s0 = (0.1 * rng.standard_normal((B, H, N, N))).astype(np.float32)
    dy = dsT = None
    if backward:
        dy = rnd(rng.standard_normal(shape))
        dsT = np.zeros((B, H, N, N), dtype=np.float32)
    return Inputs(r=r, w=w, k=k, v=v, a=a, b=b, s0=s0, dy=dy, dsT=dsT, dtype=dtype,
                  meta=dict(B=B, T=T, H=H, N=N, seed=seed, shape=shape))


def generate_workload(wl: Workload, seed: int = 0, *, T: Optional[int] = None,
                      B: Optional[int] = None) -> Inputs:
    """Inputs for a named workload; ``T``/``B`` may shrink it (same recipe)."""
    TT = wl.T if T is None else T
    BB = wl.B if B is None else B
    if wl.decode_steps:
        return generate(BB, TT, wl.H, wl.N, dtype=wl.dtype, seed=seed, random_s0=True,
                        token_shape=(TT, BB, wl.H, wl.N))
    return generate(BB, TT, wl.H, wl.N, dtype=wl.dtype, seed=seed,
                    random_s0=wl.random_s0, backward=wl.backward)


# ---------------------------------------------------------------------------
# Special-case inputs: the regimes the pages single out.  As above, these only
# draw and round inputs.
# ---------------------------------------------------------------------------

EDGE_KINDS = ("linear", "replace", "correlated", "swap", "steep_decay", "dyadic")

# Smallest decay the chunked form is asked to take: w^16 = 1e-28 (the chunk
# algebra divides by running products of 16 decays).
STEEP_DECAY = float(np.exp(np.log(1e-28) / 16))


def generate_edge(kind: str, B: int, T: int, H: int, N: int = 64, *, dtype: str = "bf16",
                  seed: int = 0, random_s0: bool = True, backward: bool = False,
                  pool: int = 3) -> Inputs:
    """Inputs for one special regime (``kind`` in ``EDGE_KINDS``), shape [B, T, H, N].

    * ``linear``: w = 1 and a = b = 0 (linear attention: "Paper Review: RWKV-7
      Goose", Background information on delta rule); r, k, v ~ N(0, 1).
    * ``replace``: w = 1, alpha = 1, k = kappa (write key = unit removal key),
      with kappa drawn per token from ``pool`` unit keys per head, so keys repeat
      inside every chunk (exact value replacement: "RWKV-7 Goose with Expressive
      Dynamic State Evolution", Abstract).
    * ``correlated``: removal keys with cosine about 0.8 to a shared direction
      per head, alpha in [0.9, 1], w in [0.95, 1], k ~ N(0, 1).
    * ``swap``: w = 1, alpha = 2 and kappa = (e_i - e_j) / sqrt(2) for random
      i != j per token, so the transition swaps two key columns ("copy" state
      transitions: "Paper Review", Architecture).
    * ``steep_decay``: a quarter of the channels decay at STEEP_DECAY (w^16 =
      1e-28, the edge of the chunked form's domain), the rest as in ``generate``.
    * ``dyadic``: every entry of r, k, v, a, b in {0, +-1/2, +-1} (a and b with
      two non-zeros per token), w in {1/2, 1}, s0 in {0, +-1/2}: sums of such
      values are exact in fp32 while they stay small.
    Draw order (PCG64 ``seed``): r, k, v, then the kind's own draws, then s0, dy.
    """
    if kind not in EDGE_KINDS:
        raise ValueError(f"kind must be one of {EDGE_KINDS}")
    shape = (B, T, H, N)
    rng = np.random.default_rng(seed)

    def rnd(x: np.ndarray) -> np.ndarray:
        x32 = np.asarray(x).astype(np.float32)
        return round_to_bf16(x32) if dtype == "bf16" else x32

    def unit(x: np.ndarray) -> np.ndarray:
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    if kind == "dyadic":
        vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0])
        r = vals[rng.integers(0, 5, shape)]
        k = vals[rng.integers(0, 5, shape)]
        v = vals[rng.integers(0, 5, shape)]
        w = np.where(rng.random(shape) < 0.5, 0.5, 1.0)
        a = np.zeros(shape)
        b = np.zeros(shape)
        idx = rng.integers(0, N, shape[:-1] + (2,))
        sgn = vals[rng.integers(1, 5, shape[:-1] + (4,))]
        np.put_along_axis(a, idx, sgn[..., :2], axis=-1)
        np.put_along_axis(b, idx[..., ::-1], sgn[..., 2:], axis=-1)
    else:
        r = rng.standard_normal(shape)
        k = rng.standard_normal(shape)
        v = rng.standard_normal(shape)
        if kind == "linear":
            w = np.ones(shape)
            a = np.zeros(shape)
            b = np.zeros(shape)
        elif kind == "replace":
            keys = unit(rng.standard_normal((B, H, pool, N)))
            pick = rng.integers(0, pool, (B, T, H))
            kappa = keys[np.arange(B)[:, None, None], np.arange(H)[None, None, :], pick]
            w = np.ones(shape)
            a = -kappa
            b = kappa
            k = kappa
        elif kind == "correlated":
            base = unit(rng.standard_normal((B, 1, H, N)))
            kappa = unit(base + 0.55 * unit(rng.standard_normal(shape)))
            alpha = rng.uniform(0.9, 1.0, shape)
            w = rng.uniform(0.95, 1.0, shape)
            a = -kappa
            b = kappa * alpha
        elif kind == "swap":
            i = rng.integers(0, N, (B, T, H))
            j = (i + rng.integers(1, N, (B, T, H))) % N
            kappa = np.zeros(shape)
            np.put_along_axis(kappa, i[..., None], 1.0, axis=-1)
            np.put_along_axis(kappa, j[..., None], -1.0, axis=-1)
            kappa /= np.sqrt(2.0)
            w = np.ones(shape)
            a = -kappa
            b = 2.0 * kappa
        else:  # steep_decay
            u = rng.standard_normal(shape)
            w = np.exp(-DECAY_SCALE * _sigmoid(u))
            w = np.where(rng.random(shape) < 0.25, STEEP_DECAY, w)
            kappa = unit(rng.standard_normal(shape))
            alpha = _sigmoid(rng.standard_normal(shape))
            a = -kappa
            b = kappa * alpha
    s0 = None
    if random_s0:
        if kind == "dyadic":
            s0 = (np.array([0.0, 0.5, -0.5])[rng.integers(0, 3, (B, H, N, N))]).astype(np.float32)
        else:
            s0 = (0.1 * rng.standard_normal((B, H, N, N))).astype(np.float32)
    dy = dsT = None
    if backward:
        dy = rnd(rng.standard_normal(shape))
        dsT = np.zeros((B, H, N, N), dtype=np.float32)
    return Inputs(r=rnd(r), w=rnd(w), k=rnd(k), v=rnd(v), a=rnd(a), b=rnd(b), s0=s0, dy=dy,
                  dsT=dsT, dtype=dtype, meta=dict(B=B, T=T, H=H, N=N, seed=seed, kind=kind))


# ---------------------------------------------------------------------------
# Inputs of the step after the read-out (current-token term, per-head
# normalisation, gate).  The pages give no values for its learned parts; the
# recipe takes a gate in (0, 1) and parts of order one.
# ---------------------------------------------------------------------------

@dataclass
class EpilogueInputs:
    g: np.ndarray       # [B, T, H, N] gate, sigmoid(N(0, 1)), rounded like the tokens
    u: np.ndarray       # [H, N] fp32 current-token weights, 0.5 N(0, 1)
    gamma: np.ndarray   # [H, N] fp32, 1 + 0.2 N(0, 1)
    beta: np.ndarray    # [H, N] fp32, 0.2 N(0, 1)
    y: np.ndarray       # [B, T, H, N] a stand-in read-out, 0.3 + N(0, 1) (mean off zero)


def generate_epilogue(B: int, T: int, H: int, N: int = 64, *, dtype: str = "bf16",
                      seed: int = 0) -> EpilogueInputs:
    """Learned parts (and a stand-in read-out for the step on its own).  Draw
    order (PCG64 ``seed``): g, u, gamma, beta, y; fp64 rounded to fp32, and
    g, y again to bf16 for bf16 workloads."""
    if dtype not in ("fp32", "bf16"):
        raise ValueError(f"dtype must be fp32 or bf16, got {dtype!r}")
    rng = np.random.default_rng(seed)

    def rnd(x: np.ndarray) -> np.ndarray:
        x32 = np.asarray(x).astype(np.float32)
        return round_to_bf16(x32) if dtype == "bf16" else x32

    g = rnd(_sigmoid(rng.standard_normal((B, T, H, N))))
    u = (0.5 * rng.standard_normal((H, N))).astype(np.float32)
    gamma = (1.0 + 0.2 * rng.standard_normal((H, N))).astype(np.float32)
    beta = (0.2 * rng.standard_normal((H, N))).astype(np.float32)
    y = rnd(0.3 + rng.standard_normal((B, T, H, N)))
    return EpilogueInputs(g=g, u=u, gamma=gamma, beta=beta, y=y)
