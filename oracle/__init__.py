"""fp64 CPU oracle for the WKV7 recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never calls it and shares no code with it.

Functions take numpy arrays (any float dtype; upcast exactly to fp64) in the
layouts ``[B, T, H, N]`` for token tensors and ``[B, H, N, N]`` for states,
and return fp64 arrays.  The recurrence and its sources on the RWKV-7 pages
are documented in ``wkv7_oracle.c``.

Parity pins (see the CPU tests): linear-attention and decay-only closed
forms, exact value replacement, the DeltaNet SGD step, the Householder swap,
exact rational arithmetic on dyadic inputs, brute-force matrix products,
linearity / permutation invariants, decode = forward, continuation, chunked =
sequential, and central finite differences for the gradients; for the step
after the read-out (``epilogue``), a hand-worked fixture, the two-channel
closed form, the one-hot term, and identity / moment / linearity / gate /
affine / invariance properties.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv7_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain fp64, OpenMP over heads)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.wkv7_oracle_forward.argtypes = [I, I, I, I] + [P] * 6 + [P, P, P, I]
        lib.wkv7_oracle_forward_chunked.argtypes = [I, I, I, I, I] + [P] * 6 + [P, P, P, I]
        lib.wkv7_oracle_decode_step.argtypes = [I, I, I] + [P] * 6 + [P, P, I]
        lib.wkv7_oracle_backward.argtypes = [I, I, I, I] + [P] * 6 + [P, P, P] + [P] * 7 + [I]
        lib.wkv7_oracle_backward_chunked.argtypes = ([I, I, I, I, I] + [P] * 6 + [P, P, P]
                                                     + [P] * 7 + [I])
        lib.wkv7_oracle_epilogue.argtypes = [I, I, I, I] + [P] * 8 + [ctypes.c_double, I, P, I]
        lib.wkv7_oracle_max_threads.restype = I
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().wkv7_oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _shape(r):
    if r.ndim != 4:
        raise ValueError("token tensors must be [B, T, H, N]")
    return r.shape


def forward(r, w, k, v, a, b, s0=None, *, nthreads: int = 0, chunk_len: int = 0):
    """y [B,T,H,N] and final state [B,H,N,N], fp64.

    ``chunk_len > 0`` runs the chunked rearrangement instead (same result up
    to rounding); it exists to pin the chunk algebra.
    """
    lib = _load()
    ins = [_f64(x) for x in (r, w, k, v, a, b)]
    B, T, H, N = _shape(ins[0])
    for x in ins:
        if x.shape != (B, T, H, N):
            raise ValueError("all token tensors must share one shape")
    s0 = _f64(s0)
    if s0 is not None and s0.shape != (B, H, N, N):
        raise ValueError("s0 must be [B, H, N, N]")
    y = np.zeros((B, T, H, N))
    sT = np.zeros((B, H, N, N))
    if chunk_len > 0:
        lib.wkv7_oracle_forward_chunked(B, T, H, N, chunk_len, *map(_ptr, ins), _ptr(s0),
                                        _ptr(y), _ptr(sT), nthreads)
    else:
        lib.wkv7_oracle_forward(B, T, H, N, *map(_ptr, ins), _ptr(s0), _ptr(y), _ptr(sT),
                                nthreads)
    return y, sT


def backward(r, w, k, v, a, b, s0=None, dy=None, dsT=None, *, nthreads: int = 0,
             chunk_len: int = 0):
    """Gradients (dr, dw, dk, dv, da, db, ds0) of <dy, y> + <dsT, S_T>, fp64."""
    lib = _load()
    ins = [_f64(x) for x in (r, w, k, v, a, b)]
    B, T, H, N = _shape(ins[0])
    s0 = _f64(s0)
    dy = _f64(dy) if dy is not None else np.zeros((B, T, H, N))
    dsT = _f64(dsT)
    outs = [np.zeros((B, T, H, N)) for _ in range(6)]
    ds0 = np.zeros((B, H, N, N))
    if chunk_len > 0:
        lib.wkv7_oracle_backward_chunked(B, T, H, N, chunk_len, *map(_ptr, ins), _ptr(s0),
                                         _ptr(dy), _ptr(dsT), *map(_ptr, outs), _ptr(ds0),
                                         nthreads)
    else:
        lib.wkv7_oracle_backward(B, T, H, N, *map(_ptr, ins), _ptr(s0), _ptr(dy), _ptr(dsT),
                                 *map(_ptr, outs), _ptr(ds0), nthreads)
    return tuple(outs) + (ds0,)


def decode_step(r, w, k, v, a, b, state, *, nthreads: int = 0):
    """One token on resident states.  Inputs [B,H,N]; returns (y, new_state)."""
    lib = _load()
    ins = [_f64(x) for x in (r, w, k, v, a, b)]
    B, H, N = ins[0].shape
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    if st.shape != (B, H, N, N):
        raise ValueError("state must be [B, H, N, N]")
    y = np.zeros((B, H, N))
    lib.wkv7_oracle_decode_step(B, H, N, *map(_ptr, ins), _ptr(st), _ptr(y), nthreads)
    return y, st


def epilogue(y, r, k, v, g=None, u=None, gamma=None, beta=None, *, eps: float = 1e-5,
             mode: int = 1, nthreads: int = 0):
    """The step after the read-out (wkv7_oracle.c), fp64: with s = r . (u * k),
    mode 0: g (y + s v); mode 1: g (norm(y) + s v); mode 2: g norm(y + s v).

    Token tensors [B, T, H, N]; u, gamma, beta [H, N]; None means g = 1, u = 0,
    gamma = 1, beta = 0."""
    lib = _load()
    toks = [_f64(x) for x in (y, r, k, v)]
    B, T, H, N = _shape(toks[0])
    for x in toks:
        if x.shape != (B, T, H, N):
            raise ValueError("token tensors must share one shape")
    g = _f64(g)
    if g is not None and g.shape != (B, T, H, N):
        raise ValueError("g must have the token tensors' shape")
    per_head = [_f64(x) for x in (u, gamma, beta)]
    for x in per_head:
        if x is not None and x.shape != (H, N):
            raise ValueError("u, gamma, beta must be [H, N]")
    if mode not in (0, 1, 2):
        raise ValueError("mode must be 0, 1 or 2")
    out = np.zeros((B, T, H, N))
    lib.wkv7_oracle_epilogue(B, T, H, N, *map(_ptr, toks), _ptr(g), *map(_ptr, per_head),
                             float(eps), int(mode), _ptr(out), nthreads)
    return out


def select_heads(x: Optional[np.ndarray], pairs, state: bool = False):
    """Gather (b, h) pairs into a batch of single-head problems.

    Token tensors [B,T,H,N] -> [P,T,1,N]; states [B,H,N,N] -> [P,1,N,N].
    """
    if x is None:
        return None
    if state:
        return np.stack([x[b_, h_] for b_, h_ in pairs])[:, None]
    return np.stack([x[b_, :, h_] for b_, h_ in pairs])[:, :, None]
