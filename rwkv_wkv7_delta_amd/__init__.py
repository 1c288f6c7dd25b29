"""WKV7 (RWKV-7 "Goose" generalised delta rule) on MI355X -- Python binding.

A thin ctypes layer over the C ABI in ``include/wkv7.h`` (``libwkv7.so``):
argument checks and marshalling only, every step of the computation runs in
the HIP kernels.  Tensors are torch CUDA (HIP) tensors; work is enqueued on
the current torch stream.  There is no CPU fallback: if the library is not
built, every call raises.

Per head the state S (N x N, row = value channel, column = key channel)
evolves as ``S <- S (diag(w_t) + a_t b_t^T) + v_t k_t^T`` and ``y_t = S r_t``
("Paper Review: RWKV-7 Goose", Architecture and The approach).  Passing
``a = b = None`` selects the decay-only recurrence ``S <- S diag(w_t) + v_t k_t^T``
(a = b = 0; RWKV-6-style vector-decay linear attention), with specialised
kernels that skip the removal terms; its backward returns ``da = db = None``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwkv7.so")

WKV7_OK = 0
WKV7_ERR_INVALID_ARG = 1
WKV7_ERR_UNSUPPORTED = 2
WKV7_ERR_WORKSPACE = 3
WKV7_ERR_LAUNCH = 4
WKV7_ERR_STATIC_SCRATCH = 5
STATIC_SCRATCH_BYTES = 16 << 20
WKV7_F32 = 0
WKV7_BF16 = 1
HEAD_SIZE = 64
TAPE_CHUNK = 16
TAPE_BLOCK = 32

EXPORTED = ("wkv7_abi_version", "wkv7_status_string", "wkv7_tape_bytes", "wkv7_ckpt_bytes",
            "wkv7_workspace_bytes", "wkv7_backward_workspace_bytes", "wkv7_forward",
            "wkv7_forward_ckpt", "wkv7_forward_split_workspace_bytes", "wkv7_forward_split_plan",
            "wkv7_forward_split",
            "wkv7_forward_split_static",
            "wkv7_backward", "wkv7_backward_ckpt", "wkv7_backward_adjoint", "wkv7_backward_gradients",
            "wkv7_backward_overlapped", "wkv7_decode_step", "wkv7_epilogue",
            "wkv7_forward_epilogue")


class WKV7Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().wkv7_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


class EpilogueParams(ctypes.Structure):
    _fields_ = [("u", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("mode", ctypes.c_int32)]


class SplitPlan(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("split_from", ctypes.c_int32), ("nseg", ctypes.c_int32),
                ("seg_len", ctypes.c_int32)]


WKV7_SPLIT_NONE, WKV7_SPLIT_MAPS, WKV7_SPLIT_SEQUENTIAL = 0, 1, 2


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("dtype", ctypes.c_int32), ("chunk_len", ctypes.c_int32)]


_lib = None


def lib():
    """Load libwkv7.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m rwkv_wkv7_delta_amd.build` (no CPU fallback exists)")
        try:
            import torch  # noqa: F401  (load torch's HIP runtime first)
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(Desc)
        L.wkv7_abi_version.restype = ctypes.c_int
        L.wkv7_status_string.argtypes = [ctypes.c_int]
        L.wkv7_status_string.restype = ctypes.c_char_p
        L.wkv7_tape_bytes.argtypes = [D]
        L.wkv7_tape_bytes.restype = Z
        L.wkv7_ckpt_bytes.argtypes = [D]
        L.wkv7_ckpt_bytes.restype = Z
        L.wkv7_workspace_bytes.argtypes = [D]
        L.wkv7_workspace_bytes.restype = Z
        L.wkv7_backward_workspace_bytes.argtypes = [D, ctypes.c_int]
        L.wkv7_backward_workspace_bytes.restype = Z
        L.wkv7_forward.argtypes = [D] + [P] * 6 + [P, P, P, P, P]
        L.wkv7_forward.restype = ctypes.c_int
        L.wkv7_forward_ckpt.argtypes = [D] + [P] * 6 + [P, P, P, P, P]
        L.wkv7_forward_ckpt.restype = ctypes.c_int
        L.wkv7_forward_split_workspace_bytes.argtypes = [D, I]
        L.wkv7_forward_split_workspace_bytes.restype = Z
        L.wkv7_forward_split_plan.argtypes = [D, I, ctypes.POINTER(SplitPlan)]
        L.wkv7_forward_split_plan.restype = ctypes.c_int
        L.wkv7_forward_split.argtypes = [D] + [P] * 6 + [P, P, P, P, I, P, Z, P]
        L.wkv7_forward_split.restype = ctypes.c_int
        L.wkv7_forward_split_static.argtypes = [D] + [P] * 6 + [P, P, P, P, I, P]
        L.wkv7_forward_split_static.restype = ctypes.c_int
        for name in ("wkv7_backward", "wkv7_backward_adjoint", "wkv7_backward_gradients"):
            fn = getattr(L, name)
            fn.argtypes = [D] + [P] * 6 + [P, P, P, P] + [P] * 6 + [P, P, Z, P]
            fn.restype = ctypes.c_int
        L.wkv7_backward_ckpt.argtypes = [D] + [P] * 6 + [P, P, P, P] + [P] * 6 + [P, P]
        L.wkv7_backward_ckpt.restype = ctypes.c_int
        L.wkv7_backward_overlapped.argtypes = [D] + [P] * 6 + [P, P, P, P] + [P] * 6 + [P, P, Z, P, P]
        L.wkv7_backward_overlapped.restype = ctypes.c_int
        L.wkv7_decode_step.argtypes = [I, I, I, I] + [P] * 6 + [P, P, P]
        L.wkv7_decode_step.restype = ctypes.c_int
        E = ctypes.POINTER(EpilogueParams)
        L.wkv7_epilogue.argtypes = [D] + [P] * 5 + [E, P, P]
        L.wkv7_epilogue.restype = ctypes.c_int
        L.wkv7_forward_epilogue.argtypes = [D] + [P] * 7 + [P, E, P, P, P]
        L.wkv7_forward_epilogue.restype = ctypes.c_int
        _lib = L
    return _lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return WKV7_F32
    if t.dtype == torch.bfloat16:
        return WKV7_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def _check_tokens(ts, shape, dtype):
    for t in ts:
        if t is None:
            raise ValueError("token tensors are required")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("token tensors must be contiguous device tensors")
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
            raise ValueError(f"token tensor shape/dtype mismatch: {tuple(t.shape)} {t.dtype}")


def _check_pair(a, b, shape, dtype):
    """a and b: both token tensors, or both None (a = b = 0)."""
    if (a is None) != (b is None):
        raise ValueError("a and b must both be given or both be None")
    if a is not None:
        _check_tokens((a, b), shape, dtype)


def _check_state(t, shape):
    torch = _torch()
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
        raise ValueError("states must be contiguous float32 device tensors")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"state shape {tuple(t.shape)} != {tuple(shape)}")


def make_desc(B: int, T: int, H: int, N: int, dtype: int, chunk_len: int) -> Desc:
    return Desc(B, T, H, N, dtype, chunk_len)


def tape_bytes(desc: Desc) -> int:
    return int(lib().wkv7_tape_bytes(ctypes.byref(desc)))


def ckpt_bytes(desc: Desc) -> int:
    return int(lib().wkv7_ckpt_bytes(ctypes.byref(desc)))


def workspace_bytes(desc: Desc, with_tape: bool = True) -> int:
    """Backward scratch with or without a tape passed in (``with_tape``)."""
    return int(lib().wkv7_backward_workspace_bytes(ctypes.byref(desc), 1 if with_tape else 0))


def split_workspace_bytes(desc: Desc, segments: int = 0) -> int:
    return int(lib().wkv7_forward_split_workspace_bytes(ctypes.byref(desc), segments))


def split_plan(desc: Desc, segments: int = 0) -> SplitPlan:
    """The plan wkv7_forward_split would run (kind, split_from, nseg, seg_len)."""
    plan = SplitPlan()
    st = lib().wkv7_forward_split_plan(ctypes.byref(desc), segments, ctypes.byref(plan))
    if st != WKV7_OK:
        raise WKV7Error(st, "wkv7_forward_split_plan")
    return plan


def split_tape(tape, B: int, T: int, H: int, N: int = HEAD_SIZE):
    """Views of a forward tape: Z [B, T, H, N] (removal read-outs z_t = S_{t-1} a_t)
    and the states entering every 32-token block [B, H, ceil(T/32), N (key j),
    N (value i)], both bf16."""
    nblk = (T + TAPE_BLOCK - 1) // TAPE_BLOCK
    ntok = B * T * H * N
    z = tape[:ntok].view(B, T, H, N)
    st = tape[ntok:ntok + B * H * nblk * N * N].view(B, H, nblk, N, N)
    return z, st


def forward(r, w, k, v, a, b, s0=None, *, chunk_len: int = 0, want_state: bool = True,
            want_tape: bool = False, out=None, segments: Optional[int] = None, workspace=None,
            tape_out=None, want_ckpt: bool = False, static_scratch: bool = False):
    """Run the recurrence over [B, T, H, N] inputs.

    Returns ``(y, sT, tape)``; ``sT`` / ``tape`` are None unless requested (the
    tape is a flat bf16 tensor for ``backward``; ``split_tape`` gives its parts).
    ``chunk_len`` 0 = sequential scan, 16 = chunked bf16-MFMA form.
    ``segments`` (not None) selects wkv7_forward_split: 0 = the library's
    choice, 1 = no split, n >= 2 = every head in up to n time segments;
    ``workspace`` is then its device scratch (allocated here when None), or,
    with ``static_scratch``, wkv7_forward_split_static runs instead, with the
    library's own fixed scratch (nothing is allocated for it).
    ``tape_out`` (a bf16 device tensor of at least ``tape_bytes`` bytes) receives
    the tape instead of a new allocation.  ``want_ckpt`` selects
    wkv7_forward_ckpt instead: the third result is then the fp32 state entering
    every 16 tokens, [B, H, ceil(T/16), N, N], which ``backward(...,
    chunk_len=0, ckpt=...)`` reads.
    """
    torch = _torch()
    B, T, H, N = r.shape
    _check_tokens((r, w, k, v), r.shape, r.dtype)
    _check_pair(a, b, r.shape, r.dtype)
    _check_state(s0, (B, H, N, N))
    desc = make_desc(B, T, H, N, _dtype_code(r), chunk_len)
    y = out if out is not None else torch.empty_like(r)
    sT = torch.empty((B, H, N, N), device=r.device, dtype=torch.float32) if want_state else None
    if want_ckpt:
        if want_tape or tape_out is not None or segments is not None:
            raise ValueError("want_ckpt excludes the tape and the split forward")
        nst = (T + TAPE_CHUNK - 1) // TAPE_CHUNK
        ck = torch.empty((B, H, nst, N, N), device=r.device, dtype=torch.float32)
        st = lib().wkv7_forward_ckpt(ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                                     _ptr(a), _ptr(b), _ptr(s0), _ptr(y), _ptr(sT), _ptr(ck),
                                     _stream())
        if st != WKV7_OK:
            raise WKV7Error(st, "wkv7_forward_ckpt")
        return y, sT, ck
    ck = None
    if tape_out is not None:
        if not tape_out.is_cuda or not tape_out.is_contiguous() or \
                tape_out.numel() * tape_out.element_size() < tape_bytes(desc):
            raise ValueError("tape_out must be a contiguous device tensor of tape_bytes(desc) bytes")
        ck = tape_out
    elif want_tape:
        nbytes = tape_bytes(desc)
        ck = torch.empty(max(nbytes // 2, 8), device=r.device, dtype=torch.bfloat16)
    if segments is None:
        st = lib().wkv7_forward(ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a),
                                _ptr(b), _ptr(s0), _ptr(y), _ptr(sT), _ptr(ck), _stream())
        if st != WKV7_OK:
            raise WKV7Error(st, "wkv7_forward")
        return y, sT, ck
    if static_scratch:
        st = lib().wkv7_forward_split_static(ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                                             _ptr(a), _ptr(b), _ptr(s0), _ptr(y), _ptr(sT), _ptr(ck),
                                             segments, _stream())
        if st != WKV7_OK:
            raise WKV7Error(st, "wkv7_forward_split_static")
        return y, sT, ck
    wsb = split_workspace_bytes(desc, segments)
    ws = workspace
    if ws is None and wsb > 0:
        ws = torch.empty(wsb // 4, device=r.device, dtype=torch.float32)
    if ws is not None:
        wsb = ws.numel() * ws.element_size()
    st = lib().wkv7_forward_split(ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a),
                                  _ptr(b), _ptr(s0), _ptr(y), _ptr(sT), _ptr(ck), segments,
                                  _ptr(ws), wsb, _stream())
    if st != WKV7_OK:
        raise WKV7Error(st, "wkv7_forward_split")
    return y, sT, ck


EPI_PLAIN, EPI_NORM_TERM, EPI_TERM_NORM = 0, 1, 2


def _epilogue_params(u, gamma, beta, eps: float, mode: int, H: int, N: int) -> EpilogueParams:
    torch = _torch()
    for t in (u, gamma, beta):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32
                              or tuple(t.shape) != (H, N)):
            raise ValueError("u, gamma, beta must be contiguous float32 device tensors of [H, N]")
    return EpilogueParams(_ptr(u), _ptr(gamma), _ptr(beta), float(eps), int(mode))


def epilogue(y, r, k, v, g=None, u=None, gamma=None, beta=None, *, eps: float = 1e-5,
             mode: int = EPI_NORM_TERM, out=None):
    """The step after the read-out (wkv7_epilogue): with s = r . (u * k) per token
    and head, mode 0: g (y + s v); 1: g (norm(y) + s v); 2: g norm(y + s v).
    Token tensors [B, T, H, N] (y's dtype); u, gamma, beta float32 [H, N] or
    None (no term / 1 / 0); g None = 1.  ``out`` may be ``y`` (in place)."""
    torch = _torch()
    B, T, H, N = y.shape
    _check_tokens([y] + [t for t in (r, k, v) if t is not None or u is not None], y.shape, y.dtype)
    if g is not None:
        _check_tokens((g,), y.shape, y.dtype)
    o = out if out is not None else torch.empty_like(y)
    _check_tokens((o,), y.shape, y.dtype)
    prm = _epilogue_params(u, gamma, beta, eps, mode, H, N)
    desc = make_desc(B, T, H, N, _dtype_code(y), 0)
    st = lib().wkv7_epilogue(ctypes.byref(desc), _ptr(y), _ptr(r), _ptr(k), _ptr(v), _ptr(g),
                             ctypes.byref(prm), _ptr(o), _stream())
    if st != WKV7_OK:
        raise WKV7Error(st, "wkv7_epilogue")
    return o


def forward_epilogue(r, w, k, v, a, b, s0=None, g=None, u=None, gamma=None, beta=None, *,
                     eps: float = 1e-5, mode: int = EPI_NORM_TERM, chunk_len: int = 16,
                     want_state: bool = True, out=None):
    """The recurrence and then the step after the read-out (wkv7_forward_epilogue;
    fused into the chunked kernel when chunk_len = 16).  Returns ``(out, sT)``."""
    torch = _torch()
    B, T, H, N = r.shape
    _check_tokens((r, w, k, v), r.shape, r.dtype)
    _check_pair(a, b, r.shape, r.dtype)
    _check_state(s0, (B, H, N, N))
    if g is not None:
        _check_tokens((g,), r.shape, r.dtype)
    o = out if out is not None else torch.empty_like(r)
    _check_tokens((o,), r.shape, r.dtype)
    sT = torch.empty((B, H, N, N), device=r.device, dtype=torch.float32) if want_state else None
    prm = _epilogue_params(u, gamma, beta, eps, mode, H, N)
    desc = make_desc(B, T, H, N, _dtype_code(r), chunk_len)
    st = lib().wkv7_forward_epilogue(ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                                     _ptr(a), _ptr(b), _ptr(s0), _ptr(g), ctypes.byref(prm),
                                     _ptr(o), _ptr(sT), _stream())
    if st != WKV7_OK:
        raise WKV7Error(st, "wkv7_forward_epilogue")
    return o, sT


_STAGES = {"all": "wkv7_backward", "adjoint": "wkv7_backward_adjoint",
           "gradients": "wkv7_backward_gradients", "overlapped": "wkv7_backward_overlapped"}


def backward(r, w, k, v, a, b, dy, s0=None, dsT=None, tape=None, *, chunk_len: int = 16,
             want_ds0: bool = True, workspace=None, stage: str = "all", grads=None, ds0=None,
             aux_stream=None, ckpt=None):
    """Gradients of ``<dy, y> + <dsT, S_T>``: returns (dr, dw, dk, dv, da, db, ds0).

    ``tape`` is the one ``forward(..., want_tape=True)`` returned for the same
    inputs, or None (the forward is then re-run inside the call).  ``ckpt``
    (``chunk_len=0`` only) is the fp32 checkpoint of ``forward(...,
    want_ckpt=True)``: the sequential reverse pass then reads it
    (wkv7_backward_ckpt) instead of re-running the scan.  ``stage``
    selects the whole backward ("all") or one of its two stages ("adjoint",
    then "gradients" with the same ``workspace``, ``grads`` and ``ds0``).
    ``aux_stream`` (a torch stream) runs the whole backward on two streams
    (wkv7_backward_overlapped).  With ``a = b = None`` (a = b = 0) da and db
    are not formed: they are returned (and may be passed in ``grads``) as None.
    """
    torch = _torch()
    B, T, H, N = r.shape
    _check_tokens((r, w, k, v, dy), r.shape, r.dtype)
    _check_pair(a, b, r.shape, r.dtype)
    _check_state(s0, (B, H, N, N))
    _check_state(dsT, (B, H, N, N))
    desc = make_desc(B, T, H, N, _dtype_code(r), chunk_len)
    nab = 6 if a is not None else 4
    if grads is None:
        grads = [torch.empty_like(r) for _ in range(nab)] + [None] * (6 - nab)
    grads = list(grads)
    if len(grads) != 6:
        raise ValueError("grads holds (dr, dw, dk, dv, da, db)")
    _check_tokens(grads[:nab], r.shape, r.dtype)
    if a is None:
        _check_pair(grads[4], grads[5], r.shape, r.dtype)
    if ds0 is None and want_ds0:
        ds0 = torch.empty((B, H, N, N), device=r.device, dtype=torch.float32)
    _check_state(ds0, (B, H, N, N))
    if ckpt is not None:
        nst = (T + TAPE_CHUNK - 1) // TAPE_CHUNK
        _check_state(ckpt, (B, H, nst, N, N))
        if tape is not None or aux_stream is not None or stage != "all" or chunk_len != 0:
            raise ValueError("ckpt goes with chunk_len=0, no tape, the whole backward")
        st = lib().wkv7_backward_ckpt(ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                                      _ptr(a), _ptr(b), _ptr(s0), _ptr(dy), _ptr(dsT), _ptr(ckpt),
                                      *[_ptr(x) for x in grads], _ptr(ds0), _stream())
        if st != WKV7_OK:
            raise WKV7Error(st, "wkv7_backward_ckpt")
        return tuple(grads) + (ds0,)
    wsb = workspace_bytes(desc, tape is not None)
    ws = workspace
    if ws is None:
        ws = torch.empty(max(wsb // 4, 4), device=r.device, dtype=torch.float32)
    else:
        wsb = ws.numel() * ws.element_size()
    name = _STAGES["overlapped" if aux_stream is not None else stage]
    if aux_stream is not None and stage != "all":
        raise ValueError("aux_stream applies to the whole backward only")
    extra = (aux_stream.cuda_stream,) if aux_stream is not None else ()
    st = getattr(lib(), name)(ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a),
                              _ptr(b), _ptr(s0), _ptr(dy), _ptr(dsT), _ptr(tape),
                              *[_ptr(x) for x in grads], _ptr(ds0), _ptr(ws), wsb, _stream(),
                              *extra)
    if st != WKV7_OK:
        raise WKV7Error(st, name)
    return tuple(grads) + (ds0,)


def decode_step(r, w, k, v, a, b, state, out=None):
    """One token on resident states [B, H, N, N] (updated in place); returns y [B, H, N]."""
    torch = _torch()
    B, H, N = r.shape
    _check_tokens((r, w, k, v), r.shape, r.dtype)
    _check_pair(a, b, r.shape, r.dtype)
    _check_state(state, (B, H, N, N))
    y = out if out is not None else torch.empty_like(r)
    st = lib().wkv7_decode_step(B, H, N, _dtype_code(r), _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                                _ptr(a), _ptr(b), _ptr(state), _ptr(y), _stream())
    if st != WKV7_OK:
        raise WKV7Error(st, "wkv7_decode_step")
    return y
