"""Thin ctypes binding of librwkv7_wkv.so (the C ABI of include/rwkv7_wkv.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels of the library.  torch provides device memory and the stream; the
functions take CUDA (HIP) tensors and pass their data pointers and
``torch.cuda.current_stream().cuda_stream`` (unless a stream is given).

There is no CPU fallback: if the library is not built, :func:`lib` raises.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

STATUS = {
    0: "RWKV7_OK", 1: "RWKV7_ERR_NULL", 2: "RWKV7_ERR_SHAPE", 3: "RWKV7_ERR_DTYPE",
    4: "RWKV7_ERR_UNSUPPORTED", 5: "RWKV7_ERR_ALIGN", 6: "RWKV7_ERR_ALIAS",
    7: "RWKV7_ERR_WORKSPACE", 8: "RWKV7_ERR_HIP",
}
DT_F32, DT_BF16, DT_BF16_W32 = 0, 1, 2
ALGOS = {"auto": 0, "scan": 1, "chunked": 2}
N_HEAD = 64


class Rwkv7Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({_status_str(code)})")


class Prologue(ctypes.Structure):
    _fields_ = [("k_k", ctypes.c_void_p), ("k_a", ctypes.c_void_p), ("g", ctypes.c_void_p)]


class Epilogue(ctypes.Structure):
    _fields_ = [("ln_w", ctypes.c_void_p), ("ln_b", ctypes.c_void_p),
                ("r_k", ctypes.c_void_p), ("eps", ctypes.c_float)]


_lib = None


def lib():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(
                f"librwkv7_wkv.so is not built ({_build.LIB}); run "
                "`python -m linear_rnn_sequence_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(_build.LIB)
        vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.rwkv7_wkv_forward.argtypes = [vp] * 9 + [ci] * 6 + [ctypes.POINTER(Epilogue), vp,
                                                             sz, vp]
        L.rwkv7_wkv_forward.restype = ci
        L.rwkv7_wkv_forward_noalloc.argtypes = [vp] * 9 + [ci] * 6 + [ctypes.POINTER(Epilogue),
                                                                     vp]
        L.rwkv7_wkv_forward_noalloc.restype = ci
        L.rwkv7_wkv_forward_workspace.argtypes = [ci] * 6
        L.rwkv7_wkv_forward_workspace.restype = sz
        L.rwkv7_wkv_decode.argtypes = [vp] * 8 + [ci] * 4 + [ctypes.POINTER(Epilogue), vp]
        L.rwkv7_wkv_decode.restype = ci
        L.rwkv7_wkv_forward_fused.argtypes = ([vp] * 5 + [ctypes.POINTER(Prologue)] + [vp] * 3
                                              + [ci] * 6 + [ctypes.POINTER(Epilogue), vp, sz,
                                                            vp])
        L.rwkv7_wkv_forward_fused.restype = ci
        L.rwkv7_wkv_decode_fused.argtypes = ([vp] * 5 + [ctypes.POINTER(Prologue)] + [vp] * 2
                                             + [ci] * 4 + [ctypes.POINTER(Epilogue), vp])
        L.rwkv7_wkv_decode_fused.restype = ci
        L.rwkv7_wkv_forward_bidir.argtypes = [vp] * 9 + [ci] * 6 + [ctypes.POINTER(Epilogue),
                                                                   vp, sz, vp]
        L.rwkv7_wkv_forward_bidir.restype = ci
        L.rwkv7_wkv_forward_bidir_workspace.argtypes = [ci] * 6
        L.rwkv7_wkv_forward_bidir_workspace.restype = sz
        L.rwkv7_wkv_forward_train.argtypes = [vp] * 10 + [ci] * 6 + [vp, sz, vp]
        L.rwkv7_wkv_forward_train.restype = ci
        L.rwkv7_wkv_backward.argtypes = [vp] * 16 + [ci] * 6 + [vp, sz, vp]
        L.rwkv7_wkv_backward.restype = ci
        L.rwkv7_wkv_backward_workspace.argtypes = [ci] * 6
        L.rwkv7_wkv_backward_workspace.restype = sz
        L.rwkv7_stream_copy.argtypes = [vp, vp, sz, vp]
        L.rwkv7_stream_copy.restype = ci
        L.rwkv7_status_str.argtypes = [ci]
        L.rwkv7_status_str.restype = ctypes.c_char_p
        L.rwkv7_abi_version.argtypes = []
        L.rwkv7_abi_version.restype = ci
        _lib = L
    return _lib


def _status_str(code: int) -> str:
    try:
        return lib().rwkv7_status_str(code).decode()
    except Exception:  # pragma: no cover - only for messages
        return "?"


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(torch, dt):
    if dt == torch.bfloat16:
        return DT_BF16
    if dt == torch.float32:
        return DT_F32
    raise TypeError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _stream(torch, stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _epilogue(epilogue):
    if epilogue is None:
        return None, ()
    keep = tuple(x for x in (epilogue.get("ln_w"), epilogue.get("ln_b"), epilogue["r_k"])
                 if x is not None)
    e = Epilogue(
        ln_w=None if epilogue.get("ln_w") is None else epilogue["ln_w"].data_ptr(),
        ln_b=None if epilogue.get("ln_b") is None else epilogue["ln_b"].data_ptr(),
        r_k=epilogue["r_k"].data_ptr(),
        eps=float(epilogue.get("eps", 64e-5)),
    )
    return ctypes.byref(e), (e, keep)


def _inputs_dtype(torch, r, w, k, v, kappa, a):
    """Check the six per-token inputs and return the ABI dtype code: one dtype for
    all, or bf16 with a float32 decay w (RWKV7_DT_BF16_W32)."""
    _check_same(torch, (r, k, v, kappa, a), r.shape, r.dtype)
    if r.dtype == torch.bfloat16 and w.dtype == torch.float32:
        _check_same(torch, (w,), r.shape, torch.float32)
        return DT_BF16_W32
    _check_same(torch, (w,), r.shape, r.dtype)
    return _dtype_code(torch, r.dtype)


def _check_same(torch, xs, shape, dtype):
    for x in xs:
        if tuple(x.shape) != tuple(shape):
            raise ValueError(f"shape {tuple(x.shape)} != {tuple(shape)}")
        if x.dtype != dtype:
            raise TypeError("all per-token inputs must share one dtype")
        if not x.is_contiguous():
            raise ValueError("inputs must be contiguous")
        if x.device.type != "cuda":
            raise ValueError("inputs must live on the GPU")


def _check_tensor(torch, t, name, shape, dtype, device):
    """A state, output, epilogue or workspace tensor: the kernels trust the sizes the
    C interface cannot see, so shape, dtype, layout and device are checked here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}, not {t.device}")


def _check_epilogue(torch, epilogue, H, N, device):
    if epilogue is None:
        return
    for key in ("ln_w", "ln_b", "r_k"):
        t = epilogue.get(key)
        if t is None:
            if key == "r_k":
                raise ValueError("the epilogue needs r_k")
            continue
        if t.dtype != torch.float32 or t.numel() != H * N or not t.is_contiguous():
            raise ValueError(f"epilogue {key} must be a contiguous float32 tensor of H*N "
                             f"= {H * N} elements")
        if t.device != device:
            raise ValueError(f"epilogue {key} must live on {device}")


def _check_workspace(torch, ws, device):
    if ws is not None and (not ws.is_contiguous() or ws.device != device):
        raise ValueError(f"the workspace must be a contiguous tensor on {device}")


# dtype names of the workspace queries
DTYPE_NAMES = {"f32": DT_F32, "float32": DT_F32, "bf16": DT_BF16, "bfloat16": DT_BF16,
               "bf16_w32": DT_BF16_W32}


def _dtype_name_code(dtype):
    try:
        return DTYPE_NAMES[dtype]
    except KeyError:
        raise ValueError(f"dtype must be one of {sorted(DTYPE_NAMES)}, not {dtype!r}") from None


def forward_workspace_bytes(B, T, H, N=N_HEAD, *, dtype="bf16", algo="auto") -> int:
    dt = _dtype_name_code(dtype)
    return int(lib().rwkv7_wkv_forward_workspace(B, T, H, N, dt, ALGOS[algo]))


def forward(r, w, k, v, kappa, a, s0=None, *, algo="auto", epilogue=None, y=None, s_out=None,
            want_state=True, workspace=None, stream=None):
    """rwkv7_wkv_forward.  Inputs [B,T,H,N] (bf16 or f32, one dtype; or bf16 with a f32
    decay w), s0 [B,H,N,N] f32.

    Returns (y, s_out).  ``epilogue``: dict of f32 device tensors ln_w, ln_b ([H*N] or
    None), r_k ([H,N] or [H*N]) and float eps.  ``s_out`` may be ``s0`` (in place).
    """
    import torch

    B, T, H, N = r.shape
    dt = _inputs_dtype(torch, r, w, k, v, kappa, a)
    f32, dev = torch.float32, r.device
    _check_tensor(torch, s0, "s0", (B, H, N, N), f32, dev)
    _check_tensor(torch, y, "y", r.shape, r.dtype, dev)
    _check_tensor(torch, s_out, "s_out", (B, H, N, N), f32, dev)
    _check_epilogue(torch, epilogue, H, N, dev)
    _check_workspace(torch, workspace, dev)
    if y is None:
        y = torch.empty_like(r)
    if s_out is None and want_state:
        s_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    need = lib().rwkv7_wkv_forward_workspace(B, T, H, N, dt, ALGOS[algo])
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=r.device)
    epi_ptr, keep = _epilogue(epilogue)
    code = lib().rwkv7_wkv_forward(
        _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(kappa), _ptr(a), _ptr(s0), _ptr(y),
        _ptr(s_out), B, T, H, N, dt, ALGOS[algo], epi_ptr, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(torch, stream))
    del keep
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_forward")
    return y, s_out


def forward_noalloc(r, w, k, v, kappa, a, s0=None, *, y, s_out=None, algo="auto",
                    epilogue=None, stream=None):
    """rwkv7_wkv_forward_noalloc: the forward without a workspace argument, for callers
    that cannot allocate (the library's fixed device array serves as the chunked
    path's workspace; calls that overlap in time on one device race on it).  ``y``
    (and ``s_out``, if the final state is wanted) must be given.  Returns (y, s_out)."""
    import torch

    B, T, H, N = r.shape
    dt = _inputs_dtype(torch, r, w, k, v, kappa, a)
    f32, dev = torch.float32, r.device
    if y is None:
        raise ValueError("forward_noalloc needs y")
    _check_tensor(torch, s0, "s0", (B, H, N, N), f32, dev)
    _check_tensor(torch, y, "y", r.shape, r.dtype, dev)
    _check_tensor(torch, s_out, "s_out", (B, H, N, N), f32, dev)
    _check_epilogue(torch, epilogue, H, N, dev)
    epi_ptr, keep = _epilogue(epilogue)
    code = lib().rwkv7_wkv_forward_noalloc(
        _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(kappa), _ptr(a), _ptr(s0), _ptr(y),
        _ptr(s_out), B, T, H, N, dt, ALGOS[algo], epi_ptr, _stream(torch, stream))
    del keep
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_forward_noalloc")
    return y, s_out


def forward_fused(r, w, k, v, a, k_k, k_a, g=None, s0=None, *, algo="auto", epilogue=None,
                  y=None, s_out=None, want_state=True, workspace=None, stream=None):
    """rwkv7_wkv_forward_fused: the recurrence fed from raw keys k.  The kernels form
    kappa = normalise(k * k_k) and k + k (a-1) k_a, and multiply y (after the epilogue) by
    the gate g if given.  k_k, k_a: f32 [H*N] (or [H,N]); g like r.  Returns (y, s_out)."""
    import torch

    B, T, H, N = r.shape
    _check_same(torch, (r, w, k, v, a) + (() if g is None else (g,)), r.shape, r.dtype)
    dt = _dtype_code(torch, r.dtype)
    for prm in (k_k, k_a):
        if prm.dtype != torch.float32 or prm.numel() != H * N or not prm.is_contiguous():
            raise ValueError("k_k and k_a must be contiguous float32 tensors of H*N elements")
        if prm.device != r.device:
            raise ValueError(f"k_k and k_a must live on {r.device}")
    f32, dev = torch.float32, r.device
    _check_tensor(torch, s0, "s0", (B, H, N, N), f32, dev)
    _check_tensor(torch, y, "y", r.shape, r.dtype, dev)
    _check_tensor(torch, s_out, "s_out", (B, H, N, N), f32, dev)
    _check_epilogue(torch, epilogue, H, N, dev)
    _check_workspace(torch, workspace, dev)
    if y is None:
        y = torch.empty_like(r)
    if s_out is None and want_state:
        s_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    need = lib().rwkv7_wkv_forward_workspace(B, T, H, N, dt, ALGOS[algo])
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=r.device)
    pro = Prologue(k_k=k_k.data_ptr(), k_a=k_a.data_ptr(),
                   g=None if g is None else g.data_ptr())
    epi_ptr, keep = _epilogue(epilogue)
    code = lib().rwkv7_wkv_forward_fused(
        _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), ctypes.byref(pro), _ptr(s0), _ptr(y),
        _ptr(s_out), B, T, H, N, dt, ALGOS[algo], epi_ptr, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(torch, stream))
    del keep
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_forward_fused")
    return y, s_out


def forward_bidir(r, w, k, v, kappa, a, s0=None, *, algo="auto", epilogue=None, y=None,
                  s_out=None, want_state=True, workspace=None, stream=None):
    """rwkv7_wkv_forward_bidir: readouts of the pass over tokens 0..T-1 plus those of the
    pass over T-1..0, epilogue on the sum.  s0 / s_out [2,B,H,N,N] f32 (forward, reverse).
    Returns (y, s_out)."""
    import torch

    B, T, H, N = r.shape
    dt = _inputs_dtype(torch, r, w, k, v, kappa, a)
    f32, dev = torch.float32, r.device
    _check_tensor(torch, s0, "s0", (2, B, H, N, N), f32, dev)
    _check_tensor(torch, y, "y", r.shape, r.dtype, dev)
    _check_tensor(torch, s_out, "s_out", (2, B, H, N, N), f32, dev)
    _check_epilogue(torch, epilogue, H, N, dev)
    _check_workspace(torch, workspace, dev)
    if y is None:
        y = torch.empty_like(r)
    if s_out is None and want_state:
        s_out = torch.empty((2, B, H, N, N), dtype=torch.float32, device=r.device)
    need = lib().rwkv7_wkv_forward_bidir_workspace(B, T, H, N, dt, ALGOS[algo])
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=r.device)
    epi_ptr, keep = _epilogue(epilogue)
    code = lib().rwkv7_wkv_forward_bidir(
        _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(kappa), _ptr(a), _ptr(s0), _ptr(y),
        _ptr(s_out), B, T, H, N, dt, ALGOS[algo], epi_ptr, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(torch, stream))
    del keep
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_forward_bidir")
    return y, s_out


def forward_bidir_workspace_bytes(B, T, H, N=N_HEAD, *, dtype="bf16", algo="auto") -> int:
    dt = _dtype_name_code(dtype)
    return int(lib().rwkv7_wkv_forward_bidir_workspace(B, T, H, N, dt, ALGOS[algo]))


CKPT_INTERVAL = 16  # RWKV7_CKPT_INTERVAL


def forward_train(r, w, k, v, kappa, a, s0=None, *, algo="auto", y=None, s_out=None,
                  s_ckpt=None, want_state=True, workspace=None, stream=None):
    """rwkv7_wkv_forward_train (no epilogue).  Returns (y, s_out, s_ckpt) with
    s_ckpt [B,H,ceil(T/16),N,N] f32, the state before every 16th token."""
    import torch

    B, T, H, N = r.shape
    dt = _inputs_dtype(torch, r, w, k, v, kappa, a)
    f32, dev = torch.float32, r.device
    nck = (T + CKPT_INTERVAL - 1) // CKPT_INTERVAL
    _check_tensor(torch, s0, "s0", (B, H, N, N), f32, dev)
    _check_tensor(torch, y, "y", r.shape, r.dtype, dev)
    _check_tensor(torch, s_out, "s_out", (B, H, N, N), f32, dev)
    _check_tensor(torch, s_ckpt, "s_ckpt", (B, H, nck, N, N), f32, dev)
    _check_workspace(torch, workspace, dev)
    if y is None:
        y = torch.empty_like(r)
    if s_out is None and want_state:
        s_out = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    if s_ckpt is None:
        s_ckpt = torch.empty((B, H, nck, N, N), dtype=torch.float32, device=r.device)
    need = lib().rwkv7_wkv_forward_workspace(B, T, H, N, dt, ALGOS[algo])
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=r.device)
    code = lib().rwkv7_wkv_forward_train(
        _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(kappa), _ptr(a), _ptr(s0), _ptr(y),
        _ptr(s_out), _ptr(s_ckpt), B, T, H, N, dt, ALGOS[algo], _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(torch, stream))
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_forward_train")
    return y, s_out, s_ckpt


def backward_workspace_bytes(B, T, H, N=N_HEAD, *, dtype="bf16", algo="auto") -> int:
    """rwkv7_wkv_backward_workspace."""
    dt = _dtype_name_code(dtype)
    return int(lib().rwkv7_wkv_backward_workspace(B, T, H, N, dt, ALGOS[algo]))


def backward(r, w, k, v, kappa, a, dy, s_ckpt, ds_T=None, *, grads=None, ds0=None,
             want_ds0=True, algo="auto", workspace=None, stream=None):
    """rwkv7_wkv_backward.  Returns (dr, dw, dk, dv, dkappa, da, ds0): the gradients of
    sum_t <y_t, dy_t> + <S_T, ds_T> for the inputs of :func:`forward_train`.  ``grads``
    may pass the six output tensors; ``ds0`` may be ``ds_T`` (in place).  ``algo`` is
    "auto", "scan" or "chunked" (head size 64 only); a workspace, where the algorithm
    needs one (chunked; scan at head size 128), is allocated here unless ``workspace``
    (a uint8 device tensor of at least backward_workspace_bytes) is given.  With a
    float32 decay w (other inputs bf16), dw is float32 too."""
    import torch

    B, T, H, N = r.shape
    dt = _inputs_dtype(torch, r, w, k, v, kappa, a)
    _check_same(torch, (dy,), r.shape, r.dtype)
    f32, dev = torch.float32, r.device
    nck = (T + CKPT_INTERVAL - 1) // CKPT_INTERVAL
    _check_tensor(torch, s_ckpt, "s_ckpt", (B, H, nck, N, N), f32, dev)
    _check_tensor(torch, ds_T, "ds_T", (B, H, N, N), f32, dev)
    _check_tensor(torch, ds0, "ds0", (B, H, N, N), f32, dev)
    _check_workspace(torch, workspace, dev)
    if grads is not None:
        if len(grads) != 6:
            raise ValueError("grads must hold the six gradient tensors (dr, dw, dk, dv, "
                             "dkappa, da)")
        for i, (name, gt) in enumerate(zip(("dr", "dw", "dk", "dv", "dkappa", "da"), grads)):
            _check_tensor(torch, gt, name, r.shape, w.dtype if i == 1 else r.dtype, dev)
            if gt is None:
                raise ValueError(f"{name} is required")
    if grads is None:
        grads = tuple(torch.empty_like(w if i == 1 else r) for i in range(6))
    if ds0 is None and want_ds0:
        ds0 = torch.empty((B, H, N, N), dtype=torch.float32, device=r.device)
    need = int(lib().rwkv7_wkv_backward_workspace(B, T, H, N, dt, ALGOS[algo]))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=r.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().rwkv7_wkv_backward(
        _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(kappa), _ptr(a), _ptr(dy), _ptr(s_ckpt),
        _ptr(ds_T), *(_ptr(g) for g in grads), _ptr(ds0), B, T, H, N, dt, ALGOS[algo],
        _ptr(workspace), nbytes, _stream(torch, stream))
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_backward")
    return (*grads, ds0)


def decode(r, w, k, v, kappa, a, state, *, epilogue=None, y=None, stream=None):
    """rwkv7_wkv_decode.  Inputs [B,H,N]; ``state`` [B,H,N,N] f32 updated in place.
    Returns y [B,H,N]."""
    import torch

    B, H, N = r.shape
    dt = _inputs_dtype(torch, r, w, k, v, kappa, a)
    _check_tensor(torch, state, "state", (B, H, N, N), torch.float32, r.device)
    if state is None:
        raise ValueError("decode needs the state")
    _check_tensor(torch, y, "y", r.shape, r.dtype, r.device)
    _check_epilogue(torch, epilogue, H, N, r.device)
    if y is None:
        y = torch.empty_like(r)
    epi_ptr, keep = _epilogue(epilogue)
    code = lib().rwkv7_wkv_decode(_ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(kappa), _ptr(a),
                                  _ptr(state), _ptr(y), B, H, N, dt, epi_ptr,
                                  _stream(torch, stream))
    del keep
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_decode")
    return y


def decode_fused(r, w, k, v, a, k_k, k_a, state, *, g=None, epilogue=None, y=None,
                 stream=None):
    """rwkv7_wkv_decode_fused: one token per resident state, fed from raw keys k through
    the fused time-mix prologue (k_k, k_a: f32 [H*N]) and gated by g ([B,H,N]) if given.
    Returns y [B,H,N]."""
    import torch

    B, H, N = r.shape
    _check_same(torch, (r, w, k, v, a) + (() if g is None else (g,)), r.shape, r.dtype)
    dt = _dtype_code(torch, r.dtype)
    for prm in (k_k, k_a):
        if prm.dtype != torch.float32 or prm.numel() != H * N or not prm.is_contiguous():
            raise ValueError("k_k and k_a must be contiguous float32 tensors of H*N elements")
        if prm.device != r.device:
            raise ValueError(f"k_k and k_a must live on {r.device}")
    _check_tensor(torch, state, "state", (B, H, N, N), torch.float32, r.device)
    if state is None:
        raise ValueError("decode needs the state")
    _check_tensor(torch, y, "y", r.shape, r.dtype, r.device)
    _check_epilogue(torch, epilogue, H, N, r.device)
    if y is None:
        y = torch.empty_like(r)
    pro = Prologue(k_k=k_k.data_ptr(), k_a=k_a.data_ptr(),
                   g=None if g is None else g.data_ptr())
    epi_ptr, keep = _epilogue(epilogue)
    code = lib().rwkv7_wkv_decode_fused(_ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a),
                                        ctypes.byref(pro), _ptr(state), _ptr(y), B, H, N, dt,
                                        epi_ptr, _stream(torch, stream))
    del keep
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_wkv_decode_fused")
    return y


def prepare_decode(r, w, k, v, kappa, a, state, *, y, epilogue=None, stream=None):
    """Marshal the arguments of one rwkv7_wkv_decode call once and return a
    zero-argument callable that enqueues it (for launch loops where Python-side
    argument handling would otherwise dominate).  The tensors must stay alive and
    unchanged in address while the callable is used."""
    import torch

    B, H, N = r.shape
    dt = _inputs_dtype(torch, r, w, k, v, kappa, a)
    if y is None or state is None:
        raise ValueError("prepare_decode needs y and the state")
    _check_tensor(torch, y, "y", r.shape, r.dtype, r.device)
    _check_tensor(torch, state, "state", (B, H, N, N), torch.float32, r.device)
    _check_epilogue(torch, epilogue, H, N, r.device)
    epi_ptr, keep = _epilogue(epilogue)
    fn = lib().rwkv7_wkv_decode
    args = (_ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(kappa), _ptr(a), _ptr(state), _ptr(y),
            B, H, N, dt, epi_ptr, _stream(torch, stream))

    def launch():
        code = fn(*args)
        if code != 0:
            raise Rwkv7Error(code, "rwkv7_wkv_decode")

    launch.keep = (keep, r, w, k, v, kappa, a, state, y)
    return launch


def stream_copy(src, dst, *, stream=None):
    """rwkv7_stream_copy: copy the bytes of ``src`` into ``dst`` (contiguous device
    tensors of equal byte size) with the library's streaming copy kernel, the
    measured HBM ceiling for one read and one write of every byte."""
    import torch

    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("stream_copy needs contiguous tensors")
    if src.device.type != "cuda" or dst.device != src.device:
        raise ValueError("stream_copy needs two tensors on the same GPU")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("stream_copy needs tensors of equal byte size")
    code = lib().rwkv7_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(torch, stream))
    if code != 0:
        raise Rwkv7Error(code, "rwkv7_stream_copy")
    return dst


def abi_version() -> int:
    return int(lib().rwkv7_abi_version())
