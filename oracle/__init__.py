"""WKV7 oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It never touches a GPU and shares no code with the HIP
path (the two meet only through the seeded inputs of ``synth``).

Two independent CPU evaluations of the RWKV-7 WKV7 recurrence:

* :func:`forward` -- the C loops of ``wkv7_oracle.c`` in IEEE double (or the
  fp32 twin), threaded over (batch, head).  This is the oracle proper.
* :func:`forward_numpy` -- the same definition written with numpy matrix
  operations per token (vectorised over batch and head), used to cross-check
  the C loops.

Both follow the state update and readout of the RWKV-7 "Goose" author
response (paperhub), numpy time_mixing listing, which the ARWKV verdict
(pith.science, arXiv 2501.15570, key_machinery field) restates in row-vector
form:

    S_t = S_{t-1} diag(w_t) - (S_{t-1} kappa_t)(kappa_t * a_t)^T + v_t k_t^T
    y_t = S_t r_t

with S[i][j], i the value index and j the key index, followed by the optional
per-head GroupNorm (population variance, eps inside the square root) and the
current-token bonus (sum_j r_j k_j r_k[h, j]) v added after the norm.

Inputs are float arrays of layout [B, T, H, N]; states [B, H, N, N]; the
epilogue parameters ln_w, ln_b ([H*N]) and r_k ([H, N] or [H*N]).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        for name, ct in (("wkv7_oracle_forward_f64", ctypes.c_double),
                         ("wkv7_oracle_forward_f32", ctypes.c_float)):
            fn = getattr(lib, name)
            p = ctypes.POINTER(ct)
            fn.argtypes = [p] * 9 + [ctypes.c_long] * 4 + [p, p, p, ctypes.c_double,
                                                          ctypes.c_int, ctypes.c_int]
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(r, w, k, v, kappa, a, s0=None, epilogue=None, *, precision="f64", threads=None):
    """Run the recurrence on the CPU.

    Returns (y [B,T,H,N], S_T [B,H,N,N]) in float64 (or float32 for the twin).
    ``epilogue`` is None or a dict with keys ln_w, ln_b, r_k, eps (ln_w / ln_b may be None,
    meaning 1 and 0).
    """
    dt = np.float64 if precision == "f64" else np.float32
    ct = ctypes.c_double if precision == "f64" else ctypes.c_float
    fn = getattr(_load(), "wkv7_oracle_forward_" + precision)
    arrs = [np.ascontiguousarray(x, dtype=dt) for x in (r, w, k, v, kappa, a)]
    B, T, H, N = arrs[0].shape
    for x in arrs:
        if x.shape != (B, T, H, N):
            raise ValueError("all per-token inputs must share the shape [B,T,H,N]")
    S0 = None if s0 is None else np.ascontiguousarray(s0, dtype=dt)
    if S0 is not None and S0.shape != (B, H, N, N):
        raise ValueError("s0 must have shape [B,H,N,N]")
    y = np.empty((B, T, H, N), dtype=dt)
    sT = np.empty((B, H, N, N), dtype=dt)

    def ptr(x):
        return None if x is None else x.ctypes.data_as(ctypes.POINTER(ct))

    if epilogue is not None:
        ln_w = epilogue.get("ln_w")
        ln_b = epilogue.get("ln_b")
        ln_w = None if ln_w is None else np.ascontiguousarray(ln_w, dtype=dt).reshape(H * N)
        ln_b = None if ln_b is None else np.ascontiguousarray(ln_b, dtype=dt).reshape(H * N)
        r_k = np.ascontiguousarray(epilogue["r_k"], dtype=dt).reshape(H * N)
        eps = float(epilogue.get("eps", 64e-5))
    else:
        ln_w = ln_b = r_k = None
        eps = 0.0
    rc = fn(*[ptr(x) for x in arrs], ptr(S0), ptr(y), ptr(sT), B, T, H, N,
            ptr(ln_w), ptr(ln_b), ptr(r_k), eps, int(epilogue is not None),
            int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return y, sT


def decode(r, w, k, v, kappa, a, state, epilogue=None, *, precision="f64", threads=None):
    """One token for each of B resident states: inputs [B,H,N], state [B,H,N,N].

    Returns (y [B,H,N], new state).  This is the recurrence at T = 1."""
    add_t = [np.asarray(x)[:, None] for x in (r, w, k, v, kappa, a)]
    y, s = forward(*add_t, s0=state, epilogue=epilogue, precision=precision, threads=threads)
    return y[:, 0], s


def forward_numpy(r, w, k, v, kappa, a, s0=None, epilogue=None):
    """Independent numpy evaluation, one token at a time, vectorised over (b, h).

    The per-token step is written with einsum/broadcast products in float64.
    """
    r, w, k, v, kappa, a = (np.asarray(x, dtype=np.float64) for x in (r, w, k, v, kappa, a))
    B, T, H, N = r.shape
    S = np.zeros((B, H, N, N)) if s0 is None else np.array(s0, dtype=np.float64)
    y = np.empty((B, T, H, N))
    for t in range(T):
        kap, at = kappa[:, t], a[:, t]
        removal = np.einsum("bhij,bhj->bhi", S, kap)              # S_{t-1} kappa
        S = (S * w[:, t][:, :, None, :]
             - removal[..., :, None] * (kap * at)[..., None, :]
             + v[:, t][..., :, None] * k[:, t][..., None, :])
        out = np.einsum("bhij,bhj->bhi", S, r[:, t])
        if epilogue is not None:
            out = group_norm_heads(out, epilogue.get("ln_w"), epilogue.get("ln_b"),
                                   epilogue.get("eps", 64e-5))
            rk = np.asarray(epilogue["r_k"], dtype=np.float64).reshape(H, N)
            out = out + bonus(r[:, t], k[:, t], rk, v[:, t])
        y[:, t] = out
    return y, S


def group_norm_heads(z, ln_w=None, ln_b=None, eps=64e-5):
    """Per-head GroupNorm of z [..., H, N]: population variance, eps inside sqrt,
    then the per-channel affine over the flattened H*N channels."""
    z = np.asarray(z, dtype=np.float64)
    H, N = z.shape[-2:]
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    out = (z - mu) / np.sqrt(var + eps)
    if ln_w is not None:
        out = out * np.asarray(ln_w, dtype=np.float64).reshape(H, N)
    if ln_b is not None:
        out = out + np.asarray(ln_b, dtype=np.float64).reshape(H, N)
    return out


def bonus(r, k, r_k, v):
    """Current-token bonus (sum_j r_j k_j r_k[h, j]) * v, for [..., H, N] inputs."""
    s = np.sum(np.asarray(r, np.float64) * np.asarray(k, np.float64)
               * np.asarray(r_k, np.float64), axis=-1, keepdims=True)
    return s * np.asarray(v, np.float64)


def forward_bidir(r, w, k, v, kappa, a, s0=None, epilogue=None, *, threads=None):
    """Bidirectional reading of the recurrence (RWKV-7 "Goose" summary, §9
    Multimodal Experiments: AudioRWKV-7 uses a bidirectional RWKV-7; the page
    gives no formula).  The plain reading: run the recurrence over tokens
    0..T-1 from s0[0] and over tokens T-1..0 from s0[1], add the two readouts of
    each token, then apply the optional per-head GroupNorm and bonus to the sum.

    Returns (y [B,T,H,N], S [2,B,H,N,N]): the final state of each pass (the
    reverse pass ends after token 0).  float64, through :func:`forward`.
    """
    ins = [np.asarray(x) for x in (r, w, k, v, kappa, a)]
    s0f = s0r = None
    if s0 is not None:
        s0f, s0r = np.asarray(s0)[0], np.asarray(s0)[1]
    y_f, s_f = forward(*ins, s0=s0f, threads=threads)
    y_r, s_r = forward(*(np.ascontiguousarray(x[:, ::-1]) for x in ins), s0=s0r,
                       threads=threads)
    y = y_f + y_r[:, ::-1]
    if epilogue is not None:
        H, N = y.shape[-2:]
        y = group_norm_heads(y, epilogue.get("ln_w"), epilogue.get("ln_b"),
                             epilogue.get("eps", 64e-5))
        rk = np.asarray(epilogue["r_k"], dtype=np.float64).reshape(H, N)
        y = y + bonus(np.asarray(ins[0], np.float64), np.asarray(ins[2], np.float64), rk,
                      np.asarray(ins[3], np.float64))
    return y, np.stack([s_f, s_r])


def prologue(k, a, k_k, k_a):
    """The time-mix prologue of the RWKV-7 "Goose" author response (paperhub),
    numpy time_mixing listing, on per-token keys k and rates a ([..., H, N]):
      kk     = k * k_k, then L2-normalised per head with a 1e-12 floor -> kappa
      k_tilde = k + k * (a - 1) * k_a
    k_k, k_a are per-channel parameters ([H*N] or [H, N]).  float64.
    Returns (kappa, k_tilde)."""
    k = np.asarray(k, np.float64)
    a = np.asarray(a, np.float64)
    H, N = k.shape[-2:]
    kk = k * np.asarray(k_k, np.float64).reshape(H, N)
    nrm = np.sqrt(np.sum(kk * kk, axis=-1, keepdims=True))
    kappa = kk / np.maximum(nrm, 1e-12)
    k_t = k + k * (a - 1.0) * np.asarray(k_a, np.float64).reshape(H, N)
    return kappa, k_t


def forward_fused(r, w, k, v, a, k_k, k_a, g=None, s0=None, epilogue=None, *, threads=None):
    """The recurrence fed from raw keys through :func:`prologue`, with the
    optional epilogue and then the output gate y * g (the listing returns
    Wo @ (y * g); the projection is outside the recurrence).  float64."""
    kappa, k_t = prologue(k, a, k_k, k_a)
    y, sT = forward(r, w, k_t, v, kappa, a, s0=s0, epilogue=epilogue, threads=threads)
    if g is not None:
        y = y * np.asarray(g, np.float64)
    return y, sT
