"""Gradients of the WKV7 recurrence -- TEST INFRASTRUCTURE ONLY.

Only the tests and the benchmark's CPU-baseline leg may import this module.
It never touches a GPU and shares no code with the HIP path.

The training path differentiates the bare recurrence (no GroupNorm or bonus;
those are ordinary elementwise and normalisation operations of the layer).
The recurrence is the one of the RWKV-7 "Goose" author response (paperhub),
numpy time_mixing listing, restated in row-vector form by the ARWKV verdict
(pith.science, arXiv 2501.15570, key_machinery field):

    S_t = S_{t-1} diag(w_t) - (S_{t-1} kappa_t)(kappa_t * a_t)^T + v_t k_t^T
    y_t = S_t r_t

For given output cotangents dy ([B,T,H,N]) and dS_T ([B,H,N,N], or zero), the
gradients are those of the scalar

    L = sum_t <y_t, dy_t> + <S_T, dS_T>

with respect to r, w, k, v, kappa, a and S_0.  They come from PyTorch's
reverse-mode differentiation of a plain per-token loop in float64 on the CPU:
the loop is the definition above written out (vectorised over batch and head
only), and autograd supplies the derivative.  Nothing is fused or reordered.
"""
from __future__ import annotations

import numpy as np

NAMES = ("r", "w", "k", "v", "kappa", "a")


def _torch():
    import torch

    return torch


def forward_torch(r, w, k, v, kappa, a, s0):
    """The recurrence as a float64 torch loop: (y [B,T,H,N], S_T [B,H,N,N])."""
    torch = _torch()
    S = s0
    ys = []
    for t in range(r.shape[1]):
        kap_t = kappa[:, t]                                    # [B,H,N]
        u = torch.einsum("bhij,bhj->bhi", S, kap_t)            # S_{t-1} kappa_t
        S = (S * w[:, t, :, None, :]                           # decay of key column j
             - u[..., :, None] * (kap_t * a[:, t])[..., None, :]
             + v[:, t, :, :, None] * k[:, t, :, None, :])
        ys.append(torch.einsum("bhij,bhj->bhi", S, r[:, t]))   # S_t r_t
    y = torch.stack(ys, 1) if ys else r.new_zeros(r.shape)
    return y, S


def backward(r, w, k, v, kappa, a, dy, s0=None, ds_T=None, *, b_idx=None, h_idx=None):
    """Gradients of L (module docstring) as float64 numpy arrays.

    Inputs are numpy arrays [B,T,H,N] (any float dtype; the exact values are
    used), s0 / ds_T [B,H,N,N] or None (zero).  ``b_idx`` / ``h_idx`` restrict
    the computation to a subset of sequences and heads (the heads are
    independent), returning arrays over that subset only.

    Returns dict with keys r, w, k, v, kappa, a ([B',T,H',N]) and s0 ([B',H',N,N]).
    """
    torch = _torch()

    def sel(x, head_axis):
        x = np.asarray(x, dtype=np.float64)
        if b_idx is not None:
            x = x[np.asarray(b_idx)]
        if h_idx is not None:
            x = np.take(x, np.asarray(h_idx), axis=head_axis)
        return torch.from_numpy(np.ascontiguousarray(x))

    ins = [sel(x, 2).requires_grad_(True) for x in (r, w, k, v, kappa, a)]
    B, T, H, N = ins[0].shape
    S0 = (sel(s0, 1) if s0 is not None else torch.zeros(B, H, N, N, dtype=torch.float64))
    S0.requires_grad_(True)
    dyt = sel(dy, 2)
    y, S_T = forward_torch(*ins, S0)
    L = (y * dyt).sum()
    if ds_T is not None:
        L = L + (S_T * sel(ds_T, 1)).sum()
    grads = torch.autograd.grad(L, ins + [S0], allow_unused=True)
    out = {}
    for name, x, g in zip(NAMES + ("s0",), ins + [S0], grads):
        out[name] = (torch.zeros_like(x) if g is None else g).detach().numpy()
    return out


def loss(y, S_T, dy, ds_T=None):
    """L of the module docstring from given outputs (float64)."""
    val = float(np.sum(np.asarray(y, np.float64) * np.asarray(dy, np.float64)))
    if ds_T is not None:
        val += float(np.sum(np.asarray(S_T, np.float64) * np.asarray(ds_T, np.float64)))
    return val
