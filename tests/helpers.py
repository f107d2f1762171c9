"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
run the oracle on the same bits, and compare with the stated bound
max|y - y_ref| / max|y_ref|."""
from __future__ import annotations

import numpy as np

import oracle
import synth

NAMES = ("r", "w", "k", "v", "kappa", "a")
TOL = {"f32": 1e-5, "bf16": 2e-2}


def to_device(x: synth.Inputs, torch, device="cuda"):
    """Per-token inputs as device tensors holding exactly the generator's bits."""
    out = {}
    for n in NAMES:
        arr = x[n]
        if arr.dtype == np.uint16:
            t = torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
        out[n] = t
    out["s0"] = None if x["s0"] is None else torch.from_numpy(x["s0"]).to(device)
    if x["epi"] is not None:
        e = x["epi"]
        out["epi"] = {
            "ln_w": None if e["ln_w"] is None else torch.from_numpy(e["ln_w"]).to(device),
            "ln_b": None if e["ln_b"] is None else torch.from_numpy(e["ln_b"]).to(device),
            "r_k": torch.from_numpy(np.ascontiguousarray(e["r_k"])).to(device),
            "eps": float(e["eps"]),
        }
    else:
        out["epi"] = None
    return out


def oracle_forward(x: synth.Inputs, *, b_idx=None, h_idx=None, threads=None):
    """Oracle on the same bits; optionally on a sample of batches / heads."""
    args = [x.as_f64(n) for n in NAMES]
    s0 = x["s0"]
    epi = x["epi"]
    if b_idx is not None or h_idx is not None:
        bi = slice(None) if b_idx is None else np.asarray(b_idx)
        hi = slice(None) if h_idx is None else np.asarray(h_idx)
        args = [a[bi][:, :, hi] for a in args]
        if s0 is not None:
            s0 = s0[bi][:, hi]
        if epi is not None:
            H = x["meta"]["H"]
            hh = np.arange(H)[hi]
            epi = dict(epi)
            epi["r_k"] = np.asarray(epi["r_k"]).reshape(H, -1)[hh]
            for key in ("ln_w", "ln_b"):
                if epi.get(key) is not None:
                    epi[key] = np.asarray(epi[key]).reshape(H, -1)[hh].reshape(-1)
    return oracle.forward(*args, s0=s0, epilogue=epi, threads=threads)


def to_f64(t):
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    e = rel_err(got, ref)
    assert e <= tol, f"{what}: max|err|/max|ref| = {e:.3e} > {tol:.1e}"
    return e
