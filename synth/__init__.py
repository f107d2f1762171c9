"""Seeded synthetic inputs for the WKV7 recurrence.

This module is shared by the tests, the benchmark and the smoke check.  It
draws the per-token vectors (r, w, k, v, kappa, a), the initial state and the
epilogue parameters, and rounds them to the storage type.  It holds none of the
recurrence's arithmetic: it only draws numbers and applies the input
parameterisations that the pages give for the producers of these vectors.

Sources for the recipes (the trained models and their activations are not
available, so these draws stand in for them):

* RWKV-7 "Goose" author response (paperhub), the numpy time_mixing listing:
  decay w = exp(-sigmoid(.)/sqrt(e)); in-context learning rate a = sigmoid(.);
  removal key kappa = L2-normalised per head with a floor of 1e-12 on the
  norm; per-head GroupNorm with eps = 64e-5 and affine ln_w, ln_b; bonus
  weights r_k of shape (H, N).
* RWKV-7 "Goose" summary (paperlayer, arXiv 2503.14456v2), App. F: the decay
  multiplier stays above 0.545, which the w recipe guarantees.

Layouts are C-order [B, T, H, N] for the per-token vectors, [B, H, N, N] for
states (row = value index i, column = key index j), [H*N] for ln_w / ln_b and
[H, N] for r_k.  bf16 data is returned as uint16 bit patterns produced by
round-to-nearest-even from float32.
"""
from __future__ import annotations

import math

import numpy as np

N_HEAD_SIZE = 64
GN_EPS = 64e-5

# ---------------------------------------------------------------------------
# bf16 helpers (bit level, round to nearest even)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    NaN inputs map to a quiet NaN.  Overflowing values round to +-inf as IEEE
    rounding prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# draw recipes
# ---------------------------------------------------------------------------


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _normalise_last(x: np.ndarray) -> np.ndarray:
    nrm = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(nrm, 1e-12)).astype(np.float32)


_INV_SQRT_E = 1.0 / math.sqrt(math.e)


def decay_from_logit(z: np.ndarray) -> np.ndarray:
    """w = exp(-sigmoid(z)/sqrt(e)); lies in (exp(-1/sqrt(e)), 1) = (0.5452, 1)."""
    return np.exp(-_sigmoid(z.astype(np.float32)) * np.float32(_INV_SQRT_E)).astype(np.float32)


def _correlated_keys(rng, B, T, H, N, cos, flip):
    """Removal keys [B,T,H,N] float32 sharing a direction per (b, h) (see draw)."""
    f32 = np.float32
    if flip is not None:
        base = np.where(rng.random((B, 1, H, N)) < 0.5, f32(-1.0), f32(1.0))
        flips = np.where(rng.random((B, T, H, N)) < flip, f32(-1.0), f32(1.0))
        return (base * flips * f32(1.0 / math.sqrt(N))).astype(f32)
    d = _normalise_last(rng.standard_normal((B, 1, H, N), dtype=f32)).astype(np.float64)
    n = rng.standard_normal((B, T, H, N), dtype=f32).astype(np.float64) / math.sqrt(N)
    if cos >= 1.0:
        return np.broadcast_to(d, (B, T, H, N)).astype(f32)
    alpha = math.sqrt(cos / (1.0 - cos))
    return _normalise_last(alpha * d + n)


class Inputs(dict):
    """Dict of arrays plus metadata (shape, dtype name, epilogue flag)."""

    @property
    def dtype(self) -> str:
        return self["meta"]["dtype"]

    def as_f32(self, name: str) -> np.ndarray:
        x = self[name]
        if x is None:
            return None
        if x.dtype == np.uint16:
            return bf16_bits_to_f32(x)
        return np.asarray(x, dtype=np.float32)

    def as_f64(self, name: str) -> np.ndarray:
        x = self.as_f32(name)
        return None if x is None else x.astype(np.float64)


def draw(
    B: int,
    T: int,
    H: int,
    N: int = N_HEAD_SIZE,
    *,
    seed: int,
    dtype: str = "bf16",
    s0: str = "zero",
    s0_std: float = 0.1,
    w_recipe: str = "default",
    a_mean: float = 0.0,
    epilogue: bool = False,
    kappa_cos: float | None = None,
    kappa_signs: float | None = None,
    k_align: bool = False,
    a_const: float | None = None,
    w_const: float | None = None,
) -> Inputs:
    """Draw one forward-pass input set.

    Draw order (fixed, numpy PCG64 ``default_rng(seed)``): r, w-noise, k, v,
    kappa-noise, a-noise, [w-bias], S0, [r_k, ln_w, ln_b].

    w_recipe:
      "default" : w = exp(-sigmoid(z + 0.5)/sqrt(e)), z ~ N(0,1)
      "wide"    : w = exp(-sigmoid(z + beta)/sqrt(e)), beta ~ N(0, std 2) per (h, j),
                  fixed over b and t (a per-channel bias, as the listing's w_bias)
      "slow"    : w = clamp(exp(-sigmoid(z - 8)/sqrt(e)), 0.99, 1)
    s0: "zero" or "normal" (N(0, s0_std), float32).
    dtype: "bf16", "f32", or "bf16_w32" (bf16 except w, which stays float32).

    Removal keys correlated within a sequence (the delta-rule regime of the
    RWKV-7 "Goose" summary, §2 Background and App. D.3: repeated or similar
    keys overwrite what the state holds for them).  These draws come after all
    of the above, so the other draws are the same with or without them:
      kappa_cos   : kappa = normalise(alpha d + n / sqrt(N)) with one unit
                    direction d ~ normalised N(0, I) per (b, h) and n ~ N(0, I)
                    per token, alpha = sqrt(c / (1 - c)): the mean pairwise
                    cosine of two tokens' keys is close to c (c = 1: one
                    repeated key);
      kappa_signs : kappa = s / sqrt(N) with s in {-1, +1}^N: one sign pattern
                    per (b, h), each sign flipped independently per token with
                    this probability p (mean cosine (1 - 2p)^2).  For N = 64 every
                    entry is +-1/8, so the bf16 key has norm exactly 1;
      k_align     : the written key is k = sqrt(N) kappa (the listing forms kappa
                    from k, so the two point the same way); for N = 64 a power
                    of two times kappa, so bf16(k) = 8 bf16(kappa);
      a_const, w_const : every a (every w) equal to this value.
    """
    rng = np.random.default_rng(seed)
    shp = (B, T, H, N)
    f32 = np.float32
    r = rng.standard_normal(shp, dtype=f32)
    wz = rng.standard_normal(shp, dtype=f32)
    k = rng.standard_normal(shp, dtype=f32)
    v = rng.standard_normal(shp, dtype=f32)
    kz = rng.standard_normal(shp, dtype=f32)
    az = rng.standard_normal(shp, dtype=f32)
    if w_recipe == "default":
        w = decay_from_logit(wz + f32(0.5))
    elif w_recipe == "wide":
        beta = rng.standard_normal((H, N), dtype=f32) * f32(2.0)
        w = decay_from_logit(wz + beta[None, None])
    elif w_recipe == "slow":
        w = np.clip(decay_from_logit(wz - f32(8.0)), f32(0.99), f32(1.0))
    else:
        raise ValueError(f"unknown w_recipe {w_recipe!r}")
    del wz
    kappa = _normalise_last(kz)
    del kz
    a = _sigmoid(az + f32(a_mean)).astype(f32)
    del az
    if kappa_cos is not None or kappa_signs is not None:
        kappa = _correlated_keys(rng, B, T, H, N, kappa_cos, kappa_signs)
    if k_align:
        k = (kappa * f32(math.sqrt(N))).astype(f32)
    if a_const is not None:
        a = np.full(shp, a_const, dtype=f32)
    if w_const is not None:
        w = np.full(shp, w_const, dtype=f32)
    if s0 == "zero":
        S0 = None
    elif s0 == "normal":
        S0 = (rng.standard_normal((B, H, N, N), dtype=f32) * f32(s0_std)).astype(f32)
    else:
        raise ValueError(f"unknown s0 recipe {s0!r}")
    epi = None
    if epilogue:
        r_k = (rng.standard_normal((H, N), dtype=f32) * f32(0.1)).astype(f32)
        ln_w = (f32(1.0) + rng.standard_normal(H * N, dtype=f32) * f32(0.1)).astype(f32)
        ln_b = (rng.standard_normal(H * N, dtype=f32) * f32(0.1)).astype(f32)
        epi = {"ln_w": ln_w, "ln_b": ln_b, "r_k": r_k, "eps": GN_EPS}

    def store(x):
        if dtype in ("bf16", "bf16_w32"):
            return f32_to_bf16_bits(x)
        if dtype == "f32":
            return np.ascontiguousarray(x, dtype=f32)
        raise ValueError(dtype)

    # "bf16_w32": bf16 vectors, except the decay w, kept as float32
    w_st = np.ascontiguousarray(w, dtype=f32) if dtype == "bf16_w32" else store(w)
    out = Inputs(
        r=store(r), w=w_st, k=store(k), v=store(v), kappa=store(kappa), a=store(a),
        s0=S0, epi=epi,
        meta={"B": B, "T": T, "H": H, "N": N, "dtype": dtype, "seed": seed},
    )
    return out


def prologue_extras(B: int, T: int, H: int, N: int = N_HEAD_SIZE, *, seed: int,
                    dtype: str = "bf16"):
    """Parameters of the fused time-mix prologue and the output gate: k_k, k_a
    [H*N] float32 ~ N(1, 0.1) (per-channel scales near one; the pages give no
    values) and g [B,T,H,N] ~ N(0, 1) stored in ``dtype``.  numpy PCG64
    ``default_rng(seed)``, drawn in that order."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    k_k = (f32(1.0) + rng.standard_normal(H * N, dtype=f32) * f32(0.1)).astype(f32)
    k_a = (f32(1.0) + rng.standard_normal(H * N, dtype=f32) * f32(0.1)).astype(f32)
    g = rng.standard_normal((B, T, H, N), dtype=f32)
    if dtype == "bf16":
        g = f32_to_bf16_bits(g)
    elif dtype != "f32":
        raise ValueError(dtype)
    return k_k, k_a, g


def cotangents(B: int, T: int, H: int, N: int = N_HEAD_SIZE, *, seed: int,
               dtype: str = "bf16", with_state: bool = True, std: float = 1.0):
    """Output cotangents for the training path: dy [B,T,H,N] ~ N(0, std) stored in
    ``dtype`` (bf16 bits or float32) and, if ``with_state``, ds_T [B,H,N,N] ~ N(0, std)
    float32.  numpy PCG64 ``default_rng(seed)``, drawn in that order."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    dy = (rng.standard_normal((B, T, H, N), dtype=f32) * f32(std)).astype(f32)
    ds_T = ((rng.standard_normal((B, H, N, N), dtype=f32) * f32(std)).astype(f32)
            if with_state else None)
    if dtype == "bf16":
        dy = f32_to_bf16_bits(dy)
    elif dtype != "f32":
        raise ValueError(dtype)
    return dy, ds_T


# ---------------------------------------------------------------------------
# the five workloads (sizes of the 0.19B..2.9B model shapes, head size 64)
# ---------------------------------------------------------------------------

CONFIGS = {
    0: dict(name="tiny fp32 forward B1 T64 H1", B=1, T=64, H=1, dtype="f32", s0="zero",
            w_recipe="default", a_mean=0.0, epilogue=False),
    1: dict(name="0.19B-shape prefill B4 T1024 H12 bf16", B=4, T=1024, H=12, dtype="bf16",
            s0="normal", w_recipe="default", a_mean=0.0, epilogue=False),
    2: dict(name="2.9B-shape prefill B8 T4096 H40 bf16 + fused epilogue", B=8, T=4096, H=40,
            dtype="bf16", s0="zero", w_recipe="wide", a_mean=0.0, epilogue=True),
    4: dict(name="long-context B1 T65536 H40 bf16, slow decay, near-full replacement", B=1,
            T=65536, H=40, dtype="bf16", s0="zero", w_recipe="slow", a_mean=2.0,
            epilogue=False),
}

# decode workload: 32 layers x B256 x H40 resident fp32 states, 64 single-token steps
DECODE = dict(name="2.9B-shape decode 32 layers x B256 x H40, 64 steps", layers=32, B=256,
              H=40, N=64, steps=64, dtype="bf16", seed=3, s0_std=0.1)


def config_inputs(idx: int, *, T: int | None = None, B: int | None = None,
                  H: int | None = None) -> Inputs:
    """Inputs for forward workload ``idx`` (seed = idx).  T/B/H may be shrunk for tests."""
    c = dict(CONFIGS[idx])
    return draw(B if B is not None else c["B"], T if T is not None else c["T"],
                H if H is not None else c["H"], N_HEAD_SIZE, seed=idx, dtype=c["dtype"],
                s0=c["s0"], w_recipe=c["w_recipe"], a_mean=c["a_mean"],
                epilogue=c["epilogue"])


# ---------------------------------------------------------------------------
# decode inputs, drawn on the device with torch's generator (5.4 GB of state)
# ---------------------------------------------------------------------------


def decode_states_device(torch, device, *, layers, B, H, N, seed, std=0.1):
    """Resident states [layers, B, H, N, N] float32 ~ N(0, std), drawn on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    st = torch.empty((layers, B, H, N, N), dtype=torch.float32, device=device)
    for l in range(layers):
        st[l].normal_(0.0, std, generator=g)
    return st


def decode_step_inputs_device(torch, device, *, B, H, N, seed, count=1):
    """``count`` independent single-token input sets, each [B, H, N] bf16, as one tensor
    per name with a leading ``count`` axis.  Recipe as the tiny forward workload:
    r, k, v ~ N(0,1); a = sigmoid(N(0,1)); w = exp(-sigmoid(N(0,1)+0.5)/sqrt(e));
    kappa = L2-normalised N(0,1) per head."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shp = (count, B, H, N)

    def nrm():
        return torch.randn(shp, generator=g, device=device, dtype=torch.float32)

    r = nrm()
    w = torch.exp(-torch.sigmoid(nrm() + 0.5) * _INV_SQRT_E)
    k = nrm()
    v = nrm()
    kz = nrm()
    kappa = kz / torch.clamp(torch.linalg.vector_norm(kz, dim=-1, keepdim=True), min=1e-12)
    a = torch.sigmoid(nrm())
    bf = torch.bfloat16
    return {n: x.to(bf).contiguous() for n, x in
            dict(r=r, w=w, k=k, v=v, kappa=kappa, a=a).items()}


def sequence_inputs_device(torch, device, *, B, T, H, N, seed, s0_std=None, rows=4096):
    """Per-token inputs [B, T, H, N] bf16 drawn on ``device`` (for sizes whose host
    copies would be impractical), with the recipe of the tiny forward workload:
    r, k, v ~ N(0,1); a = sigmoid(N(0,1)); w = exp(-sigmoid(N(0,1)+0.5)/sqrt(e));
    kappa = L2-normalised N(0,1) per (b, t, h).  Drawn ``rows`` sequences at a
    time (bounded float32 temporaries), names in the order r, w, k, v, kappa, a
    per block.  With ``s0_std``, also "s0" [B, H, N, N] float32 ~ N(0, s0_std)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    bf = torch.bfloat16
    out = {n: torch.empty((B, T, H, N), dtype=bf, device=device)
           for n in ("r", "w", "k", "v", "kappa", "a")}
    for b0 in range(0, B, rows):
        b1 = min(B, b0 + rows)
        shp = (b1 - b0, T, H, N)

        def nrm():
            return torch.randn(shp, generator=g, device=device, dtype=torch.float32)

        out["r"][b0:b1] = nrm().to(bf)
        out["w"][b0:b1] = torch.exp(-torch.sigmoid(nrm() + 0.5) * _INV_SQRT_E).to(bf)
        out["k"][b0:b1] = nrm().to(bf)
        out["v"][b0:b1] = nrm().to(bf)
        kz = nrm()
        out["kappa"][b0:b1] = (kz / torch.clamp(torch.linalg.vector_norm(kz, dim=-1, keepdim=True),
                                                min=1e-12)).to(bf)
        out["a"][b0:b1] = torch.sigmoid(nrm()).to(bf)
    if s0_std is not None:
        s0 = torch.empty((B, H, N, N), dtype=torch.float32, device=device)
        s0.normal_(0.0, s0_std, generator=g)
        out["s0"] = s0
    return out
