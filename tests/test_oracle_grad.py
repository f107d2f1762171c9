"""Pins for the gradient oracle (oracle/grad.py), none of which use autograd:

* the differentiated float64 loop equals the pinned C oracle's forward;
* directional central differences of the C oracle's forward;
* exact finite differences where the loss is affine in an input (S_0, v, r);
* the one-token gradients written out by hand;
* causality: tokens after the last nonzero cotangent get no gradient.

Page titles used in the citations:
  [listing]  RWKV-7 "Goose" author response (paperhub), numpy time_mixing listing
  [ARWKV]    ARWKV verdict (pith.science, arXiv 2501.15570), key_machinery field
"""
import numpy as np
import pytest

import oracle
from oracle import grad as og

torch = pytest.importorskip("torch")
NAMES = og.NAMES


def rand_case(rng, B=1, T=5, H=2, N=8, s0=True, dsT=True):
    d = dict(r=rng.standard_normal((B, T, H, N)), k=rng.standard_normal((B, T, H, N)),
             v=rng.standard_normal((B, T, H, N)), w=rng.uniform(0.55, 1.0, (B, T, H, N)),
             a=rng.uniform(0.0, 1.0, (B, T, H, N)))
    kap = rng.standard_normal((B, T, H, N))
    d["kappa"] = kap / np.linalg.norm(kap, axis=-1, keepdims=True)
    S0 = rng.standard_normal((B, H, N, N)) * 0.3 if s0 else None
    dy = rng.standard_normal((B, T, H, N))
    dsT_ = rng.standard_normal((B, H, N, N)) if dsT else None
    return d, S0, dy, dsT_


def c_loss(d, S0, dy, dsT):
    """L evaluated through the C oracle (independent of the torch loop)."""
    y, sT = oracle.forward(*(d[n] for n in NAMES), s0=S0)
    return og.loss(y, sT, dy, dsT)


def rel(x, ref):
    return np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300)


# [listing], [ARWKV]: the loop that is differentiated is the pinned recurrence
def test_torch_loop_equals_c_oracle():
    rng = np.random.default_rng(1)
    d, S0, _, _ = rand_case(rng, B=2, T=9, H=3, N=16)
    y_c, s_c = oracle.forward(*(d[n] for n in NAMES), s0=S0)
    y_t, s_t = og.forward_torch(*(torch.from_numpy(d[n]) for n in NAMES), torch.from_numpy(S0))
    assert rel(y_t.numpy(), y_c) < 1e-13 and rel(s_t.numpy(), s_c) < 1e-13


@pytest.mark.parametrize("seed", [2, 3])
def test_directional_central_differences(seed):
    rng = np.random.default_rng(seed)
    d, S0, dy, dsT = rand_case(rng)
    g = og.backward(*(d[n] for n in NAMES), dy, s0=S0, ds_T=dsT)
    eps = 1e-5
    for name in NAMES + ("s0",):
        for _ in range(3):
            delta = rng.standard_normal(S0.shape if name == "s0" else d[name].shape)
            plus, minus = dict(d), dict(d)
            if name == "s0":
                lp = c_loss(d, S0 + eps * delta, dy, dsT)
                lm = c_loss(d, S0 - eps * delta, dy, dsT)
            else:
                plus[name] = d[name] + eps * delta
                minus[name] = d[name] - eps * delta
                lp, lm = c_loss(plus, S0, dy, dsT), c_loss(minus, S0, dy, dsT)
            fd = (lp - lm) / (2 * eps)
            an = float(np.sum(g[name] * delta))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_exact_differences_where_affine():
    """y and S_T are linear in (S_0, v) jointly and y_t is linear in r_t while
    S_T ignores r ([listing]), so L changes by exactly the gradient entry when
    one such input element moves by 1."""
    rng = np.random.default_rng(4)
    d, S0, dy, dsT = rand_case(rng, B=1, T=4, H=1, N=4)
    g = og.backward(*(d[n] for n in NAMES), dy, s0=S0, ds_T=dsT)
    L0 = c_loss(d, S0, dy, dsT)
    for i in range(4):
        for j in range(4):
            E = np.zeros_like(S0)
            E[0, 0, i, j] = 1.0
            assert abs(c_loss(d, S0 + E, dy, dsT) - L0 - g["s0"][0, 0, i, j]) < 1e-11
    for name in ("v", "r"):
        for t in range(4):
            for i in range(4):
                dd = dict(d)
                dd[name] = d[name].copy()
                dd[name][0, t, 0, i] += 1.0
                assert abs(c_loss(dd, S0, dy, dsT) - L0 - g[name][0, t, 0, i]) < 1e-11


def test_one_token_closed_form():
    """T = 1 by hand.  With b = a*kappa, u = S0 kappa, S1 = S0 diag(w) - u b^T + v k^T
    and G = dy r^T + dS_T (the cotangent of S1):
      dr = S1^T dy, dv = G k, dk = G^T v, dw_j = sum_i G_ij S0_ij, db = -G^T u,
      du = -G b, dkappa = S0^T du + a*db, da = kappa*db, dS0 = G diag(w) + du kappa^T."""
    rng = np.random.default_rng(5)
    d, S0, dy, dsT = rand_case(rng, B=1, T=1, H=1, N=6)
    g = og.backward(*(d[n] for n in NAMES), dy, s0=S0, ds_T=dsT)
    x = {n: d[n][0, 0, 0] for n in NAMES}
    s0, dy1, G0 = S0[0, 0], dy[0, 0, 0], dsT[0, 0]
    b = x["a"] * x["kappa"]
    u = s0 @ x["kappa"]
    S1 = s0 * x["w"][None, :] - np.outer(u, b) + np.outer(x["v"], x["k"])
    G = np.outer(dy1, x["r"]) + G0
    db = -G.T @ u
    du = -G @ b
    want = dict(r=S1.T @ dy1, v=G @ x["k"], k=G.T @ x["v"], w=(G * s0).sum(0),
                kappa=s0.T @ du + x["a"] * db, a=x["kappa"] * db,
                s0=G * x["w"][None, :] + np.outer(du, x["kappa"]))
    for n, ref in want.items():
        got = g[n][0, 0] if n == "s0" else g[n][0, 0, 0]
        assert rel(got, ref) < 1e-13, n


def test_causality_and_zero_cotangent():
    rng = np.random.default_rng(6)
    d, S0, dy, _ = rand_case(rng, B=1, T=7, H=2, N=8, dsT=False)
    dy[:, 4:] = 0.0
    g = og.backward(*(d[n] for n in NAMES), dy, s0=S0)
    for n in NAMES:
        assert np.all(g[n][:, 4:] == 0.0), n
        assert np.abs(g[n][:, :4]).max() > 0.0, n
    z = og.backward(*(d[n] for n in NAMES), np.zeros_like(dy), s0=S0)
    assert all(np.all(z[n] == 0.0) for n in NAMES + ("s0",))


def test_head_subset_matches_full():
    rng = np.random.default_rng(7)
    d, S0, dy, dsT = rand_case(rng, B=3, T=3, H=4, N=4)
    full = og.backward(*(d[n] for n in NAMES), dy, s0=S0, ds_T=dsT)
    sub = og.backward(*(d[n] for n in NAMES), dy, s0=S0, ds_T=dsT, b_idx=[2, 0], h_idx=[1, 3])
    for n in NAMES:
        assert np.array_equal(sub[n], full[n][[2, 0]][:, :, [1, 3]])
    assert np.array_equal(sub["s0"], full["s0"][[2, 0]][:, [1, 3]])


def _mutants():
    """Plausible mistakes in the differentiated loop."""
    def decay_on_value(r, w, k, v, kappa, a, s0):
        S, ys = s0, []
        for t in range(r.shape[1]):
            u = torch.einsum("bhij,bhj->bhi", S, kappa[:, t])
            S = (S * w[:, t, :, :, None] - u[..., :, None] * (kappa[:, t] * a[:, t])[..., None, :]
                 + v[:, t, :, :, None] * k[:, t, :, None, :])
            ys.append(torch.einsum("bhij,bhj->bhi", S, r[:, t]))
        return torch.stack(ys, 1), S

    def probe_after_decay(r, w, k, v, kappa, a, s0):
        S, ys = s0, []
        for t in range(r.shape[1]):
            Sd = S * w[:, t, :, None, :]
            u = torch.einsum("bhij,bhj->bhi", Sd, kappa[:, t])
            S = Sd - u[..., :, None] * (kappa[:, t] * a[:, t])[..., None, :] \
                + v[:, t, :, :, None] * k[:, t, :, None, :]
            ys.append(torch.einsum("bhij,bhj->bhi", S, r[:, t]))
        return torch.stack(ys, 1), S

    def readout_old_state(r, w, k, v, kappa, a, s0):
        S, ys = s0, []
        for t in range(r.shape[1]):
            ys.append(torch.einsum("bhij,bhj->bhi", S, r[:, t]))
            u = torch.einsum("bhij,bhj->bhi", S, kappa[:, t])
            S = (S * w[:, t, :, None, :] - u[..., :, None] * (kappa[:, t] * a[:, t])[..., None, :]
                 + v[:, t, :, :, None] * k[:, t, :, None, :])
        return torch.stack(ys, 1), S

    return [decay_on_value, probe_after_decay, readout_old_state]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_mutated_loop_fails_pins(mutant, monkeypatch):
    monkeypatch.setattr(og, "forward_torch", mutant)
    with pytest.raises(AssertionError):
        test_directional_central_differences(2)
