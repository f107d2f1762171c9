"""Pins for the CPU oracle: closed forms, invariants, exact special cases and
brute force in exact rationals, each tied to the passage it follows.

Page titles used in the citations:
  [listing]  RWKV-7 "Goose" author response (paperhub), numpy time_mixing listing
  [ARWKV]    ARWKV verdict (pith.science, arXiv 2501.15570), key_machinery field
  [summary]  RWKV-7 "Goose" summary (paperlayer, arXiv 2503.14456v2), with its section
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
NAMES = ("r", "w", "k", "v", "kappa", "a")


def rand_inputs(rng, B, T, H, N, *, unit_kappa=True, w_lo=0.55, a_hi=1.0, s0=True):
    r = rng.standard_normal((B, T, H, N))
    k = rng.standard_normal((B, T, H, N))
    v = rng.standard_normal((B, T, H, N))
    w = rng.uniform(w_lo, 1.0, (B, T, H, N))
    a = rng.uniform(0.0, a_hi, (B, T, H, N))
    kap = rng.standard_normal((B, T, H, N))
    if unit_kappa:
        kap /= np.linalg.norm(kap, axis=-1, keepdims=True)
    S0 = rng.standard_normal((B, H, N, N)) * 0.3 if s0 else None
    return dict(r=r, w=w, k=k, v=v, kappa=kap, a=a), S0


def run(d, S0=None, **kw):
    return oracle.forward(d["r"], d["w"], d["k"], d["v"], d["kappa"], d["a"], s0=S0, **kw)


def rel(x, ref):
    return np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300)


# --------------------------------------------------------------------------
# the pages' equation, worked by hand ([listing]: update then readout)
# --------------------------------------------------------------------------

def test_hand_worked_example_exact():
    g = json.load(open(os.path.join(HERE, "golden", "hand_n2_t2.json")))
    sh = lambda x: np.array(x, dtype=np.float64)[None, :, None, :]  # [1,T,1,N]
    S0 = np.array(g["s0"], dtype=np.float64)[None, None]
    for prec in ("f64", "f32"):
        y, sT = oracle.forward(sh(g["r"]), sh(g["w"]), sh(g["k"]), sh(g["v"]), sh(g["kappa"]),
                               sh(g["a"]), s0=S0, precision=prec)
        assert np.array_equal(y[0, :, 0, :], np.array(g["y"])), prec
        assert np.array_equal(sT[0, 0], np.array(g["s_T"])), prec


# --------------------------------------------------------------------------
# T = 1 closed form ([listing]; [ARWKV])
# --------------------------------------------------------------------------

def test_single_step_closed_form():
    rng = np.random.default_rng(1)
    d, S0 = rand_inputs(rng, 2, 1, 3, 64)
    y, sT = run(d, S0)
    x = {n: d[n][:, 0] for n in d}  # [B,H,N]
    Sr = np.einsum("bhij,bhj->bhi", S0, x["w"] * x["r"])
    Sk = np.einsum("bhij,bhj->bhi", S0, x["kappa"])
    ar = np.sum(x["a"] * x["kappa"] * x["r"], -1, keepdims=True)
    kr = np.sum(x["k"] * x["r"], -1, keepdims=True)
    y_ref = Sr - Sk * ar + x["v"] * kr
    S_ref = (S0 * x["w"][:, :, None, :] - Sk[..., None] * (x["a"] * x["kappa"])[:, :, None, :]
             + x["v"][..., None] * x["k"][:, :, None, :])
    assert rel(y[:, 0], y_ref) < 1e-13
    assert rel(sT, S_ref) < 1e-14
    # zero initial state: y_1 = v (k . r)
    y0, _ = run(d, None)
    assert rel(y0[:, 0], x["v"] * kr) < 1e-14


# --------------------------------------------------------------------------
# a = 0, w = 1: plain linear attention ([summary] §2 Background, §4 Method)
# --------------------------------------------------------------------------

def test_linear_attention_special_case():
    rng = np.random.default_rng(2)
    d, S0 = rand_inputs(rng, 2, 40, 2, 16)
    d["a"][:] = 0.0
    d["w"][:] = 1.0
    y, sT = run(d, S0)
    for b in range(2):
        for h in range(2):
            R, K, V = d["r"][b, :, h], d["k"][b, :, h], d["v"][b, :, h]
            Y = R @ S0[b, h].T + np.tril(R @ K.T) @ V
            S = S0[b, h] + V.T @ K
            assert rel(y[b, :, h], Y) < 1e-12
            assert rel(sT[b, h], S) < 1e-12


# --------------------------------------------------------------------------
# a = 0, general w: diagonal (RWKV-6-like) transition ([summary] §3, §4)
# --------------------------------------------------------------------------

def test_diagonal_decay_closed_form():
    rng = np.random.default_rng(3)
    T, N = 32, 16
    d, S0 = rand_inputs(rng, 1, T, 1, N)
    d["a"][:] = 0.0
    y, sT = run(d, S0)
    W, R, K, V = d["w"][0, :, 0], d["r"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0]
    gam = np.cumprod(W, axis=0)  # gamma_t = prod_{s<=t} w_s
    Y = np.zeros((T, N))
    for t in range(T):
        Y[t] = S0[0, 0] @ (gam[t] * R[t])
        for s in range(t + 1):
            Y[t] += V[s] * np.sum(K[s] * R[t] * gam[t] / gam[s])
    S_T = S0[0, 0] * gam[-1][None, :] + sum(np.outer(V[s], K[s] * gam[-1] / gam[s])
                                            for s in range(T))
    assert rel(y[0, :, 0], Y) < 1e-12
    assert rel(sT[0, 0], S_T) < 1e-12


# --------------------------------------------------------------------------
# a = 1, w = 1, unit kappa: delta-rule replacement at the current key
# ([summary] §2 Background "DeltaNet", App. F state evolution)
# --------------------------------------------------------------------------

def test_delta_rule_replacement():
    rng = np.random.default_rng(4)
    T, N = 12, 32
    d, S0 = rand_inputs(rng, 1, T, 2, N)
    d["a"][:] = 1.0
    d["w"][:] = 1.0
    for t in range(1, T + 1):
        dt = {n: x[:, :t] for n, x in d.items()}
        _, St = run(dt, S0)
        kap, k, v = d["kappa"][0, t - 1], d["k"][0, t - 1], d["v"][0, t - 1]  # [H,N]
        lhs = np.einsum("hij,hj->hi", St[0], kap)
        rhs = v * np.sum(k * kap, -1, keepdims=True)
        assert np.abs(lhs - rhs).max() < 1e-12 * max(1.0, np.abs(rhs).max())


# --------------------------------------------------------------------------
# elementary transitions: identity / swap / copy from a key and a binary gate,
# exact in floating point ([summary] App. D.3 lemmas; c absorbed in |kappa|)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_elementary_transitions_bitwise(prec):
    rng = np.random.default_rng(5)
    N = 8
    S0 = rng.integers(-8, 9, (1, 1, N, N)).astype(np.float64)
    base = dict(r=rng.standard_normal((1, 1, 1, N)), k=rng.standard_normal((1, 1, 1, N)),
                v=np.zeros((1, 1, 1, N)), w=np.ones((1, 1, 1, N)))
    i, j = 2, 5
    e = np.eye(N)
    # swap columns i and j: kappa = e_i - e_j, a = 1
    d = dict(base, kappa=(e[i] - e[j])[None, None, None], a=np.ones((1, 1, 1, N)))
    _, S1 = run(d, S0, precision=prec)
    want = S0.copy()
    want[..., [i, j]] = want[..., [j, i]]
    assert np.array_equal(S1, want)
    # copy column i into column j: kappa = e_j - e_i, a = e_j
    d = dict(base, kappa=(e[j] - e[i])[None, None, None], a=e[j][None, None, None])
    _, S1 = run(d, S0, precision=prec)
    want = S0.copy()
    want[..., j] = want[..., i]
    assert np.array_equal(S1, want)
    # a = 0: identity whatever the key
    d = dict(base, kappa=rng.standard_normal((1, 1, 1, N)), a=np.zeros((1, 1, 1, N)))
    _, S1 = run(d, S0, precision=prec)
    assert np.array_equal(S1, S0)


# --------------------------------------------------------------------------
# c = 2 in the construction vs c = 1 in the model: w = 1/2, a = 1, unit kappa,
# v = 0 gives half of a Householder reflection ([summary] App. D.3)
# --------------------------------------------------------------------------

def test_half_householder():
    rng = np.random.default_rng(6)
    N = 16
    S0 = rng.standard_normal((1, 1, N, N))
    kap = rng.standard_normal(N)
    kap /= np.linalg.norm(kap)
    d = dict(r=rng.standard_normal((1, 1, 1, N)), k=rng.standard_normal((1, 1, 1, N)),
             v=np.zeros((1, 1, 1, N)), w=np.full((1, 1, 1, N), 0.5),
             kappa=kap[None, None, None], a=np.ones((1, 1, 1, N)))
    _, S1 = run(d, S0)
    want = 0.5 * S0[0, 0] @ (np.eye(N) - 2.0 * np.outer(kap, kap))
    assert rel(S1[0, 0], want) < 1e-14
    # with kappa = (e_i - e_j)/sqrt(2) this is half a column swap
    e = np.eye(N)
    d["kappa"] = ((e[1] - e[9]) / np.sqrt(2.0))[None, None, None]
    _, S1 = run(d, S0)
    sw = S0[0, 0].copy()
    sw[:, [1, 9]] = sw[:, [9, 1]]
    assert rel(S1[0, 0], 0.5 * sw) < 1e-15


# --------------------------------------------------------------------------
# transition spectrum in [-1, 1]: with w = 1, a = alpha in [0, 2], unit kappa
# and v = 0 the Frobenius norm never grows; alpha = 2 is a reflection and keeps
# it ([summary] §4 Time Mixing eigenvalues; author response on singular values)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("alpha", [0.0, 0.3, 1.0, 1.7, 2.0])
def test_norm_non_increasing(alpha):
    rng = np.random.default_rng(7)
    N, T = 24, 30
    d, S0 = rand_inputs(rng, 1, T, 1, N)
    d["w"][:] = 1.0
    d["a"][:] = alpha
    d["v"][:] = 0.0
    norms = [np.linalg.norm(S0)]
    for t in range(1, T + 1):
        _, St = run({n: x[:, :t] for n, x in d.items()}, S0)
        norms.append(np.linalg.norm(St))
    norms = np.array(norms)
    assert np.all(np.diff(norms) <= 1e-12 * norms[0])
    if alpha == 2.0:
        assert np.abs(norms / norms[0] - 1).max() < 1e-13
    if 0.0 < alpha < 2.0:
        assert norms[-1] < norms[0]


# --------------------------------------------------------------------------
# state passing: two segments equal one pass ([summary] §8 chunked pre-fill,
# constant-memory recurrence)
# --------------------------------------------------------------------------

def test_state_passing_bitwise():
    rng = np.random.default_rng(8)
    d, S0 = rand_inputs(rng, 2, 50, 3, 32)
    y, sT = run(d, S0)
    d1 = {n: x[:, :23] for n, x in d.items()}
    d2 = {n: x[:, 23:] for n, x in d.items()}
    y1, s1 = run(d1, S0)
    y2, s2 = run(d2, s1)
    assert np.array_equal(np.concatenate([y1, y2], 1), y)
    assert np.array_equal(s2, sT)
    # zero-length run returns the initial state
    y0, s0 = run({n: x[:, :0] for n, x in d.items()}, S0)
    assert y0.shape[1] == 0 and np.array_equal(s0, S0)


# --------------------------------------------------------------------------
# linearity and independence ([listing]: y and S are linear in (S0, v);
# S does not read r; y_t reads r_t only)
# --------------------------------------------------------------------------

def test_linearity_and_independence():
    rng = np.random.default_rng(9)
    d, S0 = rand_inputs(rng, 1, 20, 2, 16)
    d2, S0b = rand_inputs(rng, 1, 20, 2, 16)
    al, be = 0.75, -1.5
    y1, s1 = run(d, S0)
    y2, s2 = run(dict(d, v=d2["v"]), S0b)
    y3, s3 = run(dict(d, v=al * d["v"] + be * d2["v"]), al * S0 + be * S0b)
    assert rel(y3, al * y1 + be * y2) < 1e-12
    assert rel(s3, al * s1 + be * s2) < 1e-12
    # S_T independent of r
    _, s4 = run(dict(d, r=d2["r"]), S0)
    assert np.array_equal(s4, s1)
    # changing r at one step changes y at that step only
    r = d["r"].copy()
    r[:, 7] = d2["r"][:, 7]
    y5, _ = run(dict(d, r=r), S0)
    diff = np.abs(y5 - y1).max(axis=(0, 2, 3))
    assert diff[7] > 0 and np.all(np.delete(diff, 7) == 0)


# --------------------------------------------------------------------------
# symmetries ([listing]: heads independent; value rows independent; the key
# index only enters through inner products)
# --------------------------------------------------------------------------

def test_symmetries():
    rng = np.random.default_rng(10)
    B, T, H, N = 3, 15, 4, 16
    d, S0 = rand_inputs(rng, B, T, H, N)
    y, sT = run(d, S0)
    pb, ph = rng.permutation(B), rng.permutation(H)
    dp = {n: x[pb][:, :, ph] for n, x in d.items()}
    yp, sp = run(dp, S0[pb][:, ph])
    assert np.array_equal(yp, y[pb][:, :, ph]) and np.array_equal(sp, sT[pb][:, ph])
    # value-index permutation (rows of S0, entries of v)
    pi = rng.permutation(N)
    yv, sv = run(dict(d, v=d["v"][..., pi]), S0[:, :, pi, :])
    assert np.array_equal(yv, y[..., pi]) and np.array_equal(sv, sT[:, :, pi, :])
    # key-index permutation (w, k, kappa, a, r and the columns of S0)
    pj = rng.permutation(N)
    dk = {n: (x[..., pj] if n != "v" else x) for n, x in d.items()}
    yk, sk = run(dk, S0[..., pj])
    assert rel(yk, y) < 1e-12 and rel(sk, sT[..., pj]) < 1e-12


# --------------------------------------------------------------------------
# brute force in exact rationals, dense transition matrix form
# S_t = S_{t-1} A_t + v_t k_t^T with A_t = diag(w_t) - kappa_t (a_t*kappa_t)^T
# ([ARWKV] row-vector form of the update; [listing] readout y = S r)
# --------------------------------------------------------------------------

def _dyadic(rng, shape, lo=-8, hi=8, den=8):
    return rng.integers(lo, hi + 1, shape) / den


@pytest.mark.parametrize("N,T,seed", [(2, 6, 0), (3, 5, 1), (4, 6, 2), (4, 3, 3)])
def test_bruteforce_exact_rationals(N, T, seed):
    rng = np.random.default_rng(100 + seed)
    d = dict(r=_dyadic(rng, (1, T, 1, N)), k=_dyadic(rng, (1, T, 1, N)),
             v=_dyadic(rng, (1, T, 1, N)), kappa=_dyadic(rng, (1, T, 1, N)),
             w=rng.integers(1, 9, (1, T, 1, N)) / 8, a=rng.integers(0, 17, (1, T, 1, N)) / 8)
    S0 = _dyadic(rng, (1, 1, N, N))
    y, sT = run(d, S0)
    Fr = lambda x: Fraction(float(x))
    S = [[Fr(S0[0, 0, i, j]) for j in range(N)] for i in range(N)]
    for t in range(T):
        g = {n: [Fr(x) for x in d[n][0, t, 0]] for n in d}
        A = [[(g["w"][p] if p == q else Fraction(0)) - g["kappa"][p] * g["a"][q] * g["kappa"][q]
              for q in range(N)] for p in range(N)]
        S = [[sum(S[i][p] * A[p][q] for p in range(N)) + g["v"][i] * g["k"][q]
              for q in range(N)] for i in range(N)]
        yt = [sum(S[i][q] * g["r"][q] for q in range(N)) for i in range(N)]
        ref = np.array([float(x) for x in yt])
        assert np.abs(y[0, t, 0] - ref).max() <= 1e-14 * max(1.0, np.abs(ref).max())
    refS = np.array([[float(x) for x in row] for row in S])
    assert np.abs(sT[0, 0] - refS).max() <= 1e-14 * max(1.0, np.abs(refS).max())


# --------------------------------------------------------------------------
# epilogue: per-head GroupNorm (population variance, eps = 64e-5 inside the
# square root, affine per channel) then the bonus, added after the norm
# ([listing] group_norm and the bonus line; [summary] App. F normalisation)
# --------------------------------------------------------------------------

def test_epilogue_against_torch_group_norm():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    B, T, H, N = 2, 9, 3, 64
    d, S0 = rand_inputs(rng, B, T, H, N)
    ln_w = 1 + 0.1 * rng.standard_normal(H * N)
    ln_b = 0.1 * rng.standard_normal(H * N)
    r_k = 0.1 * rng.standard_normal((H, N))
    epi = dict(ln_w=ln_w, ln_b=ln_b, r_k=r_k, eps=64e-5)
    y, sT = run(d, S0, epilogue=epi)
    z, sT2 = run(d, S0)
    assert np.array_equal(sT, sT2)  # the epilogue never touches the state
    gn = torch.nn.functional.group_norm(torch.from_numpy(z.reshape(B * T, H * N)), H,
                                        torch.from_numpy(ln_w), torch.from_numpy(ln_b),
                                        eps=64e-5).numpy().reshape(B, T, H, N)
    bon = np.einsum("bthj,bthj,hj->bth", d["r"], d["k"], r_k)[..., None] * d["v"]
    assert rel(y, gn + bon) < 1e-12


def test_group_norm_invariants():
    rng = np.random.default_rng(12)
    B, T, H, N = 1, 6, 2, 64
    d, S0 = rand_inputs(rng, B, T, H, N)
    epi = dict(ln_w=None, ln_b=None, r_k=np.zeros((H, N)), eps=64e-5)
    y, _ = run(d, S0, epilogue=epi)
    z, _ = run(d, S0)
    var = z.var(axis=-1)
    assert np.abs(y.mean(axis=-1)).max() < 1e-13
    assert rel(y.var(axis=-1), var / (var + 64e-5)) < 1e-12
    # scaling the state and values by c scales z by c; the norm removes it up to eps
    c = 1e3
    yc, _ = run(dict(d, v=c * d["v"]), c * S0, epilogue=epi)
    want = (z - z.mean(-1, keepdims=True)) / np.sqrt(var[..., None] + 64e-5 / c**2)
    assert rel(yc, want) < 1e-12


# --------------------------------------------------------------------------
# two implementations of the oracle agree; the fp32 twin sits near fp32 rounding
# --------------------------------------------------------------------------

def test_numpy_cross_check_and_fp32_floor():
    rng = np.random.default_rng(13)
    d, S0 = rand_inputs(rng, 2, 64, 3, 64)
    epi = dict(ln_w=1 + 0.1 * rng.standard_normal(3 * 64), ln_b=0.1 * rng.standard_normal(3 * 64),
               r_k=0.1 * rng.standard_normal((3, 64)), eps=64e-5)
    for e in (None, epi):
        y, sT = run(d, S0, epilogue=e)
        yn, sn = oracle.forward_numpy(d["r"], d["w"], d["k"], d["v"], d["kappa"], d["a"], S0, e)
        assert rel(y, yn) < 1e-13 and rel(sT, sn) < 1e-13
        y32, s32 = run(d, S0, epilogue=e, precision="f32")
        assert rel(y32, y) < 2e-6 and rel(s32, sT) < 2e-6


def test_decode_is_one_step():
    rng = np.random.default_rng(14)
    d, S0 = rand_inputs(rng, 3, 1, 2, 64)
    y, sT = run(d, S0)
    yd, sd = oracle.decode(*(d[n][:, 0] for n in ("r", "w", "k", "v", "kappa", "a")), S0)
    assert np.array_equal(yd, y[:, 0]) and np.array_equal(sd, sT)


# --------------------------------------------------------------------------
# bidirectional reading ([summary] §9, AudioRWKV-7; formula not on the page)
# --------------------------------------------------------------------------

def test_bidir_brute_force_and_symmetry():
    """Against per-token loops written here (the readout of token t from the
    state after tokens 0..t plus from the state after tokens T-1..t), and the
    time-reversal symmetry: reversing the sequence and swapping the two initial
    states reverses y and swaps the final states."""
    rng = np.random.default_rng(91)
    d, _ = rand_inputs(rng, 2, 7, 3, 5)
    S0 = rng.standard_normal((2, 2, 3, 5, 5)) * 0.3
    y, S = oracle.forward_bidir(*(d[n] for n in NAMES), s0=S0)
    want = np.zeros_like(y)
    for (order, s_init) in ((range(7), S0[0]), (range(6, -1, -1), S0[1])):
        St = s_init.copy()
        for t in order:
            kap, at = d["kappa"][:, t], d["a"][:, t]
            u = np.einsum("bhij,bhj->bhi", St, kap)
            St = (St * d["w"][:, t][:, :, None, :] - u[..., None] * (kap * at)[:, :, None, :]
                  + d["v"][:, t][..., None] * d["k"][:, t][:, :, None, :])
            want[:, t] += np.einsum("bhij,bhj->bhi", St, d["r"][:, t])
    assert rel(y, want) < 1e-13
    rev = {n: np.ascontiguousarray(d[n][:, ::-1]) for n in NAMES}
    y2, S2 = oracle.forward_bidir(*(rev[n] for n in NAMES), s0=S0[::-1])
    assert rel(y2[:, ::-1], y) < 1e-13 and rel(S2[::-1], S) < 1e-13


def test_bidir_single_token_and_epilogue():
    """T = 1: both passes see the one token, so y = S1_f r + S1_r r; the epilogue
    normalises that sum (then adds the bonus once)."""
    rng = np.random.default_rng(92)
    d, _ = rand_inputs(rng, 1, 1, 2, 64)
    S0 = rng.standard_normal((2, 1, 2, 64, 64)) * 0.3
    y1, _ = oracle.forward(*(d[n] for n in NAMES), s0=S0[0])
    y2, _ = oracle.forward(*(d[n] for n in NAMES), s0=S0[1])
    y, _ = oracle.forward_bidir(*(d[n] for n in NAMES), s0=S0)
    assert rel(y, y1 + y2) < 1e-14
    epi = {"ln_w": rng.standard_normal(128), "ln_b": rng.standard_normal(128),
           "r_k": rng.standard_normal((2, 64)), "eps": 64e-5}
    ye, _ = oracle.forward_bidir(*(d[n] for n in NAMES), s0=S0, epilogue=epi)
    ref = oracle.group_norm_heads(y1 + y2, epi["ln_w"], epi["ln_b"]) + oracle.bonus(
        d["r"], d["k"], epi["r_k"], d["v"])
    assert rel(ye, ref) < 1e-13


# --------------------------------------------------------------------------
# time-mix prologue and output gate ([listing]: kk, k, normalisation, y * g)
# --------------------------------------------------------------------------

def test_prologue_worked_example():
    """N = 2, one head, by hand: k = (3, 4), k_k = (1, 2), k_a = (0.5, 1), a = (0.5, 0)
    -> kk = (3, 8), |kk| = sqrt(73); k_tilde = (3 - 0.75, 4 - 4) = (2.25, 0)."""
    k = np.array([[[[3.0, 4.0]]]])
    a = np.array([[[[0.5, 0.0]]]])
    kap, kt = oracle.prologue(k, a, np.array([1.0, 2.0]), np.array([0.5, 1.0]))
    assert np.allclose(kap[0, 0, 0], np.array([3.0, 8.0]) / np.sqrt(73.0), rtol=0, atol=1e-15)
    assert np.array_equal(kt[0, 0, 0], np.array([2.25, 0.0]))


def test_prologue_invariants():
    rng = np.random.default_rng(93)
    k = rng.standard_normal((2, 5, 3, 64))
    a = rng.uniform(0, 1, (2, 5, 3, 64))
    k_k, k_a = rng.standard_normal(3 * 64), rng.standard_normal(3 * 64)
    kap, kt = oracle.prologue(k, a, k_k, k_a)
    assert np.allclose(np.linalg.norm(kap, axis=-1), 1.0, atol=1e-14)   # unit removal key
    _, kt1 = oracle.prologue(k, np.ones_like(a), k_k, k_a)
    assert np.array_equal(kt1, k)                                       # a = 1: k unchanged
    _, kt0 = oracle.prologue(k, a, k_k, np.zeros_like(k_a))
    assert np.array_equal(kt0, k)                                       # k_a = 0: unchanged
    kz, _ = oracle.prologue(np.zeros_like(k), a, k_k, k_a)
    assert np.array_equal(kz, np.zeros_like(k))                         # 1e-12 floor: no NaN
    # the normalisation ignores the scale of k_k
    kap2, _ = oracle.prologue(k, a, 3.0 * k_k, k_a)
    assert rel(kap2, kap) < 1e-14


def test_forward_fused_composes():
    """Fused = prologue then the pinned recurrence, then the gate; a gate of ones
    changes nothing and the gate scales y channel by channel."""
    rng = np.random.default_rng(94)
    d, S0 = rand_inputs(rng, 2, 9, 2, 64)
    k_k, k_a = rng.standard_normal(128), rng.standard_normal(128)
    g = rng.standard_normal(d["r"].shape)
    kap, kt = oracle.prologue(d["k"], d["a"], k_k, k_a)
    y_ref, s_ref = oracle.forward(d["r"], d["w"], kt, d["v"], kap, d["a"], s0=S0)
    y1, s1 = oracle.forward_fused(d["r"], d["w"], d["k"], d["v"], d["a"], k_k, k_a, s0=S0)
    yg, _ = oracle.forward_fused(d["r"], d["w"], d["k"], d["v"], d["a"], k_k, k_a, g=g, s0=S0)
    assert np.array_equal(y1, y_ref) and np.array_equal(s1, s_ref)
    assert np.array_equal(yg, y_ref * g)


def test_forward_fused_worked_example():
    """Prologue, recurrence, GroupNorm, bonus and gate on one N = 4 token, worked by
    hand (tests/golden/fused_gate_n4_t1.json, exact dyadic values): fails if the
    gate moves before the norm or the bonus, if the bonus uses the raw key, or if
    kappa is formed after the booster ([listing]: group_norm, the bonus line,
    Wo @ (y * g))."""
    gd = json.load(open(os.path.join(HERE, "golden", "fused_gate_n4_t1.json")))
    sh = lambda x: np.array(x, dtype=np.float64)[None, None, None, :]  # [1,1,1,N]
    epi = dict(ln_w=np.array(gd["ln_w"], float), ln_b=np.array(gd["ln_b"], float),
               r_k=np.array(gd["r_k"], float), eps=gd["eps"])
    y, sT = oracle.forward_fused(sh(gd["r"]), sh(gd["w"]), sh(gd["k"]), sh(gd["v"]),
                                 sh(gd["a"]), np.array(gd["k_k"], float),
                                 np.array(gd["k_a"], float), g=sh(gd["g"]),
                                 s0=np.array(gd["s0"], float)[None, None], epilogue=epi)
    assert np.array_equal(y[0, 0, 0], np.array(gd["y"], float))
    assert np.array_equal(sT[0, 0], np.array(gd["s_T"], float))
