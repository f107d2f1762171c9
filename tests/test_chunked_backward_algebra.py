"""The algebra of the chunked backward, in float64 on the CPU: the per-chunk
formulas the bf16 MFMA kernels follow (derivative of the chunked form of the
RWKV-7 "Goose" summary, §4 Method) reproduce the float64 autograd oracle's
gradients, with the decay gradient formed either way: with every term of dlg,
or without the same-token terms (the diagonals of dMkr and dMbr, the first
sub-diagonals of dMkk and dMbk), which cancel exactly.  No GPU; this checks the
derivation, not the kernels."""
import numpy as np
import pytest

import synth
from oracle import grad as og

NAMES = ("r", "w", "k", "v", "kappa", "a")
C = 16


def states_before_chunks(r, w, k, v, kap, a, s0):
    """The state before every 16th token and the final state (plain recurrence)."""
    T = r.shape[0]
    S = s0.copy()
    out = []
    for t in range(T):
        if t % C == 0:
            out.append(S.copy())
        S = S * w[t][None, :] - np.outer(S @ kap[t], kap[t] * a[t]) + np.outer(v[t], k[t])
    return out, S


def chunked_backward(r, w, k, v, kap, a, dy, s0, dsT, drop_same_token):
    """Gradients of one head ([T, N] inputs) by the chunk formulas."""
    T, N = r.shape
    ck, S_T = states_before_chunks(r, w, k, v, kap, a, s0)
    g_out = {n: np.zeros((T, N)) for n in NAMES}
    dS = dsT.copy()
    same_token_max = 0.0
    for c in reversed(range(len(ck))):
        sl = slice(c * C, min(T, c * C + C))
        L = sl.stop - sl.start
        R, W, K, V, KP, A, DY = r[sl], w[sl], k[sl], v[sl], kap[sl], a[sl], dy[sl]
        S0 = ck[c]
        S_C = ck[c + 1] if c + 1 < len(ck) else S_T
        G = np.cumprod(W, axis=0)
        Gp = np.vstack([np.ones((1, N)), G[:-1]])
        Kp, Rp, Km, Bm = KP * Gp, R * G, K / G, (A * KP) / G
        low, slow = np.tril(np.ones((L, L))), np.tril(np.ones((L, L)), -1)
        Mkk, Mbk = slow * (Kp @ Km.T), slow * (Kp @ Bm.T)
        Mkr, Mbr = low * (Rp @ Km.T), low * (Rp @ Bm.T)
        X = np.linalg.inv(np.eye(L) + Mbk)
        U = X @ (Kp @ S0.T + Mkk @ V)
        dSh = dS * G[-1][None, :]
        # reverse chain
        dU = -Bm @ dSh.T - Mbr.T @ DY
        dZ = X.T @ dU
        dS0 = dSh + DY.T @ Rp + dZ.T @ Kp
        # value-side and chunk-matrix cotangents
        dV = Km @ dSh.T + Mkr.T @ DY + Mkk.T @ dZ
        dMkr, dMbr = low * (DY @ V.T), -low * (DY @ U.T)
        dMkk, dMbk = slow * (dZ @ V.T), -slow * (dZ @ U.T)
        dKm = V @ dSh + dMkr.T @ Rp + dMkk.T @ Kp
        dBm = -U @ dSh + dMbr.T @ Rp + dMbk.T @ Kp
        dRp = DY @ S0 + dMkr @ Km + dMbr @ Bm
        dKp = dZ @ S0 + dMkk @ Km + dMbk @ Bm
        # decay terms per token
        sub = lambda M: np.r_[np.diag(M, -1), 0.0][:, None]   # M[t+1, t] at row t
        dRp_l, dKm_l, dBm_l, dKp_l = dRp, dKm, dBm, dKp
        if drop_same_token:
            dRp_l = dRp - np.diag(dMkr)[:, None] * Km - np.diag(dMbr)[:, None] * Bm
            Kp_next = np.vstack([Kp[1:], np.zeros((1, N))])
            dKm_l = dKm - np.diag(dMkr)[:, None] * Rp - sub(dMkk) * Kp_next
            dBm_l = dBm - np.diag(dMbr)[:, None] * Rp - sub(dMbk) * Kp_next
            prev = np.vstack([np.zeros((1, N)), (sub(dMkk) * Km + sub(dMbk) * Bm)[:-1]])
            dKp_l = dKp - prev
            # what was dropped from each token's dlg: zero up to rounding
            dropped = ((dRp - dRp_l) * Rp - (dKm - dKm_l) * Km - (dBm - dBm_l) * Bm
                       + np.vstack([((dKp - dKp_l) * Kp)[1:], np.zeros((1, N))]))
            scale = np.abs((dRp - dRp_l) * Rp).max() + 1e-300
            same_token_max = max(same_token_max, np.abs(dropped).max() / scale)
        dlg = dRp_l * Rp - dKm_l * Km - dBm_l * Bm
        dlg[:-1] += (dKp_l * Kp)[1:]
        dlg[-1] += (dS * S_C).sum(0)          # exit state
        dw = np.cumsum(dlg[::-1], axis=0)[::-1] / W
        db = dBm / G
        g_out["r"][sl] = dRp * G
        g_out["w"][sl] = dw
        g_out["k"][sl] = dKm / G
        g_out["v"][sl] = dV
        g_out["kappa"][sl] = dKp * Gp + db * A
        g_out["a"][sl] = db * KP
        dS = dS0
    g_out["s0"] = dS
    return g_out, same_token_max


@pytest.mark.parametrize("T", [1, 2, 16, 37])
@pytest.mark.parametrize("drop_same_token", [False, True])
def test_chunk_formulas_match_autograd(T, drop_same_token):
    x = synth.draw(1, T, 1, seed=900 + T, dtype="f32", s0="normal", w_recipe="wide", a_mean=1.0)
    dy, ds_T = synth.cotangents(1, T, 1, seed=901 + T, dtype="f32")
    ins = [x.as_f64(n) for n in NAMES]
    ref = og.backward(*ins, dy.astype(np.float64), s0=x["s0"], ds_T=ds_T.astype(np.float64))
    got, same = chunked_backward(*(t[0, :, 0] for t in ins), dy[0, :, 0].astype(np.float64),
                                 x["s0"][0, 0].astype(np.float64),
                                 ds_T[0, 0].astype(np.float64), drop_same_token)
    for n in NAMES:
        e = np.abs(got[n] - ref[n][0, :, 0]).max() / np.abs(ref[n]).max()
        assert e < 1e-10, (n, e)
    assert np.abs(got["s0"] - ref["s0"][0, 0]).max() / np.abs(ref["s0"]).max() < 1e-10
    if drop_same_token:
        assert same < 1e-12  # the dropped terms cancel (relative to their size)
