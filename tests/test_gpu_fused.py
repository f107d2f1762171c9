"""GPU parity of the fused time-mix prologue and output gate
(rwkv7_wkv_forward_fused) against the oracle: kappa = normalise(k * k_k),
k <- k + k (a-1) k_a from raw keys, the recurrence, the optional epilogue, then
y * g.  Bounds as the forward: 1e-5 (fp32), 2e-2 (bf16)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import TOL, assert_close, to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
RAW = ("r", "w", "k", "v", "a")


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def dev(arr):
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def f64(arr):
    return synth.bf16_bits_to_f32(arr).astype(np.float64) if arr.dtype == np.uint16 else \
        np.asarray(arr, np.float64)


def run(wkv, B, T, H, dtype, algo, epi, gate, s0, seed):
    x = synth.draw(B, T, H, seed=seed, dtype=dtype, s0=s0, w_recipe="wide", epilogue=epi)
    k_k, k_a, g = synth.prologue_extras(B, T, H, seed=seed + 1, dtype=dtype)
    d_epi = None
    if x["epi"] is not None:
        e = x["epi"]
        d_epi = {"ln_w": dev(e["ln_w"]), "ln_b": dev(e["ln_b"]),
                 "r_k": dev(np.ascontiguousarray(e["r_k"])), "eps": e["eps"]}
    s0d = None if x["s0"] is None else dev(x["s0"])
    y, s = wkv.forward_fused(*(dev(x[n]) for n in RAW), dev(k_k), dev(k_a),
                             g=dev(g) if gate else None, s0=s0d, algo=algo, epilogue=d_epi)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward_fused(*(x.as_f64(n) for n in RAW), k_k, k_a,
                                        g=f64(g) if gate else None, s0=x["s0"], epilogue=x["epi"])
    tol = TOL["f32" if dtype == "f32" else "bf16"]
    what = f"{dtype} {algo} B{B} T{T} H{H} epi={epi} gate={gate}"
    assert_close(to_f64(y), y_ref, tol, what + " y")
    assert_close(to_f64(s), s_ref, tol, what + " S")


@pytest.mark.parametrize("dtype,algo", [("f32", "scan"), ("bf16", "scan"), ("bf16", "chunked")])
@pytest.mark.parametrize("B,H,T", [(2, 3, 37), (1, 2, 300), (1, 1, 1)])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("gate", [False, True])
def test_fused_sweep(wkv, dtype, algo, B, H, T, epi, gate):
    run(wkv, B, T, H, dtype, algo, epi, gate, "normal", seed=T + 3 * H + B)


def test_fused_segmented(wkv):
    assert wkv.forward_workspace_bytes(1, 5000, 2) > 0
    run(wkv, 1, 5000, 2, "bf16", "chunked", True, True, "normal", seed=61)


def test_fused_29b_shape(wkv):
    run(wkv, 8, 4096, 40, "bf16", "chunked", True, True, "zero", seed=62)


def test_fused_zero_keys_stay_finite(wkv):
    """A token whose keys are all zero: the 1e-12 floor keeps kappa at zero."""
    B, T, H = 1, 20, 2
    x = synth.draw(B, T, H, seed=63, dtype="bf16")
    k = x["k"].copy()
    k[:, 5] = 0
    k_k, k_a, _ = synth.prologue_extras(B, T, H, seed=64)
    ins = [dev(x[n]) if n != "k" else dev(k) for n in RAW]
    y, s = wkv.forward_fused(*ins, dev(k_k), dev(k_a))
    torch.cuda.synchronize()
    raw = [x.as_f64(n) if n != "k" else f64(k) for n in RAW]
    y_ref, s_ref = oracle.forward_fused(*raw, k_k, k_a)
    assert_close(to_f64(y), y_ref, TOL["bf16"], "zero keys y")
    assert_close(to_f64(s), s_ref, TOL["bf16"], "zero keys S")


@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("gate", [False, True])
def test_decode_fused(wkv, N, dtype, epi, gate):
    """One decode step from raw keys (rwkv7_wkv_decode_fused) against the oracle's
    prologue + recurrence at T = 1."""
    B, H = 6, 3
    x = synth.draw(B, 1, H, N, seed=N + B, dtype=dtype, s0="normal", epilogue=epi)
    k_k, k_a, g = synth.prologue_extras(B, 1, H, N, seed=N + 7, dtype=dtype)
    d_epi = None
    if x["epi"] is not None:
        e = x["epi"]
        d_epi = {"ln_w": dev(e["ln_w"]), "ln_b": dev(e["ln_b"]),
                 "r_k": dev(np.ascontiguousarray(e["r_k"])), "eps": e["eps"]}
    st = dev(x["s0"]).clone()
    y = wkv.decode_fused(*(dev(x[n][:, 0]) for n in RAW), dev(k_k), dev(k_a), st,
                         g=dev(g[:, 0]) if gate else None, epilogue=d_epi)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward_fused(*(x.as_f64(n) for n in RAW), k_k, k_a,
                                        g=f64(g) if gate else None, s0=x["s0"], epilogue=x["epi"])
    tol = TOL["f32" if dtype == "f32" else "bf16"]
    assert_close(to_f64(y), y_ref[:, 0], tol, "decode fused y")
    assert_close(to_f64(st), s_ref, tol, "decode fused S")
