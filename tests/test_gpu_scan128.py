"""Prefill at head size 128 through the scan kernel (fp32 and bf16 inputs,
fp32 decay, epilogue, bidirectional and fused-prologue entry points) against
the oracle, which takes any head size.  Bounds: 1e-5 (fp32), 2e-2 (bf16)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import NAMES, TOL, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def tol(dtype):
    return TOL["f32" if dtype == "f32" else "bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "bf16_w32"])
@pytest.mark.parametrize("B,H,T", [(2, 3, 37), (1, 2, 100), (1, 1, 1)])
@pytest.mark.parametrize("epi", [False, True])
def test_scan_n128(wkv, dtype, B, H, T, epi):
    x = synth.draw(B, T, H, 128, seed=T + H, dtype=dtype, s0="normal", w_recipe="wide",
                   epilogue=epi)
    d = to_device(x, torch)
    assert wkv.forward_workspace_bytes(B, T, H, 128) == 0
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], epilogue=d["epi"], algo="scan")
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward(*(x.as_f64(n) for n in NAMES), s0=x["s0"], epilogue=x["epi"])
    assert_close(to_f64(y), y_ref, tol(dtype), "y")
    assert_close(to_f64(s), s_ref, tol(dtype), "S")


def test_bidir_n128(wkv):
    x = synth.draw(2, 50, 2, 128, seed=8, dtype="bf16", epilogue=True)
    d = to_device(x, torch)
    y, s = wkv.forward_bidir(*(d[n] for n in NAMES), epilogue=d["epi"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward_bidir(*(x.as_f64(n) for n in NAMES), epilogue=x["epi"])
    assert_close(to_f64(y), y_ref, TOL["bf16"], "bidir y")
    assert_close(to_f64(s), s_ref, TOL["bf16"], "bidir S")


def test_fused_n128(wkv):
    B, T, H = 2, 40, 2
    x = synth.draw(B, T, H, 128, seed=9, dtype="f32", s0="normal")
    k_k, k_a, g = synth.prologue_extras(B, T, H, 128, seed=10, dtype="f32")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y, s = wkv.forward_fused(*(dev(x[n]) for n in ("r", "w", "k", "v", "a")), dev(k_k),
                             dev(k_a), g=dev(g), s0=dev(x["s0"]))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward_fused(*(x.as_f64(n) for n in ("r", "w", "k", "v", "a")), k_k,
                                        k_a, g=g.astype(np.float64), s0=x["s0"])
    assert_close(to_f64(y), y_ref, TOL["f32"], "fused y")
    assert_close(to_f64(s), s_ref, TOL["f32"], "fused S")


def test_n128_refusals(wkv):
    x = synth.draw(1, 20, 1, 128, seed=11, dtype="bf16")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    with pytest.raises(wkv.Rwkv7Error):  # the chunked kernel is bf16 only
        wkv.forward(*(t.float() for t in ins), algo="chunked")
    with pytest.raises(wkv.Rwkv7Error):  # the training forward too
        wkv.forward_train(*(t.float() for t in ins), algo="chunked")
