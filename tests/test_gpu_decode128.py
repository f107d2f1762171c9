"""Decode at head size 128 (rwkv7_wkv_decode with N = 128) against the oracle,
which takes any head size: single steps with and without the epilogue, in
fp32, bf16 and bf16 with a float32 decay, and a run of steps replayed by the
oracle as one sequence.  Bounds: 1e-5 (fp32), 2e-2 (bf16)."""
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


@pytest.mark.parametrize("dtype", ["f32", "bf16", "bf16_w32"])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("B,H", [(4, 3), (1, 1), (33, 5)])
def test_decode_n128_step(wkv, dtype, epi, B, H):
    x = synth.draw(B, 1, H, 128, seed=B * 10 + H, dtype=dtype, s0="normal", epilogue=epi)
    d = to_device(x, torch)
    st = d["s0"].clone()
    y = wkv.decode(*(d[n][:, 0].contiguous() for n in NAMES), st, epilogue=d["epi"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward(*(x.as_f64(n) for n in NAMES), s0=x["s0"], epilogue=x["epi"])
    tol = TOL["f32" if dtype == "f32" else "bf16"]
    assert_close(to_f64(y), y_ref[:, 0], tol, "y")
    assert_close(to_f64(st), s_ref, tol, "S")


def test_decode_n128_run(wkv):
    """40 steps through the resident state equal one 40-token sequence."""
    B, T, H = 6, 40, 4
    x = synth.draw(B, T, H, 128, seed=77, dtype="bf16", s0="normal", w_recipe="wide",
                   epilogue=True)
    d = to_device(x, torch)
    st = d["s0"].clone()
    ys = [wkv.decode(*(d[n][:, t].contiguous() for n in NAMES), st, epilogue=d["epi"])
          for t in range(T)]
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward(*(x.as_f64(n) for n in NAMES), s0=x["s0"], epilogue=x["epi"])
    assert_close(to_f64(torch.stack(ys, 1)), y_ref, TOL["bf16"], "y run")
    assert_close(to_f64(st), s_ref, TOL["bf16"], "S run")


def test_forward_n128_chunked_refused_for_f32(wkv):
    x = synth.draw(1, 4, 1, 128, seed=1, dtype="f32")
    d = to_device(x, torch)
    with pytest.raises(wkv.Rwkv7Error):
        wkv.forward(*(d[n] for n in NAMES), algo="chunked")
