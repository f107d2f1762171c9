"""GPU parity of the bidirectional forward (rwkv7_wkv_forward_bidir) against
the oracle's bidirectional reading: the readouts of the pass over tokens
0..T-1 plus those of the pass over T-1..0, epilogue on the sum.  Bounds as the
forward: 1e-5 (fp32 inputs), 2e-2 (bf16 inputs), for y and both final states."""
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


def two_states(rng, B, H, kind):
    if kind == "zero":
        return None
    return (rng.standard_normal((2, B, H, 64, 64)) * 0.1).astype(np.float32)


def check(wkv, x, S0, algo, what, in_place=False):
    dt = x["meta"]["dtype"]
    d = to_device(x, torch)
    s0 = None if S0 is None else torch.from_numpy(S0).cuda()
    kw = {}
    if in_place and s0 is not None:
        kw["s_out"] = s0
    y, s = wkv.forward_bidir(*(d[n] for n in NAMES), s0=s0, algo=algo, epilogue=d["epi"], **kw)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward_bidir(*(x.as_f64(n) for n in NAMES), s0=S0,
                                        epilogue=x["epi"])
    tol = TOL["f32" if dt == "f32" else "bf16"]
    assert_close(to_f64(y), y_ref, tol, f"{what} y")
    assert_close(to_f64(s), s_ref, tol, f"{what} S")
    if in_place and s0 is not None:
        assert s.data_ptr() == s0.data_ptr()


@pytest.mark.parametrize("dtype,algo", [("f32", "scan"), ("bf16", "scan"), ("bf16", "chunked"),
                                        ("bf16_w32", "chunked")])
@pytest.mark.parametrize("B,H,T", [(2, 3, 37), (1, 2, 300), (3, 1, 16), (1, 1, 1)])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("s0", ["zero", "normal"])
def test_bidir_sweep(wkv, dtype, algo, B, H, T, epi, s0):
    rng = np.random.default_rng(T * 10 + H)
    x = synth.draw(B, T, H, seed=T + 7 * H + B, dtype=dtype,
                   w_recipe="slow" if dtype == "bf16_w32" else "wide", epilogue=epi)
    check(wkv, x, two_states(rng, B, H, s0), algo, f"{dtype} {algo} B{B} H{H} T{T} epi={epi}")


def test_bidir_segmented_in_place(wkv):
    """Long sequence, few heads: both passes of the chunked path split the
    sequence into parallel segments; s_out == s0."""
    rng = np.random.default_rng(5)
    assert wkv.forward_bidir_workspace_bytes(1, 6000, 2) > 1 * 6000 * 2 * 64 * 4
    x = synth.draw(1, 6000, 2, seed=55, dtype="bf16", w_recipe="wide", epilogue=True)
    check(wkv, x, two_states(rng, 1, 2, "normal"), "chunked", "segmented", in_place=True)


def test_bidir_29b_shape(wkv):
    x = synth.config_inputs(2)
    check(wkv, x, None, "chunked", "2.9B shape")


def test_bidir_T0_and_small_workspace(wkv):
    z = torch.empty((2, 0, 3, 64), dtype=torch.bfloat16, device="cuda")
    s0 = torch.randn(2, 2, 3, 64, 64, device="cuda")
    _, s = wkv.forward_bidir(z, z, z, z, z, z, s0=s0)
    torch.cuda.synchronize()
    assert torch.equal(s, s0)
    x = synth.draw(1, 64, 2, seed=3, dtype="bf16")
    d = to_device(x, torch)
    need = wkv.forward_bidir_workspace_bytes(1, 64, 2)
    assert need == 64 * 2 * 64 * 4
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(wkv.Rwkv7Error):
        wkv.forward_bidir(*(d[n] for n in NAMES), workspace=ws)
