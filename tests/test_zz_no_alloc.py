"""rwkv7_wkv_forward_noalloc, the forward for callers that cannot allocate,
against rwkv7_wkv_forward on the same inputs, through the C ABI (ctypes): two
calls in a row, the second with a smaller input, each bitwise equal to the
existing entry point (the same kernels run; only the workspace's address
differs), and a call that needs no workspace."""
import ctypes

import numpy as np
import pytest

import synth
from linear_rnn_sequence_amd import wkv as W
from tests.helpers import NAMES, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def call_noalloc(wkv, d, y, s_out):
    """The C entry point itself, argument by argument."""
    L = wkv.lib()
    B, T, H, N = d["r"].shape
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    epi = None
    keep = None
    if d["epi"] is not None:
        e = d["epi"]
        keep = W.Epilogue(ln_w=e["ln_w"].data_ptr(), ln_b=e["ln_b"].data_ptr(),
                            r_k=e["r_k"].data_ptr(), eps=e["eps"])
        epi = ctypes.byref(keep)
    code = L.rwkv7_wkv_forward_noalloc(
        *(ptr(d[n]) for n in NAMES), ptr(d["s0"]), ptr(y), ptr(s_out), B, T, H, N,
        W.DT_BF16, W.ALGOS["chunked"], epi,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert code == 0, W.Rwkv7Error(code, "rwkv7_wkv_forward_noalloc")


def same_as_forward(wkv, B, T, H, seed, epilogue, split):
    x = synth.draw(B, T, H, seed=seed, dtype="bf16", s0="normal", w_recipe="wide",
                   epilogue=epilogue)
    d = to_device(x, torch)
    assert (wkv.forward_workspace_bytes(B, T, H) > 0) == split
    y_ref, s_ref = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo="chunked",
                               epilogue=d["epi"])
    y = torch.full_like(y_ref, float("nan"))
    s_out = torch.full_like(s_ref, float("nan"))
    call_noalloc(wkv, d, y, s_out)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), f"y differs (B{B} T{T} H{H})"
    assert torch.equal(s_out, s_ref), f"final state differs (B{B} T{T} H{H})"
    return y, s_out


def test_noalloc_matches_forward_twice_then_smaller(wkv):
    # first call: split into segments, the workspace in the library's array
    same_as_forward(wkv, 1, 8229, 2, seed=601, epilogue=True, split=True)
    # second call, smaller: fewer heads and tokens, the array reused
    same_as_forward(wkv, 1, 4100, 1, seed=602, epilogue=False, split=True)
    # no workspace needed
    same_as_forward(wkv, 2, 300, 3, seed=603, epilogue=True, split=False)


def test_noalloc_binding_and_in_place(wkv):
    x = synth.draw(1, 5000, 3, seed=604, dtype="bf16", s0="normal", w_recipe="slow",
                   a_mean=2.0)
    d = to_device(x, torch)
    y_ref, s_ref = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo="chunked")
    st = d["s0"].clone()
    y = torch.empty_like(y_ref)
    wkv.forward_noalloc(*(d[n] for n in NAMES), s0=st, y=y, s_out=st, algo="chunked")
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(st, s_ref)
    assert not np.isnan(st.cpu().numpy()).any()
