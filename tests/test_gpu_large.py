"""GPU parity past 2^31 elements: offsets into every tensor are 64-bit.

Calls whose per-token tensors hold just over 2^31 elements (B = 2^18 + 1,
T = 64, H = 2, N = 64: 4 GiB per bf16 input; at N = 128, B = 2^17 + 1) and
whose states just over 2^31 (or 2^32) floats, run as one call each: the
chunked and the scan forward, the chunked forward at head size 128, the decode
over a state pool past 2^31 floats, and the training path (stored states past
2^33 floats, both backwards).  The heads at both ends of the batch are checked
in full against the oracle (the rest of the batch only runs); bound 2e-2 as
for every bf16 call.  Inputs are drawn on the device (synth's tiny-forward
recipe) and need up to ~130 GB of device memory."""
import numpy as np
import pytest

import synth
from tests.helpers import NAMES, assert_close

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 2e-2
BS = [0, -1]  # first and last sequence
HS = [0, 1]


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def tok64(t, B):
    """float64 host copy of [B,T,H,N] tensor t at sequences BS and heads HS."""
    idx = [b % B for b in BS]
    return t[idx][:, :, HS].double().cpu().numpy()


def st64(t, B):
    """float64 host copy of [B,H,...] tensor t at sequences BS and heads HS."""
    idx = [b % B for b in BS]
    return t[idx][:, HS].double().cpu().numpy()


def big_inputs(B, T, H, N, seed, s0=True):
    x = synth.sequence_inputs_device(torch, "cuda", B=B, T=T, H=H, N=N, seed=seed,
                                     s0_std=0.1 if s0 else None)
    assert B * T * H * N > 2 ** 31
    return x


@pytest.mark.parametrize("N,B", [(64, (1 << 18) + 1), (128, (1 << 17) + 1)])
def test_forward_past_2_31(wkv, N, B):
    import oracle

    T, H = 64, 2
    x = big_inputs(B, T, H, N, seed=7001 + N)
    assert x["s0"].numel() > 2 ** 31
    ins = [x[n] for n in NAMES]
    ref_in = [tok64(t, B) for t in ins]
    y_ref, s_ref = oracle.forward(*ref_in, s0=st64(x["s0"], B))
    algos = ["chunked", "scan"] if N == 64 else ["chunked"]
    y = torch.empty_like(ins[0])
    s_out = torch.empty_like(x["s0"])
    for algo in algos:
        wkv.forward(*ins, s0=x["s0"], algo=algo, y=y, s_out=s_out)
        torch.cuda.synchronize()
        assert_close(tok64(y, B), y_ref, TOL, f"N{N} {algo} y")
        assert_close(st64(s_out, B), s_ref, TOL, f"N{N} {algo} S_T")


def test_decode_past_2_31(wkv):
    import oracle

    B, H, N = (1 << 18) + 1, 2, 64
    state = synth.decode_states_device(torch, "cuda", layers=1, B=B, H=H, N=N, seed=7101)[0]
    assert state.numel() > 2 ** 31
    x = synth.decode_step_inputs_device(torch, "cuda", B=B, H=H, N=N, seed=7102)
    ins = [x[n][0] for n in NAMES]
    idx = [b % B for b in BS]
    ref_in = [t[idx][:, HS].double().cpu().numpy() for t in ins]
    y_ref, s_ref = oracle.decode(*ref_in, st64(state, B))
    y = wkv.decode(*ins, state)
    torch.cuda.synchronize()
    assert_close(y[idx][:, HS].double().cpu().numpy(), y_ref, TOL, "decode y")
    assert_close(st64(state, B), s_ref, TOL, "decode state")


def test_train_past_2_31(wkv):
    from oracle import grad as og

    B, T, H, N = (1 << 18) + 1, 64, 2, 64
    x = big_inputs(B, T, H, N, seed=7201, s0=False)
    ins = [x[n] for n in NAMES]
    g = torch.Generator(device="cuda")
    g.manual_seed(7202)
    dy = torch.randn((B, T, H, N), generator=g, device="cuda").to(torch.bfloat16)
    _, _, ck = wkv.forward_train(*ins, algo="chunked", want_state=False)
    assert ck.numel() > 2 ** 33
    ref = og.backward(*(tok64(t, B) for t in ins), tok64(dy, B))
    grads = tuple(torch.empty_like(ins[0]) for _ in range(6))
    ds0 = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    for algo in ("chunked", "scan"):
        wkv.backward(*ins, dy, ck, None, grads=grads, ds0=ds0, algo=algo)
        torch.cuda.synchronize()
        for n, gt in zip(NAMES, grads):
            assert_close(tok64(gt, B), ref[n], TOL, f"{algo} d{n}")
        assert_close(st64(ds0, B), ref["s0"], TOL, f"{algo} ds0")
