"""GPU parity of the training path at head size 128 through the C ABI: the
forward with state storage (the chunked kernel for bf16, the scan for any
dtype) and the token-by-token backward (four workgroups of 32 value rows per
head, their partial column sums added by a second kernel; long sequences in
slices with the state cotangent carried between them), against the gradient
oracle (float64 autograd of the plain loop, which takes any head size).  The
pages tune their kernels for head size 64 and name larger heads as less
efficient (RWKV-7 "Goose" summary, §8 Speed and Memory).

Bounds as at head size 64: max|g - g_ref| / max|g_ref| <= 1e-4 for fp32
inputs and <= 2e-2 for bf16 inputs, per gradient tensor."""
import numpy as np
import pytest

import synth
from tests.helpers import NAMES, TOL, assert_close, rel_err, to_device, to_f64
from tests.test_gpu_train import TOL_GRAD, cot_device, oracle_ckpts, run_and_check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
N = 128


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


@pytest.mark.parametrize("dtype,algo", [("f32", "scan"), ("bf16", "scan"), ("bf16", "chunked")])
def test_train_forward_stores_states_128(wkv, dtype, algo):
    x = synth.draw(2, 77, 3, N, seed=1101, dtype=dtype, s0="normal", w_recipe="wide")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    y0, s0 = wkv.forward(*ins, s0=d["s0"], algo=algo)
    y1, s1, ck = wkv.forward_train(*ins, s0=d["s0"], algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(s0, s1)  # storing states changes nothing
    assert tuple(ck.shape) == (2, 3, 5, N, N)
    assert torch.equal(ck[:, :, 0], d["s0"])
    assert_close(to_f64(ck), oracle_ckpts(x), TOL[dtype], "stored states")


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 40, 100])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward128_sweep_T(wkv, T, dtype):
    x = synth.draw(1, T, 2, N, seed=1300 + T, dtype=dtype, s0="normal")
    dy, ds_T = synth.cotangents(1, T, 2, N, seed=1400 + T, dtype=dtype)
    run_and_check(wkv, x, dy, ds_T, what=f"N128 {dtype} T={T}")


@pytest.mark.parametrize("B,H,T", [(2, 3, 37), (3, 1, 129)])
@pytest.mark.parametrize("with_dsT", [False, True])
@pytest.mark.parametrize("s0", ["zero", "normal"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward128_sweep(wkv, B, H, T, with_dsT, s0, dtype):
    x = synth.draw(B, T, H, N, seed=B * 1000 + H * 100 + T + 7, dtype=dtype, s0=s0,
                   w_recipe="wide")
    dy, ds_T = synth.cotangents(B, T, H, N, seed=17 + T, dtype=dtype, with_state=with_dsT)
    run_and_check(wkv, x, dy, ds_T, what=f"N128 {dtype} B{B} H{H} T{T} dsT={with_dsT} s0={s0}")


def test_backward128_after_chunked_forward(wkv):
    """States stored by the chunked forward at 128 (bf16 MFMA) feed the same
    backward: gradients within the bf16 bound of the oracle, and of the run
    whose states came from the scan."""
    x = synth.draw(2, 200, 2, N, seed=1021, dtype="bf16", s0="normal", w_recipe="wide")
    dy, ds_T = synth.cotangents(2, 200, 2, N, seed=1022, dtype="bf16")
    _, (_, _, ck_c) = run_and_check(wkv, x, dy, ds_T, algo="chunked", what="N128 chunked fwd")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    dyt, _, dst = cot_device(dy, ds_T, "bf16")
    outs = []
    for algo in ("scan", "chunked"):
        _, _, ck = wkv.forward_train(*ins, s0=d["s0"], algo=algo)
        outs.append(wkv.backward(*ins, dyt, ck, dst))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert rel_err(to_f64(a), to_f64(b)) <= TOL_GRAD["bf16"]


def test_backward128_fp32_decay(wkv):
    """bf16 inputs with a float32 decay (dw float32 too), slow decays near 1."""
    from oracle import grad as og

    B, T, H = 2, 100, 2
    x = synth.draw(B, T, H, N, seed=1031, dtype="bf16_w32", w_recipe="slow", a_mean=2.0,
                   s0="normal")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    _, _, ck = wkv.forward_train(*ins, s0=d["s0"])
    dy_bits, ds_T = synth.cotangents(B, T, H, N, seed=1032, dtype="bf16")
    dy = torch.from_numpy(dy_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dst = torch.from_numpy(ds_T).cuda()
    *g, ds0 = wkv.backward(*ins, dy, ck, dst)
    torch.cuda.synchronize()
    assert g[1].dtype == torch.float32 and g[0].dtype == torch.bfloat16
    ref = og.backward(*(x.as_f64(n) for n in NAMES),
                      synth.bf16_bits_to_f32(dy_bits).astype(np.float64), s0=x["s0"],
                      ds_T=ds_T.astype(np.float64))
    for n, gt in zip(NAMES, g):
        assert_close(to_f64(gt), ref[n], TOL_GRAD["bf16"], f"N128 w32 d{n}")
    assert_close(to_f64(ds0), ref["s0"], TOL_GRAD["bf16"], "N128 w32 ds0")


def test_backward128_slices(wkv):
    """B4 H64: one slice holds 96 tokens, so T = 200 runs as three slices (96,
    96, 8 tokens) with the state cotangent carried between them; four (b, h)
    pairs checked in full against the oracle, and ds0 written over ds_T or not at
    all gives the same bits."""
    B, T, H = 4, 200, 64
    assert wkv.backward_workspace_bytes(B, T, H, N, algo="scan") == \
        5 * 4 * B * H * N * 4 * 96 + B * H * N * N * 4
    x = synth.draw(B, T, H, N, seed=1041, dtype="bf16", s0="normal", w_recipe="wide")
    dy, ds_T = synth.cotangents(B, T, H, N, seed=1042, dtype="bf16")
    errs, _ = run_and_check(wkv, x, dy, ds_T, algo="scan", b_idx=[0, 3], h_idx=[0, 63],
                            what="N128 slices")
    print("N128 slices:", {k: f"{v:.2e}" for k, v in errs.items()})
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    dyt, _, dst = cot_device(dy, ds_T, "bf16")
    _, _, ck = wkv.forward_train(*ins, s0=d["s0"], algo="scan")
    ref = wkv.backward(*ins, dyt, ck, dst)
    buf = dst.clone()
    got = wkv.backward(*ins, dyt, ck, buf, ds0=buf)
    nods0 = wkv.backward(*ins, dyt, ck, dst, want_ds0=False)
    torch.cuda.synchronize()
    assert torch.equal(got[6], ref[6]) and got[6].data_ptr() == buf.data_ptr()
    for a, b, c in zip(ref[:6], got[:6], nods0[:6]):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_backward128_T0_copies_state_cotangent(wkv):
    z = torch.empty((2, 0, 3, N), dtype=torch.bfloat16, device="cuda")
    dst = torch.randn(2, 3, N, N, device="cuda")
    ck = torch.empty((2, 3, 0, N, N), device="cuda")
    *g, ds0 = wkv.backward(z, z, z, z, z, z, z, ck, dst)
    torch.cuda.synchronize()
    assert torch.equal(ds0, dst)
