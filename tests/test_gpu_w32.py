"""bf16 inputs with a float32 decay (RWKV7_DT_BF16_W32) against the oracle on
the same values: slow forgetting, w in (0.99, 1), which bf16 rounds to exactly
1 for most channels.  Bound 2e-2 (bf16 inputs)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import NAMES, assert_close, oracle_forward, rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 2e-2


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def slow(B, T, H, seed, **kw):
    return synth.draw(B, T, H, seed=seed, dtype="bf16_w32", w_recipe="slow", a_mean=2.0, **kw)


@pytest.mark.parametrize("algo", ["chunked", "scan"])
@pytest.mark.parametrize("B,H,T,epi", [(2, 3, 300, False), (1, 4, 1000, True), (3, 1, 47, True)])
def test_forward_fp32_decay(wkv, algo, B, H, T, epi):
    x = slow(B, T, H, seed=T + H, s0="normal", epilogue=epi)
    assert x["w"].dtype == np.float32 and x["r"].dtype == np.uint16
    d = to_device(x, torch)
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo=algo, epilogue=d["epi"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_forward(x)
    assert_close(to_f64(y), y_ref, TOL, f"{algo} y")
    assert_close(to_f64(s), s_ref, TOL, f"{algo} S")


def test_fp32_decay_matters(wkv):
    """Slow decay with slow replacement (a ~ sigmoid(N(-3, 1))): the same draws
    with w rounded to bf16 land far outside the bound of the float32-decay
    result (an input effect: they match the oracle run on the rounded w), while
    the float32-decay path stays inside it."""
    x = synth.draw(1, 2000, 2, seed=5, dtype="bf16_w32", w_recipe="slow", a_mean=-3.0)
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    y32, _ = wkv.forward(*ins, algo="chunked")
    ins16 = list(ins)
    ins16[1] = ins[1].to(torch.bfloat16)
    y16, _ = wkv.forward(*ins16, algo="chunked")
    torch.cuda.synchronize()
    y_ref, _ = oracle_forward(x)
    w16 = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x["w"])).astype(np.float64)
    y_ref16, _ = oracle.forward(*(w16 if n == "w" else x.as_f64(n) for n in NAMES))
    assert rel_err(to_f64(y32), y_ref) <= TOL
    assert rel_err(to_f64(y16), y_ref16) <= TOL
    assert rel_err(to_f64(y16), y_ref) > 4 * TOL


def test_segmented_fp32_decay(wkv):
    assert wkv.forward_workspace_bytes(1, 6000, 2, dtype="bf16") > 0
    x = slow(1, 6000, 2, seed=9, s0="normal")
    d = to_device(x, torch)
    st = d["s0"].clone()
    y, _ = wkv.forward(*(d[n] for n in NAMES), s0=st, s_out=st, algo="chunked")
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_forward(x)
    assert_close(to_f64(y), y_ref, TOL, "segmented y")
    assert_close(to_f64(st), s_ref, TOL, "segmented S")


@pytest.mark.parametrize("epi", [False, True])
def test_decode_fp32_decay(wkv, epi):
    x = slow(8, 1, 5, seed=13, s0="normal", epilogue=epi)
    d = to_device(x, torch)
    st = d["s0"].clone()
    y = wkv.decode(*(d[n][:, 0].contiguous() for n in NAMES), st, epilogue=d["epi"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_forward(x)
    assert_close(to_f64(y), y_ref[:, 0], TOL, "decode y")
    assert_close(to_f64(st), s_ref, TOL, "decode S")


def test_train_forward_fp32_decay_stores_states(wkv):
    x = slow(1, 100, 2, seed=17, s0="normal")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    y, s, ck = wkv.forward_train(*ins, s0=d["s0"], algo="chunked")
    y0, s0 = wkv.forward(*ins, s0=d["s0"], algo="chunked")
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(s, s0)
    _, s16 = oracle.forward(*(x.as_f64(n)[:, :16] for n in NAMES), s0=x["s0"])
    assert_close(to_f64(ck[:, :, 1]), s16, TOL, "stored state at token 16")


@pytest.mark.parametrize("B,H,T,with_dsT", [(1, 2, 100, True), (2, 3, 300, True),
                                            (1, 1, 17, True), (1, 2, 16, False),
                                            (2, 1, 1, False)])
def test_backward_fp32_decay_chunked(wkv, B, H, T, with_dsT):
    """Both backward algorithms with a float32 decay (dw float32 as well) against
    the float64 autograd oracle on the same values."""
    from oracle import grad as og

    x = slow(B, T, H, seed=40 + T, s0="normal")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    _, _, ck = wkv.forward_train(*ins, s0=d["s0"], algo="chunked")
    dy_bits, ds_T = synth.cotangents(B, T, H, seed=41 + T, dtype="bf16", with_state=with_dsT)
    dy = torch.from_numpy(dy_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dst = None if ds_T is None else torch.from_numpy(ds_T).cuda()
    *g, ds0 = wkv.backward(*ins, dy, ck, dst)
    torch.cuda.synchronize()
    assert g[1].dtype == torch.float32 and g[0].dtype == torch.bfloat16
    ref = og.backward(*(x.as_f64(n) for n in NAMES),
                      synth.bf16_bits_to_f32(dy_bits).astype(np.float64), s0=x["s0"],
                      ds_T=None if ds_T is None else ds_T.astype(np.float64))
    for n, gt in zip(NAMES, g):
        assert_close(to_f64(gt), ref[n], TOL, f"d{n}")
    assert_close(to_f64(ds0), ref["s0"], TOL, "ds0")
    *g, ds0 = wkv.backward(*ins, dy, ck, dst, algo="scan")
    torch.cuda.synchronize()
    assert g[1].dtype == torch.float32 and g[0].dtype == torch.bfloat16
    for n, gt in zip(NAMES, g):
        assert_close(to_f64(gt), ref[n], TOL, f"scan d{n}")
    assert_close(to_f64(ds0), ref["s0"], TOL, "scan ds0")


def test_backward_fp32_decay_ds0_in_place_and_optional(wkv):
    """ds0 written over ds_T, or not at all: the six gradients are the same bits."""
    x = slow(1, 50, 2, seed=61, s0="normal")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    _, _, ck = wkv.forward_train(*ins, s0=d["s0"])
    dy_bits, ds_T = synth.cotangents(1, 50, 2, seed=62, dtype="bf16")
    dy = torch.from_numpy(dy_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dst = torch.from_numpy(ds_T).cuda()
    ref = wkv.backward(*ins, dy, ck, dst)
    buf = dst.clone()
    got = wkv.backward(*ins, dy, ck, buf, ds0=buf)
    nods0 = wkv.backward(*ins, dy, ck, dst, want_ds0=False)
    torch.cuda.synchronize()
    assert torch.equal(got[6], ref[6]) and got[6].data_ptr() == buf.data_ptr()
    for a, b, c in zip(ref[:6], got[:6], nods0[:6]):
        assert torch.equal(a, b) and torch.equal(a, c)
    assert ref[1].dtype == torch.float32 and nods0[6] is None
