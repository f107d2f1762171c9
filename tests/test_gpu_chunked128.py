"""GPU parity of the chunked-parallel prefill at head size 128 (bf16 MFMA,
float32 state; eight chain waves, two prep groups of 64 keys) against the
oracle through the C ABI.  The pages tune their kernels for head size 64 and
name larger heads as less efficient (RWKV-7 "Goose" summary, §8 Speed and
Memory); the oracle takes any head size.  Bound (bf16 inputs): max|err| /
max|ref| <= 2e-2 for y and the final state."""
import numpy as np
import pytest

import synth
from tests.helpers import NAMES, assert_close, oracle_forward, rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 2e-2
N = 128


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def run(wkv, x, algo="chunked", d=None):
    d = d or to_device(x, torch)
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo=algo, epilogue=d["epi"])
    torch.cuda.synchronize()
    return y, s


def check(wkv, x, what, algo="chunked"):
    y, s = run(wkv, x, algo)
    y_ref, s_ref = oracle_forward(x)
    ey = assert_close(to_f64(y), y_ref, TOL, f"{what} y")
    es = assert_close(to_f64(s), s_ref, TOL, f"{what} S_T")
    return ey, es


def test_auto_picks_chunked_at_128(wkv):
    assert wkv.forward_workspace_bytes(1, 100000, 1, N) == 0  # no segments at 128
    x = synth.draw(1, 40, 2, N, seed=1281, dtype="bf16", s0="normal")
    d = to_device(x, torch)
    ya, sa = run(wkv, x, "auto", d)
    yc, sc = run(wkv, x, "chunked", d)
    assert torch.equal(ya, yc) and torch.equal(sa, sc)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 64, 200, 1000])
def test_chunked128_sweep_T(wkv, T):
    x = synth.draw(1, T, 1, N, seed=1300 + T, dtype="bf16", s0="normal")
    check(wkv, x, f"N128 T={T}")


@pytest.mark.parametrize("B,H,T", [(2, 3, 37), (1, 5, 256), (3, 2, 130)])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("w_recipe", ["wide", "slow"])
def test_chunked128_sweep(wkv, B, H, T, epi, w_recipe):
    x = synth.draw(B, T, H, N, seed=B * 100 + H * 10 + T, dtype="bf16", s0="normal",
                   w_recipe=w_recipe, a_mean=2.0 if w_recipe == "slow" else 0.0, epilogue=epi)
    check(wkv, x, f"N128 B{B} H{H} T{T} epi={epi} {w_recipe}")


def test_chunked128_fp32_decay(wkv):
    x = synth.draw(2, 300, 2, N, seed=1310, dtype="bf16_w32", s0="normal", w_recipe="slow",
                   a_mean=2.0, epilogue=True)
    check(wkv, x, "N128 fp32 decay")


@pytest.mark.parametrize("cos,align,rate,w", [(0.99, False, "one", 1.0), (0.9, False, "s2", 0.995),
                                              (0.8, True, "one", 0.995)])
def test_chunked128_correlated_keys(wkv, cos, align, rate, w):
    ra = dict(a_const=1.0) if rate == "one" else dict(a_mean=2.0)
    x = synth.draw(2, 200, 2, N, seed=1320, dtype="bf16", kappa_cos=cos, k_align=align,
                   w_const=w, s0="normal", **ra)
    check(wkv, x, f"N128 correlated cos={cos}")


def test_chunked128_matches_scan(wkv):
    x = synth.draw(2, 300, 3, N, seed=1330, dtype="bf16", s0="normal", w_recipe="wide",
                   epilogue=True)
    d = to_device(x, torch)
    yc, sc = run(wkv, x, "chunked", d)
    ys, ss = run(wkv, x, "scan", d)
    assert rel_err(to_f64(yc), to_f64(ys)) <= TOL
    assert rel_err(to_f64(sc), to_f64(ss)) <= TOL


def test_chunked128_in_place_and_chained(wkv):
    """s_out == s0, and three calls with the state passed between them equal one."""
    x = synth.draw(1, 480, 2, N, seed=1340, dtype="bf16", s0="normal", w_recipe="slow",
                   a_mean=2.0)
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    y1, s1 = wkv.forward(*ins, s0=d["s0"], algo="chunked")
    st = d["s0"].clone()
    ys = []
    for i in range(3):
        sl = slice(160 * i, 160 * (i + 1))
        y, _ = wkv.forward(*(t[:, sl].contiguous() for t in ins), s0=st, s_out=st,
                           algo="chunked")
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_forward(x)
    assert_close(to_f64(y1), y_ref, TOL, "one call y")
    assert_close(to_f64(torch.cat(ys, 1)), y_ref, TOL, "chained y")
    assert_close(to_f64(st), s_ref, TOL, "chained S (in place)")
    assert rel_err(to_f64(st), to_f64(s1)) <= TOL


def test_chunked128_exact_transitions(wkv):
    """Swaps on disjoint key pairs within each chunk, v = 0, w = 1, small integer
    states: every intermediate is a small integer, so the final state is exact."""
    rng = np.random.default_rng(1350)
    B, H, T = 2, 2, 70
    S0 = rng.integers(-8, 9, (B, H, N, N)).astype(np.float32)
    kap = np.zeros((B, T, H, N), np.float32)
    a = np.zeros((B, T, H, N), np.float32)
    for t in range(T):
        i = 2 * (t % 16) + 64 * (t % 2)
        kap[:, t, :, i] = 1.0
        kap[:, t, :, i + 1] = -1.0
        a[:, t, :, :] = 1.0 if t % 3 else 0.0
    r = rng.integers(-2, 3, (B, T, H, N)).astype(np.float32)
    vecs = dict(r=r, w=np.ones_like(r), k=r[..., ::-1].copy(), v=np.zeros_like(r), kappa=kap,
                a=a)
    import oracle
    _, s_ref = oracle.forward(*(vecs[n] for n in NAMES), s0=S0)
    ins = [torch.from_numpy(np.ascontiguousarray(vecs[n])).to("cuda", torch.bfloat16)
           for n in NAMES]
    _, s = wkv.forward(*ins, s0=torch.from_numpy(S0).cuda(), algo="chunked")
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(s), s_ref)


def test_chunked128_rejected_where_not_built(wkv):
    """At head size 128 the chunked algorithm serves the plain and the training
    forward; the bidirectional forward and the backward refuse it."""
    x = synth.draw(1, 20, 1, N, seed=1360, dtype="bf16")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    y, s, ck = wkv.forward_train(*ins, algo="chunked")
    y0, s0 = wkv.forward(*ins, algo="chunked")
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(s, s0)
    with pytest.raises(wkv.Rwkv7Error):
        wkv.forward_bidir(*ins, algo="chunked")
    with pytest.raises(wkv.Rwkv7Error):
        wkv.backward(*ins, ins[0], ck, None, algo="chunked")
