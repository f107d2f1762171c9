"""GPU parity of the sequential scan and the decode step against the oracle,
through the C ABI.  Bound: max|y - y_ref| / max|y_ref| <= 1e-5 for fp32 inputs
and <= 2e-2 for bf16 inputs, for y and for the final state."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import NAMES, TOL, assert_close, oracle_forward, to_device, to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()  # fails loudly if the HIP library is missing
    return m


def run_forward(wkv, x, algo, **kw):
    d = to_device(x, torch)
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo=algo, epilogue=d["epi"], **kw)
    torch.cuda.synchronize()
    return y, s


def check_forward(wkv, x, algo, *, b_idx=None, h_idx=None, what=""):
    y, s = run_forward(wkv, x, algo)
    y_ref, s_ref = oracle_forward(x, b_idx=b_idx, h_idx=h_idx)
    y, s = to_f64(y), to_f64(s)
    if b_idx is not None or h_idx is not None:
        bi = slice(None) if b_idx is None else np.asarray(b_idx)
        hi = slice(None) if h_idx is None else np.asarray(h_idx)
        y, s = y[bi][:, :, hi], s[bi][:, hi]
    tol = TOL[x.dtype]
    ey = assert_close(y, y_ref, tol, f"{what} y")
    es = assert_close(s, s_ref, tol, f"{what} S_T")
    return ey, es


# ---------------------------------------------------------------------------
# the tiny fp32 workload and seeded sweeps over tile edges and ragged tails
# ---------------------------------------------------------------------------

def test_scan_tiny_fp32(wkv):
    x = synth.config_inputs(0)
    ey, es = check_forward(wkv, x, "scan", what="cfg0")
    print(f"cfg0 scan: y err {ey:.2e}, S err {es:.2e}")


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 63, 64, 65, 200])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_sweep_T(wkv, T, dtype):
    x = synth.draw(1, T, 1, seed=1000 + T, dtype=dtype, s0="normal")
    check_forward(wkv, x, "scan", what=f"T={T} {dtype}")


@pytest.mark.parametrize("B,H,T", [(3, 5, 37), (2, 1, 129), (1, 7, 48)])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("s0", ["zero", "normal"])
def test_scan_sweep_batch_heads(wkv, B, H, T, epi, s0):
    x = synth.draw(B, T, H, seed=B * 100 + H * 10 + T, dtype="bf16", s0=s0, w_recipe="wide",
                   epilogue=epi)
    check_forward(wkv, x, "scan", what=f"B{B} H{H} T{T} epi={epi} s0={s0}")


def test_scan_fp32_epilogue(wkv):
    x = synth.draw(2, 70, 3, seed=77, dtype="f32", s0="normal", epilogue=True)
    check_forward(wkv, x, "scan", what="fp32 epilogue")


def test_scan_019b_shape(wkv):
    x = synth.config_inputs(1)
    ey, es = check_forward(wkv, x, "scan", what="cfg1 scan")
    print(f"cfg1 scan: y err {ey:.2e}, S err {es:.2e}")


def test_scan_29b_shape_sampled_heads(wkv):
    x = synth.config_inputs(2)
    ey, es = check_forward(wkv, x, "scan", b_idx=[0, 5, 7], h_idx=[0, 13, 39], what="cfg2 scan")
    print(f"cfg2 scan (sampled heads): y err {ey:.2e}, S err {es:.2e}")


# ---------------------------------------------------------------------------
# boundary cases of the forward entry point
# ---------------------------------------------------------------------------

def test_zero_length_copies_state(wkv):
    x = synth.draw(2, 0, 3, seed=5, dtype="bf16", s0="normal")
    d = to_device(x, torch)
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo="scan")
    torch.cuda.synchronize()
    assert torch.equal(s, d["s0"])
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=None, algo="scan")
    torch.cuda.synchronize()
    assert torch.count_nonzero(s).item() == 0


def test_in_place_state_and_split_equals_single_pass(wkv):
    x = synth.draw(2, 90, 3, seed=6, dtype="bf16", s0="normal")
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    y_full, s_full = wkv.forward(*ins, s0=d["s0"], algo="scan")
    st = d["s0"].clone()
    ys = []
    for lo, hi in ((0, 23), (23, 64), (64, 90)):
        y, _ = wkv.forward(*(t[:, lo:hi].contiguous() for t in ins), s0=st, s_out=st,
                           algo="scan")
        ys.append(y)
    torch.cuda.synchronize()
    # the scan's per-token arithmetic does not depend on where a call starts
    assert torch.equal(torch.cat(ys, 1), y_full)
    assert torch.equal(st, s_full)


def test_hand_worked_example_embedded(wkv):
    """The N=2 worked example of tests/golden, embedded in a 64-wide head (zeros
    elsewhere); every intermediate is a small dyadic rational, so the result is exact."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_n2_t2.json")))
    T = 2
    vec = {}
    for n in NAMES:
        a = np.zeros((1, T, 1, 64), np.float32)
        a[0, :, 0, :2] = np.array(g[n], np.float32)
        vec[n] = a
    vec["w"][0, :, 0, 2:] = 1.0
    s0 = np.zeros((1, 1, 64, 64), np.float32)
    s0[0, 0, :2, :2] = np.array(g["s0"], np.float32)
    for dt in (torch.float32, torch.bfloat16):
        ins = [torch.from_numpy(vec[n]).to("cuda", dt) for n in NAMES]
        y, s = wkv.forward(*ins, s0=torch.from_numpy(s0).cuda(), algo="scan")
        torch.cuda.synchronize()
        yc = to_f64(y)
        assert np.array_equal(yc[0, :, 0, :2], np.array(g["y"]))
        assert np.count_nonzero(yc[0, :, 0, 2:]) == 0
        assert np.array_equal(to_f64(s)[0, 0, :2, :2], np.array(g["s_T"]))


@pytest.mark.parametrize("entry", ["scan", "decode"])
def test_elementary_transitions_bitwise(wkv, entry):
    """Swap / copy / identity transitions from a key and a binary gate (v = 0,
    w = 1, integer state) are exact in any precision: the GPU must match bitwise."""
    rng = np.random.default_rng(3)
    B, H, N = 2, 3, 64
    S0 = rng.integers(-64, 65, (B, H, N, N)).astype(np.float32)
    e = np.eye(N, dtype=np.float32)
    cases = [((e[3] - e[40]), np.ones(N, np.float32)),            # swap 3 <-> 40
             ((e[17] - e[5]), e[17]),                              # column 17 <- column 5
             (rng.standard_normal(N).astype(np.float32), np.zeros(N, np.float32))]  # identity
    for kap, a in cases:
        # bf16-exact values, so the GPU and the oracle see the same numbers
        r = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32)))
        vecs = dict(r=r, w=np.ones(N, np.float32), k=r[::-1].copy(), v=np.zeros(N, np.float32),
                    kappa=kap.astype(np.float32), a=a.astype(np.float32))
        want = oracle.forward(*(np.broadcast_to(vecs[n], (B, 1, H, N)) for n in NAMES), s0=S0)[1]
        ins = {n: torch.from_numpy(np.ascontiguousarray(np.broadcast_to(vecs[n], (B, 1, H, N))))
               .to("cuda", torch.bfloat16) for n in NAMES}
        st = torch.from_numpy(S0).cuda()
        if entry == "scan":
            _, s = wkv.forward(*(ins[n] for n in NAMES), s0=st, algo="scan")
        else:
            wkv.decode(*(ins[n][:, 0].contiguous() for n in NAMES), st)
            s = st
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(s), want)


# ---------------------------------------------------------------------------
# decode: one token over resident states
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("epi", [False, True])
def test_decode_steps(wkv, dtype, epi):
    B, H, steps = 5, 7, 4
    x = synth.draw(B, steps, H, seed=31, dtype=dtype, s0="normal", epilogue=epi)
    d = to_device(x, torch)
    st = d["s0"].clone()
    ys = []
    for t in range(steps):
        ys.append(wkv.decode(*(d[n][:, t].contiguous() for n in NAMES), st, epilogue=d["epi"]))
    torch.cuda.synchronize()
    y = np.stack([to_f64(v) for v in ys], 1)
    y_ref, s_ref = oracle_forward(x)
    assert_close(y, y_ref, TOL[dtype], "decode y")
    assert_close(to_f64(st), s_ref, TOL[dtype], "decode S")


def test_decode_29b_pool_slices(wkv):
    """Layer-major pool [L, B=256, H=40, N, N]; each call updates one layer's slice."""
    L, B, H, N = 2, 256, 40, 64
    pool = synth.decode_states_device(torch, "cuda", layers=L, B=B, H=H, N=N, seed=3)
    s0 = pool.cpu().numpy()
    inp = synth.decode_step_inputs_device(torch, "cuda", B=B, H=H, N=N, seed=4, count=3 * L)
    ys = {}
    for t in range(3):
        for l in range(L):
            ys[(t, l)] = wkv.decode(*(inp[n][t * L + l] for n in NAMES), pool[l])
    torch.cuda.synchronize()
    host = {n: inp[n].float().cpu().numpy() for n in NAMES}
    for l in range(L):
        seq = {n: np.stack([host[n][t * L + l] for t in range(3)], 1) for n in NAMES}
        y_ref, s_ref = oracle.forward(*(seq[n] for n in NAMES), s0=s0[l])
        y = np.stack([to_f64(ys[(t, l)]) for t in range(3)], 1)
        assert_close(y, y_ref, 2e-2, f"pool layer {l} y")
        assert_close(to_f64(pool[l]), s_ref, 2e-2, f"pool layer {l} S")


def test_decode_matches_scan(wkv):
    x = synth.draw(3, 6, 4, seed=12, dtype="f32", s0="normal")
    d = to_device(x, torch)
    y_scan, s_scan = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo="scan")
    st = d["s0"].clone()
    ys = [wkv.decode(*(d[n][:, t].contiguous() for n in NAMES), st) for t in range(6)]
    torch.cuda.synchronize()
    assert_close(to_f64(torch.stack(ys, 1)), to_f64(y_scan), 1e-5, "decode vs scan y")
    assert_close(to_f64(st), to_f64(s_scan), 1e-5, "decode vs scan S")
