"""GPU parity in the delta-rule regime: removal keys that repeat or correlate
within a sequence, so that each key overwrites what the state holds for it
(RWKV-7 "Goose" summary, §2 Background: the delta rule as a special case, and
App. D.3), with rates a = sigmoid(N(2, 1)) or 1 and decays 0.995 or 1.  Here
the chunked form couples the removal probes of a chunk's tokens strongly, and
the triangular inverse it needs is far from the identity.

Covered: the chunked forward (one call, split into parallel segments, fused
prologue, bidirectional), the chunked backward, the scan and decode, and the
replacement invariant S_t kappa_t = v_t (k_t . kappa_t) on the chunked
kernel's stored states.  Bound: max|err| / max|ref| <= 2e-2 (bf16 inputs)."""
import numpy as np
import pytest

import oracle
import synth
from oracle import grad as og
from tests.helpers import NAMES, assert_close, oracle_forward, to_device, to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 2e-2

# (mean pairwise cosine of the removal keys, written key along the removal key)
KEYS = [(0.5, False), (0.9, False), (0.99, False), (1.0, False), (0.5, True), (0.8, True)]
RATES = [("s2", 0.995), ("s2", 1.0), ("one", 0.995), ("one", 1.0)]


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def draw(B, T, H, seed, cos, align, rate, w, **kw):
    ra = dict(a_const=1.0) if rate == "one" else dict(a_mean=2.0)
    return synth.draw(B, T, H, seed=seed, dtype="bf16", kappa_cos=cos, k_align=align,
                      w_const=w, **ra, **kw)


def check_forward(wkv, x, algo, what):
    d = to_device(x, torch)
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo=algo, epilogue=d["epi"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_forward(x)
    assert_close(to_f64(y), y_ref, TOL, what + " y")
    assert_close(to_f64(s), s_ref, TOL, what + " S")


@pytest.mark.parametrize("cos,align", KEYS)
@pytest.mark.parametrize("rate,w", RATES)
def test_chunked_correlated_keys(wkv, cos, align, rate, w):
    x = draw(2, 300, 3, 500 + int(cos * 100) + 7 * align, cos, align, rate, w, s0="normal")
    check_forward(wkv, x, "chunked", f"chunked cos={cos} align={align} a={rate} w={w}")


@pytest.mark.parametrize("cos,align", [(0.99, False), (1.0, False), (0.8, True)])
def test_chunked_correlated_keys_epilogue_wide_decay(wkv, cos, align):
    """The 2.9B-shape recipe's widened decays and the fused epilogue."""
    ra = dict(a_mean=2.0)
    x = synth.draw(2, 257, 4, seed=510, dtype="bf16", kappa_cos=cos, k_align=align,
                   w_recipe="wide", epilogue=True, **ra)
    check_forward(wkv, x, "chunked", f"chunked+epilogue cos={cos} align={align}")


@pytest.mark.parametrize("cos,align,rate,w", [(0.99, False, "one", 1.0), (0.9, False, "s2", 0.995),
                                              (0.8, True, "one", 0.995)])
def test_scan_correlated_keys(wkv, cos, align, rate, w):
    x = draw(2, 200, 2, 520, cos, align, rate, w, s0="normal")
    check_forward(wkv, x, "scan", f"scan cos={cos}")


@pytest.mark.parametrize("cos,align,rate,w", [(0.99, False, "one", 1.0), (1.0, False, "s2", 0.995),
                                              (0.8, True, "one", 1.0)])
def test_segmented_correlated_keys(wkv, cos, align, rate, w):
    """Long enough to be split into parallel time segments, whose transitions
    are the products of the chunks' transitions."""
    assert wkv.forward_workspace_bytes(1, 8229, 2) > 0
    x = draw(1, 8229, 2, 530, cos, align, rate, w, s0="normal")
    check_forward(wkv, x, "chunked", f"segmented cos={cos} align={align} a={rate} w={w}")


@pytest.mark.parametrize("cos,rate,w", [(0.99, "one", 1.0), (0.9, "s2", 0.995)])
def test_fused_correlated_keys(wkv, cos, rate, w):
    """Raw keys along a shared direction: the prologue's kappa = normalise(k * k_k)
    inherits the correlation (k_k ~ N(1, 0.1))."""
    B, T, H = 2, 200, 2
    x = draw(B, T, H, 540, cos, True, rate, w, s0="normal", epilogue=True)
    k_k, k_a, g = synth.prologue_extras(B, T, H, seed=541)
    d = to_device(x, torch)
    dev = lambda a: (torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
                     if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    y, s = wkv.forward_fused(d["r"], d["w"], d["k"], d["v"], d["a"], dev(k_k), dev(k_a),
                             g=dev(g), s0=d["s0"], algo="chunked", epilogue=d["epi"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward_fused(*(x.as_f64(n) for n in ("r", "w", "k", "v", "a")), k_k,
                                        k_a, g=synth.bf16_bits_to_f32(g).astype(np.float64),
                                        s0=x["s0"], epilogue=x["epi"])
    assert_close(to_f64(y), y_ref, TOL, "fused y")
    assert_close(to_f64(s), s_ref, TOL, "fused S")


@pytest.mark.parametrize("cos,rate,w", [(0.99, "one", 1.0), (0.9, "s2", 0.995)])
def test_bidir_correlated_keys(wkv, cos, rate, w):
    x = draw(2, 150, 2, 550, cos, False, rate, w, epilogue=True)
    d = to_device(x, torch)
    y, s = wkv.forward_bidir(*(d[n] for n in NAMES), algo="chunked", epilogue=d["epi"])
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.forward_bidir(*(x.as_f64(n) for n in NAMES), epilogue=x["epi"])
    assert_close(to_f64(y), y_ref, TOL, "bidir y")
    assert_close(to_f64(s), s_ref, TOL, "bidir S")


def test_decode_correlated_keys(wkv):
    """Single-token steps over the same correlated sequence, the state kept."""
    x = draw(2, 48, 3, 560, 0.99, False, "one", 1.0, s0="normal")
    d = to_device(x, torch)
    st = d["s0"].clone()
    ys = []
    for t in range(48):
        y = wkv.decode(*(d[n][:, t].contiguous() for n in NAMES), st)
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_forward(x)
    assert_close(to_f64(torch.stack(ys, 1)), y_ref, TOL, "decode y")
    assert_close(to_f64(st), s_ref, TOL, "decode S")


@pytest.mark.parametrize("cos,align,rate,w", [(0.99, False, "one", 1.0), (1.0, False, "s2", 0.995),
                                              (0.9, False, "one", 0.995), (0.8, True, "one", 1.0)])
def test_chunked_backward_correlated_keys(wkv, cos, align, rate, w):
    B, T, H = 1, 100, 2
    x = draw(B, T, H, 570, cos, align, rate, w, s0="normal")
    dy, ds_T = synth.cotangents(B, T, H, seed=571)
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    dyt = torch.from_numpy(dy.view(np.int16)).cuda().view(torch.bfloat16)
    _, _, ck = wkv.forward_train(*ins, s0=d["s0"], algo="chunked")
    *g, ds0 = wkv.backward(*ins, dyt, ck, torch.from_numpy(ds_T).cuda(), algo="chunked")
    torch.cuda.synchronize()
    ref = og.backward(*(x.as_f64(n) for n in NAMES), synth.bf16_bits_to_f32(dy).astype(np.float64),
                      s0=x["s0"], ds_T=ds_T.astype(np.float64))
    for n, gt in zip(NAMES, g):
        assert_close(to_f64(gt), ref[n], TOL, f"backward d{n} cos={cos} a={rate} w={w}")
    assert_close(to_f64(ds0), ref["s0"], TOL, "backward ds0")


@pytest.mark.parametrize("flip,align", [(0.02, False), (0.1, False), (0.0, True)])
def test_replacement_invariant_on_stored_states(wkv, flip, align):
    """a = 1, w = 1 and removal keys of norm exactly 1 (entries +-1/8): after every
    token the state maps its removal key to the written value, S_t kappa_t =
    v_t (k_t . kappa_t), whatever it held before.  Checked on the chunked
    training forward's stored states (the state after every 16th token) and
    its final state, in float64 from the stored float32 states.  The bound is
    the state's: relative to the larger of max|v_t (k_t . kappa_t)| and the
    largest state entry (with written keys independent of the removal keys the
    state grows to ~20x the response checked here, and its float32 entries
    carry the chunked form's bf16-operand error relative to their own size)."""
    B, T, H = 2, 200, 2
    x = synth.draw(B, T, H, seed=580, dtype="bf16", kappa_signs=flip, k_align=align,
                   a_const=1.0, w_const=1.0, s0="normal")
    assert np.array_equal(np.linalg.norm(x.as_f64("kappa"), axis=-1), np.ones((B, T, H)))
    d = to_device(x, torch)
    _, s_T, ck = wkv.forward_train(*(d[n] for n in NAMES), s0=d["s0"], algo="chunked")
    torch.cuda.synchronize()
    ck, s_T = to_f64(ck), to_f64(s_T)  # ck[:, :, c] = state before token 16c
    kap, k, v = x.as_f64("kappa"), x.as_f64("k"), x.as_f64("v")
    ts = list(range(15, T - 1, 16)) + [T - 1]
    states = [ck[:, :, (t + 1) // 16] for t in ts[:-1]] + [s_T]
    lhs = np.stack([np.einsum("bhij,bhj->bhi", S, kap[:, t]) for S, t in zip(states, ts)])
    rhs = np.stack([v[:, t] * np.sum(k[:, t] * kap[:, t], -1, keepdims=True) for t in ts])
    scale = max(np.abs(rhs).max(), max(np.abs(S).max() for S in states))
    err = np.abs(lhs - rhs).max() / scale
    assert np.isfinite(lhs).all() and err <= TOL, (
        f"S_t kappa_t vs v_t (k_t . kappa_t), flip={flip}: {err:.3e} > {TOL}")
