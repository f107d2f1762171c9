"""GPU parity of the chunked-parallel prefill (bf16 MFMA, fp32 state) against
the oracle through the C ABI.  Bound (bf16 inputs): max|err| / max|ref| <= 2e-2
for y and for the final state."""
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


def run(wkv, x, algo="chunked", d=None, **kw):
    d = d or to_device(x, torch)
    y, s = wkv.forward(*(d[n] for n in NAMES), s0=d["s0"], algo=algo, epilogue=d["epi"], **kw)
    torch.cuda.synchronize()
    return y, s


def check(wkv, x, what, **kw):
    y, s = run(wkv, x)
    y_ref, s_ref = oracle_forward(x, **kw)
    y, s = to_f64(y), to_f64(s)
    if kw:
        bi = kw.get("b_idx")
        hi = kw.get("h_idx")
        bi = slice(None) if bi is None else np.asarray(bi)
        hi = slice(None) if hi is None else np.asarray(hi)
        y, s = y[bi][:, :, hi], s[bi][:, hi]
    ey = assert_close(y, y_ref, TOL, f"{what} y")
    es = assert_close(s, s_ref, TOL, f"{what} S_T")
    return ey, es


def test_auto_picks_chunked_for_bf16(wkv):
    assert wkv.forward_workspace_bytes(2, 64, 3) >= 0
    x = synth.draw(1, 40, 2, seed=1, dtype="bf16", s0="normal")
    d = to_device(x, torch)
    ya, sa = run(wkv, x, algo="auto", d=d)
    yc, sc = run(wkv, x, algo="chunked", d=d)
    assert torch.equal(ya, yc) and torch.equal(sa, sc)


@pytest.mark.parametrize("T", [1, 2, 3, 15, 16, 17, 31, 32, 33, 47, 64, 65, 200, 1000])
def test_chunked_sweep_T(wkv, T):
    x = synth.draw(1, T, 1, seed=2000 + T, dtype="bf16", s0="normal")
    check(wkv, x, f"T={T}")


@pytest.mark.parametrize("B,H,T", [(3, 5, 37), (2, 1, 129), (1, 7, 48), (4, 3, 256)])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("s0", ["zero", "normal"])
@pytest.mark.parametrize("w_recipe", ["wide", "slow"])
def test_chunked_sweep(wkv, B, H, T, epi, s0, w_recipe):
    x = synth.draw(B, T, H, seed=B * 100 + H * 10 + T, dtype="bf16", s0=s0, w_recipe=w_recipe,
                   a_mean=2.0 if w_recipe == "slow" else 0.0, epilogue=epi)
    check(wkv, x, f"B{B} H{H} T{T} epi={epi} s0={s0} {w_recipe}")


def test_chunked_019b_shape(wkv):
    x = synth.config_inputs(1)
    ey, es = check(wkv, x, "cfg1")
    print(f"0.19B shape chunked: y err {ey:.2e}, S err {es:.2e}")


def test_chunked_29b_shape_with_epilogue(wkv):
    x = synth.config_inputs(2)
    ey, es = check(wkv, x, "cfg2")
    print(f"2.9B shape chunked+epilogue: y err {ey:.2e}, S err {es:.2e}")


def test_chunked_long_context_single_pass_and_segments(wkv):
    """T = 65536, slow decay, near-full replacement: one call (which splits the
    sequence into parallel segments) and 32 calls of 2048 tokens (each split
    into shorter segments of its own) with the state passed between them, both
    against the oracle, and the drift between the two."""
    x = synth.config_inputs(4)
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    assert wkv.forward_workspace_bytes(1, 65536, 40) > 0  # split into segments
    # the 2048-token calls are split too (into as many segments as the CUs allow)
    assert 0 < wkv.forward_workspace_bytes(1, 2048, 40) <= wkv.forward_workspace_bytes(1, 65536,
                                                                                       40)
    y1, s1 = wkv.forward(*ins, algo="chunked")
    st = torch.zeros_like(s1)
    ys = []
    for seg in range(32):
        sl = slice(seg * 2048, (seg + 1) * 2048)
        y, _ = wkv.forward(*(t[:, sl].contiguous() for t in ins), s0=st, s_out=st,
                           algo="chunked")
        ys.append(y)
    torch.cuda.synchronize()
    yseg = torch.cat(ys, 1)
    y_ref, s_ref = oracle_forward(x)
    e1 = assert_close(to_f64(y1), y_ref, TOL, "single pass y")
    assert_close(to_f64(s1), s_ref, TOL, "single pass S")
    e2 = assert_close(to_f64(yseg), y_ref, TOL, "segmented y")
    assert_close(to_f64(st), s_ref, TOL, "segmented S")
    drift = rel_err(to_f64(yseg), to_f64(y1))
    print(f"long context: single {e1:.2e}, segmented {e2:.2e}, drift {drift:.2e}")
    assert drift <= TOL


# Few heads and long sequences: the time axis is split into segments run in
# parallel; their transitions and offsets are combined into each segment's
# entry state (linearity of the update in the state).
# (1, 1, 512 / 640 / 768 / 896) give 4, 5, 6 and 7 segments, so the combine
# kernel's four-slot loop ends at every position of its last trip; the others
# give 32, 58, 35 and 63 segments.
@pytest.mark.parametrize("B,H,T", [(1, 1, 4096), (1, 2, 8229), (2, 3, 5000), (1, 1, 20000),
                                   (1, 1, 512), (1, 1, 640), (1, 1, 768), (1, 1, 896)])
@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("s0", ["zero", "normal"])
def test_segmented_sweep(wkv, B, H, T, epi, s0):
    assert wkv.forward_workspace_bytes(B, T, H) > 0
    x = synth.draw(B, T, H, seed=7 * T + B + H, dtype="bf16", s0=s0, w_recipe="wide",
                   epilogue=epi)
    check(wkv, x, f"segmented B{B} H{H} T{T} epi={epi} s0={s0}")


def test_segmented_in_place_and_pieces(wkv):
    """s_out == s0 with a split sequence, against the same tokens run as pieces
    of 2000 (each split differently) with the state passed between them."""
    x = synth.draw(1, 10000, 2, seed=71, dtype="bf16", s0="normal", w_recipe="slow",
                   a_mean=2.0, epilogue=True)
    d = to_device(x, torch)
    ins = [d[n] for n in NAMES]
    st = d["s0"].clone()
    y1, _ = wkv.forward(*ins, s0=st, s_out=st, epilogue=d["epi"], algo="chunked")
    sp = d["s0"].clone()
    ys = []
    for i in range(5):
        sl = slice(i * 2000, (i + 1) * 2000)
        y, _ = wkv.forward(*(t[:, sl].contiguous() for t in ins), s0=sp, s_out=sp,
                           epilogue=d["epi"], algo="chunked")
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle_forward(x)
    assert_close(to_f64(y1), y_ref, TOL, "split y")
    assert_close(to_f64(st), s_ref, TOL, "split S in place")
    assert_close(to_f64(torch.cat(ys, 1)), y_ref, TOL, "pieces y")
    assert rel_err(to_f64(st), to_f64(sp)) <= TOL


def test_segmented_workspace_too_small(wkv):
    x = synth.draw(1, 4096, 1, seed=72, dtype="bf16")
    d = to_device(x, torch)
    need = wkv.forward_workspace_bytes(1, 4096, 1)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(wkv.Rwkv7Error):
        wkv.forward(*(d[n] for n in NAMES), algo="chunked", workspace=ws)


def test_chunked_matches_scan(wkv):
    x = synth.draw(2, 300, 4, seed=44, dtype="bf16", s0="normal", w_recipe="wide",
                   epilogue=True)
    d = to_device(x, torch)
    yc, sc = run(wkv, x, "chunked", d=d)
    ys, ss = run(wkv, x, "scan", d=d)
    assert rel_err(to_f64(yc), to_f64(ys)) <= TOL
    assert rel_err(to_f64(sc), to_f64(ss)) <= TOL


def _transition_inputs(rng, T, B=2, H=3, N=64):
    """Per chunk, swaps on disjoint column pairs (so M_bk = 0 inside a chunk)
    with v = 0, w = 1 and small integer states: every intermediate is a small
    integer and the chunked form is exact."""
    S0 = rng.integers(-8, 9, (B, H, N, N)).astype(np.float32)
    kap = np.zeros((B, T, H, N), np.float32)
    a = np.zeros((B, T, H, N), np.float32)
    for t in range(T):
        pair = 2 * (t % 16)
        i, j = pair, pair + 1
        kap[:, t, :, i] = 1.0
        kap[:, t, :, j] = -1.0
        a[:, t, :, :] = 1.0 if t % 3 else 0.0
    r = rng.integers(-2, 3, (B, T, H, N)).astype(np.float32)
    vecs = dict(r=r, w=np.ones_like(r), k=r[..., ::-1].copy(), v=np.zeros_like(r), kappa=kap,
                a=a)
    return vecs, S0


@pytest.mark.parametrize("T", [1, 2, 16, 40, 4096 + 40])
def test_chunked_exact_transitions(wkv, T):
    """Exact also when the sequence is split: each segment's transition is a
    permutation matrix and its offset zero."""
    rng = np.random.default_rng(T)
    vecs, S0 = _transition_inputs(rng, T, B=1 if T > 4096 else 2)
    _, s_ref = oracle.forward(*(vecs[n] for n in NAMES), s0=S0)
    ins = [torch.from_numpy(np.ascontiguousarray(vecs[n])).to("cuda", torch.bfloat16)
           for n in NAMES]
    y, s = wkv.forward(*ins, s0=torch.from_numpy(S0).cuda(), algo="chunked")
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(s), s_ref)


def test_chunked_rejects_fp32(wkv):
    x = synth.draw(1, 8, 1, seed=3, dtype="f32")
    d = to_device(x, torch)
    with pytest.raises(wkv.Rwkv7Error):
        wkv.forward(*(d[n] for n in NAMES), algo="chunked")


@pytest.mark.parametrize("kind", ["lower end", "uniform"])
def test_chunked_decay_domain(wkv, kind):
    """The chunked form's stated decay domain 2^-6 <= w <= 1 (include/rwkv7_wkv.h):
    at its lower end every w = 2^-6, so the decay ratios inside a 16-token chunk
    reach 2^90; and w drawn uniformly over the domain."""
    if kind == "lower end":
        x = synth.draw(2, 200, 3, seed=81, dtype="bf16", s0="normal", w_const=2.0 ** -6)
    else:
        x = synth.draw(2, 200, 3, seed=82, dtype="bf16", s0="normal")
        rng = np.random.default_rng(83)
        w = rng.uniform(2.0 ** -6, 1.0, x["w"].shape).astype(np.float32)
        x["w"] = synth.f32_to_bf16_bits(w)
    assert synth.bf16_bits_to_f32(x["w"]).min() >= 2.0 ** -6
    check(wkv, x, f"decay domain, {kind}")


@pytest.mark.parametrize("epi", [False, True])
def test_variants_agree_bitwise(wkv, epi):
    """A launch with no more workgroups than compute units runs the variant whose
    ninth wave forms the triangular inverse; a larger one runs the eight-wave
    form.  Both do the same arithmetic, so the first batch of a large call equals
    a call made of that batch alone, bit for bit (readouts, final state and, in
    the training forward, every stored state).  T < 512 keeps both calls in one
    time segment."""
    H, T = 40, 500
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B = cus // H + 1  # B * H workgroups > compute units
    x = synth.draw(B, T, H, seed=4242, dtype="bf16", s0="normal", epilogue=epi)
    d = to_device(x, torch)
    y, s = run(wkv, x, d=d)
    one = {n: d[n][:1].contiguous() for n in NAMES}
    y1, s1 = wkv.forward(*(one[n] for n in NAMES), s0=d["s0"][:1].contiguous(), algo="chunked",
                         epilogue=d["epi"])
    torch.cuda.synchronize()
    assert torch.equal(y[:1], y1) and torch.equal(s[:1], s1)
    if not epi:
        _, st, ck = wkv.forward_train(*(d[n] for n in NAMES), s0=d["s0"], algo="chunked")
        _, st1, ck1 = wkv.forward_train(*(one[n] for n in NAMES), s0=d["s0"][:1].contiguous(),
                                        algo="chunked")
        torch.cuda.synchronize()
        assert torch.equal(st[:1], st1) and torch.equal(ck[:1], ck1)
    # and both agree with the oracle on that batch
    y_ref, s_ref = oracle_forward(x, b_idx=[0])
    assert_close(to_f64(y1), y_ref, TOL, "one batch y")
    assert_close(to_f64(s1), s_ref, TOL, "one batch S_T")
