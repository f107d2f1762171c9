"""GPU checks of the non-finite contract (include/rwkv7_wkv.h): a NaN or Inf in
one token's inputs of one (batch, head) propagates to that pair's readouts from
that token on and to its final state, never to another pair, and never to the
readouts of earlier tokens -- for the chunked algorithm, of earlier 16-token
chunks (the tokens of its own chunk before it may become non-finite too, since
the chunk's tokens meet in one matrix product).  Each run is compared with the
same inputs without the non-finite value."""
import numpy as np
import pytest

import synth
from tests.helpers import NAMES, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

B, T, H = 2, 100, 3
T0 = 37  # token that receives the non-finite value (chunk 2 holds tokens 32..47)


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def poisoned(d, name, value):
    out = {n: (t.clone() if torch.is_tensor(t) else t) for n, t in d.items()}
    out[name][0, T0, 1, 5] = value  # batch 0, token T0, head 1, channel 5
    return out


def split_check(y_clean, y_bad, s_clean, s_bad, first_affected):
    """Untouched pairs and earlier tokens bitwise equal; the pair's readout at T0
    and its final state non-finite."""
    yc, yb = y_clean.float().cpu(), y_bad.float().cpu()
    sc, sb = s_clean.cpu(), s_bad.cpu()
    others = [(b, h) for b in range(B) for h in range(H) if (b, h) != (0, 1)]
    for b, h in others:
        assert torch.equal(yc[b, :, h], yb[b, :, h]), (b, h)
        assert torch.equal(sc[b, h], sb[b, h]), (b, h)
    assert torch.equal(yc[0, :first_affected, 1], yb[0, :first_affected, 1])
    assert not torch.isfinite(yb[0, T0, 1]).all()
    assert not torch.isfinite(sb[0, 1]).all()


@pytest.mark.parametrize("name", ["v", "kappa", "r", "k", "w"])
@pytest.mark.parametrize("value", [float("nan"), float("inf")])
@pytest.mark.parametrize("dtype,algo", [("f32", "scan"), ("bf16", "scan"), ("bf16", "chunked")])
@pytest.mark.parametrize("epi", [False, True])
def test_forward_nonfinite_input(wkv, name, value, dtype, algo, epi):
    if name == "w" and value == float("inf"):
        pytest.skip("an infinite decay lies outside every algorithm's domain; NaN covers w")
    x = synth.draw(B, T, H, seed=91, dtype=dtype, s0="normal", epilogue=epi)
    d = to_device(x, torch)
    bad = poisoned(d, name, value)
    run = lambda dd: wkv.forward(*(dd[n] for n in NAMES), s0=dd["s0"], algo=algo,
                                 epilogue=dd["epi"])
    yc, sc = run(d)
    yb, sb = run(bad)
    torch.cuda.synchronize()
    if name == "r" and not epi:
        # the readout alone: only y at T0 changes (the state never sees r)
        assert not torch.isfinite(yb[0, T0, 1].float()).all()
        assert torch.equal(sc.cpu(), sb.cpu())
        return
    first = T0 if algo == "scan" else T0 // 16 * 16
    if name == "r":  # with the epilogue: the readout's norm, not the state
        assert not torch.isfinite(yb[0, T0, 1].float()).all()
        assert torch.equal(yc[0, :first, 1].cpu(), yb[0, :first, 1].cpu())
        return
    split_check(yc, yb, sc, sb, first)


@pytest.mark.parametrize("name", ["v", "kappa", "w"])
def test_decode_nonfinite_input(wkv, name):
    """One step of single-token decode per token of the sequence: the poisoned
    pair's state turns non-finite at T0, the others and the earlier steps not."""
    x = synth.draw(B, T, H, seed=92, dtype="bf16", s0="normal")
    d = to_device(x, torch)
    bad = poisoned(d, name, float("nan"))

    def run(dd):
        st = dd["s0"].clone()
        ys = [wkv.decode(*(dd[n][:, t].contiguous() for n in NAMES), st) for t in range(T)]
        return torch.stack(ys, 1), st

    yc, sc = run(d)
    yb, sb = run(bad)
    torch.cuda.synchronize()
    split_check(yc, yb, sc, sb, T0)
