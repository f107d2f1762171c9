"""Decode launches captured in a HIP graph (as the benchmark replays them):
every replay, with eager work and synchronisations in between, must equal the
eager run bit for bit."""
import numpy as np
import pytest

import synth
from tests.helpers import NAMES

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


def test_decode_graph_replays_match_eager(wkv):
    L, B, H, N, steps, reps = 3, 8, 5, 64, 4, 3
    pool0 = synth.decode_states_device(torch, "cuda", layers=L, B=B, H=H, N=N, seed=21)
    inp = synth.decode_step_inputs_device(torch, "cuda", B=B, H=H, N=N, seed=22,
                                          count=steps * L)

    # eager reference: `reps` runs of steps x layers, snapshots after each run
    pool_e = pool0.clone()
    y_e = torch.empty((steps * L, B, H, N), dtype=torch.bfloat16, device="cuda")
    snaps = []
    for _ in range(reps):
        for t in range(steps):
            for l in range(L):
                wkv.decode(*(inp[n][t * L + l] for n in NAMES), pool_e[l], y=y_e[t * L + l])
        torch.cuda.synchronize()
        snaps.append((pool_e.clone(), y_e.clone()))

    # captured graph of the same launch sequence
    pool_g = pool0.clone()
    y_g = torch.empty_like(y_e)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        for t in range(steps):
            for l in range(L):
                wkv.decode(*(inp[n][t * L + l] for n in NAMES), pool_g[l], y=y_g[t * L + l])
    torch.cuda.synchronize()
    assert torch.equal(pool_g, pool0)  # capture runs nothing
    side = pool0[0].clone()
    for rep in range(reps):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(pool_g, snaps[rep][0]), f"replay {rep}: state differs"
        assert torch.equal(y_g, snaps[rep][1]), f"replay {rep}: y differs"
        # eager work between replays
        wkv.decode(*(inp[n][0] for n in NAMES), side)
        _ = (side * 2).sum().item()
        torch.cuda.synchronize()
    assert np.isfinite(pool_g.cpu().numpy()).all()
