"""The streaming copy kernel that the benchmark uses as its measured HBM ceiling:
every byte copied exactly, nothing written past the end, ragged last workgroups
included."""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def wkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_rnn_sequence_amd as m

    m.lib()
    return m


# 16-byte pieces: one piece, less than a wave, one workgroup (512 pieces) exactly,
# one more than a workgroup, several workgroups with a ragged last one, ~64 MB
@pytest.mark.parametrize("pieces", [1, 37, 512, 513, 2048, 5 * 512 + 333, 4 * 1024 * 1024 + 7])
def test_stream_copy_exact_and_bounded(wkv, pieces):
    g = torch.Generator(device="cuda").manual_seed(pieces)
    n = 4 * pieces
    src = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device="cuda", generator=g)
    guard = 1024
    dst = torch.full((n + guard,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    wkv.stream_copy(src, dst[:n])
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert bool((dst[n:] == 0x5A5A5A5A).all())


def test_stream_copy_rejects_overlap_and_size(wkv):
    x = torch.zeros(1024, dtype=torch.float32, device="cuda")
    with pytest.raises(wkv.Rwkv7Error):
        wkv.stream_copy(x[:512], x[256:768])
    with pytest.raises(ValueError):
        wkv.stream_copy(x[:512], x[512:1000])
