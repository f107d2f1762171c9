"""The binding rejects every state, output, epilogue and workspace tensor whose
shape, dtype, layout or device the kernels would misread, before any call
into the library (the C interface sees only pointers, not sizes).  CPU only:
stand-in tensors carry just the attributes the checks read; a call that got
past the checks would fail on them, so every case must raise in the checks."""
import pytest

torch = pytest.importorskip("torch")
import linear_rnn_sequence_amd as wkv  # noqa: E402


class Dev:
    def __init__(self, kind="cuda", index=0):
        self.type, self.index = kind, index

    def __eq__(self, other):
        return isinstance(other, Dev) and (self.type, self.index) == (other.type, other.index)

    def __repr__(self):
        return f"{self.type}:{self.index}"


class Fake:
    def __init__(self, shape, dtype=torch.bfloat16, device=None, contiguous=True):
        self.shape, self.dtype = tuple(shape), dtype
        self.device = device or Dev()
        self._contig = contiguous

    def is_contiguous(self):
        return self._contig

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n

    def element_size(self):
        return 2 if self.dtype == torch.bfloat16 else 4

    def data_ptr(self):
        raise AssertionError("the checks should have rejected this call first")


B, T, H, N = 2, 5, 3, 64
F32 = torch.float32


def ins(dtype=torch.bfloat16):
    return [Fake((B, T, H, N), dtype) for _ in range(6)]


def state(shape=(B, H, N, N), **kw):
    return Fake(shape, F32, **kw)


BAD_STATES = [
    ("shape", lambda: state((H, N, N))),
    ("heads", lambda: state((B, H - 1, N, N))),
    ("dtype", lambda: Fake((B, H, N, N), torch.bfloat16)),
    ("layout", lambda: state(contiguous=False)),
    ("device", lambda: state(device=Dev("cuda", 1))),
]


@pytest.mark.parametrize("what,make", BAD_STATES)
@pytest.mark.parametrize("arg", ["s0", "s_out"])
def test_forward_rejects_bad_state(what, make, arg):
    with pytest.raises((ValueError, TypeError)):
        wkv.forward(*ins(), **{arg: make()})


@pytest.mark.parametrize("what,make", BAD_STATES)
def test_forward_train_rejects_bad_states(what, make):
    with pytest.raises((ValueError, TypeError)):
        wkv.forward_train(*ins(), s0=make())
    with pytest.raises(ValueError):  # T = 5 stores one state per (b, h), not two
        wkv.forward_train(*ins(), s_ckpt=Fake((B, H, 2, N, N), F32))


def test_forward_rejects_bad_output_and_workspace():
    with pytest.raises(TypeError):
        wkv.forward(*ins(), y=Fake((B, T, H, N), F32))
    with pytest.raises(ValueError):
        wkv.forward(*ins(), y=Fake((B, T - 1, H, N)))
    with pytest.raises(ValueError):
        wkv.forward(*ins(), workspace=Fake((64,), torch.uint8, contiguous=False))


@pytest.mark.parametrize("key,bad", [("r_k", Fake((H * N,), torch.bfloat16)),
                                     ("r_k", Fake((H * N - 1,), F32)),
                                     ("ln_w", Fake((H * N,), F32, contiguous=False)),
                                     ("ln_b", Fake((H * N,), F32, device=Dev("cuda", 2)))])
def test_epilogue_rejected(key, bad):
    epi = {"ln_w": None, "ln_b": None, "r_k": Fake((H * N,), F32), "eps": 64e-5}
    epi[key] = bad
    with pytest.raises(ValueError):
        wkv.forward(*ins(), epilogue=epi)
    with pytest.raises(ValueError):
        wkv.decode(*(Fake((B, H, N)) for _ in range(6)), state(), epilogue=epi)


def test_bidir_states_have_two_passes():
    with pytest.raises(ValueError):
        wkv.forward_bidir(*ins(), s0=state())
    with pytest.raises(ValueError):
        wkv.forward_bidir(*ins(), s_out=state())


def test_decode_rejects_bad_state():
    for _, make in BAD_STATES:
        with pytest.raises((ValueError, TypeError)):
            wkv.decode(*(Fake((B, H, N)) for _ in range(6)), make())
    with pytest.raises(ValueError):
        wkv.decode(*(Fake((B, H, N)) for _ in range(6)), None)
    kk = Fake((H * N,), F32)
    with pytest.raises(ValueError):
        wkv.decode_fused(*(Fake((B, H, N)) for _ in range(5)), kk, kk, state((B - 1, H, N, N)))
    with pytest.raises(ValueError):
        wkv.prepare_decode(*(Fake((B, H, N)) for _ in range(6)), state((1, H, N, N)),
                           y=Fake((B, H, N)))


def test_backward_rejects_bad_tensors():
    base = ins()
    dy = Fake((B, T, H, N))
    ck = Fake((B, H, 1, N, N), F32)
    with pytest.raises(ValueError):
        wkv.backward(*base, dy, Fake((B, H, 2, N, N), F32))
    with pytest.raises((ValueError, TypeError)):
        wkv.backward(*base, dy, ck, ds_T=Fake((B, H, N, N), torch.bfloat16))
    with pytest.raises(ValueError):
        wkv.backward(*base, dy, ck, ds0=state((B, 1, N, N)))
    grads = [Fake((B, T, H, N)) for _ in range(6)]
    grads[3] = Fake((B, T, H, N), F32)
    with pytest.raises(TypeError):
        wkv.backward(*base, dy, ck, grads=tuple(grads))
    with pytest.raises(ValueError):
        wkv.backward(*base, dy, ck, grads=tuple(grads[:5]))
    # float32 decay: dw float32, the other gradients bf16
    w32 = ins()
    w32[1] = Fake((B, T, H, N), F32)
    grads = [Fake((B, T, H, N)) for _ in range(6)]  # dw bf16: wrong under a float32 decay
    with pytest.raises(TypeError):
        wkv.backward(*w32, dy, ck, grads=tuple(grads))
