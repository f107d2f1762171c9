"""Host-side checks of the C ABI that need no GPU: the built library loads,
exports every function include/rwkv7_wkv.h declares, and rejects bad
arguments before anything is enqueued (these calls launch nothing)."""
import ctypes
import os
import re

import pytest

from linear_rnn_sequence_amd import build as hbuild
from linear_rnn_sequence_amd import wkv

HEADER = os.path.join(hbuild.INCLUDE, "rwkv7_wkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hbuild.LIB),
                                reason="librwkv7_wkv.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rwkv7_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"rwkv7_wkv_forward", "rwkv7_wkv_decode", "rwkv7_wkv_forward_workspace",
            "rwkv7_status_str", "rwkv7_abi_version"} <= set(names)
    L = ctypes.CDLL(hbuild.LIB)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert wkv.abi_version() == 2
    L = wkv.lib()
    for code in range(9):
        assert L.rwkv7_status_str(code)
    assert L.rwkv7_status_str(0) == b"ok"


def _gpu_visible():
    try:
        import torch

        return torch.cuda.device_count() > 0  # counts devices without initialising one
    except Exception:  # pragma: no cover
        return False


# The validation tests pass fake, suitably aligned device addresses that the
# library must reject before any use.  They run only where no GPU is visible:
# after a regression in the validation a call could otherwise enqueue a kernel
# on unmapped memory.
fake_addresses = pytest.mark.skipif(_gpu_visible(),
                                    reason="fake device addresses: run where no GPU is visible")

# fake, suitably aligned device addresses: validation must reject before use
A = 1 << 40
STRIDE = 1 << 32


def fake(i, off=0):
    return ctypes.c_void_p(A + i * STRIDE + off)


def fwd(B=2, T=8, H=3, N=64, dt=1, algo=1, s0=fake(6), y=fake(7), s_out=fake(8), ins=None,
        epi=None, ws=None, ws_bytes=0):
    ins = ins or [fake(i) for i in range(6)]
    return wkv.lib().rwkv7_wkv_forward(*ins, s0, y, s_out, B, T, H, N, dt, algo, epi, ws,
                                       ws_bytes, None)


@fake_addresses
def test_forward_validation_codes():
    assert fwd(N=32) == 4                      # only head size 64
    assert fwd(B=0) == 2 and fwd(H=0) == 2 and fwd(T=-1) == 2
    assert fwd(dt=7) == 3 and fwd(algo=9) == 3
    assert fwd(dt=0, algo=2) == 4              # chunked is bf16 only
    ins = [fake(i) for i in range(6)]
    ins[3] = None
    assert fwd(ins=ins) == 1                   # NULL input
    assert fwd(y=None) == 1
    ins = [fake(i) for i in range(6)]
    ins[2] = fake(2, 8)
    assert fwd(ins=ins) == 5                   # misaligned input
    assert fwd(s_out=fake(8, 4)) == 5
    assert fwd(y=fake(0, 64)) == 6             # y overlaps r
    assert fwd(s_out=fake(6, 16)) == 6         # s_out overlaps s0 without being equal
    assert fwd(s_out=fake(3)) == 6             # s_out overlaps v
    e = wkv.Epilogue(ln_w=None, ln_b=None, r_k=None, eps=64e-5)
    assert fwd(epi=ctypes.byref(e)) == 1       # epilogue needs r_k
    e = wkv.Epilogue(ln_w=A + 9 * STRIDE + 4, ln_b=None, r_k=A + 10 * STRIDE, eps=64e-5)
    assert fwd(epi=ctypes.byref(e)) == 5
    # T == 0 needs no per-token pointers; overflowing sizes are rejected
    assert fwd(B=1 << 30, H=1 << 30) == 2


@fake_addresses
def test_decode_validation_codes():
    L = wkv.lib()

    def dec(B=2, H=3, N=64, dt=1, state=fake(6), y=fake(7), ins=None, epi=None):
        ins = ins or [fake(i) for i in range(6)]
        return L.rwkv7_wkv_decode(*ins, state, y, B, H, N, dt, epi, None)

    assert dec(N=96) == 4
    assert dec(B=0) == 2
    assert dec(dt=5) == 3
    assert dec(state=None) == 1 and dec(y=None) == 1
    assert dec(state=fake(6, 8)) == 5
    assert dec(y=fake(6, 64)) == 6             # y inside the state
    assert dec(state=fake(1)) == 6             # state overlaps w
    # one 256-thread workgroup per head (1024 at N = 128): a grid of more than
    # 2^32 - 1 threads is a shape error, the largest one that fits is not
    assert dec(B=(1 << 24) + 1, H=1) == 2
    assert dec(B=(1 << 24) - 1, H=1) != 2
    assert dec(B=1 << 22, H=1, N=128) == 2
    assert dec(B=(1 << 22) - 1, H=1, N=128) != 2


def test_workspace_query_is_pure():
    L = wkv.lib()
    assert L.rwkv7_wkv_forward_workspace(1, 64, 1, 64, 0, 1) == 0   # scan needs none
    assert L.rwkv7_wkv_forward_workspace(1, 64, 1, 32, 1, 2) == 0   # unsupported -> 0


def test_workspace_query_segments():
    """Long sequences of few heads are split into segments (up to two
    workgroups per compute unit, at least 128 tokens each); each segment keeps
    three float32 N x N states in the workspace.  Many heads, short sequences
    or the scan need none."""
    L = wkv.lib()
    per_seg = 3 * 64 * 64 * 4
    big = L.rwkv7_wkv_forward_workspace(1, 65536, 1, 64, 1, 2)
    assert big > 0 and big % per_seg == 0 and 2 <= big // per_seg <= 64
    assert L.rwkv7_wkv_forward_workspace(1, 65536, 1, 64, 1, 0) == big  # auto = chunked
    assert L.rwkv7_wkv_forward_workspace(1, 511, 1, 64, 1, 2) == 0
    assert L.rwkv7_wkv_forward_workspace(64, 65536, 64, 64, 1, 2) == 0
    assert L.rwkv7_wkv_forward_workspace(1, 65536, 1, 64, 1, 1) == 0
    assert L.rwkv7_wkv_forward_workspace(1, 4096, 1, 64, 1, 2) == 32 * per_seg  # 128 tokens each
    assert L.rwkv7_wkv_forward_workspace(1, 512, 1, 64, 1, 2) == 4 * per_seg
    assert L.rwkv7_wkv_forward_workspace(200, 4096, 1, 64, 1, 2) == 0   # B*H > CUs / 2


def fwd_train(B=2, T=8, H=3, N=64, dt=1, algo=1, s0=fake(6), y=fake(7), s_out=fake(8),
              ck=fake(9), ins=None):
    ins = ins or [fake(i) for i in range(6)]
    return wkv.lib().rwkv7_wkv_forward_train(*ins, s0, y, s_out, ck, B, T, H, N, dt, algo, None,
                                             0, None)


@fake_addresses
def test_forward_train_validation_codes():
    assert fwd_train(N=32) == 4
    assert fwd_train(B=0) == 2 and fwd_train(T=-1) == 2
    assert fwd_train(ck=None) == 1                   # stored states required
    assert fwd_train(ck=fake(9, 8)) == 5             # misaligned
    assert fwd_train(ck=fake(6)) == 6                # on top of s0
    assert fwd_train(ck=fake(0, 64)) == 6            # inside r
    assert fwd_train(y=fake(9, 4096)) == 6           # y inside the stored states
    assert fwd_train(dt=0, algo=2) == 4              # chunked needs bf16
    # T == 0 stores nothing: no stored-state buffer needed (s_out NULL: nothing to do)
    assert fwd_train(T=0, ck=None, s_out=None) == 0


def bwd(B=2, T=8, H=3, N=64, dt=1, ins=None, dy=fake(6), ck=fake(7), dsT=fake(8), outs=None,
        ds0=fake(15), algo=1, ws=None, ws_bytes=0):
    ins = ins or [fake(i) for i in range(6)]
    outs = outs or [fake(9 + i) for i in range(6)]
    return wkv.lib().rwkv7_wkv_backward(*ins, dy, ck, dsT, *outs, ds0, B, T, H, N, dt, algo,
                                        ws, ws_bytes, None)


@fake_addresses
def test_backward_validation_codes():
    assert bwd(N=96) == 4
    assert bwd(N=128, algo=2) == 4                 # the chunked backward is built for 64
    assert bwd(N=128) == 7                         # token by token at 128: a workspace
    assert bwd(B=0) == 2 and bwd(H=0) == 2 and bwd(T=-1) == 2
    assert bwd(dt=7) == 3
    assert bwd(dy=None) == 1 and bwd(ck=None) == 1
    assert bwd(outs=[fake(9 + i) for i in range(5)] + [None]) == 1
    assert bwd(ins=[fake(i) for i in range(5)] + [None]) == 1
    assert bwd(dy=fake(6, 2)) == 5
    assert bwd(ds0=fake(15, 4)) == 5
    assert bwd(outs=[fake(9)] * 6) == 6                            # outputs overlap
    assert bwd(outs=[fake(9 + i) for i in range(5)] + [fake(0)]) == 6   # da on top of r
    assert bwd(ds0=fake(7, 64)) == 6                              # ds0 inside the states
    assert bwd(ds0=fake(8, 16)) == 6                              # ds0 partly over ds_T
    # ds0 == ds_T is the in-place case: passes validation (T == 0 then has nothing to do)
    assert bwd(T=0, ds0=fake(8), dsT=fake(8), ck=None, dy=None) == 0
    assert bwd(T=0, ds0=None, ck=None) == 0


@fake_addresses
def test_fp32_decay_dtype_codes():
    # RWKV7_DT_BF16_W32 = 2: accepted by forward (scan and chunked) and decode
    # validation, and by both backward algorithms (dw float32 too); w spans 4 bytes
    # per element
    assert fwd(dt=2, algo=1, T=0, s_out=None) == 0
    assert fwd(dt=2, algo=2, T=0, s_out=None) == 0
    assert fwd(dt=3) == 3
    B, T, H = 2, 8, 3
    half_w = B * T * H * 64 * 2
    assert fwd(dt=2, y=fake(1, half_w)) == 6     # y over the float32 w's second half
    outs = [fake(9 + i) for i in range(6)]
    outs[2] = fake(10, half_w)                    # dk over the float32 dw's second half
    assert bwd(dt=2, algo=1, outs=outs) == 6      # token by token: w and dw float32 too
    L = wkv.lib()
    need = L.rwkv7_wkv_backward_workspace(B, T, H, 64, 2, 0)
    assert need == L.rwkv7_wkv_backward_workspace(B, T, H, 64, 1, 2) > 0
    assert L.rwkv7_wkv_backward_workspace(B, T, H, 64, 2, 1) == 0
    assert bwd(dt=2, algo=0) == 7                 # auto -> chunked, which needs a workspace
    assert bwd(dt=2, algo=2, T=0, ds0=None, ck=None) == 0
    outs = [fake(9 + i) for i in range(6)]
    outs[2] = fake(10, half_w)                    # dk over the float32 dw's second half
    assert bwd(dt=2, algo=2, outs=outs, ws=fake(20), ws_bytes=need) == 6
    assert L.rwkv7_wkv_forward_workspace(1, 65536, 1, 64, 2, 0) == \
        L.rwkv7_wkv_forward_workspace(1, 65536, 1, 64, 1, 0)


def test_bidir_workspace_query():
    L = wkv.lib()
    assert L.rwkv7_wkv_forward_bidir_workspace(2, 0, 3, 64, 1, 0) == 0
    assert L.rwkv7_wkv_forward_bidir_workspace(2, 10, 3, 64, 1, 0) == 2 * 10 * 3 * 64 * 4
    assert L.rwkv7_wkv_forward_bidir_workspace(2, 10, 3, 32, 1, 0) == 0
    big = L.rwkv7_wkv_forward_bidir_workspace(1, 65536, 1, 64, 1, 2)
    assert big == 65536 * 64 * 4 + L.rwkv7_wkv_forward_workspace(1, 65536, 1, 64, 1, 2)
    assert L.rwkv7_wkv_forward_bidir_workspace(1, 65536, 1, 64, 0, 1) == 65536 * 64 * 4


@fake_addresses
def test_bidir_validation_codes():
    L = wkv.lib()

    def bid(B=2, T=8, H=3, s0=fake(6), s_out=fake(7), ws=fake(8), ws_bytes=1 << 20, dt=1):
        return L.rwkv7_wkv_forward_bidir(*[fake(i) for i in range(6)], s0, fake(9), s_out, B, T,
                                         H, 64, dt, 1, None, ws, ws_bytes, None)
    assert bid(ws=None) == 7                       # workspace required
    assert bid(ws_bytes=100) == 7
    st = 2 * 3 * 64 * 64 * 4
    assert bid(s_out=fake(6, st)) == 6             # s_out over s0's second state
    assert bid(T=0, s_out=None) == 0


_Pro = wkv.Prologue


@fake_addresses
def test_fused_validation_codes():
    L = wkv.lib()

    def fu(pro=None, dt=1, T=8, y=fake(9), s_out=fake(10)):
        p = None if pro is None else ctypes.byref(pro)
        return L.rwkv7_wkv_forward_fused(*[fake(i) for i in range(5)], p, fake(6), y, s_out, 2,
                                         T, 3, 64, dt, 1, None, None, 0, None)
    ok = _Pro(k_k=A + 11 * STRIDE, k_a=A + 12 * STRIDE, g=A + 13 * STRIDE)
    assert fu(None) == 1
    assert fu(_Pro(k_k=None, k_a=A + 12 * STRIDE, g=None)) == 1
    assert fu(_Pro(k_k=A + 11 * STRIDE + 4, k_a=A + 12 * STRIDE, g=None)) == 5
    assert fu(ok, dt=2) == 4                           # no fused prologue with float32 w
    assert fu(ok, y=fake(13, 128)) == 6                # y over the gate
    assert fu(ok, s_out=fake(13)) == 6                 # s_out over the gate
    assert fu(ok, T=0, s_out=None) == 0                # no kappa argument needed


@fake_addresses
def test_decode_head_size_128_validation():
    L = wkv.lib()
    ins = [fake(i) for i in range(6)]

    def dec(N, state=fake(6), y=fake(7)):
        return L.rwkv7_wkv_decode(*ins, state, y, 2, 3, N, 1, None, None)
    assert dec(96) == 4 and dec(256) == 4
    # N = 128: the state spans 2*3*128*128*4 bytes, so y just inside its end overlaps
    assert dec(128, y=fake(6, 2 * 3 * 128 * 128 * 4 - 16)) == 6
    assert L.rwkv7_wkv_forward_workspace(1, 64, 1, 128, 1, 0) == 0


@fake_addresses
def test_forward_head_size_128_validation():
    assert fwd(N=96) == 4
    assert fwd(N=128, algo=2, dt=0) == 4           # chunked is bf16 only, at 128 too
    L = wkv.lib()
    # the chunked kernel at 128 runs the plain forward only
    assert L.rwkv7_wkv_forward_bidir(*[fake(i) for i in range(6)], None, fake(7), None, 2, 8,
                                     3, 128, 1, 2, None, fake(8), 1 << 24, None) == 4
    pro = _Pro(k_k=A + 11 * STRIDE, k_a=A + 12 * STRIDE, g=None)
    assert L.rwkv7_wkv_forward_fused(*[fake(i) for i in range(5)], ctypes.byref(pro), None,
                                     fake(7), None, 2, 8, 3, 128, 1, 2, None, None, 0,
                                     None) == 4
    # the training forward at 128 (scan and chunked): the stored states span
    # 2*3*128*128*4 bytes (one interval at T = 8), so y just inside their end overlaps
    ck_bytes = 2 * 3 * 128 * 128 * 4
    assert fwd_train(N=128, y=fake(9, ck_bytes - 16)) == 6
    assert fwd_train(N=128, algo=2, y=fake(9, ck_bytes - 16)) == 6
    assert fwd_train(N=128, algo=2, ck=fake(9, 8)) == 5
    assert fwd(N=128, T=0, s_out=None) == 0        # scan at 128 passes validation


@fake_addresses
def test_decode_fused_validation_codes():
    L = wkv.lib()

    def dfu(pro=None, dt=1, N=64, y=fake(7), state=fake(6)):
        p = None if pro is None else ctypes.byref(pro)
        return L.rwkv7_wkv_decode_fused(*[fake(i) for i in range(5)], p, state, y, 2, 3, N, dt,
                                        None, None)
    ok = _Pro(k_k=A + 11 * STRIDE, k_a=A + 12 * STRIDE, g=A + 13 * STRIDE)
    assert dfu(None) == 1
    assert dfu(_Pro(k_k=A + 11 * STRIDE, k_a=None, g=None)) == 1
    assert dfu(_Pro(k_k=A + 11 * STRIDE, k_a=A + 12 * STRIDE + 8, g=None)) == 5
    assert dfu(ok, dt=2) == 4
    assert dfu(ok, N=96) == 4
    assert dfu(ok, y=fake(13, 64)) == 6            # y over the gate
    assert dfu(ok, state=fake(11)) == 6            # state over k_k


@fake_addresses
def test_stream_copy_validation_codes():
    L = wkv.lib()
    src, dst = A, A + STRIDE
    assert L.rwkv7_stream_copy(src, dst, 0, None) == 0          # nothing to do, no launch
    assert L.rwkv7_stream_copy(None, dst, 64, None) == 1
    assert L.rwkv7_stream_copy(src, None, 64, None) == 1
    assert L.rwkv7_stream_copy(src + 8, dst, 64, None) == 5
    assert L.rwkv7_stream_copy(src, dst + 4, 64, None) == 5
    assert L.rwkv7_stream_copy(src, dst, 72, None) == 2          # not a multiple of 16
    assert L.rwkv7_stream_copy(src, src + 32, 64, None) == 6     # overlapping ranges
    assert L.rwkv7_stream_copy(src + 32, src, 64, None) == 6


@fake_addresses
def test_backward_chunked_workspace_codes():
    L = wkv.lib()
    B, T, H = 2, 40, 3
    need = L.rwkv7_wkv_backward_workspace(B, T, H, 64, 1, 2)
    assert need == B * H * 1 * 64 * 64 * 2   # 8 KiB per head and group of 8 chunks (3 chunks)
    assert L.rwkv7_wkv_backward_workspace(B, T, H, 64, 1, 0) == need    # auto -> chunked
    assert L.rwkv7_wkv_backward_workspace(B, T, H, 64, 0, 0) == 0       # f32 -> scan
    assert L.rwkv7_wkv_backward_workspace(B, T, H, 64, 1, 1) == 0
    assert L.rwkv7_wkv_backward_workspace(B, 0, H, 64, 1, 2) == 0
    assert L.rwkv7_wkv_backward_workspace(B, T, H, 128, 1, 2) == 0   # chunked: 64 only
    ws = fake(20)
    assert bwd(T=T, algo=2) == 7                              # no workspace
    assert bwd(T=T, algo=2, ws=ws, ws_bytes=need - 16) == 7   # too small
    assert bwd(T=T, algo=2, ws=fake(20, 8), ws_bytes=need) == 5
    assert bwd(T=T, algo=2, ws=fake(7), ws_bytes=need) == 6   # over the stored states
    assert bwd(T=T, algo=2, ws=fake(12), ws_bytes=need) == 6  # over dk
    assert bwd(T=T, algo=2, dt=0) == 4                        # chunked is bf16 only
    assert bwd(T=T, algo=9) == 3
    assert bwd(T=0, algo=2, ds0=None, ck=None) == 0           # nothing to do
    # gradient grid of B*H x ceil(chunks / 8) workgroups past 2^31: refused up front
    Bb, Hb, Tb = 1 << 15, 1 << 10, 1 << 13
    needb = L.rwkv7_wkv_backward_workspace(Bb, Tb, Hb, 64, 1, 2)
    assert bwd(B=Bb, H=Hb, T=Tb, algo=2, ws=ws, ws_bytes=needb) == 2


def test_binding_workspace_dtype_names():
    # the binding's workspace queries name dtypes as strings; each maps to its own code
    assert wkv.backward_workspace_bytes(2, 40, 3, dtype="bf16_w32") == \
        wkv.backward_workspace_bytes(2, 40, 3, dtype="bf16") == 2 * 3 * 1 * 64 * 64 * 2
    # one 8 KiB slot per (b, h) and group of 8 chunks: 129 chunks make 17 groups
    assert wkv.backward_workspace_bytes(1, 129 * 16, 1, dtype="bf16") == 17 * 64 * 64 * 2
    assert wkv.backward_workspace_bytes(2, 40, 3, dtype="f32") == 0          # auto -> scan
    assert wkv.forward_workspace_bytes(1, 65536, 1, dtype="bf16_w32") == \
        wkv.forward_workspace_bytes(1, 65536, 1, dtype="bfloat16") > 0
    assert wkv.forward_bidir_workspace_bytes(1, 65536, 1, dtype="float32") == \
        wkv.lib().rwkv7_wkv_forward_bidir_workspace(1, 65536, 1, 64, 0, 0)
    with pytest.raises(ValueError):
        wkv.backward_workspace_bytes(2, 40, 3, dtype="fp16")


@fake_addresses
def test_backward_head_size_128_workspace_codes():
    """Token by token at head size 128: four workgroups of 32 value rows per head
    leave float32 partial column sums (5 sums x 4 parts per element) in the
    workspace; sequences are cut into slices of whole 16-token intervals so that
    one slice's sums stay within 256 MiB, and the cotangent of the state is
    carried between slices (B*H*128*128*4 bytes, only when there are several)."""
    L = wkv.lib()
    per_tok = lambda B, H: 5 * 4 * B * H * 128 * 4
    # one slice: T rounded up to whole intervals
    assert L.rwkv7_wkv_backward_workspace(2, 40, 3, 128, 1, 1) == per_tok(2, 3) * 48
    assert L.rwkv7_wkv_backward_workspace(2, 40, 3, 128, 1, 0) == per_tok(2, 3) * 48  # auto
    assert L.rwkv7_wkv_backward_workspace(2, 40, 3, 128, 0, 0) == per_tok(2, 3) * 48  # f32
    assert L.rwkv7_wkv_backward_workspace(2, 40, 3, 128, 2, 0) == per_tok(2, 3) * 48  # w32
    assert L.rwkv7_wkv_backward_workspace(2, 0, 3, 128, 1, 1) == 0
    # several slices: 96 tokens each at B4 H64, plus the carried cotangent
    slice_len = (256 << 20) // per_tok(4, 64) // 16 * 16
    assert slice_len == 96
    assert L.rwkv7_wkv_backward_workspace(4, 1000, 64, 128, 1, 1) == \
        per_tok(4, 64) * 96 + 4 * 64 * 128 * 128 * 4
    # at least one interval per slice, however many heads
    assert L.rwkv7_wkv_backward_workspace(4096, 100, 64, 128, 1, 1) == \
        per_tok(4096, 64) * 16 + 4096 * 64 * 128 * 128 * 4
    need = L.rwkv7_wkv_backward_workspace(2, 40, 3, 128, 1, 1)
    assert bwd(T=40, N=128, ws=fake(20), ws_bytes=need - 16) == 7
    assert bwd(T=40, N=128, ws=fake(20, 8), ws_bytes=need) == 5
    assert bwd(T=40, N=128, ws=fake(12), ws_bytes=need) == 6   # over dk
    assert bwd(T=40, N=128, ws=fake(7), ws_bytes=need) == 6    # over the stored states
    assert bwd(T=0, N=128, ds0=None, ck=None) == 0             # nothing to do


@fake_addresses
def test_launch_grid_limits():
    """Every grid's extent in threads fits in 32 bits: one workgroup per head of
    4N threads (scan), 512 (chunked at 64) or 1024 (chunked at 128); the
    token-by-token backward: 256 per head at 64, four of 256 at 128.  Calls just
    under a limit fail later in validation instead (overlapping fake buffers, a
    missing workspace).  Head channels are indexed in 32 bits: H * N < 2^31."""
    assert fwd(B=1 << 24, H=1, algo=1) == 2
    assert fwd(B=(1 << 24) - 1, H=1, algo=1) != 2
    assert fwd(B=1 << 23, H=1, algo=2) == 2
    assert fwd(B=(1 << 23) - 1, H=1, algo=2) != 2
    assert fwd(B=1 << 23, H=1, N=128, algo=1) == 2
    assert fwd(B=(1 << 23) - 1, H=1, N=128, algo=1) != 2
    assert fwd(B=1 << 22, H=1, N=128, algo=2) == 2
    assert fwd(B=(1 << 22) - 1, H=1, N=128, algo=2) != 2
    assert bwd(B=1 << 24, H=1, algo=1) == 2
    assert bwd(B=(1 << 24) - 1, H=1, algo=1) != 2
    assert bwd(B=1 << 22, H=1, N=128) == 2
    assert bwd(B=(1 << 22) - 1, H=1, N=128) != 2
    # T == 0 launches no recurrence kernel: only H * N < 2^31 applies then
    assert fwd(B=1 << 24, H=1, T=0, s_out=None) == 0
    assert fwd(B=1, H=1 << 25, T=0, s_out=None) == 2
    assert fwd(B=1, H=(1 << 25) - 1, T=0, s_out=None) == 0
    assert fwd(B=1, H=1 << 24, N=128, T=0, s_out=None) == 2
    assert bwd(B=1 << 24, H=1, T=0, ds0=None, ck=None) == 0
    assert bwd(B=1, H=1 << 25, T=0, ds0=None, ck=None) == 2
