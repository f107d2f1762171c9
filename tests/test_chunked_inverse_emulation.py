"""The unit lower-triangular inverse X = (I + N)^-1 of the chunked kernels,
emulated on the CPU step by step: bf16 rounding (nearest even) wherever the
kernels convert an MFMA operand, float32 everywhere else.  No GPU; this checks
the numerical method the kernels follow, not the kernels themselves.

Within a chunk of 16 tokens, N[t, s] = Kp_t . Bm_s (s < t) couples the removal
probes of the chunk's tokens (the chunked form of the diagonal-plus-rank-one
transition, RWKV-7 "Goose" summary, §4 Method).  When removal keys repeat or
correlate -- the delta-rule regime of the summary's §2 Background and App. D.3,
where a key overwrites what the state holds for it -- N approaches the
all-ones strict lower triangle, whose inverse is I minus the first
sub-diagonal.

* The product form (I - N)(I + N^2)(I + N^4)(I + N^8), with every power rounded
  to bf16, forms intermediate entries up to C(14, 7) = 3432 that must cancel to
  entries of size 1; bf16 cannot hold them, and the result is off by 4.0 on one
  repeated key.  The kernels used it before; it is kept here to show that this
  test detects the failure.
* The blocked form the kernels use now: the four 4 x 4 diagonal blocks by
  forward substitution in float32, then two levels of block substitution,
  X <- X - X (N_l X), where N_l holds the entries of N below the diagonal
  blocks of the current size (4, then 8).  Every intermediate is a block of
  the true inverse or the product of such a block with a block of N, so
  nothing grows; the products run on the float32 matrix-core instruction
  (float32 operands and accumulation), so X keeps float32 accuracy.
"""
import numpy as np
import pytest

import oracle
import synth

C = 16
F32 = np.float32


def bf(x):
    """float32 -> nearest-even bf16, returned as float32."""
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, F32)))


def mm(a, b):
    """Matrix-core product: float32 accumulation (bf16-valued or float32 operands)."""
    return np.matmul(np.asarray(a, F32), np.asarray(b, F32)).astype(F32)


def inverse_product_form(n):
    """(I - N)(I + N^2)(I + N^4)(I + N^8), each power rounded to bf16 (the former form)."""
    eye = np.eye(C, dtype=F32)
    n2 = mm(bf(n), bf(n))
    n4 = mm(bf(n2), bf(n2))
    n8 = mm(bf(n4), bf(n4))
    f1 = (mm(bf(eye - n), bf(n2)) + (eye - n)).astype(F32)
    g = (mm(bf(f1), bf(n4)) + f1).astype(F32)
    return (mm(bf(g), bf(n8)) + g).astype(F32)


def level_mask(size):
    """Entries (t, s) in one diagonal block of 2*size, t in its lower half, s in its upper."""
    t, s = np.meshgrid(np.arange(C), np.arange(C), indexing="ij")
    return (t // (2 * size) == s // (2 * size)) & ((t // size) % 2 == 1) & ((s // size) % 2 == 0)


def inverse_blocked(n):
    """The kernels' blocked inverse of I + N (N strictly lower, float32)."""
    n = np.asarray(n, F32)
    x = np.zeros(n.shape, F32)
    for b in range(0, C, 4):  # 4 x 4 diagonal blocks, forward substitution in float32
        for c in range(b, b + 4):
            for t in range(b, b + 4):
                acc = F32(1.0) if t == c else F32(0.0)
                for s in range(b, t):
                    acc = F32(acc - n[..., t, s] * x[..., s, c])
                x[..., t, c] = acc
    for size in (4, 8):  # block substitution, float32 products
        nl = np.where(level_mask(size), n, F32(0.0)).astype(F32)
        t_ = mm(nl, x)
        x = (x - mm(x, t_)).astype(F32)
    return x


def chunk_n(kappa, a, w):
    """N of one chunk from its removal keys, rates and decays ([.., C, 64] float32),
    as the kernels form it: Kp = kappa G_{t-1}, Bm = a kappa / G_t rounded to bf16,
    N = stril(Kp Bm^T) accumulated in float32."""
    g = np.cumprod(w, axis=-2, dtype=F32)
    gp = np.concatenate([np.ones_like(g[..., :1, :]), g[..., :-1, :]], axis=-2)
    kp = bf(kappa * gp)
    bm = bf((a * kappa).astype(F32) * (F32(1.0) / g))
    return np.where(np.tril(np.ones((C, C), bool), -1), mm(kp, np.swapaxes(bm, -1, -2)), F32(0.0))


def rel_to_exact(x, n):
    ref = np.linalg.inv(np.eye(C) + np.asarray(n, np.float64))
    return np.abs(x - ref).max() / np.abs(ref).max()


def test_repeated_key():
    """One repeated unit key, a = 1, w = 1: N is the strict lower triangle of ones
    and the inverse is I minus the first sub-diagonal."""
    n = np.tril(np.ones((C, C), F32), -1)
    exact = np.eye(C) - np.eye(C, k=-1)
    assert np.abs(inverse_product_form(n) - exact).max() >= 1.0   # the former form fails
    assert np.array_equal(inverse_blocked(n), exact.astype(F32))   # exact here


@pytest.mark.parametrize("cos", [0.0, 0.5, 0.9, 0.99, 1.0])
@pytest.mark.parametrize("a_rate,w", [("s2", 0.995), ("s2", 1.0), ("one", 1.0), ("s0", 0.995)])
def test_correlated_keys(cos, a_rate, w):
    """Chunks of removal keys with mean pairwise cosine `cos` (synth's correlated
    recipe); a = sigmoid(N(2, 1)), sigmoid(N(0, 1)) or 1; constant w."""
    kw = dict(a_const=1.0) if a_rate == "one" else dict(a_mean=2.0 if a_rate == "s2" else 0.0)
    d = synth.draw(4, C, 8, seed=41, dtype="f32", w_const=w,
                   kappa_cos=cos if cos > 0 else None, **kw)
    to_chunks = lambda x: np.ascontiguousarray(np.swapaxes(d.as_f32(x), 1, 2))  # [B,H,C,N]
    n = chunk_n(bf(to_chunks("kappa")), bf(to_chunks("a")), bf(to_chunks("w")))
    assert rel_to_exact(inverse_blocked(n), n) < 1e-5
    if cos >= 0.9 and a_rate != "s0":
        assert rel_to_exact(inverse_product_form(n), n) > 2e-2   # where the former form broke


def chunked_forward(r, w, k, v, kap, a, inverse):
    """One head ([T, 64] bf16-valued float32 inputs, zero initial state) through the
    chunked form with the kernels' rounding points: Kp, Rp, Km, Bm, the C x C
    matrices (float32 diagonals of M_kr, M_br), -X, the state S^T and
    rhs = M_kk V + Kp S0^T, and -U rounded to bf16; products accumulate in
    float32; the state is carried in float32."""
    T, N = r.shape
    z = np.zeros((N, N), F32)  # S^T
    y = np.zeros((T, N), F32)
    low, slow = np.tril(np.ones((C, C), bool)), np.tril(np.ones((C, C), bool), -1)
    for c0 in range(0, T, C):
        sl = slice(c0, c0 + C)
        g = np.cumprod(w[sl], axis=0, dtype=F32)
        gp = np.vstack([np.ones((1, N), F32), g[:-1]])
        ig = (F32(1.0) / g).astype(F32)
        b = (a[sl] * kap[sl]).astype(F32)
        kp, rp, km, bm = bf(kap[sl] * gp), bf(r[sl] * g), bf(k[sl] * ig), bf(b * ig)
        mkk = bf(np.where(slow, mm(kp, km.T), 0))
        mkr, mbr = mm(rp, km.T), mm(rp, bm.T)
        i = np.arange(C)
        mkr[i, i] = np.sum(r[sl] * k[sl], axis=1, dtype=F32)
        mbr[i, i] = np.sum(r[sl] * b, axis=1, dtype=F32)
        mkr, mbr = bf(np.where(low, mkr, 0)), bf(np.where(low, mbr, 0))
        n = np.where(slow, mm(kp, bm.T), F32(0.0))
        xneg = bf(-inverse(n))
        zb = bf(z)
        u = bf(mm(xneg, bf(mm(mkk, v[sl]) + mm(kp, zb))))  # -U
        y[sl] = mm(rp, zb) + mm(mkr, v[sl]) + mm(mbr, u)
        z = ((z + mm(km.T, v[sl]) + mm(bm.T, u)) * g[-1][:, None]).astype(F32)
    return y, z.T


@pytest.mark.parametrize("cos,k_align", [(0.9, False), (0.99, False), (1.0, False), (0.8, True)])
def test_chunked_form_against_oracle(cos, k_align):
    """The whole chunked form, emulated with the kernels' rounding points, against
    the float64 oracle on correlated keys with a = 1, w = 1: within the bf16
    bound with the blocked inverse; far outside it with the product form."""
    d = synth.draw(1, 128, 3, seed=43, dtype="bf16", a_const=1.0, w_const=1.0,
                   kappa_cos=cos, k_align=k_align)
    ins = {x: d.as_f32(x) for x in ("r", "w", "k", "v", "kappa", "a")}
    y_ref, s_ref = oracle.forward(*(d.as_f64(x) for x in ("r", "w", "k", "v", "kappa", "a")))
    for inverse, ok in ((inverse_blocked, True), (inverse_product_form, False)):
        ys, ss = [], []
        for h in range(3):
            y, s = chunked_forward(*(ins[x][0, :, h] for x in ("r", "w", "k", "v", "kappa", "a")),
                                   inverse)
            ys.append(bf(y))
            ss.append(s)
        y = np.stack(ys, axis=1)[None]
        s = np.stack(ss)[None]
        err = max(np.abs(y - y_ref).max() / np.abs(y_ref).max(),
                  np.abs(s - s_ref).max() / np.abs(s_ref).max())
        assert (err <= 1e-2) if ok else (err > 2e-2), (inverse.__name__, err)
