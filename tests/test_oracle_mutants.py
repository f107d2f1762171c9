"""The pins are strong enough: each plausible mistake planted in a copy of the C
oracle (a dropped term, a wrong sign, a wrong or transposed index, a misplaced
eps, ...) makes at least one pin of test_oracle.py fail.

Everything here runs on the CPU: the mutants are compiled with gcc into a
temporary directory and swapped in for the oracle library while the pins run.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle as pins

SRC = open(obuild.SRC).read()

MUTANTS = {
    "removal sign": ("- u[i] * (kap[o + j] * a[o + j])", "+ u[i] * (kap[o + j] * a[o + j])"),
    "decay on value index": ("S[i * N + j] * w[o + j]", "S[i * N + j] * w[o + i]"),
    "rate on value index": ("(kap[o + j] * a[o + j])", "(kap[o + j] * a[o + i])"),
    "write transposed": ("+ v[o + i] * k[o + j]", "+ v[o + j] * k[o + i]"),
    "removal probe transposed": ("S[i * N + j] * kap[o + j]", "S[j * N + i] * kap[o + j]"),
    "readout transposed": ("S[i * N + j] * r[o + j]", "S[j * N + i] * r[o + j]"),
    "decay dropped": ("S[i * N + j] * w[o + j] -", "S[i * N + j] -"),
    "write dropped": ("+ v[o + i] * k[o + j];", ";"),
    "rate dropped": ("(kap[o + j] * a[o + j])", "(kap[o + j])"),
    "sample variance": ("var /= (REAL)N;", "var /= (REAL)(N - 1);"),
    "eps outside sqrt": ("SQRT(var + (REAL)J->eps)", "(SQRT(var) + (REAL)J->eps)"),
    "bonus without r_k": ("r[o + j] * k[o + j] * r_k[h * N + j]", "r[o + j] * k[o + j]"),
    "bonus normalised": ("+ c + bonus * v[o + i]", "+ c + bonus * v[o + i] * inv"),
    "affine swapped": ("* inv * g + c", "* inv * c + g"),
    "initial state ignored": ("if (s0) memcpy", "if (0) memcpy"),
    "time reversed": ("((b * T + t) * H + h) * N", "((b * T + (T - 1 - t)) * H + h) * N"),
    "state not stored": ("if (s_out) memcpy", "if (0) memcpy"),
}

PIN_CALLS = [
    ("hand example", lambda: pins.test_hand_worked_example_exact()),
    ("single step", lambda: pins.test_single_step_closed_form()),
    ("linear attention", lambda: pins.test_linear_attention_special_case()),
    ("diagonal decay", lambda: pins.test_diagonal_decay_closed_form()),
    ("delta rule", lambda: pins.test_delta_rule_replacement()),
    ("transitions", lambda: pins.test_elementary_transitions_bitwise("f64")),
    ("householder", lambda: pins.test_half_householder()),
    ("state passing", lambda: pins.test_state_passing_bitwise()),
    ("linearity", lambda: pins.test_linearity_and_independence()),
    ("brute force", lambda: pins.test_bruteforce_exact_rationals(3, 5, 1)),
    ("group norm", lambda: pins.test_epilogue_against_torch_group_norm()),
    ("norm invariants", lambda: pins.test_group_norm_invariants()),
]


def _compile(src: str, path: str):
    cpath = path + ".c"
    with open(cpath, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-pthread", cpath, "-o", path, "-lm"], check=True)


def _as_oracle_lib(path):
    lib = ctypes.CDLL(path)
    for name, ct in (("wkv7_oracle_forward_f64", ctypes.c_double),
                     ("wkv7_oracle_forward_f32", ctypes.c_float)):
        fn = getattr(lib, name)
        p = ctypes.POINTER(ct)
        fn.argtypes = [p] * 9 + [ctypes.c_long] * 4 + [p, p, p, ctypes.c_double, ctypes.c_int,
                                                      ctypes.c_int]
        fn.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    assert old in SRC, f"mutation site for {name!r} not found"
    path = str(tmp_path / "libmutant.so")
    _compile(SRC.replace(old, new), path)
    oracle._load()
    monkeypatch.setattr(oracle, "_lib", _as_oracle_lib(path))
    caught = []
    for pin, call in PIN_CALLS:
        try:
            call()
        except AssertionError:
            caught.append(pin)
    assert caught, f"no pin caught the planted mistake {name!r}"


def test_unmodified_source_passes_every_pin(tmp_path, monkeypatch):
    path = str(tmp_path / "libclean.so")
    _compile(SRC, path)
    oracle._load()
    monkeypatch.setattr(oracle, "_lib", _as_oracle_lib(path))
    for pin, call in PIN_CALLS:
        call()


# ---------------------------------------------------------------------------
# Planted mistakes in the Python oracle's fused prologue / gate composition
# (oracle.prologue and oracle.forward_fused).  Each mutant is a copy of the
# function's source with one mistake, executed in the oracle's namespace; the
# hand-worked fused example must fail for every one of them.
# ---------------------------------------------------------------------------
import inspect  # noqa: E402

_FUSED_SRC = inspect.getsource(oracle.forward_fused)
_PRO_SRC = inspect.getsource(oracle.prologue)
_GATE_LATE = ("    y, sT = forward(r, w, k_t, v, kappa, a, s0=s0, epilogue=epilogue, threads=threads)\n"
              "    if g is not None:\n"
              "        y = y * np.asarray(g, np.float64)\n")

FUSED_MUTANTS = {
    # the gate multiplies the readouts before the GroupNorm
    "gate before norm": ("forward_fused", _FUSED_SRC, _GATE_LATE,
                         "    y, sT = forward(r, w, k_t, v, kappa, a, s0=s0, threads=threads)\n"
                         "    if g is not None:\n"
                         "        y = y * np.asarray(g, np.float64)\n"
                         "    if epilogue is not None:\n"
                         "        H, N = y.shape[-2:]\n"
                         "        y = group_norm_heads(y, epilogue.get('ln_w'), epilogue.get('ln_b'),\n"
                         "                             epilogue.get('eps', 64e-5))\n"
                         "        y = y + bonus(r, k_t, np.asarray(epilogue['r_k']).reshape(H, N), v)\n"),
    # the gate multiplies after the norm but before the bonus is added
    "gate before bonus": ("forward_fused", _FUSED_SRC, _GATE_LATE,
                          "    y, sT = forward(r, w, k_t, v, kappa, a, s0=s0, threads=threads)\n"
                          "    if epilogue is not None:\n"
                          "        H, N = y.shape[-2:]\n"
                          "        y = group_norm_heads(y, epilogue.get('ln_w'), epilogue.get('ln_b'),\n"
                          "                             epilogue.get('eps', 64e-5))\n"
                          "    if g is not None:\n"
                          "        y = y * np.asarray(g, np.float64)\n"
                          "    if epilogue is not None:\n"
                          "        y = y + bonus(r, k_t, np.asarray(epilogue['r_k']).reshape(H, N), v)\n"),
    # the raw key is written (and used by the bonus) instead of the boosted one
    "raw key written": ("forward_fused", _FUSED_SRC, "forward(r, w, k_t, v,", "forward(r, w, k, v,"),
    # the removal key is formed from the boosted key
    "kappa after booster": ("prologue", _PRO_SRC, "kk = k * np.asarray(k_k",
                            "kk = (k + k * (a - 1.0) * np.asarray(k_a, np.float64).reshape(H, N))"
                            " * np.asarray(k_k"),
    # the removal key is not normalised
    "kappa not normalised": ("prologue", _PRO_SRC, "kappa = kk / np.maximum(nrm, 1e-12)",
                             "kappa = kk"),
}


@pytest.mark.parametrize("name", sorted(FUSED_MUTANTS))
def test_planted_fused_mistake_is_caught(name, monkeypatch):
    fname, src, old, new = FUSED_MUTANTS[name]
    assert old in src, f"mutation site for {name!r} not found"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    monkeypatch.setattr(oracle, fname, ns[fname])
    if fname == "prologue":  # forward_fused looks the prologue up in the module
        ns2 = dict(vars(oracle))
        exec(compile(_FUSED_SRC, "<forward_fused>", "exec"), ns2)
        monkeypatch.setattr(oracle, "forward_fused", ns2["forward_fused"])
    with pytest.raises(AssertionError):
        pins.test_forward_fused_worked_example()


def test_unmodified_fused_passes_the_pin():
    pins.test_forward_fused_worked_example()
