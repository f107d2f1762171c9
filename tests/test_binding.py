"""Host-side checks of the Python binding that need no GPU: no top-level name is
defined twice (a later definition would silently replace the first), and the
tensor-dtype and dtype-name maps give the C ABI's codes."""
import ast
import os

import pytest

import linear_rnn_sequence_amd
from linear_rnn_sequence_amd import wkv

torch = pytest.importorskip("torch")


def test_no_top_level_name_defined_twice():
    path = os.path.join(os.path.dirname(linear_rnn_sequence_amd.__file__), "wkv.py")
    tree = ast.parse(open(path).read())
    names = [n.name for n in tree.body if isinstance(n, (ast.FunctionDef, ast.ClassDef))]
    dup = sorted({n for n in names if names.count(n) > 1})
    assert not dup, dup


def test_dtype_maps():
    assert wkv._dtype_code(torch, torch.float32) == wkv.DT_F32 == 0
    assert wkv._dtype_code(torch, torch.bfloat16) == wkv.DT_BF16 == 1
    assert wkv._dtype_name_code("bf16_w32") == wkv.DT_BF16_W32 == 2
    assert wkv._dtype_name_code("float32") == 0 and wkv._dtype_name_code("bfloat16") == 1
    with pytest.raises(ValueError):
        wkv._dtype_name_code("fp16")
