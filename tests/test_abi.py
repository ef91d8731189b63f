"""The C-ABI library: it loads, exports every entry point include/moe_ffn.h
declares, and rejects bad arguments before touching the GPU (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_ffn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def b():
    from quantized_moe_wave_amd import binding

    return binding


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("moe_ffn_create", "moe_ffn_reserve", "moe_ffn_forward", "moe_ffn_debug_routing", "moe_ffn_destroy",
              "moe_ffn_last_error", "moe_ffn_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(b):
    from quantized_moe_wave_amd.build import LIB

    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(b.lib(), n)


def test_abi_version(b):
    assert b.abi_version() == 3


def _shape(b, H=256, E=8, k=2, I=256):
    return b.MoeFfnShape(H, E, k, I)


def _create(b, shape, gb=None, ub=None, db=None, ptr=None):
    H, E, I = shape.hidden_dim, shape.num_experts, shape.moe_intermediate
    gbytes = E * I * max(H // 256, 0) * 144
    dbytes = E * H * max(I // 256, 0) * 144
    out = ctypes.c_void_p()
    st = b.lib().moe_ffn_create(ctypes.byref(shape), ptr, gbytes if gb is None else gb, ptr,
                                gbytes if ub is None else ub, ptr, dbytes if db is None else db, ptr, None, None,
                                ctypes.byref(out))
    return st, out.value, b.lib().moe_ffn_last_error().decode()


@pytest.mark.parametrize("dims,frag", [
    ((256, 0, 2, 256), "num_experts=0"),
    ((256, 8, 0, 256), "num_experts_per_tok=0"),
    ((256, 8, 2, 0), "moe_intermediate=0"),
    ((256, 8, 9, 256), "exceeds num_experts"),
    ((300, 8, 2, 256), "multiples of 256"),
    ((256, 8, 2, 100), "multiples of 256"),
    ((256, 2000, 2, 256), "must be <="),
    ((256, 128, 65, 256), "must be <="),
])
def test_invalid_shapes(b, dims, frag):
    st, h, msg = _create(b, _shape(b, *dims))
    assert st == 1 and h is None and frag in msg


def test_blob_size_mismatch(b):
    st, h, msg = _create(b, _shape(b), gb=1000)
    assert st == 3 and "blob sizes" in msg
    st, h, msg = _create(b, _shape(b), db=1)
    assert st == 3


def test_null_pointers_rejected(b):
    st, h, msg = _create(b, _shape(b))
    assert st == 2 and "NULL" in msg
    assert b.lib().moe_ffn_create(None, None, 0, None, 0, None, 0, None, None, None, None) == 2


def test_null_handle_calls(b):
    lib = b.lib()
    assert lib.moe_ffn_forward(None, 1, None, None, None, None, None) == 2
    assert lib.moe_ffn_reserve(None, 4, None) == 2
    assert lib.moe_ffn_debug_routing(None, None, None, None, None, None) == 2
    assert lib.moe_ffn_destroy(None) == 0
    assert "handle" in lib.moe_ffn_last_error().decode()
