"""Host-side checks of the C ABI: the library loads, exports every function include/gpt2.h
declares (and the binding knows each signature), and rejects bad arguments before it
touches a device. No kernel is launched here."""
import ctypes
import os
import re

import pytest

from decoder_only_transformer_05_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt2.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gpt2_build", "gpt2_forward", "gpt2_backward", "gpt2_adamw_step",
                     "gpt2_zero_grad", "gpt2_free"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in gpt2.h but not exported"
        assert name in binding.SIGNATURES, f"{name} has no binding signature"
    assert set(binding.SIGNATURES) == set(declared_functions())


def test_version_string():
    assert b"gfx950" in binding.lib().gpt2_version()


@pytest.mark.parametrize("dims", [
    (1, 18, 4, 27, 16),     # C % H != 0
    (1, 18, 3, 27, 16),     # C % 4 != 0
    (1, 24, 4, 27, 16),     # head size 6 not a multiple of 4
    (0, 16, 4, 27, 16),     # L < 1
    (1, 16, 4, 0, 16),      # V < 1
    (1, 16, 4, 27, 0),      # maxT < 1
    (1, 1024, 4, 27, 16),   # head size 256 > 128
    (1, 4096, 32, 27, 16),  # C above 2048
    (1, 16, 4, 1 << 21, 16),  # V at 2^21: the token sort keeps tokens in 21 bits
])
def test_build_rejects_bad_shapes_without_a_device(dims):
    lib = binding.lib()
    h = ctypes.c_void_p()
    rc = lib.gpt2_build(ctypes.byref(h), *dims)
    assert rc == -1 and not h.value
    assert lib.gpt2_last_global_error()


def test_null_arguments_are_errors_not_crashes():
    lib = binding.lib()
    assert lib.gpt2_build(None, 1, 16, 4, 27, 16) == -1
    assert lib.gpt2_forward(None, None, None, 1, 1, None) == -1
    assert lib.gpt2_backward(None) == -1
    assert lib.gpt2_adamw_step(None, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1) == -1
    assert lib.gpt2_zero_grad(None) == -1
    assert lib.gpt2_num_params(None) == 0
    lib.gpt2_free(None)
    h = ctypes.c_void_p()
    # preallocation with T above maxT
    assert lib.gpt2_build_ex(ctypes.byref(h), 1, 16, 4, 27, 16, 0, 2, 17, None) == -1
    # unsupported dtype
    assert lib.gpt2_build_ex(ctypes.byref(h), 1, 16, 4, 27, 16, 7, 0, 0, None) == -1
