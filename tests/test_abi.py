"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/nvfp4moe.h declares, and rejects bad arguments before any
HIP call (so these run on a host without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    import quantization_nvfp4_quantize_amd as q
    return q._lib


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "nvfp4_quantize" in names and "moe_expert_ffn_nvfp4" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in nvfp4moe.h but not exported"


def test_binding_covers_header():
    import quantization_nvfp4_quantize_amd as q
    assert sorted(q.EXPORTS) == declared_functions()


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert lib.nvfp4_status_string(s)
    assert lib.nvfp4_version() >= 1


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("M,K", [(-1, 16), (4, 0), (4, 15), (4, 24)])
def test_quantize_rejects_bad_shape(lib, M, K):
    st = lib.nvfp4_quantize(FAKE, M, K, FAKE, FAKE, FAKE, None, None, 0, None)
    assert st == -1
    assert b"nvfp4_quantize" in lib.nvfp4_last_error()


def test_quantize_rejects_null_and_misaligned(lib):
    assert lib.nvfp4_quantize(None, 4, 16, FAKE, FAKE, FAKE, None, None, 0, None) == -1
    assert lib.nvfp4_quantize(FAKE, 4, 16, None, FAKE, FAKE, None, None, 0, None) == -1  # no gs_out
    assert lib.nvfp4_quantize(ctypes.c_void_p(0x10002), 4, 16, FAKE, FAKE, FAKE, None, None, 0, None) == -1


def test_quantize_workspace_too_small(lib):
    need = lib.nvfp4_quantize_workspace_size(4, 16)
    assert need > 0
    st = lib.nvfp4_quantize(FAKE, 4, 16, None, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert st == -3
    assert b"workspace" in lib.nvfp4_last_error()


def test_dequantize_rejects(lib):
    assert lib.nvfp4_dequantize(FAKE, FAKE, FAKE, 4, 16, 2, FAKE, None) == -1
    assert lib.nvfp4_dequantize(FAKE, FAKE, FAKE, 4, 17, 0, FAKE, None) == -1
    assert lib.nvfp4_dequantize(None, FAKE, FAKE, 4, 16, 0, FAKE, None) == -1
