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


def test_pair_scales_rejects(lib):
    # odd row count, a row length that is not a multiple of 64, null,
    # misaligned, overlapping: all rejected before any launch; nothing to do
    # for zero rows
    assert lib.nvfp4_pair_scales(FAKE, 3, 64, ctypes.c_void_p(0x20000), None) == -1
    assert lib.nvfp4_pair_scales(FAKE, 4, 48, ctypes.c_void_p(0x20000), None) == -1
    assert b"C % 64" in lib.nvfp4_last_error()
    assert lib.nvfp4_pair_scales(None, 4, 64, ctypes.c_void_p(0x20000), None) == -1
    assert lib.nvfp4_pair_scales(ctypes.c_void_p(0x10008), 4, 64, ctypes.c_void_p(0x20000), None) == -1
    assert lib.nvfp4_pair_scales(FAKE, 4, 64, ctypes.c_void_p(0x10000 + 128), None) == -1
    assert b"overlap" in lib.nvfp4_last_error()
    assert lib.nvfp4_pair_scales(None, 0, 64, None, None) == 0


def test_gemm_stage_rejects(lib):
    # K not a multiple of 64, N2 not a multiple of 256, negative M
    assert lib.nvfp4_gemm_swiglu_quant(FAKE, FAKE, FAKE, 4, 48, FAKE, FAKE, FAKE, 256, FAKE, None,
                                       FAKE, FAKE, None, 0, None) == -2
    assert lib.nvfp4_gemm_swiglu_quant(FAKE, FAKE, FAKE, 4, 64, FAKE, FAKE, FAKE, 128, FAKE, None,
                                       FAKE, FAKE, None, 0, None) == -2
    assert lib.nvfp4_gemm_swiglu_quant(FAKE, FAKE, FAKE, -1, 64, FAKE, FAKE, FAKE, 256, FAKE, None,
                                       FAKE, FAKE, None, 0, None) == -1
    assert lib.nvfp4_gemm_swiglu_quant(None, FAKE, FAKE, 4, 64, FAKE, FAKE, FAKE, 256, FAKE, None,
                                       FAKE, FAKE, None, 0, None) == -1
    # the NVFP4 activation operand (M * K / 2 bytes) above 4 GiB
    assert lib.nvfp4_gemm_swiglu_quant(FAKE, FAKE, FAKE, (1 << 27) + 1, 64, FAKE, FAKE, FAKE, 256,
                                       FAKE, None, FAKE, FAKE, None, 0, None) == -2
    # with a workspace, the f16 copy of the activations (M * K * 2 bytes) above 4 GiB
    assert lib.nvfp4_gemm_swiglu_quant(FAKE, FAKE, FAKE, (1 << 25) + 1, 64, FAKE, FAKE, FAKE, 256,
                                       FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == -2
    assert b"4 GiB" in lib.nvfp4_last_error()
    # a workspace smaller than the f16 copy
    need = lib.nvfp4_gemm_swiglu_quant_workspace_size(4, 64, 256)
    assert need >= 4 * 64 * 2
    assert lib.nvfp4_gemm_swiglu_quant(FAKE, FAKE, FAKE, 4, 64, FAKE, FAKE, FAKE, 256,
                                       FAKE, None, FAKE, FAKE, FAKE, need - 1, None) == -3
    assert b"workspace" in lib.nvfp4_last_error()
    # M == 0 is a valid no-op
    assert lib.nvfp4_gemm_swiglu_quant(None, None, None, 0, 64, None, None, None, 256, None, None,
                                       None, None, None, 0, None) == 0


def _moe_args(**kw):
    import quantization_nvfp4_quantize_amd as q
    f = dict(T=4, H=256, I=128, E=8, topk=2, x=0x10000, x_gs_in=None, topk_ids=0x10000,
             topk_w=0x10000, w1_q=0x10000, w1_sf=0x10000, w1_gs=0x10000, w2_q=0x10000,
             w2_sf=0x10000, w2_gs=0x10000, a2_gs=0x10000, out=0x10000, out_dtype=1)
    f.update(kw)
    a = q.MoeArgs()
    for k, v in f.items():
        setattr(a, k, v)
    return a


def test_moe_rejects(lib):
    import quantization_nvfp4_quantize_amd as q
    by = ctypes.byref
    assert lib.moe_expert_ffn_nvfp4(None, FAKE, 1 << 30, None) == -1
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(H=200)), FAKE, 1 << 30, None) == -2
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(I=96)), FAKE, 1 << 30, None) == -2
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(E=0)), FAKE, 1 << 30, None) == -1
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(E=513)), FAKE, 1 << 30, None) == -2
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(topk=33)), FAKE, 1 << 30, None) == -2
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(out_dtype=3)), FAKE, 1 << 30, None) == -1
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(w2_gs=None)), FAKE, 1 << 30, None) == -1
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(x=0x10008)), FAKE, 1 << 30, None) == -1
    # row-paired weight scales are read 16 bytes at a time
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(w1_sf_paired=0x10004)), FAKE, 1 << 30, None) == -1
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(w2_sf_paired=0x10008)), FAKE, 1 << 30, None) == -1
    # GEMM tiling: 0 (automatic), 32, 256 or 288 (mixed) only
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(tile_rows=64)), FAKE, 1 << 30, None) == -1
    assert b"tile_rows" in lib.nvfp4_last_error()
    # a second stream needs its two events
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(aux_stream=0x1234)), FAKE, 1 << 30, None) == -1
    assert b"aux_events" in lib.nvfp4_last_error()
    # 32-row tiles (alone or in the mixed tiling) need H and I multiples of 256 (or 128)
    for tr in (32, 288):
        assert lib.moe_expert_ffn_nvfp4(by(_moe_args(I=384, tile_rows=tr)), FAKE, 1 << 30, None) == -2
        assert b"multiples of 256" in lib.nvfp4_last_error()
    # the workspace follows the tile height (the tile list is sized per tile)
    small = lib.moe_expert_ffn_nvfp4_workspace_size(by(_moe_args(T=4096, tile_rows=32)))
    large = lib.moe_expert_ffn_nvfp4_workspace_size(by(_moe_args(T=4096, tile_rows=256)))
    assert small > large > 0
    # f16 operands above 4 GiB: x (T * H * 2) and the L2 input (T * k * I * 2)
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(T=1 << 19, H=1 << 13)), FAKE, 1 << 30, None) == -2
    assert b"4 GiB" in lib.nvfp4_last_error()
    assert lib.moe_expert_ffn_nvfp4(by(_moe_args(T=1 << 17, topk=8, I=1 << 12)), FAKE, 1 << 30,
                                    None) == -2
    a = _moe_args()
    need = lib.moe_expert_ffn_nvfp4_workspace_size(by(a))
    assert need > 0
    assert lib.moe_expert_ffn_nvfp4(by(a), FAKE, need - 1, None) == -3
    assert b"workspace" in lib.nvfp4_last_error()
    del q


def test_linear_rejects(lib):
    # shape checks come before any pointer is used
    assert lib.nvfp4_linear(FAKE, 4, 48, None, FAKE, FAKE, FAKE, 256, 0, FAKE, None, FAKE, 1 << 30, None) == -2
    assert lib.nvfp4_linear(FAKE, 4, 64, None, FAKE, FAKE, FAKE, 200, 0, FAKE, None, FAKE, 1 << 30, None) == -2
    assert lib.nvfp4_linear(FAKE, -1, 64, None, FAKE, FAKE, FAKE, 256, 0, FAKE, None, FAKE, 1 << 30, None) == -1
    assert lib.nvfp4_linear(FAKE, 4, 64, None, FAKE, FAKE, FAKE, 256, 2, FAKE, None, FAKE, 1 << 30, None) == -1
    assert lib.nvfp4_linear(None, 4, 64, None, FAKE, FAKE, FAKE, 256, 0, FAKE, None, FAKE, 1 << 30, None) == -1
    assert lib.nvfp4_linear(ctypes.c_void_p(0x10008), 4, 64, None, FAKE, FAKE, FAKE, 256, 0, FAKE, None, FAKE,
                            1 << 30, None) == -1
    # out is written with 16-byte stores: an offset out pointer is rejected
    for off in (4, 8):
        assert lib.nvfp4_linear(FAKE, 4, 64, None, FAKE, FAKE, FAKE, 256, 1, ctypes.c_void_p(0x10000 + off), None,
                                FAKE, 1 << 30, None) == -1
        assert b"misaligned" in lib.nvfp4_last_error()
    need = lib.nvfp4_linear_workspace_size(4, 64, 256)
    assert need > 0
    assert lib.nvfp4_linear(FAKE, 4, 64, None, FAKE, FAKE, FAKE, 256, 0, FAKE, None, FAKE, need - 1, None) == -3
    assert b"workspace" in lib.nvfp4_last_error()
    # an empty batch is a no-op
    assert lib.nvfp4_linear(None, 0, 64, None, None, None, None, 256, 0, None, None, None, 0, None) == 0


def test_build_scripts_need_no_built_library(tmp_path):
    """build() must work on a fresh checkout, before any .so exists: the
    oracle's build submodule resolves without loading the default oracle, and
    both build scripts load by path without importing their packages."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import importlib, sys; sys.path.insert(0, %r); "
            "import oracle; m = oracle.build; "
            "assert m.__name__ == 'oracle.build', m; "
            "assert oracle._default is None; "
            "import __graft_entry__ as g; "
            "h = g._load_script('quantization_nvfp4_quantize_amd/build.py', '_t'); "
            "assert callable(h.build); "
            "assert 'quantization_nvfp4_quantize_amd' not in sys.modules") % root
    subprocess.run([sys.executable, "-c", code], check=True, cwd=str(tmp_path))


def test_mxfp4_rejects_bad_args(lib):
    """The MXFP4 entry points validate before any launch."""
    assert lib.mxfp4_quantize(FAKE, 4, 48, FAKE, FAKE, None) == -1  # K % 32
    assert lib.mxfp4_quantize(None, 4, 64, FAKE, FAKE, None) == -1
    assert lib.mxfp4_quantize(ctypes.c_void_p(0x10008), 4, 64, FAKE, FAKE, None) == -1  # x misaligned
    assert lib.mxfp4_quantize(FAKE, 0, 64, None, None, None) == 0  # empty: nothing to do
    assert lib.mxfp4_dequantize(FAKE, FAKE, 4, 64, 2, FAKE, None) == -1  # out_dtype
    ws = lib.mxfp4_linear_workspace_size(4, 256, 256)
    assert ws >= 4 * 256 // 2 + 4 * 256 // 32
    assert lib.mxfp4_linear(FAKE, 4, 192, FAKE, FAKE, 256, 0, FAKE, FAKE, ws, None) == -2  # K % 128
    assert lib.mxfp4_linear(FAKE, 4, 256, FAKE, FAKE, 128, 0, FAKE, FAKE, ws, None) == -2  # N % 256
    assert lib.mxfp4_linear(FAKE, 4, 256, FAKE, FAKE, 256, 0, FAKE, FAKE, ws - 1, None) == -3
    assert lib.mxfp4_linear(FAKE, 4, 256, None, FAKE, 256, 0, FAKE, FAKE, ws, None) == -1
    assert lib.mxfp4_linear(FAKE, 4, 256, FAKE, FAKE, 256, 0, FAKE, ctypes.c_void_p(0x10010), ws, None) == -1
    assert b"mxfp4_linear" in lib.nvfp4_last_error()


def test_moe_noalloc_rejects_before_any_launch(lib):
    """The allocation-free MoE entry point validates like the workspace one
    and rejects a call whose workspace exceeds its static buffer with
    NVFP4_ERR_WORKSPACE, before touching the device."""
    by = ctypes.byref
    assert lib.moe_expert_ffn_nvfp4_noalloc(None, None) == -1
    assert lib.moe_expert_ffn_nvfp4_noalloc(by(_moe_args(H=200)), None) == -2
    big = _moe_args(T=16384, H=7168, I=2048, E=256, topk=8)
    assert lib.moe_expert_ffn_nvfp4_workspace_size(by(big)) > 64 << 20
    assert lib.moe_expert_ffn_nvfp4_noalloc(by(big), None) == -3
    msg = lib.nvfp4_last_error()
    assert b"noalloc" in msg and b"static buffer" in msg
    dec = _moe_args(T=128, H=7168, I=2048, E=256, topk=8, out_dtype=1)
    assert lib.moe_expert_ffn_nvfp4_workspace_size(by(dec)) <= 64 << 20
