"""The C ABI library on the CPU: it loads, exports every function include/*.h declares, and rejects
bad arguments on the host before any GPU work (no compute calls here)."""
import ctypes
import glob
import os
import re

import pytest

from mixture_experts_layer_top_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src))
    return names


def test_library_exports_every_declared_function():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("library not built")
    names = _declared()
    assert {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer"} <= names
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(moe.EXPORTED) == names


def test_status_strings():
    L = moe.lib()
    for s in range(5):
        assert L.moe_status_string(s).startswith(b"MOE_")


def test_host_side_argument_errors():
    L = moe.lib()
    # bad shapes are rejected before any pointer is touched
    assert L.moe_route(None, 4, 8, 0, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, 4, 8, 9, None, None, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_route(None, 4, 600, 2, None, None, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_route(None, 4, 8, 2, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, 0, 8, 2, None, None, None) == moe.MOE_OK  # T = 0: no-op
    assert L.moe_quant_act(None, 2, 100, None, None, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(None, None, None, 3, 2, 256, None, None, None) == moe.MOE_ERR_INVALID_ARG
    p = moe.problem(8, 256, 512, 8, 2)
    assert L.moe_layer_workspace_bytes(ctypes.byref(p)) > 0
    bad = moe.problem(8, 250, 512, 8, 2)
    assert L.moe_layer_workspace_bytes(ctypes.byref(bad)) == 0
    w = moe.Weights()
    assert L.moe_layer(ctypes.byref(bad), None, None, ctypes.byref(w), None, None, None, 0,
                       None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_layer(ctypes.byref(p), None, None, ctypes.byref(w), None, None, None, 0,
                       None) == moe.MOE_ERR_INVALID_ARG
    # misaligned weight pointer
    w2 = moe.Weights(w_gate=16, w_up=18, w_down=32)
    assert L.moe_layer(ctypes.byref(p), None, None, ctypes.byref(w2), None, None, None, 0,
                       None) == moe.MOE_ERR_INVALID_ARG
    # workspace too small (pointers non-null and aligned but never dereferenced on this path)
    w3 = moe.Weights(w_gate=256, w_up=512, w_down=768)
    assert L.moe_layer(ctypes.byref(p), 1024, 2048, ctypes.byref(w3), 4096, None, 8192, 16,
                       None) == moe.MOE_ERR_WORKSPACE
    fp8 = moe.problem(8, 256, 512, 8, 2, fp8=True)
    assert L.moe_layer(ctypes.byref(fp8), 1024, 2048, ctypes.byref(w3), 4096, None, 8192, 1 << 40,
                       None) == moe.MOE_ERR_INVALID_ARG  # fp8 without scales
    T0 = moe.problem(0, 256, 512, 8, 2)
    assert L.moe_layer(ctypes.byref(T0), None, None, ctypes.byref(w3), None, None, None, 0,
                       None) == moe.MOE_OK


def test_workspace_sizes_scale():
    L = moe.lib()
    a = moe.problem(64, 256, 512, 8, 2)
    b = moe.problem(128, 256, 512, 8, 2)
    assert L.moe_layer_workspace_bytes(ctypes.byref(b)) > L.moe_layer_workspace_bytes(ctypes.byref(a))
    assert L.moe_permute_workspace_bytes(64, 8, 2) > 0
    assert L.moe_grouped_ffn_workspace_bytes(ctypes.byref(a)) > 0


def test_mxfp4_tile_argument_errors():
    """moe_mxfp4_tile rejects bad arguments on the host, before any launch."""
    L = moe.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    a = (ctypes.addressof(buf) + 15) // 16 * 16
    b = a + 8192
    assert L.moe_mxfp4_tile(None, b, 16, 128, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp4_tile(a, None, 16, 128, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp4_tile(a + 8, b, 16, 128, None) == moe.MOE_ERR_INVALID_ARG  # misaligned
    assert L.moe_mxfp4_tile(a, a + 16, 16, 128, None) == moe.MOE_ERR_INVALID_ARG  # overlap
    assert L.moe_mxfp4_tile(a, b, 15, 128, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_mxfp4_tile(a, b, 16, 96, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_mxfp4_tile(a, b, -16, 128, None) == moe.MOE_ERR_INVALID_ARG
