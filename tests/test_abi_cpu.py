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
    w3t = moe.Weights(w_gate=256, w_up=512, w_down=768, layout=moe.LAYOUT_TILED)
    assert L.moe_layer(ctypes.byref(fp8), 1024, 2048, ctypes.byref(w3t), 4096, None, 8192, 1 << 40,
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


@pytest.mark.parametrize("name,bytes_per_128", [("moe_mxfp4_tile", 64), ("moe_fp8_tile", 128)])
def test_weight_tile_argument_errors(name, bytes_per_128):
    """moe_mxfp4_tile and moe_fp8_tile reject bad arguments on the host, before any launch."""
    L = moe.lib()
    fn = getattr(L, name)
    buf = ctypes.create_string_buffer(1 << 16)
    a = (ctypes.addressof(buf) + 15) // 16 * 16
    b = a + 8192
    assert fn(None, b, 16, 128, None) == moe.MOE_ERR_INVALID_ARG
    assert fn(a, None, 16, 128, None) == moe.MOE_ERR_INVALID_ARG
    assert fn(a + 8, b, 16, 128, None) == moe.MOE_ERR_INVALID_ARG  # misaligned
    assert fn(a, b + 8, 16, 128, None) == moe.MOE_ERR_INVALID_ARG
    assert fn(a, a + 16, 16, 128, None) == moe.MOE_ERR_INVALID_ARG  # overlap
    assert fn(a + 512, a, 16, 128, None) == moe.MOE_ERR_INVALID_ARG  # overlap, dst below src
    assert fn(a, b, 15, 128, None) == moe.MOE_ERR_UNSUPPORTED
    assert fn(a, b, 16, 96, None) == moe.MOE_ERR_UNSUPPORTED
    assert fn(a, b, -16, 128, None) == moe.MOE_ERR_INVALID_ARG
    assert fn(a, b, 16, -128, None) == moe.MOE_ERR_INVALID_ARG
    # 16 rows x 128 elements are 1 KB of MXFP4 and 2 KB of fp8: a destination 1 KB above the
    # source overlaps only the fp8 source (the MXFP4 case would launch, so it is not called here)
    if bytes_per_128 == 128:
        assert fn(a, a + 1024, 16, 128, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(a, a + 2032, 16, 128, None) == moe.MOE_ERR_INVALID_ARG


def test_offset_limits():
    """The kernels use 32-bit byte offsets: shapes whose activation, h or y buffers or one expert's
    matrix reach 4 GiB are rejected (MOE_ERR_UNSUPPORTED), just below the limit they are not."""
    L = moe.lib()
    ws = L.moe_layer_workspace_bytes

    def ok(*a, **kw):
        return ws(ctypes.byref(moe.problem(*a, **kw))) > 0

    # T*k*max(d, f)*2 against 2^32: n = T*k rows
    assert ok(1 << 20, 128, 256, 8, 8) is False          # 2^23 * 256 * 2 = 2^32
    assert ok(1 << 20, 128, 128, 8, 8) is True            # 2^31
    assert ok((1 << 20) - 1, 256, 128, 8, 8) is True      # just below 2^32 (d is the wide one)
    assert ok(131072, 7168, 2048, 384, 8) is False        # Kimi-shaped, 16x the workload's T
    assert ok(8192, 7168, 2048, 384, 8) is True           # the Kimi-shaped workload itself
    assert ok(37450, 7168, 2048, 384, 8) is False         # 299600 * 7168 * 2 >= 2^32
    assert ok(37449, 7168, 2048, 384, 8) is True          # 299592 * 7168 * 2 < 2^32
    # a shared expert's h [T][f_sh]
    assert ok(1 << 16, 128, 128, 8, 1, shared_f=1 << 15) is False
    # one expert's [f][d] matrix
    assert ok(4, 65536, 32768, 8, 2) is False
    assert ok(4, 65536, 32640, 8, 2) is True
    big = moe.problem(131072, 7168, 2048, 384, 8)
    w = moe.Weights(w_gate=256, w_up=512, w_down=768)
    assert L.moe_layer(ctypes.byref(big), 1024, 2048, ctypes.byref(w), 4096, None, 8192, 1 << 40,
                       None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_grouped_ffn(ctypes.byref(big), 1024, None, 2048, 4096, ctypes.byref(w), 8192,
                             16384, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_grouped_ffn_workspace_bytes(ctypes.byref(big)) == 0
    # activation quantisation: T * d / 128 groups; permute's gather: T * k * d / 128 scales
    assert L.moe_quant_act(1024, 1 << 24, 128 * 128, 2048, 4096, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_permute(1024, 1 << 20, 8, 8, 2048, 4096, 256 * 128, moe.DTYPE_FP8, 256, 512, 768,
                         1280, 8192, None, 16384, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED


def test_narrow_weight_formats_need_the_tiled_layout():
    """fp8 and mxfp4 weight bytes have the same size in either layout, so the caller tags them:
    row-major bytes of these formats (or bf16 weights tagged tiled) are rejected before any work."""
    L = moe.lib()
    ptrs = dict(w_gate=256, w_up=512, w_down=768, s_gate=1024, s_up=1280, s_down=1536,
                e_gate=1792, e_up=2048, e_down=2304)
    for wd in (moe.DTYPE_FP8, moe.DTYPE_MXFP4):
        p = moe.problem(8, 256, 512, 8, 2, wdtype=wd)
        row = moe.Weights(**ptrs, layout=moe.LAYOUT_ROW_MAJOR)
        tiled = moe.Weights(**ptrs, layout=moe.LAYOUT_TILED)
        assert L.moe_layer(ctypes.byref(p), 4096, 8192, ctypes.byref(row), 16384, None, 32768, 16,
                           None) == moe.MOE_ERR_INVALID_ARG
        # tagged tiled, the call gets as far as the (too small) workspace
        assert L.moe_layer(ctypes.byref(p), 4096, 8192, ctypes.byref(tiled), 16384, None, 32768, 16,
                           None) == moe.MOE_ERR_WORKSPACE
        assert L.moe_grouped_ffn(ctypes.byref(p), 4096, 4352, 8192, 12288, ctypes.byref(row),
                                 16384, 32768, 16, None) == moe.MOE_ERR_INVALID_ARG
    # the E8M0 scale arrays are staged with 4-byte loads: each must be 4-byte aligned
    for name in ("e_gate", "e_up", "e_down"):
        for wd in (moe.DTYPE_MXFP4, moe.DTYPE_MXFP4_A8):
            p = moe.problem(8, 256, 512, 8, 2, wdtype=wd)
            off = moe.Weights(**dict(ptrs, **{name: ptrs[name] + 2}), layout=moe.LAYOUT_TILED)
            assert L.moe_layer(ctypes.byref(p), 4096, 8192, ctypes.byref(off), 16384, None, 32768,
                               16, None) == moe.MOE_ERR_INVALID_ARG
    # MFMA tiles exist for mxfp4 weights with mxfp8 activations, not with bf16 activations
    tiled = moe.Weights(**ptrs, layout=moe.LAYOUT_TILED)
    for wd, want in ((moe.DTYPE_MXFP4, moe.MOE_ERR_UNSUPPORTED),
                     (moe.DTYPE_MXFP4_A8, moe.MOE_ERR_WORKSPACE)):
        p = moe.problem(8, 256, 512, 8, 2, wdtype=wd, config=moe.CONFIG_MFMA)
        assert L.moe_layer(ctypes.byref(p), 4096, 8192, ctypes.byref(tiled), 16384, None, 32768,
                           16, None) == want
    bf = moe.problem(8, 256, 512, 8, 2)
    assert L.moe_layer(ctypes.byref(bf), 4096, 8192,
                       ctypes.byref(moe.Weights(w_gate=256, w_up=512, w_down=768,
                                                layout=moe.LAYOUT_TILED)),
                       16384, None, 32768, 16, None) == moe.MOE_ERR_INVALID_ARG


def test_binding_tags_only_tiled_tensors():
    """The binding sets the tiled tag only when every fp8 / mxfp4 weight tensor came from
    fp8_tile / mxfp4_tile (marked by them); bf16 weights are always row-major."""
    import torch
    g = torch.zeros((2, 128, 128), dtype=torch.uint8)
    u, dn = torch.zeros_like(g), torch.zeros_like(g)
    s = torch.ones((2, 1, 1), dtype=torch.float32)
    ew = moe.ExpertWeights(gate=g, up=u, down=dn, s_gate=s, s_up=s, s_down=s)
    assert ew.struct().layout == moe.LAYOUT_ROW_MAJOR
    for t in (g, u):
        t._moe_tiled = True
    assert ew.struct().layout == moe.LAYOUT_ROW_MAJOR  # down is still row-major
    dn._moe_tiled = True
    assert ew.struct().layout == moe.LAYOUT_TILED
    bf = moe.ExpertWeights(gate=torch.zeros((2, 128, 128), dtype=torch.int16),
                           up=torch.zeros((2, 128, 128), dtype=torch.int16),
                           down=torch.zeros((2, 128, 128), dtype=torch.int16))
    assert bf.struct().layout == moe.LAYOUT_ROW_MAJOR


def test_noalloc_rejects_problems_beyond_its_scratch():
    """moe_layer_noalloc checks the workspace its problem needs against the static scratch on the
    host, before any device call."""
    L = moe.lib()
    ws = L.moe_layer_workspace_bytes
    small = moe.problem(256, 7168, 2048, 256, 8)  # DeepSeek-V3-shaped decode, T = 256
    big = moe.problem(512, 7168, 2048, 256, 8)
    assert 0 < ws(ctypes.byref(small)) <= moe.NOALLOC_SCRATCH_BYTES < ws(ctypes.byref(big))
    w = moe.Weights(w_gate=256, w_up=512, w_down=768)
    assert L.moe_layer_noalloc(ctypes.byref(big), 1024, 2048, ctypes.byref(w), 4096, None,
                               None) == moe.MOE_ERR_WORKSPACE
    mixtral = moe.problem(4096, 4096, 14336, 8, 2)
    assert L.moe_layer_noalloc(ctypes.byref(mixtral), 1024, 2048, ctypes.byref(w), 4096, None,
                               None) == moe.MOE_ERR_WORKSPACE
    bad = moe.problem(8, 250, 512, 8, 2)  # invalid problems keep moe_layer's codes
    assert L.moe_layer_noalloc(ctypes.byref(bad), 1024, 2048, ctypes.byref(w), 4096, None,
                               None) == moe.MOE_ERR_UNSUPPORTED
    assert b"static scratch" in L.moe_status_string(moe.MOE_ERR_WORKSPACE)


def test_policy_configs():
    """config 16 + i forces selection policy i for bf16 weights; other values are rejected, and the
    streaming-only formats reject policies."""
    L = moe.lib()
    ws = L.moe_layer_workspace_bytes
    for i in range(moe.NUM_POLICIES):
        assert ws(ctypes.byref(moe.problem(64, 256, 512, 8, 2, config=moe.CONFIG_POLICY0 + i))) > 0
    for bad in (3, 15, moe.CONFIG_POLICY0 + moe.NUM_POLICIES, -2):
        assert ws(ctypes.byref(moe.problem(64, 256, 512, 8, 2, config=bad))) == 0
    fp8 = moe.problem(64, 256, 512, 8, 2, fp8=True, config=moe.CONFIG_POLICY0)
    w = moe.Weights(w_gate=256, w_up=512, w_down=768)
    assert L.moe_layer(ctypes.byref(fp8), 1024, 2048, ctypes.byref(w), 4096, None, 8192, 16,
                       None) == moe.MOE_ERR_UNSUPPORTED


def test_fused_config_limits():
    """MOE_CONFIG_FUSED runs the whole layer of one bf16 token in one launch: more tokens, other
    weight formats, a shared expert, d_model or d_ff above 8192, and the grouped FFN entry point are
    rejected before any device work; the layer workspace starts with the launch's 36 KB of counters."""
    L = moe.lib()
    ws = L.moe_layer_workspace_bytes
    F = moe.CONFIG_FUSED
    ok = moe.problem(1, 7168, 2048, 256, 8, config=F)
    assert ws(ctypes.byref(ok)) > moe.FUSED_SYNC_BYTES
    assert ws(ctypes.byref(moe.problem(0, 256, 512, 8, 2, config=F))) > 0  # T = 0: a no-op call
    assert ws(ctypes.byref(moe.problem(1, 8192, 8192, 8, 2, config=F))) > 0
    for bad in (moe.problem(2, 256, 512, 8, 2, config=F),
                moe.problem(1, 256, 512, 8, 2, fp8=True, config=F),
                moe.problem(1, 256, 512, 8, 2, shared_f=256, config=F),
                moe.problem(1, 8320, 512, 8, 2, config=F),
                moe.problem(1, 256, 8320, 8, 2, config=F),
                moe.problem(1, 256, 512, 8, 2, wdtype=moe.DTYPE_MXFP4, config=F)):
        assert ws(ctypes.byref(bad)) == 0
        w = moe.Weights(w_gate=256, w_up=512, w_down=768)
        assert L.moe_layer(ctypes.byref(bad), 1024, 2048, ctypes.byref(w), 4096, None, 8192, 1 << 20,
                           None) == moe.MOE_ERR_UNSUPPORTED
    # the grouped FFN has no fused form
    w = moe.Weights(w_gate=256, w_up=512, w_down=768)
    assert L.moe_grouped_ffn(ctypes.byref(ok), 1024, None, 2048, 4096, ctypes.byref(w), 8192,
                             12288, 1 << 20, None) == moe.MOE_ERR_UNSUPPORTED
    # every layer workspace holds the counters, so the fused and automatic forms of a problem need
    # the same bytes
    auto = moe.problem(1, 7168, 2048, 256, 8)
    assert ws(ctypes.byref(ok)) == ws(ctypes.byref(auto))
