"""Thin Python binding of libmoe_mi355x.so (the C ABI in include/moe_mi355x.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.  torch is
used for device memory (output and workspace tensors) and for the current HIP stream.  If the
library is not built this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB may point at another build of the same library (e.g. to compare two builds).
LIB_PATH = os.environ.get("MOE_MI355X_LIB", os.path.join(_PKG, "libmoe_mi355x.so"))

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
DTYPE_BF16, DTYPE_FP8, DTYPE_MXFP4, DTYPE_MXFP4_A8 = 0, 1, 2, 3
CONFIG_AUTO, CONFIG_STREAM, CONFIG_MFMA, CONFIG_FUSED = -1, 0, 1, 2
FUSED_SYNC_BYTES = 36864    # the fused single-token launch's counters at the workspace's start
CONFIG_POLICY0, NUM_POLICIES = 16, 8  # config = 16 + i forces selection policy i (bf16)
LAYOUT_ROW_MAJOR, LAYOUT_TILED = 0, 1

_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("has_shared", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("config", ctypes.c_int32)]


WEIGHT_POINTERS = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                   "sh_gate", "sh_up", "sh_down", "s_sh_gate", "s_sh_up", "s_sh_down",
                   "e_gate", "e_up", "e_down")


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_POINTERS] + [("layout", ctypes.c_int32)]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_ids", "topk_w", "counts", "offsets", "perm_src", "slot_dst", "eeff", "policy")]


class MoEError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the library (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_top_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_route": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp]),
            "moe_permute": (_i, [_vp, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _sz, _vp]),
            "moe_permute_workspace_bytes": (_sz, [_i, _i, _i]),
            "moe_quant_act": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
            "moe_quant_act_mx": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
            "moe_grouped_ffn": (_i, [ctypes.POINTER(Problem), _vp, _vp, _vp, _vp,
                                     ctypes.POINTER(Weights), _vp, _vp, _sz, _vp]),
            "moe_grouped_ffn_workspace_bytes": (_sz, [ctypes.POINTER(Problem)]),
            "moe_combine": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
            "moe_layer": (_i, [ctypes.POINTER(Problem), _vp, _vp, ctypes.POINTER(Weights), _vp,
                               ctypes.POINTER(Routing), _vp, _sz, _vp]),
            "moe_layer_workspace_bytes": (_sz, [ctypes.POINTER(Problem)]),
            "moe_layer_traced": (_i, [ctypes.POINTER(Problem), _vp, _vp, ctypes.POINTER(Weights), _vp,
                                      ctypes.POINTER(Routing), _vp, _sz, ctypes.POINTER(_vp), _i, _vp]),
            "moe_status_string": (ctypes.c_char_p, [_i]),
            "moe_mxfp4_tile": (_i, [_vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp]),
            "moe_fp8_tile": (_i, [_vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp]),
            "moe_layer_noalloc": (_i, [ctypes.POINTER(Problem), _vp, _vp, ctypes.POINTER(Weights),
                                       _vp, ctypes.POINTER(Routing), _vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


EXPORTED = ("moe_route", "moe_permute", "moe_permute_workspace_bytes", "moe_quant_act",
            "moe_quant_act_mx",
            "moe_grouped_ffn", "moe_grouped_ffn_workspace_bytes", "moe_combine", "moe_layer",
            "moe_layer_workspace_bytes", "moe_layer_traced", "moe_status_string", "moe_mxfp4_tile",
            "moe_fp8_tile", "moe_layer_noalloc")

NOALLOC_SCRATCH_BYTES = 128 << 20  # MOE_NOALLOC_SCRATCH_BYTES

TRACE_EVENTS = 8
TRACE_PHASES = ("route", "permute", "quant", "select", "gate_up", "down", "combine")


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoEError(f"{what}: {lib().moe_status_string(status).decode()}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t):
    if not t.is_cuda:
        raise MoEError("tensors must live on the GPU")
    return t.device


@dataclass
class ExpertWeights:
    """Device tensors of the expert weights in the library's storage layout."""
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    s_gate: torch.Tensor | None = None
    s_up: torch.Tensor | None = None
    s_down: torch.Tensor | None = None
    sh_gate: torch.Tensor | None = None
    sh_up: torch.Tensor | None = None
    sh_down: torch.Tensor | None = None
    s_sh_gate: torch.Tensor | None = None
    s_sh_up: torch.Tensor | None = None
    s_sh_down: torch.Tensor | None = None
    e_gate: torch.Tensor | None = None  # mxfp4: uint8 E8M0 scales [E, f, d/32] / [E, d, f/32]
    e_up: torch.Tensor | None = None
    e_down: torch.Tensor | None = None
    act_mx8: bool = False  # mxfp4 weights: quantise activations (and h) to MXFP8 (MOE_DTYPE_MXFP4_A8)

    def struct(self) -> Weights:
        w = Weights()
        for name in WEIGHT_POINTERS:
            key = {"w_gate": "gate", "w_up": "up", "w_down": "down"}.get(name, name)
            setattr(w, name, _ptr(getattr(self, key)))
        w.layout = LAYOUT_ROW_MAJOR
        if self.wdtype != DTYPE_BF16:
            # fp8 / mxfp4 bytes count as tiled only if every weight tensor came from fp8_tile or
            # mxfp4_tile (the library rejects row-major bytes of these formats)
            mats = [self.gate, self.up, self.down] + (
                [self.sh_gate, self.sh_up, self.sh_down] if self.has_shared else [])
            if all(getattr(t, "_moe_tiled", False) for t in mats):
                w.layout = LAYOUT_TILED
        return w

    @property
    def wdtype(self) -> int:
        if self.e_gate is not None:
            return DTYPE_MXFP4_A8 if self.act_mx8 else DTYPE_MXFP4
        return DTYPE_FP8 if self.gate.dtype == torch.uint8 else DTYPE_BF16

    @property
    def fp8(self) -> bool:
        return self.wdtype == DTYPE_FP8

    @property
    def d_model(self) -> int:
        """d from the gate weights' last dim (two mxfp4 elements per byte)."""
        return self.gate.shape[2] * (2 if self.wdtype in (DTYPE_MXFP4, DTYPE_MXFP4_A8) else 1)

    @property
    def has_shared(self) -> bool:
        return self.sh_gate is not None


def problem(T, d, f, E, k, fp8=False, shared_f=0, config=CONFIG_AUTO, wdtype=None) -> Problem:
    if wdtype is None:
        wdtype = DTYPE_FP8 if fp8 else DTYPE_BF16
    return Problem(T, d, f, E, k, wdtype, 1 if shared_f else 0, shared_f, config)


# ------------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------------

def route(logits: torch.Tensor, k: int):
    T, E = logits.shape
    dev = _dev(logits)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream()), "moe_route")
    return ids, w


def permute(ids: torch.Tensor, E: int, x: torch.Tensor | None = None,
            x_scale: torch.Tensor | None = None):
    """Returns counts, offsets, perm_src, slot_dst (and x_perm, x_perm_scale if x is given).
    x: bf16 [T, d] as int16 bits, or e4m3 [T, d] uint8 (with x_scale [T, d/128])."""
    T, k = ids.shape
    dev = _dev(ids)
    n = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm_src = torch.empty(n, dtype=torch.int32, device=dev)
    slot_dst = torch.empty(n, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, lib().moe_permute_workspace_bytes(T, E, k)), dtype=torch.uint8, device=dev)
    xp = xps = None
    d = 0
    act = DTYPE_BF16
    if x is not None:
        d = x.shape[1]
        act = DTYPE_FP8 if x.dtype == torch.uint8 else DTYPE_BF16
        xp = torch.empty((n, d), dtype=x.dtype, device=dev)
        if x_scale is not None:
            xps = torch.empty((n, d // 128), dtype=torch.float32, device=dev)
    _check(lib().moe_permute(_ptr(ids), T, E, k, _ptr(x), _ptr(x_scale), d, act, _ptr(counts),
                             _ptr(offsets), _ptr(perm_src), _ptr(slot_dst), _ptr(xp), _ptr(xps),
                             _ptr(ws), ws.numel(), _stream()), "moe_permute")
    return counts, offsets, perm_src, slot_dst, xp, xps


def mxfp4_tile(w: torch.Tensor) -> torch.Tensor:
    """Row-major MXFP4 bytes [..., rows, cols/2] (uint8) -> the library's tiled layout (same shape;
    every leading dimension folds into the rows)."""
    w = w.contiguous()
    out = torch.empty_like(w)
    rows = w.numel() // w.shape[-1]
    _check(lib().moe_mxfp4_tile(_ptr(w), _ptr(out), rows, 2 * w.shape[-1], _stream()),
           "moe_mxfp4_tile")
    out._moe_tiled = True
    return out


def fp8_tile(w: torch.Tensor) -> torch.Tensor:
    """Row-major fp8 weight bytes [..., rows, cols] (uint8) -> the library's tiled layout."""
    w = w.contiguous()
    out = torch.empty_like(w)
    rows = w.numel() // w.shape[-1]
    _check(lib().moe_fp8_tile(_ptr(w), _ptr(out), rows, w.shape[-1], _stream()), "moe_fp8_tile")
    out._moe_tiled = True
    return out


def quant_act(x: torch.Tensor):
    T, d = x.shape
    dev = _dev(x)
    xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, d // 128), dtype=torch.float32, device=dev)
    _check(lib().moe_quant_act(_ptr(x), T, d, _ptr(xq), _ptr(xs), _stream()), "moe_quant_act")
    return xq, xs


def quant_act_mx(x: torch.Tensor):
    """bf16 [T, d] (int16 bits) -> MXFP8: e4m3 codes [T, d] and E8M0 scale codes [T, d/32]."""
    T, d = x.shape
    dev = _dev(x)
    xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
    xe = torch.empty((T, d // 32), dtype=torch.uint8, device=dev)
    _check(lib().moe_quant_act_mx(_ptr(x), T, d, _ptr(xq), _ptr(xe), _stream()), "moe_quant_act_mx")
    return xq, xe


def grouped_ffn(x_perm, x_perm_scale, counts, offsets, weights: ExpertWeights, T: int, k: int,
                config: int = CONFIG_AUTO):
    n, d = x_perm.shape
    E = counts.shape[0]
    f = weights.gate.shape[1]
    p = problem(T, d, f, E, k, config=config, wdtype=weights.wdtype)
    dev = _dev(x_perm)
    y = torch.empty((n, d), dtype=torch.int16, device=dev)
    ws = torch.empty(max(1, lib().moe_grouped_ffn_workspace_bytes(ctypes.byref(p))),
                     dtype=torch.uint8, device=dev)
    w = weights.struct()
    _check(lib().moe_grouped_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(x_perm_scale), _ptr(counts),
                                 _ptr(offsets), ctypes.byref(w), _ptr(y), _ptr(ws), ws.numel(),
                                 _stream()), "moe_grouped_ffn")
    return y


def combine(y_perm, slot_dst, topk_w, shared_y=None):
    T, k = topk_w.shape
    d = y_perm.shape[1]
    out = torch.empty((T, d), dtype=torch.int16, device=_dev(y_perm))
    _check(lib().moe_combine(_ptr(y_perm), _ptr(slot_dst), _ptr(topk_w), T, k, d, _ptr(shared_y),
                             _ptr(out), _stream()), "moe_combine")
    return out


class Layer:
    """The whole layer with a workspace kept between calls (no allocation per call)."""

    def __init__(self, weights: ExpertWeights, T: int, E: int, k: int, config: int = CONFIG_AUTO,
                 device=None):
        d = weights.d_model
        f = weights.gate.shape[1]
        shf = weights.sh_gate.shape[0] if weights.has_shared else 0
        self.weights = weights
        self.p = problem(T, d, f, E, k, shared_f=shf, config=config, wdtype=weights.wdtype)
        self.w = weights.struct()
        dev = device if device is not None else weights.gate.device
        # (zeroed once: the fused single-token launch keeps its counters, which every call
        # leaves zero, in the first FUSED_SYNC_BYTES)
        self.ws = torch.zeros(max(1, lib().moe_layer_workspace_bytes(ctypes.byref(self.p))),
                              dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, d), dtype=torch.int16, device=dev)

    def __call__(self, logits, x, keep: dict | None = None, out=None):
        r = Routing()
        if keep:
            for name in keep:
                setattr(r, name, _ptr(keep[name]))
        out = self.out if out is None else out
        _check(lib().moe_layer(ctypes.byref(self.p), _ptr(logits), _ptr(x), ctypes.byref(self.w),
                               _ptr(out), ctypes.byref(r), _ptr(self.ws), self.ws.numel(),
                               _stream()), "moe_layer")
        return out

    def traced(self, logits, x, events, keep: dict | None = None, out=None):
        """Same as __call__, recording the TRACE_EVENTS hipEvent_t handles in `events` at the
        phase boundaries (see moe_layer_traced in the C header)."""
        r = Routing()
        if keep:
            for name in keep:
                setattr(r, name, _ptr(keep[name]))
        out = self.out if out is None else out
        arr = (ctypes.c_void_p * TRACE_EVENTS)(*events)
        _check(lib().moe_layer_traced(ctypes.byref(self.p), _ptr(logits), _ptr(x),
                                      ctypes.byref(self.w), _ptr(out), ctypes.byref(r),
                                      _ptr(self.ws), self.ws.numel(), arr, TRACE_EVENTS,
                                      _stream()), "moe_layer_traced")
        return out


def layer(logits, x, weights: ExpertWeights, k: int, config: int = CONFIG_AUTO, keep_routing=False):
    """One call of the whole layer; returns out (bf16 bits, int16) and optionally the routing."""
    T, E = logits.shape
    L = Layer(weights, T, E, k, config)
    keep = None
    if keep_routing:
        dev = logits.device
        n = T * k
        keep = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                    topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
                    counts=torch.empty(E, dtype=torch.int32, device=dev),
                    offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                    perm_src=torch.empty(n, dtype=torch.int32, device=dev),
                    slot_dst=torch.empty(n, dtype=torch.int32, device=dev))
    out = L(logits, x, keep)
    return (out, keep) if keep_routing else out


def layer_noalloc(logits, x, weights: ExpertWeights, k: int, out=None, config: int = CONFIG_AUTO,
                  keep: dict | None = None):
    """The whole layer on the library's static per-GPU scratch (moe_layer_noalloc): nothing is
    allocated for the call apart from `out` when the caller passes none."""
    T, E = logits.shape
    d = weights.d_model
    f = weights.gate.shape[1]
    shf = weights.sh_gate.shape[0] if weights.has_shared else 0
    p = problem(T, d, f, E, k, shared_f=shf, config=config, wdtype=weights.wdtype)
    w = weights.struct()
    if out is None:
        out = torch.empty((T, d), dtype=torch.int16, device=logits.device)
    r = Routing()
    if keep:
        for name in keep:
            setattr(r, name, _ptr(keep[name]))
    _check(lib().moe_layer_noalloc(ctypes.byref(p), _ptr(logits), _ptr(x), ctypes.byref(w),
                                   _ptr(out), ctypes.byref(r), _stream()), "moe_layer_noalloc")
    return out
