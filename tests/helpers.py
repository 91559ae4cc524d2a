"""Shared test plumbing: input upload, oracle weight access, comparisons."""
from __future__ import annotations

import numpy as np
import torch

from mixture_experts_layer_top_amd import inputs as I

BF16_TOL = 2e-2
FP8_TOL = 6e-2


def act_of(p) -> str:
    """The oracle's activation format for a workload."""
    return "fp8" if p.wdtype == I.WDT_FP8 else "mxfp8" if p.act_mx8 else "bf16"


def tol_of(p) -> float:
    """8-bit activations (fp8, MXFP8) take the fp8 bar, bf16 activations the bf16 one."""
    return FP8_TOL if act_of(p) != "bf16" else BF16_TOL


def bits_to_f64(t) -> np.ndarray:
    """bf16 bit patterns (int16 tensor / uint16 array) -> float64 (test-side decode)."""
    a = t.cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Inputs:
    """One workload's inputs: numpy copies for the oracle, device tensors for the library."""

    def __init__(self, p: I.Problem, device="cuda", weights=None):
        self.p = p
        self.logits = I.gen_logits(p)
        self.x = I.gen_x(p)
        self.W = weights if weights is not None else I.gen_weights(p, device)
        self.d_logits = torch.from_numpy(self.logits).to(device)
        self.d_x = torch.from_numpy(self.x.view(np.int16)).to(device)
        self._cache = {}

    def expert_weights(self):
        from mixture_experts_layer_top_amd.moe import ExpertWeights
        W = self.W
        kw = dict(gate=W["gate"], up=W["up"], down=W["down"])
        if self.p.wdtype == I.WDT_FP8:
            # the library reads its tiled layout; the oracle keeps the generator's row-major bytes
            from mixture_experts_layer_top_amd.moe import fp8_tile
            if getattr(self, "_tiled", None) is None:
                names = ("gate", "up", "down") + (("sh_gate", "sh_up", "sh_down") if self.p.shared else ())
                self._tiled = {n: fp8_tile(W[n]) for n in names}
            kw.update({n: self._tiled[n] for n in ("gate", "up", "down")})
            kw.update(s_gate=W["s_gate"], s_up=W["s_up"], s_down=W["s_down"])
        if self.p.wdtype == I.WDT_MXFP4:
            # the library reads its tiled layout; the oracle keeps the generator's row-major bytes
            from mixture_experts_layer_top_amd.moe import mxfp4_tile
            if getattr(self, "_tiled", None) is None:
                self._tiled = {n: mxfp4_tile(W[n]) for n in ("gate", "up", "down")}
            kw.update(self._tiled)
            kw.update(e_gate=W["s_gate"], e_up=W["s_up"], e_down=W["s_down"], act_mx8=self.p.act_mx8)
        if self.p.shared:
            kw.update(sh_gate=W["sh_gate"], sh_up=W["sh_up"], sh_down=W["sh_down"])
            if self.p.wdtype == I.WDT_FP8:
                kw.update({n: self._tiled[n] for n in ("sh_gate", "sh_up", "sh_down")})
                kw.update(s_sh_gate=W["s_sh_gate"], s_sh_up=W["s_sh_up"], s_sh_down=W["s_sh_down"])
        return ExpertWeights(**kw)

    # The oracle reads the generator's weight bytes.  On a GPU machine they were generated there by the
    # same device-independent generator (tests check CPU == GPU generation bit for bit), and are
    # copied back per expert; no HIP-library output is involved.
    def get(self, e):
        if e not in self._cache:
            r = {n: self.W[n][e].cpu().numpy() for n in ("gate", "up", "down")}
            if self.p.wdtype in (I.WDT_FP8, I.WDT_MXFP4):
                r.update({"s_" + n: self.W["s_" + n][e].cpu().numpy() for n in ("gate", "up", "down")})
            if len(self._cache) > 24:
                self._cache.clear()
            self._cache[e] = r
        return self._cache[e]

    def get_shared(self):
        """The shared expert's stored weights for the oracle, as a getter (None without one)."""
        if not self.p.shared:
            return None
        r = {n: self.W["sh_" + n].cpu().numpy() for n in ("gate", "up", "down")}
        if self.p.wdtype == I.WDT_FP8:
            r.update({"s_" + n: self.W["s_sh_" + n].cpu().numpy() for n in ("gate", "up", "down")})
        return lambda: r


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    m = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (m if m > 0 else 1.0))
