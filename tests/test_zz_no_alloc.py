"""GPU: moe_layer_noalloc -- the layer on the library's static per-GPU scratch, for callers that
cannot allocate -- against moe_layer with a caller workspace, through the C ABI.  Two calls in a
row, the second with a smaller input, so the second runs on scratch that still holds the first
call's contents: each must give moe_layer's output and routing outputs bit for bit (the same
kernels run), and the small cases also lie within the oracle's tolerance."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from mixture_experts_layer_top_amd import inputs as I
from oracle import moe_oracle as O

from helpers import BF16_TOL, FP8_TOL, Inputs, bits_to_f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_top_amd import moe as m
    m.lib()
    return m


ROUTING = ("topk_ids", "topk_w", "counts", "offsets", "perm_src", "slot_dst")


def _keep(p):
    return dict(topk_ids=torch.empty((p.T, p.k), dtype=torch.int32, device="cuda"),
                topk_w=torch.empty((p.T, p.k), dtype=torch.float32, device="cuda"),
                counts=torch.empty(p.E, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(p.E + 1, dtype=torch.int32, device="cuda"),
                perm_src=torch.empty(p.T * p.k, dtype=torch.int32, device="cuda"),
                slot_dst=torch.empty(p.T * p.k, dtype=torch.int32, device="cuda"))


def _both(moe, inp):
    """moe_layer_noalloc, then moe_layer with its own workspace, on the same inputs."""
    p = inp.p
    ew = inp.expert_weights()
    k_na, k_ws = _keep(p), _keep(p)
    out_na = moe.layer_noalloc(inp.d_logits, inp.d_x, ew, p.k, keep=k_na)
    torch.cuda.synchronize()
    out_na = out_na.clone()
    out_ws = moe.Layer(ew, p.T, p.E, p.k)(inp.d_logits, inp.d_x, k_ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws)
    for n in ROUTING:
        assert torch.equal(k_na[n], k_ws[n]), n
    return out_na


def _oracle_ok(inp, out, tol):
    p = inp.p
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get, inp.get_shared(),
                      act_fp8=p.wdtype == I.WDT_FP8)["out"]
    assert rel_err(bits_to_f64(out), ref) <= tol


SMALL_BF16 = I.Problem("na_bf16", 180, T=300, d=1024, f=512, E=64, k=8, routing="dirichlet",
                       alpha=0.3)
SMALL_FP8 = I.Problem("na_fp8", 181, T=96, d=512, f=256, E=32, k=4, routing="dirichlet", alpha=1.0,
                      wdtype=I.WDT_FP8, shared=True, shared_f=256)


@pytest.mark.parametrize("p, T2", [(SMALL_BF16, 7), (SMALL_BF16, 1), (SMALL_FP8, 5)],
                         ids=["bf16_300_then_7", "bf16_300_then_1", "fp8_96_then_5"])
def test_noalloc_matches_layer_two_calls(moe, p, T2):
    tol = FP8_TOL if p.wdtype == I.WDT_FP8 else BF16_TOL
    first = Inputs(p)
    out1 = _both(moe, first)
    _oracle_ok(first, out1, tol)
    second = Inputs(replace(p, T=T2, name=f"{p.name}_T{T2}"), weights=first.W)
    out2 = _both(moe, second)
    _oracle_ok(second, out2, tol)


def test_noalloc_full_decode_shape(moe):
    """DeepSeek-V3-shaped bf16 decode at T = 256 (about 100 MiB of the 128 MiB scratch), then
    the single-token path on the same scratch."""
    W = I.gen_weights(I.DSV3, "cuda")
    _both(moe, Inputs(I.dsv3_point(256, 1.0), weights=W))
    _both(moe, Inputs(I.dsv3_point(1, 1.0), weights=W))


def test_noalloc_rejects_large_problem(moe):
    inp = Inputs(replace(SMALL_BF16, T=4096, d=4096, f=2048, name="na_big"))
    with pytest.raises(moe.MoEError, match="WORKSPACE"):
        moe.layer_noalloc(inp.d_logits, inp.d_x, inp.expert_weights(), inp.p.k)
