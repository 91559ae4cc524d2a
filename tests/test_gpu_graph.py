"""GPU: the whole layer captured in a HIP graph (torch.cuda.graph over the library's launches on the
capture stream) and replayed.  The library allocates, clears and synchronises nothing on the host
side, so every launch of moe_layer is capturable; its counters and queues are cleared by its own
kernels.  Each replay must give the eager call's output bit for bit and lie within the tolerance
of the oracle's output (2e-2 * max|ref|, 6e-2 for fp8 weights), with eager work of other layers
between the replays; new inputs copied into the captured buffers must give the eager result for
those inputs, again within the tolerance of the oracle's output for them."""
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


def _p(name, cfg_index, **kw):
    base = dict(T=64, d=256, f=512, E=8, k=2)
    base.update(kw)
    return I.Problem(name, cfg_index, **base)


GRAPH_CASES = [
    # single token: routing inside the gate/up kernel, then the streaming down GEMM
    _p("graph_T1", 170, T=1, d=1024, f=512, E=64, k=8, routing="dirichlet", alpha=1.0),
    # decode front end (route + permute + select in one launch), light MFMA and streaming tiles
    _p("graph_T16", 171, T=16, d=512, f=512, E=32, k=4, routing="dirichlet", alpha=1.0),
    # separate route / permute / select launches, MFMA tiles of several heights
    _p("graph_T300", 172, T=300, d=384, f=640, E=6, k=2),
    # last-round split in K (counters and partial-sum slots cleared by the selection kernel)
    _p("graph_split", 173, T=1100, d=512, f=1024, E=1, k=1),
    # block-scaled fp8 experts with the shared expert and activation quantisation
    _p("graph_fp8", 174, T=32, d=512, f=256, E=16, k=4, routing="dirichlet", alpha=1.0,
       wdtype=I.WDT_FP8, shared=True, shared_f=256),
]


def _layer(moe, inp):
    return moe.Layer(inp.expert_weights(), inp.p.T, inp.p.E, inp.p.k)


def _oracle_out(inp):
    p = inp.p
    return O.moe_layer(inp.logits, inp.x, p.k, inp.get, inp.get_shared(),
                       act_fp8=p.wdtype == I.WDT_FP8)["out"]


@pytest.mark.parametrize("p", GRAPH_CASES, ids=lambda p: p.name)
def test_layer_graph_replay(moe, p):
    tol = FP8_TOL if p.wdtype == I.WDT_FP8 else BF16_TOL
    inp = Inputs(p)
    ref = _oracle_out(inp)
    L = _layer(moe, inp)
    eager = L(inp.d_logits, inp.d_x).clone()
    torch.cuda.synchronize()
    assert rel_err(bits_to_f64(eager), ref) <= tol

    static_logits = inp.d_logits.clone()
    static_x = inp.d_x.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L(static_logits, static_x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = L(static_logits, static_x)
    torch.cuda.synchronize()

    # eager work of another layer (own workspace) between the replays
    other = Inputs(replace(p, name=p.name + "_other", cfg_index=p.cfg_index + 50), weights=inp.W)
    L_other = _layer(moe, other)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        assert rel_err(bits_to_f64(out), ref) <= tol
        L_other(other.d_logits, other.d_x)
        torch.cuda.synchronize()

    # new inputs through the captured buffers
    static_logits.copy_(other.d_logits)
    static_x.copy_(other.d_x)
    g.replay()
    torch.cuda.synchronize()
    fresh = _layer(moe, other)(other.d_logits, other.d_x)
    torch.cuda.synchronize()
    assert torch.equal(out, fresh)
    assert not torch.equal(fresh, eager)
    assert rel_err(bits_to_f64(out), _oracle_out(other)) <= tol
