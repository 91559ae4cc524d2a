"""GPU parity at the full workload sizes, in the launch configuration bench.py times (automatic tile
selection, one moe_layer call).  Routing ids, counts, offsets and both permutations are compared
with the oracle in full, bit for bit, and topk_w within 2e-6.  Outputs are compared with the oracle
within 2e-2 * max|ref| (bf16 and MXFP4 weights) or 6e-2 * max|ref| (fp8):
  * the Mixtral-shaped prefill layer, every DeepSeek-V3-shaped decode point, both fp8 points and
    every MXFP4 point: every token, against the whole-layer oracle (points that share one set of
    expert weights are computed together, each expert's weights decoded once);
  * the Kimi-K2-shaped prefill layer (8192 tokens, about 330 active experts): 256 random tokens
    plus, for each of the 16 heaviest experts, the owners of the first, the last and a random row
    of every 256-row m-tile of its segment (full tiles, the short tail tiles that the chunked and
    longest-first orders make segments of their own, split pieces), each computed token by token.
Properties that hold at any size are checked on the whole output: a second call gives identical
bits and every value is finite."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from mixture_experts_layer_top_amd import inputs as I
from oracle import moe_oracle as O

from helpers import BF16_TOL, FP8_TOL, Inputs, act_of, bits_to_f64, rel_err, tol_of

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

ROUTING = ("topk_ids", "topk_w", "counts", "offsets", "perm_src", "slot_dst")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_top_amd import moe as m
    m.lib()
    return m


def _run(moe, inp, config=-1):
    """One layer call keeping every routing output, and a second call that must give the same
    bits."""
    p = inp.p
    L = moe.Layer(inp.expert_weights(), p.T, p.E, p.k, config=config)
    keep = dict(topk_ids=torch.empty((p.T, p.k), dtype=torch.int32, device="cuda"),
                topk_w=torch.empty((p.T, p.k), dtype=torch.float32, device="cuda"),
                counts=torch.empty(p.E, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(p.E + 1, dtype=torch.int32, device="cuda"),
                perm_src=torch.empty(p.T * p.k, dtype=torch.int32, device="cuda"),
                slot_dst=torch.empty(p.T * p.k, dtype=torch.int32, device="cuda"))
    out = L(inp.d_logits, inp.d_x, keep).clone()
    again = L(inp.d_logits, inp.d_x).clone()
    torch.cuda.synchronize()
    assert torch.equal(out, again)  # deterministic
    got = bits_to_f64(out)
    assert np.isfinite(got).all()
    return got, {n: keep[n].cpu().numpy() for n in ROUTING}


def _check_routing(p, keep, ids, w, counts, offsets, perm_src, slot_dst):
    assert np.array_equal(keep["topk_ids"], ids)
    assert np.abs(keep["topk_w"] - w).max() <= 2e-6
    assert np.array_equal(keep["counts"], counts)
    assert int(counts.sum()) == p.T * p.k
    assert np.array_equal(keep["offsets"], offsets)
    assert np.array_equal(keep["perm_src"], perm_src)
    assert np.array_equal(keep["slot_dst"], slot_dst)


def _check_whole(moe, inp, ref, tol, config=-1):
    """Every routing output and every output value against a whole-layer oracle result."""
    got, keep = _run(moe, inp, config)
    _check_routing(inp.p, keep, ref["ids"], ref["w"], ref["counts"], ref["offsets"],
                   ref["perm_src"], ref["slot_dst"])
    err = rel_err(got, ref["out"])
    assert err <= tol, err
    return err


def _oracle_points(inps):
    """Whole-layer oracle results of several workload points that share one set of weights."""
    first = inps[0]
    return O.moe_layers([(i.logits, i.x) for i in inps], first.p.k, first.get,
                        first.get_shared(), act=act_of(first.p))


# ------------------------------------------------------------------------------------------------
# Mixtral-shaped prefill: the whole output
# ------------------------------------------------------------------------------------------------

def test_mixtral_prefill_full(moe):
    inp = Inputs(I.MIXTRAL)
    ref = O.moe_layer(inp.logits, inp.x, inp.p.k, inp.get)
    _check_whole(moe, inp, ref, BF16_TOL)


# ------------------------------------------------------------------------------------------------
# DeepSeek-V3-shaped decode: all 12 points, every token
# ------------------------------------------------------------------------------------------------

DSV3_POINTS = [I.dsv3_point(T, a) for T in I.DSV3_TS for a in I.DSV3_ALPHAS]


@pytest.fixture(scope="module")
def dsv3(moe):
    W = I.gen_weights(I.DSV3, "cuda")
    inps = [Inputs(p, weights=W) for p in DSV3_POINTS]
    refs = _oracle_points(inps)
    return {i.p.name: (i, r) for i, r in zip(inps, refs)}


@pytest.mark.parametrize("p", DSV3_POINTS, ids=lambda p: p.name)
def test_dsv3_decode_full(moe, dsv3, p):
    inp, ref = dsv3[p.name]
    _check_whole(moe, inp, ref, BF16_TOL)


# the single-token points through the one-launch layer (MOE_CONFIG_FUSED)
@pytest.mark.parametrize("p", [p for p in DSV3_POINTS if p.T == 1], ids=lambda p: p.name)
def test_dsv3_decode_fused_full(moe, dsv3, p):
    inp, ref = dsv3[p.name]
    _check_whole(moe, inp, ref, BF16_TOL, config=moe.CONFIG_FUSED)


# ------------------------------------------------------------------------------------------------
# block-scaled fp8 with the shared expert: both points, every token
# ------------------------------------------------------------------------------------------------

FP8_POINTS = [I.fp8_point(T) for T in I.FP8_TS]


@pytest.fixture(scope="module")
def fp8(moe):
    first = Inputs(FP8_POINTS[0])
    inps = [first] + [Inputs(p, weights=first.W) for p in FP8_POINTS[1:]]
    refs = _oracle_points(inps)
    return {i.p.name: (i, r) for i, r in zip(inps, refs)}


@pytest.mark.parametrize("p", FP8_POINTS, ids=lambda p: p.name)
def test_fp8_decode_full(moe, fp8, p):
    inp, ref = fp8[p.name]
    got, keep = _run(moe, inp)
    _check_routing(p, keep, ref["ids"], ref["w"], ref["counts"], ref["offsets"], ref["perm_src"],
                   ref["slot_dst"])
    assert rel_err(got, ref["out"]) <= FP8_TOL


# ------------------------------------------------------------------------------------------------
# MXFP4 routed experts (bf16 activations): T = 1, 16, 64, 256, every token
# ------------------------------------------------------------------------------------------------

MXFP4_POINTS = [replace(I.MXFP4, T=T, name=f"{I.MXFP4.name}_T{T}") for T in I.DSV3_TS]


@pytest.fixture(scope="module")
def mxfp4(moe):
    first = Inputs(MXFP4_POINTS[0])
    inps = [first] + [Inputs(p, weights=first.W) for p in MXFP4_POINTS[1:]]
    refs = _oracle_points(inps)
    return {i.p.name: (i, r) for i, r in zip(inps, refs)}


@pytest.mark.parametrize("p", MXFP4_POINTS, ids=lambda p: p.name)
def test_mxfp4_decode_full(moe, mxfp4, p):
    inp, ref = mxfp4[p.name]
    _check_whole(moe, inp, ref, BF16_TOL)


# ------------------------------------------------------------------------------------------------
# MXFP4 experts with MXFP8 activations (scaled f8f6f4 MFMA): T = 1, 16, 64, 256, every token
# ------------------------------------------------------------------------------------------------

MXA8_POINTS = [replace(I.MXFP4_A8, T=T, name=f"{I.MXFP4_A8.name}_T{T}") for T in I.DSV3_TS]


@pytest.fixture(scope="module")
def mxa8(moe, mxfp4):
    W = next(iter(mxfp4.values()))[0].W  # the same weights as the W4A16 points
    inps = [Inputs(p, weights=W) for p in MXA8_POINTS]
    refs = _oracle_points(inps)
    return {i.p.name: (i, r) for i, r in zip(inps, refs)}


@pytest.mark.parametrize("p", MXA8_POINTS, ids=lambda p: p.name)
def test_mxfp4_a8_decode_full(moe, mxa8, p):
    inp, ref = mxa8[p.name]
    _check_whole(moe, inp, ref, tol_of(p))


# ------------------------------------------------------------------------------------------------
# Kimi-K2-shaped prefill: routing in full, outputs on a dense sample
# ------------------------------------------------------------------------------------------------

def _kimi_tokens(counts, offsets, perm_src, k, T, seed=0):
    rng = np.random.default_rng(seed)
    tok = set(rng.choice(T, 256, replace=False).tolist()) | {0, T - 1}
    for e in np.argsort(-counts, kind="stable")[:16]:
        c, r0 = int(counts[e]), int(offsets[e])
        for m0 in range(0, c, 256):
            m1 = min(c, m0 + 256)
            for r in {m0, m1 - 1, int(rng.integers(m0, m1))}:
                tok.add(int(perm_src[r0 + r]) // k)
    return np.array(sorted(tok))


def test_kimi_prefill_full(moe):
    inp = Inputs(I.KIMI)
    p = inp.p
    ids, w = O.route(inp.logits, p.k)
    counts, offsets = O.histogram(ids, p.E)
    perm_src, slot_dst = O.permute(ids, p.E)
    got, keep = _run(moe, inp)
    _check_routing(p, keep, ids, w, counts, offsets, perm_src, slot_dst)
    tok = _kimi_tokens(counts, offsets, perm_src, p.k, p.T)
    assert tok.size >= 256 + 16
    ref = O.moe_tokens(tok, inp.logits, inp.x, p.k, inp.get)["out"]
    err = rel_err(got[tok], ref)
    assert err <= BF16_TOL, err
    del inp
    torch.cuda.empty_cache()
