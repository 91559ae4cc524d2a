"""GPU parity: the HIP library (through its C ABI) against the CPU fp64 oracle on the same seeded
inputs.  Routing, counts, offsets and permutations must match bit for bit; topk_w within 2e-6;
outputs within 2e-2 * max|ref| (bf16 weights) or 6e-2 * max|ref| (fp8 weights)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from mixture_experts_layer_top_amd import inputs as I
from oracle import moe_oracle as O

from helpers import BF16_TOL, FP8_TOL, Inputs, act_of, bits_to_f64, rel_err, tol_of
from oracle import mxfp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_top_amd import moe as m
    m.lib()
    return m


def _small(name, **kw):
    base = dict(cfg_index=100, T=64, d=256, f=512, E=8, k=2)
    base.update(kw)
    return I.Problem(name, **base)


# ------------------------------------------------------------------------------------------------
# route
# ------------------------------------------------------------------------------------------------

ROUTE_CASES = [(64, 8, 2), (300, 1, 1), (257, 64, 8), (100, 65, 3), (64, 256, 8), (33, 384, 8),
               (17, 512, 8), (50, 8, 8), (4096, 8, 2)]


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
def test_route_random(moe, T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = moe.route(torch.from_numpy(L).cuda(), k)
    rids, rw = O.route(L, k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.abs(w.cpu().numpy() - rw).max() <= 2e-6


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (256, 8), (384, 8), (512, 5)])
def test_route_planted_ties(moe, E, k):
    rng = np.random.default_rng(E)
    L = rng.integers(-2, 3, size=(200, E)).astype(np.float32)
    L[::7] = 0.0
    L[1::7] = -0.0
    L[2::7, ::2] = -0.0
    ids, w = moe.route(torch.from_numpy(L).cuda(), k)
    rids, rw = O.route(L, k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.abs(w.cpu().numpy() - rw).max() <= 2e-6


@pytest.mark.parametrize("T,alpha", [(1, 0.1), (16, 1.0), (64, 10.0), (256, 0.1)])
def test_route_dirichlet_workloads(moe, T, alpha):
    p = I.dsv3_point(T, alpha)
    L = I.gen_logits(p)
    ids, w = moe.route(torch.from_numpy(L).cuda(), p.k)
    rids, rw = O.route(L, p.k)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.abs(w.cpu().numpy() - rw).max() <= 2e-6


# ------------------------------------------------------------------------------------------------
# permute
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (64, 8, 2), (1000, 16, 4), (2048, 256, 8),
                                   (8192, 384, 8), (3, 512, 8), (700, 1, 1)])
def test_permute_bit_exact(moe, T, E, k):
    rng = np.random.default_rng(T + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:, :3] += 2.0  # skew: some experts heavy, several tails
    rids, _ = O.route(L, k)
    x = rng.integers(-30000, 30000, size=(T, 128)).astype(np.int16)
    counts, offsets, perm_src, slot_dst, xp, _ = moe.permute(
        torch.from_numpy(rids).cuda(), E, torch.from_numpy(x).cuda())
    rc, ro = O.histogram(rids, E)
    rps, rsd = O.permute(rids, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm_src.cpu().numpy(), rps)
    assert np.array_equal(slot_dst.cpu().numpy(), rsd)
    assert np.array_equal(xp.cpu().numpy(), x[rps // k])


# ------------------------------------------------------------------------------------------------
# combine and grouped FFN, each fed with the oracle's own intermediates
# ------------------------------------------------------------------------------------------------

# d / 8 threads per token row: 48 (one 256-thread workgroup with idle lanes), 64 and 192
# (64-thread workgroups), 256 (256), 896 (seven of 128, the Kimi-K2 and DeepSeek-V3 width)
@pytest.mark.parametrize("T,E,k,d", [(77, 16, 4, 384), (33, 8, 2, 512), (50, 12, 3, 1536),
                                     (19, 16, 8, 2048), (41, 64, 8, 7168)])
def test_combine_matches_oracle(moe, T, E, k, d):
    rng = np.random.default_rng(3 + d)
    L = rng.standard_normal((T, E)).astype(np.float32)
    rids, rw = O.route(L, k)
    _, rsd = O.permute(rids, E)
    y = I.f32_to_bf16_bits(rng.standard_normal((T * k, d)).astype(np.float32))
    sh = I.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w32 = rw.astype(np.float32)
    for shared in (None, sh):
        out = moe.combine(torch.from_numpy(y.view(np.int16)).cuda(),
                          torch.from_numpy(rsd.astype(np.int32)).cuda(),
                          torch.from_numpy(w32).cuda(),
                          None if shared is None else torch.from_numpy(shared.view(np.int16)).cuda())
        S = None if shared is None else bits_to_f64(shared)
        ref = O.combine(bits_to_f64(y), rsd, w32.astype(np.float64), S)
        got = bits_to_f64(out)
        # one bf16 rounding of an fp32 sum: within 2^-8 relative (plus fp32 summation noise)
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


GFFN = [
    _small("gffn_tiny"),
    _small("gffn_ragged", T=300, d=384, f=640, E=6, k=2, cfg_index=101),
    _small("gffn_one", T=5, d=128, f=128, E=3, k=1, cfg_index=102),
    _small("gffn_skew", T=200, d=256, f=256, E=40, k=4, routing="dirichlet", alpha=0.1, cfg_index=103),
]


@pytest.mark.parametrize("config", [-1, 0, 1])
@pytest.mark.parametrize("p", GFFN, ids=lambda p: p.name)
def test_grouped_ffn_matches_oracle(moe, p, config):
    inp = Inputs(p)
    rids, _ = O.route(inp.logits, p.k)
    counts, offsets = O.histogram(rids, p.E)
    perm_src, _ = O.permute(rids, p.E)
    x_perm = inp.x[perm_src // p.k]
    y = moe.grouped_ffn(torch.from_numpy(x_perm.view(np.int16)).cuda(), None,
                        torch.from_numpy(counts.astype(np.int32)).cuda(),
                        torch.from_numpy(offsets.astype(np.int32)).cuda(),
                        inp.expert_weights(), p.T, p.k, config=config)
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get)["y_perm"]
    got = bits_to_f64(y)
    assert rel_err(got, ref) <= BF16_TOL


# ------------------------------------------------------------------------------------------------
# the whole layer
# ------------------------------------------------------------------------------------------------

LAYER = [
    I.TINY,
    _small("layer_ragged", T=300, d=384, f=640, E=6, k=2, cfg_index=104),
    _small("layer_e1k1", T=40, d=256, f=384, E=1, k=1, cfg_index=105),
    _small("layer_skew", T=333, d=256, f=512, E=48, k=6, routing="dirichlet", alpha=0.1, cfg_index=106),
    _small("layer_T1", T=1, d=512, f=256, E=16, k=4, routing="dirichlet", alpha=1.0, cfg_index=107),
    _small("layer_big_expert", T=700, d=128, f=256, E=4, k=1, routing="dirichlet", alpha=0.1,
           cfg_index=108),
    # long-K down GEMMs (d_ff = 4096) whose experts end in a short MFMA tile of 64 rows (320 rows),
    # of 65 rows -> a 128-row tile (321), and two experts with different tails (560 over 2)
    _small("layer_down_tail64", T=320, d=128, f=4096, E=1, k=1, cfg_index=113),
    _small("layer_down_tail65", T=321, d=128, f=4096, E=1, k=1, cfg_index=114),
    _small("layer_down_tail2e", T=560, d=128, f=4096, E=2, k=1, cfg_index=115),
    # down GEMM of 8 column tiles per expert with light (<= 8 rows) and heavier experts: 43 light
    # experts beside heavier ones worth 392 down tiles, so on 256 CUs the light ones join the MFMA
    # list; with 240 heavy tiles (below one round) they stay on the streaming tiles and the GEMM
    # runs both launches
    _small("layer_down_promote", T=300, d=2048, f=256, E=96, k=4, routing="dirichlet", alpha=1.0,
           cfg_index=116),
    _small("layer_down_split", T=160, d=2048, f=256, E=64, k=4, routing="dirichlet", alpha=1.0,
           cfg_index=116),
]


def _check_layer(moe, inp, config=-1, tol=BF16_TOL, runs=1):
    p = inp.p
    out, keep = moe.layer(inp.d_logits, inp.d_x, inp.expert_weights(), p.k, config=config,
                          keep_routing=True)
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get, inp.get_shared(), act=act_of(p))
    assert np.array_equal(keep["topk_ids"].cpu().numpy(), ref["ids"])
    assert np.abs(keep["topk_w"].cpu().numpy() - ref["w"]).max() <= 2e-6
    assert np.array_equal(keep["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(keep["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(keep["perm_src"].cpu().numpy(), ref["perm_src"])
    assert np.array_equal(keep["slot_dst"].cpu().numpy(), ref["slot_dst"])
    err = rel_err(bits_to_f64(out), ref["out"])
    assert err <= tol, err
    first = out.clone()
    for _ in range(runs - 1):
        again = moe.layer(inp.d_logits, inp.d_x, inp.expert_weights(), p.k, config=config)
        assert torch.equal(again, first)  # bitwise deterministic
    return err


@pytest.mark.parametrize("config", [-1, 0, 1])
@pytest.mark.parametrize("p", LAYER, ids=lambda p: p.name)
def test_layer_matches_oracle(moe, p, config):
    _check_layer(moe, Inputs(p), config=config, runs=2)


# One token (bf16, no shared expert, d <= 8192): every workgroup of the gate/up kernel routes the
# token itself and takes its tiles' experts from that; its first workgroup also writes the routing
# outputs and the down GEMM's segments.  Cases: each width of the routing's per-lane candidates
# (E <= 64, 128, 256, 512), both streaming tile widths (d below 4096: 32 columns, else 16), more
# tiles than workgroups (f = 4096, k = 8: 2048 gate/up tiles of 16 columns), f above 8192, and d
# above the staging limit (the general path).  The down GEMM runs on the segments the gate/up
# kernel wrote.
DECODE1 = [
    _small("decode1_E64_k1", T=1, d=256, f=256, E=64, k=1, cfg_index=160),
    _small("decode1_E128", T=1, d=1024, f=512, E=128, k=6, routing="dirichlet", alpha=0.3,
           cfg_index=161),
    _small("decode1_E256", T=1, d=4096, f=384, E=256, k=8, routing="dirichlet", alpha=1.0,
           cfg_index=162),
    _small("decode1_E512", T=1, d=512, f=384, E=512, k=8, cfg_index=163),
    _small("decode1_many_tiles", T=1, d=4096, f=4096, E=8, k=8, cfg_index=164),
    _small("decode1_wide_d", T=1, d=8320, f=256, E=8, k=2, cfg_index=165),
    _small("decode1_wide_f", T=1, d=256, f=8320, E=4, k=2, cfg_index=167),
]


@pytest.mark.parametrize("config", [-1, 0])
@pytest.mark.parametrize("p", DECODE1, ids=lambda p: p.name)
def test_decode1_matches_oracle(moe, p, config):
    _check_layer(moe, Inputs(p), config=config, runs=2)


# The whole single-token layer in one launch (config FUSED): every single-token shape whose d and f
# stay within 8192 (so both tile widths of each GEMM, every routing width, more tiles than
# workgroups), against the oracle; then three calls on one Layer: the device counters that order
# the launch's phases must return to zero after each call (the same bits every time, the counter
# block zero afterwards, the error flag clear), and the result must equal the multi-launch path's
# bits (the same tiles in the same order, read through LDS and coherent loads).
FUSED = [p for p in DECODE1 if p.d <= 8192 and p.f <= 8192]


@pytest.mark.parametrize("p", FUSED, ids=lambda p: p.name)
def test_fused_decode_matches_oracle(moe, p):
    inp = Inputs(p)
    _check_layer(moe, inp, config=moe.CONFIG_FUSED)
    L = moe.Layer(inp.expert_weights(), 1, p.E, p.k, config=moe.CONFIG_FUSED)
    outs = []
    for _ in range(3):
        outs.append(L(inp.d_logits, inp.d_x).clone())
        torch.cuda.synchronize()
        sync = L.ws[:moe.FUSED_SYNC_BYTES].view(torch.int32).cpu().numpy()
        assert not sync.any(), np.flatnonzero(sync)[:8]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    multi = moe.layer(inp.d_logits, inp.d_x, inp.expert_weights(), p.k, config=-1)
    assert torch.equal(multi, outs[0])


def test_fused_ties(moe):
    inp = Inputs(_small("fused_ties", T=1, d=256, f=256, E=256, k=8, cfg_index=168))
    rng = np.random.default_rng(7)
    L = rng.integers(-1, 2, size=(1, 256)).astype(np.float32)
    L[0, ::5] = -0.0
    L[0, 1::5] = 0.0
    inp.logits = L
    inp.d_logits = torch.from_numpy(L).cuda()
    _check_layer(moe, inp, config=moe.CONFIG_FUSED)


# Ties inside the single-token routing: equal logits (and +0.0 / -0.0) go to the lower expert id.
@pytest.mark.parametrize("E,k", [(64, 8), (256, 8), (512, 3)])
def test_decode1_ties(moe, E, k):
    inp = Inputs(_small(f"decode1_ties_E{E}", T=1, d=256, f=256, E=E, k=k, cfg_index=166))
    rng = np.random.default_rng(E + k)
    L = rng.integers(-1, 2, size=(1, E)).astype(np.float32)
    L[0, ::5] = -0.0
    L[0, 1::5] = 0.0
    inp.logits = L
    inp.d_logits = torch.from_numpy(L).cuda()
    _check_layer(moe, inp, config=-1)


# MFMA tiles take a height of 64, 128 or 256 token rows from the rows they hold; one expert whose
# row count sits at each boundary, with K of 2 K-steps (the three-stage ring of the short tiles
# then reloads its last step) and of 6.
TILE_HEIGHTS = [
    _small(f"heights_T{T}_d{d}", T=T, d=d, f=f, E=1, k=1, cfg_index=120 + i)
    for i, (T, d, f) in enumerate(
        [(T, 128, 384) for T in (1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 320, 385)]
        + [(T, 384, 128) for T in (40, 100, 300)])
]


@pytest.mark.parametrize("p", TILE_HEIGHTS, ids=lambda p: p.name)
def test_mfma_tile_heights(moe, p):
    _check_layer(moe, Inputs(p), config=1)


# More tiles than workgroups, so one persistent workgroup runs tiles of different heights in turn.
def test_mfma_mixed_heights_persistent(moe):
    p = _small("heights_mixed", T=2000, d=256, f=2048, E=8, k=2, routing="dirichlet", alpha=1.0,
               cfg_index=140)
    for config in (1, -1):
        _check_layer(moe, Inputs(p), config=config, runs=2)


# Last-round split in K: tiles past the last whole round of CUs run as 2 or 4 K-pieces whose fp32
# partial sums an epilogue kernel adds in piece order.  1100 rows = 4 full m-tiles + a 128-row
# short one; 1050 rows = 4 full m-tiles + a 32-row one.  f = 1024: 40 gate/up and 10 down tiles,
# all split 4 ways; f = 8192: 320 gate/up tiles, one whole round + 64 tiles split 4 ways (256
# pieces).  Runs must agree bit for bit.
@pytest.mark.parametrize("T,f", [(1100, 1024), (1100, 8192), (1050, 1024), (1050, 8192)])
def test_mfma_last_round_split(moe, T, f):
    cfg = 141 + (f > 1024) if T == 1100 else 143 + (f > 1024)
    p = _small(f"split_T{T}_f{f}", T=T, d=512, f=f, E=1, k=1, cfg_index=cfg)
    for config in (1, -1):
        _check_layer(moe, Inputs(p), config=config, runs=3)


# Tile orders at a size the oracle still checks in full: the long-K gate/up GEMM (d = 4096, 848
# tiles on 256 CUs) takes the two-class order, with two heavy experts whose short last m-tiles
# become segments of their own, 46 light experts and full-height single tiles; the down GEMM
# (K = 2048) takes the mixed order.  (Routing draw: Dirichlet(0.3) over 64 experts, seed 150.)
def test_mfma_order_modes(moe):
    p = I.Problem("order_modes", 150, T=1000, d=4096, f=2048, E=64, k=2, routing="dirichlet",
                  alpha=0.3)
    _check_layer(moe, Inputs(p), config=-1, runs=2)


def _planted_inputs(p, counts):
    """Inputs whose routing gives exactly `counts` rows per expert (each count <= T): the T*k
    slots are dealt in expert order, token t taking the experts at positions t, t + T, ..., which
    are distinct, with logits far above every other expert's and strictly decreasing in j."""
    counts = np.asarray(counts)
    assert counts.sum() == p.T * p.k and counts.max() <= p.T
    deal = np.repeat(np.arange(p.E), counts).reshape(p.k, p.T)
    inp = Inputs(p)
    lg = (inp.logits - 20.0).astype(np.float32)
    for j in range(p.k):
        lg[np.arange(p.T), deal[j]] = np.float32(10.0 - 0.5 * j)
    inp.logits = lg
    inp.d_logits = torch.from_numpy(lg).to("cuda")
    return inp


# The two-class order at its edges (long-K gate/up lists of at least three rounds of 256 CUs):
# every tile full-height (16 experts of exactly three m-tiles, 768 tiles, no short class), and a
# short class that dwarfs the full one (one expert of two m-tiles against 47 of 64 rows: 32 full
# and 752 short tiles, so only two CUs of an XCD start on full tiles and the rest steal them).
@pytest.mark.parametrize("case", ["full_only", "few_full"])
def test_mfma_two_class_edges(moe, case):
    if case == "full_only":
        p = I.Problem("two_class_full", 151, T=6144, d=4096, f=2048, E=16, k=2)
        counts = [768] * 16
    else:
        p = I.Problem("two_class_few", 152, T=1760, d=4096, f=2048, E=64, k=2)
        counts = [512] + [64] * 47 + [0] * 16
    inp = _planted_inputs(p, counts)
    _check_layer(moe, inp, config=-1, runs=2)


def test_generator_device_independent(moe):
    for p, which, e in ((I.TINY, "gate", 3), (I.DSV3, "down", 200), (I.FP8, "up", 7),
                        (I.MXFP4, "gate", 11)):
        a = I.gen_expert_weight(p, which, e, "cpu")
        b = I.gen_expert_weight(p, which, e, "cuda").cpu()
        assert torch.equal(a, b)
    for p, which, e in ((I.FP8, "down", 5), (I.MXFP4, "down", 9)):
        a = I.gen_expert_scales(p, which, e, "cpu")
        b = I.gen_expert_scales(p, which, e, "cuda").cpu()
        assert torch.equal(a, b)


def test_t0_is_noop(moe):
    p = I.TINY
    W = Inputs(p).expert_weights()
    L = moe.Layer(W, 0, p.E, p.k)
    out = L(torch.empty((0, p.E), device="cuda"), torch.empty((0, p.d), dtype=torch.int16, device="cuda"))
    assert out.shape == (0, p.d)


# ------------------------------------------------------------------------------------------------
# fp8: activation quantisation (bit-exact) and the block-scaled layer
# ------------------------------------------------------------------------------------------------

def _all_bf16_below_448():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (b.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    return b[keep]


def test_quant_act_exhaustive_bf16(moe):
    """A 448 in every 128-block makes s = 1 exactly, so q must be the oracle's encoding of every
    finite bf16 value of magnitude <= 448 (all binades, subnormals, both zeros, every tie)."""
    vals = _all_bf16_below_448()
    per, d = 127, 1024
    nblk = (vals.size + per - 1) // per
    nblk += (-nblk) % (d // 128)  # whole rows of 8 blocks
    pad = np.full(nblk * per - vals.size, 0x3F80, np.uint16)  # 1.0
    body = np.concatenate([vals, pad]).reshape(nblk, per)
    blocks = np.concatenate([np.full((nblk, 1), 0x43E0, np.uint16), body], axis=1)  # 448.0 first
    x = blocks.reshape(-1, d)
    xq, xs = moe.quant_act(torch.from_numpy(x.view(np.int16)).cuda())
    rq, rs = O.quant_act_e4m3(x)
    assert np.array_equal(xs.cpu().numpy(), rs)
    assert np.all(rs == 1.0)
    assert np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("scale", [1.0, 1e-3, 37.0, 1e-30])
def test_quant_act_random(moe, scale):
    rng = np.random.default_rng(int(scale * 1000) + 1)
    x = (rng.standard_normal((37, 640)) * scale).astype(np.float32)
    x[3, 128:256] = 0.0
    x[5, :128] = -0.0
    x[7, 256:384] = rng.integers(-3, 4, 128)
    bits = I.f32_to_bf16_bits(x)
    xq, xs = moe.quant_act(torch.from_numpy(bits.view(np.int16)).cuda())
    rq, rs = O.quant_act_e4m3(bits)
    assert np.array_equal(xs.cpu().numpy(), rs)
    assert np.array_equal(xq.cpu().numpy(), rq)


FP8_SMALL = [
    I.Problem("fp8_tiny", 110, T=24, d=256, f=256, E=16, k=4, routing="dirichlet", alpha=1.0,
              wdtype=I.WDT_FP8, shared=True, shared_f=256),
    I.Problem("fp8_ragged", 111, T=150, d=384, f=512, E=12, k=3, routing="dirichlet", alpha=0.3,
              wdtype=I.WDT_FP8, shared=True, shared_f=384),
    I.Problem("fp8_noshared", 112, T=70, d=256, f=384, E=8, k=2, wdtype=I.WDT_FP8),
]


@pytest.mark.parametrize("p", FP8_SMALL, ids=lambda p: p.name)
def test_fp8_layer_matches_oracle(moe, p):
    _check_layer(moe, Inputs(p), tol=FP8_TOL, runs=2)


def test_fp8_grouped_ffn_matches_oracle(moe):
    p = FP8_SMALL[1]
    inp = Inputs(p)
    rids, _ = O.route(inp.logits, p.k)
    counts, offsets = O.histogram(rids, p.E)
    perm_src, _ = O.permute(rids, p.E)
    xq, xs = O.quant_act_e4m3(inp.x)
    y = moe.grouped_ffn(torch.from_numpy(xq[perm_src // p.k]).cuda(),
                        torch.from_numpy(xs[perm_src // p.k]).cuda(),
                        torch.from_numpy(counts.astype(np.int32)).cuda(),
                        torch.from_numpy(offsets.astype(np.int32)).cuda(),
                        inp.expert_weights(), p.T, p.k)
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get, None, act_fp8=True)["y_perm"]
    assert rel_err(bits_to_f64(y), ref) <= FP8_TOL


# fp8 experts on the LDS-staged MFMA tiles (256 token rows x 256 weight rows, one 128-wide K block
# per stage).  Forced (config 1) on every fp8 shape above plus: several 256-row m-tiles per expert
# with ragged tails and the shared expert's T rows (T = 600, k = 2, E = 4), an odd number of K
# blocks and a down tile whose second 128 columns lie past d (d = 384), five gate/up tiles
# (f = 640), and a longer K (d = 2048) under skewed routing.  Automatic selection puts experts of
# more than 128 rows on the MFMA tiles when a GEMM's MFMA tiles fill a round of CUs: on the
# prefill-shaped case the gate/up GEMM qualifies (512 tiles) and the down GEMM (128) streams.
FP8_MFMA = [
    I.Problem("fp8_mfma_ragged", 113, T=600, d=384, f=640, E=4, k=2, wdtype=I.WDT_FP8,
              shared=True, shared_f=384),
    I.Problem("fp8_mfma_long_k", 114, T=520, d=2048, f=256, E=8, k=2, routing="dirichlet",
              alpha=0.3, wdtype=I.WDT_FP8),
]
FP8_PREFILL = I.Problem("fp8_prefill", 115, T=4096, d=1024, f=2048, E=8, k=2, wdtype=I.WDT_FP8)


@pytest.mark.parametrize("p", FP8_SMALL + FP8_MFMA, ids=lambda p: p.name)
def test_fp8_mfma_layer_matches_oracle(moe, p):
    _check_layer(moe, Inputs(p), config=1, tol=FP8_TOL, runs=2)


def test_fp8_prefill_auto_matches_oracle(moe):
    _check_layer(moe, Inputs(FP8_PREFILL), config=-1, tol=FP8_TOL, runs=2)


def test_fp8_mfma_grouped_ffn_matches_oracle(moe):
    p = FP8_MFMA[0]
    inp = Inputs(p)
    rids, _ = O.route(inp.logits, p.k)
    counts, offsets = O.histogram(rids, p.E)
    perm_src, _ = O.permute(rids, p.E)
    xq, xs = O.quant_act_e4m3(inp.x)
    y = moe.grouped_ffn(torch.from_numpy(xq[perm_src // p.k]).cuda(),
                        torch.from_numpy(xs[perm_src // p.k]).cuda(),
                        torch.from_numpy(counts.astype(np.int32)).cuda(),
                        torch.from_numpy(offsets.astype(np.int32)).cuda(),
                        inp.expert_weights(), p.T, p.k, config=1)
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get, None, act_fp8=True)["y_perm"]
    assert rel_err(bits_to_f64(y), ref) <= FP8_TOL


# ------------------------------------------------------------------------------------------------
# MXFP4 experts (E2M1 pairs with E8M0 scales per 32; bf16 activations; streaming tiles only).  The
# tile converts the weights to bf16 exactly, so the bar is the bf16 one.  K-loop cases: K / WK / 32
# steps per wavefront against batches of 8 (one token group) or 4 steps: remainder only (d = 256,
# 384), whole batches plus a remainder (d = 384 at 4-step batches), an even (d = 4096) and an odd
# (d = 1536) number of pipelined batches; one token (the general path: the single-token kernel is
# bf16 only); three token-group widths (T = 64 and 300 reach passes of 33-64 rows).
# ------------------------------------------------------------------------------------------------

MXFP4_SMALL = [
    I.Problem("mx_tiny", 120, T=64, d=256, f=512, E=8, k=2, wdtype=I.WDT_MXFP4),
    I.Problem("mx_ragged", 121, T=300, d=384, f=640, E=6, k=2, wdtype=I.WDT_MXFP4),
    I.Problem("mx_long_k", 122, T=40, d=4096, f=1024, E=16, k=4, routing="dirichlet", alpha=1.0,
              wdtype=I.WDT_MXFP4),
    I.Problem("mx_odd_batches", 123, T=24, d=1536, f=256, E=8, k=2, wdtype=I.WDT_MXFP4),
    I.Problem("mx_T1", 124, T=1, d=1024, f=512, E=32, k=4, routing="dirichlet", alpha=1.0,
              wdtype=I.WDT_MXFP4),
]


@pytest.mark.parametrize("config", [-1, 0])
@pytest.mark.parametrize("p", MXFP4_SMALL, ids=lambda p: p.name)
def test_mxfp4_layer_matches_oracle(moe, p, config):
    _check_layer(moe, Inputs(p), config=config, tol=BF16_TOL, runs=2)


def test_mxfp4_grouped_ffn_matches_oracle(moe):
    p = MXFP4_SMALL[2]
    inp = Inputs(p)
    rids, _ = O.route(inp.logits, p.k)
    counts, offsets = O.histogram(rids, p.E)
    perm_src, _ = O.permute(rids, p.E)
    x_perm = torch.from_numpy(np.ascontiguousarray(inp.x[perm_src // p.k]).view(np.int16)).cuda()
    y = moe.grouped_ffn(x_perm, None, torch.from_numpy(counts.astype(np.int32)).cuda(),
                        torch.from_numpy(offsets.astype(np.int32)).cuda(),
                        inp.expert_weights(), p.T, p.k)
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get)["y_perm"]
    assert rel_err(bits_to_f64(y), ref) <= BF16_TOL


def test_mxfp4_tile_layout(moe):
    """The tiled layout, restated from its definition: 16-row blocks, 128-element chunks, 1 KB per
    (block, chunk) ordered [g][row][elements 32 g .. 32 g + 31]."""
    rows, cols = 48, 384
    src = np.random.default_rng(5).integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    got = moe.mxfp4_tile(torch.from_numpy(src).cuda()).cpu().numpy().reshape(-1)
    want = np.empty(rows * cols // 2, np.uint8)
    o = 0
    for nb in range(rows // 16):
        for c in range(cols // 128):
            for g in range(4):
                for r in range(16):
                    want[o:o + 16] = src[16 * nb + r, 64 * c + 16 * g:64 * c + 16 * g + 16]
                    o += 16
    assert np.array_equal(got, want)


def test_fp8_tile_layout(moe):
    """The fp8 tiled layout, restated from its definition: 16-row blocks, 128-element chunks, 2 KB
    per (block, chunk) ordered [h][g][row][elements 32 g + 16 h .. + 15]."""
    rows, cols = 32, 256
    src = np.random.default_rng(6).integers(0, 256, size=(rows, cols), dtype=np.uint8)
    got = moe.fp8_tile(torch.from_numpy(src).cuda()).cpu().numpy().reshape(-1)
    want = np.empty(rows * cols, np.uint8)
    o = 0
    for nb in range(rows // 16):
        for c in range(cols // 128):
            for h in range(2):
                for g in range(4):
                    for r in range(16):
                        b0 = 128 * c + 32 * g + 16 * h
                        want[o:o + 16] = src[16 * nb + r, b0:b0 + 16]
                        o += 16
    assert np.array_equal(got, want)


def test_mxfp4_rejects_mfma_config(moe):
    inp = Inputs(MXFP4_SMALL[0])
    with pytest.raises(moe.MoEError, match="UNSUPPORTED"):
        moe.Layer(inp.expert_weights(), inp.p.T, inp.p.E, inp.p.k, config=1)(inp.d_logits, inp.d_x)


# ------------------------------------------------------------------------------------------------
# MXFP4 experts with MXFP8 activations on the scaled f8f6f4 MFMA: x and h quantised per 32 channels
# (E4M3 codes, E8M0 scales; bit-exact quantiser), outputs at the 8-bit bar.  Same K-loop cases as
# the W4A16 tiles: one chunk per wavefront or none (d = 256, 384), whole pipelined pairs plus an
# odd chunk (d = 1536, 4096), one token, passes of up to 16, 32 and 64 rows.
# ------------------------------------------------------------------------------------------------

def test_quant_act_mx_exhaustive_bf16(moe):
    """A 448 in every block of 32 gives scale code 127 (E = 0): every other element's code is then
    the oracle's encoding of it -- all finite bf16 values of magnitude <= 448."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (b.astype(np.uint32) << 16).view(np.float32)
    vals = b[np.isfinite(v) & (np.abs(v) <= 448.0)]
    per, d = 31, 1024
    nblk = (vals.size + per - 1) // per
    nblk += (-nblk) % (d // 32)
    body = np.concatenate([vals, np.full(nblk * per - vals.size, 0x3F80, np.uint16)]).reshape(nblk, per)
    x = np.concatenate([np.full((nblk, 1), 0x43E0, np.uint16), body], axis=1).reshape(-1, d)
    xq, xe = moe.quant_act_mx(torch.from_numpy(x.view(np.int16)).cuda())
    rq, re = mxfp8.quant_act(x)
    assert np.all(re == 127)
    assert np.array_equal(xe.cpu().numpy(), re)
    assert np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0, 1e-30, 1e30])
def test_quant_act_mx_random(moe, scale):
    rng = np.random.default_rng(int(min(scale, 1e6) * 1000) + 7)
    x = (rng.standard_normal((41, 640)) * scale).astype(np.float32)
    x[3, 32:64] = 0.0
    x[5, :32] = -0.0
    x[7, 64:96] = rng.integers(-3, 4, 32)
    x[9, 96:128] = 448.0 * scale
    bits = I.f32_to_bf16_bits(x)
    xq, xe = moe.quant_act_mx(torch.from_numpy(bits.view(np.int16)).cuda())
    rq, re = mxfp8.quant_act(bits)
    assert np.array_equal(xe.cpu().numpy(), re)
    assert np.array_equal(xq.cpu().numpy(), rq)


MXA8_SMALL = [replace(p, name=p.name + "_a8", act_mx8=True) for p in MXFP4_SMALL]


# config 1: the LDS-staged MFMA tiles (256 x 256, one 128-value chunk per stage, both operands'
# E8M0 scales applied by the scaled MFMA) on every shape: several m-tiles with ragged tails
# (T = 300, k = 2, E = 6), an odd number of K chunks and a down tile half past d (d = 384), long K
# (d = 4096), one token (a tile of one row).  Automatic selection puts experts of more than 64 rows
# on them when a GEMM's MFMA tiles fill a round of CUs: the prefill-shaped case's gate/up GEMM
# (512 tiles) does, its down GEMM (128) streams.
@pytest.mark.parametrize("config", [-1, 0, 1])
@pytest.mark.parametrize("p", MXA8_SMALL, ids=lambda p: p.name)
def test_mxfp4_a8_layer_matches_oracle(moe, p, config):
    _check_layer(moe, Inputs(p), config=config, tol=FP8_TOL, runs=2)


MXA8_PREFILL = I.Problem("mx_a8_prefill", 125, T=4096, d=1024, f=2048, E=8, k=2,
                         wdtype=I.WDT_MXFP4, act_mx8=True)


def test_mxfp4_a8_prefill_auto_matches_oracle(moe):
    _check_layer(moe, Inputs(MXA8_PREFILL), config=-1, tol=FP8_TOL, runs=2)


def test_mxfp4_a8_grouped_ffn_matches_oracle(moe):
    p = MXA8_SMALL[2]
    inp = Inputs(p)
    rids, _ = O.route(inp.logits, p.k)
    counts, offsets = O.histogram(rids, p.E)
    perm_src, _ = O.permute(rids, p.E)
    x_perm = torch.from_numpy(np.ascontiguousarray(inp.x[perm_src // p.k]).view(np.int16)).cuda()
    y = moe.grouped_ffn(x_perm, None, torch.from_numpy(counts.astype(np.int32)).cuda(),
                        torch.from_numpy(offsets.astype(np.int32)).cuda(),
                        inp.expert_weights(), p.T, p.k)
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get, act="mxfp8")["y_perm"]
    assert rel_err(bits_to_f64(y), ref) <= FP8_TOL


def test_mxfp4_a8_mfma_grouped_ffn_matches_oracle(moe):
    p = MXA8_SMALL[1]
    inp = Inputs(p)
    rids, _ = O.route(inp.logits, p.k)
    counts, offsets = O.histogram(rids, p.E)
    perm_src, _ = O.permute(rids, p.E)
    x_perm = torch.from_numpy(np.ascontiguousarray(inp.x[perm_src // p.k]).view(np.int16)).cuda()
    y = moe.grouped_ffn(x_perm, None, torch.from_numpy(counts.astype(np.int32)).cuda(),
                        torch.from_numpy(offsets.astype(np.int32)).cuda(),
                        inp.expert_weights(), p.T, p.k, config=1)
    ref = O.moe_layer(inp.logits, inp.x, p.k, inp.get, act="mxfp8")["y_perm"]
    assert rel_err(bits_to_f64(y), ref) <= FP8_TOL
