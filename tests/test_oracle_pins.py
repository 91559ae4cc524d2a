"""Pins for the CPU oracle: checks against things other than the oracle itself (closed forms,
special cases that reduce to textbook or library routines, brute force on tiny inputs, invariants,
the fp8 format's own table and a hand-worked example).  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import fp8_e4m3 as fp8
from oracle import moe_oracle as O
from mixture_experts_layer_top_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------------------
# fp8 codec
# ------------------------------------------------------------------------------------------------

def _golden_e4m3():
    rows = []
    for line in open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_decode_matches_spec_table():
    for code, val in _golden_e4m3():
        got = fp8.decode(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_decode_structure():
    v = fp8.decode(np.arange(256, dtype=np.uint8))
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)  # monotone in the code
    assert pos.max() == 448.0 and pos[1] == 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    assert np.array_equal(v[128:255], -v[:127])
    # within a binade consecutive values differ by a constant step of 2^(E-10)
    for e in range(1, 16):
        seg = pos[e * 8:(e + 1) * 8] if e < 15 else pos[120:127]
        assert np.all(np.diff(seg) == 2.0 ** (e - 10))


def test_e4m3_encode_roundtrip_and_rounding():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(codes)), codes)
    pos = fp8.decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2  # exact in float64
    enc = fp8.encode(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)  # ties go to the even mantissa
    assert np.array_equal(enc, want.astype(np.uint8))
    # just off the midpoints goes to the nearer one
    assert np.array_equal(fp8.encode(np.nextafter(mids, 0)), lo.astype(np.uint8))
    assert np.array_equal(fp8.encode(np.nextafter(mids, 1e9)), (lo + 1).astype(np.uint8))
    # saturation, signed zero, tiny values
    assert fp8.encode(np.array([1e6, 464.0, 449.0]))[0] == 0x7E
    assert np.all(fp8.encode(np.array([1e6, 464.0, 449.0])) == 0x7E)
    assert fp8.encode(np.array([-1e30]))[0] == 0xFE
    assert fp8.encode(np.array([-0.0]))[0] == 0x80
    assert fp8.encode(np.array([2.0 ** -10]))[0] == 0x00  # half the smallest subnormal: tie -> even 0
    assert fp8.encode(np.array([-2.0 ** -11]))[0] == 0x80
    assert fp8.encode(np.array([1.5 * 2.0 ** -9]))[0] == 0x02


def test_e4m3_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(3000) * 100, rng.standard_normal(1000) * 0.01])
    enc = fp8.encode(v)
    allv = fp8.decode(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(allv)
    for x, c in zip(v, enc):
        err = np.abs(allv[finite] - min(max(x, -448), 448))
        assert abs(fp8.decode(np.array([c]))[0] - min(max(x, -448), 448)) == err.min()


# ------------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------------

def _brute_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]


def test_route_brute_force_with_planted_ties():
    rng = np.random.default_rng(1)
    for trial in range(200):
        E = int(rng.integers(1, 20))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 6))
        L = rng.integers(-3, 4, size=(T, E)).astype(np.float32)  # many exact ties
        if trial % 3 == 0:
            L = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = O.route(L, k)
        for t in range(T):
            assert list(ids[t]) == _brute_topk(L[t], k)
            sel = [float(L[t, e]) for e in ids[t]]
            den = sum(math.exp(v - sel[0]) for v in sel)
            for j in range(k):
                assert abs(w[t, j] - math.exp(sel[j] - sel[0]) / den) < 1e-15


def test_route_signed_zero_is_a_tie():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    ids, w = O.route(L, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]
    assert np.all(w == 0.5)


def test_route_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((7, 9)).astype(np.float32)
    ids, w = O.route(L, 9)
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    for t in range(7):
        assert np.allclose(w[t], full[t, ids[t]], rtol=0, atol=1e-15)
        assert sorted(ids[t].tolist()) == list(range(9))


def test_route_special_cases():
    L = np.full((3, 6), 0.25, np.float32)
    ids, w = O.route(L, 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3 and np.all(w == 0.25)
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 8)).astype(np.float32)
    _, w1 = O.route(L, 1)
    assert np.all(w1 == 1.0)
    ids2, w2 = O.route(L, 2)
    gap = L[np.arange(50), ids2[:, 0]].astype(np.float64) - L[np.arange(50), ids2[:, 1]]
    assert np.allclose(w2[:, 0], scipy.special.expit(gap), rtol=0, atol=1e-15)  # closed form k=2
    _, w8 = O.route(L, 5)
    assert np.allclose(w8.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w8, axis=1) <= 0)


# ------------------------------------------------------------------------------------------------
# dispatch
# ------------------------------------------------------------------------------------------------

def test_histogram_and_permutation_invariants():
    rng = np.random.default_rng(4)
    for _ in range(30):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(0, 60))
        L = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = O.route(L, k) if T else (np.zeros((0, k), np.int32), None)
        counts, offsets = O.histogram(ids, E)
        assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
        for t in range(T):
            assert len(set(ids[t].tolist())) == k  # every token routed to k distinct experts
        perm_src, slot_dst = O.permute(ids, E)
        n = T * k
        assert np.array_equal(perm_src[slot_dst], np.arange(n))  # bijection
        assert np.array_equal(slot_dst[perm_src], np.arange(n))
        # same as a library stable sort of the slots by expert
        assert np.array_equal(perm_src, np.argsort(ids.ravel(), kind="stable"))
        flat = ids.ravel()
        for e in range(E):
            seg = perm_src[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e)  # each row sits in its expert's segment
            assert np.all(np.diff(seg) > 0)  # stable
        payload = rng.standard_normal((n, 3))
        assert np.array_equal(payload[perm_src][slot_dst], payload)  # permute then inverse


# ------------------------------------------------------------------------------------------------
# experts and the layer
# ------------------------------------------------------------------------------------------------

def test_silu_identities():
    z = np.linspace(-30, 30, 1001)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(O.silu(z) - O.silu(-z), z, rtol=0, atol=1e-12)
    assert np.allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([-1000.0]))[0] == 0.0


def _bits(a):
    return I.f32_to_bf16_bits(np.asarray(a, np.float32))


def _weights_from_list(experts):
    def get(e):
        return {n: _bits(experts[e][n]) for n in ("gate", "up", "down")}
    return get


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    res = O.moe_layer(np.array(g["logits"], np.float32), _bits(g["x"]), g["k"],
                      _weights_from_list(g["experts"]))
    assert res["ids"].tolist() == g["ids"]
    assert np.allclose(res["w"], g["w"], rtol=0, atol=1e-15)
    assert res["counts"].tolist() == g["counts"]
    assert res["offsets"].tolist() == g["offsets"]
    assert res["perm_src"].tolist() == g["perm_src"]
    assert res["slot_dst"].tolist() == g["slot_dst"]
    assert np.allclose(res["out"], g["out"], rtol=0, atol=1e-15)


def _textbook_swiglu(x, Wg, Wu, Wd):
    """Dense SwiGLU FFN written out with explicit loops: out_i = sum_n Wd[i][n] * silu(g_n) * u_n."""
    d, f = len(x), len(Wg)
    out = []
    g = [sum(Wg[n][i] * x[i] for i in range(d)) for n in range(f)]
    u = [sum(Wu[n][i] * x[i] for i in range(d)) for n in range(f)]
    h = [g[n] / (1.0 + math.exp(-g[n])) * u[n] for n in range(f)]
    for i in range(d):
        out.append(sum(Wd[i][n] * h[n] for n in range(f)))
    return out


def _rand_problem(rng, T, d, f, E):
    x = _bits(rng.standard_normal((T, d)))
    W = [{n: _bits(rng.standard_normal(s) * 0.2)
          for n, s in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f)))} for _ in range(E)]
    return x, W


def test_E1_k1_is_dense_swiglu():
    rng = np.random.default_rng(6)
    T, d, f = 5, 6, 7
    x, W = _rand_problem(rng, T, d, f, 1)
    L = rng.standard_normal((T, 1)).astype(np.float32)
    res = O.moe_layer(L, x, 1, lambda e: W[e])
    xd = O.bf16_bits_to_f64(x).tolist()
    Wd = {n: O.bf16_bits_to_f64(W[0][n]).tolist() for n in W[0]}
    for t in range(T):
        ref = _textbook_swiglu(xd[t], Wd["gate"], Wd["up"], Wd["down"])
        assert np.allclose(res["out"][t], ref, rtol=1e-13, atol=1e-13)
    assert np.all(res["w"] == 1.0)


def test_identical_experts_give_the_dense_ffn():
    rng = np.random.default_rng(7)
    T, d, f, E, k = 9, 8, 5, 6, 3
    x, W = _rand_problem(rng, T, d, f, 1)
    L = rng.standard_normal((T, E)).astype(np.float32)
    res = O.moe_layer(L, x, k, lambda e: W[0])  # every expert the same
    xd = O.bf16_bits_to_f64(x).tolist()
    Wd = {n: O.bf16_bits_to_f64(W[0][n]).tolist() for n in W[0]}
    for t in range(T):
        ref = _textbook_swiglu(xd[t], Wd["gate"], Wd["up"], Wd["down"])
        assert np.allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)


def test_zero_inputs_give_zero():
    rng = np.random.default_rng(8)
    T, d, f, E, k = 6, 4, 3, 5, 2
    x, W = _rand_problem(rng, T, d, f, E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    res = O.moe_layer(L, np.zeros_like(x), k, lambda e: W[e])
    assert np.all(res["out"] == 0)
    Wz = [dict(w, down=np.zeros_like(w["down"])) for w in W]
    res = O.moe_layer(L, x, k, lambda e: Wz[e])
    assert np.all(res["out"] == 0)


def test_direct_per_token_form_equals_permuted_layer():
    rng = np.random.default_rng(9)
    T, d, f, E, k = 13, 8, 6, 7, 3
    x, W = _rand_problem(rng, T, d, f, E)
    L = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    res = O.moe_layer(L, x, k, lambda e: W[e])
    tok = O.moe_tokens(np.arange(T), L, x, k, lambda e: W[e])
    assert np.allclose(res["out"], tok["out"], rtol=1e-13, atol=1e-13)
    part = O.moe_tokens(np.array([3, 11]), L, x, k, lambda e: W[e])
    assert np.allclose(part["out"], res["out"][[3, 11]], rtol=1e-13, atol=1e-13)
    # and a fully naive triple loop for every token
    xd = O.bf16_bits_to_f64(x)
    for t in range(T):
        ids = _brute_topk(L[t], k)
        sel = [float(L[t, e]) for e in ids]
        den = sum(math.exp(v - sel[0]) for v in sel)
        acc = np.zeros(d)
        for j, e in enumerate(ids):
            Wd = {n: O.bf16_bits_to_f64(W[e][n]).tolist() for n in W[e]}
            acc += math.exp(sel[j] - sel[0]) / den * np.array(
                _textbook_swiglu(xd[t].tolist(), Wd["gate"], Wd["up"], Wd["down"]))
        assert np.allclose(res["out"][t], acc, rtol=1e-12, atol=1e-12)


def test_shared_expert_adds_with_weight_one():
    rng = np.random.default_rng(10)
    T, d, f, E, k = 6, 4, 3, 5, 2
    x, W = _rand_problem(rng, T, d, f, E + 1)
    L = rng.standard_normal((T, E)).astype(np.float32)
    base = O.moe_layer(L, x, k, lambda e: W[e])
    withs = O.moe_layer(L, x, k, lambda e: W[e], get_shared=lambda: W[E])
    xd = O.bf16_bits_to_f64(x).tolist()
    Wd = {n: O.bf16_bits_to_f64(W[E][n]).tolist() for n in W[E]}
    for t in range(T):
        ref = _textbook_swiglu(xd[t], Wd["gate"], Wd["up"], Wd["down"])
        assert np.allclose(withs["out"][t] - base["out"][t], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# fp8 activation quantisation and weights
# ------------------------------------------------------------------------------------------------

def test_act_quant_properties():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 384)).astype(np.float32) * np.array([1, 1e-3, 50, 1], np.float32)[:, None]
    x[3, 128:256] = 0.0
    bits = I.f32_to_bf16_bits(x)
    q, s = O.quant_act_e4m3(bits)
    xv = O.bf16_bits_to_f32(bits)
    assert s.dtype == np.float32 and s.shape == (4, 3)
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] == 0)
    deq = O.dequant_act_e4m3(q, s)
    blocks = xv.reshape(4, 3, 128)
    for t in range(4):
        for b in range(3):
            amax = np.abs(blocks[t, b]).max()
            if amax == 0:
                continue
            assert s[t, b] == np.float32(amax / np.float32(448))
            # the largest element lands on +-448 (or the nearest code below it)
            r = np.abs(fp8.decode(q[t, b * 128:(b + 1) * 128])).max()
            assert r in (448.0, 416.0)
            # every element within half a quantisation step of its value
            v = blocks[t, b].astype(np.float64)
            dq = deq[t, b * 128:(b + 1) * 128]
            step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(v) / s[t, b], 2.0 ** -6))) - 3),
                              2.0 ** -9) * s[t, b]
            assert np.all(np.abs(dq - v) <= step / 2 * (1 + 1e-6))
    # brute force: each code is the nearest of the 254 finite values to fp32(x / s)
    allv = fp8.decode(np.arange(256, dtype=np.uint8))
    fin = ~np.isnan(allv)
    for t in range(4):
        for i in range(0, 384, 7):
            r = float(np.float32(xv[t, i]) / s[t, i // 128])
            best = np.abs(allv[fin] - r).min()
            assert abs(fp8.decode(q[t:t + 1, i])[0] - r) == best


def test_block_dequant():
    codes = np.full((256, 128), 0x38, np.uint8)  # all 1.0
    scales = np.array([[0.5], [2.0]], np.float32)
    v = O.dequant_e4m3_blocks(codes, scales)
    assert np.all(v[:128] == 0.5) and np.all(v[128:] == 2.0)


# ------------------------------------------------------------------------------------------------
# the tolerance is attainable: an oracle variant with GPU-like rounding passes it
# ------------------------------------------------------------------------------------------------

def _gen_problem_weights(p):
    import torch  # noqa: F401  (the generator runs torch ops on the CPU)
    W = I.gen_weights(p, "cpu")

    def get(e):
        r = {n: W[n][e].numpy() for n in ("gate", "up", "down")}
        if p.wdtype == I.WDT_FP8:
            r.update({"s_" + n: W["s_" + n][e].numpy() for n in ("gate", "up", "down")})
        return r

    def get_sh():
        r = {n: W["sh_" + n].numpy() for n in ("gate", "up", "down")}
        if p.wdtype == I.WDT_FP8:
            r.update({"s_" + n: W["s_sh_" + n].numpy() for n in ("gate", "up", "down")})
        return r
    return get, (get_sh if p.shared else None)


def test_tolerance_attainable_bf16_tiny():
    p = I.TINY
    get, _ = _gen_problem_weights(p)
    L, x = I.gen_logits(p), I.gen_x(p)
    ref = O.moe_layer(L, x, p.k, get)["out"]
    emu = O.moe_layer_emulated(L, x, p.k, get)
    err = np.abs(emu - ref).max() / np.abs(ref).max()
    assert err <= 2e-2 / 2, err  # comfortably inside the bound


def test_tolerance_attainable_fp8_small():
    from dataclasses import replace
    p = replace(I.FP8, T=24, d=256, f=256, E=16, k=4, shared_f=256, name="fp8_small")
    get, get_sh = _gen_problem_weights(p)
    L, x = I.gen_logits(p), I.gen_x(p)
    ref = O.moe_layer(L, x, p.k, get, get_sh, act_fp8=True)["out"]
    emu = O.moe_layer_emulated(L, x, p.k, get, get_sh, act_fp8=True)
    err = np.abs(emu - ref).max() / np.abs(ref).max()
    assert err <= 6e-2 / 2, err


# ------------------------------------------------------------------------------------------------
# the emulated variant's rounding steps
# ------------------------------------------------------------------------------------------------

def _finite_f32_sample(n, seed):
    """Random float32 bit patterns over the whole finite range (every binade, subnormals, both
    signs), plus the values next to the bfloat16 overflow boundary."""
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> np.uint32(23)) & np.uint32(255)) != 255]
    edge = np.arange(0x7F7F0000, 0x7F800000, 97, dtype=np.uint32)  # near float32 / bf16 max
    sub = np.arange(0, 1 << 23, 4099, dtype=np.uint32)              # float32 subnormals
    u = np.concatenate([u, edge, sub])
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    return u.view(np.float32)


def test_bf16_rounding_matches_integer_rounding_and_torch():
    """On float32-representable values the oracle's bf16 rounding equals the generator's integer
    round-half-even on the bit pattern and torch's float32 -> bfloat16 conversion (two routes that
    share nothing with the oracle's frexp/quantum arithmetic)."""
    import torch
    v = _finite_f32_sample(2_000_000, 21)
    got = O.f64_to_bf16_f64(v.astype(np.float64))
    via_bits = O.bf16_bits_to_f64(I.f32_to_bf16_bits(v))
    via_torch = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, via_bits)
    assert np.array_equal(got, via_torch)
    assert np.array_equal(np.signbit(got), np.signbit(v))


def test_bf16_rounding_hand_worked():
    """Float64 values that float32 cannot hold: one rounding, straight from float64 (going through
    float32 first would round twice and lose the sticky bits)."""
    t = 2.0 ** -133  # bf16 subnormal quantum
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite bf16
    cases = [
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),  # above the midpoint: up (via fp32: tie -> 1)
        (1.0 + 2.0 ** -8, 1.0),                          # tie, 1.0000000 is even
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),          # tie between ...001 and ...010: even
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 1.0),             # just below the midpoint
        (1.5 * t, 2 * t),                                # subnormal tie: 1 (odd) vs 2 (even)
        (0.5 * t, 0.0),                                  # tie with zero: zero is even
        (0.5 * t + 2.0 ** -170, t),                      # just above it
        (2.0 ** -126 - 2.0 ** -140, 2.0 ** -126),        # rounds up into the normal range
        ((2.0 - 2.0 ** -8) * 2.0 ** 127, math.inf),      # tie between max (odd) and 2^128 (even)
        ((2.0 - 2.0 ** -8 - 2.0 ** -20) * 2.0 ** 127, big),
        (3.39e38, big),                                  # above max, below max + half a step
        (1.0e39, math.inf),
        (1e-300, 0.0),
    ]
    for v, want in cases:
        for sgn in (1.0, -1.0):
            got = float(O.f64_to_bf16_f64(np.array([sgn * v]))[0])
            assert got == sgn * want, (sgn * v, got, sgn * want)
            assert math.copysign(1.0, got) == sgn


def test_requant_rows_matches_activation_quantiser():
    """quant_rows_e4m3_f64 (the emulated fp8 requantisation of h) on bf16-representable rows equals
    dequantising the activation quantiser's codes and scales, which takes the bits themselves."""
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((9, 640)) * np.array([1, 1e-3, 40, 1, 3e-6, 1, 1, 200, 1],
                                                  np.float32)[:, None]).astype(np.float32)
    x[3, 128:256] = 0.0
    x[5, :128] = -0.0
    x[6, 256:384] = rng.integers(-4, 5, 128)
    bits = I.f32_to_bf16_bits(x)
    q, s = O.quant_act_e4m3(bits)
    want = O.dequant_act_e4m3(q, s)
    got = O.quant_rows_e4m3_f64(O.bf16_bits_to_f64(bits))
    assert np.array_equal(got, want)


def test_requant_rows_hand_worked():
    """One 128-wide group worked by hand: amax 896 gives s = 2 exactly; 896 -> 448 (code 0x7E);
    3 -> 1.5; 2.3 -> 1.15 -> 1.125 (step 1/8 in [1, 2)); 0.01 -> 0.005 -> 3 * 2^-9 (subnormal step
    2^-9: 0.005 / 2^-9 = 2.56); -700 -> -350 -> -352 (step 32 in [256, 448]).  Values are then
    multiplied back by s."""
    row = np.zeros((1, 128))
    row[0, :5] = [896.0, 3.0, 2.3, 0.01, -700.0]
    got = O.quant_rows_e4m3_f64(row)[0]
    want = np.zeros(128)
    want[:5] = [896.0, 3.0, 2.25, 2 * 3 * 2.0 ** -9, -704.0]
    assert np.array_equal(got, want)


def test_layers_sharing_weights_equal_separate_layers():
    """moe_layers (several calls decoding each expert once) gives each call's moe_layer result,
    computed here expert by expert without it: the per-token direct form for each call."""
    rng = np.random.default_rng(23)
    T_list, d, f, E, k = (1, 7, 30), 128, 128, 6, 2
    W = {e: {n: I.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32) * 0.05)
             for n, s in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f)))} for e in range(E + 1)}
    calls = [(rng.standard_normal((T, E)).astype(np.float32),
              I.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))) for T in T_list]
    for shared in (None, (lambda: W[E])):
        got = O.moe_layers(calls, k, lambda e: W[e], shared)
        for (L, x), r in zip(calls, got):
            direct = O.moe_tokens(np.arange(L.shape[0]), L, x, k, lambda e: W[e], shared)
            assert np.allclose(r["out"], direct["out"], rtol=1e-12, atol=1e-14)
            ids, _ = O.route(L, k)
            assert np.array_equal(r["ids"], ids)


# ------------------------------------------------------------------------------------------------
# storage decoding helpers: bf16 bits, block-scaled e4m3 weights and activations, the weight and
# activation dispatch
# ------------------------------------------------------------------------------------------------

def test_bf16_bits_hand_worked():
    """bfloat16 is the top half of a float32: sign, 8 exponent bits (bias 127), 7 mantissa bits."""
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x4049: 3.140625,   # 1.1001001b * 2^1
        0x3E80: 0.25, 0x0001: 2.0 ** -133,                          # min subnormal
        0x0080: 2.0 ** -126,                                        # min normal
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,                     # max finite
        0x7F80: math.inf, 0xFF80: -math.inf, 0x0000: 0.0,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    want = np.array(list(cases.values()))
    assert np.array_equal(O.bf16_bits_to_f64(bits), want)
    assert np.array_equal(O.bf16_bits_to_f32(bits), want.astype(np.float32))
    neg0 = O.bf16_bits_to_f64(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0
    # int16 storage (the binding's dtype) is read as the same bit patterns
    assert np.array_equal(O.bf16_bits_to_f64(bits.view(np.int16)), want)
    assert math.isnan(O.bf16_bits_to_f64(np.array([0x7FC0], np.uint16))[0])


def _e4m3_spec(code: int) -> float:
    """E4M3FN by its definition: sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at
    exponent 0, S.1111.111 NaN."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_dequant_e4m3_blocks_by_element():
    """Block (i // 128, j // 128) scales element (i, j): a 256 x 384 weight with a 2 x 3 scale grid
    of distinct powers of two and random non-NaN codes, checked element by element."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(256, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11          # no NaN codes
    scales = np.array([[0.5, 2.0, 8.0], [0.25, 4.0, 16.0]], np.float32)
    got = O.dequant_e4m3_blocks(codes, scales)
    for i in range(0, 256, 17):
        for j in range(0, 384, 13):
            assert got[i, j] == _e4m3_spec(int(codes[i, j])) * float(scales[i // 128, j // 128])
    assert got[127, 255] == _e4m3_spec(int(codes[127, 255])) * 2.0
    assert got[128, 256] == _e4m3_spec(int(codes[128, 256])) * 16.0


def test_dequant_act_e4m3_by_element():
    """Activation scales are per token and 128 channels: token t's group g scales [128 g, 128 g +
    128) of row t only."""
    rng = np.random.default_rng(8)
    q = rng.integers(0, 256, size=(3, 256)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x22
    s = np.array([[1.0, 0.5], [4.0, 0.125], [3.0, 6.0]], np.float32)
    got = O.dequant_act_e4m3(q, s)
    for t in range(3):
        for c in range(256):
            assert got[t, c] == _e4m3_spec(int(q[t, c])) * float(s[t, c // 128])


def test_decode_weight_and_layer_input_dispatch():
    """decode_weight: int16/uint16 bf16 bits, uint8 codes with fp32 block scales (e4m3) or uint8
    E8M0 scales (mxfp4); layer_input: bf16 values unchanged, fp8 and mxfp8 through their
    quantise-dequantise pairs."""
    from oracle import mxfp4, mxfp8
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 16, size=(128, 128)).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80     # finite only
    assert np.array_equal(O.decode_weight(bits.view(np.int16)), O.bf16_bits_to_f64(bits))
    codes = rng.integers(0, 0x7F, size=(128, 256)).astype(np.uint8)
    sc = np.array([[2.0, 0.5]], np.float32)
    assert np.array_equal(O.decode_weight(codes, sc), O.dequant_e4m3_blocks(codes, sc))
    packed = rng.integers(0, 256, size=(16, 64)).astype(np.uint8)
    e8 = rng.integers(120, 134, size=(16, 4)).astype(np.uint8)
    assert np.array_equal(O.decode_weight(packed, e8), mxfp4.dequant(packed, e8))
    with pytest.raises(ValueError):
        O.decode_weight(codes)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    xb = I.f32_to_bf16_bits(x)
    v, q, s = O.layer_input(xb)
    assert q is None and s is None and np.array_equal(v, O.bf16_bits_to_f64(xb))
    v, q, s = O.layer_input(xb, act="fp8")
    q2, s2 = O.quant_act_e4m3(xb)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.array_equal(v, O.dequant_act_e4m3(q2, s2))
    assert np.array_equal(O.layer_input(xb, act_fp8=True)[0], v)
    v, q, s = O.layer_input(xb, act="mxfp8")
    q3, s3 = mxfp8.quant_act(xb)
    assert np.array_equal(q, q3) and np.array_equal(s, s3)
    assert np.array_equal(v, mxfp8.dequant_rows(q3, s3))
    with pytest.raises(ValueError):
        O.layer_input(xb, act="int4")
