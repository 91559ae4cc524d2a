"""Pins for the oracle's MXFP8 activation quantiser (oracle/mxfp8.py): E4M3 elements with one E8M0
scale per 32 channels, the scale exponent from the block's largest magnitude.  Checked against
direct power-of-two comparisons, every finite bf16 value, scale invariance, brute force and
hand-worked blocks.  CPU only."""
import numpy as np

from mixture_experts_layer_top_amd import inputs as I
from oracle import fp8_e4m3 as fp8
from oracle import moe_oracle as O
from oracle import mxfp8

FINITE = fp8.decode(np.arange(256, dtype=np.uint8))
FINITE = FINITE[~np.isnan(FINITE)]


def test_shared_exponent_is_the_smallest_that_fits():
    """E is the smallest integer with amax <= 448 * 2^E, clamped to [-127, 127]: checked by comparing
    with 448 * 2^E and 448 * 2^(E-1) directly, over every binade of float32 (subnormals included)."""
    rng = np.random.default_rng(31)
    u = rng.integers(1, 0x7F800000, size=200_000, dtype=np.uint64).astype(np.uint32)
    amax = np.concatenate([u.view(np.float32).astype(np.float64),
                           448.0 * 2.0 ** np.arange(-20, 20), np.nextafter(448.0, 0) * 2.0 ** np.arange(-20, 20)])
    E = mxfp8.shared_exponent(amax)
    inside = (E > -127) & (E < 127)
    assert np.all(amax[inside] <= 448.0 * 2.0 ** E[inside])
    assert np.all(amax[inside] > 448.0 * 2.0 ** (E[inside] - 1))
    assert np.all(amax[E == -127] <= 448.0 * 2.0 ** -127)  # clamped below
    assert E.max() <= 127
    assert mxfp8.shared_exponent(np.array([0.0, 448.0, 449.0, 224.0, 224.5]))[0] == 0
    assert list(mxfp8.shared_exponent(np.array([448.0, 449.0, 224.0, 224.5]))) == [0, 1, -1, 0]


def test_every_bf16_value_in_a_unit_scale_block():
    """A block whose largest magnitude is 448 has E = 0 (scale code 127): every other element's
    code is then E4M3's own encoding of it -- all finite bf16 values of magnitude <= 448."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (b.astype(np.uint32) << 16).view(np.float32)
    vals = b[np.isfinite(v) & (np.abs(v) <= 448.0)]
    per = 31
    n = (vals.size + per - 1) // per
    body = np.concatenate([vals, np.full(n * per - vals.size, 0x3F80, np.uint16)]).reshape(n, per)
    x = np.concatenate([np.full((n, 1), 0x43E0, np.uint16), body], axis=1)  # 448.0 first
    x = x[: n - n % 4].reshape(-1, 128)
    q, s = mxfp8.quant_act(x)
    assert np.all(s == 127)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(q, fp8.encode(xv))


def test_codes_are_nearest_and_scale_invariant():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((16, 256)) * np.exp(rng.uniform(-20, 20, (16, 1)))
    bits = I.f32_to_bf16_bits(x.astype(np.float32))
    q, s = mxfp8.quant_act(bits)
    xv = O.bf16_bits_to_f64(bits)
    E = s.astype(np.int64) - 127
    for t in range(16):
        for c in range(0, 256, 5):
            r = xv[t, c] * 2.0 ** -E[t, c // 32]
            got = fp8.decode(q[t:t + 1, c])[0]
            if abs(r) >= 448:
                assert got == np.copysign(448.0, r)
            else:
                assert abs(got - r) == np.abs(FINITE - r).min()
    # the block's largest element lands in (224, 448] before rounding, so its code lies in
    # [224, 448] and nothing saturates
    blk = np.abs(fp8.decode(q)).reshape(16, 8, 32).max(axis=2)
    assert np.all((blk >= 224) & (blk <= 448))
    # scaling a block by 2^m shifts its scale code by m and leaves its codes alone
    for m in (-9, 1, 13):
        q2, s2 = mxfp8.quant_act(I.f32_to_bf16_bits((xv * 2.0 ** m).astype(np.float32)))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2.astype(np.int64), s.astype(np.int64) + m)


def test_hand_worked_blocks():
    """amax 1000: 448 * 2 = 896 < 1000 <= 448 * 4, so E = 2 and the scale code is 129.  1000 / 4 = 250
    lies in [128, 256) with step 16: 240 or 256, nearer 256 (-> 1024); 3 / 4 = 0.75 and
    -0.5 / 4 = -0.125 are E4M3 values; 0.1 / 4 = 0.025 lies in [2^-6, 2^-5) with step 2^-9:
    0.025 / 2^-9 = 12.8 -> 13 * 2^-9 (-> 0.1015625); 0 stays 0.  A block of zeros has scale code
    127 and zero codes (-0 keeps its sign).  A block whose largest magnitude is 2^-130 needs
    E = -138, clamped to -127 (code 0): 2^-130 * 2^127 = 0.125."""
    x = np.zeros((3, 32))
    x[0, :5] = [3.0, 1000.0, -0.5, 0.1, 0.0]
    x[1, 7] = -0.0
    x[2, 0] = 2.0 ** -130
    q, s = mxfp8.quant_rows(x)
    assert list(s[:, 0]) == [129, 127, 0]
    d = mxfp8.dequant_rows(q, s)
    assert list(d[0, :5]) == [3.0, 1024.0, -0.5, 13 * 2.0 ** -9 * 4, 0.0]
    assert q[1, 7] == 0x80 and np.all(np.delete(q[1], 7) == 0)
    assert d[2, 0] == 2.0 ** -130 and fp8.decode(q[2:3, 0])[0] == 0.125


def test_layer_with_mxfp8_activations():
    """E = 1, k = 1 with MXFP8 activations is the dense SwiGLU FFN on the dequantised activations
    (written out as loops), and the rounding-emulating variant (fp32 GEMMs, h requantised to MXFP8,
    bf16 y and output) stays well inside the 6e-2 bound."""
    rng = np.random.default_rng(33)
    T, d, f = 5, 64, 96
    x = I.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    W = {n: I.f32_to_bf16_bits((rng.standard_normal(sh) * 0.1).astype(np.float32))
         for n, sh in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f)))}
    L = rng.standard_normal((T, 1)).astype(np.float32)
    out = O.moe_layer(L, x, 1, lambda e: W, act="mxfp8")["out"]
    xd = mxfp8.dequant_rows(*mxfp8.quant_act(x))
    Wd = {n: O.bf16_bits_to_f64(W[n]) for n in W}
    for t in range(T):
        h = []
        for j in range(f):
            g = sum(xd[t, i] * Wd["gate"][j, i] for i in range(d))
            u = sum(xd[t, i] * Wd["up"][j, i] for i in range(d))
            h.append(g / (1.0 + np.exp(-g)) * u)
        for i in range(0, d, 7):
            ref = sum(h[j] * Wd["down"][i, j] for j in range(f))
            assert abs(out[t, i] - ref) <= 1e-12 * max(1.0, abs(ref))
    # tolerance sanity on a small MXFP4 problem
    p = I.Problem("mx8_small", 190, T=48, d=256, f=256, E=8, k=2, wdtype=I.WDT_MXFP4)
    import torch  # noqa: F401  (the generator runs torch ops on the CPU)
    Wm = I.gen_weights(p, "cpu")

    def get(e):
        return {**{n: Wm[n][e].numpy() for n in ("gate", "up", "down")},
                **{"s_" + n: Wm["s_" + n][e].numpy() for n in ("gate", "up", "down")}}
    Lg, xg = I.gen_logits(p), I.gen_x(p)
    ref = O.moe_layer(Lg, xg, p.k, get, act="mxfp8")["out"]
    emu = O.moe_layer_emulated(Lg, xg, p.k, get, act="mxfp8")
    assert np.abs(emu - ref).max() / np.abs(ref).max() <= 6e-2 / 2
