"""The seeded input generator: determinism, distributions, device independence (CPU side)."""
import math
import numpy as np
import torch

from mixture_experts_layer_top_amd import inputs as I


def test_fmix32_python_and_torch_agree():
    rng = np.random.default_rng(0)
    vals = [int(v) for v in rng.integers(0, 2**32, size=2000, dtype=np.uint64)] + [0, 1, 2**32 - 1]
    t = I._fmix32(torch.tensor(vals, dtype=torch.int64))
    assert [I._fmix32_int(v) for v in vals] == t.tolist()


def test_determinism():
    p = I.dsv3_point(16, 0.1)
    assert np.array_equal(I.gen_logits(p), I.gen_logits(p))
    assert np.array_equal(I.gen_x(p), I.gen_x(p))
    a = I.gen_expert_weight(I.TINY, "gate", 3)
    b = I.gen_expert_weight(I.TINY, "gate", 3)
    assert torch.equal(a, b)
    assert not torch.equal(a, I.gen_expert_weight(I.TINY, "gate", 4))
    assert not torch.equal(a, I.gen_expert_weight(I.TINY, "up", 3))


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000).astype(np.float32)
    bits = I.f32_to_bf16_bits(v)
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    up = ((bits.astype(np.uint32) + 1) << 16).view(np.float32).astype(np.float64)
    dn = ((bits.astype(np.uint32) - 1) << 16).view(np.float32).astype(np.float64)
    err = np.abs(back - v)
    assert np.all(err <= np.abs(up - v)) and np.all(err <= np.abs(dn - v))
    # hashed path rounds the same way as the numpy path
    key = I.stream_key(9, 4, 0)
    tb = I.hashed_normal_bf16(key, 5000, 0.02, "cpu")
    h = I.hash_stream(key, 0, 5000, "cpu")
    s = ((h & 255) + ((h >> 8) & 255) + ((h >> 16) & 255) + (h >> 24) - 510).numpy()
    f = (s.astype(np.float32) * np.float32(0.02 / I._IH4_STD)).astype(np.float32)
    assert np.array_equal(tb.numpy().view(np.uint16), I.f32_to_bf16_bits(f))


def test_hashed_normal_moments_and_independence():
    a = I.hashed_normal_bf16(I.stream_key(1, 4, 0), 1 << 20, 0.02, "cpu")
    b = I.hashed_normal_bf16(I.stream_key(1, 4, 1), 1 << 20, 0.02, "cpu")
    fa = (a.numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fb = (b.numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(fa.mean()) < 1e-4 and abs(fa.std() - 0.02) < 2e-4
    assert abs(np.corrcoef(fa, fb)[0, 1]) < 5e-3
    assert abs(np.corrcoef(fa[:-1], fa[1:])[0, 1]) < 5e-3


def test_fp8_codes_and_scales():
    c = I.hashed_e4m3_codes(I.stream_key(4, 4, 0), 1 << 18, "cpu").numpy()
    assert not np.any((c & 0x7F) == 0x7F)  # never NaN
    mag = c & 0x7F
    assert 0.4 < np.mean(c >> 7) < 0.6
    # magnitudes concentrate around the half-normal's scale (exponent fields 12..14 = 32..256)
    ef = mag >> 3
    assert np.mean((ef >= 12) & (ef <= 14)) > 0.7
    s = I.hashed_block_scales(I.stream_key(4, 20, 0), 4096, "cpu").numpy()
    assert s.dtype == np.float32 and s.min() >= 2.0 ** -13 and s.max() < 2.0 ** -12


def test_gumbel_top1_frequency_matches_p():
    from dataclasses import replace
    p = replace(I.DSV3, T=20000, E=16, alpha=1.0, name="stat")
    L = I.gen_logits(p).astype(np.float64)
    prob = I.gen_dirichlet_p(p)
    top1 = np.argmax(L, axis=1)
    obs = np.bincount(top1, minlength=16)
    exp = prob * p.T
    chi2 = np.sum((obs - exp) ** 2 / exp)
    assert chi2 < 60  # 15 dof: far below this unless the construction is wrong


def test_dirichlet_mean():
    from dataclasses import replace
    ps = [I.gen_dirichlet_p(replace(I.DSV3, T=t, alpha=1.0)) for t in range(200)]
    assert abs(np.mean(ps) - 1 / 256) < 1e-6
    assert np.allclose(np.sum(ps, axis=1), 1.0)


def test_shapes():
    W = I.gen_weights(I.TINY, "cpu")
    assert W["gate"].shape == (8, 512, 256) and W["down"].shape == (8, 256, 512)
    assert W["gate"].dtype == torch.int16
    assert I.gen_logits(I.TINY).shape == (64, 8) and I.gen_x(I.TINY).shape == (64, 256)


# Dirichlet effective-experts model: the closed-form expected entropy against Monte Carlo draws of
# the same distribution, its limits, monotonicity, and the inverse (alpha from a target count).
def test_expected_entropy_closed_form_vs_monte_carlo():
    rng = np.random.default_rng(7)
    for E, alpha in ((256, 0.1), (256, 1.0), (384, 0.3), (8, 10.0)):
        draws = rng.dirichlet(np.full(E, alpha), size=400)
        d = np.maximum(draws, 1e-300)
        h = -(d * np.log(d)).sum(axis=1)
        assert abs(h.mean() - I.expected_entropy(E, alpha)) <= 0.02 * I.expected_entropy(E, alpha) + 3 * h.std() / 20


def test_expected_eeff_limits_and_monotone():
    E = 256
    vals = [I.expected_eeff(E, a) for a in (1e-4, 1e-2, 0.1, 1.0, 10.0, 1e4)]
    assert all(x < y for x, y in zip(vals, vals[1:]))
    assert vals[0] < 1.05 and abs(vals[-1] - E) / E < 0.01
    # a uniform p (alpha -> infinity) has entropy ln E exactly
    assert abs(I.expected_entropy(E, 1e9) - math.log(E)) < 1e-6


def test_alpha_for_eeff_round_trip():
    for E in (8, 256, 384):
        for alpha in (0.05, 0.3, 1.0, 7.0):
            target = I.expected_eeff(E, alpha)
            assert abs(I.alpha_for_eeff(E, target) / alpha - 1.0) < 1e-6


def test_effective_experts_of_counts():
    assert abs(I.effective_experts(np.array([5, 5, 5, 5, 0])) - 4.0) < 1e-12
    assert abs(I.effective_experts(np.array([7, 0, 0])) - 1.0) < 1e-12
