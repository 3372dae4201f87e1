"""Pins of the oracle's bf16 AdamW without master weights (train_gpt2.cu,
adamw_kernel3's stochastic-rounding path): the rounding step against its
exact expectation, the noise against uniformity and bijectivity, and the
whole update against cases whose result is fixed without the noise.  The
per-call seed generator (the page's xorshift*) is the page's definition on
both sides; its values are not pinned to an outside source (any seed gives
a valid rounding)."""

import numpy as np

import oracle


def _f32_from_bits(u):
    return float(np.array([u], np.uint32).view(np.float32)[0])


def test_rounding_is_exactly_unbiased_over_all_thresholds():
    # x = lower + L/65536 ulp: exactly L of the 65536 thresholds round it up,
    # so the mean over all thresholds is x itself
    for hi in (0x3F80, 0x4049, 0xBE00, 0x0085):
        for L in (0, 1, 0x3FFF, 0x8000, 0xC001, 0xFFFF):
            x = _f32_from_bits((hi << 16) | L)
            ups = sum(oracle.sr_bf16(x, r) == hi + 1 for r in range(0, 65536, 1))
            downs = sum(oracle.sr_bf16(x, r) == hi for r in range(0, 65536, 1))
            assert ups == L and downs == 65536 - L, (hex(hi), L)


def test_bf16_exact_values_are_kept():
    for hi in (0x0000, 0x3F80, 0xC2C8, 0x7F7F):
        x = _f32_from_bits(hi << 16)
        assert all(oracle.sr_bf16(x, r) == hi for r in (0, 1, 0x7FFF, 0xFFFF))


def test_noise_is_a_bijection_with_uniform_low_bits():
    # SquirrelNoise5 is a composition of bijections of 32-bit words (odd
    # multiplies, additions, right xor-shifts): distinct positions, distinct
    # values; its low 16 bits (the rounding threshold) are uniform
    seed = 0x9E3779B9
    vals = np.array([oracle.noise2d(x, y, seed) for y in range(256) for x in range(512)], np.uint64)
    assert len(np.unique(vals)) == vals.size
    counts = np.bincount((vals & 0xFF).astype(np.int64), minlength=256)
    exp = vals.size / 256
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 350  # 255 degrees of freedom: mean 255, sd 22.6


def test_update_without_step_keeps_parameters():
    # g = m = v = 0 and no weight decay: the update is exactly zero and the
    # bf16-exact parameters come back unchanged, whatever the noise
    rng = np.random.default_rng(1)
    p = (rng.integers(0, 2 ** 16, 5000) & 0x7F7F).astype(np.uint16)
    z = np.zeros(p.size, np.float32)
    q, m, v = oracle.adamw_sr(p, z, z, z, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 12345)
    assert np.array_equal(q, p) and not m.any() and not v.any()


def test_decay_only_update_rounds_without_bias():
    # g = 0, wd > 0: x = p - lr * (wd * p) for every element; with one p for
    # all n elements, the fraction rounded up matches x's position between
    # its two bf16 neighbours within binomial noise
    n = 1 << 18
    p0 = 0x3F80  # 1.0
    p = np.full(n, p0, np.uint16)
    z = np.zeros(n, np.float32)
    lr, wd = 0.013, 0.37
    one = np.float32(1.0)
    x = one - np.float32(lr) * (np.float32(wd) * one)
    xb = int(np.array([x], np.float32).view(np.uint32)[0])
    lower, frac = xb >> 16, (xb & 0xFFFF) / 65536.0
    q, _, _ = oracle.adamw_sr(p, z, z, z, lr, 0.9, 0.999, 1e-8, wd, 1, 777)
    assert set(np.unique(q).tolist()) <= {lower, lower + 1}
    up = float(np.mean(q == lower + 1))
    assert abs(up - frac) < 5 * np.sqrt(frac * (1 - frac) / n) + 1e-9
