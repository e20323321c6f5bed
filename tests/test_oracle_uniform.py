"""Pins of the oracle's uniform quantizer against what the pages and IEEE arithmetic fix.

The pages fix: the zero point is the group minimum, the step is the range over
2^B - 1, each element goes to the nearest step, so the error is at most half a
step ("The KV cache has a geometry problem", section "Quantization error in
practice"); keys are grouped per channel and values per token (same page,
sections on keys and values; KIVI post, "Method"); groups of 32 with a
floating-point zero point (KIVI post, "Experiments").
"""
import numpy as np
import pytest

from oracle import kvq_oracle as O


def _f16(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


# ---- IEEE binary16 conversion: values fixed by the standard ----------------
@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (65520.0, 0x7C00),
    (1.0 + 2.0 ** -11, 0x3C00),              # tie -> even mantissa
    (1.0 + 3 * 2.0 ** -11, 0x3C02),          # tie -> even (up)
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002),
    (-0.0, 0x8000), (0.1, 0x2E66), (1.0 / 3.0, 0x3555),
])
def test_rne16_ieee_values(x, bits):
    assert int(O.f32_to_f16_bits(np.float32(x))) == bits


def test_f16_widening_exact():
    allbits = np.arange(0, 0x7C00, dtype=np.uint16)       # every finite non-negative fp16
    f = O.f16_to_f32(allbits)
    # fp16 value = (1 + m/1024) 2^(e-15), or m 2^-24 for e == 0
    e = (allbits >> 10).astype(np.int64)
    m = (allbits & 0x3FF).astype(np.float64)
    ref = np.where(e == 0, m * 2.0 ** -24, (1 + m / 1024) * 2.0 ** (e - 15))
    assert np.array_equal(f.astype(np.float64), ref)


# ---- closed-form error bound ------------------------------------------------
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("spread", [1e-3, 1.0, 300.0])
def test_error_bound(bits, spread):
    rng = np.random.default_rng(bits * 1000 + int(spread * 7))
    x = (rng.standard_normal((4000, 32)) * spread + rng.standard_normal((4000, 1)) * spread)
    xb = _f16(x)
    xf = O.f16_to_f32(xb).astype(np.float64)
    c, s_h, m_h = O.uniform_quantize_groups(xb, bits)
    xh = O.uniform_dequant(c, s_h, m_h).astype(np.float64)
    s = O.f16_to_f32(s_h).astype(np.float64)[:, None]
    L = 2 ** bits - 1
    step = (xf.max(1) - xf.min(1))[:, None] / L              # exact step, float64
    # stored scale is the step rounded to fp16 (plus one fp32 rounding)
    assert np.all(np.abs(s - step) <= step * 2.0 ** -10 + 1e-30)
    ulp = np.spacing(np.maximum(np.abs(xf), np.abs(xf.min(1))[:, None]).astype(np.float32))
    bound = s / 2 + L * np.abs(step - s) + 4 * ulp.astype(np.float64)
    assert np.all(np.abs(xf - xh) <= bound)
    assert c.max() <= L


# ---- exact round trip: groups whose values are a + j 2^e with every level present
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("a,e", [(0.0, 0), (-3.0, -2), (12.5, -1), (-1000.0, 3), (0.25, -8)])
def test_exact_round_trip(bits, a, e):
    L = 2 ** bits - 1
    rng = np.random.default_rng(bits + 10 * (e + 20))
    j = np.concatenate([np.arange(L + 1), rng.integers(0, L + 1, 32 - (L + 1))])
    rng.shuffle(j)
    x = a + j * 2.0 ** e
    xb = _f16(x)
    assert np.array_equal(O.f16_to_f32(xb).astype(np.float64), x)    # exact fp16 inputs
    c, s_h, m_h = O.uniform_quantize_groups(xb[None], bits)
    assert np.array_equal(c[0], j)
    assert float(O.f16_to_f32(s_h)[0]) == 2.0 ** e
    assert float(O.f16_to_f32(m_h)[0]) == a + 0.0
    xh = O.uniform_dequant(c, s_h, m_h)[0].astype(np.float64)
    assert np.array_equal(xh, x)


def test_constant_group_and_signed_zero():
    for v in (0.0, -0.0, 7.25, -3.5):
        xb = _f16(np.full(32, v))
        c, s_h, m_h = O.uniform_quantize_groups(xb[None], 2)
        assert not c.any()
        assert int(s_h[0]) == 0                      # +0, never -0
        assert float(O.f16_to_f32(m_h)[0]) == v + 0.0
        assert int(m_h[0]) != 0x8000
        assert np.array_equal(O.uniform_dequant(c, s_h, m_h)[0], O.f16_to_f32(xb) + np.float32(0))


@pytest.mark.parametrize("bits", [2, 4])
def test_extremes_map_to_end_codes(bits):
    rng = np.random.default_rng(5)
    xb = _f16(rng.standard_normal((500, 32)) * 3)
    x = O.f16_to_f32(xb)
    c, _, _ = O.uniform_quantize_groups(xb, bits)
    rows = np.arange(500)
    assert np.all(c[rows, x.argmin(1)] == 0)
    assert np.all(c[rows, x.argmax(1)] == 2 ** bits - 1)


# ---- brute force: the code is the nearest level of the stored grid ----------
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_nearest_level_brute_force(bits):
    rng = np.random.default_rng(100 + bits)
    L = 2 ** bits - 1
    xb = _f16(rng.uniform(-5, 5, (3000, 32)) * rng.uniform(0.01, 50, (3000, 1)))
    x = O.f16_to_f32(xb).astype(np.float64)
    c, s_h, m_h = O.uniform_quantize_groups(xb, bits)
    s = O.f16_to_f32(s_h).astype(np.float64)[:, None]
    m = O.f16_to_f32(m_h).astype(np.float64)[:, None]
    grid = m[..., None] + s[..., None] * np.arange(L + 1)          # [G, 1, L+1]
    d = np.abs(x[..., None] - grid)
    best = d.argmin(-1)
    dbest = np.take_along_axis(d, best[..., None], -1)[..., 0]
    dcode = np.take_along_axis(d, c[..., None].astype(np.int64), -1)[..., 0]
    # equal to the nearest level, or an exact/near tie (fp32 rounding of (x - min)/s)
    near_tie = np.abs(dcode - dbest) <= 1e-6 * (np.abs(x) + s)
    assert np.all((c == best) | near_tie)
    assert np.mean(c == best) > 0.999


def test_ties_round_half_to_even():
    # min 0, max 3 -> step 1: (x - 0) * 1 = k + 1/2 exactly
    x = np.zeros(32)
    x[1] = 3.0
    x[2:5] = [0.5, 1.5, 2.5]
    c, s_h, _ = O.uniform_quantize_groups(_f16(x)[None], 2)
    assert float(O.f16_to_f32(s_h)[0]) == 1.0
    assert list(c[0, 2:5]) == [0, 2, 2]


# ---- axis invariants ---------------------------------------------------------
def test_per_channel_key_outlier_isolation():
    rng = np.random.default_rng(7)
    k = _f16(rng.standard_normal((1, 1, 128, 64)))
    kc, ks, km = O.quantize_keys_per_channel(k, 2)
    k2 = k.copy()
    k2[..., 17] = _f16(O.f16_to_f32(k[..., 17]) * 100)
    kc2, ks2, km2 = O.quantize_keys_per_channel(k2, 2)
    other = np.arange(64) != 17
    assert np.array_equal(kc[..., other], kc2[..., other])
    assert np.array_equal(ks[..., other], ks2[..., other])
    assert np.array_equal(km[..., other], km2[..., other])
    assert not np.array_equal(ks[..., 17], ks2[..., 17])


def test_per_token_value_isolation():
    rng = np.random.default_rng(8)
    v = _f16(rng.standard_normal((1, 1, 64, 128)))
    vc, vs, vm = O.quantize_values_per_token(v, 2)
    v2 = v.copy()
    v2[..., 9, :] = _f16(rng.standard_normal(128) * 40)
    vc2, vs2, vm2 = O.quantize_values_per_token(v2, 2)
    other = np.arange(64) != 9
    assert np.array_equal(vc[..., other, :], vc2[..., other, :])
    assert np.array_equal(vs[..., other, :], vs2[..., other, :])
    assert np.array_equal(vm[..., other, :], vm2[..., other, :])


def test_key_axis_ordering_on_outlier_channels():
    """Informational ordering: with fixed outlier key channels, per-channel grouping
    reconstructs keys better than per-token grouping (the geometry page reports this
    ordering for real keys)."""
    import kvq_synth as S
    g = S.key_gains(11, 1, 128, 3, 100.0)
    k = S.gen_tensor(11, S.TID_K, 1, 1, 512, 128, gains=g)
    x = O.f16_to_f32(k).astype(np.float64)
    c1, s1, m1 = O.quantize_keys_per_channel(k, 2)
    e_ch = np.abs(O.dequant_keys_per_channel(c1, s1, m1) - x).mean()
    c2, s2, m2 = O.quantize_keys_per_token(k, 2)
    e_tok = np.abs(O.dequant_values_per_token(c2, s2, m2) - x).mean()
    assert e_ch < e_tok
