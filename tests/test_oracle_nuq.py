"""Pins of the oracle's non-uniform datatype and dense-and-sparse outliers (KVQuant
review: abstract items (iii) and (iv), "Proposed method").

- With the identity code book {0..7} the nuq3 quantizer is the uniform 3-bit
  quantizer, bit for bit (the normalization reading).
- Every element maps to the nearest code-book level (brute force).
- Outliers: exactly k per vector, all at least as large in magnitude as every
  dense entry, ties broken towards lower indices, kept exactly; none with bp = 0.
"""
import numpy as np
import pytest

import kvq_synth as S
from oracle import kvq_oracle as O

IDENT = np.arange(8).astype(np.float16).view(np.uint16)


def _f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def test_outlier_count_rounds_up():
    assert O.outlier_count(1048576, 100) == 10486
    assert O.outlier_count(100, 100) == 1
    assert O.outlier_count(101, 100) == 2
    assert O.outlier_count(4096, 0) == 0
    assert O.outlier_count(128, 100) == 2


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_identity_lut_equals_uniform_3bit(seed):
    rng = np.random.default_rng(seed)
    x = _f16(rng.standard_normal(512) * rng.uniform(0.1, 30))
    c, s, m, oi, xh = O.nuq_quantize_vector(x, IDENT, 0)
    cu, su, mu = O.uniform_quantize_groups(x[None], 3)
    assert np.array_equal(c, cu[0]) and s == su[0] and m == mu[0]
    assert np.array_equal(xh, O.uniform_dequant(cu, su, mu)[0])
    assert oi.size == 0


def test_identity_lut_values_per_token():
    v = S.gen_tensor(4, S.TID_V, 1, 1, 64, 128)[0, 0]
    c, s, m, xh = O.nuq_quantize_values(v, IDENT)
    cu, su, mu = O.uniform_quantize_groups(v, 3)
    assert np.array_equal(c, cu) and np.array_equal(s, su) and np.array_equal(m, mu)


def test_nearest_level_brute_force():
    lut = S.nuq3_lut()
    L = O.f16_to_f32(lut).astype(np.float64)
    rng = np.random.default_rng(9)
    x = _f16(rng.standard_normal(4000) * 2)
    c, s, m, oi, xh = O.nuq_quantize_vector(x, lut, 0)
    sf, mf = float(O.f16_to_f32(s)), float(O.f16_to_f32(m))
    xn = (O.f16_to_f32(x).astype(np.float64) - mf) / sf
    d = np.abs(xn[:, None] - L[None, :])
    best = d.argmin(1)
    dc = d[np.arange(len(c)), c]
    assert np.all((c == best) | (np.abs(dc - d.min(1)) <= 1e-5))
    assert np.mean(c == best) > 0.999


def test_ties_go_to_even_index():
    lut = _f16([0, 1, 2, 3, 4, 5, 6, 7])
    # min 0, max 7 -> scale 1; 2.5 is a tie between levels 2 and 3 -> 2; 3.5 -> 4
    x = _f16([0, 7, 2.5, 3.5, 6.5, 0.5])
    c, *_ = O.nuq_quantize_vector(x, lut, 0)
    assert list(c[2:]) == [2, 4, 6, 0]


def test_outliers_largest_magnitudes_ties_to_lower_index():
    x = np.zeros(200)
    x[:] = np.linspace(-1, 1, 200)
    x[[3, 50, 120]] = [9.0, -9.0, 9.0]     # three equal magnitudes: tie
    x[77] = -20.0
    xb = _f16(x)
    c, s, m, oi, xh = O.nuq_quantize_vector(xb, S.nuq3_lut(), 3)
    assert list(oi) == [3, 50, 77]
    assert np.array_equal(xh[oi], O.f16_to_f32(xb)[oi])


@pytest.mark.parametrize("bp", [0, 100, 250])
def test_outlier_invariants_keys(bp):
    B, H, N, D = 1, 1, 640, 128
    k = S.gen_tensor(12, S.TID_K, B, H, N, D, gains=S.key_gains(12, H, D, 3, 100.0))[0, 0]
    lut = S.nuq3_lut()
    codes, sc, mn, rp, ent, xh = O.nuq_quantize_keys(k, lut, bp)
    kk = O.outlier_count(N, bp)
    assert rp[0] == 0 and rp[-1] == D * kk and np.all(np.diff(rp) >= 0)
    cols = (ent & 0xFF).astype(np.int64)
    vals = (ent >> 16).astype(np.uint16)
    rows = np.repeat(np.arange(N), np.diff(rp))
    assert np.array_equal(vals, k[rows, cols])                  # exact fp16 values
    assert np.array_equal((ent >> 8) & 0xFF, rows % 32)         # token within its block
    for t in range(N):                                          # columns ascending per row
        seg = cols[rp[t]:rp[t + 1]]
        assert np.all(np.diff(seg) > 0)
    mag = (k & 0x7FFF).astype(np.int64)
    is_out = np.zeros((N, D), bool)
    is_out[rows, cols] = True
    for d in range(D):
        assert is_out[:, d].sum() == kk
        if kk:
            assert mag[is_out[:, d], d].min() >= mag[~is_out[:, d], d].max()
            # dense min/max exclude outliers
            xd = O.f16_to_f32(k[~is_out[:, d], d])
            assert O.f16_to_f32(mn[d]) == xd.min() + np.float32(0)
    x = O.f16_to_f32(k)
    assert np.array_equal(xh[is_out], x[is_out])
    assert not codes[is_out].any()                              # outlier positions: code 0
    if bp == 0:
        c0, s0, m0, _, xh0 = O.nuq_quantize_vector(k[:, 5], lut, 0)
        assert np.array_equal(codes[:, 5], c0) and sc[5] == s0


def test_all_outliers_degenerate():
    x = _f16([1.0, -2.0, 3.0])
    c, s, m, oi, xh = O.nuq_quantize_vector(x, S.nuq3_lut(), 3)
    assert s == 0 and m == 0 and not c.any()
    assert np.array_equal(xh, O.f16_to_f32(x))


def test_nuq_head_identity_lut_no_outliers_is_per_channel_int3_over_context():
    """With the identity code book, no outliers and no RoPE, a head's keys are the uniform
    3-bit quantizer applied to each channel over the whole context."""
    k = S.gen_tensor(31, S.TID_K, 1, 1, 96, 128)[0, 0]
    v = S.gen_tensor(31, S.TID_V, 1, 1, 96, 128)[0, 0]
    h = O.nuq_head(k, v, IDENT, IDENT, 0, 64, 32, 0.0)
    cu, su, mu = O.uniform_quantize_groups(k[:64].T, 3)      # groups = channels over tokens
    assert np.allclose(h["k_hat"][:64], O.uniform_dequant(cu, su, mu).T)
    assert np.array_equal(h["k_hat"][64:], O.f16_to_f32(k[64:]))


def test_rope_query_rounds_rotation():
    q = S.gen_tensor(2, S.TID_Q, 1, 2, 1, 128)[:, :, 0]
    r = O.rope_query_f16(q, 1000, 1e4)
    ref = O.rope_f64(O.f16_to_f32(q).astype(np.float64)[0][:, None, :], np.array([1000]), 1e4)
    assert np.array_equal(r[0], O.f32_to_f16_bits(ref[:, 0, :].astype(np.float32)))
    assert np.array_equal(O.rope_query_f16(q, 0, 1e4), q)


# ---- dense-and-sparse values: outliers isolated for each token's vector (KVQuant review,
# abstract item (iv)); the table's "-1%" rows keep 1 % of each vector exactly.
@pytest.mark.parametrize("bp", [100, 250, 1000])
def test_outlier_invariants_values(bp):
    N, D = 96, 128
    v = S.gen_tensor(14, S.TID_V, 1, 1, N, D)[0, 0].copy()
    v[5, 17] = _f16(300.0)                        # a clear outlier channel in token 5
    v[9, 3] = v[9, 100] = _f16(-64.0)             # a tie: both kept when k >= 2
    lut = S.nuq3_lut()
    codes, sc, mn, ent, xh = O.nuq_quantize_values(v, lut, bp)
    kk = O.outlier_count(D, bp)
    assert ent.shape == (N, kk)
    cols = (ent & 0xFFFF).astype(np.int64)
    assert np.all(np.diff(cols, axis=1) > 0)                     # ascending, distinct
    assert np.array_equal((ent >> 16).astype(np.uint16), np.take_along_axis(v, cols, 1))
    mag = (v & 0x7FFF).astype(np.int64)
    x = O.f16_to_f32(v)
    for t in range(N):
        out = np.zeros(D, bool)
        out[cols[t]] = True
        assert mag[t, out].min() >= mag[t, ~out].max()
        # ties at the threshold go to the lower channels
        thr = mag[t, out].min()
        tied = np.nonzero(mag[t] == thr)[0]
        assert np.array_equal(out[tied], np.arange(len(tied)) < out[tied].sum())
        assert O.f16_to_f32(mn[t]) == x[t, ~out].min() + np.float32(0)
        assert np.array_equal(xh[t, out], x[t, out])
    assert 17 in cols[5] and {3, 100} <= set(cols[9])
    # without outliers the dense path is the per-token quantizer already pinned
    c0, s0, m0, xh0 = O.nuq_quantize_values(v, lut)
    assert O.f16_to_f32(m0[5]) <= O.f16_to_f32(mn[5])


def test_value_outliers_by_hand():
    """Token [1, 2, 9, 3] with one outlier: 9 is kept; the dense range is [1, 3], so the
    scale is 2/7 and the min 1 (identity code book: levels 0..7)."""
    v = _f16([[1.0, 2.0, 9.0, 3.0]])
    codes, sc, mn, ent, xh = O.nuq_quantize_values(v, IDENT, 2500)
    assert ent.shape == (1, 1) and ent[0, 0] == (2 | (int(_f16(9.0)) << 16))
    assert O.f16_to_f32(mn[0]) == 1.0
    assert sc[0] == _f16(2.0 / 7.0)
    assert xh[0, 2] == 9.0
    s = O.f16_to_f32(sc[0])
    assert np.array_equal(codes[0, [0, 1, 3]], np.rint((np.float32([1, 2, 3]) - 1) / s))
    assert codes[0, 2] == 0                       # an outlier's position stores code 0


def test_nuq_head_value_outliers_change_only_the_outlier_values():
    """Attention reads the exact value at every value outlier."""
    rng = np.random.default_rng(4)
    x = O.f32_to_f16_bits(rng.standard_normal((64, 128)).astype(np.float32))
    h = O.nuq_head(x, x, S.nuq3_lut(), S.nuq3_lut(), 100, 64, 0, 0.0, v_outlier_bp=100)
    cols = (h["v_ent"] & 0xFFFF).astype(np.int64)
    rows = np.repeat(np.arange(64), cols.shape[1])
    assert np.array_equal(h["v_hat"][rows, cols.ravel()], O.f16_to_f32(x)[rows, cols.ravel()])


@pytest.mark.parametrize("bits", [2, 4])
def test_identity_lut_equals_uniform_at_other_widths(bits):
    """nuq2 / nuq4 with the identity code book {0 .. 2^B - 1} are the uniform B-bit
    quantizer, per vector and per token, bit for bit."""
    ident = np.arange(1 << bits).astype(np.float16).view(np.uint16)
    rng = np.random.default_rng(bits)
    x = _f16(rng.standard_normal(256) * 7.0)
    c, s, m, oi, xh = O.nuq_quantize_vector(x, ident, 0)
    cu, su, mu = O.uniform_quantize_groups(x[None], bits)
    assert np.array_equal(c, cu[0]) and s == su[0] and m == mu[0]
    v = S.gen_tensor(6, S.TID_V, 1, 1, 32, 128)[0, 0]
    c, s, m, xh = O.nuq_quantize_values(v, ident)
    cu, su, mu = O.uniform_quantize_groups(v, bits)
    assert np.array_equal(c, cu) and np.array_equal(s, su) and np.array_equal(m, mu)


@pytest.mark.parametrize("bits", [2, 4])
def test_code_books_of_other_widths(bits):
    """The stand-in code books: 2^B ascending levels from 0 to 2^B - 1, symmetric about the
    middle (normal quantiles)."""
    lut = O.f16_to_f32(S.nuq_lut(bits))
    n = 1 << bits
    assert lut.shape == (n,) and lut[0] == 0 and lut[-1] == n - 1
    assert np.all(np.diff(lut) > 0)
    np.testing.assert_allclose(lut + lut[::-1], n - 1, atol=0.01)


# ---- Q-Norm (KVQuant review, "Proposed method" and findings: the dequantized distribution
# is matched to the statistics before quantization; it helps most at 2 bits).
@pytest.mark.parametrize("bits,bp", [(2, 0), (2, 100), (3, 100), (4, 0)])
def test_qnorm_matches_mean_and_std(bits, bp):
    rng = np.random.default_rng(30 + bits)
    x = _f16(rng.standard_normal(4096) * 3.0 + 1.5)
    lut = S.nuq_lut(bits)
    k = O.outlier_count(4096, bp)
    c0, s0, m0, oi0, xh0 = O.nuq_quantize_vector(x, lut, k)
    c, s, m, oi, xh = O.nuq_quantize_vector(x, lut, k, qnorm=True)
    assert np.array_equal(c, c0) and np.array_equal(oi, oi0)     # codes and outliers unchanged
    dense = np.ones(4096, bool)
    dense[oi] = False
    xf = O.f16_to_f32(x)[dense].astype(np.float64)
    got = xh[dense].astype(np.float64)
    # the fp16 metadata round a and b: the moments match to within that rounding
    assert abs(got.mean() - xf.mean()) <= 2e-3 * xf.std()
    assert abs(got.std() / xf.std() - 1.0) <= 2e-3
    # and plain dequantization does not match them as closely at 2 bits
    if bits == 2:
        assert abs(xh0[dense].std() / xf.std() - 1.0) > 5e-3
    assert np.array_equal(xh[oi], O.f16_to_f32(x)[oi])


def test_qnorm_by_hand():
    """x = [0, 0, 3, 3] with the identity 2-bit code book: codes [0, 0, 3, 3], x_hat = x,
    so a = 1, b = 0 and the metadata stay.  x = [0, 1, 1, 3]: scale 1, codes [0, 1, 1, 3],
    again exact.  A constant vector has var_hat = 0: a = 1 and b = 0."""
    ident = np.arange(4).astype(np.float16).view(np.uint16)
    for vals in ([0.0, 0.0, 3.0, 3.0], [0.0, 1.0, 1.0, 3.0]):
        x = _f16(vals)
        a = O.nuq_quantize_vector(x, ident, 0)
        b = O.nuq_quantize_vector(x, ident, 0, qnorm=True)
        assert a[1] == b[1] and a[2] == b[2] and np.array_equal(b[4], O.f16_to_f32(x))
    x = _f16([2.0, 2.0, 2.0])
    c, s, m, oi, xh = O.nuq_quantize_vector(x, ident, 0, qnorm=True)
    assert s == 0 and O.f16_to_f32(m) == 2.0 and np.array_equal(xh, [2.0, 2.0, 2.0])


def test_qnorm_on_keys_and_values_of_a_head():
    k = S.gen_tensor(8, S.TID_K, 1, 1, 256, 128)[0, 0]
    lut = S.nuq_lut(2)
    h0 = O.nuq_head(k, k, lut, lut, 100, 256, 0, 0.0)
    h1 = O.nuq_head(k, k, lut, lut, 100, 256, 0, 0.0, qnorm=True)
    assert np.array_equal(h0["k_codes"], h1["k_codes"])
    assert np.array_equal(h0["v_codes"], h1["v_codes"])
    assert not np.array_equal(h0["k_meta"], h1["k_meta"])
    # per key channel: dequantized std within 0.5 % of the original's after Q-Norm
    x = O.f16_to_f32(k).astype(np.float64)
    r0 = np.abs(h0["k_hat"].std(0) / x.std(0) - 1).mean()
    r1 = np.abs(h1["k_hat"].std(0) / x.std(0) - 1).mean()
    assert r1 < r0 and r1 < 5e-3


def _exact_sum(vals) -> float:
    """The exact rational sum of float values, rounded once to float64 (Fraction -> float
    is correctly rounded): an independent route to the definition."""
    from fractions import Fraction
    return float(sum((Fraction(float(v)) for v in vals), Fraction(0)))


def test_exact_moments_are_correctly_rounded_sums():
    """Q-Norm's sum x and sum x^2 are the exact sums rounded once.  The vector mixes one
    large value with many fp16 subnormals, so that adding x^2 left to right and numpy's
    pairwise sum give different float64 results; the oracle must give the exact one."""
    big = _f16([256.0, -96.0])
    tiny = np.full(4096, 1, np.uint16)                 # 2^-24 each (smallest subnormal)
    x_bits = np.concatenate([big, tiny, _f16(np.linspace(-3.0, 3.0, 1001))])
    x = O.f16_to_f32(x_bits).astype(np.float64)
    sq = (x * x)
    seq = 0.0
    for v in sq.tolist():
        seq += v
    exact_sq = _exact_sum(sq.tolist())
    assert seq != exact_sq                             # the order matters for this vector
    mean, var = O.exact_moments(O.f16_to_f32(x_bits))
    n = len(x)
    assert mean == _exact_sum(x.tolist()) / n
    assert var == max(exact_sq / n - mean * mean, 0.0)


def test_exact_moments_ignore_the_order():
    """Permuting the entries leaves the moments (and so the Q-Norm metadata) bit for bit
    unchanged, on vectors whose naive float64 sums of x^2 depend on the order."""
    rng = np.random.default_rng(77)
    mags = np.exp2(rng.integers(-24, 15, 5000).astype(np.float64)) * rng.uniform(1, 2, 5000)
    x_bits = _f16(mags * np.where(rng.random(5000) < 0.5, -1.0, 1.0))
    x = O.f16_to_f32(x_bits)
    naive = set()
    ref = O.exact_moments(x)
    lut = S.nuq_lut(2)
    meta0 = O.nuq_quantize_vector(x_bits, lut, 50, qnorm=True)[1:3]
    for i in range(6):
        p = rng.permutation(len(x))
        acc = 0.0
        for v in (x[p].astype(np.float64) ** 2).tolist():     # left to right
            acc += v
        naive.add(acc)
        assert O.exact_moments(x[p]) == ref
        assert O.nuq_quantize_vector(x_bits[p], lut, 50, qnorm=True)[1:3] == meta0
    assert len(naive) > 1                              # a naive sum would not be stable
