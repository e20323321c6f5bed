"""Pins of the oracle's RoPE and decode attention.

RoPE is applied to keys after dequantization ("The KV cache has a geometry
problem", section on rotary embeddings; KVQuant review, abstract item (ii)).
Attention is textbook scaled dot-product attention over the whole cache; the
pins are a library routine (torch's CPU scaled_dot_product_attention in
float64), closed forms and special cases.
"""
import numpy as np
import pytest
import torch

import kvq_synth as S
from oracle import kvq_oracle as O


# ---- RoPE --------------------------------------------------------------------
def test_rope_identity_at_zero_and_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 128))
    assert np.array_equal(O.rope_f64(x[:1], np.array([0]), 1e4), x[:1])
    y = O.rope_f64(x, np.array([1, 7, 1000, 65535, 1048575]), 1e4)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_matches_complex_rotation():
    """Pair (2i, 2i+1) as a complex number times exp(i t theta^(-2i/D))."""
    rng = np.random.default_rng(1)
    D = 16
    x = rng.standard_normal((3, D))
    pos = np.array([2, 33, 999])
    z = x[:, 0::2] + 1j * x[:, 1::2]
    freq = 1e4 ** (-np.arange(D // 2) * 2.0 / D)
    zr = z * np.exp(1j * pos[:, None] * freq[None, :])
    y = O.rope_f64(x, pos, 1e4)
    assert np.allclose(y[:, 0::2], zr.real, atol=1e-12)
    assert np.allclose(y[:, 1::2], zr.imag, atol=1e-12)


def test_rope_unit_vector_by_hand():
    e2 = np.zeros((1, 4))
    e2[0, 2] = 1.0
    y = O.rope_f64(e2, np.array([1]), 100.0)          # freq_1 = 100^(-1/2) = 0.1
    assert np.allclose(y[0], [0, 0, np.cos(0.1), np.sin(0.1)], atol=1e-15)


def test_rope_scores_depend_on_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    s0 = O.rope_f64(q, np.array([50]), 1e4) @ O.rope_f64(k, np.array([20]), 1e4).T
    s1 = O.rope_f64(q, np.array([50 + 777]), 1e4) @ O.rope_f64(k, np.array([20 + 777]), 1e4).T
    assert abs(s0 - s1).max() < 1e-9


# ---- attention ---------------------------------------------------------------
def _sdpa(q, k, v, scale):
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    kt = torch.from_numpy(np.asarray(k, np.float64))
    vt = torch.from_numpy(np.asarray(v, np.float64))
    hq, hkv = qt.shape[1], kt.shape[1]
    kt = kt.repeat_interleave(hq // hkv, dim=1)
    vt = vt.repeat_interleave(hq // hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[:, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,T", [(1, 1, 1), (2, 2, 37), (8, 2, 100), (4, 1, 300)])
def test_attention_matches_torch_sdpa(hq, hkv, T):
    rng = np.random.default_rng(hq * 100 + T)
    q = rng.standard_normal((2, hq, 64))
    k = rng.standard_normal((2, hkv, T, 64)) * 3
    v = rng.standard_normal((2, hkv, T, 64))
    sc = O.default_sm_scale(64)
    o = O.decode_attention_f64(q, k, v, sc)
    assert o.dtype == np.float32
    assert np.allclose(o, _sdpa(q, k, v, sc), rtol=1e-6, atol=1e-7)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 1, 9, 32))
    k = rng.standard_normal((1, 1, 9, 32))
    # one token -> its value
    o1 = O.decode_attention_f64(rng.standard_normal((1, 1, 32)), k[:, :, :1], v[:, :, :1], 0.3)
    assert np.allclose(o1[0, 0], v[0, 0, 0])
    # zero query -> equal scores -> mean of values
    o2 = O.decode_attention_f64(np.zeros((1, 1, 32)), k, v, 0.3)
    assert np.allclose(o2[0, 0], v[0, 0].mean(0), atol=1e-7)
    # GQA equals MHA over replicated kv heads
    q = rng.standard_normal((1, 4, 32))
    og = O.decode_attention_f64(q, k, v, 0.2)
    om = O.decode_attention_f64(q, np.repeat(k, 4, 1), np.repeat(v, 4, 1), 0.2)
    assert np.array_equal(og, om)


def test_uniform_cache_attention_with_only_window_is_fp16_attention():
    """n_packed = 0: attention runs on the fp16 window alone."""
    w = S.WORKLOADS["tiny"]
    k = S.gen_tensor(w.seed, S.TID_K, 1, 1, 64, 128, gains=w.gains())
    v = S.gen_tensor(w.seed, S.TID_V, 1, 1, 64, 128)
    q = S.gen_tensor(w.seed, S.TID_Q, 1, 1, 1, 128)[:, :, 0]
    c = O.uniform_cache(k, v, 2, 2, 0, 64)
    o = O.decode_attention_f64(O.f16_to_f32(q), c["k_hat"], c["v_hat"], 0.125)
    ref = _sdpa(O.f16_to_f32(q), O.f16_to_f32(k), O.f16_to_f32(v), 0.125)
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-7)
