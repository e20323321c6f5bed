"""Pins of the oracle's streaming cache: a token is appended, the newest tokens stay in
fp16, and a full window is quantized as a group ("The KV cache has a geometry
problem", section "The systems tax"; KIVI post, "Method").

Streaming n tokens from empty must equal one-shot quantization of the same
tokens, bit for bit, with the window holding the rest."""
import numpy as np
import pytest

import kvq_synth as S
from oracle import kvq_oracle as O


@pytest.mark.parametrize("R", [32, 128])
@pytest.mark.parametrize("n", [1, 31, 32, 33, 127, 128, 129, 300, 640])
def test_streaming_equals_one_shot(R, n):
    B, H, D = 2, 2, 64
    k = S.gen_tensor(21, S.TID_K, B, H, n, D, gains=S.key_gains(21, H, D, 2, 50.0))
    v = S.gen_tensor(21, S.TID_V, B, H, n, D)
    sc = O.StreamingCache(B, H, D, 2, 4, residual_len=R)
    for t in range(n):
        sc.append(k[:, :, t], v[:, :, t])
    r = (n - 1) % R + 1
    N = n - r
    assert (sc.n_packed, sc.n_resid) == (N, r)
    kc, ks, km = O.quantize_keys_per_channel(k[:, :, :N], 2)
    vc, vs, vm = O.quantize_values_per_token(v[:, :, :N], 4)
    assert np.array_equal(sc.k_codes, kc) and np.array_equal(sc.v_codes, vc)
    assert np.array_equal(sc.k_scale, ks) and np.array_equal(sc.k_min, km)
    assert np.array_equal(sc.v_scale, vs) and np.array_equal(sc.v_min, vm)
    assert np.array_equal(sc.k_res[:, :, :r], k[:, :, N:])
    assert np.array_equal(sc.v_res[:, :, :r], v[:, :, N:])


def test_window_semantics_of_tiny_workload():
    """512 packed + 128 fp16 tokens is the state after streaming 640 tokens with R = 128."""
    sc = O.StreamingCache(1, 1, 32, 2, 2, residual_len=128)
    z = np.zeros((1, 1, 32), np.uint16)
    for _ in range(640):
        sc.append(z, z)
    assert (sc.n_packed, sc.n_resid) == (512, 128)
    sc.append(z, z)
    assert (sc.n_packed, sc.n_resid) == (640, 1)


def test_dequant_window_is_fp16_exact():
    B, H, D, n = 1, 1, 32, 70
    k = S.gen_tensor(3, S.TID_K, B, H, n, D)
    v = S.gen_tensor(3, S.TID_V, B, H, n, D)
    sc = O.StreamingCache(B, H, D, 2, 2, residual_len=32)
    for t in range(n):
        sc.append(k[:, :, t], v[:, :, t])
    kd, vd = sc.dequant()
    assert kd.shape == (1, 1, n, D)
    assert np.array_equal(kd[:, :, 64:], O.f16_to_f32(k[:, :, 64:]))
    assert np.array_equal(vd[:, :, 64:], O.f16_to_f32(v[:, :, 64:]))


# ---- attention-sink window ("The KV cache has a geometry problem", section on where
# research goes: InnerQ keeps full-precision windows for the recent tokens and for the
# attention-sink tokens).  Reading: the sink is the sequence's first sink_len tokens,
# filled before anything else and never quantized; token order is sink, packed, window.
@pytest.mark.parametrize("S_len,R,n", [(4, 32, 3), (4, 32, 4), (4, 32, 5), (4, 32, 37),
                                       (4, 32, 100), (32, 128, 300), (7, 64, 200)])
def test_streaming_with_sink_equals_one_shot(S_len, R, n):
    B, H, D = 2, 2, 64
    k = S.gen_tensor(41, S.TID_K, B, H, n, D, gains=S.key_gains(41, H, D, 2, 50.0))
    v = S.gen_tensor(41, S.TID_V, B, H, n, D)
    sc = O.StreamingCache(B, H, D, 2, 4, residual_len=R, sink_len=S_len)
    for t in range(n):
        sc.append(k[:, :, t], v[:, :, t])
    ns = min(n, S_len)
    rest = n - ns
    r = (rest - 1) % R + 1 if rest else 0
    N = rest - r
    assert (sc.n_sink, sc.n_packed, sc.n_resid) == (ns, N, r)
    # the sink holds the first tokens exactly and takes no part in the quantizer
    assert np.array_equal(sc.k_sink[:, :, :ns], k[:, :, :ns])
    assert np.array_equal(sc.v_sink[:, :, :ns], v[:, :, :ns])
    kc, ks, km = O.quantize_keys_per_channel(k[:, :, ns:ns + N], 2)
    vc, vs, vm = O.quantize_values_per_token(v[:, :, ns:ns + N], 4)
    assert np.array_equal(sc.k_codes, kc) and np.array_equal(sc.v_codes, vc)
    assert np.array_equal(sc.k_scale, ks) and np.array_equal(sc.v_min, vm)
    one = O.uniform_cache(k, v, 2, 4, N, r, n_sink=ns)
    kd, vd = sc.dequant()
    assert np.array_equal(kd, one["k_hat"]) and np.array_equal(vd, one["v_hat"])
    assert np.array_equal(kd[:, :, :ns], O.f16_to_f32(k[:, :, :ns]))


def test_sink_only_cache_is_fp16_attention():
    """Every token in the sink: attention over the exact fp16 keys and values."""
    torch = pytest.importorskip("torch")
    B, H, D, n = 1, 2, 64, 24
    k = S.gen_tensor(5, S.TID_K, B, H, n, D)
    v = S.gen_tensor(5, S.TID_V, B, H, n, D)
    q = S.gen_tensor(5, S.TID_Q, B, H, 1, D)[:, :, 0]
    sc = O.StreamingCache(B, H, D, 2, 2, residual_len=32, sink_len=32)
    for t in range(n):
        sc.append(k[:, :, t], v[:, :, t])
    assert (sc.n_sink, sc.n_packed, sc.n_resid) == (n, 0, 0)
    kd, vd = sc.dequant()
    out = O.decode_attention_f64(O.f16_to_f32(q), kd, vd, 0.125)
    qt = torch.from_numpy(O.f16_to_f32(q).astype(np.float64))[:, :, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(O.f16_to_f32(k).astype(np.float64)),
        torch.from_numpy(O.f16_to_f32(v).astype(np.float64)), scale=0.125)[:, :, 0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-6, atol=1e-7)


def test_nuq_sink_shifts_rotation_positions_by_its_length():
    """With a sink of S tokens the packed keys sit at positions S.. : rotating the no-sink
    result by S more positions (R(a + b) = R(b) R(a)) gives the same keys."""
    rng = np.random.default_rng(2)
    D, Sn, N, r, theta = 32, 5, 64, 3, 1e4
    x = O.f32_to_f16_bits(rng.standard_normal((Sn + N + r, D)).astype(np.float32))
    lut = O.f32_to_f16_bits(np.arange(8, dtype=np.float32))
    with_sink = O.nuq_head(x, x, lut, lut, 100, N, r, theta, n_sink=Sn)
    plain = O.nuq_head(x[Sn:], x[Sn:], lut, lut, 100, N, r, 0.0)
    shifted = O.rope_f64(plain["k_hat"], np.arange(N + r) + Sn, theta)
    np.testing.assert_allclose(with_sink["k_hat"][Sn:], shifted, rtol=0, atol=1e-9)
    assert np.array_equal(with_sink["ent"], plain["ent"])          # statistics skip the sink
    np.testing.assert_allclose(with_sink["k_hat"][:Sn],
                               O.rope_f64(O.f16_to_f32(x[:Sn]), np.arange(Sn), theta),
                               rtol=0, atol=1e-12)
