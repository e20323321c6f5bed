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
