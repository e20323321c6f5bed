"""GPU parity of the uniform (KIVI-style) path against the oracle, through the C ABI.

Codes, metadata, window contents and counters must be bit-exact; attention
outputs must satisfy |o - ref| <= 2e-3 + 1e-2 |ref| against the oracle's float64
attention over its own dequantized cache."""
import numpy as np
import pytest

import kvq_synth as S
from oracle import kvq_oracle as O
from tests.kvq_testlib import (assert_close, build_uniform_cache, decode, dev, host_words,
                               oracle_uniform_attention)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("decode_attention_10_amd")


def _kv(seed, B, H, T, D=128, n_out=3, gain=100.0):
    g = S.key_gains(seed, H, D, n_out, gain)
    return (S.gen_tensor(seed, S.TID_K, B, H, T, D, gains=g),
            S.gen_tensor(seed, S.TID_V, B, H, T, D))


@pytest.mark.parametrize("kb,vb", [(2, 2), (4, 2), (2, 4), (4, 4)])
def test_quantize_bit_exact_with_offset_and_strides(kb, vb):
    B, H, T, cap = 2, 3, 192, 224
    k, v = _kv(100 + kb * 10 + vb, B, H, T)
    cache = K.KVCache(B, H, cap, k_bits=kb, v_bits=vb, residual_len=0)
    kd, vd = dev(k), dev(v)
    off, n = 32, 128                     # tokens [32, 160) from the source's tokens [32, 160)
    K.kvq_quantize_keys(cache.c, kd[:, :, off:], H * T * 128, T * 128, 128, off, n)
    K.kvq_quantize_values(cache.c, vd[:, :, off:], H * T * 128, T * 128, 128, off, n)
    kw = host_words(cache.buf("k_codes")).reshape(B, H, cap // 32, 32, 128 * kb // 32)
    km = host_words(cache.buf("k_meta")).reshape(B, H, cap // 32, 128)
    vw = host_words(cache.buf("v_codes")).reshape(B, H, cap // 32, 128 * vb)
    vm = host_words(cache.buf("v_meta")).reshape(B, H, cap, 4)
    kc, ks, kmn = O.quantize_keys_per_channel(k[:, :, off:off + n], kb)
    vc, vs, vmn = O.quantize_values_per_token(v[:, :, off:off + n], vb)
    b0, b1 = off // 32, (off + n) // 32
    assert np.array_equal(kw[:, :, b0:b1], O.pack_k_codes(kc, kb))
    assert np.array_equal(km[:, :, b0:b1], O.pack_meta(ks, kmn))
    assert np.array_equal(vw[:, :, b0:b1], O.pack_v_codes(vc, vb))
    assert np.array_equal(vm[:, :, off:off + n], O.pack_meta(vs, vmn))
    # nothing outside the range was written
    assert not kw[:, :, :b0].any() and not kw[:, :, b1:].any()
    assert not vm[:, :, :off].any() and not vm[:, :, off + n:].any()


def test_quantize_degenerate_groups():
    """Constant groups, signed zeros, tiny and huge ranges, subnormal fp16 inputs."""
    B, H, T = 1, 2, 64
    rng = np.random.default_rng(5)
    x = rng.standard_normal((B, H, T, 128)).astype(np.float32)
    x[0, 0, :32, 5] = 3.25                          # constant key group
    x[0, 0, :32, 6] = -0.0
    x[0, 0, :32, 7] = np.where(np.arange(32) % 2, 0.0, -0.0)
    x[0, 1, 3, :32] = 7.0                           # constant value group
    x[0, 1, 4, :32] = np.linspace(-6e-8, 6e-8, 32)  # fp16 subnormals
    x[0, 1, 5, :] = np.linspace(-65504, 65504, 128)
    x[0, 0, 32:, 9] *= 1e-4
    k = x.astype(np.float16).view(np.uint16)
    cache = K.KVCache(B, H, T, k_bits=2, v_bits=4, residual_len=0)
    kd = dev(k)
    K.kvq_quantize_keys(cache.c, kd, H * T * 128, T * 128, 128, 0, T)
    K.kvq_quantize_values(cache.c, kd, H * T * 128, T * 128, 128, 0, T)
    kc, ks, kmn = O.quantize_keys_per_channel(k, 2)
    vc, vs, vmn = O.quantize_values_per_token(k, 4)
    assert np.array_equal(host_words(cache.buf("k_codes")).reshape(O.pack_k_codes(kc, 2).shape),
                          O.pack_k_codes(kc, 2))
    assert np.array_equal(host_words(cache.buf("k_meta")).reshape(B, H, 2, 128),
                          O.pack_meta(ks, kmn))
    assert np.array_equal(host_words(cache.buf("v_codes")).reshape(O.pack_v_codes(vc, 4).shape),
                          O.pack_v_codes(vc, 4))
    assert np.array_equal(host_words(cache.buf("v_meta")).reshape(B, H, T, 4),
                          O.pack_meta(vs, vmn))


@pytest.mark.parametrize("R,n,kb,vb", [(32, 1, 2, 2), (32, 33, 2, 4), (128, 128, 4, 2),
                                       (128, 129, 2, 2), (128, 300, 4, 4), (64, 200, 2, 2)])
def test_streaming_append_bit_exact(R, n, kb, vb):
    B, H = 2, 2
    k, v = _kv(7 + n, B, H, n)
    cap = ((n + R) // R) * R
    cache = K.KVCache(B, H, cap, k_bits=kb, v_bits=vb, residual_len=R)
    ref = O.StreamingCache(B, H, 128, kb, vb, residual_len=R)
    kd, vd = dev(k), dev(v)
    kstep = [kd[:, :, t].contiguous() for t in range(n)]
    vstep = [vd[:, :, t].contiguous() for t in range(n)]
    for t in range(n):
        K.kvq_append_flush(cache.c, kstep[t], vstep[t])
        ref.append(k[:, :, t], v[:, :, t])
    assert (cache.n_packed, cache.n_resid) == (ref.n_packed, ref.n_resid)
    N = ref.n_packed
    nb = N // 32
    kw = host_words(cache.buf("k_codes")).reshape(B, H, cap // 32, 32, 128 * kb // 32)
    vw = host_words(cache.buf("v_codes")).reshape(B, H, cap // 32, 128 * vb)
    km = host_words(cache.buf("k_meta")).reshape(B, H, cap // 32, 128)
    vm = host_words(cache.buf("v_meta")).reshape(B, H, cap, 4)
    assert np.array_equal(kw[:, :, :nb], O.pack_k_codes(ref.k_codes, kb))
    assert np.array_equal(vw[:, :, :nb], O.pack_v_codes(ref.v_codes, vb))
    assert np.array_equal(km[:, :, :nb], O.pack_meta(ref.k_scale, ref.k_min))
    assert np.array_equal(vm[:, :, :N], O.pack_meta(ref.v_scale, ref.v_min))
    r = ref.n_resid
    kr = cache.buf("k_resid").cpu().numpy().view(np.uint16).reshape(B, H, R, 128)
    vr = cache.buf("v_resid").cpu().numpy().view(np.uint16).reshape(B, H, R, 128)
    assert np.array_equal(kr[:, :, :r], ref.k_res[:, :, :r])
    assert np.array_equal(vr[:, :, :r], ref.v_res[:, :, :r])


DECODE_CASES = [
    # B, Hkv, GQ, n_packed, n_resid, kb, vb, R
    (1, 1, 1, 512, 128, 2, 2, 128),     # the tiny workload's shape
    (2, 2, 1, 0, 1, 2, 2, 128),         # window only, one token
    (1, 2, 2, 32, 0, 4, 2, 128),        # one block, no window
    (2, 2, 4, 1024, 127, 2, 2, 128),
    (1, 1, 8, 4096, 33, 4, 4, 128),
    (3, 2, 1, 96, 128, 2, 4, 128),
    (1, 3, 2, 2048, 1, 4, 2, 64),
    (2, 1, 4, 8192, 0, 2, 2, 0),        # no window at all, many splits
    (1, 4, 1, 160, 1000, 2, 2, 1024),   # long window: 32 chunks
    # grouped queries on the matrix cores: every bit pair, one head per workgroup
    # (heads >= CUs) and split heads with the window in a middle split
    (1, 2, 2, 3072, 77, 4, 4, 128),
    (2, 3, 4, 1536, 128, 4, 4, 128),
    (1, 1, 4, 40960, 100, 2, 2, 128),
    (64, 5, 4, 96, 5, 2, 2, 128),
    (48, 6, 2, 64, 31, 2, 4, 128),
    # one query head per kv head with a workgroup per head (heads >= CUs: 8-wave groups,
    # streaming loads, one block in flight): every bit pair, a window-only cache and
    # mostly idle waves
    (64, 4, 1, 256, 77, 2, 2, 128),
    (32, 8, 1, 1024, 128, 2, 4, 128),
    (20, 16, 1, 512, 5, 4, 2, 128),
    (128, 2, 1, 96, 0, 4, 4, 128),
    (64, 4, 1, 0, 100, 2, 2, 128),
]


@pytest.mark.parametrize("B,Hkv,GQ,N,r,kb,vb,R", DECODE_CASES)
def test_decode_matches_oracle(B, Hkv, GQ, N, r, kb, vb, R):
    seed = 1000 + B * 100 + Hkv * 10 + GQ + N
    k, v = _kv(seed, B, Hkv, N + r)
    q = S.gen_tensor(seed, S.TID_Q, B, Hkv * GQ, 1, 128)[:, :, 0]
    cache = build_uniform_cache(K, k, v, N, r, kb, vb, R, cap=max(32, N + 32))
    sm = O.default_sm_scale(128)
    out, _ = decode(K, cache, q, sm)
    ref, _ = oracle_uniform_attention(k, v, q, N, r, kb, vb, sm)
    assert np.isfinite(out).all()
    assert_close(out, ref, f"decode B{B} Hkv{Hkv} GQ{GQ} N{N} r{r} K{kb}V{vb}")


def test_decode_empty_cache_is_zero():
    cache = K.KVCache(1, 2, 64, residual_len=32)
    q = S.gen_tensor(3, S.TID_Q, 1, 2, 1, 128)[:, :, 0]
    out, _ = decode(K, cache, q, 0.1)
    assert not out.any()


@pytest.mark.parametrize("B,Hkv,GQ,N,r", [(2, 2, 2, 4096, 64), (1, 4, 1, 16384, 64),
                                          (8, 32, 1, 2048, 128)])
def test_decode_workspace_needs_no_initialization_and_repeats(B, Hkv, GQ, N, r):
    """Repeated calls give the same bytes: every plan fixes which wave sums which block,
    so the fp32 sums run in the same order (split plans with one and two query heads per
    kv head, and one workgroup per head with 8 blocks per wave)."""
    k, v = _kv(77, B, Hkv, N + r)
    q = S.gen_tensor(77, S.TID_Q, B, Hkv * GQ, 1, 128)[:, :, 0]
    cache = build_uniform_cache(K, k, v, N, r, 2, 2, 128, cap=N)
    out1, ws = decode(K, cache, q, 0.09)
    ref, _ = oracle_uniform_attention(k, v, q, N, r, 2, 2, 0.09)
    assert_close(out1, ref, "first call")
    ws.fill_(0xFF)                                # garbage (NaN patterns) in the workspace
    qd = dev(q)
    out2 = torch.empty_like(torch.from_numpy(out1)).cuda()
    K.kvq_decode_attn(cache.c, qd, Hkv * GQ, 0.09, 0.0, out2, ws, ws.numel())
    torch.cuda.synchronize()
    assert np.array_equal(out1, out2.cpu().numpy())   # same plan, same arithmetic order


# ---- attention-sink window: the sequence's first tokens kept in fp16 for good
# ("The KV cache has a geometry problem", section on where research goes)
@pytest.mark.parametrize("S_len,R,n,kb,vb", [(4, 32, 3, 2, 2), (4, 32, 40, 2, 4),
                                             (32, 128, 300, 4, 2), (7, 64, 200, 2, 2)])
def test_streaming_append_with_sink_bit_exact(S_len, R, n, kb, vb):
    B, H = 2, 2
    k, v = _kv(70 + n, B, H, n)
    cap = max(32, ((n + R) // R) * R)
    cache = K.KVCache(B, H, cap, k_bits=kb, v_bits=vb, residual_len=R, sink_len=S_len)
    ref = O.StreamingCache(B, H, 128, kb, vb, residual_len=R, sink_len=S_len)
    kd, vd = dev(k), dev(v)
    for t in range(n):
        K.kvq_append_flush(cache.c, kd[:, :, t].contiguous(), vd[:, :, t].contiguous())
        ref.append(k[:, :, t], v[:, :, t])
    assert (cache.n_sink, cache.n_packed, cache.n_resid) == (ref.n_sink, ref.n_packed,
                                                              ref.n_resid)
    ns, N, r = ref.n_sink, ref.n_packed, ref.n_resid
    ks = cache.buf("k_sink").cpu().numpy().view(np.uint16).reshape(B, H, S_len, 128)
    vs = cache.buf("v_sink").cpu().numpy().view(np.uint16).reshape(B, H, S_len, 128)
    assert np.array_equal(ks[:, :, :ns], ref.k_sink[:, :, :ns])
    assert np.array_equal(vs[:, :, :ns], ref.v_sink[:, :, :ns])
    nb = N // 32
    kw = host_words(cache.buf("k_codes")).reshape(B, H, cap // 32, 32, 128 * kb // 32)
    vw = host_words(cache.buf("v_codes")).reshape(B, H, cap // 32, 128 * vb)
    vm = host_words(cache.buf("v_meta")).reshape(B, H, cap, 4)
    assert np.array_equal(kw[:, :, :nb], O.pack_k_codes(ref.k_codes, kb))
    assert np.array_equal(vw[:, :, :nb], O.pack_v_codes(ref.v_codes, vb))
    assert np.array_equal(vm[:, :, :N], O.pack_meta(ref.v_scale, ref.v_min))
    kr = cache.buf("k_resid").cpu().numpy().view(np.uint16).reshape(B, H, R, 128)
    assert np.array_equal(kr[:, :, :r], ref.k_res[:, :, :r])


SINK_CASES = [
    # B, Hkv, GQ, n_sink, sink_len, n_packed, n_resid, kb, vb, R
    (1, 2, 1, 4, 4, 512, 77, 2, 2, 128),        # vector kernel, split contexts
    (2, 2, 1, 100, 128, 1024, 0, 4, 2, 128),    # ragged sink chunk, no window
    (1, 2, 2, 32, 32, 3072, 5, 2, 2, 128),      # matrix-core kernel
    (1, 1, 4, 7, 16, 40960, 100, 2, 2, 128),    # matrix-core kernel, many splits
    (3, 1, 8, 20, 32, 96, 31, 2, 4, 64),        # 8 query heads per kv head
    (1, 1, 1, 30, 32, 0, 0, 2, 2, 32),          # sink only
    (2, 3, 1, 32, 32, 0, 17, 2, 2, 32),         # sink and window, nothing packed
    (64, 5, 4, 3, 4, 96, 5, 2, 2, 128),         # one head per workgroup
]


@pytest.mark.parametrize("B,Hkv,GQ,ns,S_len,N,r,kb,vb,R", SINK_CASES)
def test_decode_with_sink_matches_oracle(B, Hkv, GQ, ns, S_len, N, r, kb, vb, R):
    seed = 3000 + B * 100 + Hkv * 10 + GQ + N + ns
    k, v = _kv(seed, B, Hkv, ns + N + r)
    q = S.gen_tensor(seed, S.TID_Q, B, Hkv * GQ, 1, 128)[:, :, 0]
    cache = build_uniform_cache(K, k, v, N, r, kb, vb, R, cap=max(32, N + 32), n_sink=ns,
                                sink_len=S_len)
    sm = O.default_sm_scale(128)
    out, _ = decode(K, cache, q, sm)
    ref, _ = oracle_uniform_attention(k, v, q, N, r, kb, vb, sm, n_sink=ns)
    assert np.isfinite(out).all()
    assert_close(out, ref, f"sink decode B{B} Hkv{Hkv} GQ{GQ} sink{ns} N{N} r{r} K{kb}V{vb}")
