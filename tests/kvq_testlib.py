"""Helpers shared by the GPU tests: moving synthetic inputs to the device, building a
cache through the library, and computing the oracle's answer for the same inputs."""
from __future__ import annotations

import numpy as np

import kvq_synth as S
from oracle import kvq_oracle as O

TOL_ABS, TOL_REL = 2e-3, 1e-2     # attention output gate: |o - ref| <= abs + rel * |ref|


def dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_words(t) -> np.ndarray:
    """A device byte buffer as little-endian uint32 words on the host."""
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint32)


def assert_close(o: np.ndarray, ref: np.ndarray, what: str = ""):
    err = np.abs(o.astype(np.float64) - ref.astype(np.float64))
    bound = TOL_ABS + TOL_REL * np.abs(ref.astype(np.float64))
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                           f"max abs err {err.max():.3e}, worst err/bound {(err / bound).max():.3f}")
    return float(err.max())


def build_uniform_cache(K, k: np.ndarray, v: np.ndarray, n_packed: int, n_resid: int,
                        kb: int, vb: int, R: int, cap: int | None = None, n_sink: int = 0,
                        sink_len: int = 0):
    """Copy tokens [0, n_sink) of host K/V ([B][H][T][D] fp16 bits) into the sink, quantize
    the next n_packed tokens on the GPU and copy the n_resid after them into the window.
    Returns the KVCache."""
    import torch
    B, H, T, D = k.shape
    cap = cap if cap is not None else max(32, n_packed)
    cache = K.KVCache(B, H, cap, k_bits=kb, v_bits=vb, residual_len=R, sink_len=sink_len)
    kd, vd = dev(k), dev(v)
    p0, p1 = n_sink, n_sink + n_packed
    if n_sink:
        ks = cache.buf("k_sink").view(torch.int16).view(B, H, sink_len, D)
        vs = cache.buf("v_sink").view(torch.int16).view(B, H, sink_len, D)
        ks[:, :, :n_sink] = kd[:, :, :n_sink]
        vs[:, :, :n_sink] = vd[:, :, :n_sink]
    if n_packed:
        K.kvq_quantize_keys(cache.c, kd[:, :, p0:], H * T * D, T * D, D, 0, n_packed)
        K.kvq_quantize_values(cache.c, vd[:, :, p0:], H * T * D, T * D, D, 0, n_packed)
    if n_resid:
        kr = cache.buf("k_resid").view(torch.int16).view(B, H, R, D)
        vr = cache.buf("v_resid").view(torch.int16).view(B, H, R, D)
        kr[:, :, :n_resid] = kd[:, :, p1:p1 + n_resid]
        vr[:, :, :n_resid] = vd[:, :, p1:p1 + n_resid]
    cache.c.n_packed = n_packed
    cache.c.n_resid = n_resid
    cache.c.n_sink = n_sink
    torch.cuda.synchronize()
    return cache


def decode(K, cache, q: np.ndarray, sm_scale: float, rope_theta: float = 0.0):
    """Run kvq_decode_attn for host q [B][Hq][D]; returns the output on the host."""
    import torch
    B, Hq, D = q.shape
    qd = dev(q)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    ws_bytes = K.kvq_workspace_bytes(cache.c, Hq, K.KVQ_OP_DECODE_ATTN)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    K.kvq_decode_attn(cache.c, qd, Hq, sm_scale, rope_theta, out, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


def oracle_uniform_attention(k, v, q, n_packed, n_resid, kb, vb, sm_scale, n_sink=0):
    c = O.uniform_cache(k, v, kb, vb, n_packed, n_resid, n_sink=n_sink)
    return O.decode_attention_f64(O.f16_to_f32(q), c["k_hat"], c["v_hat"], sm_scale), c


def workload_inputs(w: S.Workload, tokens: int, heads_sel=None, batch_sel=None):
    """Host K, V (fp16 bits [B][Hkv][tokens][D]) for a workload, optionally a subset of heads."""
    g = w.gains()
    k = S.gen_tensor(w.seed, S.TID_K, w.batch, w.kv_heads, tokens, w.head_dim, gains=g,
                     heads_sel=heads_sel, batch_sel=batch_sel)
    v = S.gen_tensor(w.seed, S.TID_V, w.batch, w.kv_heads, tokens, w.head_dim,
                     heads_sel=heads_sel, batch_sel=batch_sel)
    return k, v


def workload_query(w: S.Workload, step: int = 0, heads_sel=None, batch_sel=None):
    return S.gen_tensor(w.seed, S.TID_Q, w.batch, w.q_heads, 1, w.head_dim, t0=step,
                        heads_sel=heads_sel, batch_sel=batch_sel)[:, :, 0]
