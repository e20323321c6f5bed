"""Streams and HIP graphs, through the C ABI.

A decode launched on a non-default stream equals the same decode on the default stream.
Library calls captured in a HIP graph (decodes, a run of appends with a flush, the
KVQuant quantizer's passes, the empty-cache decode) give the eager call's results on every
replay, with eager library work and host synchronizations between the replays.  A
captured call keeps the counters it saw at capture, so every replay repeats the same
step; its outputs must be bit-identical to the eager call's (same plan, same arithmetic
order).  Parity of those eager results with the oracle is checked once per case here and
in depth by the other GPU tests."""
import numpy as np
import pytest

import kvq_synth as S
from oracle import kvq_oracle as O
from tests.kvq_testlib import (assert_close, build_uniform_cache, dev, host_words,
                               oracle_uniform_attention)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("decode_attention_10_amd")

SM = 0.0883883


def _kv(seed, B, H, T, D=128):
    g = S.key_gains(seed, H, D, 3, 100.0)
    return (S.gen_tensor(seed, S.TID_K, B, H, T, D, gains=g),
            S.gen_tensor(seed, S.TID_V, B, H, T, D))


def _queries(seed, B, Hq, n):
    return [S.gen_tensor(seed, S.TID_Q, B, Hq, 1, 128, t0=i)[:, :, 0] for i in range(n)]


def _workspace(cache, Hq):
    wsb = K.kvq_workspace_bytes(cache.c, Hq, K.KVQ_OP_DECODE_ATTN)
    return torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda"), wsb


def _nan_out(B, Hq):
    return torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")


# (B, Hkv, GQ, N, r, kb, vb): split plan + merge launch (vector kernel), the matrix-core
# kernel with a merge, one workgroup per head (no merge), 8 query heads per kv head
DECODES = [(1, 2, 1, 4096, 40, 2, 2), (2, 2, 4, 2048, 17, 4, 2), (4, 64, 1, 1024, 128, 2, 2),
           (1, 2, 8, 512, 3, 2, 4)]


@pytest.mark.parametrize("B,Hkv,GQ,N,r,kb,vb", DECODES)
def test_decode_on_a_side_stream_equals_the_default_stream(B, Hkv, GQ, N, r, kb, vb):
    k, v = _kv(500 + N + r, B, Hkv, N + r)
    cache = build_uniform_cache(K, k, v, N, r, kb, vb, 128, cap=N)
    Hq = Hkv * GQ
    q = _queries(500, B, Hq, 1)[0]
    qd = dev(q)
    ws0, wsb = _workspace(cache, Hq)
    ws1, _ = _workspace(cache, Hq)
    out0, out1 = _nan_out(B, Hq), _nan_out(B, Hq)
    K.kvq_decode_attn(cache.c, qd, Hq, SM, 0.0, out0, ws0, wsb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    K.kvq_decode_attn(cache.c, qd, Hq, SM, 0.0, out1, ws1, wsb, stream=side)
    torch.cuda.synchronize()
    a, b = out0.cpu().numpy(), out1.cpu().numpy()
    ref, _ = oracle_uniform_attention(k, v, q, N, r, kb, vb, SM)
    assert_close(a, ref, f"decode B{B} Hkv{Hkv} GQ{GQ} N{N} r{r}")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("B,Hkv,GQ,N,r,kb,vb", DECODES)
def test_decode_graph_replays_equal_eager_calls(B, Hkv, GQ, N, r, kb, vb):
    k, v = _kv(600 + N + r, B, Hkv, N + r)
    cache = build_uniform_cache(K, k, v, N, r, kb, vb, 128, cap=N)
    Hq = Hkv * GQ
    qs = _queries(600, B, Hq, 4)
    ws_e, wsb = _workspace(cache, Hq)
    eager = []
    for q in qs:
        out = _nan_out(B, Hq)
        K.kvq_decode_attn(cache.c, dev(q), Hq, SM, 0.0, out, ws_e, wsb)
        torch.cuda.synchronize()
        eager.append(out.cpu().numpy())
    ref, _ = oracle_uniform_attention(k, v, qs[0], N, r, kb, vb, SM)
    assert_close(eager[0], ref, f"decode B{B} Hkv{Hkv} GQ{GQ} N{N} r{r}")

    q_g, out_g = dev(qs[0]), _nan_out(B, Hq)
    ws_g, _ = _workspace(cache, Hq)
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap_stream):
        K.kvq_decode_attn(cache.c, q_g, Hq, SM, 0.0, out_g, ws_g, wsb)
    torch.cuda.synchronize()
    for i in range(len(qs)):
        q_g.copy_(dev(qs[i]))                     # the graph reads the buffers' contents
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        other = _nan_out(B, Hq)                   # eager library work between replays
        K.kvq_decode_attn(cache.c, dev(qs[(i + 1) % len(qs)]), Hq, SM, 0.0, other, ws_e, wsb)
        torch.cuda.synchronize()
        assert np.array_equal(out_g.cpu().numpy(), eager[i]), f"replay {i}"
        assert np.array_equal(other.cpu().numpy(), eager[(i + 1) % len(qs)]), f"eager {i}"


def test_append_and_decode_steps_replayed_from_a_graph():
    """Four (append, decode) steps across a flush (window of 32, 30 tokens in it at the
    start), captured once and replayed three times, against the same steps run eagerly on
    a twin cache built from the same tokens.  The steps change the cache (the flush
    empties the window that the first decodes read), so the cache's starting bytes are
    restored before each replay."""
    B, H, R, N0, r0, steps = 2, 3, 32, 64, 30, 4
    T = N0 + r0 + steps
    k, v = _kv(701, B, H, T)
    qs = _queries(701, B, H, steps)
    eager_cache = build_uniform_cache(K, k, v, N0, r0, 2, 4, R, cap=N0 + 2 * R)
    graph_cache = build_uniform_cache(K, k, v, N0, r0, 2, 4, R, cap=N0 + 2 * R)
    kd, vd = dev(k), dev(v)
    knew = [kd[:, :, N0 + r0 + i].contiguous() for i in range(steps)]
    vnew = [vd[:, :, N0 + r0 + i].contiguous() for i in range(steps)]
    qd = [dev(q) for q in qs]
    ws_e, wsb = _workspace(eager_cache, H)
    ws_g, _ = _workspace(graph_cache, H)
    names = ("k_codes", "k_meta", "v_codes", "v_meta", "k_resid", "v_resid")
    start = {n: graph_cache.buf(n).clone() for n in names}

    eager = []
    for i in range(steps):
        K.kvq_append_flush(eager_cache.c, knew[i], vnew[i])
        out = _nan_out(B, H)
        K.kvq_decode_attn(eager_cache.c, qd[i], H, SM, 0.0, out, ws_e, wsb)
        torch.cuda.synchronize()
        eager.append(out.cpu().numpy())
    assert (eager_cache.n_packed, eager_cache.n_resid) == (N0 + R, r0 + steps - R)
    n_last = N0 + r0 + steps
    ref, _ = oracle_uniform_attention(k, v, qs[-1], N0 + R, n_last - N0 - R, 2, 4, SM)
    assert_close(eager[-1], ref, "last eager step")

    outs = [_nan_out(B, H) for _ in range(steps)]
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap_stream):
        for i in range(steps):
            K.kvq_append_flush(graph_cache.c, knew[i], vnew[i])
            K.kvq_decode_attn(graph_cache.c, qd[i], H, SM, 0.0, outs[i], ws_g, wsb)
    torch.cuda.synchronize()
    final = _nan_out(B, H)
    for rep in range(3):
        for n in names:
            graph_cache.buf(n).copy_(start[n])
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        K.kvq_decode_attn(eager_cache.c, qd[0], H, SM, 0.0, final, ws_e, wsb)
        torch.cuda.synchronize()
        for i in range(steps):
            assert np.array_equal(outs[i].cpu().numpy(), eager[i]), f"replay {rep} step {i}"
        for n in names:
            assert np.array_equal(host_words(graph_cache.buf(n)),
                                  host_words(eager_cache.buf(n))), f"replay {rep}: {n}"


def test_nuq_quantize_and_decode_replayed_from_a_graph():
    """The KVQuant key quantizer (histogram, select, statistics, codes and CSR passes, its
    scratch cleared by fill kernels), the value quantizer and a RoPE decode, captured and
    replayed three times: every replay rewrites the eager call's bytes and output."""
    B, H, N, bp, theta = 1, 2, 2048 + 64, 100, 1e4
    k, v = _kv(801, B, H, N)
    lut = S.nuq_lut(3)
    lk = dev(lut)

    def nuq_cache():
        c = K.KVCache(B, H, N, k_bits=3, v_bits=3, residual_len=0, kind=K.KVQ_NUQ, lut=lk,
                      outlier_bp=bp)
        c.c.vq.lut = lk.data_ptr()
        return c

    kd, vd = dev(k), dev(v)
    q = O.rope_query_f16(_queries(801, B, H, 1)[0], N, theta)
    qd = dev(q)
    wsq = K.kvq_workspace_bytes(nuq_cache().c, 0, K.KVQ_OP_QUANTIZE_KEYS)

    def run(c, wq, wd, out, stream=None):
        K.kvq_quantize_keys(c.c, kd, H * N * 128, N * 128, 128, 0, N, wq, wsq, stream=stream)
        K.kvq_quantize_values(c.c, vd, H * N * 128, N * 128, 128, 0, N, stream=stream)
        c.c.n_packed = N
        K.kvq_decode_attn(c.c, qd, H, SM, theta, out, wd, wsd, stream=stream)
        c.c.n_packed = 0

    ce, cg = nuq_cache(), nuq_cache()
    wsd = K.kvq_workspace_bytes(ce.c, H, K.KVQ_OP_DECODE_ATTN)
    wq_e = torch.empty(wsq, dtype=torch.uint8, device="cuda")
    wq_g = torch.empty(wsq, dtype=torch.uint8, device="cuda")
    wd_e = torch.empty(max(wsd, 16), dtype=torch.uint8, device="cuda")
    wd_g = torch.empty(max(wsd, 16), dtype=torch.uint8, device="cuda")
    out_e, out_g = _nan_out(B, H), _nan_out(B, H)
    run(ce, wq_e, wd_e, out_e)
    torch.cuda.synchronize()
    want = out_e.cpu().numpy()
    kh = np.zeros((B, H, N, 128))
    vh = np.zeros((B, H, N, 128))
    for h in range(H):
        ref = O.nuq_head(k[0, h], v[0, h], lut, lut, bp, N, 0, theta)
        kh[0, h], vh[0, h] = ref["k_hat"], ref["v_hat"]
    assert_close(want, O.decode_attention_f64(O.f16_to_f32(q), kh, vh, SM), "eager nuq decode")

    names = ("k_codes", "k_meta", "v_codes", "v_meta", "k_csr_rowptr", "k_csr_ent")
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap_stream):
        run(cg, wq_g, wd_g, out_g)
    torch.cuda.synchronize()
    for rep in range(3):
        for name in names:
            cg.buf(name).fill_(0x5A)               # stale bytes the replay must overwrite
        wq_g.fill_(0xFF)
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        run(ce, wq_e, wd_e, out_e)                 # eager library work between replays
        torch.cuda.synchronize()
        assert np.array_equal(out_g.cpu().numpy(), want), f"replay {rep}"
        assert np.array_equal(out_e.cpu().numpy(), want), f"eager {rep}"
        for name in names[:-1]:
            assert np.array_equal(host_words(cg.buf(name)), host_words(ce.buf(name))), \
                f"replay {rep}: {name}"
        rp = host_words(ce.buf("k_csr_rowptr")).reshape(B, H, N + 1)
        eg = host_words(cg.buf("k_csr_ent")).reshape(B, H, -1)
        ee = host_words(ce.buf("k_csr_ent")).reshape(B, H, -1)
        for h in range(H):
            nnz = int(rp[0, h, N])
            assert nnz > 0 and np.array_equal(eg[0, h, :nnz], ee[0, h, :nnz]), \
                f"replay {rep}: CSR entries of head {h}"


def test_empty_cache_decode_in_a_graph_writes_zeros():
    cache = K.KVCache(2, 2, 64, residual_len=32)
    q = dev(_queries(9, 2, 4, 1)[0])
    out = _nan_out(2, 4)
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap_stream):
        K.kvq_decode_attn(cache.c, q, 4, SM, 0.0, out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (out.cpu().numpy() == 0).all(), f"replay {rep}"
