"""The C ABI on the host: the library loads, exports every function include/kvq.h
declares, agrees with the header's struct layout, and rejects bad arguments before
anything reaches the GPU (no GPU needed)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import decode_attention_10_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert len(names) >= 8
    lib = C.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(K.EXPORTS) == names


def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "kvq.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(kvq_cache), sizeof(kvq_qparams),
         offsetof(kvq_cache, kq), offsetof(kvq_cache, k_codes), offsetof(kvq_cache, csr_capacity),
         offsetof(kvq_cache, n_resid), offsetof(kvq_qparams, lut), offsetof(kvq_cache, sink_len),
         offsetof(kvq_cache, k_sink), offsetof(kvq_cache, v_sink), offsetof(kvq_cache, n_sink));
  return 0;
}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(prog), "-o", str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                       check=True).stdout.split()))
    want = [C.sizeof(K.kvq_cache), C.sizeof(K.kvq_qparams), K.kvq_cache.kq.offset,
            K.kvq_cache.k_codes.offset, K.kvq_cache.csr_capacity.offset,
            K.kvq_cache.n_resid.offset, K.kvq_qparams.lut.offset, K.kvq_cache.sink_len.offset,
            K.kvq_cache.k_sink.offset, K.kvq_cache.v_sink.offset, K.kvq_cache.n_sink.offset]
    assert got == want


def _desc(kind=K.KVQ_UNIFORM, kb=2, vb=2, B=2, H=3, cap=256, R=128):
    c = K.kvq_cache()
    c.batch, c.kv_heads, c.head_dim, c.residual_len, c.capacity_tokens = B, H, 128, R, cap
    lut = 0x1000 if kind == K.KVQ_NUQ else None
    c.kq = K.make_qparams(kind, kb, K.KVQ_AXIS_CHANNEL, lut, 0)
    c.vq = K.make_qparams(kind, vb, K.KVQ_AXIS_TOKEN, lut, 0)
    return c


def test_layout_bytes_uniform():
    c = _desc(kb=4, vb=2)
    s = K.kvq_layout_bytes(c)
    bh, cap, D = 6, 256, 128
    assert s[K.KVQ_BUF_K_CODES] == bh * cap * D * 4 // 8
    assert s[K.KVQ_BUF_V_CODES] == bh * cap * D * 2 // 8
    assert s[K.KVQ_BUF_K_META] == bh * (cap // 32) * D * 4
    assert s[K.KVQ_BUF_V_META] == bh * cap * (D // 32) * 4
    assert s[K.KVQ_BUF_K_RESID] == s[K.KVQ_BUF_V_RESID] == bh * 128 * D * 2
    assert s[K.KVQ_BUF_K_CSR_ROWPTR] == s[K.KVQ_BUF_K_CSR_ENT] == 0
    assert s[K.KVQ_BUF_K_SINK] == s[K.KVQ_BUF_V_SINK] == 0
    c.sink_len = 20
    s = K.kvq_layout_bytes(c)
    assert s[K.KVQ_BUF_K_SINK] == s[K.KVQ_BUF_V_SINK] == bh * 20 * D * 2


def test_layout_bytes_nuq_and_csr_capacity():
    c = _desc(kind=K.KVQ_NUQ, kb=3, vb=3, B=1, H=32, cap=1048576, R=0)
    c.kq.outlier_bp = 100
    need = K.kvq_csr_entries_needed(c)
    assert need == 128 * 10486
    c.csr_capacity = need
    s = K.kvq_layout_bytes(c)
    assert s[K.KVQ_BUF_K_CODES] == 32 * 1048576 * 128 * 3 // 8
    assert s[K.KVQ_BUF_K_META] == 32 * 128 * 4
    assert s[K.KVQ_BUF_V_META] == 32 * 1048576 * 4
    assert s[K.KVQ_BUF_K_CSR_ROWPTR] == 32 * (1048576 + 1) * 4
    assert s[K.KVQ_BUF_K_CSR_ENT] == 32 * need * 4


@pytest.mark.parametrize("mutate,status", [
    (lambda c: setattr(c.kq, "bits", 3), K.KVQ_ERR_UNSUPPORTED),
    (lambda c: setattr(c.kq, "bits", 0), K.KVQ_ERR_INVALID_ARG),
    (lambda c: setattr(c.kq, "axis", K.KVQ_AXIS_TOKEN), K.KVQ_ERR_UNSUPPORTED),
    (lambda c: setattr(c.vq, "axis", K.KVQ_AXIS_CHANNEL), K.KVQ_ERR_UNSUPPORTED),
    (lambda c: setattr(c.kq, "axis", 7), K.KVQ_ERR_INVALID_ARG),
    (lambda c: setattr(c.kq, "group_size", 64), K.KVQ_ERR_UNSUPPORTED),
    (lambda c: setattr(c, "head_dim", 100), K.KVQ_ERR_INVALID_ARG),
    (lambda c: setattr(c, "residual_len", 100), K.KVQ_ERR_INVALID_ARG),
    (lambda c: setattr(c, "capacity_tokens", 100), K.KVQ_ERR_INVALID_ARG),
    (lambda c: setattr(c, "batch", 0), K.KVQ_ERR_INVALID_ARG),
    (lambda c: setattr(c.vq, "kind", K.KVQ_NUQ), K.KVQ_ERR_UNSUPPORTED),
    (lambda c: setattr(c, "sink_len", -1), K.KVQ_ERR_INVALID_ARG),
    (lambda c: (setattr(c.kq, "kind", K.KVQ_NUQ), setattr(c.vq, "kind", K.KVQ_NUQ),
                setattr(c.kq, "group_size", 0), setattr(c.vq, "group_size", 0),
                setattr(c.kq, "lut", 0x1000), setattr(c.vq, "lut", 0x1000),
                setattr(c.kq, "bits", 5), setattr(c.vq, "bits", 5)), K.KVQ_ERR_UNSUPPORTED),
    (lambda c: (setattr(c.kq, "kind", K.KVQ_NUQ), setattr(c.vq, "kind", K.KVQ_NUQ),
                setattr(c.kq, "group_size", 0), setattr(c.vq, "group_size", 0),
                setattr(c.kq, "lut", 0x1000), setattr(c.vq, "lut", 0x1000),
                setattr(c.kq, "bits", 4), setattr(c.vq, "bits", 2)), K.KVQ_ERR_UNSUPPORTED),
    (lambda c: setattr(c, "sink_len", 1025), K.KVQ_ERR_INVALID_ARG),
])
def test_descriptor_errors(mutate, status):
    c = _desc()
    mutate(c)
    with pytest.raises(K.KvqError) as e:
        K.kvq_layout_bytes(c)
    assert e.value.status == status
    assert K.kvq_last_error()


def test_mixed_kinds_unsupported():
    c = _desc()
    c.vq = K.make_qparams(K.KVQ_NUQ, 3, K.KVQ_AXIS_TOKEN, 0x1000, 0)
    with pytest.raises(K.KvqError) as e:
        K.kvq_layout_bytes(c)
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED


FAKE = 0x7F0000000000      # never dereferenced: every call below fails its host checks


def _fake_buffers(c):
    for i, n in enumerate(["k_codes", "k_meta", "v_codes", "v_meta", "k_resid", "v_resid"]):
        setattr(c, n, FAKE + 0x100000 * (i + 1))


def test_quantize_argument_errors():
    c = _desc()
    _fake_buffers(c)
    cases = [
        (dict(k=None), K.KVQ_ERR_INVALID_ARG),
        (dict(k=FAKE + 8), K.KVQ_ERR_ALIGNMENT),
        (dict(off=16), K.KVQ_ERR_INVALID_ARG),
        (dict(n=48), K.KVQ_ERR_INVALID_ARG),
        (dict(off=224, n=64), K.KVQ_ERR_CAPACITY),
        (dict(st=64), K.KVQ_ERR_INVALID_ARG),
        (dict(st=132), K.KVQ_ERR_ALIGNMENT),
    ]
    for kw, status in cases:
        a = dict(k=FAKE, sb=0, sh=0, st=128, off=0, n=32)
        a.update(kw)
        with pytest.raises(K.KvqError) as e:
            K.kvq_quantize_keys(c, a["k"], a["sb"], a["sh"], a["st"], a["off"], a["n"], stream=0)
        assert e.value.status == status, kw


def test_append_errors_leave_state_unchanged():
    c = _desc(cap=128, R=128)
    _fake_buffers(c)
    c.n_packed, c.n_resid = 128, 128          # full window, no room to flush
    with pytest.raises(K.KvqError) as e:
        K.kvq_append_flush(c, FAKE, FAKE, stream=0)
    assert e.value.status == K.KVQ_ERR_CAPACITY
    assert (c.n_packed, c.n_resid) == (128, 128)
    c.n_resid = 129
    with pytest.raises(K.KvqError) as e:
        K.kvq_append_flush(c, FAKE, FAKE, stream=0)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    c2 = _desc(R=0)
    _fake_buffers(c2)
    with pytest.raises(K.KvqError) as e:
        K.kvq_append_flush(c2, FAKE, FAKE, stream=0)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG


def test_decode_argument_errors():
    c = _desc()
    _fake_buffers(c)
    c.n_packed, c.n_resid = 64, 5
    cases = [
        (dict(hq=4), K.KVQ_ERR_INVALID_ARG),           # not a multiple of kv_heads = 3
        (dict(hq=15), K.KVQ_ERR_UNSUPPORTED),          # 5 query heads per kv head
        (dict(hq=48), K.KVQ_ERR_UNSUPPORTED),          # 16 per kv head
        (dict(theta=1e4), K.KVQ_ERR_UNSUPPORTED),      # RoPE is for nuq caches
        (dict(theta=-1.0), K.KVQ_ERR_INVALID_ARG),
        (dict(scale=float("inf")), K.KVQ_ERR_INVALID_ARG),
        (dict(q=FAKE + 4), K.KVQ_ERR_ALIGNMENT),
        (dict(out=None), K.KVQ_ERR_INVALID_ARG),
    ]
    for kw, status in cases:
        a = dict(hq=3, theta=0.0, scale=0.1, q=FAKE, out=FAKE, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        with pytest.raises(K.KvqError) as e:
            K.kvq_decode_attn(c, a["q"], a["hq"], a["scale"], a["theta"], a["out"], a["ws"],
                              a["wsb"], stream=0)
        assert e.value.status == status, kw


def test_decode_needs_workspace_for_split_contexts():
    """A long context over few heads is split across workgroups: the partials need the
    workspace, so a missing or short one is rejected before any launch."""
    c = _desc(B=1, H=1, cap=1 << 20)
    _fake_buffers(c)
    c.n_packed, c.n_resid = 1 << 20, 0
    need = K.kvq_workspace_bytes(c, 1, K.KVQ_OP_DECODE_ATTN)
    assert need > 0
    for ws, wsb in [(None, need), (FAKE, need - 4)]:
        with pytest.raises(K.KvqError) as e:
            K.kvq_decode_attn(c, FAKE, 1, 0.1, 0.0, FAKE, ws, wsb, stream=0)
        assert e.value.status == K.KVQ_ERR_INVALID_ARG


def test_sink_errors_leave_state_unchanged():
    """The sink fills first: an append while it has room needs its buffers; counters
    outside [0, sink_len] are rejected by append and decode alike."""
    c = _desc(R=128)
    _fake_buffers(c)
    c.sink_len = 4
    c.k_sink = c.v_sink = None
    with pytest.raises(K.KvqError) as e:
        K.kvq_append_flush(c, FAKE, FAKE, stream=0)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    assert (c.n_sink, c.n_packed, c.n_resid) == (0, 0, 0)
    c.n_sink = 5
    with pytest.raises(K.KvqError) as e:
        K.kvq_append_flush(c, FAKE, FAKE, stream=0)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    with pytest.raises(K.KvqError) as e:
        K.kvq_decode_attn(c, FAKE, 3, 0.1, 0.0, FAKE, FAKE, 1 << 20, stream=0)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    c.n_sink = 2                                 # tokens in the sink but no sink buffers
    with pytest.raises(K.KvqError) as e:
        K.kvq_decode_attn(c, FAKE, 3, 0.1, 0.0, FAKE, FAKE, 1 << 20, stream=0)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    assert "sink" in K.kvq_last_error()


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_layout_bytes_nuq_widths_and_value_outliers(bits):
    c = _desc(kind=K.KVQ_NUQ, kb=bits, vb=bits, B=1, H=2, cap=1024, R=0)
    c.vq.outlier_bp = 100
    s = K.kvq_layout_bytes(c)
    assert s[K.KVQ_BUF_K_CODES] == s[K.KVQ_BUF_V_CODES] == 2 * 1024 * 128 * bits // 8
    assert s[K.KVQ_BUF_V_OUT] == 2 * 1024 * 2 * 4          # 2 outliers per 128-channel token


def test_capacity_and_csr_limits():
    """The decode kernels form 32-bit word offsets within a head (block index times at most
    512 words) and the CSR row pointers are int32: capacity_tokens is capped at 2^28 and a
    head's outlier entries at 2^31 - 1, both rejected on the host."""
    c = _desc(B=1, H=1, cap=1 << 28, R=0)
    K.kvq_layout_bytes(c)                                  # the largest capacity is valid
    c.capacity_tokens = (1 << 28) + 32
    with pytest.raises(K.KvqError) as e:
        K.kvq_layout_bytes(c)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    c = _desc(B=1, H=1, cap=1024, R=0)
    c.csr_capacity = 1 << 31
    with pytest.raises(K.KvqError) as e:
        K.kvq_layout_bytes(c)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    # nuq keys: 128 channels x ceil(2^28 * 700 / 1e4) outliers per head > 2^31 - 1
    c = _desc(kind=K.KVQ_NUQ, kb=3, vb=3, B=1, H=1, cap=1 << 28, R=0)
    c.kq.outlier_bp = 700
    c.csr_capacity = (1 << 31) - 1
    _fake_buffers(c)
    c.k_csr_rowptr = FAKE + 0x900000
    c.k_csr_ent = FAKE + 0xA00000
    with pytest.raises(K.KvqError) as e:
        K.kvq_quantize_keys(c, FAKE, 0, 0, 128, 0, 1 << 28, FAKE, 1 << 40, stream=0)
    assert e.value.status == K.KVQ_ERR_CAPACITY
    assert "int32" in K.kvq_last_error()


def test_debug_build_exports_the_same_functions():
    """libkvq_debug.so (built with -DKVQ_DEBUG: device-side bounds checks) keeps the ABI."""
    path = os.path.join(os.path.dirname(K.LIB_PATH), "libkvq_debug.so")
    if not os.path.exists(path):
        pytest.skip("libkvq_debug.so is not built")
    lib = C.CDLL(path)
    for n in _declared_functions():
        assert hasattr(lib, n), n
