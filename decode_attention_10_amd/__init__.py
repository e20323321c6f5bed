"""Python binding of libkvq.so (include/kvq.h): argument marshalling only.

Every step of the quantize/append/attention path runs in the library's HIP
kernels; PyTorch is used for device memory and streams.  Importing this module
fails loudly if the library has not been built (python
decode_attention_10_amd/build.py) - there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY selects another build of the same C ABI, e.g. libkvq_debug.so (device-side
# bounds checks, synchronous entry points)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_PKG, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python decode_attention_10_amd/build.py`")

# torch first: its HIP runtime then satisfies libkvq.so's libamdhip64 dependency (same
# soname), so the library and torch share one runtime, one device context and the same
# stream handles.  Loading the library first would map a second runtime.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

# ---- constants (include/kvq.h) ----------------------------------------------------
KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_CAPACITY, KVQ_ERR_ALIGNMENT, \
    KVQ_ERR_HIP = range(6)
KVQ_AXIS_CHANNEL, KVQ_AXIS_TOKEN = 0, 1
KVQ_UNIFORM, KVQ_NUQ = 0, 1
(KVQ_BUF_K_CODES, KVQ_BUF_K_META, KVQ_BUF_V_CODES, KVQ_BUF_V_META, KVQ_BUF_K_RESID,
 KVQ_BUF_V_RESID, KVQ_BUF_K_CSR_ROWPTR, KVQ_BUF_K_CSR_ENT, KVQ_BUF_K_SINK,
 KVQ_BUF_V_SINK, KVQ_BUF_V_OUT) = range(11)
KVQ_NUM_BUFS = 11
KVQ_OP_QUANTIZE_KEYS, KVQ_OP_DECODE_ATTN = 0, 1

STATUS_NAMES = {0: "KVQ_OK", 1: "KVQ_ERR_INVALID_ARG", 2: "KVQ_ERR_UNSUPPORTED",
                3: "KVQ_ERR_CAPACITY", 4: "KVQ_ERR_ALIGNMENT", 5: "KVQ_ERR_HIP"}


class kvq_qparams(C.Structure):
    _fields_ = [("kind", C.c_int32), ("bits", C.c_int32), ("axis", C.c_int32),
                ("group_size", C.c_int32), ("lut", C.c_void_p), ("outlier_bp", C.c_int32),
                ("qnorm", C.c_int32)]


class kvq_cache(C.Structure):
    _fields_ = [("batch", C.c_int32), ("kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("residual_len", C.c_int32), ("capacity_tokens", C.c_int64),
                ("kq", kvq_qparams), ("vq", kvq_qparams),
                ("k_codes", C.c_void_p), ("k_meta", C.c_void_p), ("v_codes", C.c_void_p),
                ("v_meta", C.c_void_p), ("k_resid", C.c_void_p), ("v_resid", C.c_void_p),
                ("k_csr_rowptr", C.c_void_p), ("k_csr_ent", C.c_void_p),
                ("csr_capacity", C.c_int64), ("v_out", C.c_void_p),
                ("n_packed", C.c_int64), ("n_resid", C.c_int32),
                ("sink_len", C.c_int32), ("k_sink", C.c_void_p), ("v_sink", C.c_void_p),
                ("n_sink", C.c_int32), ("reserved", C.c_int32)]


_P = C.POINTER(kvq_cache)
_sig = {
    "kvq_layout_bytes": (C.c_int, [_P, C.POINTER(C.c_size_t)]),
    "kvq_csr_entries_needed": (C.c_int64, [_P]),
    "kvq_workspace_bytes": (C.c_size_t, [_P, C.c_int32, C.c_int32]),
    "kvq_quantize_keys": (C.c_int, [_P, C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                    C.c_int64, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kvq_quantize_values": (C.c_int, [_P, C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                      C.c_int64, C.c_int64, C.c_void_p]),
    "kvq_append_flush": (C.c_int, [_P, C.c_void_p, C.c_void_p, C.c_void_p]),
    "kvq_decode_attn": (C.c_int, [_P, C.c_void_p, C.c_int32, C.c_float, C.c_float, C.c_void_p,
                                  C.c_void_p, C.c_size_t, C.c_void_p]),
    "kvq_decode_attn_noalloc": (C.c_int, [_P, C.c_void_p, C.c_int32, C.c_float, C.c_float,
                                          C.c_void_p, C.c_void_p]),
    "kvq_last_error": (C.c_char_p, []),
}
for _n, (_r, _a) in _sig.items():
    _f = getattr(_lib, _n)
    _f.restype = _r
    _f.argtypes = _a

EXPORTS = tuple(_sig)


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != KVQ_OK:
        raise KvqError(status, kvq_last_error())


def _ptr(x) -> int | None:
    """Device/host address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- the C ABI, one wrapper per entry point ----------------------------------------
def kvq_last_error() -> str:
    return _lib.kvq_last_error().decode()


def kvq_layout_bytes(c: kvq_cache) -> list[int]:
    sizes = (C.c_size_t * KVQ_NUM_BUFS)()
    _check(_lib.kvq_layout_bytes(C.byref(c), sizes))
    return list(sizes)


def kvq_csr_entries_needed(c: kvq_cache) -> int:
    return int(_lib.kvq_csr_entries_needed(C.byref(c)))


def kvq_workspace_bytes(c: kvq_cache, q_heads: int, op: int) -> int:
    return int(_lib.kvq_workspace_bytes(C.byref(c), q_heads, op))


def kvq_quantize_keys(c: kvq_cache, k, stride_b: int, stride_h: int, stride_t: int,
                      token_offset: int, n_tokens: int, workspace=None, ws_bytes: int = 0,
                      stream=None) -> None:
    _check(_lib.kvq_quantize_keys(C.byref(c), _ptr(k), stride_b, stride_h, stride_t,
                                  token_offset, n_tokens, _ptr(workspace), ws_bytes,
                                  _stream(stream)))


def kvq_quantize_values(c: kvq_cache, v, stride_b: int, stride_h: int, stride_t: int,
                        token_offset: int, n_tokens: int, stream=None) -> None:
    _check(_lib.kvq_quantize_values(C.byref(c), _ptr(v), stride_b, stride_h, stride_t,
                                    token_offset, n_tokens, _stream(stream)))


def kvq_append_flush(c: kvq_cache, k_new, v_new, stream=None) -> None:
    _check(_lib.kvq_append_flush(C.byref(c), _ptr(k_new), _ptr(v_new), _stream(stream)))


def kvq_decode_attn(c: kvq_cache, q, q_heads: int, sm_scale: float, rope_theta: float, out,
                    workspace=None, ws_bytes: int = 0, stream=None) -> None:
    _check(_lib.kvq_decode_attn(C.byref(c), _ptr(q), q_heads, sm_scale, rope_theta, _ptr(out),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def kvq_decode_attn_noalloc(c: kvq_cache, q, q_heads: int, sm_scale: float,
                            rope_theta: float, out, stream=None) -> None:
    _check(_lib.kvq_decode_attn_noalloc(C.byref(c), _ptr(q), q_heads, sm_scale, rope_theta,
                                        _ptr(out), _stream(stream)))


# ---- device-memory plumbing --------------------------------------------------------
def make_qparams(kind: int, bits: int, axis: int, lut=None, outlier_bp: int = 0,
                 qnorm: int = 0) -> kvq_qparams:
    return kvq_qparams(kind=kind, bits=bits, axis=axis,
                       group_size=32 if kind == KVQ_UNIFORM else 0,
                       lut=_ptr(lut), outlier_bp=outlier_bp, qnorm=qnorm)


class KVCache:
    """Owns torch buffers for one cache descriptor (device memory plumbing only)."""

    def __init__(self, batch: int, kv_heads: int, capacity_tokens: int, k_bits: int = 2,
                 v_bits: int = 2, residual_len: int = 128, head_dim: int = 128,
                 kind: int = KVQ_UNIFORM, lut=None, outlier_bp: int = 0,
                 csr_capacity: int | None = None, sink_len: int = 0,
                 v_outlier_bp: int = 0, qnorm: int = 0, device="cuda"):
        import torch
        self.lut = lut
        c = kvq_cache()
        c.batch, c.kv_heads, c.head_dim = batch, kv_heads, head_dim
        c.residual_len, c.capacity_tokens = residual_len, capacity_tokens
        c.sink_len = sink_len
        c.kq = make_qparams(kind, k_bits, KVQ_AXIS_CHANNEL, lut, outlier_bp, qnorm)
        c.vq = make_qparams(kind, v_bits, KVQ_AXIS_TOKEN, lut, v_outlier_bp, qnorm)
        if csr_capacity is None:
            csr_capacity = max(0, kvq_csr_entries_needed(c))
        c.csr_capacity = csr_capacity
        sizes = kvq_layout_bytes(c)
        self.bufs = {}
        names = ["k_codes", "k_meta", "v_codes", "v_meta", "k_resid", "v_resid",
                 "k_csr_rowptr", "k_csr_ent", "k_sink", "v_sink", "v_out"]
        for i, n in enumerate(names):
            if sizes[i]:
                t = torch.zeros(sizes[i], dtype=torch.uint8, device=device)
                self.bufs[n] = t
                setattr(c, n, t.data_ptr())
        self.c = c
        self.sizes = sizes

    def buf(self, name: str, dtype=None):
        import torch
        t = self.bufs[name]
        return t.view(dtype) if dtype is not None else t

    @property
    def n_packed(self) -> int:
        return int(self.c.n_packed)

    @property
    def n_resid(self) -> int:
        return int(self.c.n_resid)

    @property
    def n_sink(self) -> int:
        return int(self.c.n_sink)
