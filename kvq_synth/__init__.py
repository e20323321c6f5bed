"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no quantization or attention arithmetic.  It produces
fp16 tensors (as raw uint16 bit patterns) from a counter-based generator so
that any element can be regenerated on its own, on the host here or on the
device by the matching kernel in ``synth.hip``.

Generator (SplitMix64, Steele/Lea/Flood 2014, as published by Vigna):
the n-th output of a stream with state ``s`` is ``mix64(s + (n + 1) * GAMMA)``.
Each element draws three consecutive outputs of its tensor's stream
(``n = 3 * idx + j``); each output gives four 16-bit uniforms, so twelve in
all.  Their sum minus 6 * 65536, times 2**-16, is an Irwin-Hall(12) variate:
mean 0, variance 1 (an approximate N(0, 1)), computed exactly in float32.  It
is multiplied by the element's gain in float32 and rounded to fp16
(round-to-nearest-even).

The element counter ``idx`` depends on the (batch, head, token, channel)
coordinate only, not on the tensor's shape, so a token appended later in a
stream draws the same value as in a one-shot tensor.

Workloads: the pages measure on Llama-2-7B/13B, Llama-3-8B and LLaMA-7B
activations (CoQA, GSM8K, LongBench, Wikitext).  No weights or datasets are
used here: K, V and q are drawn from the generator above with the models'
layer shapes, and a few fixed key channels per head are scaled up to imitate
the fixed-channel key outliers described on "The KV cache has a geometry
problem" (section on keys and fixed-channel outliers).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1

# tensor ids of the streams
TID_K = 1
TID_V = 2
TID_Q = 3
TID_OUTLIER = 4


def mix64(z):
    """SplitMix64 output function on numpy uint64 arrays (wrapping)."""
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor_id: int) -> int:
    """State of the stream for one tensor of one workload (a Python int < 2**64)."""
    return _mix64_int((seed + (tensor_id + 1) * GAMMA) & MASK64)


def elem_index(b, h, t, d):
    """Shape-independent element counter: b < 2**16, h < 2**12, t < 2**28, d < 2**8."""
    b = np.asarray(b, dtype=np.uint64)
    h = np.asarray(h, dtype=np.uint64)
    t = np.asarray(t, dtype=np.uint64)
    d = np.asarray(d, dtype=np.uint64)
    return (b << np.uint64(48)) | (h << np.uint64(36)) | (t << np.uint64(8)) | d


def ih12(key: int, idx) -> np.ndarray:
    """Irwin-Hall(12) variates (float32, exact) for element counters ``idx``."""
    idx = np.asarray(idx, dtype=np.uint64)
    k = np.uint64(key)
    total = np.zeros(idx.shape, dtype=np.int64)
    for j in range(3):
        n = idx * np.uint64(3) + np.uint64(j + 1)
        h = mix64(k + n * np.uint64(GAMMA))
        for s in range(4):
            total += ((h >> np.uint64(16 * s)) & np.uint64(0xFFFF)).astype(np.int64)
    centred = (total - 6 * 65536).astype(np.float32)       # |.| < 2**19: exact
    return centred * np.float32(2.0 ** -16)                   # power of two: exact


def outlier_channels(seed: int, heads: int, head_dim: int, n_out: int) -> np.ndarray:
    """``n_out`` distinct key channels per head, fixed for every token: int32 [heads][n_out]."""
    key = stream_key(seed, TID_OUTLIER)
    out = np.zeros((heads, n_out), dtype=np.int32)
    for h in range(heads):
        chosen: list[int] = []
        n = 0
        while len(chosen) < n_out:
            n += 1
            v = _mix64_int(key + (h * 4096 + n) * GAMMA) % head_dim
            if v not in chosen:
                chosen.append(v)
        out[h] = sorted(chosen)
    return out


def key_gains(seed: int, heads: int, head_dim: int, n_out: int, gain: float) -> np.ndarray:
    """float32 [heads][head_dim]: 1 everywhere except ``gain`` on the outlier channels."""
    g = np.ones((heads, head_dim), dtype=np.float32)
    if n_out:
        ch = outlier_channels(seed, heads, head_dim, n_out)
        for h in range(heads):
            g[h, ch[h]] = np.float32(gain)
    return g


def gen_tensor(seed: int, tensor_id: int, batch: int, heads: int, tokens: int, head_dim: int,
               gains: np.ndarray | None = None, t0: int = 0,
               heads_sel=None, batch_sel=None) -> np.ndarray:
    """fp16 bit patterns (uint16) [batch][heads][tokens][head_dim] for tokens t0 .. t0+tokens-1.

    ``heads_sel``/``batch_sel`` restrict the output to a subset of heads/batches
    (their coordinates are kept, so the values equal the full tensor's)."""
    key = stream_key(seed, tensor_id)
    bs = np.arange(batch) if batch_sel is None else np.asarray(batch_sel)
    hs = np.arange(heads) if heads_sel is None else np.asarray(heads_sel)
    b = bs[:, None, None, None]
    h = hs[None, :, None, None]
    t = (t0 + np.arange(tokens))[None, None, :, None]
    d = np.arange(head_dim)[None, None, None, :]
    idx = elem_index(b, h, t, d)
    x = ih12(key, idx)
    if gains is not None:
        x = x * np.asarray(gains, dtype=np.float32)[hs][None, :, None, :]
    return x.astype(np.float16).view(np.uint16)


def nuq_lut(bits: int) -> np.ndarray:
    """fp16 bits [2^bits]: an ascending non-uniform code book in level units [0, 2^bits - 1].

    The learned, sensitivity-weighted datatype of KVQuant is not printed on the
    pages, so a fixed normal-quantile code book stands in for it: level i sits
    at the standard-normal quantile of (2i + 1) / 2^(bits + 1), mapped affinely so that
    the first level is 0 and the last 2^bits - 1.  It is an input of the method, not
    part of it.
    """
    from statistics import NormalDist
    nd = NormalDist()
    n = 1 << bits
    z = np.array([nd.inv_cdf((2 * i + 1) / (2.0 * n)) for i in range(n)], dtype=np.float64)
    half = (n - 1) / 2.0
    lv = half + half * z / z[-1]
    return np.sort(lv.astype(np.float16)).view(np.uint16)


def nuq3_lut() -> np.ndarray:
    """The 3-bit code book (nuq_lut(3))."""
    return nuq_lut(3)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: the layer shape and the quantization settings."""
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    n_packed: int          # tokens in the packed cache
    n_resid: int           # tokens in the fp16 residual window at attention time
    k_bits: int
    v_bits: int
    kind: str              # "uniform" or "nuq"
    seed: int
    n_outlier_ch: int      # fixed outlier key channels per kv head
    outlier_gain: float
    residual_len: int = 128
    group: int = 32
    outlier_bp: int = 0    # dense-and-sparse: outliers per key channel, basis points
    rope_theta: float = 0.0
    stream_steps: int = 0  # appends (each followed by attention) after the prefill
    sink_len: int = 0      # fp16 attention-sink tokens at the sequence start (kept full)
    v_outlier_bp: int = 0  # dense-and-sparse values: outliers per token vector, basis points
    qnorm: int = 0         # 1: Q-Norm the nuq metadata

    @property
    def ctx(self) -> int:
        return self.sink_len + self.n_packed + self.n_resid

    def gains(self) -> np.ndarray:
        return key_gains(self.seed, self.kv_heads, self.head_dim, self.n_outlier_ch,
                         self.outlier_gain)


SEED_BASE = 0x4B49564900

WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 128, 512, 128, 2, 2, "uniform", SEED_BASE + 1, 4, 50.0),
    "llama2_7b": Workload("llama2_7b", 8, 32, 32, 128, 4096, 128, 2, 2, "uniform",
                          SEED_BASE + 2, 3, 100.0),
    "llama2_7b_sink": Workload("llama2_7b_sink", 8, 32, 32, 128, 4096, 128, 2, 2, "uniform",
                               SEED_BASE + 6, 3, 100.0, sink_len=32),
    "llama2_13b_k4v2": Workload("llama2_13b_k4v2", 4, 40, 40, 128, 32768, 128, 4, 2, "uniform",
                                SEED_BASE + 3, 3, 100.0),
    "llama3_8b_gqa": Workload("llama3_8b_gqa", 1, 32, 8, 128, 131072, 128, 2, 2, "uniform",
                              SEED_BASE + 4, 3, 100.0, stream_steps=1024),
    "kvquant_1m": Workload("kvquant_1m", 1, 32, 32, 128, 1048576, 0, 3, 3, "nuq",
                           SEED_BASE + 5, 3, 100.0, residual_len=0, outlier_bp=100,
                           rope_theta=1.0e4),
    "kvquant_256k_nuq2": Workload("kvquant_256k_nuq2", 1, 32, 32, 128, 262144, 0, 2, 2, "nuq",
                                  SEED_BASE + 8, 3, 100.0, residual_len=0, outlier_bp=100,
                                  rope_theta=1.0e4),
    "kvquant_256k_nuq4": Workload("kvquant_256k_nuq4", 1, 32, 32, 128, 262144, 0, 4, 4, "nuq",
                                  SEED_BASE + 9, 3, 100.0, residual_len=0, outlier_bp=100,
                                  rope_theta=1.0e4),
    "kvquant_256k_nuq2_qnorm": Workload("kvquant_256k_nuq2_qnorm", 1, 32, 32, 128, 262144, 0,
                                        2, 2, "nuq", SEED_BASE + 10, 3, 100.0, residual_len=0,
                                        outlier_bp=100, rope_theta=1.0e4, qnorm=1),
    "kvquant_256k_dense_sparse": Workload("kvquant_256k_dense_sparse", 1, 32, 32, 128, 262144, 0,
                                          3, 3, "nuq", SEED_BASE + 7, 3, 100.0, residual_len=0,
                                          outlier_bp=100, rope_theta=1.0e4, v_outlier_bp=100),
}


def n_outlier_channels(head_dim: int, frac: float = 0.02) -> int:
    """Rounded count of outlier channels for a fraction of the head dimension."""
    return int(math.floor(frac * head_dim + 0.5))


# ---- device generator (kvq_synth/synth.hip, built into libkvq_synth.so) ----------------
_synth_lib = None


def _load_synth():
    global _synth_lib
    if _synth_lib is None:
        import ctypes as C
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_synth.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: run python decode_attention_10_amd/build.py")
        import torch  # noqa: F401  (share torch's HIP runtime, see the binding)
        lib = C.CDLL(path)
        lib.kvq_synth_fill.restype = C.c_int
        lib.kvq_synth_fill.argtypes = [C.c_void_p, C.c_uint64, C.c_int32, C.c_int32, C.c_int64,
                                       C.c_int32, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p]
        _synth_lib = lib
    return _synth_lib


def fill_device(out, seed: int, tensor_id: int, batch: int, heads: int, tokens: int,
                head_dim: int, gains=None, t0: int = 0, b0: int = 0, stream=None):
    """Fill a device tensor (int16/uint16 storage, [batch][heads][tokens][head_dim]) with the
    values gen_tensor() defines.  ``gains``: device float32 [heads][head_dim] or None."""
    import torch
    lib = _load_synth()
    assert out.numel() >= batch * heads * tokens * head_dim and out.element_size() == 2
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = lib.kvq_synth_fill(out.data_ptr(), stream_key(seed, tensor_id), batch, heads, tokens,
                            head_dim, t0, b0, None if gains is None else gains.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"kvq_synth_fill failed ({rc})")
    return out
