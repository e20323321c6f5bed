"""Oracle: a plain, slow, CPU reference of the packed KV cache and its decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import or run this module.  The product path (the HIP
library and its Python binding) never calls it, and it shares no code with the
product: the two meet only through the synthetic-input generator in
``kvq_synth`` and through the packed layouts documented in ``include/kvq.h``.

Sources (cited by short name below):
  [GEOM] "The KV cache has a geometry problem, not a bits problem" (unite.ai)
  [KIVI] "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
         (Telegram post on tgoop.com, sections "Method" and "Experiments")
  [KVQ]  "KVQuant: Towards 10 Million Context Length LLM Inference with KV
         Cache Quantization" (paper review on nubint.ai: abstract items (i)-(iv),
         "Proposed method", results table)
  [AXIS] "Why KV cache quantization fails without axis-specific geometry"
         (dothoosh.com; restates [GEOM])

Precision: the quantizer is float32 (IEEE round-to-nearest-even, one rounding
per operation, no fused multiply-add) because codes and metadata must be
bit-exact against the device; numpy ufuncs apply exactly one rounding per
operation.  Attention is float64.  fp16 values travel as uint16 bit patterns.

Parity pins for every function live in tests/test_oracle_*.py.  The one part
with no pin is the choice of the nuq code book itself (an input here): "parity
unpinned" for whether it resembles KVQuant's learned datatype.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 32


# --------------------------------------------------------------------------
# fp16 <-> fp32 (IEEE binary16; numpy's conversion rounds to nearest even and
# keeps subnormals)
# --------------------------------------------------------------------------
def f16_to_f32(bits) -> np.ndarray:
    """Exact widening of fp16 bit patterns to float32."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_f16_bits(x) -> np.ndarray:
    """float32 -> fp16 bit pattern, round to nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# O1: uniform asymmetric B-bit quantizer on groups ([GEOM] "Quantization error
# in practice": the group minimum is the zero point, the step is the range
# divided by 2^B - 1, each element goes to the nearest step; [KIVI]
# "Experiments": group 32 with a floating-point zero point).
# --------------------------------------------------------------------------
def uniform_quantize_groups(x_bits: np.ndarray, bits: int):
    """Quantize groups that run along the LAST axis of ``x_bits`` (fp16 bits).

    Returns (codes uint8 same shape, scale fp16 bits, min fp16 bits), the
    metadata with the group axis removed.

    Readings: rounding is half-to-even; the code is (x - min) times the
    reciprocal of the stored fp16 scale (one reciprocal per group); a zero
    scale gives all-zero codes; -0 is stored as +0.
    """
    x = f16_to_f32(x_bits)
    levels = np.float32(2 ** bits - 1)
    mn = x.min(axis=-1) + np.float32(0.0)     # + 0 turns -0 into +0
    mx = x.max(axis=-1) + np.float32(0.0)
    min_h = f32_to_f16_bits(mn)                # exact: mn is an fp16 value
    scale_h = f32_to_f16_bits((mx - mn) / levels)
    s = f16_to_f32(scale_h)
    with np.errstate(divide="ignore"):
        inv = np.where(s == 0, np.float32(0.0), np.float32(1.0) / s).astype(np.float32)
    q = np.rint((x - mn[..., None]) * inv[..., None])
    q = np.clip(q, np.float32(0.0), levels)
    q = np.where(s[..., None] == 0, np.float32(0.0), q)
    return q.astype(np.uint8), scale_h, min_h


def uniform_dequant(codes: np.ndarray, scale_h: np.ndarray, min_h: np.ndarray) -> np.ndarray:
    """x_hat = code * scale + min, two float32 roundings (metadata broadcast on the last axis)."""
    s = f16_to_f32(scale_h)[..., None]
    m = f16_to_f32(min_h)[..., None]
    return codes.astype(np.float32) * s + m


# --------------------------------------------------------------------------
# O2: grouping axes.  Keys per channel: a group is one channel over 32
# consecutive tokens ([GEOM] "Keys: outliers in fixed channels"; [KIVI]
# "Method").  Values per token: a group is 32 consecutive channels of one token
# ([GEOM] "Values: where intuition breaks").
# --------------------------------------------------------------------------
def quantize_keys_per_channel(k_bits: np.ndarray, bits: int):
    """k_bits [..., N, D] (N % 32 == 0) -> codes [..., N, D], scale/min [..., N/32, D]."""
    *lead, n, d = k_bits.shape
    assert n % GROUP == 0
    blk = k_bits.reshape(*lead, n // GROUP, GROUP, d)
    blk = np.swapaxes(blk, -1, -2)                         # [..., nb, D, 32]
    c, s, m = uniform_quantize_groups(blk, bits)
    c = np.swapaxes(c, -1, -2).reshape(*lead, n, d)
    return c, s, m


def quantize_values_per_token(v_bits: np.ndarray, bits: int):
    """v_bits [..., N, D] (D % 32 == 0) -> codes [..., N, D], scale/min [..., N, D/32]."""
    *lead, n, d = v_bits.shape
    assert d % GROUP == 0
    grp = v_bits.reshape(*lead, n, d // GROUP, GROUP)
    c, s, m = uniform_quantize_groups(grp, bits)
    return c.reshape(*lead, n, d), s, m


def quantize_keys_per_token(k_bits: np.ndarray, bits: int):
    """The swapped axis for keys (ablation only): groups of 32 channels per token."""
    return quantize_values_per_token(k_bits, bits)


def quantize_values_per_channel(v_bits: np.ndarray, bits: int):
    """The swapped axis for values (ablation only): groups of 32 tokens per channel."""
    return quantize_keys_per_channel(v_bits, bits)


def dequant_keys_per_channel(codes, scale_h, min_h):
    *lead, n, d = codes.shape
    c = np.swapaxes(codes.reshape(*lead, n // GROUP, GROUP, d), -1, -2)
    x = uniform_dequant(c, scale_h, min_h)
    return np.swapaxes(x, -1, -2).reshape(*lead, n, d)


def dequant_values_per_token(codes, scale_h, min_h):
    *lead, n, d = codes.shape
    c = codes.reshape(*lead, n, d // GROUP, GROUP)
    return uniform_dequant(c, scale_h, min_h).reshape(*lead, n, d)


# --------------------------------------------------------------------------
# O3: packing into the library's layouts (the pages give bit budgets, not bit
# layouts; the layouts are the ones include/kvq.h documents).  Codes are
# packed least-significant-bit first into little-endian 32-bit words.
# --------------------------------------------------------------------------
def _pack_fields(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack the last axis (length L, L*bits % 32 == 0) into L*bits/32 uint32 words."""
    per = 32 // bits
    *lead, n = codes.shape
    c = codes.astype(np.uint64).reshape(*lead, n // per, per)
    sh = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    return np.bitwise_or.reduce(c << sh, axis=-1).astype(np.uint32)


def _unpack_fields(words: np.ndarray, bits: int, n: int) -> np.ndarray:
    per = 32 // bits
    w = words.astype(np.uint64)[..., None]
    sh = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    c = (w >> sh) & np.uint64((1 << bits) - 1)
    return c.reshape(*words.shape[:-1], n).astype(np.uint8)


def pack_meta(scale_h: np.ndarray, min_h: np.ndarray) -> np.ndarray:
    """Metadata word: fp16 scale in bits 0..15, fp16 min in bits 16..31."""
    return (scale_h.astype(np.uint32) | (min_h.astype(np.uint32) << np.uint32(16)))


def unpack_meta(words: np.ndarray):
    return (words & 0xFFFF).astype(np.uint16), (words >> 16).astype(np.uint16)


def pack_k_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """[..., N, D] -> [..., N/32, 32 tokens, D*bits/32 words]: token-major rows; channel d
    of a token sits at bit (bits*d) % 32 of word (bits*d) // 32."""
    *lead, n, d = codes.shape
    w = _pack_fields(codes, bits)                          # [..., N, D*bits/32]
    return w.reshape(*lead, n // GROUP, GROUP, d * bits // 32)


def unpack_k_codes(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    *lead, nb, g, _ = words.shape
    return _unpack_fields(words, bits, d).reshape(*lead, nb * g, d)


def v_code_positions(bits: int, d: int = 128):
    """Word index within a block and bit position of the code of (token j, channel c),
    for every j in 0..31 and c in 0..d-1 of a per-token value block.

    A block is cut into tiles of 8 tokens x 8 channels, stored tile after tile in the
    order (token octet, channel octet), 2*bits words per tile.  Inside a tile, token pair
    i (tokens 2i, 2i+1 of the octet) owns words i and, for 4-bit codes, i + 4; the even
    token of the pair fills the low 16 bits of those words and the odd token the high 16
    bits; the tile's channels follow one another from bit 0 of each half, ``bits`` bits
    apart (2 bits: 8 channels in one half word; 4 bits: channels 0..3 in word i, 4..7 in
    word i + 4).  Returns int arrays ``word[j, c]`` and ``bit[j, c]``."""
    j = np.arange(GROUP)[:, None]
    c = np.arange(d)[None, :]
    per_half = 16 // bits                                # channels in one half word
    tile = (j // 8) * (d // 8) + c // 8
    pair, odd = (j % 8) // 2, j % 2
    word = tile * (2 * bits) + pair + 4 * ((c % 8) // per_half)
    bit = 16 * odd + bits * ((c % 8) % per_half)
    return np.broadcast_to(word, (GROUP, d)), np.broadcast_to(bit, (GROUP, d))


def pack_v_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """[..., N, D] -> [..., N/32, D*bits words]: per block of 32 tokens, the tiled layout
    of v_code_positions."""
    *lead, n, d = codes.shape
    blk = codes.reshape(*lead, n // GROUP, GROUP, d).astype(np.uint64)
    word, bit = v_code_positions(bits, d)
    out = np.zeros((*lead, n // GROUP, d * bits), dtype=np.uint64)
    for jj in range(GROUP):
        for cc in range(d):
            out[..., word[jj, cc]] |= blk[..., jj, cc] << np.uint64(bit[jj, cc])
    return out.astype(np.uint32)


def unpack_v_codes(words: np.ndarray, bits: int) -> np.ndarray:
    *lead, nb, nw = words.shape
    d = nw // bits
    word, bit = v_code_positions(bits, d)
    w = words.astype(np.uint64)[..., word]                # [..., nb, 32, D]
    c = (w >> bit.astype(np.uint64)) & np.uint64((1 << bits) - 1)
    return c.reshape(*lead, nb * GROUP, d).astype(np.uint8)


def nuq_code_fields(bits: int):
    """Where token j's code lives in a channel's ``bits`` words of a 32-token block: a list
    per token of (word, bit position, field width, first code bit) pieces.  Token j sits in
    byte j % 4 of its words, so that the codes of four consecutive tokens 4m..4m+3 come
    out of a word as the four bytes of one shifted and masked word.

    nuq2: words 0 and 1 hold tokens 0..15 / 16..31, token j of its half at bit
    8*(j % 4) + 2*(j % 16 // 4).  nuq3 (tokens 4m..4m+3, m = j // 4): for m < 6 the whole
    3-bit code at bit 8*(j % 4) + 3*(m % 2) of word m // 2; for m = 6 and 7 the low two
    bits at bit 8*(j % 4) + 6 of word m - 6 and the high bit at bit 8*(j % 4) + m of word
    2.  nuq4: word i holds tokens 8i..8i+7, token j of its octet at bit
    8*(j % 4) + 4*(j % 8 // 4)."""
    fields = []
    for j in range(GROUP):
        k, m = j % 4, j // 4
        if bits == 4:
            fields.append([(j // 8, 8 * k + 4 * ((j % 8) // 4), 4, 0)])
        elif bits == 3:
            if m < 6:
                fields.append([(m // 2, 8 * k + 3 * (m % 2), 3, 0)])
            else:
                fields.append([(m - 6, 8 * k + 6, 2, 0), (2, 8 * k + m, 1, 2)])
        else:
            fields.append([(j // 16, 8 * k + 2 * ((j % 16) // 4), 2, 0)])
    return fields


def pack_nuq(codes: np.ndarray, bits: int) -> np.ndarray:
    """``bits``-bit codes [..., N, D] -> [..., N/32, D, bits words] (per block, channel-major)."""
    *lead, n, d = codes.shape
    blk = np.swapaxes(codes.reshape(*lead, n // GROUP, GROUP, d), -1, -2).astype(np.uint64)
    words = np.zeros((*blk.shape[:-1], bits), dtype=np.uint64)
    for j, pieces in enumerate(nuq_code_fields(bits)):
        for w, pos, width, first in pieces:
            part = (blk[..., j] >> np.uint64(first)) & np.uint64((1 << width) - 1)
            words[..., w] |= part << np.uint64(pos)
    return words.astype(np.uint32)


def unpack_nuq(words: np.ndarray, bits: int) -> np.ndarray:
    *lead, nb, d, _ = words.shape
    w64 = words.astype(np.uint64)
    out = np.zeros((*lead, nb, d, GROUP), dtype=np.uint8)
    for j, pieces in enumerate(nuq_code_fields(bits)):
        c = np.zeros(w64.shape[:-1], dtype=np.uint64)
        for w, pos, width, first in pieces:
            c |= ((w64[..., w] >> np.uint64(pos)) & np.uint64((1 << width) - 1)) << np.uint64(first)
        out[..., j] = c.astype(np.uint8)
    return np.swapaxes(out, -1, -2).reshape(*lead, nb * GROUP, d)


def pack_nuq3(codes: np.ndarray) -> np.ndarray:
    """3-bit codes [..., N, D] -> [..., N/32, D, 3 words] (per block, channel-major)."""
    return pack_nuq(codes, 3)


def unpack_nuq3(words: np.ndarray) -> np.ndarray:
    return unpack_nuq(words, 3)


# --------------------------------------------------------------------------
# Byte accounting ([KVQ] results table, KV-cache GB column).
# --------------------------------------------------------------------------
def kv_cache_bytes(layers: int, hidden: int, tokens: int, bits_per_elem: float,
                   outlier_frac: float = 0.0, outlier_bits: int = 32) -> float:
    """Bytes of K plus V for ``tokens`` tokens: 2 * layers * hidden * tokens elements at
    ``bits_per_elem``, plus ``outlier_frac`` of the elements kept as sparse entries of
    ``outlier_bits`` each (value and index; row pointers not counted)."""
    elems = 2 * layers * hidden * tokens
    return elems * bits_per_elem / 8.0 + elems * outlier_frac * outlier_bits / 8.0


# --------------------------------------------------------------------------
# O4: streaming cache with an fp16 residual window ([GEOM] "The systems tax";
# [KIVI] "Method": keep up to R recent tokens in full precision and quantize
# them as a group once enough have accumulated).  Reading: the flush is lazy
# (it happens when a token arrives and the window is already full).
# --------------------------------------------------------------------------
class StreamingCache:
    """Per-channel keys / per-token values, one window shared by K and V.

    With ``sink_len`` > 0 the first ``sink_len`` tokens of the sequence are kept in fp16
    for good and never quantized ([GEOM] "Where research goes": InnerQ keeps
    full-precision windows for both the recent tokens and the attention-sink tokens).
    Reading: the sink is the sequence's leading tokens, filled before anything else;
    token order is sink, packed, window."""

    def __init__(self, batch, heads, head_dim, k_bits, v_bits, residual_len=128, sink_len=0):
        assert residual_len % GROUP == 0
        self.B, self.H, self.D = batch, heads, head_dim
        self.kb, self.vb, self.R = k_bits, v_bits, residual_len
        self.S = sink_len
        self.k_sink = np.zeros((batch, heads, sink_len, head_dim), np.uint16)
        self.v_sink = np.zeros((batch, heads, sink_len, head_dim), np.uint16)
        self.n_sink = 0
        self.k_res = np.zeros((batch, heads, residual_len, head_dim), np.uint16)
        self.v_res = np.zeros((batch, heads, residual_len, head_dim), np.uint16)
        self.k_codes = np.zeros((batch, heads, 0, head_dim), np.uint8)
        self.v_codes = np.zeros((batch, heads, 0, head_dim), np.uint8)
        self.k_scale = np.zeros((batch, heads, 0, head_dim), np.uint16)
        self.k_min = np.zeros((batch, heads, 0, head_dim), np.uint16)
        self.v_scale = np.zeros((batch, heads, 0, head_dim // GROUP), np.uint16)
        self.v_min = np.zeros((batch, heads, 0, head_dim // GROUP), np.uint16)
        self.n_packed = 0
        self.n_resid = 0

    def _flush(self):
        kc, ks, km = quantize_keys_per_channel(self.k_res, self.kb)
        vc, vs, vm = quantize_values_per_token(self.v_res, self.vb)
        self.k_codes = np.concatenate([self.k_codes, kc], axis=2)
        self.v_codes = np.concatenate([self.v_codes, vc], axis=2)
        self.k_scale = np.concatenate([self.k_scale, ks], axis=2)
        self.k_min = np.concatenate([self.k_min, km], axis=2)
        self.v_scale = np.concatenate([self.v_scale, vs], axis=2)
        self.v_min = np.concatenate([self.v_min, vm], axis=2)
        self.n_packed += self.R
        self.n_resid = 0

    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """k_new, v_new: fp16 bits [B][H][D] for one new token."""
        if self.n_sink < self.S:
            self.k_sink[:, :, self.n_sink] = k_new
            self.v_sink[:, :, self.n_sink] = v_new
            self.n_sink += 1
            return
        if self.R == 0:
            raise ValueError("streaming needs a residual window")
        if self.n_resid == self.R:
            self._flush()
        self.k_res[:, :, self.n_resid] = k_new
        self.v_res[:, :, self.n_resid] = v_new
        self.n_resid += 1

    def dequant(self):
        """(K_hat, V_hat) float32 [B][H][n_sink + N + r][D]: the sink as fp16, the packed
        part dequantized, the window as fp16."""
        kd = dequant_keys_per_channel(self.k_codes, self.k_scale, self.k_min)
        vd = dequant_values_per_token(self.v_codes, self.v_scale, self.v_min)
        r, ns = self.n_resid, self.n_sink
        kd = np.concatenate([f16_to_f32(self.k_sink[:, :, :ns]), kd,
                             f16_to_f32(self.k_res[:, :, :r])], axis=2)
        vd = np.concatenate([f16_to_f32(self.v_sink[:, :, :ns]), vd,
                             f16_to_f32(self.v_res[:, :, :r])], axis=2)
        return kd, vd


# --------------------------------------------------------------------------
# O5/O6: non-uniform datatype with per-vector dense-and-sparse outliers
# ([KVQ] abstract (iii) non-uniform datatype nuqX, (iv) per-vector
# dense-and-sparse quantization; "Proposed method").
# Readings: the code book is given in level units [0, 2^B - 1] with the same
# (min, scale) normalization as the uniform quantizer, so the identity code
# book reproduces the uniform quantizer; each element goes to the nearest code
# book level (ties to the even index); outliers are the ceil(n * bp / 10000)
# largest magnitudes of the vector (ties: lower index first), kept exactly and
# excluded from the min/max; outlier positions store code 0.
# --------------------------------------------------------------------------
def outlier_count(n: int, bp: int) -> int:
    """ceil(n * bp / 10000) in integer arithmetic."""
    return (n * bp + 9999) // 10000


def select_outliers(x_bits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest |x| of a 1-D vector of fp16 bits (ties: lower index first)."""
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    mag = (np.asarray(x_bits, dtype=np.uint16) & 0x7FFF).astype(np.int64)
    order = np.argsort(-mag, kind="stable")
    return np.sort(order[:k])


def nuq_code(xn: np.ndarray, lut_f32: np.ndarray) -> np.ndarray:
    """Index of the nearest code-book level for normalized values (ties: even index)."""
    mid = (lut_f32[:-1] + lut_f32[1:]) * np.float32(0.5)
    c = (xn[..., None] > mid).sum(axis=-1)
    cc = np.minimum(c, len(mid) - 1)
    tie = (c < len(mid)) & (xn == mid[cc]) & (c % 2 == 1)
    return (c + tie).astype(np.uint8)


def exact_moments(x_dense: np.ndarray):
    """(E[x], E[x^2] - E[x]^2, clamped at 0) of float values in float64, where sum x and
    sum x^2 are the exact sums rounded once (math.fsum is correctly rounded; x * x of an
    fp16 value is exact in float64).  The result does not depend on the order of the
    entries."""
    x = np.asarray(x_dense, dtype=np.float64)
    n = x.shape[0]
    mean = math.fsum(x.tolist()) / n
    var = max(math.fsum((x * x).tolist()) / n - mean * mean, 0.0)
    return mean, var


def qnorm_params(x_dense: np.ndarray, codes_dense: np.ndarray, lut: np.ndarray,
                 scale_h, min_h):
    """Q-Norm ([KVQ] "Proposed method" and findings: the dequantized distribution is made to
    match the statistics taken before quantization).  Reading: per vector, over its dense
    entries, the affine map x_hat -> a * x_hat + b that gives the dequantized values the
    mean and standard deviation of the original ones; it folds into the metadata as
    scale' = a * scale, min' = a * min + b (codes unchanged).

    Moments in float64: the original's from the values (E[x], E[x^2] - E[x]^2), the
    dequantized ones from the code histogram (level by level, ascending), each level's
    value lut[c] * scale + min in float32.  a = sqrt(var / var_hat) (1 when var_hat is 0),
    b = mean - a * mean_hat; the new metadata are a * scale and a * min + b rounded to
    float32, then to fp16.  Returns (scale_h', min_h').

    Reading of the summation (the page fixes no order): sum x and sum x^2 are the exact
    sums rounded once to float64 (math.fsum; x^2 of an fp16 value is exact in float64),
    so the result does not depend on the order in which the entries are added."""
    n = x_dense.shape[0]
    if n == 0:
        return scale_h, min_h
    mean, var = exact_moments(x_dense)
    s, m = f16_to_f32(scale_h), f16_to_f32(min_h)
    levels = (lut * s + m).astype(np.float32).astype(np.float64)
    cnt = np.bincount(np.asarray(codes_dense, dtype=np.int64), minlength=len(lut))
    m1 = 0.0
    m2 = 0.0
    for c in range(len(lut)):
        m1 += float(cnt[c]) * levels[c]
        m2 += float(cnt[c]) * levels[c] * levels[c]
    mean_hat = m1 / n
    var_hat = max(m2 / n - mean_hat * mean_hat, 0.0)
    a = math.sqrt(var / var_hat) if var_hat > 0.0 else 1.0
    b = mean - a * mean_hat
    new_s = f32_to_f16_bits(np.float32(a * float(s)))
    new_m = f32_to_f16_bits(np.float32(a * float(m) + b))
    return new_s, new_m


def nuq_quantize_vector(x_bits: np.ndarray, lut_bits: np.ndarray, n_outliers: int = 0,
                        qnorm: bool = False):
    """One vector (fp16 bits, 1-D).  Returns (codes, scale_h, min_h, outlier_idx, x_hat).
    With qnorm the returned metadata (and x_hat) are the Q-Norm-corrected ones."""
    lut = f16_to_f32(lut_bits)
    bits = int(round(math.log2(len(lut))))
    x = f16_to_f32(x_bits)
    out_idx = select_outliers(x_bits, n_outliers)
    dense = np.ones(x.shape[0], dtype=bool)
    dense[out_idx] = False
    if dense.any():
        mn = x[dense].min() + np.float32(0.0)
        mx = x[dense].max() + np.float32(0.0)
    else:
        mn = mx = np.float32(0.0)
    min_h = f32_to_f16_bits(mn)
    scale_h = f32_to_f16_bits((mx - mn) / np.float32(2 ** bits - 1))
    s = f16_to_f32(scale_h)
    if s == 0:
        codes = np.zeros(x.shape[0], dtype=np.uint8)
    else:
        inv = np.float32(1.0) / s
        xn = (x - mn) * inv
        codes = nuq_code(xn, lut)
    # An outlier's exact value replaces its dequantized one in attention, so the code
    # stored at its position is never read for its value; the pages leave it open.  Code 0
    # is stored there (reading: any fixed code works), which lets a decoder form the
    # replaced value from the metadata alone.
    codes[out_idx] = 0
    if qnorm:
        scale_h, min_h = qnorm_params(x[dense], codes[dense], lut, scale_h, min_h)
        s, mn = f16_to_f32(scale_h), f16_to_f32(min_h)
    xhat = lut[codes] * s + mn
    xhat[out_idx] = x[out_idx]
    return codes, scale_h, min_h, out_idx, xhat


def nuq_quantize_keys(k_bits: np.ndarray, lut_bits: np.ndarray, outlier_bp: int,
                      qnorm: bool = False):
    """Keys of one head [N][D]: per channel over the whole context, with outliers.

    Returns codes [N][D], scale/min [D], CSR (row_ptr int32 [N+1], entries uint32: column in
    bits 0..7, the row's token modulo 32 (its place in its 32-token block) in bits 8..12 and
    the fp16 value in bits 16..31, rows = tokens, columns ascending), and the dequantized
    keys x_hat float32 [N][D] (pre-RoPE)."""
    n, d = k_bits.shape
    k = outlier_count(n, outlier_bp)
    codes = np.zeros((n, d), np.uint8)
    scale = np.zeros(d, np.uint16)
    mins = np.zeros(d, np.uint16)
    xhat = np.zeros((n, d), np.float32)
    is_out = np.zeros((n, d), bool)
    for ch in range(d):
        c, s, m, oi, xh = nuq_quantize_vector(k_bits[:, ch], lut_bits, k, qnorm)
        codes[:, ch], scale[ch], mins[ch], xhat[:, ch] = c, s, m, xh
        is_out[oi, ch] = True
    counts = is_out.sum(axis=1)
    row_ptr = np.zeros(n + 1, np.int32)
    row_ptr[1:] = np.cumsum(counts)
    tt, cc = np.nonzero(is_out)                   # row-major: tokens, then channels ascending
    ent = (cc.astype(np.uint32) | ((tt % GROUP).astype(np.uint32) << np.uint32(8))
           | (k_bits[tt, cc].astype(np.uint32) << np.uint32(16)))
    return codes, scale, mins, row_ptr, ent.astype(np.uint32), xhat


def nuq_quantize_values(v_bits: np.ndarray, lut_bits: np.ndarray, outlier_bp: int = 0,
                        qnorm: bool = False):
    """Values of one head [N][D]: per token over all D channels.

    Without outliers returns codes [N][D], scale/min [N], x_hat float32 [N][D].  With
    outlier_bp > 0 each token's vector is quantized dense-and-sparse like a key channel
    ([KVQ] abstract (iv): outliers isolated for each vector): its ceil(D * bp / 10000)
    largest magnitudes are kept exactly, and a fifth array [N][k] of entries (channel in
    bits 0..15, fp16 value in bits 16..31, channels ascending) is returned after scale/min."""
    n, d = v_bits.shape
    if outlier_bp > 0 or qnorm:
        k = outlier_count(d, outlier_bp)
        codes = np.zeros((n, d), np.uint8)
        scale = np.zeros(n, np.uint16)
        mins = np.zeros(n, np.uint16)
        ent = np.zeros((n, k), np.uint32)
        xhat = np.zeros((n, d), np.float32)
        for t in range(n):
            c, sc, mn, oi, xh = nuq_quantize_vector(v_bits[t], lut_bits, k, qnorm)
            codes[t], scale[t], mins[t], xhat[t] = c, sc, mn, xh
            ent[t] = oi.astype(np.uint32) | (v_bits[t, oi].astype(np.uint32) << np.uint32(16))
        if outlier_bp == 0:
            return codes, scale, mins, xhat
        return codes, scale, mins, ent, xhat
    codes = np.zeros((n, d), np.uint8)
    scale = np.zeros(n, np.uint16)
    mins = np.zeros(n, np.uint16)
    lut = f16_to_f32(lut_bits)
    x = f16_to_f32(v_bits)
    mn = x.min(axis=1) + np.float32(0.0)
    mx = x.max(axis=1) + np.float32(0.0)
    mins[:] = f32_to_f16_bits(mn)
    scale[:] = f32_to_f16_bits((mx - mn) / np.float32(len(lut) - 1))
    s = f16_to_f32(scale)
    with np.errstate(divide="ignore"):
        inv = np.where(s == 0, np.float32(0.0), np.float32(1.0) / s).astype(np.float32)
    xn = (x - mn[:, None]) * inv[:, None]
    codes[:] = nuq_code(xn, lut)
    codes[s == 0] = 0
    xhat = lut[codes] * s[:, None] + mn[:, None]
    return codes, scale, mins, xhat


# --------------------------------------------------------------------------
# O7: rotary position embedding applied after dequantization ([GEOM] "Rotary
# embeddings complicate keys": quantize keys before the rotation and apply it
# after; [KVQ] abstract (ii)).  Readings: interleaved pairs (2i, 2i+1),
# frequency theta^(-2i/D), angle t * freq, all in float64.
# --------------------------------------------------------------------------
def rope_f64(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate x [..., T, D] (float64) at integer positions [T]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    freq = np.power(np.float64(theta), -2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# --------------------------------------------------------------------------
# O8: decode attention over the dequantized cache, float64 ([GEOM] "Why the KV
# cache is a problem": every generated token reads the whole cache; the score,
# softmax and weighted sum are textbook attention).  GQA: query head h reads kv
# head h // (Hq / Hkv).
# --------------------------------------------------------------------------
def decode_attention_f64(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
                         sm_scale: float) -> np.ndarray:
    """q [B][Hq][D]; k_hat, v_hat [B][Hkv][T][D] (any float) -> out float32 [B][Hq][D]."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k_hat.shape[1]
    g = hq // hkv
    out = np.zeros((bsz, hq, d), np.float64)
    for b in range(bsz):
        for h in range(hq):
            kh = np.asarray(k_hat[b, h // g], dtype=np.float64)
            vh = np.asarray(v_hat[b, h // g], dtype=np.float64)
            if kh.shape[0] == 0:
                continue
            s = (kh @ q[b, h]) * sm_scale
            p = np.exp(s - s.max())
            out[b, h] = (p @ vh) / p.sum()
    return out.astype(np.float32)


def default_sm_scale(head_dim: int) -> float:
    """1/sqrt(D) (textbook scaled dot-product attention; not on the pages)."""
    return 1.0 / math.sqrt(head_dim)


# --------------------------------------------------------------------------
# Whole-cache helpers used by the tests (compositions of the functions above).
# --------------------------------------------------------------------------
def uniform_cache(k_bits, v_bits, k_b, v_b, n_packed, n_resid, n_sink=0):
    """One-shot cache for tokens [0, n_sink + n_packed + n_resid): an fp16 sink of the first
    n_sink tokens, the packed part, the fp16 window.

    k_bits/v_bits: fp16 bits [B][H][T][D] with T >= n_sink + n_packed + n_resid.
    Returns a dict of the packed buffers (library layouts) and the dequantized K/V."""
    p0, p1 = n_sink, n_sink + n_packed
    kp, vp = k_bits[:, :, p0:p1], v_bits[:, :, p0:p1]
    kc, ks, km = quantize_keys_per_channel(kp, k_b)
    vc, vs, vm = quantize_values_per_token(vp, v_b)
    kd = dequant_keys_per_channel(kc, ks, km)
    vd = dequant_values_per_token(vc, vs, vm)
    kr = k_bits[:, :, p1:p1 + n_resid]
    vr = v_bits[:, :, p1:p1 + n_resid]
    return {
        "k_codes": pack_k_codes(kc, k_b),
        "k_meta": pack_meta(ks, km),
        "v_codes": pack_v_codes(vc, v_b),
        "v_meta": pack_meta(vs, vm),
        "k_hat": np.concatenate([f16_to_f32(k_bits[:, :, :p0]), kd, f16_to_f32(kr)], axis=2),
        "v_hat": np.concatenate([f16_to_f32(v_bits[:, :, :p0]), vd, f16_to_f32(vr)], axis=2),
    }


def rope_query_f16(q_bits: np.ndarray, position: int, theta: float) -> np.ndarray:
    """The query of the token at ``position``, rotated in float64 and rounded to fp16 bits
    (the decode call receives it already rotated)."""
    q = f16_to_f32(q_bits).astype(np.float64)
    shp = q.shape
    r = rope_f64(q.reshape(-1, 1, shp[-1]), np.array([position]), theta)
    return f32_to_f16_bits(r.reshape(shp).astype(np.float32))


def nuq_head(k_bits: np.ndarray, v_bits: np.ndarray, lut_k: np.ndarray, lut_v: np.ndarray,
             outlier_bp: int, n_packed: int, n_resid: int, theta: float, n_sink: int = 0,
             v_outlier_bp: int = 0, qnorm: bool = False):
    """One (batch, head) of a KVQuant-style cache: tokens [0, n_sink) kept in fp16 (the
    sink), tokens [n_sink, n_sink + n_packed) quantized (keys per channel with outliers over
    the quantized tokens only, values per token), the next n_resid tokens kept in fp16.
    Returns the packed buffers and the float64 keys (RoPE applied at positions 0.. in that
    order when theta > 0) and values attention reads."""
    p0, p1 = n_sink, n_sink + n_packed
    bk, bv = int(round(math.log2(len(lut_k)))), int(round(math.log2(len(lut_v))))
    kp, vp = k_bits[p0:p1], v_bits[p0:p1]
    kc, ks, km, rp, ent, kx = nuq_quantize_keys(kp, lut_k, outlier_bp, qnorm)
    if v_outlier_bp > 0:
        vc, vs, vm, v_ent, vx = nuq_quantize_values(vp, lut_v, v_outlier_bp, qnorm)
    else:
        vc, vs, vm, vx = nuq_quantize_values(vp, lut_v, 0, qnorm)
        v_ent = np.zeros((n_packed, 0), np.uint32)
    kw = k_bits[p1:p1 + n_resid]
    vw = v_bits[p1:p1 + n_resid]
    k_hat = np.concatenate([f16_to_f32(k_bits[:p0]), kx, f16_to_f32(kw)],
                           axis=0).astype(np.float64)
    v_hat = np.concatenate([f16_to_f32(v_bits[:p0]), vx, f16_to_f32(vw)],
                           axis=0).astype(np.float64)
    if theta > 0:
        k_hat = rope_f64(k_hat, np.arange(p1 + n_resid), theta)
    return {
        "k_codes": pack_nuq(kc[None], bk)[0] if n_packed else np.zeros((0, k_bits.shape[1], bk), np.uint32),
        "k_meta": pack_meta(ks, km),
        "v_codes": pack_nuq(vc[None], bv)[0] if n_packed else np.zeros((0, k_bits.shape[1], bv), np.uint32),
        "v_meta": pack_meta(vs, vm),
        "rowptr": rp, "ent": ent, "v_ent": v_ent, "k_hat": k_hat, "v_hat": v_hat,
    }
