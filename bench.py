"""Benchmark of the packed-KV hot path on one MI355X, over the five workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME ...]
                    [--no-cpu-baseline] [--cpu-budget SECONDS]

Workloads (kvq_synth.WORKLOADS), run in this order by default:
  tiny             B1 H1, 512 packed + 128 fp16 window, int2 K/V
  llama2_7b        B8 H32, 4096 + 128, int2 K/V
  llama2_13b_k4v2  B4 H40, 32768 + 128, int4 K / int2 V
  llama3_8b_gqa    B1 Hq32 / Hkv8, 131072 + 128, int2 K/V, streaming appends
  kvquant_1m       B1 H32, 1,048,576 tokens, nuq3 K (pre-RoPE, 1 % CSR outliers) / nuq3 V
The headline line (value, roofline) is kvquant_1m, the largest configuration that fits
one GPU; every workload gets its own block under "workloads".

A step of a uniform workload is one decode step of one layer: append the new token's
K/V to the fp16 window (the first step of the timed run finds the window full and first
quantizes it into the packed cache: the per-channel key and per-token value quantizers)
and then decode attention over the whole cache.  Layer caches rotate (copies carved out
of one allocation per buffer, > 768 MB in all, at most 256 copies) so that the decode
streams its cache from HBM rather than the 256 MB Infinity Cache; each layer's counters
are restored after its step.  A step of kvquant_1m is one decode over the one-shot
quantized context (quantize is timed separately).  Exactly --steps steps are captured in
one HIP graph and replayed once in the timed region (after --warmup eager steps and one
untimed replay that uploads the graph), bracketed by device synchronizations:
ms_per_step = wall / steps.

value / decode GB/s: algorithmic bytes of one decode (codes, metadata, CSR, fp16 window
and sink, q, out) / mean decode time, from HIP events on the launch stream around each
of >= 10 replays of a decode-only graph (each >= 64 decodes over the rotating layer
copies; 4 decodes for kvquant_1m); p10 / p50 / p90 of the per-replay means.
quantize GB/s: fp16 K/V read + everything written, over the whole context.

cpu_baseline: the oracle (oracle/kvq_oracle.py, unchanged) timed on the host on a bounded
sample of each workload, once on 1 thread and once on every core this process may use
(worker processes started from a fork server launched before the first GPU call; each
worker runs 1 BLAS thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E peak, GB/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "decode_attention_10_amd", "csrc")
KERNEL_SOURCES = {
    "decode_uniform_kernel": ("decode_uniform.hip", "decode_common.h", "kvq_common.h"),
    "decode_gqa_kernel": ("decode_gqa.hip", "decode_common.h", "kvq_common.h"),
    "decode_nuq_kernel": ("decode_nuq.hip", "kvq_common.h"),
}
METRIC = "decode-attn HBM GB/s on packed KV (% of peak); tokens*ctx/s; quantize GB/s"
DEFAULT_WORKLOADS = ("tiny", "llama2_7b", "llama2_13b_k4v2", "llama3_8b_gqa", "kvquant_1m")
HEADLINE = "kvquant_1m"
MIN_ROTATION_BYTES = 768e6
MAX_LAYERS = 256
MIN_DECODE_REPLAYS = 10
MIN_DECODES_PER_REPLAY = 64
NUQ_CPU_TOKENS = 65536      # oracle sample of a 1M-token head: its first 65,536 tokens


# ---------------------------------------------------------------------------------------
# byte accounting
# ---------------------------------------------------------------------------------------
def decode_bytes(w, n_packed: int, n_resid: int) -> int:
    """Algorithmic bytes one decode launch must move: packed codes and metadata, the fp16
    window and attention-sink tokens, q and the fp32 output."""
    bh = w.batch * w.kv_heads
    D = w.head_dim
    codes = bh * n_packed * D * (w.k_bits + w.v_bits) // 8
    meta = bh * (n_packed // 32) * D * 4 + bh * n_packed * (D // 32) * 4
    window = 2 * bh * (n_resid + w.sink_len) * D * 2
    return codes + meta + window + w.batch * w.q_heads * D * (2 + 4)


def nuq_decode_bytes(w, n_packed: int, heads: int | None = None) -> int:
    """Algorithmic bytes of one decode over a nuq cache: B-bit codes of K and V, per-channel
    key metadata, per-token value metadata, the CSR of key outliers (row pointers and one
    4-byte entry per outlier), the value outliers (4 bytes each), q and out."""
    bh = w.batch * (w.kv_heads if heads is None else heads)
    hq = bh * (w.q_heads // w.kv_heads)
    D = w.head_dim
    k_out = (n_packed * w.outlier_bp + 9999) // 10000
    v_out = (D * w.v_outlier_bp + 9999) // 10000
    codes = bh * n_packed * D * (w.k_bits + w.v_bits) // 8
    meta = bh * D * 4 + bh * n_packed * 4
    csr = (bh * (n_packed + 1) * 4 + bh * D * k_out * 4) if w.outlier_bp else 0
    return codes + meta + csr + bh * n_packed * v_out * 4 + hq * D * (2 + 4)


def nuq_quantize_bytes(w, n_tokens: int, heads: int | None = None) -> int:
    """One-shot nuq quantize: fp16 K and V read once, codes, metadata and CSR written."""
    bh = w.batch * (w.kv_heads if heads is None else heads)
    D = w.head_dim
    k_out = (n_tokens * w.outlier_bp + 9999) // 10000
    read = 2 * bh * n_tokens * D * 2
    written = bh * n_tokens * D * (w.k_bits + w.v_bits) // 8 + bh * D * 4 + bh * n_tokens * 4
    if w.outlier_bp:
        written += bh * (n_tokens + 1) * 4 + bh * D * k_out * 4
    written += bh * n_tokens * ((D * w.v_outlier_bp + 9999) // 10000) * 4
    return read + written


def quantize_bytes(w, n_tokens: int, heads: int | None = None) -> int:
    """Prefill quantize: fp16 K and V read, packed codes and metadata written."""
    bh = w.batch * w.kv_heads if heads is None else heads
    D = w.head_dim
    read = 2 * bh * n_tokens * D * 2
    written = bh * n_tokens * D * (w.k_bits + w.v_bits) // 8 + \
        bh * (n_tokens // 32) * D * 4 + bh * n_tokens * (D // 32) * 4
    return read + written


# ---------------------------------------------------------------------------------------
# counter summaries committed under profiles/
# ---------------------------------------------------------------------------------------
def kernel_source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of ``kernel`` on ``workload`` from the committed counter summary
    ``profiles/<kernel>_<workload>_traffic.txt``: rocprofv3 FETCH_SIZE and WRITE_SIZE of the
    kernel's dispatches, each scaled by what the same counter reads for a plain copy of known
    size.  None when there is no summary or it was taken on other kernel sources."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_source_digest(kernel):
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def uniform_decode_kernel(w) -> str:
    """The decode kernel the library runs for a uniform cache: the matrix-core kernel for 2
    or 4 query heads per kv head, else the vector kernel."""
    return "decode_gqa_kernel" if w.q_heads // w.kv_heads in (2, 4) else "decode_uniform_kernel"


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample (runs in worker processes)
# ---------------------------------------------------------------------------------------
def cpu_cores() -> int:
    """Cores this process may use (capped at 16, the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_unit_inputs(w, unit: int):
    """Host inputs of one (batch, kv head) unit: fp16 K, V and the unit's queries.  nuq
    units are the head's first NUQ_CPU_TOKENS tokens, quantized as a context of their own."""
    import kvq_synth as S
    b, h = divmod(unit, w.kv_heads)
    gq = w.q_heads // w.kv_heads
    T = NUQ_CPU_TOKENS if w.kind == "nuq" else w.ctx
    k = S.gen_tensor(w.seed, S.TID_K, w.batch, w.kv_heads, T, w.head_dim, gains=w.gains(),
                     heads_sel=[h], batch_sel=[b])
    v = S.gen_tensor(w.seed, S.TID_V, w.batch, w.kv_heads, T, w.head_dim,
                     heads_sel=[h], batch_sel=[b])
    q = S.gen_tensor(w.seed, S.TID_Q, w.batch, w.q_heads, 1, w.head_dim,
                     heads_sel=list(range(h * gq, (h + 1) * gq)), batch_sel=[b])[:, :, 0]
    return k, v, q


def _cpu_uniform_unit(w, k, v, q):
    """Oracle quantize (keys per channel, values per token, packing) and one decode (unpack,
    dequantize, fp16 sink and window, float64 attention) of one unit.  Returns
    (quantize seconds, decode seconds)."""
    from oracle import kvq_oracle as O
    S0, S1 = w.sink_len, w.sink_len + w.n_packed
    t0 = time.perf_counter()
    kc, ks, km = O.quantize_keys_per_channel(k[:, :, S0:S1], w.k_bits)
    vc, vs, vm = O.quantize_values_per_token(v[:, :, S0:S1], w.v_bits)
    pk = (O.pack_k_codes(kc, w.k_bits), O.pack_meta(ks, km))
    pv = (O.pack_v_codes(vc, w.v_bits), O.pack_meta(vs, vm))
    t1 = time.perf_counter()
    kd = O.dequant_keys_per_channel(O.unpack_k_codes(pk[0], w.k_bits, w.head_dim),
                                    *O.unpack_meta(pk[1]))
    vd = O.dequant_values_per_token(O.unpack_v_codes(pv[0], w.v_bits), *O.unpack_meta(pv[1]))
    kd = np.concatenate([O.f16_to_f32(k[:, :, :S0]), kd, O.f16_to_f32(k[:, :, S1:])], axis=2)
    vd = np.concatenate([O.f16_to_f32(v[:, :, :S0]), vd, O.f16_to_f32(v[:, :, S1:])], axis=2)
    O.decode_attention_f64(O.f16_to_f32(q), kd, vd, O.default_sm_scale(w.head_dim))
    return t1 - t0, time.perf_counter() - t1


def _cpu_nuq_unit(w, k, v, q):
    """Oracle nuq quantize (keys per channel with CSR outliers, values per token, packing) and
    one decode (unpack, code-book dequantization, outliers, RoPE in float64, attention) of
    one unit.  Returns (quantize seconds, decode seconds)."""
    import kvq_synth as S
    from oracle import kvq_oracle as O
    L = S.nuq_lut(w.k_bits)
    kh, vh = k[0, 0], v[0, 0]
    n = kh.shape[0]
    t0 = time.perf_counter()
    kc, ks, km, rp, ent, _ = O.nuq_quantize_keys(kh, L, w.outlier_bp)
    vc, vs, vm, _ = O.nuq_quantize_values(vh, L, 0)
    pk = (O.pack_nuq(kc, w.k_bits), O.pack_meta(ks, km))
    pv = (O.pack_nuq(vc, w.v_bits), O.pack_meta(vs, vm))
    t1 = time.perf_counter()
    lut = O.f16_to_f32(L)
    s, m = (O.f16_to_f32(x) for x in O.unpack_meta(pk[1]))
    kd = lut[O.unpack_nuq(pk[0], w.k_bits)] * s[None, :] + m[None, :]
    rows = np.repeat(np.arange(n), np.diff(rp))
    kd[rows, (ent & 0xFF).astype(np.int64)] = O.f16_to_f32((ent >> 16).astype(np.uint16))
    s, m = (O.f16_to_f32(x) for x in O.unpack_meta(pv[1]))
    vd = lut[O.unpack_nuq(pv[0], w.v_bits)] * s[:, None] + m[:, None]
    kr = O.rope_f64(kd, np.arange(n), w.rope_theta)
    qr = O.rope_query_f16(q, n, w.rope_theta)
    O.decode_attention_f64(O.f16_to_f32(qr), kr[None, None], vd[None, None],
                           O.default_sm_scale(w.head_dim))
    return t1 - t0, time.perf_counter() - t1


def _cpu_unit_bytes(w):
    """(quantize bytes, decode bytes) of one sample unit, in the metric's accounting."""
    if w.kind == "nuq":
        return (nuq_quantize_bytes(w, NUQ_CPU_TOKENS, heads=1),
                nuq_decode_bytes(w, NUQ_CPU_TOKENS, heads=1))
    bh = w.batch * w.kv_heads
    return quantize_bytes(w, w.n_packed, heads=1), decode_bytes(w, w.n_packed, w.n_resid) // bh


def cpu_leg_worker(name: str, index: int, workers: int, budget_s: float, barrier, results):
    """One worker of a CPU-baseline leg: prepares its units' inputs, waits for the other
    workers, then runs oracle quantize + decode over its units (unit index, index + workers,
    ...) until ``budget_s`` of timed work; puts (index, units, quantize s, decode s,
    quantize bytes, decode bytes, wall s) on ``results``."""
    try:
        from threadpoolctl import threadpool_limits

        import kvq_synth as S
        w = S.WORKLOADS[name]
        n_units = w.batch * w.kv_heads
        mine = [u % n_units for u in range(index, index + 2 * workers, workers)][:2]
        qb, db = _cpu_unit_bytes(w)
        unit_fn = _cpu_nuq_unit if w.kind == "nuq" else _cpu_uniform_unit
        with threadpool_limits(limits=1):
            inputs = [_cpu_unit_inputs(w, u) for u in mine]
            if barrier is not None:
                barrier.wait(timeout=300)
            tq = td = 0.0
            runs = 0
            w0 = time.perf_counter()
            while tq + td < budget_s:
                a, b = unit_fn(w, *inputs[runs % len(inputs)])
                tq += a
                td += b
                runs += 1
            wall = time.perf_counter() - w0
        results.put((index, runs, tq, td, runs * qb, runs * db, wall))
    except BaseException as e:                      # reported by the parent
        if barrier is not None:
            barrier.abort()
        results.put((index, f"{type(e).__name__}: {e}"))


def start_cpu_leg(ctx, name: str, workers: int, budget_s: float):
    """Starts a leg's worker processes (forked by the fork server) and returns a handle."""
    q = ctx.Queue()
    barrier = ctx.Barrier(workers) if workers > 1 else None
    procs = [ctx.Process(target=cpu_leg_worker, args=(name, i, workers, budget_s, barrier, q))
             for i in range(workers)]
    for p in procs:
        p.start()
    # the barrier stays referenced until the leg ends: dropping it would unlink its
    # semaphores before the workers have opened them
    return procs, q, workers, barrier


def finish_cpu_leg(handle, name: str, timeout_s: float = 600.0):
    import kvq_synth as S
    procs, q, workers, _barrier = handle
    got = [q.get(timeout=timeout_s) for _ in range(workers)]
    for p in procs:
        p.join()
    errors = [g[1] for g in got if len(g) == 2]
    if errors:
        raise RuntimeError(f"CPU baseline of {name} failed: {errors[0]}")
    w = S.WORKLOADS[name]
    runs = sum(g[1] for g in got)
    tq, td = max(g[2] for g in got), max(g[3] for g in got)
    qbytes, dbytes = sum(g[4] for g in got), sum(g[5] for g in got)
    # the workers ran side by side: aggregate rate = all bytes / the longest worker's time
    if w.kind == "nuq":
        unit = (f"{NUQ_CPU_TOKENS}-token prefix of a head quantized as a context of its own "
                f"(nuq{w.k_bits} keys with {w.outlier_bp / 100:g}% CSR outliers, nuq{w.v_bits} "
                f"values, RoPE theta {w.rope_theta:g})")
    else:
        unit = f"(batch, kv head) unit at the full context ({w.ctx} tokens)"
    return {"decode_gbs": round(dbytes / td / 1e9, 4), "quantize_gbs": round(qbytes / tq / 1e9, 4),
            "cores": workers, "unit_runs": runs,
            "sample": f"{runs} unit runs over {workers} worker(s), each {unit} of {name}: oracle "
                      f"quantize + pack, then unpack + dequantize + float64 attention; "
                      f"{td:.1f} s decode / {tq:.1f} s quantize timed on {workers} core(s)"}


# ---------------------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------------------
def time_replays(graph, replays: int, per_replay: int, stream):
    """Replays ``graph`` ``replays`` times with HIP events on ``stream`` around each replay.
    Returns (mean seconds per unit over the whole run, [p10, p50, p90] of the per-replay
    means)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record(stream)
    for i in range(replays):
        graph.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e-3 / per_replay for i in range(replays)])
    mean = ev[0].elapsed_time(ev[replays]) * 1e-3 / (replays * per_replay)
    return mean, [float(np.percentile(per, p)) for p in (10, 50, 90)]


def timed_steps(graph, steps: int, stream, restore=None):
    """The timed region: one replay of the ``steps``-step graph between two device
    synchronizations, after one untimed replay (the graph's first launch uploads it) and
    ``restore`` (which puts back any state the untimed replay changed).  Returns (wall
    seconds, device seconds from events)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph.replay()
    if restore is not None:
        restore()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) * 1e-3


class LayerArena:
    """``layers`` cache descriptors of one shape whose buffers are slices of one allocation
    per buffer slot (device memory plumbing only)."""

    def __init__(self, K, template, layers: int, device):
        import ctypes

        import torch
        sizes = K.kvq_layout_bytes(template)
        names = ["k_codes", "k_meta", "v_codes", "v_meta", "k_resid", "v_resid",
                 "k_csr_rowptr", "k_csr_ent", "k_sink", "v_sink", "v_out"]
        self.layers, self.slots = layers, {}
        descs = [K.kvq_cache() for _ in range(layers)]
        for d in descs:
            ctypes.memmove(ctypes.byref(d), ctypes.byref(template), ctypes.sizeof(template))
        for i, n in enumerate(names):
            if not sizes[i]:
                continue
            stride = (sizes[i] + 255) // 256 * 256
            buf = torch.empty(layers * stride, dtype=torch.uint8, device=device)
            self.slots[n] = (buf, stride, sizes[i])
            for l, d in enumerate(descs):
                setattr(d, n, buf.data_ptr() + l * stride)
        self.descs = descs

    def view(self, name: str, layer: int = 0):
        buf, stride, size = self.slots[name]
        return buf[layer * stride: layer * stride + size]

    def replicate(self):
        """Copies layer 0's bytes of every slot into every other layer (one copy per slot)."""
        for buf, stride, size in self.slots.values():
            v = buf.view(self.layers, stride)
            v[1:, :size] = v[0:1, :size]


def gpu_uniform(w, steps: int, warmup: int) -> dict:
    import torch

    import decode_attention_10_amd as K
    import kvq_synth as S
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    B, Hkv, Hq, D, N, R = w.batch, w.kv_heads, w.q_heads, w.head_dim, w.n_packed, w.residual_len
    S0, T = w.sink_len, w.ctx
    cap = N + R

    gains = torch.from_numpy(w.gains()).to(dev)
    k_src = torch.empty((B, Hkv, T + 1, D), dtype=torch.int16, device=dev)
    v_src = torch.empty((B, Hkv, T + 1, D), dtype=torch.int16, device=dev)
    S.fill_device(k_src, w.seed, S.TID_K, B, Hkv, T + 1, D, gains=gains)
    S.fill_device(v_src, w.seed, S.TID_V, B, Hkv, T + 1, D)
    q = torch.empty((B, Hq, 1, D), dtype=torch.int16, device=dev)
    S.fill_device(q, w.seed, S.TID_Q, B, Hq, 1, D)
    k_new = k_src[:, :, T].contiguous()
    v_new = v_src[:, :, T].contiguous()

    per_layer = decode_bytes(w, N, w.n_resid)
    layers = max(1, min(MAX_LAYERS, math.ceil(MIN_ROTATION_BYTES / per_layer)))
    tpl = K.kvq_cache()
    tpl.batch, tpl.kv_heads, tpl.head_dim, tpl.residual_len, tpl.capacity_tokens = B, Hkv, D, R, cap
    tpl.sink_len = S0
    tpl.kq = K.make_qparams(K.KVQ_UNIFORM, w.k_bits, K.KVQ_AXIS_CHANNEL)
    tpl.vq = K.make_qparams(K.KVQ_UNIFORM, w.v_bits, K.KVQ_AXIS_TOKEN)
    arena = LayerArena(K, tpl, layers, dev)
    c0 = arena.descs[0]
    sT = (Hkv * (T + 1) * D, (T + 1) * D, D)
    k_pk, v_pk = k_src[:, :, S0:], v_src[:, :, S0:]       # first packed token

    def prefill():
        K.kvq_quantize_keys(c0, k_pk, sT[0], sT[1], sT[2], 0, N)
        K.kvq_quantize_values(c0, v_pk, sT[0], sT[1], sT[2], 0, N)

    prefill()
    arena.view("k_resid").view(torch.int16).view(B, Hkv, R, D)[:, :, :w.n_resid] = \
        k_src[:, :, S0 + N:T]
    arena.view("v_resid").view(torch.int16).view(B, Hkv, R, D)[:, :, :w.n_resid] = \
        v_src[:, :, S0 + N:T]
    if S0:
        arena.view("k_sink").view(torch.int16).view(B, Hkv, S0, D)[:] = k_src[:, :, :S0]
        arena.view("v_sink").view(torch.int16).view(B, Hkv, S0, D)[:] = v_src[:, :, :S0]
    arena.replicate()
    for c in arena.descs:
        c.n_packed, c.n_resid, c.n_sink = N, w.n_resid, S0
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws_bytes = K.kvq_workspace_bytes(c0, Hq, K.KVQ_OP_DECODE_ATTN)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    sm = 1.0 / math.sqrt(D)

    # prefill quantize rate (keys + values over the whole packed context, into layer 0,
    # which holds the same bytes afterwards)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        prefill()
    reps = 20
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        prefill()
    e1.record(stream)
    torch.cuda.synchronize()
    quant_ms = e0.elapsed_time(e1) / reps
    quant_gbs = quantize_bytes(w, N) / (quant_ms * 1e-3) / 1e9

    # the step: append (the window is full at step 0, 128, ...: flush first) + decode
    def step(i: int) -> int:
        c = arena.descs[i % layers]
        flush = i % R == 0
        c.n_packed, c.n_resid = N, (R if flush else w.n_resid - 1)
        K.kvq_append_flush(c, k_new, v_new)
        nbytes = decode_bytes(w, int(c.n_packed), int(c.n_resid))
        K.kvq_decode_attn(c, q, Hq, sm, 0.0, out, ws, ws_bytes)
        c.n_packed, c.n_resid = N, w.n_resid
        return nbytes

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    cap_stream = torch.cuda.Stream()
    step_graph, dec_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    # a decode-only replay goes over every layer copy `rounds` times (>= 64 decodes)
    rounds = max(1, math.ceil(MIN_DECODES_PER_REPLAY / layers))
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(step_graph, stream=cap_stream):
            nbytes = [step(i) for i in range(steps)]
        with torch.cuda.graph(dec_graph, stream=cap_stream):
            for _ in range(rounds):
                for c in arena.descs:
                    K.kvq_decode_attn(c, q, Hq, sm, 0.0, out, ws, ws_bytes)
    torch.cuda.synchronize()
    wall, dev_s = timed_steps(step_graph, steps, stream)
    dec_graph.replay()
    mean_dec_s, pct = time_replays(dec_graph, MIN_DECODE_REPLAYS, rounds * layers, stream)
    dec_bytes = decode_bytes(w, N, w.n_resid)
    gbs = dec_bytes / mean_dec_s / 1e9
    kern = uniform_decode_kernel(w)
    res = {
        "workload": (f"{w.name}: batch {B}, {Hq} q / {Hkv} kv heads, head_dim {D}, "
                     + (f"{S0} fp16 sink + " if S0 else "")
                     + f"{N} packed + {w.n_resid} fp16 window tokens, K int{w.k_bits} "
                     f"per-channel / V int{w.v_bits} per-token, group 32"),
        "steps": steps, "ms_per_step": round(wall / steps * 1e3, 5),
        "ms_per_step_device": round(dev_s / steps * 1e3, 5),
        "step_bytes_mean": int(np.mean(nbytes)), "flushes_in_timed_steps": (steps + R - 1) // R,
        "decode_us": round(mean_dec_s * 1e6, 3),
        "decode_us_p10_p50_p90": [round(x * 1e6, 3) for x in pct],
        "decode_replays": MIN_DECODE_REPLAYS, "decodes_per_replay": rounds * layers,
        "layers_rotated": layers,
        "decode_gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_ctx_per_s": round(B * T / mean_dec_s, 1),
        "quantize_gbs": round(quant_gbs, 1), "quantize_ms_prefill": round(quant_ms, 4),
        "kernel": kern, "bytes_per_launch": dec_bytes,
        "traffic": measured_traffic(kern, w.name),
    }
    del arena, k_src, v_src, ws
    torch.cuda.empty_cache()
    return res


def gpu_nuq(w, steps: int, warmup: int) -> dict:
    """KVQuant-style workload: one-shot quantize of the whole context (timed as the quantize
    rate), then decode steps over it (a step is one decode; there is no window)."""
    import torch

    import decode_attention_10_amd as K
    import kvq_synth as S
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    B, Hkv, Hq, D, N = w.batch, w.kv_heads, w.q_heads, w.head_dim, w.n_packed
    gains = torch.from_numpy(w.gains()).to(dev)
    k_src = torch.empty((B, Hkv, N, D), dtype=torch.int16, device=dev)
    v_src = torch.empty_like(k_src)
    S.fill_device(k_src, w.seed, S.TID_K, B, Hkv, N, D, gains=gains)
    S.fill_device(v_src, w.seed, S.TID_V, B, Hkv, N, D)
    lut = torch.from_numpy(S.nuq_lut(w.k_bits).view(np.int16)).to(dev)
    c = K.KVCache(B, Hkv, N, k_bits=w.k_bits, v_bits=w.v_bits, residual_len=0, kind=K.KVQ_NUQ,
                  lut=lut, outlier_bp=w.outlier_bp, v_outlier_bp=w.v_outlier_bp, qnorm=w.qnorm)
    wsq = K.kvq_workspace_bytes(c.c, 0, K.KVQ_OP_QUANTIZE_KEYS)
    ws_q = torch.empty(wsq, dtype=torch.uint8, device=dev)
    sT = (Hkv * N * D, N * D, D)

    def quantize():
        K.kvq_quantize_keys(c.c, k_src, sT[0], sT[1], sT[2], 0, N, ws_q, wsq)
        K.kvq_quantize_values(c.c, v_src, sT[0], sT[1], sT[2], 0, N)

    quantize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        quantize()
    e1.record(stream)
    torch.cuda.synchronize()
    quant_ms = e0.elapsed_time(e1) / reps
    quant_gbs = nuq_quantize_bytes(w, N) / (quant_ms * 1e-3) / 1e9
    del ws_q, k_src, v_src
    torch.cuda.empty_cache()
    c.c.n_packed, c.c.n_resid = N, 0

    q = torch.empty((B, Hq, 1, D), dtype=torch.int16, device=dev)
    S.fill_device(q, w.seed, S.TID_Q, B, Hq, 1, D)    # any query: timing does not depend on it
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    wsd = K.kvq_workspace_bytes(c.c, Hq, K.KVQ_OP_DECODE_ATTN)
    ws_d = torch.empty(max(wsd, 16), dtype=torch.uint8, device=dev)
    sm = 1.0 / math.sqrt(D)

    def decode():
        K.kvq_decode_attn(c.c, q, Hq, sm, w.rope_theta, out, ws_d, wsd)

    for _ in range(max(warmup, 1)):
        decode()
    torch.cuda.synchronize()
    per_replay = 4
    step_graph, dec_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(step_graph, stream=cap_stream):
            for _ in range(steps):
                decode()
        with torch.cuda.graph(dec_graph, stream=cap_stream):
            for _ in range(per_replay):
                decode()
    torch.cuda.synchronize()
    wall, dev_s = timed_steps(step_graph, steps, stream)
    dec_graph.replay()
    mean_dec_s, pct = time_replays(dec_graph, MIN_DECODE_REPLAYS, per_replay, stream)
    nbytes = nuq_decode_bytes(w, N)
    gbs = nbytes / mean_dec_s / 1e9
    res = {
        "workload": (f"{w.name}: batch {B}, {Hq} heads, head_dim {D}, {N} tokens, "
                     f"nuq{w.k_bits} keys per channel pre-RoPE with {w.outlier_bp / 100:g}% CSR "
                     f"outliers, nuq{w.v_bits} values per token"
                     + (f" with {w.v_outlier_bp / 100:g}% outliers" if w.v_outlier_bp else "")
                     + (", Q-Norm" if w.qnorm else "") + f", RoPE theta {w.rope_theta:g}"),
        "steps": steps, "ms_per_step": round(wall / steps * 1e3, 5),
        "ms_per_step_device": round(dev_s / steps * 1e3, 5),
        "decode_us": round(mean_dec_s * 1e6, 3),
        "decode_us_p10_p50_p90": [round(x * 1e6, 3) for x in pct],
        "decode_replays": MIN_DECODE_REPLAYS, "decodes_per_replay": per_replay,
        "decode_gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_ctx_per_s": round(B * N / mean_dec_s, 1),
        "quantize_gbs": round(quant_gbs, 1), "quantize_ms_prefill": round(quant_ms, 3),
        "kernel": "decode_nuq_kernel", "bytes_per_launch": nbytes,
        "traffic": measured_traffic("decode_nuq_kernel", w.name),
    }
    del c, ws_d
    torch.cuda.empty_cache()
    return res


def copy_calibration(mib: int) -> dict:
    """A plain device-to-device copy of ``mib`` MiB, five times: the known-size reference
    for the FETCH_SIZE and WRITE_SIZE counters."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}


def copy_bandwidth(mib: int = 1024) -> float:
    """GB/s of a plain device-to-device copy (bytes read + bytes written): the streaming
    rate this machine reaches outside the library, reported next to the 8 TB/s peak."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 10
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / t / 1e9


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="steps in the timed region")
    ap.add_argument("--warmup", type=int, default=5, help="untimed eager steps before it")
    ap.add_argument("--workload", nargs="*", default=None,
                    help=f"workloads to run (default: {' '.join(DEFAULT_WORKLOADS)})")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=6.0,
                    help="seconds of timed oracle work per workload and leg")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain copy of this size (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the path shards by "
              f"(batch, kv head) with no communication, and no multi-GPU run is built",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    names = list(args.workload) if args.workload else list(DEFAULT_WORKLOADS)

    # The CPU baseline's workers come from a fork server started now, before the first GPU
    # call: no process that has touched the GPU ever forks or execs.
    cpu = not args.no_cpu_baseline and not args.copy_calibration_mib
    ctx = None
    single_handles = {}
    if cpu:
        ctx = mp.get_context("forkserver")
        ctx.set_forkserver_preload([])
        p = ctx.Process(target=time.sleep, args=(0,))
        p.start()
        p.join()
        # The 1-thread legs (one process per workload, each on one core of the host's
        # share) run beside the GPU measurements; the all-cores legs run after them.
        for n in names:
            single_handles[n] = start_cpu_leg(ctx, n, 1, args.cpu_budget)

    import torch

    import decode_attention_10_amd as K  # noqa: F401  (fails loudly without the library)
    import kvq_synth as S
    if args.copy_calibration_mib:
        print(json.dumps(copy_calibration(args.copy_calibration_mib)))
        return 0
    torch.cuda.set_device(0)

    results = {}
    for n in names:
        w = S.WORKLOADS[n]
        print(f"[bench] {n}", file=sys.stderr, flush=True)
        results[n] = (gpu_nuq if w.kind == "nuq" else gpu_uniform)(w, args.steps, args.warmup)
    copy_gbs = copy_bandwidth()

    cores = cpu_cores()
    if cpu:
        single = {}
        for n in names:
            single[n] = finish_cpu_leg(single_handles[n], n)
        print("[bench] 1-thread oracle legs done", file=sys.stderr, flush=True)
        for n in names:
            print(f"[bench] oracle on {cores} cores: {n}", file=sys.stderr, flush=True)
            allc = finish_cpu_leg(start_cpu_leg(ctx, n, cores, args.cpu_budget), n)
            results[n]["cpu_baseline"] = {"single_thread": single[n], "all_cores": allc}

    head = HEADLINE if HEADLINE in results else names[-1]
    h = results[head]
    res = {
        "metric": METRIC,
        "value": h["decode_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": h["steps"],
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": h["workload"]},
        "decode_us": h["decode_us"], "decode_us_p10_p50_p90": h["decode_us_p10_p50_p90"],
        "tokens_ctx_per_s": h["tokens_ctx_per_s"], "quantize_gbs": h["quantize_gbs"],
        "copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(h["decode_gbs"] / copy_gbs, 4),
        "roofline": {"bound": "hbm", "achieved": h["decode_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": h["frac_of_peak"], "traffic": h["traffic"],
                     "kernel": h["kernel"], "bytes_per_launch": h["bytes_per_launch"]},
    }
    if cpu:
        cb = results[head]["cpu_baseline"]
        a = cb["all_cores"]
        res["cpu_baseline"] = {"value": a["decode_gbs"], "unit": "GB/s", "cores": a["cores"],
                               "kind": "oracle", "sample": a["sample"],
                               "single_thread": {"value": cb["single_thread"]["decode_gbs"],
                                                 "cores": 1,
                                                 "sample": cb["single_thread"]["sample"]}}
    res["workloads"] = results
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
