"""Benchmark of the packed-KV decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one decode step of one layer: append the new token's K/V to the fp16
window (every 128th step the window is full and is first quantized into the packed
cache: the per-channel key and per-token value quantizers) and then decode attention
over the whole cache.  The layer caches rotate (several copies, > 768 MB in all) so
that every step streams its cache from HBM rather than from the 256 MB Infinity
Cache.  Each layer's state is restored after its step, so every decode sees the
configured context.

The launch-bound step loop is captured in HIP graphs (one round of 128 steps per
graph) and the timed region replays them, so ms_per_step is GPU time, not Python
launch overhead.

Printed: one JSON line.  value = decode-attention GB/s: algorithmic bytes of codes,
metadata, fp16 window, q and out per decode / mean decode time, from HIP events on
the launch stream around replays of a decode-only graph (kernel plus the small gap
between launches); p10 / p50 / p90 of the per-replay means beside it.  Also
tokens*ctx/s, prefill quantize GB/s, the roofline of the decode kernel, the rate of a
plain 1 GiB device copy on the same box (and value as a fraction of it) and the oracle
timed on a bounded host sample.  KVQuant-style workloads (--workload kvquant_...) time
one decode per step over a one-shot quantized context.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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


def uniform_decode_kernel(w) -> str:
    """The decode kernel the library runs for a uniform cache: the matrix-core kernel for 2
    or 4 query heads per kv head, else the vector kernel."""
    return "decode_gqa_kernel" if w.q_heads // w.kv_heads in (2, 4) else "decode_uniform_kernel"


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


def time_replays(graph, rounds: int, per_replay: int, stream):
    """Replays ``graph`` ``rounds`` times with HIP events on ``stream`` around each replay.
    Returns (mean seconds per step over the whole run, [p10, p50, p90] of the per-replay
    mean step time)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(rounds + 1)]
    ev[0].record(stream)
    for i in range(rounds):
        graph.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e-3 / per_replay for i in range(rounds)])
    mean = ev[0].elapsed_time(ev[rounds]) * 1e-3 / (rounds * per_replay)
    return mean, [float(np.percentile(per, q)) for q in (10, 50, 90)]


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


def decode_bytes(w, n_packed: int, n_resid: int) -> int:
    """Algorithmic bytes one decode launch must move: packed codes and metadata, the fp16
    window and attention-sink tokens, q and the fp32 output."""
    bh = w.batch * w.kv_heads
    D = w.head_dim
    codes = bh * n_packed * D * (w.k_bits + w.v_bits) // 8
    meta = bh * (n_packed // 32) * D * 4 + bh * n_packed * (D // 32) * 4
    window = 2 * bh * (n_resid + w.sink_len) * D * 2
    return codes + meta + window + w.batch * w.q_heads * D * (2 + 4)


def nuq_decode_bytes(w, n_packed: int) -> int:
    """Algorithmic bytes of one decode over a nuq cache: B-bit codes of K and V, per-channel
    key metadata, per-token value metadata, the CSR of key outliers (row pointers and one
    4-byte entry per outlier), the value outliers (4 bytes each), q and out."""
    bh = w.batch * w.kv_heads
    D = w.head_dim
    k_out = (n_packed * w.outlier_bp + 9999) // 10000
    v_out = (D * w.v_outlier_bp + 9999) // 10000
    codes = bh * n_packed * D * (w.k_bits + w.v_bits) // 8
    meta = bh * D * 4 + bh * n_packed * 4
    csr = (bh * (n_packed + 1) * 4 + bh * D * k_out * 4) if w.outlier_bp else 0
    return codes + meta + csr + bh * n_packed * v_out * 4 + w.batch * w.q_heads * D * (2 + 4)


def nuq_quantize_bytes(w, n_tokens: int) -> int:
    """One-shot nuq quantize: fp16 K and V read once, codes, metadata and CSR written."""
    bh = w.batch * w.kv_heads
    D = w.head_dim
    k_out = (n_tokens * w.outlier_bp + 9999) // 10000
    read = 2 * bh * n_tokens * D * 2
    written = bh * n_tokens * D * (w.k_bits + w.v_bits) // 8 + bh * D * 4 + bh * n_tokens * 4
    if w.outlier_bp:
        written += bh * (n_tokens + 1) * 4 + bh * D * k_out * 4
    written += bh * n_tokens * ((D * w.v_outlier_bp + 9999) // 10000) * 4
    return read + written


def quantize_bytes(w, n_tokens: int) -> int:
    """Prefill quantize: fp16 K and V read, packed codes and metadata written."""
    bh = w.batch * w.kv_heads
    D = w.head_dim
    read = 2 * bh * n_tokens * D * 2
    written = bh * n_tokens * D * (w.k_bits + w.v_bits) // 8 + \
        bh * (n_tokens // 32) * D * 4 + bh * n_tokens * (D // 32) * 4
    return read + written


def cpu_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w, budget_s: float = 40.0, timed_min_s: float = 10.0,
                 keep_units: int = 32) -> dict:
    """The oracle (unchanged) on a bounded sample: whole (batch, kv head) units of the same
    workload.  Per unit the oracle builds the packed cache from host-generated K/V (setup,
    untimed), then the timed part unpacks it, dequantizes and runs float64 attention.  The
    first pass goes over the units until ``budget_s`` of wall time; if its timed part is
    under ``timed_min_s``, the timed part is repeated over the first ``keep_units`` units'
    prepared inputs until it reaches that (or the wall budget ends).  One thread (BLAS
    pinned to 1)."""
    from threadpoolctl import threadpool_limits

    import kvq_synth as S
    from oracle import kvq_oracle as O
    T = w.ctx
    S0, S1 = w.sink_len, w.sink_len + w.n_packed
    g = w.gains()
    sm = O.default_sm_scale(w.head_dim)
    gq = w.q_heads // w.kv_heads
    done, runs, t_used, nbytes = 0, 0, 0.0, 0
    per_unit = decode_bytes(w, w.n_packed, w.n_resid) // (w.batch * w.kv_heads)
    kept = []

    def timed(k, v, q, c):
        t0 = time.perf_counter()
        kc = O.unpack_k_codes(c["k_codes"], w.k_bits, w.head_dim)
        vc = O.unpack_v_codes(c["v_codes"], w.v_bits)
        ks, km = O.unpack_meta(c["k_meta"])
        vs, vm = O.unpack_meta(c["v_meta"])
        kd = O.dequant_keys_per_channel(kc, ks, km)
        vd = O.dequant_values_per_token(vc, vs, vm)
        kd = np.concatenate([O.f16_to_f32(k[:, :, :S0]), kd, O.f16_to_f32(k[:, :, S1:])],
                            axis=2)
        vd = np.concatenate([O.f16_to_f32(v[:, :, :S0]), vd, O.f16_to_f32(v[:, :, S1:])],
                            axis=2)
        O.decode_attention_f64(O.f16_to_f32(q), kd, vd, sm)
        return time.perf_counter() - t0

    wall0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - wall0 < budget_s and done < w.batch * w.kv_heads:
            b, h = divmod(done, w.kv_heads)
            k = S.gen_tensor(w.seed, S.TID_K, w.batch, w.kv_heads, T, w.head_dim, gains=g,
                             heads_sel=[h], batch_sel=[b])
            v = S.gen_tensor(w.seed, S.TID_V, w.batch, w.kv_heads, T, w.head_dim,
                             heads_sel=[h], batch_sel=[b])
            q = S.gen_tensor(w.seed, S.TID_Q, w.batch, w.q_heads, 1, w.head_dim,
                             heads_sel=list(range(h * gq, (h + 1) * gq)), batch_sel=[b])[:, :, 0]
            c = O.uniform_cache(k, v, w.k_bits, w.v_bits, w.n_packed, w.n_resid,
                                n_sink=w.sink_len)
            if len(kept) < keep_units:
                kept.append((k, v, q, c))
            t_used += timed(k, v, q, c)
            nbytes += per_unit
            done += 1
            runs += 1
        i = 0
        while t_used < timed_min_s and time.perf_counter() - wall0 < budget_s and kept:
            t_used += timed(*kept[i % len(kept)])
            nbytes += per_unit
            runs += 1
            i += 1
    return {"value": round(nbytes / t_used / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{runs} unit decodes over {done} of {w.batch * w.kv_heads} (batch, kv "
                      f"head) units of {w.name} (after one pass over the units, repeats over "
                      f"the first {min(len(kept), done)}): unpack + dequantize + float64 "
                      f"attention, {t_used:.1f} s timed on 1 thread of {cpu_cores()} available"}


def bench_nuq(w, args) -> dict:
    """KVQuant-style workload: one-shot quantize of the whole context (timed as the
    quantize rate), then decode steps over it (a step is one decode; there is no
    streaming window), replayed from a HIP graph."""
    import torch

    import decode_attention_10_amd as K
    import kvq_synth as S
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    B, Hkv, Hq, D, N = w.batch, w.kv_heads, w.q_heads, w.head_dim, w.n_packed
    gains = torch.from_numpy(w.gains()).to(dev)
    k_src = torch.empty((B, Hkv, N, D), dtype=torch.int16, device=dev)
    v_src = torch.empty_like(k_src)
    S.fill_device(k_src, w.seed, S.TID_K, B, Hkv, N, D, gains=gains)
    S.fill_device(v_src, w.seed, S.TID_V, B, Hkv, N, D)
    lut = torch.from_numpy(S.nuq_lut(w.k_bits).view(np.int16)).to(dev)
    c = K.KVCache(B, Hkv, N, k_bits=w.k_bits, v_bits=w.v_bits, residual_len=0, kind=K.KVQ_NUQ,
                  lut=lut,
                  outlier_bp=w.outlier_bp, v_outlier_bp=w.v_outlier_bp, qnorm=w.qnorm)
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

    round_len = 16
    for _ in range(2):
        decode()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(g, stream=cap_stream):
            for _ in range(round_len):
                decode()
    torch.cuda.synchronize()
    rounds = max(1, args.steps // round_len)
    steps = rounds * round_len
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    mean_dec_s, pct = time_replays(g, rounds, round_len, stream)
    wall = time.perf_counter() - t0
    nbytes = nuq_decode_bytes(w, N)
    copy_gbs = copy_bandwidth()
    gbs = nbytes / mean_dec_s / 1e9
    return {
        "metric": "decode-attn HBM GB/s on packed KV (% of peak); tokens*ctx/s; quantize GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {B}, {Hq} heads, head_dim {D}, {N} tokens, "
                               f"nuq{w.k_bits} keys per channel pre-RoPE with "
                               f"{w.outlier_bp / 100:g}% CSR outliers, nuq{w.v_bits} values per "
                               f"token"
                               + (f" with {w.v_outlier_bp / 100:g}% outliers"
                                  if w.v_outlier_bp else "")
                               + (", Q-Norm" if w.qnorm else "")
                               + f", RoPE theta {w.rope_theta:g}"},
        "decode_us": round(mean_dec_s * 1e6, 3),
        "decode_us_p10_p50_p90": [round(x * 1e6, 3) for x in pct],
        "decode_bytes": nbytes,
        "copy_gbs": round(copy_gbs, 1),
        "frac_of_copy": round(gbs / copy_gbs, 4),
        "tokens_ctx_per_s": round(B * N / mean_dec_s, 1),
        "quantize_gbs": round(quant_gbs, 1),
        "quantize_ms_prefill": round(quant_ms, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_nuq_kernel", w.name),
                     "kernel": "decode_nuq_kernel", "bytes_per_launch": nbytes},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024, help="rounded down to whole rounds of 128")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="llama2_7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-rotation-mb", type=float, default=768.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain copy of this size (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the path shards by "
              f"(batch, kv head) with no communication, and no multi-GPU run is built",
              file=sys.stderr)
        return 2
    if args.copy_calibration_mib:
        print(json.dumps(copy_calibration(args.copy_calibration_mib)))
        return 0

    import torch

    import decode_attention_10_amd as K
    import kvq_synth as S
    w = S.WORKLOADS[args.workload]
    if w.kind == "nuq":
        res = bench_nuq(w, args)
        print(json.dumps(res))
        return 0
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    B, Hkv, Hq, D, N, R = w.batch, w.kv_heads, w.q_heads, w.head_dim, w.n_packed, w.residual_len
    S0 = w.sink_len                      # tokens [0, S0) in the fp16 sink, packed from S0
    T = w.ctx
    cap = N + R

    # ---- inputs on the device (generator kernel), prefill into the layer copies
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
    layers = max(1, math.ceil(args.min_rotation_mb * 1e6 / per_layer))
    caches = []
    sT = (B, Hkv * (T + 1) * D, (T + 1) * D, D)
    k_pk, v_pk = k_src[:, :, S0:], v_src[:, :, S0:]      # first packed token
    for _ in range(layers):
        c = K.KVCache(B, Hkv, cap, k_bits=w.k_bits, v_bits=w.v_bits, residual_len=R,
                      sink_len=S0)
        K.kvq_quantize_keys(c.c, k_pk, sT[1], sT[2], sT[3], 0, N)
        K.kvq_quantize_values(c.c, v_pk, sT[1], sT[2], sT[3], 0, N)
        kr = c.buf("k_resid").view(torch.int16).view(B, Hkv, R, D)
        vr = c.buf("v_resid").view(torch.int16).view(B, Hkv, R, D)
        kr[:, :, :w.n_resid] = k_src[:, :, S0 + N:T]
        vr[:, :, :w.n_resid] = v_src[:, :, S0 + N:T]
        if S0:
            c.buf("k_sink").view(torch.int16).view(B, Hkv, S0, D)[:] = k_src[:, :, :S0]
            c.buf("v_sink").view(torch.int16).view(B, Hkv, S0, D)[:] = v_src[:, :, :S0]
            c.c.n_sink = S0
        caches.append(c)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws_bytes = K.kvq_workspace_bytes(caches[0].c, Hq, K.KVQ_OP_DECODE_ATTN)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    sm = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()

    # prefill quantize rate (keys + values over the whole packed context), own copy
    qc = K.KVCache(B, Hkv, cap, k_bits=w.k_bits, v_bits=w.v_bits, residual_len=R)

    def prefill():
        K.kvq_quantize_keys(qc.c, k_pk, sT[1], sT[2], sT[3], 0, N)
        K.kvq_quantize_values(qc.c, v_pk, sT[1], sT[2], sT[3], 0, N)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        prefill()
    reps = 20
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)          # host enqueues behind a busy GPU
    e0.record(stream)
    for _ in range(reps):
        prefill()
    e1.record(stream)
    torch.cuda.synchronize()
    quant_ms = e0.elapsed_time(e1) / reps
    quant_gbs = quantize_bytes(w, N) / (quant_ms * 1e-3) / 1e9
    del qc

    # ---- the step: append (flush every R-th step) + decode, layers rotating.  A round of
    # R steps is captured in a HIP graph (launch-bound loop -> one graph launch); the
    # captured kernel arguments fix each step's cache state, restored after the step.
    def step(i: int) -> int:
        c = caches[i % layers].c
        flush = (i % R) == R - 1
        c.n_packed, c.n_resid = N, (R if flush else w.n_resid - 1)
        K.kvq_append_flush(c, k_new, v_new)
        nbytes = decode_bytes(w, int(c.n_packed), int(c.n_resid))
        K.kvq_decode_attn(c, q, Hq, sm, 0.0, out, ws, ws_bytes)
        c.n_packed, c.n_resid = N, w.n_resid
        return nbytes

    def decode_only(i: int) -> None:
        K.kvq_decode_attn(caches[i % layers].c, q, Hq, sm, 0.0, out, ws, ws_bytes)

    cap_stream = torch.cuda.Stream()
    round_len = R
    step_graph, dec_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    for i in range(round_len):                 # eager warm-up of every step shape
        step(i)
    torch.cuda.synchronize()
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(step_graph, stream=cap_stream):
            nbytes = [step(i) for i in range(round_len)]
        with torch.cuda.graph(dec_graph, stream=cap_stream):
            for i in range(round_len):
                decode_only(i)
    torch.cuda.synchronize()
    rounds = max(1, args.steps // round_len)
    steps = rounds * round_len
    for _ in range(max(1, args.warmup // round_len)):
        step_graph.replay()
        dec_graph.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(rounds):
        step_graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # decode kernel time: events around replays of the decode-only graph
    mean_dec_s, pct = time_replays(dec_graph, rounds, round_len, stream)
    copy_gbs = copy_bandwidth()
    dec_bytes = decode_bytes(w, N, w.n_resid)
    gbs = dec_bytes / mean_dec_s / 1e9
    tok_ctx = B * T / mean_dec_s

    res = {
        "metric": "decode-attn HBM GB/s on packed KV (% of peak); tokens*ctx/s; quantize GB/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {B}, {Hq} q / {Hkv} kv heads, head_dim {D}, "
                               + (f"{S0} fp16 sink + " if S0 else "")
                               + f"{N} packed + {w.n_resid} fp16 window tokens, K int{w.k_bits} "
                               f"per-channel / V int{w.v_bits} per-token, group 32",
                   "layers_rotated": layers, "flush_every": R},
        "decode_us": round(mean_dec_s * 1e6, 3),
        "decode_us_p10_p50_p90": [round(x * 1e6, 3) for x in pct],
        "copy_gbs": round(copy_gbs, 1),
        "frac_of_copy": round(gbs / copy_gbs, 4),
        "step_bytes_mean": int(np.mean(nbytes)),
        "tokens_ctx_per_s": round(tok_ctx, 1),
        "quantize_gbs": round(quant_gbs, 1),
        "quantize_ms_prefill": round(quant_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(uniform_decode_kernel(w), w.name),
                     "kernel": uniform_decode_kernel(w), "bytes_per_launch": dec_bytes},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
