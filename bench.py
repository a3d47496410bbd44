#!/usr/bin/env python3
"""Benchmark: causal prefill attention + KV-cache write on one MI355X.

One step = one call of prefill_attn_varlen (C ABI, one fused kernel launch)
over the Llama-2-7B-shaped layer: one sequence of T=2048 tokens, 32 heads x
128, bf16 q/k/v ~ N(0,1) from a seed, scale 1/sqrt(128), K/V cache
[1, 32, 2048, 128] written in the same launch.  Inputs are resident in HBM
before the timed region.  Prints one JSON line.

  value     = algorithmic FLOPs per step / mean step time (TFLOP/s); the
              algorithmic FLOPs count 4*D per causal (query, key) pair per head
              (QK^T and PV, 2*D each), the masked half excluded.
  roofline  = the same FLOPs / the kernel's average launch duration (the timed
              steps are single launches, back to back between two HIP events
              on the launch stream), against the dense bf16 MFMA peak
              (2.5 PFLOP/s);
              traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE and
              WRITE_SIZE counters (profiles/), scaled by a copy-kernel
              calibration, or null if the kernel source changed since.
  cpu_baseline = the float64 oracle on the host cores over the same workload.

Context fields (not part of value): cold and warm (median and p99 per
launch: cold after a 1 GiB fill that evicts L2 and the Infinity Cache before
every launch, warm back to back), measured_mfma_peak (the bf16 matrix-core
rate measured in-process by a small MFMA-loop kernel with random operands,
and with constant ones, each with its shader clock, and value as a
percentage of the random-operand rate), kernel_clock (the shader clock over
the attention kernel's loop and its phase times, from a measurement build
with per-wave clock stamps) with mfma_peak_at_kernel_clock (the published
dense rate scaled to that clock), hbm_copy_measured (a plain 1 GiB device copy),
gemm_bf16_context (a large hipBLASLt bf16 GEMM at the run's clock; it and
the MFMA peak run before the attention's warm-up, so the timed steps start
at the clock the matrix cores sustain, not while it ramps up from idle),
other_configs (the varlen batch of three prompts, the long-context mix and
the chunked workload's heaviest step, on inputs drawn on the device),
int8_cache and fp8_cache (the same step writing an INT8 or E4M3 cache).  The chunked workloads
report the heaviest step (value: through split-KV; also one-pass and paged), the decode rows alone,
and every step summed (all_steps_splitkv) with the prompt's chunks alone
against one varlen call over the whole prompt.

Options: --gpus N (only 1 is supported: the path runs on one GPU),
--steps K, --warmup W, --workload NAME, --no-cpu-baseline,
--no-other-configs, --kernel-only (only the attention step's timed launches,
for profiler runs), --copy-calib (runs only a 1 GiB device copy, for the
counter calibration).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "prefill_self_attention_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd64_T2048_H32_D128.txt")
METRIC = "prefill attention TFLOP/s + % bf16 MFMA peak (T=2048,H=32,D=128); KV GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the GPU's clocks ramp up over the first few hundred launches after idle;
    # the default warmup lets the timed steps run at the sustained clock
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="single_T2048_H32_D128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--kernel-only", action="store_true",
                    help="time only the attention step (warm-up, timed steps, per-launch pass): for profiler runs")
    ap.add_argument("--copy-calib", action="store_true")
    return ap.parse_args()


def causal_pairs(lengths, prefixes=None):
    prefixes = prefixes or [0] * len(lengths)
    return sum(n * p + n * (n + 1) // 2 for n, p in zip(lengths, prefixes))


def kernel_sha():
    """SHA-256 over every kernel source (csrc/*.hip, *.h, the generator), in
    name order: a profile taken on other sources is stale."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".py")):
            h.update(name.encode() + b"\0")
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def hbm_copy_rate(n_bytes=1 << 30, reps=10):
    """Read + write bytes per second of a plain contiguous device copy."""
    import torch
    src = torch.ones(n_bytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    ms = timed_steps(lambda: dst.copy_(src), reps, 3)
    del src, dst
    gbps = 2.0 * n_bytes / (ms * 1e-3) / 1e9
    return {"gbps_read_plus_write": round(gbps, 1), "frac_of_hbm_8tbs": round(gbps / PEAK_HBM_GBPS, 3),
            "bytes_each_way": n_bytes}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def measured_mfma_peak(blocks=2048, iters=4000, reps=5):
    """The bf16 MFMA rate measured on this part: the probe library's
    back-to-back v_mfma_f32_32x32x16_bf16 loop (8 independent accumulators
    per wave, 4 waves per work-group, 8 work-groups per CU), best of a few
    launches, with random operands (the power real data draws; the part then
    runs a lower shader clock) and with constant ones, each with the median
    shader clock of its work-groups (s_memtime cycles over s_memrealtime
    time)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "prefill_self_attention_amd", "libpa_mfma_peak.so")
    lib = ctypes.CDLL(path)
    lib.pa_mfma_peak_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    lib.pa_mfma_peak_run.restype = ctypes.c_int
    lib.pa_mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.pa_mfma_peak_flops.restype = ctypes.c_double
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def run(random_operands):
        best = None
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if lib.pa_mfma_peak_run(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clk.data_ptr()), blocks, iters,
                                    random_operands, sp) != 0:
                raise RuntimeError("mfma peak probe failed to launch")
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            if r > 0 and (best is None or ms < best[0]):
                c = clk.view(blocks, 4).cpu()
                mhz = _median(((c[:, 3] - c[:, 2]).double() / ((c[:, 1] - c[:, 0]).double() / 100.0)).tolist())
                best = (ms, mhz)
        tflops = lib.pa_mfma_peak_flops(blocks, iters) / (best[0] * 1e-3) / 1e12
        return {"tflops": round(tflops, 1), "pct_of_published_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 1),
                "shader_clock_mhz": round(best[1]), "launch_ms": round(best[0], 3)}

    rnd = run(1)
    const = run(0)
    return dict(rnd, operands="random bf16 in [-1, 1), four register sets cycled",
                kernel="v_mfma_f32_32x32x16_bf16, 8 independent accumulators per wave, %d work-groups of 4 waves"
                % blocks, constant_operands=const)


def kernel_clock(args_fn, n_launch=30):
    """Shader clock and phase times of the 64-row kernel on this workload:
    the measurement build of the library (libprefill_attn_clock.so, the same
    sources with per-wave clock stamps) runs the same varlen call
    (args_fn() -> the ctypes arguments of prefill_attn_varlen_gqa) n_launch
    times back to back; from the last launch's stamps: the median (and
    per-XCD) shader clock over each wave's loop, and the median prologue,
    loop and epilogue times and the span from the first wave's start to the
    last wave's end."""
    import ctypes
    import numpy as np
    import torch
    path = os.path.join(ROOT, "prefill_self_attention_amd", "libprefill_attn_clock.so")
    lib = ctypes.CDLL(path)
    f = lib.prefill_attn_varlen_gqa
    p_, i32 = ctypes.c_void_p, ctypes.c_int32
    f.argtypes = [p_, p_, p_, p_, i32, i32, i32, i32, i32, p_, p_, p_, ctypes.c_float, p_]
    f.restype = ctypes.c_int
    lib.pa_fwd64_clock_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    lib.pa_fwd64_clock_stamps.restype = ctypes.c_int
    for _ in range(n_launch):
        if f(*args_fn()) != 0:
            raise RuntimeError("clock-stamp build: launch failed")
    torch.cuda.synchronize()
    n = 1 << 16
    buf = np.zeros(8 * n, dtype=np.uint64)
    if lib.pa_fwd64_clock_stamps(ctypes.c_void_p(buf.ctypes.data), n) != 0:
        raise RuntimeError("clock-stamp build: copy failed")
    st = buf.reshape(n, 8).astype(np.int64)
    idx = np.nonzero(st[:, 0])[0]
    st = st[idx]
    if len(st) == 0:
        return None
    real = (st[:, :4] - st[:, 0].min()) / 100.0          # microseconds
    cyc = st[:, 4:]
    loop_us = real[:, 2] - real[:, 1]
    mhz = (cyc[:, 2] - cyc[:, 1]) / np.maximum(loop_us, 1e-3)
    xcd = (idx // 4) % 8
    return {"waves": int(len(st)),
            "loop_shader_clock_mhz": {"median": round(float(np.median(mhz))), "min": round(float(mhz.min())),
                                      "max": round(float(mhz.max())),
                                      "per_xcd_median": [round(float(np.median(mhz[xcd == x]))) for x in range(8)]},
            "median_us": {"prologue": round(float(np.median(real[:, 1] - real[:, 0])), 2),
                          "loop": round(float(np.median(loop_us)), 2),
                          "epilogue": round(float(np.median(real[:, 3] - real[:, 2])), 2)},
            "loop_us_min_max": [round(float(loop_us.min()), 2), round(float(loop_us.max()), 2)],
            "span_first_start_to_last_end_us": round(float(real[:, 3].max()), 2),
            "library": "libprefill_attn_clock.so (measurement build, per-wave s_memtime / s_memrealtime stamps)"}


def read_traffic():
    """HBM bytes per launch from the committed counter summary, if it is current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha256") != kernel_sha():
        return None, "kernel changed since the counters were taken"
    try:
        f = float(kv["fetch_kib_per_dispatch"]) * float(kv["copy_fetch_factor"])
        w = float(kv["write_kib_per_dispatch"]) * float(kv["copy_write_factor"])
    except (KeyError, ValueError):
        return None, "incomplete counter summary"
    return (f + w) * 1024.0, "ok"


def copy_calib():
    import torch
    n = 1 << 29  # 2^29 bf16 = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_each_way": 2 * n, "launches": 3}), flush=True)


def cpu_baseline(w, q, k, v, flops):
    """Time the float64 oracle on the host cores over the same workload."""
    import oracle
    oracle._load()
    t0 = time.perf_counter()
    oracle.prefill_varlen(q, k, v, w.cu_seqlens, w.scale)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": "the whole workload (%d tokens x %d heads x %d), float64, one run"
                      % (w.num_tokens, w.num_heads, w.head_dim)}


def timed_steps(fn, steps, warmup):
    """Mean time (ms) of one call of fn: `steps` calls back to back on the
    current stream, bracketed by two events (nothing recorded between them)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def launch_times(fn, steps):
    """Sorted per-call times (ms), each call between its own pair of events.
    A separate pass: the event records between calls serialise the stream and
    add a few microseconds per call, so these are not used for the step time."""
    import torch
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)


def timed(fn, steps, warmup):
    """Mean time per call (ms, back to back) and sorted per-call times."""
    ms = timed_steps(fn, steps, warmup)
    return ms, launch_times(fn, steps)


def cold_launch_times(fn, steps, flush_bytes=1 << 30):
    """Sorted per-call times (ms) with L2 and the 256 MB Infinity Cache evicted
    before every call by a 1 GiB device fill (outside the events)."""
    import torch
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        flush.zero_()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    del flush
    return sorted(a.elapsed_time(b) for a, b in evs)


def stats_us(ms_sorted):
    n = len(ms_sorted)
    return {"median": round(ms_sorted[n // 2] * 1e3, 2),
            "p99": round(ms_sorted[min(n - 1, int(math.ceil(0.99 * n)) - 1)] * 1e3, 2)}


def gemm_context(n=8192, steps=20):
    """A large plain bf16 GEMM through torch (hipBLASLt), back to back: the
    matrix rate this part sustains at the clock of the run, as context for the
    published dense peak (not a roofline denominator)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda", generator=g)
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda", generator=g)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    ms = timed_steps(lambda: torch.matmul(a, b, out=c), steps, 5)
    del a, b, c
    return {"shape": [n, n, n], "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}


def other_configs(P, steps=20, warmup=5):
    """The other configurations, each timed on inputs drawn on the device
    (N(0,1) bf16, no host copy, no CPU oracle): the varlen batch of three
    prompts, the long-context mix, and the chunked workload's heaviest step
    (last 512-token chunk of the 8192-token prompt beside 64 decode rows)
    through split-KV and through the one-pass call, with the 64 decode rows
    alone as GB/s of cached K/V read."""
    import torch
    from prefill_self_attention_amd import inputs as I
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(11)

    def rnd(*shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    res = {}
    for name, st, wu in (("varlen_10_50_2048_H32_D128", steps, warmup),
                         ("longmix_65536_plus_32768_H32_D128", 5, 2)):
        w = I.workload(name)
        N, H, HK, D = w.num_tokens, w.num_heads, w.num_kv_heads, w.head_dim
        q, k, v = rnd(N, H, D), rnd(N, HK, D), rnd(N, HK, D)
        kc, vc, out = torch.empty_like(k), torch.empty_like(v), torch.empty_like(q)
        cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device=dev)

        def fn():
            P.prefill_attn_varlen(q, k, v, cu, kc, vc, out, scale=w.scale, max_seqlen=w.max_seqlen)

        ms = timed_steps(fn, st, wu)
        flops = 4.0 * D * H * causal_pairs(w.lengths)
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"us_per_step": round(ms * 1e3, 2), "tflops": round(tf, 1),
                     "pct_bf16_mfma_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
                     "tokens": N, "sequences": len(w.lengths), "steps": st, "warmup": wu}
        del q, k, v, kc, vc, out
    # chunked: heaviest step
    wl = I.workload("chunked_8192x512_plus_64_decode_H32_D128")
    H, HK, D, R = wl.num_heads, wl.num_kv_heads, wl.head_dim, len(wl.contexts)
    c = wl.num_chunks - 1
    stp = wl.step(c)
    kc = rnd(1 + R, HK, wl.cap, D)
    vc = rnd(1 + R, HK, wl.cap, D)
    T = stp.cu_seqlens[-1]
    q, k, v = rnd(T, H, D), rnd(T, HK, D), rnd(T, HK, D)
    out = torch.empty_like(q)
    cu = torch.tensor(stp.cu_seqlens, dtype=torch.int32, device=dev)
    pre = torch.tensor(stp.prefix_lens, dtype=torch.int32, device=dev)
    ws = torch.empty(P.splitkv_workspace_size(1 + R, T, H, D, wl.cap), dtype=torch.uint8, device=dev)

    def split_step():
        P.prefill_attn_chunked_splitkv(q, k, v, cu, kc, vc, out, pre, scale=stp.scale,
                                       max_seqlen=wl.chunk_len, workspace=ws)

    def one_pass_step():
        P.prefill_attn_chunked(q, k, v, cu, kc, vc, out, pre, scale=stp.scale, max_seqlen=wl.chunk_len)

    ms_split = timed_steps(split_step, steps, warmup)
    ms_one = timed_steps(one_pass_step, steps, warmup)
    flops = 4.0 * D * H * causal_pairs(stp.lengths, stp.prefix_lens)
    # decode rows alone (rows 1..R of the cache)
    qd, kd, vd = q[wl.chunk_len:], k[wl.chunk_len:], v[wl.chunk_len:]
    outd = torch.empty_like(qd)
    cud = torch.arange(R + 1, dtype=torch.int32, device=dev)
    pred = torch.tensor(wl.contexts, dtype=torch.int32, device=dev)
    kcd, vcd = kc[1:], vc[1:]
    wsd = torch.empty(P.splitkv_workspace_size(R, R, H, D, wl.cap), dtype=torch.uint8, device=dev)

    def decode_step():
        P.prefill_attn_chunked_splitkv(qd, kd, vd, cud, kcd, vcd, outd, pred, scale=stp.scale,
                                       max_seqlen=1, workspace=wsd)

    ms_dec = timed_steps(decode_step, steps, warmup)
    dec_bytes = 2.0 * sum(x + 1 for x in wl.contexts) * HK * D * 2
    res["chunked_8192x512_plus_64_decode_H32_D128"] = {
        "step": "chunk %d of %d (prefix %d) + %d decode rows" % (c, wl.num_chunks, c * wl.chunk_len, R),
        "splitkv": {"us_per_step": round(ms_split * 1e3, 2),
                    "tflops": round(flops / (ms_split * 1e-3) / 1e12, 1)},
        "one_pass": {"us_per_step": round(ms_one * 1e3, 2),
                     "tflops": round(flops / (ms_one * 1e-3) / 1e12, 1)},
        "decode_rows_alone": {"rows": R, "context_tokens": sum(wl.contexts),
                              "us_per_step": round(ms_dec * 1e3, 2),
                              "kv_read_gbps": round(dec_bytes / (ms_dec * 1e-3) / 1e9, 1),
                              "frac_of_hbm_8tbs": round(dec_bytes / (ms_dec * 1e-3) / 8e12, 4)},
        "steps": steps, "warmup": warmup}
    del kc, vc, q, k, v, out, ws, wsd
    torch.cuda.empty_cache()
    return res


def bench_chunked(args, wl, P):
    """The heaviest step of the chunked workload (last 512-token chunk of the
    8192-token prompt beside the 64 decode rows) and, separately, the 64
    decode rows alone: TFLOP/s over the step's causal pairs and the decode
    share as GB/s of cached K/V read."""
    import torch
    dev = torch.device("cuda:0")
    H, HK, D, R = wl.num_heads, wl.num_kv_heads, wl.head_dim, len(wl.contexts)
    t = wl.tensors()
    kc = torch.zeros((1 + R, HK, wl.cap, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    for r, ctx in enumerate(wl.contexts):
        kc[1 + r, :, :ctx] = t["pre_k"][r].to(dev)
        vc[1 + r, :, :ctx] = t["pre_v"][r].to(dev)
    c = wl.num_chunks - 1
    st = wl.step(c)
    sl = slice(c * wl.chunk_len, (c + 1) * wl.chunk_len)
    # the prompt's earlier chunks are already in the cache
    kc[0, :, :c * wl.chunk_len] = t["pk"][:c * wl.chunk_len].transpose(0, 1).to(dev)
    vc[0, :, :c * wl.chunk_len] = t["pv"][:c * wl.chunk_len].transpose(0, 1).to(dev)
    q = torch.cat([t["pq"][sl], t["dq"]]).to(dev)
    k = torch.cat([t["pk"][sl], t["dk"]]).to(dev)
    v = torch.cat([t["pv"][sl], t["dv"]]).to(dev)
    out = torch.empty_like(q)
    cu = torch.tensor(st.cu_seqlens, dtype=torch.int32, device=dev)
    pre = torch.tensor(st.prefix_lens, dtype=torch.int32, device=dev)

    def step():
        P.prefill_attn_chunked(q, k, v, cu, kc, vc, out, pre, scale=st.scale, max_seqlen=wl.chunk_len)

    ms = timed_steps(step, args.steps, args.warmup)
    pairs = causal_pairs(st.lengths, st.prefix_lens)
    flops = 4.0 * D * H * pairs
    # decode rows alone: rows 1..R of the cache, one new token each
    qd, kd, vd = t["dq"].to(dev), t["dk"].to(dev), t["dv"].to(dev)
    outd = torch.empty_like(qd)
    cud = torch.arange(R + 1, dtype=torch.int32, device=dev)
    pred = torch.tensor(wl.contexts, dtype=torch.int32, device=dev)
    kcd, vcd = kc[1:], vc[1:]

    def decode():
        P.prefill_attn_chunked(qd, kd, vd, cud, kcd, vcd, outd, pred, scale=st.scale, max_seqlen=1)

    msd = timed_steps(decode, args.steps, args.warmup)
    dec_bytes = 2.0 * sum(c_ + 1 for c_ in wl.contexts) * HK * D * 2  # K and V of every context row, once per K/V head

    # the same step and decode rows through the split-KV path (plan, attention
    # over key segments, merge), workspaces allocated before timing
    ws = torch.empty(P.splitkv_workspace_size(1 + R, q.shape[0], H, D, wl.cap), dtype=torch.uint8, device=dev)
    wsd = torch.empty(P.splitkv_workspace_size(R, R, H, D, wl.cap), dtype=torch.uint8, device=dev)

    def step_split():
        P.prefill_attn_chunked_splitkv(q, k, v, cu, kc, vc, out, pre, scale=st.scale,
                                       max_seqlen=wl.chunk_len, workspace=ws)

    def decode_split():
        P.prefill_attn_chunked_splitkv(qd, kd, vd, cud, kcd, vcd, outd, pred, scale=st.scale,
                                       max_seqlen=1, workspace=wsd)

    mss = timed_steps(step_split, args.steps, args.warmup)
    msds = timed_steps(decode_split, args.steps, args.warmup)

    # and over a paged cache: the same contents in 16-token blocks placed by
    # a seeded random permutation of the pool, located through a block table
    B = 1 + R
    mb = wl.cap // 16
    perm = torch.randperm(B * mb, generator=torch.Generator().manual_seed(7)).to(dev)
    bt = perm.view(B, mb).to(torch.int32).contiguous()

    def to_pages(slab):
        pages = torch.empty((B * mb, HK, 16, D), dtype=slab.dtype, device=dev)
        pages[perm] = slab.view(B, HK, mb, 16, D).permute(0, 2, 1, 3, 4).reshape(B * mb, HK, 16, D)
        return pages

    kp, vp = to_pages(kc), to_pages(vc)
    btd = bt[1:].contiguous()

    def step_paged():
        P.prefill_attn_chunked_splitkv_paged(q, k, v, cu, kp, vp, bt, out, pre, scale=st.scale,
                                             max_seqlen=wl.chunk_len, workspace=ws)

    def decode_paged():
        P.prefill_attn_chunked_splitkv_paged(qd, kd, vd, cud, kp, vp, btd, outd, pred, scale=st.scale,
                                             max_seqlen=1, workspace=wsd)

    msp = timed_steps(step_paged, args.steps, args.warmup)
    msdp = timed_steps(decode_paged, args.steps, args.warmup)
    del kp, vp

    # every step c = 0 .. 15 through split-KV, summed (the cache already holds
    # the prompt's earlier chunks; a step rewrites its own chunk with the same
    # values), and the prompt's chunks alone (no decode rows) summed against
    # one varlen call over the whole 8192-token prompt: the chunking overhead
    L = wl.chunk_len
    pqd, pkd, pvd = t["pq"].to(dev), t["pk"].to(dev), t["pv"].to(dev)
    dq_, dk_, dv_ = t["dq"].to(dev), t["dk"].to(dev), t["dv"].to(dev)
    reps = 50
    step_us, chunk_us = [], []
    out1 = torch.empty((L, H, D), dtype=torch.bfloat16, device=dev)
    outs = torch.empty((L + R, H, D), dtype=torch.bfloat16, device=dev)
    cu1 = torch.tensor([0, L], dtype=torch.int32, device=dev)
    for c_ in range(wl.num_chunks):
        stc = wl.step(c_)
        sl_ = slice(c_ * L, (c_ + 1) * L)
        qs, ks_, vs_ = (torch.cat([a[sl_], b_]) for a, b_ in ((pqd, dq_), (pkd, dk_), (pvd, dv_)))
        cus = torch.tensor(stc.cu_seqlens, dtype=torch.int32, device=dev)
        pres = torch.tensor(stc.prefix_lens, dtype=torch.int32, device=dev)
        pre1 = torch.tensor([c_ * L], dtype=torch.int32, device=dev)

        def one_step():
            P.prefill_attn_chunked_splitkv(qs, ks_, vs_, cus, kc, vc, outs, pres, scale=st.scale,
                                           max_seqlen=L, workspace=ws)

        def one_chunk():
            P.prefill_attn_chunked_splitkv(pqd[sl_], pkd[sl_], pvd[sl_], cu1, kc[:1], vc[:1], out1, pre1,
                                           scale=st.scale, max_seqlen=L, workspace=ws)

        step_us.append(timed_steps(one_step, reps, 10) * 1e3)
        chunk_us.append(timed_steps(one_chunk, reps, 10) * 1e3)
    kc1 = torch.empty_like(pkd)
    vc1 = torch.empty_like(pvd)
    out_full = torch.empty_like(pqd)
    cu_full = torch.tensor([0, wl.prompt_len], dtype=torch.int32, device=dev)

    def one_shot():
        P.prefill_attn_varlen(pqd, pkd, pvd, cu_full, kc1, vc1, out_full, scale=st.scale, max_seqlen=wl.prompt_len)

    one_shot_us = timed_steps(one_shot, reps, 10) * 1e3
    prompt_flops = 4.0 * D * H * causal_pairs([wl.prompt_len])
    all_steps = {"steps": wl.num_chunks, "sum_us": round(sum(step_us), 1),
                 "per_step_us": [round(x, 1) for x in step_us],
                 "prompt_chunks_alone_sum_us": round(sum(chunk_us), 1),
                 "one_shot_varlen_us": round(one_shot_us, 1),
                 "chunking_overhead": round(sum(chunk_us) / one_shot_us, 3),
                 "one_shot_tflops": round(prompt_flops / (one_shot_us * 1e-6) / 1e12, 1)}
    del kc1, vc1, out_full, pqd, pkd, pvd
    # the line's value is the step through split-KV, the path for this workload;
    # the one-pass call's figures follow under one_pass
    value = flops / (mss * 1e-3) / 1e12
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mss, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "step": "chunk %d of %d (prefix %d) + %d decode rows" % (c, wl.num_chunks, c * wl.chunk_len, R),
                   "tokens": int(q.shape[0]), "num_heads": H, "num_kv_heads": HK, "head_dim": D, "causal": True,
                   "kv_cache_write": True, "scale": st.scale,
                   "path": "prefill_attn_chunked_splitkv"},
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "us_per_step": round(mss * 1e3, 2),
        "one_pass": {"ms_per_step": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "us_per_step": round(ms * 1e3, 2)},
        "decode_only": {"rows": R, "context_tokens": sum(wl.contexts), "path": "one-pass",
                        "us_per_step": round(msd * 1e3, 2),
                        "kv_read_gbps": round(dec_bytes / (msd * 1e-3) / 1e9, 1),
                        "frac_of_hbm_8tbs": round(dec_bytes / (msd * 1e-3) / 8e12, 4)},
        "splitkv": {"ms_per_step": round(mss, 5),
                    "tflops": round(flops / (mss * 1e-3) / 1e12, 2),
                    "us_per_step": round(mss * 1e3, 2),
                    "decode_only_us_per_step": round(msds * 1e3, 2),
                    "decode_kv_read_gbps": round(dec_bytes / (msds * 1e-3) / 1e9, 1),
                    "decode_frac_of_hbm_8tbs": round(dec_bytes / (msds * 1e-3) / 8e12, 4)},
        "splitkv_paged": {"ms_per_step": round(msp, 5),
                          "tflops": round(flops / (msp * 1e-3) / 1e12, 2),
                          "us_per_step": round(msp * 1e3, 2),
                          "decode_only_us_per_step": round(msdp * 1e3, 2),
                          "decode_kv_read_gbps": round(dec_bytes / (msdp * 1e-3) / 1e9, 1),
                          "block_tokens": 16, "blocks": B * mb},
        "all_steps_splitkv": all_steps,
        "roofline": None,
        "cpu_baseline": None,
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only (no sharding or collectives); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calib:
        copy_calib()
        return

    import prefill_self_attention_amd as P
    from prefill_self_attention_amd import inputs as I
    P.load()

    w = I.workload(args.workload)
    if isinstance(w, I.ChunkedWorkload):
        print(json.dumps(bench_chunked(args, w, P)))
        return
    dev = torch.device("cuda:0")
    if args.kernel_only:
        # profiler runs: N(0,1) bf16 drawn on the device (the seeded host
        # draw of the large workloads takes minutes)
        gd = torch.Generator(device=dev)
        gd.manual_seed(w.seed)
        N, H, HK, D = w.num_tokens, w.num_heads, w.num_kv_heads, w.head_dim
        qd, kd, vd = (torch.randn(s_, generator=gd, device=dev).to(torch.bfloat16)
                      for s_ in ((N, H, D), (N, HK, D), (N, HK, D)))
        q = k = v = None
    else:
        q, k, v = w.tensors()
        N, H, D = q.shape
        HK = k.shape[1]
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    kc = torch.empty_like(kd)
    vc = torch.empty_like(kd)
    max_seqlen = w.max_seqlen
    torch.cuda.synchronize()

    pairs = causal_pairs(w.lengths)
    flops = 4.0 * D * H * pairs
    kv_bytes = 2.0 * N * HK * D * 2
    # read q, k, v; write out, k_cache, v_cache
    alg_bytes = 2.0 * N * H * D * 2 + 4.0 * N * HK * D * 2

    def step():
        P.prefill_attn_varlen(qd, kd, vd, cu, kc, vc, out, scale=w.scale, max_seqlen=max_seqlen)

    # the in-process context probes first (a bf16 GEMM, the MFMA peak): the
    # peak is then taken at the clock the timed steps run at, and the timed
    # steps do not run while the clocks are still ramping up from idle
    if not args.kernel_only:
        gemm = gemm_context()
        try:
            peak = measured_mfma_peak()
        except OSError as e:  # the probe library is context, not the measured path
            peak = {"error": str(e)}
    # the timed region: K steps back to back (one kernel launch each) between
    # two events; its mean is also the kernel's average launch duration
    ms_per_step = timed_steps(step, args.steps, args.warmup)
    # per-launch spread, from a separate pass with events around every launch
    launch_ms = launch_times(step, args.steps)
    mean_launch_ms = sum(launch_ms) / len(launch_ms)

    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = value
    if args.kernel_only:
        print(json.dumps({"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s",
                          "ms_per_step": round(ms_per_step, 5), "steps": args.steps, "warmup": args.warmup,
                          "config": {"workload": w.name}, "kernel_only": True,
                          "kernel_source_sha256": kernel_sha()}), flush=True)
        return

    # the same step writing an INT8 cache (codes + one float scale per token
    # and K/V head) instead of the bf16 cache
    kq8 = torch.empty((N * HK * D,), dtype=torch.int8, device=dev)
    vq8 = torch.empty_like(kq8)
    ks8 = torch.empty((N * HK,), dtype=torch.float32, device=dev)
    vs8 = torch.empty_like(ks8)

    def step_int8():
        P.prefill_attn_varlen_int8(qd, kd, vd, cu, kq8, vq8, ks8, vs8, out, scale=w.scale,
                                   max_seqlen=max_seqlen)

    ms8 = timed_steps(step_int8, args.steps, args.warmup)

    # and an FP8 (E4M3) cache, same layout
    kf8, vf8 = kq8.view(torch.uint8), vq8.view(torch.uint8)

    def step_fp8():
        P.prefill_attn_varlen_fp8(qd, kd, vd, cu, kf8, vf8, ks8, vs8, out, scale=w.scale,
                                  max_seqlen=max_seqlen)

    msf8 = timed_steps(step_fp8, args.steps, args.warmup)

    # the shader clock the kernel runs at, from the measurement build
    clock = None
    if D == 128 and args.workload == "single_T2048_H32_D128":
        import ctypes
        try:
            clock = kernel_clock(lambda: (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), cu.data_ptr(),
                                          len(w.lengths), max_seqlen, H, HK, D, kc.data_ptr(), vc.data_ptr(),
                                          out.data_ptr(), ctypes.c_float(w.scale), None))
        except OSError as e:  # the measurement build is context, not the measured path
            clock = {"error": str(e)}

    # cold: every launch after a 1 GiB fill that evicts L2 and the Infinity Cache
    cold_ms = cold_launch_times(step, min(args.steps, 100))
    # the HBM copy rate this part sustains (a plain 1 GiB device-to-device
    # copy, read + write bytes per time): the bandwidth the cache write and
    # the decode rows are compared with
    hbm = hbm_copy_rate()
    others = other_configs(P) if args.workload == "single_T2048_H32_D128" and not args.no_other_configs else None
    cache8_bytes = 2.0 * N * HK * (D + 4)
    cold = stats_us(cold_ms)
    traffic, traffic_note = read_traffic() if args.workload == "single_T2048_H32_D128" else (None, "n/a")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_lens": w.lengths if len(w.lengths) <= 8 else
                   "%d sequences" % len(w.lengths), "tokens": N, "num_heads": H,
                   "num_kv_heads": HK, "head_dim": D,
                   "causal": True, "kv_cache_write": True, "scale": w.scale},
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        # cold (L2 and Infinity Cache evicted before each launch) beside warm
        # (back to back): median and p99 per launch, and the rate at the median
        "cold": dict(cold, tflops_at_median=round(flops / (cold["median"] * 1e-6) / 1e12, 1),
                     pct_bf16_mfma_peak_at_median=round(100.0 * flops / (cold["median"] * 1e-6) / 1e12
                                                        / PEAK_BF16_TFLOPS, 2)),
        "warm": {"median": round(launch_ms[len(launch_ms) // 2] * 1e3, 2),
                 "p99": round(launch_ms[min(len(launch_ms) - 1, int(math.ceil(0.99 * len(launch_ms))) - 1)] * 1e3, 2),
                 "mean_back_to_back": round(ms_per_step * 1e3, 2)},
        "measured_mfma_peak": peak if "error" in peak else
        dict(peak, value_pct_of_it=round(100.0 * value / peak["tflops"], 1)),
        # the kernel's own shader clock, and the published dense rate scaled
        # to it (2.5 PFLOP/s at 2.4 GHz)
        "kernel_clock": clock,
        "mfma_peak_at_kernel_clock": None if clock is None or "error" in clock else {
            "tflops": round(PEAK_BF16_TFLOPS * clock["loop_shader_clock_mhz"]["median"] / 2400.0, 1),
            "value_pct_of_it": round(100.0 * value / (PEAK_BF16_TFLOPS * clock["loop_shader_clock_mhz"]["median"]
                                                      / 2400.0), 1)},
        "kernel_source_sha256": kernel_sha(),
        # cache bytes written per step over the fused step's time: the write's
        # share of the step's HBM traffic, not a bandwidth of its own
        "kv_write_gbps": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "kv_bytes_written": kv_bytes,
        "algorithmic_hbm_gbps": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        # each launch between its own events (separate pass; the event records
        # add a few microseconds per launch)
        "launch_us": {"mean": round(mean_launch_ms * 1e3, 2),
                      "median": round(launch_ms[len(launch_ms) // 2] * 1e3, 2),
                      "p99": round(launch_ms[min(len(launch_ms) - 1,
                                                 int(math.ceil(0.99 * len(launch_ms))) - 1)] * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "algorithmic_flops": flops, "algorithmic_bytes": alg_bytes},
        "cold_launch_us": cold,
        "hbm_copy_measured": hbm,
        "gemm_bf16_context": dict(gemm, pct_of_published_peak=round(100.0 * gemm["tflops"] / PEAK_BF16_TFLOPS, 1),
                                  attention_pct_of_it=round(100.0 * value / gemm["tflops"], 1)),
        "int8_cache": {"us_per_step": round(ms8 * 1e3, 2),
                       "tflops": round(flops / (ms8 * 1e-3) / 1e12, 2),
                       "cache_bytes_written": cache8_bytes,
                       "bf16_cache_bytes": kv_bytes},
        "fp8_cache": {"us_per_step": round(msf8 * 1e3, 2),
                      "tflops": round(flops / (msf8 * 1e-3) / 1e12, 2),
                      "cache_bytes_written": cache8_bytes,
                      "format": "OCP E4M3, one float scale per (token, K/V head)"},
        "other_configs": others,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, flops)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
