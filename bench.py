#!/usr/bin/env python3
"""Benchmark: one continuous-batching decode step on one MI355X.

Workload (seeded, synthetic): 256 sequences with context lengths uniform in
[64, 4096], 32 query / 8 KV heads, head_dim 128, bf16, 16-token blocks
scattered over a pool of total blocks + 10% drawn from a shuffled free list.
A step = pa_reshape_and_cache (one new token per sequence, through
slot_mapping) + pa_decode over context + 1 (the decode kernel and, for the
sequences longer than one 512-token partition, the log-sum-exp merge).
Inputs are resident in HBM before timing starts.

With --mode prefill the line is the chunked-prefill step instead (32
sequences whose last 512 tokens are this step's chunk; append + pa_prefill),
in TFLOP/s of useful causal FLOPs against the bf16 matrix-core peak; the
default run adds it as the `chunked_prefill` object.

With --mode serve the line is this build's own measurement of what the
pages credit paged allocation with: an iteration-level batching loop (host
scheduler + block manager + the kernels) over one pool, admitting by free
blocks, against the same loop holding 4096-token reservations; generated
tokens per second of summed kernel time and of wall time, and the mean
decode batch, for both.

With --mode long the line is pa_decode over the long-context batch (32
sequences of 8192..32768 tokens, 64 q / 8 KV heads) at block size 16; the
default run adds every block size (8, 16, 32), balanced and with fixed
512-position partitions, as the `long_context` object, and the shared-prefix
step (copy-on-write + append + decode; cache-warm, logical and unique GB/s)
as the `shared_prefix` object.

With --kv fp8 the same step runs over 8-bit OCP E4M3 K/V pools (one scale
per pool): pa_reshape_and_cache_fp8 + pa_decode_fp8, B_kv counted at one byte
per element.  The default (16-bit) run also times that step and adds it as
the `fp8_kv` object.

Prints one JSON line:
  value       effective KV GB/s of the whole step = B_kv / step time, with
              B_kv = sum_s L_s * 2 * Hkv * d * 2 bytes (live K and V read
              once; tail slots of partial blocks not counted)
  roofline    pa_decode's achieved B_kv / (mean duration of its launches,
              HIP events on its stream around each call over K further
              steps) against the
              8 TB/s HBM peak; `achievable` is the same figure for
              pa_probe_gather, which issues exactly pa_decode's K/V loads and
              computes nothing (the gather pattern's own ceiling);
              `streaming_read` the same for pa_probe_stream, a plain
              streaming read of as many bytes (the device's read peak)
  cpu_baseline  the float64 CPU oracle on the same step, host cores
  host_block_manager  the host bookkeeping of the same step through the
              block manager (include/pa_block_manager.h): one appended
              token for each of the 256 sequences (pa_bm_append_batch) and
              the 256 block tables pa_decode takes (pa_bm_tables), median
              microseconds per step on the host
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention effective KV GB/s (% of HBM peak) + decode seqs/s"
HBM_PEAK_GBS = 8000.0

# HBM bytes per pa_decode call from the committed rocprofv3 FETCH_SIZE /
# WRITE_SIZE summary; reported only while the kernel sources still hash to
# the value recorded there (a changed kernel has no measured traffic).
_CSRC = os.path.join(ROOT, "paged_kv_cache_400_amd", "csrc")
TRAFFIC_SUMMARY = {
    "16": os.path.join(ROOT, "profiles", "pa_decode_streamk_mixed_step_traffic.md"),
    "fp8": os.path.join(ROOT, "profiles", "pa_decode_fp8_mixed_step_traffic.md"),
    "prefill": os.path.join(ROOT, "profiles", "pa_prefill_chunked_prefill_traffic.md"),
}
KERNEL_SOURCES = {
    "16": [os.path.join(_CSRC, f) for f in ("decode_streamk.hip", "decode_streamk.h",
                                            "pa_mfma.h", "pa_device.h", "pa_launch.h")],
    "fp8": [os.path.join(_CSRC, f) for f in ("decode_fp8.hip", "decode_streamk.h",
                                             "pa_mfma_fp8.h", "pa_mfma.h", "pa_device.h",
                                             "pa_launch.h")],
    "prefill": [os.path.join(_CSRC, f) for f in ("prefill.hip", "pa_mfma.h", "pa_device.h",
                                                 "pa_launch.h")],
}
KERNEL_NAMES = {
    ("fp8", True): "pa_decode_fp8 (pa_decode_streamk over E4M3 pools + pa_streamk_reduce)",
    ("auto", True): "pa_decode (pa_decode_streamk + pa_streamk_reduce)",
    ("auto", False): ("pa_decode, explicit partitions (pa_decode_streamk with runs cut at "
                      "partition boundaries + pa_streamk_reduce)"),
    ("mfma", True): ("pa_probe_decode_mfma (pa_decode_streamk with the matrix-core tile wave "
                     "at every group + pa_streamk_reduce)"),
    ("mfma", False): ("pa_probe_decode_mfma, explicit partitions (pa_decode_streamk with the "
                      "matrix-core tile wave + pa_streamk_reduce)"),
    ("valu", True): ("pa_decode_valu, balanced split (pa_decode_streamk with the vector-unit "
                     "tile wave + pa_streamk_reduce)"),
    ("valu", False): "pa_decode_valu, fixed partitions (pa_decode_valu + pa_splitk_reduce)",
}


def prefill_flops(seq_lens, query_start, num_q_heads: int, head_dim: int) -> int:
    """Useful floating-point operations of causal chunk attention: for each
    chunk token at position p and each query head, (p + 1) positions of a
    q.K dot product and of a P.V accumulation, 2 * d each."""
    import numpy as np
    lens = np.asarray(seq_lens, dtype=np.int64)
    qs = np.asarray(query_start, dtype=np.int64)
    n = qs[1:] - qs[:-1]
    # sum over i < n of (L - n + i + 1) = n (L - n + 1) + n (n - 1) / 2
    pos = n * (lens - n + 1) + n * (n - 1) // 2
    return int(pos.sum()) * num_q_heads * 4 * head_dim


MFMA_BF16_PEAK_TFLOPS = 2500.0


def kernel_sources_sha256(kv="16"):
    """SHA-256 over the sources the decode kernel of pool type kv is built from."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[kv]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kv="16"):
    """(bytes per call, note) from the counter summary, or (None, reason)."""
    try:
        text = open(TRAFFIC_SUMMARY[kv]).read()
    except OSError:
        return None, "no counter summary"
    fields = dict(re.findall(r"^([a-z_0-9]+): (\S+)$", text, re.M))
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256(kv):
        return None, "kernel changed since the counters were taken"
    return int(fields["traffic_bytes_per_call"]), os.path.relpath(TRAFFIC_SUMMARY[kv], ROOT)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default 50: the GPU runs below full clock "
                         "for the first ~10 ms of decode work and ~20 ms of prefill work)")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--ceiling", choices=["on", "off"], default="on",
                    help="also time pa_probe_gather (the same loads, no arithmetic)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time the oracle baseline accumulates")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="0: pa_decode's balanced split (stream-K); else explicit partitions")
    ap.add_argument("--kv", choices=["16", "fp8"], default="16",
                    help="16: bf16 pools (the headline); fp8: the same step over 8-bit E4M3 "
                         "pools (pa_reshape_and_cache_fp8 + pa_decode_fp8)")
    ap.add_argument("--mode", choices=["decode", "prefill", "serve", "long", "groups", "shared"],
                    default="decode",
                    help="decode: the mixed decode step (the headline); prefill: the chunked "
                         "prefill step (32 sequences x 512-token chunks, pa_prefill); serve: "
                         "iteration-level batching over the paged pool against 4096-token "
                         "reservations on the same pool; long: decode over the long-context "
                         "batch (32 sequences of 8192..32768 tokens, group 8) at block sizes "
                         "8, 16 and 32")
    ap.add_argument("--long-summary", choices=["on", "off"], default="on",
                    help="with --mode decode: also time the long-context batch at block sizes "
                         "8/16/32 and add a summary object")
    ap.add_argument("--shared-summary", choices=["on", "off"], default="on",
                    help="with --mode decode: also time the shared-prefix step (copy-on-write, "
                         "append, decode) and add a summary object")
    ap.add_argument("--serve-iterations", type=int, default=300,
                    help="timed iterations per policy in --mode serve (after as many untimed)")
    ap.add_argument("--prefill-summary", choices=["on", "off"], default="on",
                    help="with --mode decode: also time the chunked-prefill step and add a "
                         "summary object")
    ap.add_argument("--fp8-summary", choices=["on", "off"], default="on",
                    help="with --kv 16: also time the 8-bit step and add a summary object")
    ap.add_argument("--impl", choices=["auto", "mfma", "valu"], default="auto",
                    help="auto: pa_decode (tile wave chosen by the query group); mfma: "
                         "pa_probe_decode_mfma (matrix cores at every group); valu: "
                         "pa_decode_valu (vector unit alone)")
    ap.add_argument("--block-manager", choices=["on", "off"], default="on",
                    help="time the host block manager's bookkeeping for the same step")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB once (a transfer of "
                         "known size to scale HBM byte counters by)")
    args = ap.parse_args()
    if args.warmup is None:
        args.warmup = (PREFILL_WARMUP if args.mode == "prefill" else
                       FP8_WARMUP if args.kv == "fp8" else DECODE_WARMUP)
    return args


def host_cpu():
    """What the CPU baseline ran on: the cores this process may use
    (sched_getaffinity) and the host CPU's model name (/proc/cpuinfo)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(b, seconds):
    import oracle
    from paged_kv_cache_400_amd.workload import bits
    nk, nv, q = bits(b.new_key), bits(b.new_value), bits(b.q)
    if b.kv == "fp8":
        kp, vp = b.k_cache.numpy().copy(), b.v_cache.numpy().copy()

        def step():
            oracle.reshape_and_cache_fp8(nk, nv, kp, vp, b.slot_mapping, b.k_scale, b.v_scale,
                                         oracle.BF16)
            oracle.decode_fp8(q, kp, vp, b.block_tables, b.seq_lens, b.scale, b.k_scale,
                              b.v_scale, oracle.BF16)
    else:
        kp, vp = bits(b.k_cache).copy(), bits(b.v_cache).copy()

        def step():
            oracle.reshape_and_cache(nk, nv, kp, vp, b.slot_mapping)
            oracle.decode(q, kp, vp, b.block_tables, b.seq_lens, b.scale, oracle.BF16)
    reps, total = 0, 0.0
    while reps == 0 or total < seconds:
        t0 = time.perf_counter()
        step()
        total += time.perf_counter() - t0
        reps += 1
    t = total / reps
    return {
        "value": round(b.kv_bytes() / t / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        **host_cpu(),
        "kind": "oracle",
        "sample": (f"the whole step ({len(b.slot_mapping)}-token append + decode of all "
                   f"{b.num_seqs * b.num_q_heads} rows), float64, {reps} repetition(s) of "
                   f"{t:.2f} s"),
        "seqs_per_s": round(b.num_seqs / t, 2),
    }


def host_block_manager(b, steps=200):
    """Median host time of one decode step's bookkeeping for the bench batch:
    the manager holds the batch's sequences (random token ids, no shared
    prefixes), then each step appends one token to every sequence and fills
    the block tables and lengths pa_decode takes."""
    import numpy as np
    import paged_kv_cache_400_amd as pa
    bs, S = b.block_size, b.num_seqs
    lens = b.seq_lens.astype(np.int64)
    mb = int((lens.max() + steps) // bs + 2)
    nb = int(sum(-(-int(L) // bs) for L in lens)) + S * (steps // bs + 2)
    bm = pa.BlockManager(nb, bs)
    rng = np.random.default_rng(0)
    for s in range(S):
        bm.add_sequence(s, rng.integers(0, 1 << 15, int(lens[s])))
    ids = np.arange(S, dtype=np.int64)
    toks = rng.integers(0, 1 << 15, (steps, S)).astype(np.int32)
    out = (np.empty((S, mb), np.int32), np.empty(S, np.int32))
    times = []
    for i in range(steps):
        t0 = time.perf_counter()
        bm.append_batch(ids, toks[i])
        bm.tables(ids, mb, out=out)
        times.append(time.perf_counter() - t0)
    bm.close()
    return {"us_per_step": round(float(np.median(times)) * 1e6, 1), "seqs": S, "steps": steps,
            "ops": "append_batch (one token per sequence) + tables, through the Python binding"}


def measure(b, dev, args, kv, partition_size, with_ceiling, warmup=None):
    """Time K steps (append + decode) of batch b after W warmup steps: the K
    steps back to back between two HIP events on the current stream (the
    step time), then K more with events around each decode call (the call's
    own duration; an event between two launches costs the stream a few
    microseconds, so these are not the step time); then, optionally, K
    gather-only runs.  Returns (ms per step, ms per decode call, ms per
    gather-only run or None)."""
    import torch
    import paged_kv_cache_400_amd as pa
    S, Hq, d = b.q.shape
    ws_bytes = pa.decode_workspace_bytes(S, Hq, d, b.max_blocks_per_seq, b.block_size,
                                         partition_size)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(dev["q"])

    if kv == "fp8":
        def append():
            pa.reshape_and_cache_fp8(dev["new_key"], dev["new_value"], dev["k_cache"],
                                     dev["v_cache"], dev["slot_mapping"], b.k_scale, b.v_scale)

        def decode():
            pa.decode_fp8(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                          dev["seq_lens"], b.k_scale, b.v_scale, scale=b.scale, out=out,
                          workspace=ws)
    else:
        def append():
            pa.reshape_and_cache(dev["new_key"], dev["new_value"], dev["k_cache"],
                                 dev["v_cache"], dev["slot_mapping"])

        def decode():
            pa.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                      dev["seq_lens"], scale=b.scale, partition_size=partition_size, out=out,
                      workspace=ws, impl=args.impl)

    W = args.warmup if warmup is None else warmup
    for _ in range(W):
        append()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        append()
        decode()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        append()
        ev[i][0].record()
        decode()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms_decode = sum(a.elapsed_time(z) for a, z in ev) / K

    # the access pattern's own ceiling: the same K/V loads, nothing computed
    ceiling = None
    if with_ceiling:
        sink = torch.zeros(2, dtype=torch.int16, device="cuda:0")
        for _ in range(W):
            pa.probe_gather(dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["seq_lens"],
                            Hq, sink=sink)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record()
        for _ in range(K):
            pa.probe_gather(dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["seq_lens"],
                            Hq, sink=sink)
        c1.record()
        torch.cuda.synchronize()
        ceiling = c0.elapsed_time(c1) / K
    return ms_step, ms_decode, ceiling


def streaming_read(nbytes, steps, warmup):
    """Mean us per pa_probe_stream call over a device buffer of nbytes bytes
    (HIP events around `steps` back-to-back calls after `warmup`)."""
    import torch
    import paged_kv_cache_400_amd as pa
    buf = torch.empty(nbytes // 16 * 16, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(2, dtype=torch.int16, device="cuda:0")
    ms = time_calls(lambda: pa.probe_stream(buf, sink=sink), steps, warmup)
    del buf
    return ms * 1e3, nbytes // 16 * 16


def calibration_copy(mib):
    """One device copy of a known size (a transfer to scale HBM byte
    counters by): mib MiB read and mib MiB written."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    ms = c0.elapsed_time(c1)
    return {"bytes_read": n, "bytes_written": n, "ms": round(ms, 5),
            "gbs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}


# Warmup steps of a chunked-prefill measurement: the GPU's clocks take about
# 20 ms of matrix-core work to settle (per-dispatch durations fall by a
# quarter over the first 20 steps, then stay flat).
PREFILL_WARMUP = 50

# Warmup steps of an 8-bit decode measurement: the first ~10 ms after the
# host has prepared the batch run below full clock (the first repetition of
# 100 calls averages 198 us, the next ones 190 us); 50 steps are ~10 ms.
FP8_WARMUP = 50

# Warmup steps of a 16-bit decode measurement, for the same reason: 50 steps
# are ~17 ms (with 10, the timed steps averaged 349.7 us; with 50, 347.8).
DECODE_WARMUP = 50


def measure_prefill(b, dev, args, warmup=None):
    """K steps of the chunked-prefill step (append of the chunks' keys and
    values + pa_prefill) after W warmup steps, back to back between two HIP
    events on the current stream; then K more with events around each
    pa_prefill call.  Returns (ms per step, ms per pa_prefill call)."""
    import torch
    import paged_kv_cache_400_amd as pa
    qs = torch.from_numpy(b.query_start).to("cuda:0")
    out = torch.empty_like(dev["q"])

    def append():
        pa.reshape_and_cache(dev["new_key"], dev["new_value"], dev["k_cache"], dev["v_cache"],
                             dev["slot_mapping"])

    def attend():
        pa.prefill(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                   dev["seq_lens"], qs, scale=b.scale, out=out)

    for _ in range(args.warmup if warmup is None else warmup):
        append()
        attend()
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        append()
        attend()
    end.record()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        append()
        ev[i][0].record()
        attend()
        ev[i][1].record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K, sum(a.elapsed_time(z) for a, z in ev) / K


PREFILL_WORKLOAD = ("chunked_prefill: 32 seqs, total length uniform[1024,4096] whose last 512 "
                    "tokens are this step's chunk (16384 query tokens), causal, 32 q / 8 kv "
                    "heads, d 128, bf16 (f32 accumulate), block 16, shuffled pool of blocks+10%")


def prefill_line(args):
    import torch
    from paged_kv_cache_400_amd import workload as wl
    b = wl.make_chunked_prefill()
    dev = wl.to_device(b, "cuda:0")
    ms_step, ms_attend = measure_prefill(b, dev, args)
    fl = prefill_flops(b.seq_lens, b.query_start, b.num_q_heads, b.head_dim)
    tq = int(b.query_start[-1])
    tf = fl / (ms_attend * 1e-3) / 1e12
    res = {
        "metric": "chunked prefill attention TFLOP/s (causal useful FLOPs) + tokens/s",
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL_WORKLOAD, "num_seqs": b.num_seqs, "query_tokens": tq,
                   "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads,
                   "head_dim": b.head_dim, "block_size": b.block_size, "flops": fl,
                   "kv_bytes": b.kv_bytes()},
        "prefill_ms": round(ms_attend, 5),
        "prefill_tokens_per_s": round(tq / (ms_step * 1e-3), 1),
        "roofline": {"kernel": "pa_prefill (pa_prefill_kernel)", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
    }
    traffic, note = measured_traffic("prefill")
    if traffic is not None:
        res["roofline"]["traffic"] = traffic
        res["roofline"]["traffic_over_kv_bytes"] = round(traffic / b.kv_bytes(), 4)
    res["roofline"]["traffic_source"] = note
    if args.calibrate_copy_mib > 0:
        res["calibration_copy"] = calibration_copy(args.calibrate_copy_mib)
    if args.cpu_baseline == "on":
        import oracle
        from paged_kv_cache_400_amd.workload import bits
        kp, vp = bits(b.k_cache).copy(), bits(b.v_cache).copy()
        oracle.reshape_and_cache(bits(b.new_key), bits(b.new_value), kp, vp, b.slot_mapping)
        # a bounded sample: the first 4 sequences' chunks
        sub = 4
        qe = int(b.query_start[sub])
        t0 = time.perf_counter()
        oracle.prefill(bits(b.q)[:qe], kp, vp, b.block_tables[:sub], b.seq_lens[:sub],
                       b.query_start[:sub + 1], b.scale, oracle.BF16)
        t = time.perf_counter() - t0
        fl_sub = prefill_flops(b.seq_lens[:sub], b.query_start[:sub + 1], b.num_q_heads,
                               b.head_dim)
        res["cpu_baseline"] = {"value": round(fl_sub / t / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), **host_cpu(),
                               "kind": "oracle",
                               "sample": f"the chunks of the first {sub} sequences ({qe} query "
                                         f"tokens, all heads), float64, one run of {t:.2f} s"}
    return res


def time_calls(fn, steps, warmup):
    """Mean ms per call of fn over `steps` back-to-back calls after `warmup`
    untimed ones: HIP events on the current stream around the whole run."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(steps):
        fn()
    c1.record()
    torch.cuda.synchronize()
    return c0.elapsed_time(c1) / steps


LONG_WORKLOAD = ("long_context: 32 seqs, length uniform[8192,32768], 64 q / 8 kv heads "
                 "(group 8), d 128, bf16 (f32 accumulate), block size 8, 16 and 32 with seeded "
                 "random placement in a pool of blocks+10% (the same logical K/V for every "
                 "block size), decode only")


def long_context_summary(args, block_sizes=(8, 16, 32)):
    """pa_decode over the long-context batch at each block size: the
    balanced split (partition_size 0) and fixed 512-position partitions
    merged by log-sum-exp, plus the gather-only ceiling of the balanced
    split.  The batch's K/V (2.56 GB) is ten times the last-level cache, so
    back-to-back calls read HBM."""
    import torch
    import paged_kv_cache_400_amd as pa
    from paged_kv_cache_400_amd import workload as wl
    res = {"workload": LONG_WORKLOAD + " (bench.py --mode long)"}
    steps = max(1, min(args.steps, 50))
    for bs in block_sizes:
        b = wl.make_long_context(bs)
        dev = wl.to_device(b, "cuda:0")
        S, Hq, d = b.q.shape
        kv = b.kv_bytes()
        out = torch.empty_like(dev["q"])
        row = {"kv_bytes": kv, "num_blocks": b.num_blocks,
               "max_blocks_per_seq": b.max_blocks_per_seq}
        for name, part, impl in (("balanced", 0, "auto"), ("partitions_512", 512, "auto"),
                                 ("valu_balanced", 0, "valu")):
            need = pa.decode_workspace_bytes(S, Hq, d, b.max_blocks_per_seq, bs, part)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")
            ms = time_calls(lambda: pa.decode(dev["q"], dev["k_cache"], dev["v_cache"],
                                              dev["block_tables"], dev["seq_lens"],
                                              scale=b.scale, partition_size=part, out=out,
                                              workspace=ws, impl=impl), steps, args.warmup)
            gbs = kv / (ms * 1e-3) / 1e9
            row[name] = {"decode_ms": round(ms, 5), "gbs": round(gbs, 2),
                         "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                         "decode_seqs_per_s": round(S / (ms * 1e-3), 1)}
            del ws
        if args.ceiling == "on":
            sink = torch.zeros(2, dtype=torch.int16, device="cuda:0")
            ms = time_calls(lambda: pa.probe_gather(dev["k_cache"], dev["v_cache"],
                                                    dev["block_tables"], dev["seq_lens"], Hq,
                                                    sink=sink), steps, args.warmup)
            row["achievable_gbs"] = round(kv / (ms * 1e-3) / 1e9, 2)
            row["balanced_frac_of_achievable"] = round(ms / row["balanced"]["decode_ms"], 4)
        res[f"bs{bs}"] = row
        del dev, out
    return res


SHARED_WORKLOAD = ("shared_prefix: 64 seqs sharing the physical blocks of a 2048-token prefix "
                   "(odd-indexed seqs stop 1..15 tokens short of it and copy the partial block "
                   "on write), private tails uniform[1,512], 32 q / 8 kv heads, d 128, fp16 "
                   "(f32 accumulate), block 16")


def unique_kv_bytes(b) -> int:
    """K and V bytes of the distinct pool slots the batch's decode reads
    (shared prefix slots counted once)."""
    import numpy as np
    bs = b.block_size
    slots = []
    for s, L in enumerate(b.seq_lens):
        t = np.arange(int(L))
        slots.append(b.block_tables[s, t // bs].astype(np.int64) * bs + t % bs)
    n = len(np.unique(np.concatenate(slots))) if slots else 0
    return int(n) * 2 * b.num_kv_heads * b.head_dim * b.elem_bytes


def shared_prefix_summary(args):
    """The shared-prefix step: copy-on-write of the 32 partial prefix blocks
    (pa_copy_blocks), the tails' append (pa_reshape_and_cache) and pa_decode.
    Repeating the step is idempotent (the copy restores what the append
    overwrites).  Unique K/V (76 MB) stays in the last-level cache across
    calls, so the figures are cache-warm: logical GB/s counts every
    sequence's reads, unique GB/s each distinct slot once."""
    import torch
    import paged_kv_cache_400_amd as pa
    from paged_kv_cache_400_amd import workload as wl
    b = wl.make_shared_prefix()
    dev = wl.to_device(b, "cuda:0")
    S, Hq, d = b.q.shape
    out = torch.empty_like(dev["q"])
    need = pa.decode_workspace_bytes(S, Hq, d, b.max_blocks_per_seq, b.block_size, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")

    def copy_append():
        pa.copy_blocks(dev["k_cache"], dev["v_cache"], dev["block_mapping"])
        pa.reshape_and_cache(dev["new_key"], dev["new_value"], dev["k_cache"],
                             dev["v_cache"], dev["slot_mapping"])

    def decode():
        pa.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                  dev["seq_lens"], scale=b.scale, out=out, workspace=ws)

    # the blocks every table shares (after the copy-on-write: 127 of 128)
    nblk = min(-(-int(L) // b.block_size) for L in b.seq_lens)
    pb = 0
    while pb < nblk and (b.block_tables[:, pb] == b.block_tables[0, pb]).all():
        pb += 1
    ws_sp = torch.empty(max(pa.decode_shared_prefix_workspace_bytes(S, Hq, d, pb,
                                                                     b.block_size), 1),
                        dtype=torch.uint8, device="cuda:0")

    def decode_shared():
        pa.decode_shared_prefix(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                dev["seq_lens"], pb, scale=b.scale, out=out, workspace=ws_sp)

    def step():
        copy_append()
        decode()

    def step_shared():
        copy_append()
        decode_shared()

    steps = max(1, min(args.steps, 50))
    ms_step = time_calls(step, steps, args.warmup)
    ms_copy_append = time_calls(copy_append, steps, args.warmup)
    ms_decode = time_calls(decode, steps, args.warmup)
    ms_step_shared = time_calls(step_shared, steps, args.warmup)
    ms_shared = time_calls(decode_shared, steps, args.warmup)
    logical, unique = b.kv_bytes(), unique_kv_bytes(b)
    return {
        "workload": SHARED_WORKLOAD + " (cache-warm)",
        "cow_pairs": int(len(b.block_mapping)), "appended_tokens": int(len(b.slot_mapping)),
        "logical_kv_bytes": logical, "unique_kv_bytes": unique,
        "ms_per_step": round(ms_step, 5), "copy_append_ms": round(ms_copy_append, 5),
        "decode_ms": round(ms_decode, 5),
        "decode_logical_gbs": round(logical / (ms_decode * 1e-3) / 1e9, 2),
        "decode_unique_gbs": round(unique / (ms_decode * 1e-3) / 1e9, 2),
        "decode_seqs_per_s": round(S / (ms_decode * 1e-3), 1),
        "shared_prefix_decode": {
            "entry_point": "pa_decode_shared_prefix",
            "prefix_blocks": pb,
            "ms_per_step": round(ms_step_shared, 5),
            "decode_ms": round(ms_shared, 5),
            "decode_logical_gbs": round(logical / (ms_shared * 1e-3) / 1e9, 2),
            "decode_unique_gbs": round(unique / (ms_shared * 1e-3) / 1e9, 2),
            "decode_seqs_per_s": round(S / (ms_shared * 1e-3), 1),
            "speedup_vs_pa_decode": round(ms_decode / ms_shared, 3),
        },
    }


SERVE_WORKLOAD = ("serve: a seeded stream of requests (prompts uniform[64,1024], generations "
                  "uniform[16,512], 8 arrivals per iteration), one attention layer of 32 q / 8 kv "
                  "heads, d 128, bf16, a pool of 4096 16-token blocks (65,536 tokens), at most "
                  "256 running requests and 2048 prefill tokens per iteration")


def serve_line(args):
    """Iteration-level batching driven through the kernels: the paged pool
    (admit by free blocks, grow block by block) against 4096-token
    reservations on the same pool, decided by the C++ scheduler
    (include/pa_scheduler.h).  Each policy runs W untimed iterations (the
    ramp-up), then K timed ones."""
    from paged_kv_cache_400_amd.scheduler import Executor, NativeScheduler, seeded_requests
    nb, K = 4096, args.serve_iterations
    res = {}
    for mode in ("paged", "reserved"):
        reqs = seeded_requests(20000, seed=6, prompt=(64, 1024), gen=(16, 512), rate=8.0)
        sched = NativeScheduler(mode, reqs, num_blocks=nb, block_size=16, max_batch=256,
                                max_step_tokens=2048)
        ex = Executor(nb, 16, 32, 8, 128, seed=6)
        ex.run(sched, K)
        st = ex.run(sched, K, timed=True)
        res[mode] = {
            "generated_tokens": st["generated_tokens"], "iterations": st["iterations"],
            "mean_decode_batch": round(st["generated_tokens"] / st["iterations"], 2),
            "prefill_tokens": st["prefill_tokens"],
            "kernel_ms": round(st["kernel_ms"], 3), "wall_s": round(st["wall_s"], 3),
            "tokens_per_kernel_s": round(st["generated_tokens"] / (st["kernel_ms"] * 1e-3), 1),
            "tokens_per_wall_s": round(st["generated_tokens"] / st["wall_s"], 1),
            "kernel_ms_per_iteration": round(st["kernel_ms"] / st["iterations"], 4),
        }
    p, r = res["paged"], res["reserved"]
    return {
        "metric": "generated tokens/s of kernel time under iteration-level batching "
                  "(paged pool vs 4096-token reservations)",
        "value": p["tokens_per_kernel_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": K, "ms_per_step": p["kernel_ms_per_iteration"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": SERVE_WORKLOAD, "num_blocks": nb, "block_size": 16,
                   "scheduler": "C++ (include/pa_scheduler.h)"},
        "paged": p, "reserved": r,
        "paged_over_reserved": {
            "decode_batch": round(p["mean_decode_batch"] / r["mean_decode_batch"], 3),
            "tokens_per_kernel_s": round(p["tokens_per_kernel_s"] / r["tokens_per_kernel_s"], 3),
            "tokens_per_wall_s": round(p["tokens_per_wall_s"] / r["tokens_per_wall_s"], 3)},
    }


GROUPS_WORKLOAD = ("group sweep: the mixed step's 256 sequences (context uniform[64,4096] + 1), "
                   "8 kv heads, d 128, bf16, block 16, with 8, 16, 32 and 64 query heads "
                   "(group 1, 2, 4, 8): the same K/V bytes, 1 to 8 query heads per byte; "
                   "decode only")


def group_sweep(args, groups=(1, 2, 4, 8)):
    """The balanced split with the matrix-core tile wave (pa_probe_decode_mfma)
    against the same split with the vector-unit tile wave (pa_decode_valu,
    partition_size 0: the same runs, launch and merge), and pa_decode (which
    picks one of the two by the group), on the mixed step's K/V at each query
    group: mean us per call over back-to-back calls (HIP events), effective
    KV GB/s, and the vector kernel's time over the matrix-core one's.  One
    batch is drawn with 64 query heads; group g decodes its first 8 g heads."""
    import torch
    import paged_kv_cache_400_amd as pa
    from paged_kv_cache_400_amd import workload as wl
    ctx = wl.mixed_lengths(256, 64, 4096, 3)
    b = wl.make_decode_batch("group_sweep", ctx, 64, 8, 128, 16, "bf16", 3, append=1)
    dev = wl.to_device(b, "cuda:0")
    pa.reshape_and_cache(dev["new_key"], dev["new_value"], dev["k_cache"], dev["v_cache"],
                         dev["slot_mapping"])
    kv = b.kv_bytes()
    steps = max(1, min(args.steps, 50))
    res = {"workload": GROUPS_WORKLOAD + " (bench.py --mode groups)", "kv_bytes": kv}
    for g in groups:
        q = dev["q"][:, :8 * g].contiguous()
        S, Hq, d = q.shape
        need = pa.decode_workspace_bytes(S, Hq, d, b.max_blocks_per_seq, 16, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")
        out = torch.empty_like(q)
        row = {}
        for impl in ("mfma", "valu", "auto"):
            ms = time_calls(lambda: pa.decode(q, dev["k_cache"], dev["v_cache"],
                                              dev["block_tables"], dev["seq_lens"],
                                              scale=b.scale, out=out, workspace=ws, impl=impl),
                            steps, args.warmup)
            gbs = kv / (ms * 1e-3) / 1e9
            row[impl] = {"us": round(ms * 1e3, 2), "gbs": round(gbs, 2),
                         "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        row["valu_over_mfma_time"] = round(row["valu"]["us"] / row["mfma"]["us"], 4)
        res[f"g{g}"] = row
        del ws
    return res


def groups_line(args):
    """The group sweep as the line's workload: value = pa_decode's effective
    KV GB/s at group 4 (the mixed step itself); every group and both tile
    waves in `group_sweep`."""
    gs = group_sweep(args)
    row = gs["g4"]["auto"]
    return {
        "metric": METRIC, "value": row["gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": max(1, min(args.steps, 50)), "warmup": args.warmup,
        "ms_per_step": round(row["us"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": GROUPS_WORKLOAD, "kv_bytes": gs["kv_bytes"]},
        "roofline": {"kernel": KERNEL_NAMES[("auto", True)], "bound": "hbm",
                     "achieved": row["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": row["frac_of_hbm_peak"], "traffic": None,
                     "traffic_source": "not profiled"},
        "group_sweep": gs,
    }


def shared_line(args):
    """The shared-prefix step as the line's workload (cache-warm): value =
    logical KV GB/s of pa_decode_shared_prefix; pa_decode on the same step
    beside it in `shared_prefix`."""
    sp = shared_prefix_summary(args)
    row = sp["shared_prefix_decode"]
    return {
        "metric": METRIC, "value": row["decode_logical_gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": max(1, min(args.steps, 50)), "warmup": args.warmup,
        "ms_per_step": row["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": SHARED_WORKLOAD, "kv_bytes": sp["logical_kv_bytes"]},
        "shared_prefix": sp,
    }


def long_line(args):
    """The long-context batch as the line's workload: value = effective KV
    GB/s of pa_decode (balanced split) at block size 16; every block size
    and the fixed 512-position partitions in `long_context`."""
    lc = long_context_summary(args)
    row = lc["bs16"]["balanced"]
    return {
        "metric": METRIC, "value": row["gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": max(1, min(args.steps, 50)), "warmup": args.warmup,
        "ms_per_step": row["decode_ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": LONG_WORKLOAD, "block_size": 16,
                   "kv_bytes": lc["bs16"]["kv_bytes"]},
        "frac_of_hbm_peak": row["frac_of_hbm_peak"],
        "decode_seqs_per_s": row["decode_seqs_per_s"],
        "roofline": {"kernel": KERNEL_NAMES[("auto", True)], "bound": "hbm",
                     "achieved": row["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": row["frac_of_hbm_peak"], "traffic": None,
                     "traffic_source": "not profiled"},
        "long_context": lc,
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_400_amd as pa
    from paged_kv_cache_400_amd import workload as wl

    if args.mode == "prefill":
        print(json.dumps(prefill_line(args)), flush=True)
        return
    if args.mode == "serve":
        print(json.dumps(serve_line(args)), flush=True)
        return
    if args.mode == "groups":
        print(json.dumps(groups_line(args)), flush=True)
        return
    if args.mode == "long":
        print(json.dumps(long_line(args)), flush=True)
        return
    if args.mode == "shared":
        print(json.dumps(shared_line(args)), flush=True)
        return

    b = wl.make_mixed_step(kv=args.kv)
    dev = wl.to_device(b, "cuda:0")
    S, Hq, d = b.q.shape
    MB, bs = b.max_blocks_per_seq, b.block_size
    if args.kv == "fp8" and (args.partition_size != 0 or args.impl != "auto"):
        print("--kv fp8 runs pa_decode_fp8 (balanced split only)", file=sys.stderr)
        sys.exit(2)
    ms_step, ms_decode, ceiling = measure(b, dev, args, args.kv, args.partition_size,
                                          args.ceiling == "on")
    K = args.steps
    fp8 = args.kv == "fp8"

    kv = b.kv_bytes()
    gbs_step = kv / (ms_step * 1e-3) / 1e9
    gbs_decode = kv / (ms_decode * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(gbs_step, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 KV, bf16 q/out" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("mixed_step_fp8: 256 seqs, context uniform[64,4096] + 1 appended "
                         "token, 32 q / 8 kv heads, d 128, 8-bit E4M3 K/V pools (per-pool "
                         "scale), bf16 q/out (f32 accumulate), block 16, shuffled pool of "
                         "blocks+10%") if fp8 else
                        ("mixed_step: 256 seqs, context uniform[64,4096] + 1 appended token, "
                         "32 q / 8 kv heads, d 128, bf16 (f32 accumulate), block 16, "
                         "shuffled pool of blocks+10%"),
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": b.num_kv_heads, "head_dim": d,
            "block_size": bs, "num_blocks": b.num_blocks, "max_blocks_per_seq": MB,
            "partition_size": args.partition_size or "balanced (stream-K)", "kv_bytes": kv,
            "tokens": int(b.seq_lens.sum()),
        },
        "frac_of_hbm_peak": round(gbs_step / HBM_PEAK_GBS, 4),
        "decode_seqs_per_s": round(S / (ms_step * 1e-3), 1),
        "decode_ms": round(ms_decode, 5),
        "decode_only_gbs": round(gbs_decode, 2),
        "roofline": {
            "kernel": KERNEL_NAMES[("fp8" if fp8 else args.impl, args.partition_size == 0)],
            "bound": "hbm",
            "achieved": round(gbs_decode, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs_decode / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }
    if ceiling is not None:
        gbs_ceiling = kv / (ceiling * 1e-3) / 1e9
        res["roofline"]["achievable"] = {
            "kernel": "pa_probe_gather: the same grid and K/V loads as the decode's balanced "
                      "split, no arithmetic",
            "us": round(ceiling * 1e3, 2), "gbs": round(gbs_ceiling, 2),
            "frac_of_peak": round(gbs_ceiling / HBM_PEAK_GBS, 4),
            "decode_frac_of_achievable": round(gbs_decode / gbs_ceiling, 4),
        }
        # the same number of bytes read as a plain streaming read
        us_sr, nb_sr = streaming_read(kv, K, args.warmup)
        gbs_sr = nb_sr / (us_sr * 1e-6) / 1e9
        res["roofline"]["streaming_read"] = {
            "kernel": "pa_probe_stream: a plain streaming read of a buffer of the same size "
                      "at its peak launch shape (4 waves per CU, 8 KiB in flight each)",
            "bytes": nb_sr, "us": round(us_sr, 2), "gbs": round(gbs_sr, 2),
            "frac_of_peak": round(gbs_sr / HBM_PEAK_GBS, 4),
            "decode_frac_of_streaming_read": round(gbs_decode / gbs_sr, 4),
        }
    profiled = args.impl == "auto" and args.partition_size == 0
    traffic, note = measured_traffic(args.kv)
    if profiled and traffic is not None:
        res["roofline"]["traffic"] = traffic
        res["roofline"]["traffic_over_algorithmic"] = round(traffic / kv, 4)
    res["roofline"]["traffic_source"] = note if profiled else "not profiled"
    if args.calibrate_copy_mib > 0:
        res["calibration_copy"] = calibration_copy(args.calibrate_copy_mib)
    if args.kv == "16" and args.fp8_summary == "on" and profiled:
        del dev
        b8 = wl.make_mixed_step(kv="fp8")
        dev8 = wl.to_device(b8, "cuda:0")
        s8, d8, c8 = measure(b8, dev8, args, "fp8", 0, args.ceiling == "on",
                             warmup=max(args.warmup, FP8_WARMUP))
        kv8 = b8.kv_bytes()
        res["fp8_kv"] = {
            "workload": "the same step over 8-bit E4M3 K/V pools (bench.py --kv fp8)",
            "kv_bytes": kv8,
            "warmup": max(args.warmup, FP8_WARMUP),
            "ms_per_step": round(s8, 5),
            "value_gbs": round(kv8 / (s8 * 1e-3) / 1e9, 2),
            "decode_ms": round(d8, 5),
            "decode_gbs": round(kv8 / (d8 * 1e-3) / 1e9, 2),
            "decode_frac_of_hbm_peak": round(kv8 / (d8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_seqs_per_s": round(S / (s8 * 1e-3), 1),
            "step_speedup_vs_16bit": round(ms_step / s8, 3),
        }
        if c8 is not None:
            res["fp8_kv"]["achievable_gbs"] = round(kv8 / (c8 * 1e-3) / 1e9, 2)
            res["fp8_kv"]["decode_frac_of_achievable"] = round(c8 / d8, 4)
        del dev8
    if args.prefill_summary == "on" and profiled and args.kv == "16":
        pf = wl.make_chunked_prefill()
        devp = wl.to_device(pf, "cuda:0")
        sp, ap = measure_prefill(pf, devp, args, warmup=max(args.warmup, PREFILL_WARMUP))
        fl = prefill_flops(pf.seq_lens, pf.query_start, pf.num_q_heads, pf.head_dim)
        res["chunked_prefill"] = {
            "workload": PREFILL_WORKLOAD + " (bench.py --mode prefill)",
            "flops": fl, "prefill_ms": round(ap, 5), "ms_per_step": round(sp, 5),
            "tflops": round(fl / (ap * 1e-3) / 1e12, 2),
            "frac_of_mfma_bf16_peak": round(fl / (ap * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(int(pf.query_start[-1]) / (sp * 1e-3), 1),
        }
        del devp
    if args.long_summary == "on" and profiled and args.kv == "16":
        res["long_context"] = long_context_summary(args)
    if args.shared_summary == "on" and profiled and args.kv == "16":
        res["shared_prefix"] = shared_prefix_summary(args)
    if args.block_manager == "on":
        res["host_block_manager"] = host_block_manager(b)
        res["host_block_manager"]["frac_of_step"] = round(
            res["host_block_manager"]["us_per_step"] * 1e-3 / res["ms_per_step"], 4)
    if args.cpu_baseline == "on":
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
