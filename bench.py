#!/usr/bin/env python3
"""Benchmark of the online-softmax attention path on one MI355X.

One step = one ``osx_attn_fwd`` call on the GQA causal prefill workload (bf16,
B=2, Hq=32, Hkv=8, S=4096, d=128): every step of the single-pass attention
hot path runs in it.  The headline ``value`` is its causal-adjusted TFLOP/s
(4*B*Hq*S*S*d / 2 flops per call).  The other hot-path calls are timed in the
same run and reported under ``also``: GQA decode (GB/s over K/V), the long-row
softmax and the causal bf16 score-row softmax (GB/s: the visible inputs read
twice, or once where the row stays in registers, + 1 write), the two
three-pass softmax comparators on the long row (with their time relative to
the two-pass kernel), the fp32 4096^2 attention (TFLOP/s) with the plain and
the normalised-output recurrence, the prefill with the log-sum-exp output, the
two small latency cases (microseconds), the unfused three-kernel attention
comparator on the prefill workload (its time relative to the fused call), and,
as the reference for the HBM-bound lines, a plain 16-byte streaming read of
2 GiB on the same GPU.

Inputs are seeded synthetic tensors (``synth``), generated on the host and
copied to HBM before timing.  Durations come from HIP events recorded on the
stream the kernels run on: the timed calls run back to back in a few
consecutive windows, each bracketed by its own event pair, so the mean over
all calls (the reported rate) and the per-call min / median / max over the
windows come from the same run.

``cpu_baseline`` times the fp64 oracle on the host's cores in the same run:
every workload in full (the per-(batch, head) slices of the large ones spread
over a pool of host threads), each with its wall time and its rate under the
same algorithmic count as the GPU line.

``--gpus N`` with N > 1 exits: the library and this benchmark use one GPU.
Prints one JSON line on stdout.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 MFMA / vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PREWARM_S = 0.5            # untimed run before the warm-up steps, so clocks are up
METRIC = "attn fwd TFLOP/s (causal-adjusted) & softmax/decode GB/s, % of MI355X peak"
KERNEL_SOURCES = {
    "prefill_bf16_kernel": "online_softmax_02_amd/csrc/attn_prefill_bf16.hip",
    "decode_bf16_kernel": "online_softmax_02_amd/csrc/attn_decode_bf16.hip",
    "softmax_split": "online_softmax_02_amd/csrc/softmax_rows.hip",
    "softmax_wave_causal": "online_softmax_02_amd/csrc/softmax_rows.hip",
    "prefill_f32_kernel": "online_softmax_02_amd/csrc/attn_prefill_f32.hip",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--only", default="all",
                   choices=["all", "prefill", "unfused", "decode", "softmax", "f32", "small", "copy", "probe"],
                   help="time one workload only (for profiler runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sha_of(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(kernel: str):
    """HBM bytes per launch from committed PMC counters, or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != sha_of(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("traffic_bytes_per_launch")


WINDOWS = 5  # event windows per timed region


class Timing:
    """Result of timed(): wall seconds of the timed region, mean GPU ms per call over all calls, and the mean ms
    per call of each event window."""

    def __init__(self, wall, ms, window_ms):
        self.wall, self.ms, self.window_ms = wall, ms, window_ms

    def __iter__(self):  # (wall, ms) unpacking
        return iter((self.wall, self.ms))

    def per_call_us(self):
        w = sorted(self.window_ms)
        med = w[len(w) // 2] if len(w) % 2 else 0.5 * (w[len(w) // 2 - 1] + w[len(w) // 2])
        return {"mean": round(self.ms * 1e3, 2), "min": round(w[0] * 1e3, 2), "median": round(med * 1e3, 2),
                "max": round(w[-1] * 1e3, 2), "windows": len(w)}


def timed(torch, fn, steps, warmup):
    """Warm up, then time `steps` back-to-back calls.

    The call first runs untimed for PREWARM_S seconds (GPU clocks ramp up
    over the first few hundred milliseconds), then `warmup` times.  The timed
    calls are split into up to WINDOWS consecutive windows, each bracketed by
    a HIP event pair on the launch stream; the windows follow each other with
    no host synchronisation, so the host keeps the GPU queue full (per-call
    event pairs would count the host's argument marshalling whenever the GPU
    catches up).  Returns a Timing: the mean over all `steps` calls is the
    first window's start to the last window's end."""
    # Bring the GPU clocks up first: run the call for ~0.5 s (untimed).
    t_end = time.perf_counter() + PREWARM_S
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn(0)
        torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    stream = torch.cuda.current_stream()
    n_win = max(1, min(WINDOWS, steps))
    sizes = [steps // n_win + (1 if w < steps % n_win else 0) for w in range(n_win)]
    events = [torch.cuda.Event(enable_timing=True) for _ in range(n_win + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events[0].record(stream)
    i = 0
    for w, n in enumerate(sizes):
        for _ in range(n):
            fn(warmup + i)
            i += 1
        events[w + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    window_ms = [events[w].elapsed_time(events[w + 1]) / n for w, n in enumerate(sizes)]
    return Timing(wall, events[0].elapsed_time(events[-1]) / steps, window_ms)


def to_dev(a):
    """numpy (fp32, or bf16 bit patterns as uint16) -> CUDA tensor."""
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def attn_tensors(torch, w):
    import synth
    t0 = time.perf_counter()
    t = synth.attn_inputs(w)
    log(f"[bench] generated {w.name} in {time.perf_counter() - t0:.1f}s")
    return t, to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def bench_prefill(torch, osx, args):
    import synth
    w = synth.WORKLOADS["gqa_prefill_bf16"]
    t, q, k, v = attn_tensors(torch, w)
    out = torch.empty_like(q)
    tm = timed(torch, lambda i: osx.attn_fwd(q, k, v, causal=True, out=out), args.steps, args.warmup)
    wall, kern_ms = tm
    tflops = w.flops() / (kern_ms * 1e-3) / 1e12
    res = {"wall_s": wall, "ms_per_step": wall / args.steps * 1e3, "kernel_ms": kern_ms, "tflops": tflops,
           "per_call_us": tm.per_call_us(),
           "roofline": roofline("mfma", tflops, PEAK_BF16_TFLOPS, "TFLOP/s", traffic_for("prefill_bf16_kernel")),
           "qkv": (q, k, v)}
    return res, t, w


def bench_unfused(torch, osx, args, q, k, v, w, fused_ms):
    """The unfused three-kernel comparator on the prefill workload: S = scale q k^T to HBM (fp32), softmax in
    place, P v.  Its HBM traffic is dominated by four passes over S (written, read and rewritten by the
    softmax, read by the P v product): 16 bytes per score, plus q, k, v, o once."""
    out = torch.empty_like(q)
    ws = torch.empty(osx.attn_fwd_unfused_workspace(osx.OSX_BF16, w.batch, w.heads_q, w.heads_kv, w.seq_q, w.seq_k,
                                                    w.head_dim, True), dtype=torch.uint8, device="cuda")
    steps = max(3, args.steps // 4)
    tm = timed(torch, lambda i: osx.attn_fwd_unfused(q, k, v, causal=True, out=out, workspace=ws), steps,
               args.warmup)
    ms = tm.ms
    scores = float(w.batch * w.heads_q * w.seq_q * w.seq_k)
    nbytes = 16.0 * scores + w.bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "unit": "GB/s", "value": round(gbs, 1), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(), "bytes_per_call": nbytes, "score_matrix_bytes": 4.0 * scores,
            "tflops_causal_adjusted": round(w.flops() / (ms * 1e-3) / 1e12, 2),
            "time_vs_fused": round(ms / fused_ms, 2),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}


def bench_decode(torch, osx, args):
    import synth
    w = synth.WORKLOADS["gqa_decode_bf16"]
    t, q, k, v = attn_tensors(torch, w)
    out = torch.empty_like(q)
    ws = torch.empty(osx.attn_fwd_workspace(osx.OSX_BF16, w.batch, w.heads_q, w.heads_kv, 1, w.seq_k, w.head_dim),
                     dtype=torch.uint8, device="cuda")
    tm = timed(torch, lambda i: osx.attn_fwd(q, k, v, out=out, workspace=ws), args.steps, args.warmup)
    ms = tm.ms
    gbs = w.bytes() / (ms * 1e-3) / 1e9
    return {"workload": w.name, "unit": "GB/s", "value": round(gbs, 1), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(), "bytes_per_call": w.bytes(),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", traffic_for("decode_bf16_kernel"))}, t


def softmax_reads(osx, w):
    """Times the planned kernels read x from memory: once when a row stays in registers, twice when split."""
    return 2 if osx.softmax_rows_plan(w.rows, w.cols)["kernel_name"] == "softmax_split" else 1


def bench_softmax(torch, osx, args):
    import synth
    w = synth.WORKLOADS["softmax_1x16m"]
    x = to_dev(synth.softmax_inputs(w))
    # 5 input/output pairs (640 MiB) rotate so no call finds its data in the 256 MB MALL.
    xs = [x.clone() for _ in range(5)]
    ys = [torch.empty_like(x) for _ in range(5)]
    ws = torch.empty(osx.softmax_rows_workspace(w.rows, w.cols), dtype=torch.uint8, device="cuda")
    tm = timed(torch, lambda i: osx.softmax_rows(xs[i % 5], out=ys[i % 5], workspace=ws), args.steps, args.warmup)
    ms = tm.ms
    reads = softmax_reads(osx, w)
    gbs = w.bytes(reads) / (ms * 1e-3) / 1e9
    return {"workload": w.name, "unit": "GB/s", "value": round(gbs, 1), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(), "bytes_per_call": w.bytes(reads), "reads_of_x": reads,
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", traffic_for("softmax_split"))}


def bench_softmax_3pass(torch, osx, args, two_pass_us):
    """The three-pass comparator designs on the long-row workload, same rotation of buffers as the two-pass line.

    Algorithmic bytes: ATOMIC reads x three times and writes y once (4 x 4N);
    STASH reads x twice, writes y twice and reads it once (5 x 4N)."""
    import synth
    w = synth.WORKLOADS["softmax_1x16m"]
    x = to_dev(synth.softmax_inputs(w))
    xs = [x.clone() for _ in range(5)]
    ys = [torch.empty_like(x) for _ in range(5)]
    out = {}
    for name, method, passes in (("atomic", osx.OSX_3PASS_ATOMIC, 4), ("stash", osx.OSX_3PASS_STASH, 5)):
        ws = torch.empty(osx.softmax_rows_3pass_workspace(w.rows, w.cols, method), dtype=torch.uint8, device="cuda")
        tm = timed(torch, lambda i: osx.softmax_rows_3pass(xs[i % 5], method, out=ys[i % 5], workspace=ws),
                   args.steps, args.warmup)
        ms = tm.ms
        nbytes = passes * 4.0 * w.rows * w.cols
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"softmax_1x16m_3pass_{name}"] = {
            "workload": w.name, "unit": "GB/s", "value": round(gbs, 1), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(), "bytes_per_call": nbytes,
            "time_vs_two_pass": round(ms * 1e3 / two_pass_us, 3),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
    return out


def bench_softmax_causal(torch, osx, args):
    """Causal bf16 score rows: one wavefront per row reads the visible columns and zero-fills the rest."""
    import synth
    w = synth.WORKLOADS["softmax_causal_bf16"]
    x = to_dev(synth.softmax_inputs(w))
    # 5 input/output pairs (1.3 GB) rotate so no call finds its data in the 256 MB MALL.
    xs = [x.clone() for _ in range(5)]
    ys = [torch.empty_like(x) for _ in range(5)]
    ws = torch.empty(max(1, osx.softmax_rows_workspace(w.rows, w.cols)), dtype=torch.uint8, device="cuda")
    tm = timed(torch, lambda i: osx.softmax_rows(xs[i % 5], out=ys[i % 5], workspace=ws,
                                                 causal_period=w.causal_period, scale=w.scale),
               args.steps, args.warmup)
    ms = tm.ms
    reads = softmax_reads(osx, w)
    gbs = w.bytes(reads) / (ms * 1e-3) / 1e9
    return {"workload": w.name, "unit": "GB/s", "value": round(gbs, 1), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(), "bytes_per_call": w.bytes(reads), "reads_of_x": reads,
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", traffic_for("softmax_wave_causal"))}


def bench_f32(torch, osx, args):
    import synth
    w = synth.WORKLOADS["attn_f32_4k_d128"]
    t, q, k, v = attn_tensors(torch, w)
    out = torch.empty_like(q)
    tm = timed(torch, lambda i: osx.attn_fwd(q, k, v, out=out), args.steps, args.warmup)
    ms = tm.ms
    tf = w.flops() / (ms * 1e-3) / 1e12
    return {"workload": w.name, "unit": "TFLOP/s", "value": round(tf, 2), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(),
            "roofline": roofline("mfma", tf, PEAK_F32_TFLOPS, "TFLOP/s", traffic_for("prefill_f32_kernel"))}, t


def bench_f32_normalised(torch, osx, args, plain_us):
    """The normalised-output recurrence (O kept normalised after every block) on the same fp32 workload."""
    import synth
    w = synth.WORKLOADS["attn_f32_4k_d128"]
    _, q, k, v = attn_tensors(torch, w)
    out = torch.empty_like(q)
    tm = timed(torch, lambda i: osx.attn_fwd_normalised(q, k, v, out=out), args.steps, args.warmup)
    ms = tm.ms
    tf = w.flops() / (ms * 1e-3) / 1e12
    return {"workload": w.name, "unit": "TFLOP/s", "value": round(tf, 2), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(),
            "time_vs_unnormalised": round(ms * 1e3 / plain_us, 3),
            "roofline": roofline("mfma", tf, PEAK_F32_TFLOPS, "TFLOP/s", None)}


def bench_lse(torch, osx, args, q, k, v, w, plain_ms):
    """The prefill call that also writes each query row's log-sum-exp (osx_attn_fwd_lse)."""
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    tm = timed(torch, lambda i: osx.attn_fwd(q, k, v, causal=True, out=out, lse=lse), args.steps, args.warmup)
    ms = tm.ms
    tf = w.flops() / (ms * 1e-3) / 1e12
    return {"workload": w.name, "unit": "TFLOP/s", "value": round(tf, 2), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(),
            "time_vs_without_lse": round(ms / plain_ms, 3),
            "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", None)}


def bench_small(torch, osx, args):
    import synth
    res = {}
    w = synth.WORKLOADS["attn_f32_m64_n100_d48"]
    _, q, k, v = attn_tensors(torch, w)
    out = torch.empty_like(q)
    tm = timed(torch, lambda i: osx.attn_fwd(q, k, v, out=out), args.steps, args.warmup)
    res[w.name] = {"unit": "us", "value": round(1e3 * tm.ms, 2), "per_call_us": tm.per_call_us(),
                   "note": "launch-latency bound; roofline fraction not meaningful"}
    w = synth.WORKLOADS["softmax_4x200"]
    x = to_dev(synth.softmax_inputs(w))
    y = torch.empty_like(x)
    tm = timed(torch, lambda i: osx.softmax_rows(x, out=y), args.steps, args.warmup)
    res[w.name] = {"unit": "us", "value": round(1e3 * tm.ms, 2), "per_call_us": tm.per_call_us(),
                   "note": "launch-latency bound; roofline fraction not meaningful"}
    return res


def bench_read_probe(torch, osx, args):
    """Context for the HBM-bound lines: a plain 16-byte streaming read of 2 GiB (osx_read_probe) on the same GPU."""
    n = 1 << 29
    x = torch.ones(n, dtype=torch.int32, device="cuda")
    sink = torch.empty(osx.lib.osx_read_probe_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    tm = timed(torch, lambda i: osx.read_probe(x, sink=sink), args.steps, args.warmup)
    ms = tm.ms
    gbs = 4.0 * n / (ms * 1e-3) / 1e9
    return {"workload": "read 2 GiB", "unit": "GB/s", "value": round(gbs, 1), "call_us": round(ms * 1e3, 2),
            "per_call_us": tm.per_call_us(),
            "note": "achievable-bandwidth reference (loads only), not a step of the method",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}


def bench_copy(torch, args):
    """A plain device copy of known size (256 MiB), to calibrate the HBM byte counters."""
    n = 64 << 20
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    timed(torch, lambda i: b.copy_(a), args.steps, args.warmup)
    return {"bytes_read": 4 * n, "bytes_written": 4 * n}


def cpu_baseline(host):
    """The fp64 oracle, timed on the host's cores, on every workload in full.

    ``host`` maps workload names to the host inputs the GPU lines used (the
    rest are regenerated from their seeds).  Single-head workloads call the
    oracle once (numpy's BLAS uses every core for the products; the
    element-wise steps run on one thread); the multi-head ones spread their
    (batch, query head) slices over ``oracle.attention_heads``' pool of host
    threads.  Each entry gives the wall time and the rate under the GPU line's
    algorithmic count; the causal prefill's rate uses the causal-adjusted flop
    count although the oracle computes the dense score matrix.  The headline
    value is the causal GQA prefill's."""
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    workers = oracle.pool.default_workers()
    per = {}

    def run(name, fn, work, unit, threads, what):
        t0 = time.perf_counter()
        fn()
        el = time.perf_counter() - t0
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        per[name] = {"wall_s": round(el, 6), "value": round(work / el / scale, 6), "unit": unit,
                     "threads": threads, "what": what}
        log(f"[bench] oracle {name}: {el:.2f}s")

    W = synth.WORKLOADS
    w = W["attn_f32_m64_n100_d48"]
    t = synth.attn_inputs(w)
    run(w.name, lambda: oracle.attention(t["q"], t["k"], t["v"]), w.flops(), "TFLOP/s", cores, "oracle.attention")
    for name in ("softmax_4x200", "softmax_1x16m"):
        w = W[name]
        x = synth.softmax_inputs(w)
        run(name, lambda: oracle.softmax_rows(x), w.bytes(2 if w.cols > 8192 else 1), "GB/s", 1,
            "oracle.softmax_rows")
    w = W["attn_f32_4k_d128"]
    t = host.get(w.name) or synth.attn_inputs(w)
    run(w.name, lambda: oracle.attention(t["q"], t["k"], t["v"]), w.flops(), "TFLOP/s", cores, "oracle.attention")
    w = W["gqa_decode_bf16"]
    t = host.get(w.name) or synth.attn_inputs(w)
    run(w.name, lambda: oracle.attention_heads(t["q"], t["k"], t["v"], workers=workers), w.bytes(), "GB/s", workers,
        f"oracle.attention_heads, {w.batch * w.heads_q} heads on {workers} threads")
    w = W["gqa_prefill_bf16"]
    t = host[w.name]
    run(w.name, lambda: oracle.attention_heads(t["q"], t["k"], t["v"], causal=True, workers=workers), w.flops(),
        "TFLOP/s", workers, f"oracle.attention_heads, {w.batch * w.heads_q} heads on {workers} threads")
    head = per[w.name]
    return {"value": head["value"], "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"all {w.batch * w.heads_q} (batch, query head) slices of {w.name} (the whole workload), "
                      f"{head['wall_s']}s on a pool of {workers} host threads (BLAS one thread per call); "
                      "causal-adjusted flop count (the oracle computes the dense score matrix)",
            "per_config": per}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested; the library and this benchmark use exactly one GPU "
              "(no collectives or sharding). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import online_softmax_02_amd as osx
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    log(f"[bench] device {torch.cuda.get_device_name(0)}; library {osx.LIB_PATH}")

    if args.only == "copy":
        print(json.dumps({"copy": bench_copy(torch, args)}))
        return
    also = {}
    if args.only == "probe":
        print(json.dumps({"also": {"hbm_read_probe": bench_read_probe(torch, osx, args)}}))
        return
    if args.only in ("decode",):
        also["gqa_decode_bf16"], _ = bench_decode(torch, osx, args)
        print(json.dumps({"also": also}))
        return
    if args.only in ("softmax",):
        also["softmax_1x16m"] = bench_softmax(torch, osx, args)
        also["softmax_causal_bf16"] = bench_softmax_causal(torch, osx, args)
        also.update(bench_softmax_3pass(torch, osx, args, also["softmax_1x16m"]["call_us"]))
        print(json.dumps({"also": also}))
        return
    if args.only in ("f32",):
        also["attn_f32_4k_d128"], _ = bench_f32(torch, osx, args)
        also["attn_f32_normalised_4k_d128"] = bench_f32_normalised(torch, osx, args,
                                                                   also["attn_f32_4k_d128"]["call_us"])
        print(json.dumps({"also": also}))
        return
    if args.only in ("small",):
        print(json.dumps({"also": bench_small(torch, osx, args)}))
        return

    head, t, w = bench_prefill(torch, osx, args)
    host = {w.name: t}
    log(f"[bench] prefill {head['tflops']:.1f} TFLOP/s ({head['kernel_ms']:.3f} ms per call)")
    qkv = head.pop("qkv")
    if args.only in ("all", "unfused"):
        also["attn_unfused_gqa_prefill_bf16"] = bench_unfused(torch, osx, args, *qkv, w, head["kernel_ms"])
        log(f"[bench] unfused comparator {also['attn_unfused_gqa_prefill_bf16']['call_us']} us")
    if args.only == "all":
        also["attn_lse_gqa_prefill_bf16"] = bench_lse(torch, osx, args, *qkv, w, head["kernel_ms"])
        log(f"[bench] prefill with lse {also['attn_lse_gqa_prefill_bf16']['value']} TFLOP/s")
    del qkv
    if args.only == "unfused":
        print(json.dumps({"also": also}))
        return
    if args.only == "all":
        also["hbm_read_probe"] = bench_read_probe(torch, osx, args)
        log(f"[bench] plain streaming read {also['hbm_read_probe']['value']} GB/s")
        also["gqa_decode_bf16"], host["gqa_decode_bf16"] = bench_decode(torch, osx, args)
        log(f"[bench] decode {also['gqa_decode_bf16']['value']} GB/s")
        also["softmax_1x16m"] = bench_softmax(torch, osx, args)
        log(f"[bench] softmax {also['softmax_1x16m']['value']} GB/s")
        also["softmax_causal_bf16"] = bench_softmax_causal(torch, osx, args)
        log(f"[bench] causal bf16 softmax {also['softmax_causal_bf16']['value']} GB/s")
        also.update(bench_softmax_3pass(torch, osx, args, also["softmax_1x16m"]["call_us"]))
        log("[bench] three-pass comparators done")
        also["attn_f32_4k_d128"], host["attn_f32_4k_d128"] = bench_f32(torch, osx, args)
        log(f"[bench] fp32 attention {also['attn_f32_4k_d128']['value']} TFLOP/s")
        also["attn_f32_normalised_4k_d128"] = bench_f32_normalised(torch, osx, args,
                                                                   also["attn_f32_4k_d128"]["call_us"])
        log(f"[bench] fp32 normalised-output attention {also['attn_f32_normalised_4k_d128']['value']} TFLOP/s")
        also.update(bench_small(torch, osx, args))
    cpu = None
    if not args.no_cpu_baseline and args.only == "all":
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(host)
    rec = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), rounded to bf16)",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seq_q": w.seq_q, "seq_k": w.seq_k, "head_dim": w.head_dim, "causal": w.causal,
                   "parallelism": "none (one GPU)"},
        "kernel_ms": round(head["kernel_ms"], 4),
        "per_call_us": head["per_call_us"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
