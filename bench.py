"""Benchmark of the exact tiled attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one pass over every stage of the path, each on its own synthetic
seeded workload with inputs already resident in HBM:
  * causal GQA prefill, B=1, Hq=32, Hkv=8, N=4096, d=128, bf16 (the headline
    workload: ``value`` is its TFLOP/s),
  * kv_append of 4 new tokens + paged 4-token decode, B=32, 16-token blocks,
    cached lengths uniform in [1024, 16384],
  * split-KV decode of 1 token against 16 contiguous 32768-token caches.
Before the W warmup steps the step runs untimed for --settle-seconds (0.3 s)
so that the GPU clocks have reached their loaded level: the first ~30 ms of
work on an idle MI355X run about 10% slower. Each stage is timed with HIP
events recorded on the stream the library
launches on; the long-context prefill (N=32768), the chunked prefill against
the paged cache (8 sequences, 512 new tokens after 1k-8k cached ones), the
backward pass of the 4k prefill, the
paged 4-token decode over an fp8 (E4M3) cache and the fp32 single-head case
are timed in their own loops after the steps. Last, on the host, the 1000-chat
serving simulation compares the native block pool (paged cache) with
contiguous allocation. FLOPs count visible
(query, key) pairs x 4d; decode bytes count each visible K/V row once.
Prints ONE JSON line.
"""

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
METRIC = "prefill attention TFLOP/s and decode KV-read GB/s, % of MI355X peak"


def causal_pairs(nq, nk, q_offset=0):
    """Visible (row, key) pairs of a causal nq x nk mask, closed form."""
    tot = 0
    # row i sees min(nk, max(0, i + q_offset + 1)) keys
    for i in range(nq):
        tot += min(nk, max(0, i + q_offset + 1))
    return tot


def prefill_flops(B, Hq, N, d, causal=True):
    pairs = causal_pairs(N, N) if causal else N * N
    return 4.0 * d * B * Hq * pairs


def chunk_flops(seq_lens, Nq, Hq, d):
    """Causal chunk of Nq new rows after seq_len - Nq cached keys, per sequence."""
    return 4.0 * d * Hq * sum(causal_pairs(Nq, n, n - Nq) for n in seq_lens)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--long-steps", type=int, default=5)
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="run the step untimed for this long before the warmup steps, so the "
                         "GPU clocks reach their loaded level (the first ~30 ms of work run "
                         "about 10%% slower)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chat-sim", action="store_true",
                    help="skip the host-side 1000-chat block-pool simulation")
    ap.add_argument("--stage", default=None,
                    choices=["prefill_4k", "prefill_32k", "splitkv_decode_32k", "paged_decode_q4",
                             "paged_decode_q4_d64", "chunked_prefill_paged", "paged_decode_q4_fp8",
                             "backward_4k", "single_head_f32", "copy_1gib"],
                    help="run only this stage --steps times and exit (for profiler runs); "
                         "copy_1gib is a plain 1 GiB device copy used to calibrate HBM counters")
    return ap.parse_args()


def run_stage(args, torch, eta, inputs, dev):
    """One stage alone, --warmup + --steps launches, one summary line on stderr."""
    name = args.stage
    if name == "copy_1gib":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)  # noqa: E731
    elif name in ("prefill_4k", "prefill_32k"):
        wl = "causal_gqa_prefill_4k" if name == "prefill_4k" else "causal_gqa_prefill_32k"
        q, k, v = inputs.workload_inputs(wl, dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fn = lambda: eta.attn_prefill(q, k, v, causal=True, out=o, lse=lse)  # noqa: E731
    elif name == "single_head_f32":
        q, k, v = inputs.workload_inputs(name, dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fn = lambda: eta.attn_prefill(q, k, v, causal=False, out=o, lse=lse)  # noqa: E731
    elif name == "backward_4k":
        q, k, v, do = inputs.workload_inputs("causal_gqa_backward_4k", dev)
        o, lse = eta.attn_prefill(q, k, v, causal=True)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(eta.attn_prefill_backward_workspace_bytes(
            q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2], q.shape[3], True),
            dtype=torch.uint8, device=dev)
        fn = lambda: eta.attn_prefill_backward(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk,  # noqa
                                               dv=dv, workspace=ws)
    elif name == "chunked_prefill_paged":
        p = inputs.workload_inputs(name, dev)
        eta.kv_append(p["k_new"], p["v_new"], p["k_pool"], p["v_pool"], p["cache_lens"],
                      block_table=p["block_table"])
        fn = lambda: eta.attn_prefill_paged(p["q"], p["k_pool"], p["v_pool"], p["seq_lens"],  # noqa
                                            block_table=p["block_table"], causal=True)
    elif name == "paged_decode_q4_fp8":
        p = inputs.workload_inputs(name, dev)
        eta.kv_append_fp8(p["k_new"], p["v_new"], p["k_pool"], p["v_pool"], p["k_scale"],
                          p["v_scale"], p["cache_lens"], block_table=p["block_table"])
        fn = lambda: eta.attn_decode_paged_fp8(p["q"], p["k_pool"], p["v_pool"], p["k_scale"],  # noqa
                                               p["v_scale"], p["seq_lens"],
                                               block_table=p["block_table"], causal=True)
    elif name == "splitkv_decode_32k":
        q, kc, vc, sl = inputs.workload_inputs(name, dev)
        fn = lambda: eta.attn_decode_paged(q, kc, vc, sl, causal=True)  # noqa: E731
    else:
        p = inputs.workload_inputs(name, dev)
        eta.kv_append(p["k_new"], p["v_new"], p["k_pool"], p["v_pool"], p["cache_lens"],
                      block_table=p["block_table"])
        fn = lambda: eta.attn_decode_paged(p["q"], p["k_pool"], p["v_pool"], p["seq_lens"],  # noqa
                                           block_table=p["block_table"], causal=True)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(f"[bench] stage {name}: {args.steps} launches, {dt * 1e3:.4f} ms each (wall)",
          file=sys.stderr, flush=True)


class StageTimer:
    """Per-stage HIP events on one stream; durations summed over the timed steps."""

    def __init__(self, torch, stream, names):
        self.torch = torch
        self.stream = stream
        self.names = names
        self.pairs = {n: [] for n in names}

    def run(self, name, fn, record=True):
        if not record:
            fn()
            return
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record(self.stream)
        fn()
        ev1.record(self.stream)
        self.pairs[name].append((ev0, ev1))

    def times_ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs[name]]

    def mean_ms(self, name):
        ts = self.times_ms(name)
        return sum(ts) / len(ts)

    def stats(self, name):
        """mean, median and min of the event-timed durations, in ms"""
        ts = sorted(self.times_ms(name))
        n = len(ts)
        med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
        return {"ms": round(sum(ts) / n, 5), "ms_median": round(med, 5), "ms_min": round(ts[0], 5),
                "launches": n}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters_all_workloads.md")
CSRC = os.path.join(ROOT, "exact_tiled_attention_flashattention_amd", "csrc")


def source_fingerprint(sources):
    """First 16 hex digits of the sha256 of the kernel sources' code: comments and
    blank lines are dropped, so that a change of wording alone keeps the figure."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(CSRC, f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code.strip():
                h.update((code + "\n").encode())
    return h.hexdigest()[:16]


def counter_traffic(stage, kernel, sources):
    """HBM bytes per launch of `kernel` on `stage` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by its plain-copy calibration), or None
    when the kernel's code has changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fp = source_fingerprint(sources)
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) < 4 or parts[0] != "traffic" or parts[1] != stage or parts[2] != kernel:
                continue
            kv = dict(x.split("=", 1) for x in parts[3:] if "=" in x)
            if kv.get("sources_sha256") != fp:
                return None
            return int(kv["bytes_per_launch"])
    return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the visible cores
        return os.cpu_count()


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _single_thread(fn):
    """Run fn() with BLAS limited to one thread; None when that cannot be arranged."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t


def cpu_baselines(torch, inputs, dev, seconds=5.0):
    """The fp64 oracle, timed on the host's cores on bounded samples of every
    workload (about 20-30 s of CPU work in all), each rate scaled by the same
    convention as the GPU figure (visible pairs x 4d FLOP; each visible K/V row
    once for decode). Returns the headline workload's figure with the others
    under "per_workload"."""
    import numpy as np

    import oracle

    threads = _blas_threads()
    out = {}

    # 4k causal GQA prefill: whole heads (all 4096 rows), cycling over the 32
    q, k, v = (t.cpu() for t in inputs.workload_inputs("causal_gqa_prefill_4k", dev))
    N, d, G, Hq = q.shape[2], q.shape[3], q.shape[1] // k.shape[1], q.shape[1]
    rows = np.arange(N)
    done, t0 = 0, time.perf_counter()
    while done < 1 or (time.perf_counter() - t0 < seconds and done < 4 * Hq):
        hq = done % Hq
        oracle.attention_rows(q[0, hq], rows, k[0, hq // G], v[0, hq // G], 1 / math.sqrt(d), True)
        done += 1
    dt = time.perf_counter() - t0
    rate = prefill_flops(1, done, N, d) / dt / 1e12
    one = _single_thread(lambda: oracle.attention_rows(q[0, 0], rows, k[0, 0], v[0, 0],
                                                       1 / math.sqrt(d), True))
    out["causal_gqa_prefill_4k"] = {
        "value": round(rate, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{done} whole heads (all {N} rows; heads in order, cycling over the {Hq}), "
                  f"{dt:.1f} s",
        "single_core_value": (round(prefill_flops(1, 1, N, d) / one / 1e12, 6) if one else None),
        "whole_workload_s_estimate": round(prefill_flops(1, Hq, N, d) / (rate * 1e12), 2)}
    del q, k, v

    # 32k causal GQA prefill: every 16th row of one head (2048 rows spread over
    # the whole causal triangle, so their visible pairs average those of the
    # head), extrapolated to the workload
    q, k, v = inputs.workload_inputs("causal_gqa_prefill_32k", dev)
    N3 = q.shape[2]
    rows3 = np.arange(0, N3, 16)
    qh, kh, vh = q[0, 0, rows3].cpu(), k[0, 0].cpu(), v[0, 0].cpu()
    del q, k, v
    t0 = time.perf_counter()
    oracle.attention_rows(qh, rows3, kh, vh, 1 / math.sqrt(d), True)
    dt = time.perf_counter() - t0
    fl = 4.0 * d * float((rows3 + 1).sum())
    rate = fl / dt / 1e12
    out["causal_gqa_prefill_32k"] = {
        "value": round(rate, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"rows 0, 16, 32, ... ({rows3.size} rows) of head 0 against all {N3} keys, "
                  f"{dt:.1f} s; the whole workload is extrapolated at that rate",
        "whole_workload_s_estimate": round(prefill_flops(1, 32, N3, d) / (rate * 1e12), 1),
        "extrapolated": True}
    del qh, kh, vh

    # 16 x 32k split-KV decode: whole sequences (every head), until the budget is spent
    w4 = inputs.WORKLOADS["splitkv_decode_32k"]
    q, kc, vc, sl = inputs.workload_inputs("splitkv_decode_32k", dev)
    qc, slc = q.cpu(), sl.cpu()
    per_seq = 2 * 2 * w4["Hkv"] * w4["d"] * w4["seq_len"]
    done, t0, t_copy = 0, time.perf_counter(), 0.0
    while done < 1 or (time.perf_counter() - t0 - t_copy < seconds and done < w4["B"]):
        b = done
        tc = time.perf_counter()
        kb, vb = kc[b:b + 1].cpu(), vc[b:b + 1].cpu()  # the device-to-host copy is not timed
        t_copy += time.perf_counter() - tc
        oracle.decode_attention(qc[b:b + 1], kb, vb, slc[b:b + 1], 1 / math.sqrt(w4["d"]), True)
        done += 1
    dt = time.perf_counter() - t0 - t_copy
    del q, kc, vc
    out["splitkv_decode_32k"] = {
        "value": round(done * per_seq / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {w4['B']} sequences, every head ({dt:.1f} s of oracle time)",
        "whole_workload_s_estimate": round(w4["B"] * dt / done, 2)}

    # paged 4-token decode (bf16 cache): whole sequences through the oracle's gather
    w5 = inputs.WORKLOADS["paged_decode_q4"]
    p = inputs.workload_inputs("paged_decode_q4", dev)
    kp, vp = p["k_pool"].cpu(), p["v_pool"].cpu()
    qc, tab, seq = p["q"].cpu(), p["block_table"].cpu(), p["seq_lens"].cpu()
    del p
    done, t0, nbytes = 0, time.perf_counter(), 0
    while done < 1 or (time.perf_counter() - t0 < seconds and done < w5["B"]):
        b = done
        oracle.decode_attention(qc[b:b + 1], kp, vp, seq[b:b + 1], 1 / math.sqrt(w5["d"]), True,
                                block_table=tab[b:b + 1])
        nbytes += 2 * 2 * w5["Hkv"] * w5["d"] * int(seq[b])
        done += 1
    dt = time.perf_counter() - t0
    allb = 2 * 2 * w5["Hkv"] * w5["d"] * int(seq.sum())
    out["paged_decode_q4"] = {
        "value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"{done} of {w5['B']} sequences, every head ({dt:.1f} s)",
        "whole_workload_s_estimate": round(allb / (nbytes / dt), 2)}
    del kp, vp

    # single-head fp32 256 x 64: the whole workload, all cores and one core
    q, k, v = (t.cpu() for t in inputs.workload_inputs("single_head_f32", dev))
    n1 = q.shape[2]
    rows1 = np.arange(n1)
    reps, t0 = 0, time.perf_counter()
    while reps < 20 or time.perf_counter() - t0 < 0.5:
        oracle.attention_rows(q[0, 0], rows1, k[0, 0], v[0, 0], 0.125, False)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    one = _single_thread(lambda: [oracle.attention_rows(q[0, 0], rows1, k[0, 0], v[0, 0], 0.125,
                                                        False) for _ in range(20)])
    out["single_head_f32"] = {
        "us": round(dt * 1e6, 1), "cores": threads, "kind": "oracle",
        "sample": f"the whole workload, {reps} repetitions",
        "single_core_us": round(one / 20 * 1e6, 1) if one else None}

    head = dict(out["causal_gqa_prefill_4k"])
    head["host"] = cpu_model()
    head["host_cpus"] = os.cpu_count()
    head["per_workload"] = {k2: v2 for k2, v2 in out.items() if k2 != "causal_gqa_prefill_4k"}
    return head


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch

    import exact_tiled_attention_flashattention_amd as eta
    from exact_tiled_attention_flashattention_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    eta.library()
    dev = torch.device("cuda:0")
    if args.stage is not None:
        run_stage(args, torch, eta, inputs, dev)
        return
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] device {torch.cuda.get_device_name(dev)}; building inputs", file=sys.stderr,
          flush=True)

    # ---- inputs (seeded, generated on the device) ---------------------------------
    q2, k2, v2 = inputs.workload_inputs("causal_gqa_prefill_4k", dev)
    o2 = torch.empty_like(q2)
    l2 = torch.empty(q2.shape[:3], dtype=torch.float32, device=dev)
    w4 = inputs.WORKLOADS["splitkv_decode_32k"]
    q4, kc4, vc4, sl4 = inputs.workload_inputs("splitkv_decode_32k", dev)
    o4 = torch.empty_like(q4)
    l4 = torch.empty((w4["B"], w4["Hq"], 1), dtype=torch.float32, device=dev)
    ws4 = torch.empty(eta.attn_decode_workspace_bytes(w4["B"], w4["Hq"], w4["Hkv"], 1, w4["d"],
                                                      w4["seq_len"]), dtype=torch.uint8, device=dev)
    w5 = inputs.WORKLOADS["paged_decode_q4"]
    p5 = inputs.workload_inputs("paged_decode_q4", dev)
    L5 = p5["block_table"].shape[1] * 16
    o5 = torch.empty_like(p5["q"])
    l5 = torch.empty((w5["B"], w5["Hq"], 4), dtype=torch.float32, device=dev)
    ws5 = torch.empty(eta.attn_decode_workspace_bytes(w5["B"], w5["Hq"], w5["Hkv"], 4, w5["d"], L5),
                      dtype=torch.uint8, device=dev)
    seq5 = [int(x) for x in p5["seq_lens"].cpu()]
    torch.cuda.synchronize()

    def prefill4k():
        eta.attn_prefill(q2, k2, v2, causal=True, out=o2, lse=l2)

    def append5():
        eta.kv_append(p5["k_new"], p5["v_new"], p5["k_pool"], p5["v_pool"], p5["cache_lens"],
                      block_table=p5["block_table"])

    def decode5():
        eta.attn_decode_paged(p5["q"], p5["k_pool"], p5["v_pool"], p5["seq_lens"],
                              block_table=p5["block_table"], causal=True, workspace=ws5, out=o5,
                              lse=l5)

    def decode4():
        eta.attn_decode_paged(q4, kc4, vc4, sl4, causal=True, workspace=ws4, out=o4, lse=l4)

    stages = [("prefill_4k", prefill4k), ("kv_append_q4", append5),
              ("paged_decode_q4", decode5), ("splitkv_decode_32k", decode4)]
    timer = StageTimer(torch, stream, [n for n, _ in stages])

    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for n, fn in stages:
            timer.run(n, fn, record=False)
        torch.cuda.synchronize()
        settle += 1
    for _ in range(args.warmup):
        for n, fn in stages:
            timer.run(n, fn, record=False)
    torch.cuda.synchronize()
    print(f"[bench] clock settle {settle} steps, warmup {args.warmup} steps; timing {args.steps} "
          f"steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for n, fn in stages:
            timer.run(n, fn)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    flops2 = prefill_flops(1, 32, 4096, 128)
    ms2 = timer.mean_ms("prefill_4k")
    tflops2 = flops2 / (ms2 * 1e-3) / 1e12
    result_workloads = {
        "causal_gqa_prefill_4k": {**timer.stats("prefill_4k"), "TFLOP/s": round(tflops2, 2),
                                  "frac_of_peak": round(tflops2 / PEAK_BF16_TFLOPS, 4),
                                  "flops": flops2},
    }
    bytes4 = 2 * 2 * w4["Hkv"] * w4["d"] * w4["B"] * w4["seq_len"]
    ms4 = timer.mean_ms("splitkv_decode_32k")
    bytes5 = 2 * 2 * w5["Hkv"] * w5["d"] * sum(seq5)
    ms5 = timer.mean_ms("paged_decode_q4")
    msa = timer.mean_ms("kv_append_q4")
    result_workloads["splitkv_decode_32k"] = {
        **timer.stats("splitkv_decode_32k"), "GB/s": round(bytes4 / (ms4 * 1e-3) / 1e9, 1),
        "frac_of_peak": round(bytes4 / (ms4 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "kv_bytes": bytes4,
        "traffic_partial_kernel": counter_traffic("splitkv_decode_32k", "decode_partial_kernel<128,false>",
                                                  ["common.h", "decode.hip"])}
    result_workloads["paged_decode_q4"] = {
        **timer.stats("paged_decode_q4"), "GB/s": round(bytes5 / (ms5 * 1e-3) / 1e9, 1),
        "frac_of_peak": round(bytes5 / (ms5 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "kv_bytes": bytes5, "kv_append_ms": round(msa, 5),
        "traffic_partial_kernel": counter_traffic("paged_decode_q4", "decode_partial_kernel<128,false>",
                                                  ["common.h", "decode.hip"])}

    # long-context prefill and the fp32 single-head case, in their own loops
    print("[bench] long-context prefill", file=sys.stderr, flush=True)
    del kc4, vc4
    torch.cuda.empty_cache()
    q3, k3, v3 = inputs.workload_inputs("causal_gqa_prefill_32k", dev)
    o3 = torch.empty_like(q3)
    l3 = torch.empty(q3.shape[:3], dtype=torch.float32, device=dev)
    t3 = StageTimer(torch, stream, ["p"])
    eta.attn_prefill(q3, k3, v3, causal=True, out=o3, lse=l3)
    for _ in range(max(1, args.long_steps)):
        t3.run("p", lambda: eta.attn_prefill(q3, k3, v3, causal=True, out=o3, lse=l3))
    torch.cuda.synchronize()
    ms3 = t3.mean_ms("p")
    flops3 = prefill_flops(1, 32, 32768, 128)
    result_workloads["causal_gqa_prefill_32k"] = {
        **t3.stats("p"), "TFLOP/s": round(flops3 / (ms3 * 1e-3) / 1e12, 2),
        "frac_of_peak": round(flops3 / (ms3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops": flops3}
    del q3, k3, v3, o3, l3
    torch.cuda.empty_cache()
    # chunked prefill against the paged cache: 512 new tokens per sequence
    w6 = inputs.WORKLOADS["chunked_prefill_paged"]
    p6 = inputs.workload_inputs("chunked_prefill_paged", dev)
    eta.kv_append(p6["k_new"], p6["v_new"], p6["k_pool"], p6["v_pool"], p6["cache_lens"],
                  block_table=p6["block_table"])
    o6 = torch.empty_like(p6["q"])
    l6 = torch.empty((w6["B"], w6["Hq"], w6["Nq"]), dtype=torch.float32, device=dev)

    def chunk6():
        eta.attn_prefill_paged(p6["q"], p6["k_pool"], p6["v_pool"], p6["seq_lens"],
                               block_table=p6["block_table"], causal=True, out=o6, lse=l6)

    t6 = StageTimer(torch, stream, ["p"])
    for _ in range(3):
        chunk6()
    for _ in range(20):
        t6.run("p", chunk6)
    torch.cuda.synchronize()
    ms6 = t6.mean_ms("p")
    flops6 = chunk_flops([int(x) for x in p6["seq_lens"].cpu()], w6["Nq"], w6["Hq"], w6["d"])
    result_workloads["chunked_prefill_paged"] = {
        **t6.stats("p"), "TFLOP/s": round(flops6 / (ms6 * 1e-3) / 1e12, 2),
        "frac_of_peak": round(flops6 / (ms6 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops": flops6}
    del p6, o6, l6
    torch.cuda.empty_cache()
    # the backward pass of the 4k causal GQA prefill (dQ kernel, then dK/dV kernel)
    w8 = inputs.WORKLOADS["causal_gqa_backward_4k"]
    q8, k8, v8, do8 = inputs.workload_inputs("causal_gqa_backward_4k", dev)
    o8, l8 = eta.attn_prefill(q8, k8, v8, causal=True)
    dq8, dk8, dv8 = torch.empty_like(q8), torch.empty_like(k8), torch.empty_like(v8)
    ws8 = torch.empty(eta.attn_prefill_backward_workspace_bytes(w8["B"], w8["Hq"], w8["Hkv"],
                                                                w8["N"], w8["N"], w8["d"], True),
                      dtype=torch.uint8, device=dev)

    def bwd8():
        eta.attn_prefill_backward(q8, k8, v8, o8, l8, do8, causal=True, dq=dq8, dk=dk8, dv=dv8,
                                  workspace=ws8)

    t8 = StageTimer(torch, stream, ["p"])
    for _ in range(3):
        bwd8()
    for _ in range(20):
        t8.run("p", bwd8)
    torch.cuda.synchronize()
    ms8 = t8.mean_ms("p")
    flops8 = 2.5 * prefill_flops(w8["B"], w8["Hq"], w8["N"], w8["d"])
    result_workloads["causal_gqa_backward_4k"] = {
        **t8.stats("p"), "TFLOP/s": round(flops8 / (ms8 * 1e-3) / 1e12, 2),
        "frac_of_peak": round(flops8 / (ms8 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops": flops8,
        "flop_convention": "five products per visible pair (QK^T, dO V^T, P^T dO, dS K, dS^T Q),"
                           " 2.5x the forward's; the kernels recompute QK^T and dO V^T once more"}
    del q8, k8, v8, do8, o8, l8, dq8, dk8, dv8, ws8
    torch.cuda.empty_cache()
    # the paged 4-token decode over an E4M3 cache (one byte per element)
    w7 = inputs.WORKLOADS["paged_decode_q4_fp8"]
    p7 = inputs.workload_inputs("paged_decode_q4_fp8", dev)
    L7 = p7["block_table"].shape[1] * 16
    o7 = torch.empty_like(p7["q"])
    l7 = torch.empty((w7["B"], w7["Hq"], w7["Nq"]), dtype=torch.float32, device=dev)
    ws7 = torch.empty(eta.attn_decode_workspace_bytes(w7["B"], w7["Hq"], w7["Hkv"], w7["Nq"],
                                                      w7["d"], L7), dtype=torch.uint8, device=dev)
    seq7 = [int(x) for x in p7["seq_lens"].cpu()]

    def append7():
        eta.kv_append_fp8(p7["k_new"], p7["v_new"], p7["k_pool"], p7["v_pool"], p7["k_scale"],
                          p7["v_scale"], p7["cache_lens"], block_table=p7["block_table"])

    def decode7():
        eta.attn_decode_paged_fp8(p7["q"], p7["k_pool"], p7["v_pool"], p7["k_scale"],
                                  p7["v_scale"], p7["seq_lens"], block_table=p7["block_table"],
                                  causal=True, workspace=ws7, out=o7, lse=l7)

    t7 = StageTimer(torch, stream, ["a", "d"])
    for _ in range(3):
        append7()
        decode7()
    for _ in range(20):
        t7.run("a", append7)
        t7.run("d", decode7)
    torch.cuda.synchronize()
    ms7 = t7.mean_ms("d")
    bytes7 = 2 * 1 * w7["Hkv"] * w7["d"] * sum(seq7)
    result_workloads["paged_decode_q4_fp8"] = {
        **t7.stats("d"), "GB/s": round(bytes7 / (ms7 * 1e-3) / 1e9, 1),
        "frac_of_peak": round(bytes7 / (ms7 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "kv_bytes": bytes7, "kv_append_ms": round(t7.mean_ms("a"), 5),
        "speedup_vs_bf16_cache": round(ms5 / ms7, 3),
        "traffic_partial_kernel": counter_traffic("paged_decode_q4_fp8",
                                                  "decode_partial_kernel<128,true>",
                                                  ["common.h", "decode.hip"])}
    del p7, o7, l7, ws7
    torch.cuda.empty_cache()
    q1, k1, v1 = inputs.workload_inputs("single_head_f32", dev)
    t1 = StageTimer(torch, stream, ["p"])
    for _ in range(10):
        eta.attn_prefill(q1, k1, v1, causal=False)
    for _ in range(50):
        t1.run("p", lambda: eta.attn_prefill(q1, k1, v1, causal=False))
    torch.cuda.synchronize()
    st1 = t1.stats("p")
    result_workloads["single_head_f32"] = {"us": round(st1["ms"] * 1e3, 2),
                                           "us_median": round(st1["ms_median"] * 1e3, 2),
                                           "us_min": round(st1["ms_min"] * 1e3, 2),
                                           "launches": st1["launches"]}

    traffic = counter_traffic("prefill_4k", "prefill_bf16_kernel<128,true,false,8>",
                              ["common.h", "prefill_bf16.hip"])
    roofline = {"bound": "mfma", "achieved": round(tflops2, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops2 / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "traffic_unit": "bytes per launch (HBM read + write)",
                "kernel": "prefill_bf16_kernel<128, true, false, 8>",
                "per_launch": f"{flops2:.6g} FLOP (visible pairs x 4d) per launch"}

    # one roofline object per named workload (the decode ones against HBM)
    def _mfma(name, kernel, stage):
        r = result_workloads[name]
        return {"bound": "mfma", "achieved": r["TFLOP/s"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": r["frac_of_peak"], "kernel": kernel,
                "traffic": counter_traffic(stage, kernel.replace(" ", ""),
                                           ["common.h", "prefill_bf16.hip"]),
                "per_launch": f"{r['flops']:.6g} FLOP (visible pairs x 4d)"}

    def _hbm(name, stage, kernels):
        r = result_workloads[name]
        tr = [counter_traffic(stage, k.replace(" ", ""), ["common.h", "decode.hip"])
              for k in kernels]
        return {"bound": "hbm", "achieved": r["GB/s"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": r["frac_of_peak"], "kernel": " + ".join(kernels),
                "traffic": None if None in tr else sum(tr),
                "per_launch": f"{r['kv_bytes']} B of K/V (each visible row once)"}

    rooflines = {
        "causal_gqa_prefill_4k": roofline,
        "causal_gqa_prefill_32k": _mfma("causal_gqa_prefill_32k",
                                        "prefill_bf16_kernel<128, true, false, 8>", "prefill_32k"),
        "splitkv_decode_32k": _hbm("splitkv_decode_32k", "splitkv_decode_32k",
                                   ["decode_partial_kernel<128, false>",
                                    "decode_combine_kernel<128>"]),
        "paged_decode_q4": _hbm("paged_decode_q4", "paged_decode_q4",
                                ["decode_partial_kernel<128, false>",
                                 "decode_combine_kernel<128>"]),
        "single_head_f32": {"bound": "latency", "us": result_workloads["single_head_f32"]["us"],
                            "per_launch": "16.8 MFLOP (256 x 256 x 64 x 4), one head"},
    }

    if not args.no_chat_sim:
        from exact_tiled_attention_flashattention_amd import chat_sim

        print("[bench] 1000-chat block-pool simulation (host)", file=sys.stderr, flush=True)
        cfg = inputs.CHAT_SIM
        prompts, outputs = inputs.chat_lengths(**cfg)
        t_sim = time.perf_counter()
        sims = chat_sim.compare(prompts, outputs, cfg["capacity_tokens"], cfg["max_new_tokens"])
        result_workloads["paged_pool_chat_sim"] = {
            "chats": cfg["chats"], "capacity_tokens": cfg["capacity_tokens"],
            "lengths": f"prompt U[{cfg['prompt_lo']},{cfg['prompt_hi']}], "
                       f"output U[{cfg['output_lo']},{cfg['output_hi']}]",
            "host_seconds": round(time.perf_counter() - t_sim, 2),
            "schemes": {r["scheme"]: {k: (round(v, 4) if isinstance(v, float) else v)
                                      for k, v in r.items() if k != "scheme"} for r in sims}}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        del q2, k2, v2, p5, ws4, ws5
        torch.cuda.empty_cache()
        cpu = cpu_baselines(torch, inputs, dev)

    line = {
        "metric": METRIC,
        "value": round(tflops2, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal_gqa_prefill_4k", "B": 1, "Hq": 32, "Hkv": 8, "N": 4096,
                   "d": 128, "causal": True,
                   "step": [n for n, _ in stages],
                   "timing": "HIP events on the library's stream; ms = mean, with median and "
                             "min, over the timed launches"},
        "roofline": roofline,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
        "workloads": result_workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
