"""Benchmark of one device's ring pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --workload bwd_striped_causal_8k      # the backward pass
    python bench.py --sweep                                # L sweep, every shard, merge GB/s

A "step" here is one whole ring pass of the hot path for one device: N ring steps, each a
fused attention-step kernel (QK^T, mask, online softmax, PV, merge into the running
(O, LSE)), the double-buffered KV staging copies on the side stream, and the final cast.
Inputs are seeded synthetic N(0, 1) bf16 tensors resident in HBM before timing starts.

Prints ONE JSON line.  `value` is useful attention TFLOP/s (4 h d FLOPs per allowed
(query, key) pair; causal pairs above the diagonal do not count; the backward counts
10 h d, five products, the FlashAttention convention of 2.5 x the forward).  `roofline`
reports the dominant kernel against the bf16 dense MFMA peak, from per-launch HIP events
on the compute stream; `cpu_baseline` times the fp64 oracle on a bounded sample of the
same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOADS = {
    # name: (description, sizes, layout, causal, shard, seed)
    "striped_causal_32k": ("ring_fwd striped causal, S=262144 N=8 L=32768 h=32 n_kv=8 d=128 "
                           "bf16, shard 0", dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8),
                           "striped", True, 0, 1004),
    "zigzag_causal_32k": ("ring_fwd zigzag causal, S=262144 N=8 L=32768 h=32 n_kv=8 d=128 bf16, "
                          "shard 0", dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8),
                          "zigzag", True, 0, 1004),
    "noncausal_32k": ("ring_fwd non-causal, S=262144 N=8 L=32768 h=32 n_kv=8 d=128 bf16, shard 0",
                      dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8), "contiguous", False, 0, 1003),
    "contiguous_causal_32k_shard7": ("ring_fwd contiguous causal, S=262144 N=8 L=32768 h=32 "
                                     "n_kv=8 d=128 bf16, shard 7",
                                     dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8),
                                     "contiguous", True, 7, 1003),
    "noncausal_gqa_8k": ("ring_fwd non-causal GQA, S=65536 N=8 L=8192 h=32 n_kv=8 d=128 bf16, "
                         "shard 0", dict(b=1, L=8192, h=32, n_kv=8, d=128, N=8),
                         "contiguous", False, 0, 1002),
}
BWD_WORKLOADS = {
    "bwd_striped_causal_8k": ("ring_bwd striped causal, S=65536 N=8 L=8192 h=32 n_kv=8 d=128 "
                              "bf16, shard 0", dict(b=1, L=8192, h=32, n_kv=8, d=128, N=8),
                              "striped", True, 0, 1005),
}
# the other gradient schedule (page 1, "The Backward Pass and Gradient Exchange"): keys and
# values stay, the query shards pass by; the last field is the device (its KV shard)
BWD_STATIONARY_WORKLOADS = {
    "bwd_kv_stationary_striped_causal_8k": ("ring_bwd_kv_stationary striped causal, S=65536 N=8 L=8192 "
                                            "h=32 n_kv=8 d=128 bf16, KV shard 0",
                                            dict(b=1, L=8192, h=32, n_kv=8, d=128, N=8), "striped", True, 0,
                                            1005),
}
# all-to-all sequence parallelism (page 3, sections 4.2 and 7): one device's share, the same
# sequence and heads as the ring workloads; the last field is the device (head group)
ULYSSES_WORKLOADS = {
    "ulysses_striped_causal_32k": ("ulysses_fwd striped causal, S=262144 N=8 L=32768 h=32 n_kv=8 "
                                   "d=128 bf16, head group 0 (4 query heads, 1 KV head)",
                                   dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8), "striped", True, 0, 1007),
}
ULYSSES_WORKLOADS["ulysses_bwd_striped_causal_8k"] = (
    "ulysses_bwd striped causal, S=65536 N=8 L=8192 h=32 n_kv=8 d=128 bf16, head group 0 (4 query "
    "heads, 1 KV head)", dict(b=1, L=8192, h=32, n_kv=8, d=128, N=8), "striped", True, 0, 1008)
# heads and sequence cut together (page 3, sections 7 and 8): n_head_groups x N/n_head_groups
# devices; the last two fields are the device's head group and ring rank
USP_WORKLOADS = {
    "usp2x4_striped_causal_32k": ("usp_fwd striped causal over 4 ring shards, S=262144, 8 devices of L=32768 as "
                                  "2 head groups x 4 ring shards, h=32 n_kv=8 d=128 bf16, device (head group 0, "
                                  "ring rank 0): 16 query heads, 2 KV heads, 65536 tokens",
                                  dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8), "striped", True, 2, 0, 0, 1009),
}
ULYSSES_METRIC = ("all-to-all sequence-parallel attention TFLOP/s (bf16, causal), one device's share, "
                  "and % of MI355X MFMA peak")
# packed-document workloads (page 3, section 5): the same shapes with documents of lognormal
# length packed into the window; value counts only pairs inside a document
WORKLOADS["packed_striped_causal_32k"] = (
    "ring_fwd striped causal, packed documents (lognormal lengths, mean 4096), S=262144 N=8 "
    "L=32768 h=32 n_kv=8 d=128 bf16, shard 0", dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8),
    "striped", True, 0, 1006)
PACKED_MEAN_LEN = {"packed_striped_causal_32k": 4096}
DEFAULT_WORKLOAD = "striped_causal_32k"
METRIC = "ring-step attention TFLOP/s (bf16, causal) and % of MI355X MFMA peak"
BWD_METRIC = ("ring-step attention backward TFLOP/s (bf16, causal, 2.5x forward FLOPs) and % of "
              "MI355X MFMA peak")
XGMI_LINK_GBPS = 153.0     # one xGMI link, one direction (for the modelled ring transfer)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(inp, cfg, layout, causal, shard, budget_s=20.0, docs=None):
    """Time the fp64 oracle on whole query rows (all heads, every key of the sequence)
    until about budget_s seconds of CPU work; report useful TFLOP/s of that sample."""
    from oracle import allowed_mask, shard_attention, shard_tokens
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q = inp["q"].astype(np.float64)
    k_all = inp["k_all"].astype(np.float64)
    v_all = inp["v_all"].astype(np.float64)
    N, L, h, d = cfg["N"], cfg["L"], cfg["h"], cfg["d"]
    toks = shard_tokens(layout, N, L)
    all_pos = np.sort(np.concatenate(toks))
    rng = np.random.default_rng(99)
    rows_done, pairs, elapsed = [], 0, 0.0
    chunk = 16
    while elapsed < budget_s and len(rows_done) < L:
        rows = rng.choice(L, size=chunk, replace=False)
        t0 = time.perf_counter()
        shard_attention(q, k_all, v_all, N=N, shard=shard, layout=layout, causal=causal, rows=rows,
                        docs=docs)
        elapsed += time.perf_counter() - t0
        rows_done.extend(rows.tolist())
        if docs is not None:
            pairs += int(allowed_mask(toks[shard][rows], all_pos, causal=causal, docs=docs).sum())
        elif causal:
            pairs += int(np.searchsorted(all_pos, toks[shard][rows], side="right").sum())
        else:
            pairs += chunk * N * L
    flops = 4.0 * h * d * pairs * cfg["b"]
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(rows_done)} random query rows of shard {shard} x all {h} heads against "
                      f"all {N * L} keys (fp64 numpy, {elapsed:.1f} s)"}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "step_fwd_bf16_striped_causal_32k_hbm_bytes.md")


def measured_traffic(ring_steps):
    """HBM bytes per launch of the dominant step kernel (launches running the ring steps listed
    in `ring_steps`, e.g. [4, 3]) from the committed rocprofv3 counter summary, or None when the
    kernel source changed since the counters were taken or they describe other launches."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
        fields = dict(re.findall(r"^\s+([a-z_0-9]+): (\S+)$", text, flags=re.M))
        src = os.path.join(ROOT, fields["kernel_source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != fields["kernel_source_sha256"]:
            return None
        if fields.get("ring_steps_per_launch", "1") != ",".join(str(n) for n in ring_steps):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(mib, steps):
    """Run the library's fp32 copy kernel (reads and writes mib MiB each) `steps` times."""
    import torch

    import ring_attention_long_amd as ra
    n = mib * (1 << 20) // 4
    d = 128
    rows = n // d
    src = torch.randn(1, rows, 1, d, device="cuda:0", dtype=torch.float32)
    for _ in range(steps):
        ra.finalize(src, torch.float32)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": rows * d * 4, "bytes_written": rows * d * 4,
                                           "dispatches": steps, "kernel": "copy_f32_kernel"}}))


def overlap_fraction(copy_begin, copy_end, steps):
    """Share of a staging copy that ran while some step kernel ran ([begin, end) intervals,
    pairwise disjoint since the steps share one stream).  The driver starts a copy as soon
    as the buffer it fills is free, which can be during an earlier step than the one just
    before the step it stages, so every step interval counts."""
    inside = sum(max(0.0, min(copy_end, e) - max(copy_begin, b)) for b, e in steps)
    return inside / (copy_end - copy_begin)


def exposure_band(exposed_ms, compute_ms):
    """The pages' three bands for exposed communication over compute time."""
    r = exposed_ms / compute_ms if compute_ms > 0 else 0.0
    return "< 5 %" if r < 0.05 else ("5-15 %" if r <= 0.15 else "> 15 %")


def receive_over_compute(receive_ms, compute_ms):
    """Page 3, section 11 (the three-step check, step 3): the share of communication is the
    per-step receive time over the per-step compute time, both medians of measurements, with
    no overlap subtracted; under 5 % there is ample room to overlap, 5-15 % whether overlap
    hides it depends on the implementation, above 15 % the transfer can no longer be ignored."""
    r = float(np.median(receive_ms)) / float(np.median(compute_ms))
    band = "< 5 %" if r < 0.05 else ("5-15 %" if r <= 0.15 else "> 15 %")
    return {"ratio": round(r, 4), "band": band}


def timed_passes(one_pass, steps, stream):
    """Run `steps` passes between HIP events on `stream`: mean ms per pass, and the median,
    min and max of the individual passes (an event between passes)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        one_pass()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    mean = ev[0].elapsed_time(ev[steps]) / steps
    return mean, {"median": round(float(np.median(per)), 4), "min": round(min(per), 4),
                  "max": round(max(per), 4)}


def forward_passes(ra, q, k_all, v_all, ws, o, lse, *, shard, causal, layout, docs, steps, warmup, spl=0):
    """`warmup` untimed then `steps` timed forward ring passes (ra_ring_fwd_timed: HIP events
    around every kernel launch and staging copy on the streams they run on; spl: ring steps
    per launch, 0 the library's choice).  Returns the mean ms per pass, the per-pass
    statistics and the timings of the timed passes."""
    import torch
    timings = []

    def one_pass():
        timings.append(ra.ring_fwd_timed(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout,
                                         workspace=ws, out=o, lse_out=lse, docs=docs, steps_per_launch=spl)[2])

    for i in range(warmup):
        one_pass()
        log(f"[bench] warmup {i + 1}/{warmup}")
    torch.cuda.synchronize()
    timings.clear()
    ms, pass_stats = timed_passes(one_pass, steps, torch.cuda.current_stream())
    return ms, pass_stats, timings


def launch_stats(timings, N, shard, step_flops):
    """The kernel launches of a pass, from the timed passes: a launch running ring steps
    k .. k + n - 1 is timed at step k.  Returns [(k, n, mean ms, useful FLOPs of its steps)],
    step_flops(src) giving the FLOPs of the step holding KV shard src."""
    out = []
    for k in range(N):
        n = timings[0]["launch_steps"][k]
        if n <= 0:
            continue
        ms = float(np.mean([t["step_end_ms"][k] - t["step_begin_ms"][k] for t in timings]))
        out.append((k, n, ms, sum(step_flops((shard - j) % N) for j in range(k, k + n))))
    return out


def forward_summary(ra, accounting, q, k_all, v_all, ws, o, lse, *, cfg, shard, causal, layout, steps, warmup):
    """A short record of one more forward workload on tensors already in HBM."""
    b, L, h, d, N = (cfg[x] for x in ("b", "L", "h", "d", "N"))
    ms, pass_stats, timings = forward_passes(ra, q, k_all, v_all, ws, o, lse, shard=shard, causal=causal,
                                             layout=layout, docs=None, steps=steps, warmup=warmup)
    pairs = ra.allowed_pairs(b=b, L=L, N=N, q_shard=shard, causal=causal, layout=layout)
    value = accounting.flops_from_pairs(pairs, h, d) / (ms * 1e-3) / 1e12
    launches = launch_stats(
        timings, N, shard, lambda src: accounting.flops_from_pairs(
            ra.allowed_pairs(b=b, L=L, N=N, q_shard=shard, kv_shard=src, causal=causal, layout=layout), h, d))
    peak = accounting.MI355X_BF16_DENSE_TFLOPS
    rest = [x for x in launches if x[0] > 0] or launches  # the launches after step 0
    achieved = sum(x[3] for x in rest) / (sum(x[2] for x in rest) * 1e-3) / 1e12
    log(f"[bench] {layout} causal={causal}: {ms:.3f} ms/pass, {value:.1f} TFLOP/s useful")
    return {"value": round(value, 2), "unit": "TFLOP/s", "pct_of_bf16_peak": round(100 * value / peak, 2),
            "ms_per_pass": round(ms, 4), "pass_ms": pass_stats, "steps": steps, "warmup": warmup,
            "launch_ms": [round(x[2], 4) for x in launches], "launch_steps": [x[1] for x in launches],
            "roofline_frac": round(achieved / peak, 4)}


def cpu_baseline_bwd(inp, cfg, layout, causal, shard, budget_s=20.0):
    """Time the fp64 oracle's dQ of whole query rows (all heads, every key) until about
    budget_s seconds; report TFLOP/s counting the three products a dQ row needs (S, dP,
    dQ: 6 h d FLOPs per allowed pair)."""
    from oracle import shard_dq_rows, shard_tokens
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    x = {k: inp[k].astype(np.float64) for k in ("q", "k_all", "v_all", "dout")}
    N, L, h, d = cfg["N"], cfg["L"], cfg["h"], cfg["d"]
    toks = shard_tokens(layout, N, L)
    all_pos = np.sort(np.concatenate(toks))
    rng = np.random.default_rng(98)
    rows_done, pairs, elapsed = [], 0, 0.0
    chunk = 8
    while elapsed < budget_s and len(rows_done) < L:
        rows = rng.choice(L, size=chunk, replace=False)
        t0 = time.perf_counter()
        shard_dq_rows(x["q"], x["k_all"], x["v_all"], x["dout"], rows, N=N, shard=shard,
                      layout=layout, causal=causal)
        elapsed += time.perf_counter() - t0
        rows_done.extend(rows.tolist())
        pairs += int(np.searchsorted(all_pos, toks[shard][rows], side="right").sum()) if causal \
            else chunk * N * L
    flops = 6.0 * h * d * pairs * cfg["b"]
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"dQ of {len(rows_done)} random query rows of shard {shard} x all {h} heads "
                      f"against all {N * L} keys (fp64 numpy, {elapsed:.1f} s; 6 h d FLOPs per pair)"}


def oracle_timing():
    """The fp64 oracle on the host cores, per configuration, in useful TFLOP/s (a baseline,
    not a target).  c1 runs in full (median of 5); the large ones on a fixed sample of query
    rows (all heads, every key), extrapolated by allowed pairs."""
    import platform
    import statistics

    import synth
    from oracle import allowed_mask, shard_attention, shard_dq_rows, shard_tokens
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: p.get(k) for k in ("internal_api", "num_threads", "version")}
                for p in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    model = ""
    try:
        model = next(line.split(":", 1)[1].strip() for line in open("/proc/cpuinfo")
                     if line.startswith("model name"))
    except (OSError, StopIteration):
        model = platform.processor()
    out = {"host": {"cpu_model": model, "os_cpu_count": os.cpu_count(),
                    "sched_affinity": len(os.sched_getaffinity(0)), "blas": blas}, "configs": {}}

    def rows_sample(L, n, seed):
        # the shard's first and last rows, rows on both sides of the first and last 64-row
        # tile boundaries and of the half-shard boundary (a zigzag chunk edge), then seeded
        # random rows up to n
        edges = np.array([0, L - 1, 63, 64, L - 65, L - 64, L // 2 - 1, L // 2])
        edges = np.unique(edges[(edges >= 0) & (edges < L)])
        rng = np.random.default_rng(seed)
        rest = np.setdiff1d(np.arange(L), edges)
        return np.unique(np.concatenate([edges, rng.choice(rest, size=n - edges.size, replace=False)]))

    def fwd_case(name, cfg, layout, causal, shard, seed, dtype, n_rows=None, reps=1):
        b, L, h, d, N = cfg["b"], cfg["L"], cfg["h"], cfg["d"], cfg["N"]
        inp = synth.shard_inputs(**cfg, q_shard=shard, seed=seed, dtype=dtype)
        x = {k: inp[k].astype(np.float64) for k in ("q", "k_all", "v_all")}
        toks = shard_tokens(layout, N, L)
        all_pos = np.sort(np.concatenate(toks))
        rows = None if n_rows is None else rows_sample(L, n_rows, 7)
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            shard_attention(x["q"], x["k_all"], x["v_all"], N=N, shard=shard, layout=layout,
                            causal=causal, rows=rows)
            ts.append(time.perf_counter() - t0)
        sel = toks[shard] if rows is None else toks[shard][rows]
        pairs = int(allowed_mask(sel, all_pos, causal=causal).sum()) * b
        full_pairs = int(allowed_mask(toks[shard], all_pos, causal=causal).sum()) * b
        t = statistics.median(ts)
        tf = 4.0 * h * d * pairs / t / 1e12
        out["configs"][name] = {
            "useful_tflops": tf, "seconds": round(t, 3),
            "sample": "full shard" if rows is None else f"{rows.size} rows, all heads, every key",
            "full_shard_seconds_extrapolated": round(t * full_pairs / pairs, 1)}
        log(f"[oracle] {name}: {out['configs'][name]}")

    fwd_case("c1 fp32 S=1024 N=4 d=64 non-causal", dict(b=1, L=256, h=1, n_kv=1, d=64, N=4),
             "contiguous", False, 0, 1001, "f32", None, reps=5)
    fwd_case("c2 bf16 S=65536 N=8 non-causal GQA", dict(b=1, L=8192, h=32, n_kv=8, d=128, N=8),
             "contiguous", False, 0, 1002, "bf16", 512)
    fwd_case("c3 bf16 S=262144 N=8 contiguous causal shard 7",
             dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8), "contiguous", True, 7, 1003, "bf16", 512)
    fwd_case("c4 bf16 S=262144 N=8 striped causal shard 0",
             dict(b=1, L=32768, h=32, n_kv=8, d=128, N=8), "striped", True, 0, 1004, "bf16", 512)
    # c5: the backward's dQ rows (three products per pair)
    cfg = dict(b=1, L=8192, h=32, n_kv=8, d=128, N=8)
    inp = synth.shard_inputs(**cfg, q_shard=0, seed=1005, dtype="bf16", with_dout=True)
    x = {k: inp[k].astype(np.float64) for k in ("q", "k_all", "v_all", "dout")}
    rows = rows_sample(8192, 256, 8)
    t0 = time.perf_counter()
    shard_dq_rows(x["q"], x["k_all"], x["v_all"], x["dout"], rows, N=8, shard=0,
                  layout="striped", causal=True)
    t = time.perf_counter() - t0
    toks = shard_tokens("striped", 8, 8192)
    all_pos = np.sort(np.concatenate(toks))
    pairs = int(allowed_mask(toks[0][rows], all_pos, causal=True).sum())
    full_pairs = int(allowed_mask(toks[0], all_pos, causal=True).sum())
    out["configs"]["c5 bf16 backward S=65536 striped causal shard 0 (dQ rows)"] = {
        "useful_tflops": 6.0 * 32 * 128 * pairs / t / 1e12, "seconds": round(t, 3),
        "sample": f"dQ of {rows.size} rows, all heads, every key (6 h d FLOPs per pair)",
        "full_shard_dq_seconds_extrapolated": round(t * full_pairs / pairs, 1)}
    print(json.dumps({"oracle_timing": out}), flush=True)


def run_backward(args):
    result = measure_backward(args.workload, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        import synth
        desc, cfg, layout, causal, shard, seed = BWD_WORKLOADS[args.workload]
        inp = synth.shard_inputs(**cfg, q_shard=shard, seed=seed, dtype="bf16", with_dout=True)
        result["cpu_baseline"] = cpu_baseline_bwd(inp, cfg, layout, causal, shard, args.cpu_budget)
    print(json.dumps(result), flush=True)


def measure_backward(workload, steps, warmup):
    """Time `steps` backward ring passes (after `warmup`) of a BWD_WORKLOADS entry; returns
    the bench record without the cpu_baseline."""
    import torch

    import ring_attention_long_amd as ra
    import synth
    from ring_attention_long_amd import accounting

    desc, cfg, layout, causal, shard, seed = BWD_WORKLOADS[workload]
    b, L, h, n_kv, d, N = (cfg[k] for k in ("b", "L", "h", "n_kv", "d", "N"))
    log(f"[bench] workload {workload}: {desc}")
    inp = synth.shard_inputs(**cfg, q_shard=shard, seed=seed, dtype="bf16", with_dout=True)
    dev = torch.device("cuda:0")
    g = lambda name: torch.from_numpy(inp[name]).to(dev, torch.bfloat16)  # noqa: E731
    q, k_all, v_all, dout = g("q"), g("k_all"), g("v_all"), g("dout")
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout)
    ws = torch.empty(ra.ring_bwd_workspace_bytes(q, k_all, causal=causal, layout=layout), device=dev,
                     dtype=torch.uint8)
    out = (torch.empty((b, L, h, d), device=dev, dtype=torch.float32),
           torch.empty((N, b, L, n_kv, d), device=dev, dtype=torch.float32),
           torch.empty((N, b, L, n_kv, d), device=dev, dtype=torch.float32))
    pairs = ra.allowed_pairs(b=b, L=L, N=N, q_shard=shard, causal=causal, layout=layout)
    flops = 10.0 * h * d * pairs
    compute = torch.cuda.current_stream()

    # each pass records HIP events around every step's ra_step_bwd (both kernels) on the
    # compute stream (ra_ring_bwd_timed): the roofline comes from the timed passes
    timings = []

    def one_pass():
        timings.append(ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=causal,
                                   layout=layout, workspace=ws, out=out, timed=True)[3])

    for i in range(warmup):
        one_pass()
        log(f"[bench] warmup {i + 1}/{warmup}")
    torch.cuda.synchronize()
    timings.clear()
    ms, pass_stats = timed_passes(one_pass, steps, compute)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {steps} passes: {ms:.3f} ms/pass, {value:.1f} TFLOP/s useful")

    step_ms, step_flops = [], 0
    for k in range(N):
        src = (shard - k) % N
        if timings[0]["step_begin_ms"][k] < 0:
            continue
        step_ms.append(float(np.mean([t["step_end_ms"][k] - t["step_begin_ms"][k] for t in timings])))
        step_flops += 10.0 * h * d * ra.allowed_pairs(b=b, L=L, N=N, q_shard=shard, kv_shard=src,
                                                      causal=causal, layout=layout)
    kern_ms = sum(step_ms)
    achieved = step_flops / (kern_ms * 1e-3) / 1e12
    peak = accounting.MI355X_BF16_DENSE_TFLOPS
    result = {
        "metric": BWD_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "pass_ms": pass_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) bf16 Q/K/V/dO from seeded numpy PCG64",
        "config": {"workload": desc, "S": N * L, "N": N, "L": L, "b": b, "h": h, "n_kv": n_kv,
                   "d": d, "layout": layout, "causal": causal, "q_shard": shard,
                   "useful_tflop_per_pass": round(flops / 1e12, 4),
                   "pct_of_bf16_peak": round(100 * value / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "ra_step_bwd: bwd_dq_kernel + bwd_dkdv_kernel (10 h d FLOPs per "
                               "allowed pair; the kernels execute 14 h d)",
                     "launches": len(step_ms),
                     "avg_launch_ms": round(kern_ms / max(1, len(step_ms)), 4),
                     "timed_over": f"the {len(timings)} timed passes"},
    }
    return result


def run_backward_stationary(args):
    import torch

    import ring_attention_long_amd as ra
    import synth
    from ring_attention_long_amd import accounting

    desc, cfg, layout, causal, ks, seed = BWD_STATIONARY_WORKLOADS[args.workload]
    b, L, h, n_kv, d, N = (cfg[k] for k in ("b", "L", "h", "n_kv", "d", "N"))
    log(f"[bench] workload {args.workload}: {desc}")
    dev = torch.device("cuda:0")
    host = {name: np.stack([synth.normal(shape, seed=seed, name=name, shard=j) for j in range(N)])
            for name, shape in (("q", (b, L, h, d)), ("do", (b, L, h, d)), ("k", (b, L, n_kv, d)),
                                ("v", (b, L, n_kv, d)))}
    q_all, dout_all, k_all, v_all = (torch.from_numpy(host[n]).to(dev, torch.bfloat16) for n in ("q", "do", "k", "v"))
    # what every home device holds before the backward: its shard's O, LSE and D
    lse_l, delta_l, o_l = [], [], []
    for i in range(N):
        o, lse = ra.ring_fwd(q_all[i].contiguous(), k_all, v_all, q_shard=i, causal=causal, layout=layout)
        o_l.append(o)
        lse_l.append(lse)
        delta_l.append(ra.bwd_preprocess(o, dout_all[i].contiguous()))
    lse_all, delta_all = torch.stack(lse_l), torch.stack(delta_l)
    k, v = k_all[ks].contiguous(), v_all[ks].contiguous()
    out = (torch.empty((N, b, L, h, d), device=dev, dtype=torch.float32),
           torch.empty((b, L, n_kv, d), device=dev, dtype=torch.float32),
           torch.empty((b, L, n_kv, d), device=dev, dtype=torch.float32))
    pairs = sum(ra.allowed_pairs(b=b, L=L, N=N, q_shard=i, kv_shard=ks, causal=causal, layout=layout)
                for i in range(N))
    flops = 10.0 * h * d * pairs
    compute = torch.cuda.current_stream()

    def one_pass():
        ra.ring_bwd_kv_stationary(k, v, q_all, dout_all, lse_all, delta_all, kv_shard=ks, causal=causal,
                                  layout=layout, out=out)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    ms, pass_stats = timed_passes(one_pass, args.steps, compute)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} passes: {ms:.3f} ms/pass, {value:.1f} TFLOP/s useful")
    # the key/value-rotating schedule of device ks in the same process, for comparison
    rq = q_all[ks].contiguous()
    rout = (torch.empty((b, L, h, d), device=dev, dtype=torch.float32),
            torch.empty((N, b, L, n_kv, d), device=dev, dtype=torch.float32),
            torch.empty((N, b, L, n_kv, d), device=dev, dtype=torch.float32))
    rot = lambda: ra.ring_bwd(rq, k_all, v_all, o_l[ks], dout_all[ks].contiguous(), lse_l[ks], q_shard=ks,  # noqa: E731
                              causal=causal, layout=layout, out=rout)
    rot()
    torch.cuda.synchronize()
    rot_ms, _ = timed_passes(rot, args.steps, compute)
    rot_pairs = ra.allowed_pairs(b=b, L=L, N=N, q_shard=ks, causal=causal, layout=layout)
    peak = accounting.MI355X_BF16_DENSE_TFLOPS
    bytes_rot = accounting.bwd_bytes_per_step_kv_rotating(b, L, n_kv, d, 2)
    bytes_sta = accounting.bwd_bytes_per_step_kv_stationary(b, L, h, d, 2)
    result = {
        "metric": BWD_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "pass_ms": pass_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) bf16 Q/K/V/dO from seeded numpy PCG64",
        "config": {"workload": desc, "S": N * L, "N": N, "L": L, "b": b, "h": h, "n_kv": n_kv, "d": d,
                   "layout": layout, "causal": causal, "kv_shard": ks,
                   "useful_tflop_per_pass": round(flops / 1e12, 4),
                   "pct_of_bf16_peak": round(100 * value / peak, 2)},
        "schedules": {
            "kv_rotating_pass_ms": round(rot_ms, 4),
            "kv_rotating_tflops": round(10.0 * h * d * rot_pairs / (rot_ms * 1e-3) / 1e12, 2),
            "bytes_per_step_kv_rotating": bytes_rot, "bytes_per_step_kv_stationary": bytes_sta,
            "xgmi_model_ms_per_step_kv_rotating": round(bytes_rot / (XGMI_LINK_GBPS * 1e9) * 1e3, 4),
            "xgmi_model_ms_per_step_kv_stationary": round(bytes_sta / (XGMI_LINK_GBPS * 1e9) * 1e3, 4)},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        inp = {"q": host["q"][0], "k_all": host["k"], "v_all": host["v"], "dout": host["do"][0]}
        result["cpu_baseline"] = cpu_baseline_bwd(inp, cfg, layout, causal, 0, args.cpu_budget)
    print(json.dumps(result), flush=True)


def run_ulysses(args):
    import torch

    import ring_attention_long_amd as ra
    import synth
    from ring_attention_long_amd import accounting

    desc, cfg, layout, causal, group, seed = ULYSSES_WORKLOADS[args.workload]
    b, L, h, n_kv, d, N = (cfg[k] for k in ("b", "L", "h", "n_kv", "d", "N"))
    S = N * L
    log(f"[bench] workload {args.workload}: {desc}")
    q_np = np.stack([synth.normal((b, L, h, d), seed=seed, name="q", shard=j) for j in range(N)])
    base = synth.shard_inputs(**cfg, q_shard=0, seed=seed, dtype="bf16")
    dev = torch.device("cuda:0")
    q_all = torch.from_numpy(q_np).to(dev, torch.bfloat16)
    k_all = torch.from_numpy(base["k_all"]).to(dev, torch.bfloat16)
    v_all = torch.from_numpy(base["v_all"]).to(dev, torch.bfloat16)
    o_all = torch.zeros((N, b, L, h, d), device=dev, dtype=torch.bfloat16)
    lse_all = torch.full((N, b, h, L), float("-inf"), device=dev, dtype=torch.float32)
    ws = torch.empty(ra.ulysses_workspace_bytes(q_all, k_all, causal=causal, layout=layout), device=dev,
                     dtype=torch.uint8)
    # the device's work: every allowed pair of the whole sequence, for its h/N heads
    pairs = sum(ra.allowed_pairs(b=b, L=L, N=N, q_shard=j, causal=causal, layout=layout) for j in range(N))
    flops = accounting.flops_from_pairs(pairs, h // N, d)
    compute = torch.cuda.current_stream()

    backward = "bwd" in args.workload
    if backward:
        # the forward once (O, LSE), then the timed backward of the device's share
        ra.ulysses_fwd(q_all, k_all, v_all, head_group=group, causal=causal, layout=layout, workspace=ws,
                       out=o_all, lse_out=lse_all)
        dout_all = torch.from_numpy(np.stack([synth.normal((b, L, h, d), seed=seed, name="do", shard=j)
                                              for j in range(N)])).to(dev, torch.bfloat16)
        grads = (torch.zeros((N, b, L, h, d), device=dev, dtype=torch.float32),
                 torch.zeros((N, b, L, n_kv, d), device=dev, dtype=torch.float32),
                 torch.zeros((N, b, L, n_kv, d), device=dev, dtype=torch.float32))
        flops = flops * 10 // 4                      # five products per pair instead of two

    parts = []          # forward: HIP events around the gather, attention and scatter of every pass

    def one_pass():
        if backward:
            ra.ulysses_bwd(q_all, k_all, v_all, o_all, dout_all, lse_all, head_group=group, causal=causal,
                           layout=layout, out=grads)
        else:
            parts.append(ra.ulysses_fwd_timed(q_all, k_all, v_all, head_group=group, causal=causal, layout=layout,
                                              workspace=ws, out=o_all, lse_out=lse_all)[2])

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    parts.clear()
    ms, pass_stats = timed_passes(one_pass, args.steps, compute)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} passes: {ms:.3f} ms/pass, {value:.1f} TFLOP/s useful")
    if backward:
        result = {"metric": BWD_METRIC + " (all-to-all scheme, one device's share)", "value": round(value, 2),
                  "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                  "ms_per_step": round(ms, 4), "pass_ms": pass_stats, "higher_is_better": True,
                  "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                  "data": "synthetic: iid N(0,1) bf16 Q/K/V/dO from seeded numpy PCG64",
                  "config": {"workload": desc, "S": S, "N": N, "L": L, "b": b, "h": h, "n_kv": n_kv, "d": d,
                             "layout": layout, "causal": causal, "head_group": group,
                             "useful_tflop_per_pass": round(flops / 1e12, 4),
                             "pct_of_bf16_peak": round(100 * value / accounting.MI355X_BF16_DENSE_TFLOPS, 2)}}
        print(json.dumps(result), flush=True)
        return
    tm = {k: float(np.mean([t[k] for t in parts])) for k in parts[0]}
    peak = accounting.MI355X_BF16_DENSE_TFLOPS
    achieved = flops / (tm["attend_ms"] * 1e-3) / 1e12
    es, hg, kg = 2, h // N, n_kv // N
    gather_bytes = 2 * b * S * (hg + 2 * kg) * d * es             # read and write
    scatter_bytes = b * S * hg * d * (4 + es) + 2 * b * hg * S * 4  # fp32 O in, dtype O out, LSE
    a2a = accounting.ulysses_bytes_per_device(b, S, N, h, n_kv, d, es)
    ring = accounting.ring_kv_bytes_per_pass(b, S, N, n_kv, d, es)
    result = {
        "metric": ULYSSES_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "pass_ms": pass_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) bf16 Q/K/V from seeded numpy PCG64",
        "config": {"workload": desc, "S": S, "N": N, "L": L, "b": b, "h": h, "n_kv": n_kv, "d": d,
                   "layout": layout, "causal": causal, "head_group": group,
                   "useful_tflop_per_pass": round(flops / 1e12, 4),
                   "pct_of_bf16_peak": round(100 * value / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "step_fwd_bf16_kernel<MODE_PART> over the whole sequence",
                     "launches": 1, "avg_launch_ms": round(tm["attend_ms"], 4),
                     "timed_over": f"the {len(parts)} timed passes"},
        "exchange": {"gather_ms": round(tm["gather_ms"], 4), "scatter_ms": round(tm["scatter_ms"], 4),
                     "gather_GBps": round(gather_bytes / (tm["gather_ms"] * 1e-3) / 1e9, 1),
                     "scatter_GBps": round(scatter_bytes / (tm["scatter_ms"] * 1e-3) / 1e9, 1),
                     "alltoall_bytes_per_device": int(a2a), "ring_kv_bytes_per_pass": int(ring),
                     "alltoall_xgmi_model_ms": round(a2a / (N - 1) / (XGMI_LINK_GBPS * 1e9) * 1e3, 4),
                     "ring_xgmi_model_ms_per_step": round(ring / (N - 1) / (XGMI_LINK_GBPS * 1e9) * 1e3, 4)},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        inp = {"q": q_np[0], "k_all": base["k_all"], "v_all": base["v_all"]}
        cb = cpu_baseline(inp, cfg, layout, causal, 0, args.cpu_budget)
        cb["sample"] += "; the same rows and keys a device of this scheme attends for its heads"
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


def run_usp(args):
    import torch

    import ring_attention_long_amd as ra
    import synth
    from ring_attention_long_amd import accounting

    desc, cfg, layout, causal, N_h, g, r, seed = USP_WORKLOADS[args.workload]
    b, L, h, n_kv, d, N = (cfg[k] for k in ("b", "L", "h", "n_kv", "d", "N"))
    N_s, S = N // N_h, N * L
    log(f"[bench] workload {args.workload}: {desc}")
    dev = torch.device("cuda:0")
    mk = lambda name, heads: torch.from_numpy(np.stack([synth.normal((b, L, heads, d), seed=seed, name=name, shard=j)  # noqa: E731
                                                        for j in range(N)])).to(dev, torch.bfloat16)
    q_all, k_all, v_all = mk("q", h), mk("k", n_kv), mk("v", n_kv)
    o_all = torch.zeros((N, b, L, h, d), device=dev, dtype=torch.bfloat16)
    lse_all = torch.full((N, b, h, L), float("-inf"), device=dev, dtype=torch.float32)
    ws = torch.empty(ra.usp_workspace_bytes(q_all, k_all, n_head_groups=N_h, causal=causal, layout=layout),
                     device=dev, dtype=torch.uint8)
    # the device's work: its ring shard's rows (N_h L tokens) against the sequence, h/N_h heads
    pairs = ra.allowed_pairs(b=b, L=N_h * L, N=N_s, q_shard=r, causal=causal, layout=layout)
    flops = accounting.flops_from_pairs(pairs, h // N_h, d)
    parts = []

    def one_pass():
        parts.append(ra.usp_fwd(q_all, k_all, v_all, n_head_groups=N_h, head_group=g, ring_rank=r, causal=causal,
                                layout=layout, workspace=ws, out=o_all, lse_out=lse_all, timed=True)[2])

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    parts.clear()
    tm = {}
    for i in range(args.steps):
        one_pass()
    tm = {k: float(np.median([t[k] for t in parts])) for k in parts[0]}
    ms = tm["total_ms"]               # this device's work: its exchanges and its ring (not the others' gathers)
    value = flops / (ms * 1e-3) / 1e12
    peak = accounting.MI355X_BF16_DENSE_TFLOPS
    achieved = flops / (tm["ring_ms"] * 1e-3) / 1e12
    log(f"[bench] {args.steps} calls: device share {ms:.3f} ms, {value:.1f} TFLOP/s useful")
    es = 2
    result = {
        "metric": "two-dimensional (head x sequence) attention TFLOP/s (bf16, causal), one device's share, "
                  "and % of MI355X MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "pass_ms": {"median": round(ms, 4), "min": round(min(t["total_ms"] for t in parts), 4),
                    "max": round(max(t["total_ms"] for t in parts), 4)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: iid N(0,1) bf16 Q/K/V from seeded numpy PCG64",
        "config": {"workload": desc, "S": S, "N": N, "n_head_groups": N_h, "ring_shards": N_s, "L": L, "b": b,
                   "h": h, "n_kv": n_kv, "d": d, "layout": layout, "causal": causal, "head_group": g,
                   "ring_rank": r, "useful_tflop_per_pass": round(flops / 1e12, 4),
                   "pct_of_bf16_peak": round(100 * value / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": f"the ring over {N_s} ring shards (step kernels, merges, staging waits)",
                     "launches": N_s, "avg_launch_ms": round(tm["ring_ms"] / N_s, 4),
                     "timed_over": f"the {len(parts)} timed calls (HIP events, median)"},
        "exchange": {"gather_ms": round(tm["gather_ms"], 4), "ring_ms": round(tm["ring_ms"], 4),
                     "scatter_ms": round(tm["scatter_ms"], 4),
                     "other_ring_shards_gather_ms": round(tm["others_gather_ms"], 4),
                     "usp_bytes_per_device": int(accounting.usp_bytes_per_device(b, S, N_h, N_s, h, n_kv, d, es)),
                     "ring_bytes_per_device": int(accounting.usp_bytes_per_device(b, S, 1, N, h, n_kv, d, es)),
                     "alltoall_bytes_per_device": int(accounting.usp_bytes_per_device(b, S, N, 1, h, n_kv, d, es))},
    }
    print(json.dumps(result), flush=True)


def run_hbm_kernels(args):
    """The HBM-bound pieces alone, at the S = 262144, N = 8 one-device shapes (L = 32768,
    h = 32, n_kv = 8, d = 128): the standalone LSE merge (ra_merge_lse), the finalize
    (ra_finalize, fp32 -> bf16), and a runtime device-to-device copy of one K (or V) shard for
    reference (the ring stages K and V with its own kernel, whose launches and GB/s the
    default line's `staging` block reports).  GB/s from HIP events over `steps` calls each."""
    import torch

    import ring_attention_long_amd as ra
    from ring_attention_long_amd import accounting

    b, L, h, n_kv, d = 1, 32768, 32, 8, 128
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1009)
    oa = torch.randn((b, L, h, d), device=dev, generator=gen)
    op = torch.randn((b, L, h, d), device=dev, generator=gen)
    la = torch.randn((b, h, L), device=dev, generator=gen)
    lp = torch.randn((b, h, L), device=dev, generator=gen)
    kv = torch.randn((b, L, n_kv, d), device=dev, generator=gen).to(torch.bfloat16)
    kv_dst = torch.empty_like(kv)

    def rate(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        return {"ms": round(ms, 4), "bytes": int(nbytes), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}

    res = {"merge_lse": rate(lambda: ra.merge_lse(oa, la, op, lp), accounting.merge_bytes(b, L, h, d)),
           "finalize_bf16": rate(lambda: ra.finalize(oa), 6 * b * L * h * d),
           "kv_shard_copy": rate(lambda: kv_dst.copy_(kv), 2 * kv.numel() * 2)}
    print(json.dumps({"hbm_kernels": res, "peak_GBps": accounting.MI355X_HBM_GBPS, "steps": args.steps,
                      "shapes": {"b": b, "L": L, "h": h, "n_kv": n_kv, "d": d}}), flush=True)


def run_sweep(args):
    """Where the time goes across sizes and shards (timing only: inputs are seeded
    torch.randn bf16 on the GPU; attention time does not depend on the values)."""
    import torch

    import ring_attention_long_amd as ra
    from ring_attention_long_amd import accounting

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1004)
    h, n_kv, d, N, b = 32, 8, 128, 8, 1

    def inputs(L):
        q = torch.randn((b, L, h, d), device=dev, generator=gen).to(torch.bfloat16)
        k = torch.randn((N, b, L, n_kv, d), device=dev, generator=gen).to(torch.bfloat16)
        v = torch.randn((N, b, L, n_kv, d), device=dev, generator=gen).to(torch.bfloat16)
        return q, k, v

    def timed(q, k, v, shard, layout, causal, copy_stream="auto", reps=3, spl=1):
        # spl: ring steps per launch; 1 (one launch per step) for the per-step analyses
        ws = torch.empty(ra.ring_workspace_bytes(q, k, causal=causal, layout=layout, steps_per_launch=spl),
                         device=dev, dtype=torch.uint8)
        for _ in range(2):
            ra.ring_fwd(q, k, v, q_shard=shard, causal=causal, layout=layout, workspace=ws,
                        copy_stream=copy_stream, steps_per_launch=spl)
        runs = [ra.ring_fwd_timed(q, k, v, q_shard=shard, causal=causal, layout=layout,
                                  workspace=ws, copy_stream=copy_stream, steps_per_launch=spl)[2]
                for _ in range(reps)]
        return sorted(runs, key=lambda t: t["total_ms"])[reps // 2]

    def batched(tm, L, shard, layout, causal):
        """A pass with the library's batching of ring steps into launches."""
        starts = [k for k in range(N) if tm["launch_steps"][k] > 0]
        exposed = [max(0.0, max(tm["copy_end_ms"][k:k + tm["launch_steps"][k]]) - tm["step_end_ms"][prev])
                   for prev, k in zip(starts, starts[1:])]
        pairs = ra.allowed_pairs(b=b, L=L, N=N, q_shard=shard, causal=causal, layout=layout)
        fl = accounting.flops_from_pairs(pairs, h, d)
        return {"pass_ms": round(tm["total_ms"], 4), "tflops": round(fl / tm["total_ms"] / 1e9, 1),
                "launch_ring_steps": [tm["launch_steps"][k] for k in starts],
                "launch_ms": [round(tm["step_end_ms"][k] - tm["step_begin_ms"][k], 4) for k in starts],
                "exposed_ms_max": round(max(exposed), 4) if exposed else None}

    def summarise(tm, L, shard, layout, causal):
        steps, copies, overlapped, exposed = [], [], [], []
        intervals = [(tm["step_begin_ms"][k], tm["step_end_ms"][k]) for k in range(N)
                     if tm["step_begin_ms"][k] >= 0]
        for k in range(N):
            if tm["step_begin_ms"][k] >= 0:
                steps.append(tm["step_end_ms"][k] - tm["step_begin_ms"][k])
            if k >= 1 and tm["copy_begin_ms"][k] >= 0:
                cb, ce = tm["copy_begin_ms"][k], tm["copy_end_ms"][k]
                copies.append(ce - cb)
                sb, se = tm["step_begin_ms"][k - 1], tm["step_end_ms"][k - 1]
                if sb >= 0 and ce > cb:
                    overlapped.append(overlap_fraction(cb, ce, intervals))
                    exposed.append(max(0.0, ce - se))
        pairs = ra.allowed_pairs(b=b, L=L, N=N, q_shard=shard, causal=causal, layout=layout)
        fl = accounting.flops_from_pairs(pairs, h, d)
        return {"pass_ms": round(tm["total_ms"], 4), "tflops": round(fl / tm["total_ms"] / 1e9, 1),
                "live_steps": len(steps), "step_ms_mean": round(float(np.mean(steps)), 4) if steps else 0,
                "copy_ms_mean": round(float(np.mean(copies)), 4) if copies else 0,
                "overlap_min": round(min(overlapped), 4) if overlapped else None,
                "exposed_ms_max": round(max(exposed), 4) if exposed else None}

    out = {"sweep": {"h": h, "n_kv": n_kv, "d": d, "N": N, "b": b, "data": "torch.randn bf16, seed 1004"}}
    # (1) L sweep, striped causal shard 0 and non-causal shard 0
    rows = []
    for L in (1024, 2048, 4096, 8192, 16384, 32768):
        q, k, v = inputs(L)
        kv_bytes = accounting.kv_bytes_per_step(b, L, n_kv, d, 2)
        row = {"L": L, "S": N * L, "kv_bytes_per_step": kv_bytes,
               "xgmi_ms_per_step_model": round(kv_bytes / (XGMI_LINK_GBPS * 1e9) * 1e3, 4)}
        for layout, causal, key in (("striped", True, "striped_causal"),
                                    ("contiguous", False, "noncausal")):
            row[key] = summarise(timed(q, k, v, 0, layout, causal), L, 0, layout, causal)
            row[key + "_batched"] = batched(timed(q, k, v, 0, layout, causal, spl=0), L, 0, layout, causal)
        rows.append(row)
        log(f"[sweep] L={L}: {row}")
        del q, k, v
    out["sweep"]["L_sweep"] = rows
    for key in ("striped_causal", "noncausal"):
        cross = [r["L"] for r in rows if r[key]["step_ms_mean"] >= r["xgmi_ms_per_step_model"]]
        out["sweep"][f"L_star_xgmi_model_{key}"] = min(cross) if cross else None
        hidden = [r["L"] for r in rows if r[key]["exposed_ms_max"] is not None
                  and r[key]["exposed_ms_max"] <= 0.01 * r[key]["step_ms_mean"]]
        out["sweep"][f"L_min_copy_hidden_on_gpu_{key}"] = min(hidden) if hidden else None
    # (1b) short shards: the same pass captured in a HIP graph and replayed (the cross-stream
    #      waits become graph edges), every replay checked against the eager result
    graph_rows = []
    for L in (1024, 2048, 4096):
        q, k, v = inputs(L)
        for layout, causal in (("striped", True), ("contiguous", False)):
            ws = torch.empty(ra.ring_workspace_bytes(q, k, causal=causal, layout=layout), device=dev,
                             dtype=torch.uint8)
            o = torch.empty_like(q)
            lse = torch.empty((b, h, L), device=dev)

            def one():
                ra.ring_fwd(q, k, v, q_shard=0, causal=causal, layout=layout, workspace=ws, out=o, lse_out=lse)
            one()
            torch.cuda.synchronize()
            ref = (o.clone(), lse.clone())
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                one()
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                one()
            torch.cuda.synchronize()
            same = True
            for _ in range(3):
                graph.replay()
                torch.cuda.synchronize()
                same = same and torch.equal(o, ref[0]) and torch.equal(lse, ref[1])
                one()                     # eager work between replays
                torch.cuda.synchronize()

            def med(fn, n=20):
                ts = []
                for _ in range(n):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fn()
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1))
                return float(np.median(ts))
            eager, replay = med(one), med(graph.replay)
            graph_rows.append({"L": L, "layout": layout, "causal": causal, "steps_per_launch": "library's choice",
                               "eager_ms": round(eager, 4),
                               "graph_replay_ms": round(replay, 4), "replays_equal_eager": bool(same)})
            log(f"[sweep] graph L={L} {layout}: eager {eager:.4f} ms, replay {replay:.4f} ms, equal {same}")
        del q, k, v
    out["sweep"]["graph_replay"] = graph_rows
    # (2) every shard of each causal layout at L = 32768 (load balance across devices)
    L = 32768
    q, k, v = inputs(L)
    shards = {}
    for layout in ("contiguous", "striped", "zigzag"):
        shards[layout] = [summarise(timed(q, k, v, s, layout, True, reps=1), L, s, layout, True)
                          for s in range(N)]
        log(f"[sweep] shards {layout}: {[x['pass_ms'] for x in shards[layout]]}")
    out["sweep"]["shards_L32768"] = shards
    # (3) interference: step kernels with the copy on a side stream vs copies serialised
    side = summarise(timed(q, k, v, 0, "striped", True), L, 0, "striped", True)
    serial = summarise(timed(q, k, v, 0, "striped", True, copy_stream=None), L, 0, "striped", True)
    out["sweep"]["interference_L32768_striped"] = {
        "step_ms_mean_with_concurrent_copy": side["step_ms_mean"],
        "step_ms_mean_copies_serialised": serial["step_ms_mean"],
        "slowdown": round(side["step_ms_mean"] / serial["step_ms_mean"], 4)}
    # (4) HBM-bound kernels: merge and finalize at the L = 32768 shapes, against a torch copy
    oa = torch.randn((b, L, h, d), device=dev, generator=gen)
    op = torch.randn((b, L, h, d), device=dev, generator=gen)
    la = torch.randn((b, h, L), device=dev, generator=gen)
    lp = torch.randn((b, h, L), device=dev, generator=gen)

    def gbps(fn, nbytes, reps=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)

    merge_bytes = accounting.merge_bytes(b, L, h, d)
    dst = torch.empty_like(oa)
    out["sweep"]["hbm_GBps"] = {
        "merge_lse": gbps(lambda: ra.merge_lse(oa, la, op, lp), merge_bytes),
        "finalize_bf16": gbps(lambda: ra.finalize(oa), 6 * b * L * h * d),
        "torch_copy_fp32": gbps(lambda: dst.copy_(oa), 8 * b * L * h * d),
        "spec": 8000.0, "merge_bytes_per_call": merge_bytes}
    # (5) packed documents (page 3, section 5): mean document length against the work left
    #     and the step time, with the staged KV bytes per step unchanged
    import synth
    packed = []
    for mean_len in (1024, 4096, 16384, 65536):
        bounds = synth.document_bounds(N * L, seed=1006, mean_len=mean_len)
        row = {"mean_doc_len": mean_len, "documents": int(bounds.size - 1)}
        for layout in ("striped", "contiguous"):
            begin, end = ra.document_ranges(bounds, N=N, L=L, shard=0, layout=layout)
            docs = (torch.from_numpy(begin[None]).to(dev), torch.from_numpy(end[None]).to(dev))
            pairs = ra.allowed_pairs_packed(begin[None], end[None], N=N, q_shard=0, causal=True,
                                            layout=layout)
            fl = accounting.flops_from_pairs(pairs, h, d)
            for spl, key in ((1, layout), (0, layout + "_batched")):
                ws = torch.empty(ra.ring_workspace_bytes(q, k, causal=True, layout=layout, steps_per_launch=spl),
                                 device=dev, dtype=torch.uint8)
                for _ in range(2):
                    ra.ring_fwd(q, k, v, q_shard=0, causal=True, layout=layout, workspace=ws, docs=docs,
                                steps_per_launch=spl)
                tm = sorted((ra.ring_fwd_timed(q, k, v, q_shard=0, causal=True, layout=layout, workspace=ws,
                                               docs=docs, steps_per_launch=spl)[2] for _ in range(3)),
                            key=lambda t: t["total_ms"])[1]
                launches = [tm["step_end_ms"][kk] - tm["step_begin_ms"][kk] for kk in range(N)
                            if tm["launch_steps"][kk] > 0]
                row[key] = {"useful_tflop": round(fl / 1e12, 4), "pass_ms": round(tm["total_ms"], 4),
                            "tflops": round(fl / tm["total_ms"] / 1e9, 1),
                            "launch_ms": [round(x, 4) for x in launches]}
        packed.append(row)
        log(f"[sweep] packed {row}")
    out["sweep"]["packed_L32768_shard0"] = packed
    out["sweep"]["peak_bf16_tflops"] = accounting.MI355X_BF16_DENSE_TFLOPS
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(WORKLOADS) + sorted(BWD_WORKLOADS) + sorted(BWD_STATIONARY_WORKLOADS)
                    + sorted(ULYSSES_WORKLOADS) + sorted(USP_WORKLOADS))
    ap.add_argument("--oracle-timing", action="store_true",
                    help="CPU only: time the fp64 oracle on each configuration (full or a bounded "
                         "sample, extrapolated) and describe the host")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of one workload: L sweep of the striped causal ring pass, every "
                         "shard of each causal layout at L=32768, copy interference, merge GB/s")
    ap.add_argument("--hbm-kernels", action="store_true",
                    help="instead of a workload: the LSE merge, the finalize and a K/V shard copy "
                         "alone, with their HBM GB/s")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default workload only: skip the non-causal and backward passes measured beside it")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="instead of the ring pass, run the library's plain fp32 copy kernel "
                         "(ra_finalize, fp32) over this many MiB: the known-size reference for "
                         "scaling HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration_mb:
        return copy_calibration(args.copy_calibration_mb, args.steps)
    if args.oracle_timing:
        return oracle_timing()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring; --gpus {args.gpus} is not supported "
              "(the ring's other devices are emulated on the one GPU)", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        return run_sweep(args)
    if args.hbm_kernels:
        return run_hbm_kernels(args)
    if args.workload in BWD_WORKLOADS:
        return run_backward(args)
    if args.workload in ULYSSES_WORKLOADS:
        return run_ulysses(args)
    if args.workload in BWD_STATIONARY_WORKLOADS:
        return run_backward_stationary(args)
    if args.workload in USP_WORKLOADS:
        return run_usp(args)

    import torch

    import ring_attention_long_amd as ra
    import synth
    from ring_attention_long_amd import accounting

    desc, cfg, layout, causal, shard, seed = WORKLOADS[args.workload]
    b, L, h, n_kv, d, N = (cfg[k] for k in ("b", "L", "h", "n_kv", "d", "N"))
    log(f"[bench] workload {args.workload}: {desc}")
    inp = synth.shard_inputs(**cfg, q_shard=shard, seed=seed, dtype="bf16")
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp["q"]).to(dev, torch.bfloat16)
    k_all = torch.from_numpy(inp["k_all"]).to(dev, torch.bfloat16)
    v_all = torch.from_numpy(inp["v_all"]).to(dev, torch.bfloat16)
    ws = torch.empty(ra.ring_workspace_bytes(q, k_all, causal=causal, layout=layout),
                     device=dev, dtype=torch.uint8)
    o = torch.empty_like(q)
    lse = torch.empty((b, h, L), device=dev, dtype=torch.float32)
    docs = bounds = None
    if args.workload in PACKED_MEAN_LEN:
        bounds = synth.document_bounds(N * L, seed=seed, mean_len=PACKED_MEAN_LEN[args.workload])
        begin, end = ra.document_ranges(bounds, N=N, L=L, shard=shard, layout=layout)
        docs = (torch.from_numpy(begin[None]).to(dev), torch.from_numpy(end[None]).to(dev))

    def pairs_of(kv_shard=-1):
        if docs is None:
            return ra.allowed_pairs(b=b, L=L, N=N, q_shard=shard, kv_shard=kv_shard, causal=causal,
                                    layout=layout)
        return ra.allowed_pairs_packed(begin[None], end[None], N=N, q_shard=shard,
                                       kv_shard=kv_shard, causal=causal, layout=layout)
    pairs = pairs_of()
    flops = accounting.flops_from_pairs(pairs, h, d)

    # Every pass records HIP events around each step kernel and each staging copy on the
    # streams they run on (ra_ring_fwd_timed); the roofline's launch durations come from
    # the timed passes themselves.
    ms, pass_stats, timings = forward_passes(ra, q, k_all, v_all, ws, o, lse, shard=shard, causal=causal,
                                             layout=layout, docs=docs, steps=args.steps, warmup=args.warmup)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} passes: {ms:.3f} ms/pass, {value:.1f} TFLOP/s useful")
    launches = launch_stats(timings, N, shard, lambda src: accounting.flops_from_pairs(pairs_of(src), h, d))
    tm = sorted(timings, key=lambda t: t["total_ms"])[len(timings) // 2]   # the median pass
    kern_ms = sum(x[2] for x in launches)
    peak = accounting.MI355X_BF16_DENSE_TFLOPS
    # the roofline of the dominant kernel: the launches after step 0 (one kernel, batched or
    # per step) over their mean duration, or step 0's when it takes longer in all
    rest = [x for x in launches if x[0] > 0]
    first = [x for x in launches if x[0] == 0]
    dom = rest if sum(x[2] for x in rest) >= sum(x[2] for x in first) else first
    dom_ms = sum(x[2] for x in dom)
    achieved = sum(x[3] for x in dom) / (dom_ms * 1e-3) / 1e12
    # per staged shard k: share of its copy that ran under kernels; per launch after the
    # first: the time (if any) the copies of its shards ran on past the previous launch's end
    intervals = [(tm["step_begin_ms"][k], tm["step_end_ms"][k]) for k in range(N)
                 if tm["launch_steps"][k] > 0]
    # staging launches: one per step, or one per group of batched steps (its shards report
    # the same begin and end)
    copies = {}
    for k in range(1, N):
        cb, ce = tm["copy_begin_ms"][k], tm["copy_end_ms"][k]
        if cb >= 0 and ce > cb:
            copies[(cb, ce)] = copies.get((cb, ce), 0) + 1
    copy_launches = sorted((cb, ce, n) for (cb, ce), n in copies.items())
    overlapped = [overlap_fraction(cb, ce, intervals) for cb, ce, _ in copy_launches]
    exposed = []
    starts = [k for k in range(N) if tm["launch_steps"][k] > 0]
    for prev, k in zip(starts, starts[1:]):
        last_copy = max(tm["copy_end_ms"][k:k + tm["launch_steps"][k]])
        exposed.append(max(0.0, last_copy - tm["step_end_ms"][prev]))
    kv_bytes = accounting.kv_bytes_per_step(b, L, n_kv, d, 2)
    copy_ms = [ce - cb for cb, ce, _ in copy_launches]
    receive_ms = [(ce - cb) / n for cb, ce, n in copy_launches for _ in range(n)]   # per shard
    # compute per ring step: a launch's duration spread over the steps it ran
    per_step_ms = [x[2] / x[1] for x in launches for _ in range(x[1])]
    xgmi_ms = kv_bytes / (XGMI_LINK_GBPS * 1e9) * 1e3

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "pass_ms": pass_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: iid N(0,1) bf16 Q/K/V from seeded numpy PCG64",
        "config": {"workload": desc, "S": N * L, "N": N, "L": L, "b": b, "h": h, "n_kv": n_kv,
                   "d": d, "layout": layout, "causal": causal, "q_shard": shard,
                   "documents": None if bounds is None else int(bounds.size - 1),
                   "useful_tflop_per_pass": round(flops / 1e12, 4),
                   "pct_of_bf16_peak": round(100 * value / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic([x[1] for x in dom]) if args.workload == DEFAULT_WORKLOAD else None,
                     "kernel": "step_fwd_bf16_kernel, " + ", ".join(
                         f"ring steps {x[0]}..{x[0] + x[1] - 1}" if x[1] > 1 else f"ring step {x[0]}" for x in dom),
                     "launches": len(dom),
                     "avg_launch_ms": round(dom_ms / len(dom), 4),
                     "useful_tflop_per_launch": round(sum(x[3] for x in dom) / len(dom) / 1e12, 4),
                     "all_launches": {"ms": [round(x[2], 4) for x in launches], "ring_steps": [x[1] for x in launches],
                                      "achieved": round(sum(x[3] for x in launches) / (kern_ms * 1e-3) / 1e12, 2)},
                     "timed_over": f"the {len(timings)} timed passes"},
        "staging": {"kv_bytes_per_step": kv_bytes,
                    "copy_launch_ms": [round(x, 4) for x in copy_ms],
                    "copy_launch_shards": [n for _, _, n in copy_launches],
                    "copy_GBps": [round(2 * kv_bytes * n / ((ce - cb) * 1e-3) / 1e9, 1)
                                  for cb, ce, n in copy_launches],
                    "overlap_fraction_per_copy_launch": [round(x, 4) for x in overlapped],
                    "exposed_ms_per_launch": [round(x, 4) for x in exposed],
                    "exposed_over_compute_band": exposure_band(sum(exposed), kern_ms),
                    "receive_over_compute": {
                        "definition": "page 3 section 11: median per-step receive time / median per-step "
                                      "compute time (a launch's duration over the ring steps it ran), no "
                                      "overlap subtracted",
                        "on_gpu_copy": receive_over_compute(receive_ms, per_step_ms) if receive_ms else None,
                        "xgmi_link_model": dict(receive_over_compute([xgmi_ms], per_step_ms),
                                                receive_ms=round(xgmi_ms, 4), link_GBps=XGMI_LINK_GBPS)}},
    }
    if args.workload == DEFAULT_WORKLOAD and not args.no_extras:
        # the same run also measures the non-causal pass at the same shapes (on the same
        # tensors: the step time does not depend on the values) and the backward pass
        extras = {}
        log("[bench] also: non-causal pass at the same shapes")
        extras["noncausal_32k"] = dict(
            forward_summary(ra, accounting, q, k_all, v_all, ws, o, lse, cfg=cfg, shard=shard, causal=False,
                            layout="contiguous", steps=args.steps, warmup=args.warmup),
            workload="ring_fwd non-causal, S=262144 N=8 L=32768 h=32 n_kv=8 d=128 bf16, shard 0 (same tensors)")
        del q, k_all, v_all, ws, o, lse
        torch.cuda.empty_cache()
        log("[bench] also: backward pass")
        bwd = measure_backward("bwd_striped_causal_8k", args.steps, args.warmup)
        extras["bwd_striped_causal_8k"] = {
            "workload": bwd["config"]["workload"], "metric": bwd["metric"], "value": bwd["value"],
            "unit": "TFLOP/s", "pct_of_bf16_peak": bwd["config"]["pct_of_bf16_peak"],
            "ms_per_pass": bwd["ms_per_step"], "pass_ms": bwd["pass_ms"], "steps": bwd["steps"],
            "warmup": bwd["warmup"], "roofline_frac": bwd["roofline"]["frac"],
            "step_avg_ms": bwd["roofline"]["avg_launch_ms"]}
        result["also_measured"] = extras
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(inp, cfg, layout, causal, shard, args.cpu_budget,
                                              docs=bounds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
