#!/usr/bin/env python3
"""One-GPU benchmark of split-KV decode attention on MI355X.

A step is one decode-attention call (the split and the combine of every
partial) over one synthetic batch whose inputs are already resident in HBM. The
headline workload is a 9B-like full-attention layer (16 query / 4 KV heads,
head_dim 256, f32 KV, q f32) at 131,072 positions; other context lengths,
storage types, split counts and workloads are the rungs.

Every timed call is cold: a read of a 512 MB buffer (twice the Infinity Cache)
runs before it, outside its HIP event pair. Warm figures (calls back to back)
are reported beside the headline's, labelled as such.

Output: one compact JSON line on stdout with the metric, throughput
(algorithmic HBM GB/s of the whole call through ``attn_decode``: the split
kernel, then the combine kernel), the split kernel's roofline (HIP-event time
per cold launch on the launch stream), a short table of every rung, and the
float64 CPU oracle's throughput on bounded samples. The full record of each
rung goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
MALL_FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache
# Dense MFMA peaks of MI355X by the input type the latent kernel feeds them.
MFMA_PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0}


# Named single workloads for --only (profiling runs of one kernel).
ONLY = {
    "nine-b-f32-131072": ("qwen9b_like", (131072, "f32"), {"seed": 2000 + 131072}),
    "nine-b-f16-262144": ("qwen9b_like", (262144, "f16"), {"seed": 2000 + 262144}),
    "wide-peaky-262144": ("wide_group_peaky", (262144,), {}),
    "ragged-paged": ("ragged_paged", (), {}),
    "latent-f32-131072": ("latent_decode", (131072, "f32"), {"seed": 3000 + 131072}),
    "latent-f16-131072": ("latent_decode", (131072, "f16"), {"seed": 3000 + 131072}),
    "latent-f16-131072-project": ("latent_decode", (131072, "f16"), {"seed": 3000 + 131072}),
    "dsa-latent-f16": ("dsa_latent", (2048, 131072, "f16"), {}),
    "verify4-131072": ("spec_verify", (131072, 4, "f16"), {}),
    "prefill512-8192": ("chunked_prefill", (8192, 512, "f16"), {}),
}

# HBM traffic of the headline split kernel, measured with rocprofv3 counters
# (FETCH_SIZE and WRITE_SIZE, scaled by a copy kernel of known size) and kept
# with the hash of the kernel sources it was measured on. It is reported only
# while those sources are unchanged.
TRAFFIC_SUMMARY = os.path.join(HERE, "profiles", "gqa_split_9b-like_f32_L131072_traffic.md")
KERNEL_SOURCES = [os.path.join(HERE, "split_kv_flash_amd", "csrc", f)
                  for f in ("gqa_split.hip", "sk_device.h", "sk_internal.h", "sk_merge.h")]


def _code_only(text):
    """C++ source with comments removed and whitespace runs collapsed (string
    literals kept), so that editing a comment does not change the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """SHA-256 of the split kernel's code (comments and layout ignored)."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(n_splits):
    """Bytes per launch from the committed counter summary, or None when the
    kernel sources or the split count differ from the measured ones."""
    try:
        fields = {}
        for line in open(TRAFFIC_SUMMARY):
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
        if fields.get("kernel_source_sha256") != kernel_source_hash():
            return None
        if int(fields.get("n_splits", -1)) != n_splits:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seq-len", type=int, default=131072)
    ap.add_argument("--kv", default="f32", choices=["f32", "f16"])
    ap.add_argument("--n-splits", type=int, default=0, help="0 = the library's heuristic")
    ap.add_argument("--no-rungs", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rung-steps", type=int, default=30)
    ap.add_argument("--rung-warmup", type=int, default=10)
    ap.add_argument("--only", choices=sorted(ONLY), default=None,
                    help="time one named workload (prints its dict, no JSON line); for profiling")
    ap.add_argument("--no-one-launch", action="store_true",
                    help="with --only: leave out the one-launch timing (for a shared latent a "
                         "cooperative launch, after which rocprofv3 can crash on exit)")
    return ap.parse_args()


def decode_call(case, tensors, n_splits=0):
    from split_kv_flash_amd import DecodeCall

    return DecodeCall(
        tensors["q"], tensors["k"], tensors["v"], tensors["seq_lens"], case.seq_lens,
        scale=case.scale, block_table=tensors["block_table"], page_size=case.page_size,
        v_cols=case.head_dim_v if case.kv_shared else None, n_splits=n_splits)


def algorithmic_bytes(case, plan):
    """Algorithmic bytes of (whole call, split kernel, one-launch kernel).

    Whole call: K and V rows read once (positions < L_b), q read once, out and
    lse written once (plus one block-table entry per page when paged). Split
    kernel: K, V, q read once plus the partials it writes (B*Hq*S*(Dv+2)
    floats). One-launch kernel (split and merge in one grid): K, V, q, the
    partials of the non-empty splits written and read back once, out and lse."""
    qb = case.q.nbytes
    kv = case.kv_bytes()
    out = case.batch * case.num_q_heads * (case.head_dim_v + 1) * 4
    row = (case.head_dim_v + 2) * 4
    part = case.batch * case.num_q_heads * plan.n_splits * row
    used = sum(-(-int(L) // plan.chunk) for L in case.seq_lens) * case.num_q_heads * row
    table = 0 if case.block_table is None else sum(-(-int(L) // case.page_size) for L in case.seq_lens) * 4
    return kv + qb + out + table, kv + qb + part + table, kv + qb + table + 2 * used + out


def _pair():
    import torch

    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


# Untimed warm-up runs at least this long as well as at least W calls: after
# the host has spent seconds generating a workload the GPU has been idle, and
# the first calls then run up to 25% slower while its clocks ramp; 100 ms of
# calls still left the first of two identical timed runs 4% slower.
WARMUP_MIN_MS = 500.0


def warm_up(fn, calls, min_ms=WARMUP_MIN_MS, flush=None):
    """Runs fn at least ``calls`` times and for at least ``min_ms`` of GPU time
    (each call after a flush read when ``flush`` is given, as in the timed
    calls, so that a kernel trace of the run sees only cold launches)."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while n < calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(max(1, calls)):
            if flush is not None:
                flush.sum()
            fn()
        n += max(1, calls)
        torch.cuda.synchronize()


def time_calls(fn, steps, warmup, flush=None):
    """Per-call times in ms (one HIP event pair around each call, recorded on
    torch's current stream, which is the stream the library launches on) and
    the wall-clock ms per call (None when flushing). With ``flush`` (a device
    buffer of MALL_FLUSH_BYTES) a read of the whole buffer evicts the Infinity
    Cache before every timed call, outside the event pair; reading rather than
    writing leaves no dirty lines whose write-back would compete with the
    timed call. Warm-up: ``warmup`` calls and at least WARMUP_MIN_MS."""
    import torch

    warm_up(fn, warmup, flush=flush)
    ev = [_pair() for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        if flush is not None:
            flush.sum()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return [a.elapsed_time(b) for a, b in ev], (None if flush is not None else wall)


def kernel_avg(fn, steps, evict=None):
    """Average duration in ms of one launch of ``fn`` (a single kernel): one
    event pair around ``steps`` back-to-back launches divided by ``steps`` (the
    inputs do not change, so every launch does the same work), which is the
    per-launch duration a kernel trace reports; with ``evict`` the Infinity
    Cache is evicted before every launch and each launch is timed alone."""
    import torch

    warm_up(fn, 1, min_ms=100.0, flush=evict)
    if evict is None:
        e0, e1 = _pair()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    evs = [_pair() for _ in range(steps)]
    for e0, e1 in evs:
        evict.sum()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return statistics.mean(a.elapsed_time(b) for a, b in evs)


def median(x):
    return statistics.median(x)


def pct(x, q):
    s = sorted(x)
    return s[min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))]


def measure(case, steps, warmup, n_splits=0, flush=None, one_launch=True, tensors=None):
    """Times one workload. The call is ``attn_decode`` (the split kernel, then
    the combine kernel); the one-launch variant (``attn_decode_one_launch``:
    the last workgroups merge, or for a shared latent every workgroup after a
    grid barrier) is timed beside it, and each kernel alone. With ``flush`` every timed call and launch is
    cold (the Infinity Cache evicted before it, outside the event pair)."""
    import torch
    from synthetic.torch_io import to_device

    t = to_device(case) if tensors is None else tensors
    call = decode_call(case, t, n_splits)
    total, wall = time_calls(call.decode, steps, warmup, flush)
    split = kernel_avg(call.splitk, steps, flush)
    comb = kernel_avg(call.combine, steps)  # reads the partials the split just wrote
    whole_b, split_b, fused_b = algorithmic_bytes(case, call.plan)
    us = median(total) * 1e3
    res = {
        "workload": case.name, "n_splits": call.plan.n_splits, "chunk": call.plan.chunk,
        "us_per_call": round(us, 2), "us_p10": round(pct(total, 0.1) * 1e3, 2),
        "us_p90": round(pct(total, 0.9) * 1e3, 2),
        "split_us": round(split * 1e3, 2),
        "combine_us": round(comb * 1e3, 2),
        "GBps": round(whole_b / (us * 1e-6) / 1e9, 1),
        "frac_of_peak": round(whole_b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "split_GBps": round(split_b / (split * 1e-3) / 1e9, 1),
        "split_frac_of_peak": round(split_b / (split * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "bytes_call": whole_b, "bytes_split": split_b,
        "tokens_per_s_per_layer": round(case.batch * 1e6 / us, 1),
        "mall_flushed": flush is not None,
    }
    if one_launch:
        one, _ = time_calls(call.decode_one_launch, steps, warmup, flush)
        fused = kernel_avg(call.decode_one_launch, steps, flush)
        us1 = median(one) * 1e3
        res.update({"one_launch_us_per_call": round(us1, 2),
                    "one_launch_frac_of_peak": round(whole_b / (us1 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "one_launch_kernel_us": round(fused * 1e3, 2), "bytes_one_launch_kernel": fused_b})
    if case.kv_shared:
        # Dense contractions on MFMA: scores (Hq x Dk) and output (Hq x Dv) per position.
        flops = 2.0 * case.num_q_heads * (case.head_dim_qk + case.head_dim_v) * int(case.seq_lens.sum())
        tf = flops / (split * 1e-3) / 1e12
        if case.kv_dtype == "f32":
            # f16 MFMA on two f16 parts of every operand: three part products
            # per product, against the f16 peak; beside it, the algorithmic
            # rate against the FP32-MFMA peak.
            peak = MFMA_PEAK_TFLOPS["f16"]
            res.update({"split_TFLOPs": round(tf, 2), "part_products": 3, "mfma_peak_TFLOPs": peak,
                        "mfma_frac": round(3 * tf / peak, 4), "flops_split": flops,
                        "frac_of_fp32_mfma_peak": round(tf / MFMA_PEAK_TFLOPS["f32"], 4)})
        else:
            peak = MFMA_PEAK_TFLOPS[case.kv_dtype]
            res.update({"split_TFLOPs": round(tf, 2), "mfma_peak_TFLOPs": peak,
                        "mfma_frac": round(tf / peak, 4), "flops_split": flops})
    del call
    if tensors is None:
        del t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, split, wall


def measure_project(case, steps, warmup, w_dtype="bf16", proj_dim=128, flush=None):
    """The latent call with the per-head output projection after the merge:
    the split kernel, then the combine-project kernel (merge, then W_h o per
    head). Algorithmic bytes of the combine-project kernel: the partials of
    the non-empty splits read once, the weights read once, out and lse."""
    import numpy as np
    import torch

    import synthetic
    from synthetic.torch_io import to_device

    t = to_device(case)
    call = decode_call(case, t, 0)
    w = synthetic.projection_weights(case.num_q_heads, proj_dim, case.head_dim_v, w_dtype,
                                     seed=6000 + case.num_q_heads)
    wt = (torch.from_numpy(w.view(np.int16)).view(torch.bfloat16) if w_dtype == "bf16"
          else torch.from_numpy(w)).cuda()
    y = torch.empty(case.batch, case.num_q_heads, proj_dim, device="cuda")

    def whole():
        call.splitk()
        call.combine_project(wt, y)

    total, _ = time_calls(whole, steps, warmup, flush)
    call.splitk()
    cp = kernel_avg(lambda: call.combine_project(wt, y), steps)
    row = (case.head_dim_v + 2) * 4
    used = sum(-(-int(L) // call.plan.chunk) for L in case.seq_lens) * case.num_q_heads * row
    cp_b = used + wt.numel() * wt.element_size() + y.numel() * 4 + case.batch * case.num_q_heads * 4
    us = median(total) * 1e3
    res = {"workload": f"{case.name} + per-head projection {case.head_dim_v}->{proj_dim} ({w_dtype})",
           "n_splits": call.plan.n_splits, "chunk": call.plan.chunk,
           "us_per_call": round(us, 2), "us_p10": round(pct(total, 0.1) * 1e3, 2),
           "combine_project_us": round(cp * 1e3, 2), "bytes_combine_project": cp_b,
           "combine_project_GBps": round(cp_b / (cp * 1e-3) / 1e9, 1),
           "mall_flushed": flush is not None}
    del call, t, wt, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure_query_tiles(case, steps, warmup, flush=None):
    """Several queries per sequence (attn_query_tiles: query-tile split kernel,
    then the combine). Algorithmic bytes: K and V rows read once (positions <
    L_b), q read once, out and lse written once. Algorithmic flops: 4*D per
    visible (query, head, position) triple (scores and weighted values; the
    kernel issues twice that on MFMA for its high/low 16-bit split)."""
    import torch

    import oracle
    from split_kv_flash_amd import QueryTileCall
    from synthetic.torch_io import to_device

    t = to_device(case)
    call = QueryTileCall(t["q"], t["k"], t["v"], t["seq_lens"], case.seq_lens, scale=case.scale)
    total, _ = time_calls(call, steps, warmup, flush)
    Q = call.q_len
    vis = sum(int(x) for L in case.seq_lens for x in oracle.causal_limits(int(L), Q) if x > 0)
    flops = 4.0 * case.head_dim_qk * case.num_q_heads * vis
    byts = case.kv_bytes() + case.q.nbytes + case.batch * Q * case.num_q_heads * (case.head_dim_v + 1) * 4
    us = median(total) * 1e3
    res = {"workload": case.name, "q_len": Q, "n_splits": call.plan.n_splits, "chunk": call.plan.chunk,
           "us_per_call": round(us, 2), "us_p10": round(pct(total, 0.1) * 1e3, 2),
           "GBps": round(byts / (us * 1e-6) / 1e9, 1),
           "frac_of_peak": round(byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
           "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["f16"], 4),
           "bytes_call": byts, "flops_call": flops,
           "tokens_per_s_per_layer": round(case.batch * Q * 1e6 / us, 1),
           "mall_flushed": flush is not None}
    del call, t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def bandwidth_control(nbytes=1 << 30, reps=20):
    """Achievable-bandwidth controls on the same GPU in the same run: the
    library's streaming-read probe over 2 GiB (16-byte loads, 4 workgroups of
    512 threads per compute unit: the practical read ceiling), torch's
    read-only sum over a 1 GiB f32 tensor and a 1 GiB device-to-device copy."""
    import torch

    from split_kv_flash_amd import binding

    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    big = torch.zeros(2 * nbytes // 4, dtype=torch.float32, device="cuda")
    scratch = torch.zeros(65536, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream

    def probe():
        binding.attn_decode_read_probe(big, big.numel() * 4, 4 * cus, scratch, stream)

    out = {}
    for name, fn, traffic in (("read_kernel", probe, 2 * nbytes),
                              ("read_sum", lambda: x.sum(), nbytes),
                              ("copy", lambda: y.copy_(x), 2 * nbytes)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        out[name + "_GBps"] = round(traffic / (median(ts) * 1e-3) / 1e9, 1)
    del x, y, big, scratch
    torch.cuda.empty_cache()
    return out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return None


def cpu_baseline(case, heads, reps=3):
    """Time the float64 oracle on a bounded sample (the given query heads)."""
    import oracle

    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale,
                          q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, heads=heads)
        times.append(time.perf_counter() - t0)
    groups = sorted(set(h // case.group for _, h in heads))
    kv_per_group = case.kv_bytes() / case.num_kv_heads
    byts = kv_per_group * len(groups)
    sec = median(times)
    return {
        "value": round(byts / sec / 1e9, 3), "unit": "GB/s", "cores": _blas_threads(),
        "kind": "oracle",
        "sample": f"{case.name}: query heads {[h for _, h in heads]} (KV groups {groups}), "
                  f"median of {reps} float64 two-pass oracle calls, {sec:.2f} s each; "
                  f"bytes = K+V rows of the sampled KV groups",
        "seconds_per_call": round(sec, 3),
        "cpu": _cpu_model(),
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


def cpu_oracle_sample(case, heads, bytes_call, reps=1):
    """The float64 oracle on a sample of (sequence, head) pairs of a workload,
    scaled to the whole call by the (position, head) pairs it covers: the
    oracle's cost is one score and one weighted row per (position, head).
    Returns a short record: seconds for the sample, the estimated seconds of
    the whole call, and the call's algorithmic bytes over that estimate."""
    import oracle

    v_cols = case.head_dim_v if case.kv_shared else None
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale,
                          q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, v_cols=v_cols, heads=heads)
        times.append(time.perf_counter() - t0)
    sec = median(times)
    covered = sum(int(case.seq_lens[b]) for b, _ in heads)
    whole = int(case.seq_lens.sum()) * case.num_q_heads
    est = sec * whole / covered
    return {"w": case.name, "sample_heads": len(heads), "sample_s": round(sec, 3),
            "call_s_est": round(est, 3), "GBps_est": round(bytes_call / est / 1e9, 4)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; sharding over several GPUs is "
                                   "designed but not built (run with --gpus 1)"}))
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import synthetic
    from synthetic.torch_io import to_device

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} CUs={props.multi_processor_count} "
        f"mem={props.total_memory / 2**30:.0f} GiB")

    if args.only:
        # Cold calls, as in the full run (the flush reads show up in a kernel
        # trace as a reduction kernel of their own).
        fl = torch.zeros(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        fn, pos, kw = ONLY[args.only]
        c = getattr(synthetic, fn)(*pos, **kw)
        if args.only.endswith("-project"):
            r = measure_project(c, args.steps, args.warmup, "bf16", 128, fl)
        elif "q_len" in c.meta:
            r = measure_query_tiles(c, args.steps, args.warmup, fl)
        else:
            r, _, _ = measure(c, args.steps, args.warmup, args.n_splits, fl, one_launch=not args.no_one_launch)
        log(f"{args.only}: {r}")
        # A 1 GiB device-to-device copy: the kernel of known size that counter
        # runs scale FETCH_SIZE and WRITE_SIZE by.
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        torch.empty_like(x).copy_(x)
        torch.cuda.synchronize()
        return

    flush = torch.zeros(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    # Headline, cold: A and B runs of the same workload give the A/A noise
    # floor; a warm run (calls back to back) is reported beside them.
    case = synthetic.qwen9b_like(args.seq_len, args.kv, seed=2000 + args.seq_len)
    log(f"headline workload {case.name}: K+V {case.kv_bytes() / 1e9:.3f} GB")
    head_a, kern_a, _ = measure(case, args.steps, args.warmup, args.n_splits, flush)
    log(f"run A (cold): {head_a}")
    head_b, _, _ = measure(case, args.steps, args.warmup, args.n_splits, flush, one_launch=False)
    log(f"run B (cold): {head_b}")
    aa_spread = abs(head_a["us_per_call"] - head_b["us_per_call"]) / head_a["us_per_call"]
    warm, warm_split, _ = measure(case, args.steps, args.warmup, args.n_splits, None, one_launch=False)
    log(f"warm run: {warm}")

    split_ms = kern_a
    achieved = head_a["bytes_split"] / (split_ms * 1e-3) / 1e9
    roofline = {
        "kernel": "gqa_split_kernel",
        "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(head_a["n_splits"]),
        "avg_launch_us": round(split_ms * 1e3, 2), "launches": "cold (Infinity Cache evicted before each)",
        "algorithmic_bytes_per_launch": head_a["bytes_split"],
        "warm_avg_launch_us": round(warm_split * 1e3, 2),
    }

    control = bandwidth_control()
    log(f"bandwidth control {control}")
    roofline["frac_of_read_ceiling"] = round(achieved / control["read_kernel_GBps"], 4)

    rungs = []
    oracle_samples = []
    no_cpu = args.no_cpu_baseline

    def rung(r):
        log(f"rung {json.dumps(r)}")
        rungs.append(r)

    if not args.no_rungs:
        rs, rw = args.rung_steps, args.rung_warmup
        # Tiny GQA (4 query / 1 KV head, width 64, f32) at its longest length and 8 splits.
        c = synthetic.tiny_gqa(4096, seed=1004)
        r, _, _ = measure(c, rs, rw, 8, flush)
        rung(r)
        if not no_cpu:
            oracle_samples.append(cpu_oracle_sample(c, [(0, h) for h in range(c.num_q_heads)],
                                                    r["bytes_call"]))
        del c
        for kv in ("f32", "f16"):
            for L in (4096, 20480, 61440, 151552, 262144):
                c = synthetic.qwen9b_like(L, kv, seed=2000 + L)
                r, _, _ = measure(c, rs, rw, 0, flush)
                rung(r)
                del c
        # The 27B-like peaky layer: the planned split count, then the sweep.
        c = synthetic.wide_group_peaky(262144)
        t = to_device(c)
        r, _, _ = measure(c, rs, rw, 0, flush, tensors=t)
        rung(r)
        for S in (64, 128, 256, 512):
            r, _, _ = measure(c, rs, rw, S, flush, one_launch=False, tensors=t)
            r["workload"] += f" (S={S})"
            rung(r)
        del t
        if not no_cpu:  # one KV group of six heads
            oracle_samples.append(cpu_oracle_sample(c, [(0, h) for h in range(c.group)],
                                                    r["bytes_call"]))
        del c
        c = synthetic.ragged_paged()
        r, _, _ = measure(c, rs, rw, 0, flush)
        rung(r)
        if not no_cpu:  # every head of the first sequence
            oracle_samples.append(cpu_oracle_sample(c, [(0, h) for h in range(c.num_q_heads)],
                                                    r["bytes_call"]))
        del c
        for kv in ("f32", "f16"):
            for L in (8192, 131072):
                c = synthetic.latent_decode(L, kv, seed=3000 + L)
                r, _, _ = measure(c, rs, rw, 0, flush)
                rung(r)
                if L == 131072:
                    rung(measure_project(c, rs, rw, "bf16", 128, flush))
                    if not no_cpu:  # eight of the 96 heads
                        oracle_samples.append(cpu_oracle_sample(c, [(0, h) for h in range(8)],
                                                                r["bytes_call"]))
                del c
        for kv in ("f32", "f16"):  # sparse: top-2048 rows of a 131,072-row latent cache
            c = synthetic.dsa_latent(2048, 131072, kv)
            r, _, _ = measure(c, rs, rw, 0, flush)
            rung(r)
            del c
        # several queries per sequence (query tiles)
        for mk in (lambda: synthetic.spec_verify(131072, 4, "f16"),
                   lambda: synthetic.chunked_prefill(8192, 512, "f16"),
                   lambda: synthetic.causal_block(2048, "f16")):
            c = mk()
            rung(measure_query_tiles(c, rs, rw, flush))
            del c
    del flush
    torch.cuda.empty_cache()

    cpu = None
    if not no_cpu:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(case, [(0, h) for h in range(case.num_q_heads)])
        cpu["by_config"] = oracle_samples
        log(f"cpu baseline {cpu}")

    line = {
        "metric": "decode-attention µs/call and achieved HBM GB/s (% of peak) at 128k context",
        "value": head_a["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head_a["us_per_call"] / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) q/K/V, no dataset)",
        "config": {
            "workload": f"9B-like full-attention decode layer: batch 1, 16 query / 4 KV heads, "
                        f"head_dim 256, q f32, KV {args.kv}, context {args.seq_len}",
            "global_batch": 1, "seq_len": args.seq_len, "kv_dtype": args.kv,
            "n_splits": head_a["n_splits"], "chunk": head_a["chunk"],
            "parallelism": "single GPU", "timing": "cold calls (Infinity Cache evicted before each)",
        },
        "us_per_call": head_a["us_per_call"],
        "frac_of_peak": head_a["frac_of_peak"],
        "split_us": head_a["split_us"],
        "combine_us": head_a["combine_us"],
        "tokens_per_s_per_layer": head_a["tokens_per_s_per_layer"],
        "warm": {"us_per_call": warm["us_per_call"], "frac_of_peak": warm["frac_of_peak"],
                 "split_us": warm["split_us"]},
        "one_launch": {k: head_a[k] for k in ("one_launch_us_per_call", "one_launch_frac_of_peak",
                                             "one_launch_kernel_us")},
        "aa_noise_floor": round(aa_spread, 4),
        "bandwidth_control": control,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rungs": [brief(r) for r in rungs],
        "device": props.name,
        "cu_count": props.multi_processor_count,
    }
    if cpu:
        line["cpu_baseline_ratio"] = round(head_a["GBps"] / cpu["value"], 1)
    print(json.dumps(line, separators=(",", ":")), flush=True)


def brief(r):
    """One rung as a short record for the final line (the full record went to stderr)."""
    b = {"w": r["workload"], "S": r.get("n_splits"), "us": r["us_per_call"], "p10": r.get("us_p10")}
    for src, dst in (("frac_of_peak", "frac"), ("split_us", "split_us"),
                     ("split_frac_of_peak", "split_frac"), ("combine_us", "comb_us"),
                     ("one_launch_us_per_call", "one_us"), ("mfma_frac", "mfma_frac"),
                     ("TFLOPs", "TFLOPs"), ("combine_project_us", "cp_us"),
                     ("frac_of_fp32_mfma_peak", "fp32_mfma_frac")):
        if src in r:
            b[dst] = r[src]
    b["cold"] = r.get("mall_flushed")
    return b


if __name__ == "__main__":
    main()
