"""Benchmark: causal GQA attention forward on one MI355X.

Prints ONE JSON line.  `value` is the throughput of the dense causal GQA
prefill at the Qwen3-8B attention shape (B=2, Hq=32, Hkv=8, Sq=Skv=4096,
D=128, bf16), counting 4*D flops per visible (query, key, query-head) triple,
with inputs resident in HBM.  The same line carries:
  roofline      the attention kernel's achieved rate against the dense bf16
                MFMA peak (its average duration from HIP events recorded by
                the library around each launch, on the launch stream);
  device        compute units, the published peaks, and the busy clock the
                rocprofv3 counters give over the prefill kernel (GRBM_GUI_ACTIVE
                per XCD / kernel time, from the committed counter record,
                while the kernel sources match it);
  paged_decode  KV bytes/s of the paged decode workload (B=64, Sq=1, Hq=32,
                Hkv=8, D=128, page 64, lengths U[512, 8192]) against HBM peak,
                over whole calls (attention kernel + LSE merge) issued back to
                back with HIP events between them, rotating over three copies
                of the caches so that no call finds its data in the last-level
                cache; the attention kernel alone is reported beside it;
  paged_decode_fp8  the same decode with the caches quantized into FP8
                E4M3FN pools (half the bytes), timed the same way;
  backward      the attention backward (dq, dk, dv) of the same prefill,
                TFLOP/s counting 10*D flops per visible triple;
  other_configs median call time and TFLOP/s of the tiny causal GQA call,
                the key-padding MHA (B=4, H=16, S=2048, D=64, fp16) and the
                wide-group chunked prefill through the paged path (B=2, Hq=24,
                Hkv=2, D=256, 512 queries after 16384 keys);
  cpu_baseline  the fp64 CPU oracle on a bounded row sample of the prefill
                workload, on this host's cores, and (per_config) on bounded
                samples of the other four workloads.

Every timed leg first runs its call for at least --warmup calls AND at least
0.5 s of wall time, so the clocks have settled whatever --warmup is.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("attn fwd TFLOP/s (causal GQA prefill) + KV GB/s (paged decode), % of roofline")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA (AMD's published figure)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MIN_WARM_S = 0.5            # wall time of calls before every timed leg


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs(B, Hq, Sq, kv_lens, causal, keep_counts=None):
    """Visible (query, key, query-head) triples; kv_lens per batch entry.
    Query i sees keys j <= i + L - Sq (causal) among the first L keys."""
    total = 0
    for b in range(B):
        L = kv_lens[b]
        if keep_counts is not None:
            total += Sq * keep_counts[b]
            continue
        for i in range(Sq):
            hi = min(L, i + L - Sq + 1) if causal else L
            total += max(hi, 0)
    return total * Hq


def source_digest(path):
    """sha256 of a kernel source with comments and whitespace removed, so a
    change to comments alone keeps the recorded counters valid."""
    import hashlib
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def measured_traffic(kind, field="hbm_bytes"):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record (profiles/traffic.json), or None when a kernel source that record
    depends on changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        entry = json.load(f).get(kind)
    if not entry or not entry.get("sources"):
        return None
    for src, digest in entry["sources"].items():
        full = os.path.join(ROOT, src)
        if not os.path.exists(full) or source_digest(full) != digest:
            return None
    return entry.get(field)


def kv_bytes(kv_lens, Hkv, D, elem_bytes=2):
    return sum(kv_lens) * Hkv * D * elem_bytes * 2


# ---------------------------------------------------------------- device facts


def device_facts():
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": pr.gcnArchName, "compute_units": pr.multi_processor_count,
            "peak_bf16_tflops": PEAK_BF16_TFLOPS, "peak_hbm_gbs": PEAK_HBM_GBS,
            "peak_basis": "AMD's published MI355X figures (256 CU, 2.4 GHz; HBM3E 8 TB/s)",
            "busy_clock_ghz": measured_traffic("prefill", "busy_clock_ghz"),
            "busy_clock_basis": "GRBM_GUI_ACTIVE per XCD / the prefill kernel's average "
                                "duration, rocprofv3 counter pass of this bench "
                                "(profiles/traffic.json; null once the kernel changed)"}


# ---------------------------------------------------------------- timing helpers


def warm(fn, min_calls):
    """At least `min_calls` calls and MIN_WARM_S of wall time, then a sync."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < MIN_WARM_S:
        fn(n)
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def back_to_back(fn, steps, first=0):
    """Per-call times (ms) of `steps` calls issued back to back on the current
    stream with a HIP event between consecutive calls (no host sync inside)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn(first + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def kernel_times(mi, fn, steps, first=0):
    """Average attention-kernel and merge-kernel durations (ms) from the
    library's own events, over `steps` calls issued back to back."""
    import torch
    mi.profile_start()
    for i in range(steps):
        fn(first + i)
    torch.cuda.synchronize()
    prof = mi.profile_stop()
    return (prof["attn_ms"] / max(prof["attn_launches"], 1),
            prof["merge_ms"] / max(prof["merge_launches"], 1) if prof["merge_launches"] else 0.0)


def med(xs):
    s = sorted(xs)
    return s[len(s) // 2]


# ---------------------------------------------------------------- legs


def time_prefill(mi, w, steps, warmup):
    import torch
    dev = "cuda:0"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    call = lambda i: mi.attn_fwd_dense(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_warm = warm(call, warmup)
    mi.profile_start()
    start.record()
    for i in range(steps):
        call(i)
    end.record()
    torch.cuda.synchronize()
    prof = mi.profile_stop()
    total_ms = start.elapsed_time(end)
    return total_ms / steps, prof["attn_ms"] / max(prof["attn_launches"], 1), n_warm


def time_decode(mi, w, steps, warmup, copies=3, fp8=False):
    """Paged decode timing.  The caches (1.08 GB of visible K/V against a 256 MB
    last-level cache) rotate over `copies` identical copies, so each call reads
    data that two other calls' 2 GB of reads have evicted since it was last
    touched.  (Overwriting a scratch buffer between calls instead leaves its
    dirty lines in the cache, and the timed kernel then pays for writing them
    back: about 60 us more per call on MI355X.)  With fp8 the caches are first
    quantized into FP8 E4M3FN pools (scale = max |x| / 448) by kv_cache_write
    and read through attn_fwd_paged_varlen with one query per request."""
    import torch
    dev = "cuda:0"
    q = w.q.to(dev)
    lens, bt = w.real_seqlen_kv.to(dev), w.block_table.to(dev)
    if fp8:
        k16, v16 = w.k_cache.to(dev), w.v_cache.to(dev)
        ks = torch.tensor([float(k16.float().abs().amax()) / 448.0], device=dev)
        vs = torch.tensor([float(v16.float().abs().amax()) / 448.0], device=dev)
        k8 = torch.empty(k16.shape, dtype=torch.float8_e4m3fn, device=dev)
        v8 = torch.empty_like(k8)
        mi.kv_cache_write(k16, v16, k8, v8, torch.arange(k16.shape[0], device=dev),
                          k_scale=ks, v_scale=vs)
        del k16, v16
        caches = [(k8, v8)]
        q3 = q.reshape(w.B, w.Hq, w.D)
        cu = torch.arange(0, w.B + 1, dtype=torch.int32, device=dev)
        o = torch.empty_like(q3)
        lse = torch.empty((w.Hq, w.B), dtype=torch.float32, device=dev)

        def call(i):
            kc, vc = caches[i % copies]
            mi.attn_fwd_paged_varlen(q3, kc, vc, lens, bt, cu, w.page_size, max_seqlen_q=1,
                                     k_scale=ks, v_scale=vs, out=o, lse=lse)
    else:
        caches = [(w.k_cache.to(dev), w.v_cache.to(dev))]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)

        def call(i):
            kc, vc = caches[i % copies]
            mi.attn_fwd_paged(q, kc, vc, lens, bt, w.page_size, out=o, lse=lse)
    for _ in range(copies - 1):
        caches.append((caches[0][0].clone(), caches[0][1].clone()))
    n_warm = warm(call, warmup)
    # whole calls back to back (the library's own kernel timing off), then
    # the kernels alone from the library's events, again back to back
    call_ms = back_to_back(call, steps, first=n_warm)
    a_ms, m_ms = kernel_times(mi, call, steps, first=n_warm + steps)
    del caches
    return {"median_call_ms": med(call_ms), "min_call_ms": min(call_ms),
            "mean_call_ms": sum(call_ms) / len(call_ms), "attn_kernel_ms": a_ms,
            "merge_kernel_ms": m_ms, "cache_copies": copies, "warmup_calls": n_warm}


def time_backward(mi, w, steps, warmup):
    """Backward of the causal prefill: TFLOP/s counting 10 * D flops per
    visible (query, key, query-head) triple (five products of 2 * D:
    recomputed scores, dP, dV, dK, dQ)."""
    import torch
    dev = "cuda:0"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    g = torch.Generator(device="cpu").manual_seed(7)
    do = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
    o, lse = mi.attn_fwd_dense(q, k, v, scale=w.scale, causal=True)
    call = lambda i: mi.attn_bwd(q, k, v, o, do, lse, scale=w.scale, causal=True)
    warm(call, warmup)
    ms_list = back_to_back(call, steps)
    ms = sum(ms_list) / len(ms_list)
    triples = visible_pairs(w.B, w.Hq, w.Sq, [w.Skv] * w.B, True)
    tflops = 10 * w.D * triples / (ms * 1e-3) / 1e12
    return {"workload": w.name, "value": tflops, "unit": "TFLOP/s", "ms_per_call": ms,
            "median_call_ms": med(ms_list),
            "flops_per_call": 10 * w.D * triples, "counted": "10*D per visible triple",
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                         "traffic": measured_traffic("backward"),
                         "traffic_per_kernel": measured_traffic("backward", "per_kernel")}}


def time_other_configs(mi, steps):
    """The tiny causal GQA call, the key-padding MHA (fp16, D=64, non-causal)
    and the wide-group chunked prefill through the paged path (D=256, G=12):
    whole calls back to back, TFLOP/s at 4*D flops per visible triple against
    the dense 16-bit MFMA peak, and the attention kernel's own time."""
    import torch

    from softmax_attention_amd import workloads
    dev = "cuda:0"
    out = {}

    def record(w, call, triples, dtype):
        warm(call, 10)
        ms = back_to_back(call, steps)
        a_ms, m_ms = kernel_times(mi, call, steps)
        m = med(ms)
        tf = 4 * w.D * triples / (m * 1e-3) / 1e12
        ktf = 4 * w.D * triples / (a_ms * 1e-3) / 1e12
        out[w.name] = {"median_call_us": m * 1e3, "min_call_us": min(ms) * 1e3, "dtype": dtype,
                       "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS, "triples": triples,
                       "attn_kernel_us": a_ms * 1e3, "merge_kernel_us": m_ms * 1e3,
                       "kernel_tflops": ktf, "kernel_frac_of_peak": ktf / PEAK_BF16_TFLOPS}

    w = workloads.make(1)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    record(w, lambda i: mi.attn_fwd_dense(q, k, v, scale=w.scale, causal=True, out=o, lse=lse),
           visible_pairs(w.B, w.Hq, w.Sq, [w.Skv] * w.B, True), "bf16")

    w = workloads.make(4)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    mask = w.key_padding_mask.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    record(w, lambda i: mi.attn_fwd_dense(q, k, v, scale=w.scale, causal=False,
                                          key_padding_mask=mask, out=o, lse=lse),
           int(w.key_padding_mask.sum()) * w.Sq * w.Hq, "f16")
    del q, k, v, o, lse, w

    w = workloads.make(5)
    q, kc, vc = w.q.to(dev), w.k_cache.to(dev), w.v_cache.to(dev)
    lens, bt = w.real_seqlen_kv.to(dev), w.block_table.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    record(w, lambda i: mi.attn_fwd_paged(q, kc, vc, lens, bt, w.page_size, scale=w.scale,
                                          out=o, lse=lse),
           visible_pairs(w.B, w.Hq, w.Sq, w.kv_lengths(), True), "bf16")
    return out


# ---------------------------------------------------------------- CPU oracle


def cpu_baseline(w, target_s=12.0):
    """The fp64 oracle on a bounded sample of the prefill workload's rows."""
    import numpy as np

    import oracle
    rng = np.random.default_rng(1234)

    def sample(n):
        return [(int(rng.integers(w.B)), int(rng.integers(w.Sq)), int(rng.integers(w.Hq)))
                for _ in range(n)]

    def run(rows):
        t = time.perf_counter()
        oracle.attn_dense_rows(w.q, w.k, w.v, rows, scale=w.scale, causal=True)
        return time.perf_counter() - t

    probe = sample(256)
    t_probe = run(probe)
    n = int(min(w.B * w.Sq * w.Hq, max(256, 256 * target_s / max(t_probe, 1e-3))))
    rows = sample(n)
    dt = run(rows)
    pairs = sum(min(i + 1, w.Skv) for _, i, _ in rows)
    tflops = 4.0 * w.D * pairs / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} random (b, i, h) rows of the B=2 Hq=32 S=4096 D=128 causal prefill "
                      f"({pairs} visible pairs, {dt:.1f} s)"}


def cpu_per_config(w3=None, target_s=3.0):
    """The oracle timed on the other workloads: the tiny call whole, and
    bounded samples of the paged decode (its first requests, whole; `w3`, if
    given, is that workload already built), the key-padding MHA and the
    chunked prefill (random rows)."""
    import numpy as np
    import torch

    import oracle
    from softmax_attention_amd import workloads
    out = {}
    rng = np.random.default_rng(4321)

    w = workloads.make(1)
    t = time.perf_counter()
    oracle.attn_dense(w.q, w.k, w.v, scale=w.scale, causal=True)
    dt = time.perf_counter() - t
    pairs = visible_pairs(w.B, w.Hq, w.Sq, [w.Skv] * w.B, True)
    out[w.name] = {"seconds": dt, "sample": "whole call",
                   "tflops": 4.0 * w.D * pairs / dt / 1e12}

    w = w3 if w3 is not None else workloads.make(3)
    n = 1
    while True:
        t = time.perf_counter()
        oracle.attn_paged(w.q[:n], w.k_cache, w.v_cache, w.real_seqlen_kv[:n],
                          w.block_table[:n], w.page_size)
        dt = time.perf_counter() - t
        if dt >= target_s / 4 or n == w.B:
            break
        n = min(w.B, n * 2)
    nb = kv_bytes([int(x) for x in w.real_seqlen_kv[:n]], w.Hkv, w.D)
    out[w.name] = {"seconds": dt, "sample": f"the first {n} of {w.B} requests, whole",
                   "kv_gbs": nb / dt / 1e9}
    del w, w3

    def rows_timed(w, fn, visible_of):
        n = 64
        while True:
            rows = sorted({(int(rng.integers(w.B)), int(rng.integers(w.Sq)),
                            int(rng.integers(w.Hq))) for _ in range(n)})
            t = time.perf_counter()
            fn(rows)
            dt = time.perf_counter() - t
            if dt >= target_s / 4 or n >= w.B * w.Sq * w.Hq:
                break
            n *= 2
        pairs = sum(visible_of(b, i) for b, i, _ in rows)
        return {"seconds": dt, "sample": f"{len(rows)} random (b, i, h) rows",
                "tflops": 4.0 * w.D * pairs / dt / 1e12}

    w = workloads.make(4)
    keep = w.key_padding_mask.sum(1).tolist()
    out[w.name] = rows_timed(
        w, lambda rows: oracle.attn_dense_rows(w.q, w.k, w.v, rows, scale=w.scale, causal=False,
                                               key_padding_mask=w.key_padding_mask),
        lambda b, i: int(keep[b]))
    del w
    w = workloads.make(5)
    lens = w.kv_lengths()
    out[w.name] = rows_timed(
        w, lambda rows: oracle.attn_paged_rows(w.q, w.k_cache, w.v_cache, w.real_seqlen_kv,
                                               w.block_table, w.page_size, rows, scale=w.scale),
        lambda b, i: min(lens[b], i + lens[b] - w.Sq + 1))
    for rec in out.values():
        rec["cores"] = oracle.num_threads()
    return out


# ---------------------------------------------------------------- main


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the tiny, key-padding MHA and chunked prefill timings")
    ap.add_argument("--only", choices=["prefill", "decode", "decode_fp8", "backward", "other"],
                    default=None, help="time one workload and print its line (profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device-to-device copy 5 times and exit: the "
                         "reference kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import softmax_attention_amd as mi
    from softmax_attention_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mi.lib()

    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 5}), flush=True)
        return
    if args.only in ("decode", "decode_fp8"):
        wd = workloads.make(3)
        fp8 = args.only == "decode_fp8"
        d = time_decode(mi, wd, max(args.steps, 10), args.warmup, fp8=fp8)
        nbytes = kv_bytes(wd.kv_lengths(), wd.Hkv, wd.D) // (2 if fp8 else 1)
        print(json.dumps({"workload": wd.name + ("_fp8_e4m3" if fp8 else ""), "kv_bytes": nbytes,
                          **d}), flush=True)
        return
    if args.only == "backward":
        w = workloads.make(2)
        bw = time_backward(mi, w, args.steps, args.warmup)
        print(json.dumps(bw), flush=True)
        return
    if args.only == "other":
        print(json.dumps(time_other_configs(mi, max(args.steps, 50))), flush=True)
        return

    w = workloads.make(2)
    flops = 4.0 * w.D * visible_pairs(w.B, w.Hq, w.Sq, [w.Skv] * w.B, True)
    log(f"prefill {w.name}: {flops / 1e9:.1f} GFLOP per call")
    ms_step, ms_kernel, n_warm = time_prefill(mi, w, args.steps, args.warmup)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    log(f"prefill {ms_step * 1e3:.1f} us/step, kernel {ms_kernel * 1e3:.1f} us, "
        f"{achieved:.1f} TFLOP/s")

    dev_facts = device_facts()
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Skv": w.Skv, "D": w.D, "causal": True, "scale": w.scale,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic("prefill"),
                     "kernel": "attn_fwd_kernel<128, true, 0, 8, false> (D, bf16, dense K/V, 8 waves, plain logits)",
                     "kernel_avg_us": ms_kernel * 1e3, "warmup_calls": n_warm},
        "device": dev_facts,
    }
    del w
    if args.only == "prefill":
        print(json.dumps(line), flush=True)
        return

    if not args.no_decode:
        wd = workloads.make(3)
        nbytes = kv_bytes(wd.kv_lengths(), wd.Hkv, wd.D)
        d = time_decode(mi, wd, max(args.steps, 10), args.warmup)
        call_gbs = nbytes / (d["median_call_ms"] * 1e-3) / 1e9
        kern_gbs = nbytes / (d["attn_kernel_ms"] * 1e-3) / 1e9
        log(f"decode {wd.name}: call {d['median_call_ms'] * 1e3:.1f} us ({call_gbs:.0f} GB/s), "
            f"attention kernel {d['attn_kernel_ms'] * 1e3:.1f} us, "
            f"merge {d['merge_kernel_ms'] * 1e3:.1f} us")
        line["paged_decode"] = {
            "workload": wd.name, "value": call_gbs, "unit": "GB/s", "kv_bytes": nbytes,
            "median_call_us": d["median_call_ms"] * 1e3, "min_call_us": d["min_call_ms"] * 1e3,
            "mean_call_us": d["mean_call_ms"] * 1e3, "cache_copies": d["cache_copies"],
            "timed": "whole calls (attention + merge), back to back, events between calls",
            "roofline": {"bound": "hbm", "achieved": call_gbs, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": call_gbs / PEAK_HBM_GBS,
                         "traffic": measured_traffic("decode"),
                         "kernel": "attn_fwd_kernel<128, true, 1, 5, false> (D, bf16, paged K/V, paired decode: two KV heads per workgroup, plain logits, stream-K) + lse_merge_kernel<128, true>",
                         "attn_kernel_avg_us": d["attn_kernel_ms"] * 1e3,
                         "attn_kernel_gbs": kern_gbs,
                         "attn_kernel_frac": kern_gbs / PEAK_HBM_GBS,
                         "merge_kernel_avg_us": d["merge_kernel_ms"] * 1e3}}
        # the same decode over FP8 E4M3FN pools (half the bytes)
        d8 = time_decode(mi, wd, max(args.steps, 10), args.warmup, fp8=True)
        nb8 = nbytes // 2
        call8 = nb8 / (d8["median_call_ms"] * 1e-3) / 1e9
        kern8 = nb8 / (d8["attn_kernel_ms"] * 1e-3) / 1e9
        log(f"decode fp8 pools: call {d8['median_call_ms'] * 1e3:.1f} us ({call8:.0f} GB/s of "
            f"FP8 K/V), attention kernel {d8['attn_kernel_ms'] * 1e3:.1f} us, "
            f"merge {d8['merge_kernel_ms'] * 1e3:.1f} us")
        line["paged_decode_fp8"] = {
            "workload": wd.name + "_fp8_e4m3", "value": call8, "unit": "GB/s", "kv_bytes": nb8,
            "median_call_us": d8["median_call_ms"] * 1e3, "min_call_us": d8["min_call_ms"] * 1e3,
            "speedup_vs_16bit_call": d["median_call_ms"] / d8["median_call_ms"],
            "roofline": {"bound": "hbm", "achieved": call8, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": call8 / PEAK_HBM_GBS,
                         "traffic": measured_traffic("decode_fp8"),
                         "kernel": "attn_fwd_kernel<128, true, 3, 5, false> (D, bf16, FP8 pages, paired decode: two KV heads per workgroup, plain logits, stream-K) + lse_merge_kernel<128, true>",
                         "attn_kernel_avg_us": d8["attn_kernel_ms"] * 1e3,
                         "attn_kernel_gbs": kern8, "attn_kernel_frac": kern8 / PEAK_HBM_GBS,
                         "merge_kernel_avg_us": d8["merge_kernel_ms"] * 1e3}}

    if not args.no_backward:
        # the backward of the same prefill (dq, dk, dv from q, k, v, o, do, lse)
        w = workloads.make(2)
        bw = time_backward(mi, w, max(args.steps // 5, 5), 3)
        line["backward"] = bw
        log(f"backward {w.name}: {bw['ms_per_call'] * 1e3:.1f} us, {bw['value']:.1f} TFLOP/s")
        del w

    if not args.no_other:
        line["other_configs"] = time_other_configs(mi, max(args.steps, 50))
        for name, rec in line["other_configs"].items():
            log(f"{name}: call {rec['median_call_us']:.1f} us, {rec['tflops']:.1f} TFLOP/s, "
                f"attention kernel {rec['attn_kernel_us']:.1f} us")

    if not args.no_cpu_baseline:
        w = workloads.make(2)
        log("cpu baseline: oracle on a row sample of the prefill")
        line["cpu_baseline"] = cpu_baseline(w)
        del w
        log("cpu baseline: oracle on the other workloads")
        line["cpu_baseline"]["per_config"] = cpu_per_config(None if args.no_decode else wd)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
