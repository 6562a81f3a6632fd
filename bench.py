"""Benchmark: causal GQA attention forward on one MI355X.

Prints ONE JSON line.  `value` is the throughput of the dense causal GQA
prefill at the Qwen3-8B attention shape (B=2, Hq=32, Hkv=8, Sq=Skv=4096,
D=128, bf16), counting 4*D flops per visible (query, key, query-head) triple,
with inputs resident in HBM.  The same line carries:
  roofline      the attention kernel's achieved rate against the dense bf16
                MFMA peak (its average duration from HIP events recorded by
                the library around each launch, on the launch stream);
  paged_decode  KV bytes/s of the paged decode workload (B=64, Sq=1, Hq=32,
                Hkv=8, D=128, page 64, lengths U[512, 8192]) against HBM peak,
                timed per call, rotating over three copies of the caches so
                that no call finds its data in the last-level cache;
  paged_decode_fp8  the same decode with the caches quantized into FP8
                E4M3FN pools (half the bytes), timed the same way;
  backward      the attention backward (dq, dk, dv) of the same prefill,
                TFLOP/s counting 10*D flops per visible triple;
  other_configs median call time and TFLOP/s of the key-padding MHA (B=4,
                H=16, S=2048, D=64, fp16) and of the wide-group chunked prefill
                through the paged path (B=2, Hq=24, Hkv=2, D=256, 512 queries
                after 16384 keys);
  cpu_baseline  the fp64 CPU oracle on a bounded row sample of the prefill
                workload, on this host's cores.

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
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


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


def time_prefill(mi, w, steps, warmup):
    import torch
    dev = "cuda:0"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        mi.attn_fwd_dense(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mi.profile_start()
    start.record()
    for _ in range(steps):
        mi.attn_fwd_dense(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    end.record()
    torch.cuda.synchronize()
    prof = mi.profile_stop()
    total_ms = start.elapsed_time(end)
    return total_ms / steps, prof["attn_ms"] / max(prof["attn_launches"], 1)


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

        def call(kc, vc):
            mi.attn_fwd_paged_varlen(q3, kc, vc, lens, bt, cu, w.page_size, max_seqlen_q=1,
                                     k_scale=ks, v_scale=vs, out=o, lse=lse)
    else:
        caches = [(w.k_cache.to(dev), w.v_cache.to(dev))]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)

        def call(kc, vc):
            mi.attn_fwd_paged(q, kc, vc, lens, bt, w.page_size, out=o, lse=lse)
    for _ in range(copies - 1):
        caches.append((caches[0][0].clone(), caches[0][1].clone()))
    for i in range(warmup):
        call(*caches[i % copies])
    torch.cuda.synchronize()
    # whole calls (the library's own kernel timing off), then the kernels
    call_ms = []
    for i in range(steps):
        kc, vc = caches[(warmup + i) % copies]
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        call(kc, vc)
        e.record()
        torch.cuda.synchronize()
        call_ms.append(s.elapsed_time(e))
    a_ms = m_ms = 0.0
    a_n = m_n = 0
    for i in range(steps):
        kc, vc = caches[(warmup + steps + i) % copies]
        mi.profile_start()
        call(kc, vc)
        torch.cuda.synchronize()
        prof = mi.profile_stop()
        a_ms += prof["attn_ms"]
        a_n += prof["attn_launches"]
        m_ms += prof["merge_ms"]
        m_n += prof["merge_launches"]
    del caches
    call_ms.sort()
    return {"median_call_ms": call_ms[len(call_ms) // 2], "min_call_ms": call_ms[0],
            "attn_kernel_ms": a_ms / max(a_n, 1), "merge_kernel_ms": m_ms / max(m_n, 1),
            "cache_copies": copies}


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
    for _ in range(warmup):
        mi.attn_bwd(q, k, v, o, do, lse, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        mi.attn_bwd(q, k, v, o, do, lse, scale=w.scale, causal=True)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    triples = visible_pairs(w.B, w.Hq, w.Sq, [w.Skv] * w.B, True)
    tflops = 10 * w.D * triples / (ms * 1e-3) / 1e12
    return {"workload": w.name, "value": tflops, "unit": "TFLOP/s", "ms_per_call": ms,
            "flops_per_call": 10 * w.D * triples, "counted": "10*D per visible triple",
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                         "traffic": measured_traffic("backward"),
                         "traffic_per_kernel": measured_traffic("backward", "per_kernel")}}


def time_calls(fn, steps, warmup):
    """Median and minimum of per-call HIP-event times (ms) on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms[len(ms) // 2], ms[0]


def time_other_configs(mi, steps):
    """The key-padding MHA (fp16, D=64, non-causal) and the wide-group chunked
    prefill through the paged path (D=256, G=12): TFLOP/s of whole calls at
    4*D flops per visible triple, against the dense 16-bit MFMA peak."""
    import torch

    from softmax_attention_amd import workloads
    dev = "cuda:0"
    out = {}
    w = workloads.make(4)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    mask = w.key_padding_mask.to(dev)
    triples = int(w.key_padding_mask.sum()) * w.Sq * w.Hq
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    med, mn = time_calls(lambda: mi.attn_fwd_dense(q, k, v, scale=w.scale, causal=False,
                                                   key_padding_mask=mask, out=o, lse=lse),
                         steps, 10)
    out[w.name] = {"median_call_us": med * 1e3, "min_call_us": mn * 1e3, "dtype": "f16",
                   "tflops": 4 * w.D * triples / (med * 1e-3) / 1e12, "triples": triples}
    del q, k, v, o, lse, w
    w = workloads.make(5)
    q, kc, vc = w.q.to(dev), w.k_cache.to(dev), w.v_cache.to(dev)
    lens, bt = w.real_seqlen_kv.to(dev), w.block_table.to(dev)
    triples = visible_pairs(w.B, w.Hq, w.Sq, w.kv_lengths(), True)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    med, mn = time_calls(lambda: mi.attn_fwd_paged(q, kc, vc, lens, bt, w.page_size,
                                                   scale=w.scale, out=o, lse=lse), steps, 10)
    out[w.name] = {"median_call_us": med * 1e3, "min_call_us": mn * 1e3, "dtype": "bf16",
                   "tflops": 4 * w.D * triples / (med * 1e-3) / 1e12, "triples": triples}
    for rec in out.values():
        rec["frac_of_peak"] = rec["tflops"] / PEAK_BF16_TFLOPS
    return out


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the key-padding MHA and wide-group chunked prefill timings")
    ap.add_argument("--only", choices=["prefill", "decode", "decode_fp8", "backward"], default=None,
                    help="time one workload and print its line (for profiler runs)")
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

    w = workloads.make(2)
    flops = 4.0 * w.D * visible_pairs(w.B, w.Hq, w.Sq, [w.Skv] * w.B, True)
    print(f"[bench] prefill {w.name}: {flops / 1e9:.1f} GFLOP per call", file=sys.stderr,
          flush=True)
    ms_step, ms_kernel = time_prefill(mi, w, args.steps, args.warmup)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    print(f"[bench] prefill {ms_step * 1e3:.1f} us/step, kernel {ms_kernel * 1e3:.1f} us, "
          f"{achieved:.1f} TFLOP/s", file=sys.stderr, flush=True)

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
                     "kernel_avg_us": ms_kernel * 1e3},
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
        print(f"[bench] decode {wd.name}: call {d['median_call_ms'] * 1e3:.1f} us "
              f"({call_gbs:.0f} GB/s), attention kernel {d['attn_kernel_ms'] * 1e3:.1f} us, "
              f"merge {d['merge_kernel_ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)
        line["paged_decode"] = {
            "workload": wd.name, "value": call_gbs, "unit": "GB/s", "kv_bytes": nbytes,
            "median_call_us": d["median_call_ms"] * 1e3, "min_call_us": d["min_call_ms"] * 1e3,
            "cache_copies": d["cache_copies"],
            "roofline": {"bound": "hbm", "achieved": kern_gbs, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": kern_gbs / PEAK_HBM_GBS,
                         "traffic": measured_traffic("decode"),
                         "kernel": "attn_fwd_kernel<128, true, 1, 3, false> (D, bf16, paged K/V, 3 waves, plain logits, stream-K)",
                         "kernel_avg_us": d["attn_kernel_ms"] * 1e3,
                         "merge_kernel_avg_us": d["merge_kernel_ms"] * 1e3}}
        # the same decode over FP8 E4M3FN pools (half the bytes)
        d8 = time_decode(mi, wd, max(args.steps, 10), args.warmup, fp8=True)
        nb8 = nbytes // 2
        call8 = nb8 / (d8["median_call_ms"] * 1e-3) / 1e9
        kern8 = nb8 / (d8["attn_kernel_ms"] * 1e-3) / 1e9
        print(f"[bench] decode fp8 pools: call {d8['median_call_ms'] * 1e3:.1f} us "
              f"({call8:.0f} GB/s of FP8 K/V), attention kernel "
              f"{d8['attn_kernel_ms'] * 1e3:.1f} us, merge {d8['merge_kernel_ms'] * 1e3:.1f} us",
              file=sys.stderr, flush=True)
        line["paged_decode_fp8"] = {
            "workload": wd.name + "_fp8_e4m3", "value": call8, "unit": "GB/s", "kv_bytes": nb8,
            "median_call_us": d8["median_call_ms"] * 1e3, "min_call_us": d8["min_call_ms"] * 1e3,
            "speedup_vs_16bit_call": d["median_call_ms"] / d8["median_call_ms"],
            "roofline": {"bound": "hbm", "achieved": kern8, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": kern8 / PEAK_HBM_GBS,
                         "kernel": "attn_fwd_kernel<128, true, 3, 3, false> (D, bf16, FP8 pages, 3 waves, plain logits, stream-K)",
                         "kernel_avg_us": d8["attn_kernel_ms"] * 1e3,
                         "merge_kernel_avg_us": d8["merge_kernel_ms"] * 1e3}}
        del wd

    if not args.no_backward:
        # the backward of the same prefill (dq, dk, dv from q, k, v, o, do, lse)
        w = workloads.make(2)
        bw = time_backward(mi, w, max(args.steps // 5, 5), 3)
        line["backward"] = bw
        print(f"[bench] backward {w.name}: {bw['ms_per_call'] * 1e3:.1f} us, "
              f"{bw['value']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del w

    if not args.no_other:
        line["other_configs"] = time_other_configs(mi, max(args.steps, 50))
        for name, rec in line["other_configs"].items():
            print(f"[bench] {name}: call {rec['median_call_us']:.1f} us, "
                  f"{rec['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        w = workloads.make(2)
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
