#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

A step is one forward plus one full backward (dQ, dK, dV) of the prefill
workload: fp16 q, k, v ~ N(0, 1) of shape (8, 8, 2048, 64), causal, ALiBi
score_mod, dO ~ N(0, 1).  The headline value is forward+backward TFLOP/s on
the algorithmic flop count (causal pairs S(S+1)/2 per head; 4*D flop per pair
forward, 10*D backward).  The same JSON line also carries the forward alone,
the split-KV decode (fp16, (8, 8, 1, 64) against 2048 and 32768 keys, GB/s
of K + V + q + O + lse with K/V copies rotated so reads come from HBM), the
roofline of the dominant kernel, and the fp64 oracle timed on a bounded
sample on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-s SECONDS]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0    # MI355X dense fp16/bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def time_calls(fn, reps: int, torch) -> float:
    """Average milliseconds per call of fn() from HIP events on the current
    stream (the stream the library launches on)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_f16_causal_alibi.json")
KERNEL_SOURCES = {"fwd16_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_fwd16.hip",
                  "dq16_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_bwd16.hip",
                  "dkdv16_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_bwd16.hip"}
COPY_BYTES = 256 * 1024 * 1024    # the calibration copy of --counters


def counters_pass() -> int:
    """What the rocprofv3 --pmc runs profile: a device copy of COPY_BYTES (the
    counters' calibration), then two forward + backward steps of the prefill
    workload."""
    import torch

    import tiled_online_softmax_flashattention_amd as fa
    import workloads as W

    x = torch.ones(COPY_BYTES // 4, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    w = W.PREFILL_F16
    d = w.make()
    q, k, v, do = (d[t].cuda() for t in ("q", "k", "v", "dout"))
    kw = dict(causal=True, score_mod="alibi", scale=w.scale)
    out, lse = fa.forward(q, k, v, **kw)
    for _ in range(2):
        fa.forward(q, k, v, out=out, lse=lse, **kw)
        fa.backward(q, k, v, out, lse, do, **kw)
    torch.cuda.synchronize()
    print("counters pass done", flush=True)
    return 0


def traffic_summary(fetch_csv: str, write_csv: str, command: str) -> int:
    """Writes TRAFFIC_FILE from the counter_collection CSVs of the two
    rocprofv3 passes over --counters: per-dispatch FETCH_SIZE / WRITE_SIZE
    (KiB, summed over the device) of each kernel, scaled by what the same
    counters read for the calibration copy, with the source hash of each
    kernel."""
    import csv
    import hashlib
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        by_dispatch = defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = r["Dispatch_Id"]
            by_dispatch[key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
        for key, v in by_dispatch.items():
            vals[names[key]].append(v)
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def find(vals, frag):
        got = [v for n, v in vals.items() if frag in n]
        return sorted(x for lst in got for x in lst)

    copy_kib = COPY_BYTES / 1024
    cf = find(fetch, "copyBuffer") or find(fetch, "elementwise") or find(fetch, "copy")
    cw = find(write, "copyBuffer") or find(write, "elementwise") or find(write, "copy")
    fetch_factor = copy_kib / max(cf)
    write_factor = copy_kib / max(cw)
    out = {"command": command, "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": max(cf), "write_kib": max(cw),
                                                    "fetch_factor": round(fetch_factor, 4),
                                                    "write_factor": round(write_factor, 4)},
           "kernels": {}}
    for kern, src in KERNEL_SOURCES.items():
        f, wv = find(fetch, kern), find(write, kern)
        if not f or not wv:
            continue
        fk, wk = f[len(f) // 2], wv[len(wv) // 2]
        sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
        out["kernels"][kern] = {"fetch_kib": fk, "write_kib": wk,
                                "hbm_bytes": int(round((fk * fetch_factor + wk * write_factor) * 1024)),
                                "source": src, "source_sha256": sha}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel's source has changed since then."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))["kernels"][kernel]
        sha = hashlib.sha256(open(os.path.join(ROOT, rec["source"]), "rb").read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    return rec["hbm_bytes"] if sha == rec["source_sha256"] else None


def extra_workloads(fa, W, torch, reps: int) -> dict:
    """Forward and forward+backward times of the key-padding (bf16) and the
    long-context (fp32, head_dim 512) workloads, and a short query block
    against a long KV cache (split over keys vs. the plain forward)."""
    res = {}
    for w, kw, peak in ((W.KEYPAD_BF16, dict(score_mod="checkerboard"), PEAK_F16_TFLOPS),
                        (W.LONG_F32, dict(causal=True), PEAK_F32_TFLOPS)):
        log(f"[bench] extra: {w.name}")
        x = w.make()
        dev = {k2: (None if t is None else t.cuda()) for k2, t in x.items()}
        kw = dict(kw, key_mask=dev["key_mask"], scale=w.scale)
        q, k, v, do = dev["q"], dev["k"], dev["v"], dev["dout"]
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = torch.empty(fa.backward_workspace_bytes(fa.problem(q, k, **kw)), dtype=torch.uint8, device=q.device)
        run_fwd = fa.plan_forward(q, k, v, out, lse, **kw)
        run_bwd = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, **kw)
        run_fwd(); run_bwd()
        n = reps if w.head_dim < 512 else 2
        ms_f = time_calls(lambda i: run_fwd(), n, torch)
        ms_fb = time_calls(lambda i: (run_fwd(), run_bwd()), n, torch)
        res[w.name] = {"forward_ms": round(ms_f, 3), "fwd_bwd_ms": round(ms_fb, 3),
                       "forward_TFLOP/s": round(w.fwd_flops() / ms_f / 1e9, 1),
                       "fwd_bwd_TFLOP/s": round((w.fwd_flops() + w.bwd_flops()) / ms_fb / 1e9, 1),
                       "peak_TFLOP/s": peak, "flop_convention": "causal pairs" if w.causal else "all pairs"}
        del dev, q, k, v, do, out, grads, ws
        torch.cuda.empty_cache()

    # A block of 16 new queries after a 32752-key cache (fp16, causal, ALiBi):
    # the key-split path of fa_decode against the plain forward; K/V copies
    # are rotated so reads come from HBM.
    B, H, Sq, Skv, D = 8, 8, 16, 32768, 64
    log(f"[bench] extra: short query block {B}x{H}x{Sq} against {Skv} keys")
    gen = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn(B, H, Sq, D, device="cuda", dtype=torch.float16, generator=gen)
    kvs = [(torch.randn(B, H, Skv, D, device="cuda", dtype=torch.float16, generator=gen),
            torch.randn(B, H, Skv, D, device="cuda", dtype=torch.float16, generator=gen)) for _ in range(2)]
    kw = dict(causal=True, score_mod="alibi", q_offset=Skv - Sq)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.decode_workspace_bytes(fa.problem(q, kvs[0][0], **kw)), dtype=torch.uint8, device="cuda")
    split = [fa.plan_decode(q, k, v, out, lse, ws, **kw) for k, v in kvs]
    plain = [fa.plan_forward(q, k, v, out, lse, **kw) for k, v in kvs]
    for f in split + plain:
        f()
    ms_s = time_calls(lambda i: split[i % 2](), max(reps, 4), torch)
    ms_p = time_calls(lambda i: plain[i % 2](), max(reps, 4), torch)
    nbytes = 2 * B * H * Skv * D * 2 + 2 * B * H * Sq * D * 2 + B * H * Sq * 4
    res[f"short query block f16 causal ALiBi ({B},{H},{Sq},{D}) after {Skv - Sq} cached keys"] = {
        "split_us": round(ms_s * 1e3, 2), "split_GB/s": round(nbytes / (ms_s * 1e-3) / 1e9, 1),
        "split_frac_hbm_peak": round(nbytes / (ms_s * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "forward_unsplit_us": round(ms_p * 1e3, 2), "bytes": nbytes}
    del q, kvs, out, lse, ws, split, plain
    torch.cuda.empty_cache()

    # Block sparsity: fp16 (8, 8, 8192, 64), causal, ALiBi, with a block mask
    # of a sliding window of 8 blocks (1024 keys).  Flops count only the pairs
    # the mask and the causal rule allow.
    import numpy as np
    B, H, S, D, win = 8, 8, 8192, 64, 8
    w = W.Workload("block-sparse prefill", 8, B, H, S, S, D, "f16", causal=True, mod=W.MOD_ALIBI)
    log(f"[bench] extra: block-sparse {B}x{H}x{S}x{D}, causal ALiBi, window of {win} blocks")
    x = w.make()
    q, k, v, do = (x[t].cuda() for t in ("q", "k", "v", "dout"))
    bm = W.window_block_mask(B, H, S, S, win).cuda()
    rows = np.arange(S)
    bmh = bm[0, 0].cpu().numpy() != 0
    pairs = B * H * int(sum(((np.arange(S)[None, :] <= rows[r0:r0 + 128, None])
                             & bmh[r0 // 128][np.arange(S) // 128][None, :]).sum() for r0 in range(0, S, 128)))
    kw = dict(causal=True, score_mod="alibi", block_mask=bm)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(fa.backward_workspace_bytes(fa.problem(q, k, **kw)), dtype=torch.uint8, device="cuda")
    run_fwd = fa.plan_forward(q, k, v, out, lse, **kw)
    run_bwd = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, **kw)
    dense_fwd = fa.plan_forward(q, k, v, out, lse, causal=True, score_mod="alibi")
    run_fwd(); run_bwd(); dense_fwd()
    ms_f = time_calls(lambda i: run_fwd(), reps, torch)
    ms_fb = time_calls(lambda i: (run_fwd(), run_bwd()), reps, torch)
    ms_dense = time_calls(lambda i: dense_fwd(), reps, torch)
    res[f"block-sparse f16 causal ALiBi ({B},{H},{S},{D}), sliding window of {win} blocks"] = {
        "forward_ms": round(ms_f, 4), "fwd_bwd_ms": round(ms_fb, 4), "allowed_pairs": pairs,
        "forward_TFLOP/s": round(4.0 * D * pairs / ms_f / 1e9, 1),
        "fwd_bwd_TFLOP/s": round(14.0 * D * pairs / ms_fb / 1e9, 1),
        "dense_causal_forward_ms": round(ms_dense, 4), "peak_TFLOP/s": PEAK_F16_TFLOPS,
        "flop_convention": "pairs allowed by the block mask and the causal rule"}
    del q, k, v, do, out, lse, grads, ws, bm
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, heads: int) -> dict:
    """The fp64 oracle (as it is) on a bounded sample: the first `heads`
    (batch, head) slices of the workload, forward + backward."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl is optional
        threads = 1
    x = w.make()
    B = max(1, heads // w.heads)
    hs = min(heads, w.heads)
    sl = lambda t: t[:B, :hs].contiguous()
    kw = dict(scale=w.scale, causal=w.causal, mod=w.mod)
    # ALiBi slopes depend on the head count: pass the workload's slopes for the kept heads
    slopes = oracle.default_alibi_slopes(w.heads)[:hs] if w.mod == W.MOD_ALIBI else None
    t0 = time.perf_counter()
    oracle.forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), alibi_slopes=slopes, **kw)
    oracle.backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["dout"]), alibi_slopes=slopes, **kw)
    dt = time.perf_counter() - t0
    frac = (B * hs) / (w.batch * w.heads)
    flops = (w.fwd_flops() + w.bwd_flops()) * frac
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle forward+backward on {B * hs} of {w.batch * w.heads} (batch, head) slices "
                      f"of the prefill workload, full sequence; {dt:.1f} s wall",
            "seconds": dt, "host_cpus": len(os.sched_getaffinity(0))}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup, so the GPU clock has left its ramp")
    ap.add_argument("--reps", type=int, default=20, help="calls per per-kernel timing loop")
    ap.add_argument("--cpu-heads", type=int, default=64, help="(batch, head) slices in the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true", help="also time the key-padding and long-context workloads")
    ap.add_argument("--counters", action="store_true",
                    help="only run the calibration copy and two untimed steps (for rocprofv3 --pmc)")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write the HBM traffic summary from two rocprofv3 counter CSVs of --counters")
    args = ap.parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    if args.counters:
        return counters_pass()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (heads and batches shard with no "
              "communication; see the multi-GPU design notes); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import tiled_online_softmax_flashattention_amd as fa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    w = W.PREFILL_F16
    log(f"[bench] inputs for {w.name}")
    x = w.make()
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    kw = dict(causal=w.causal, score_mod="alibi", scale=w.scale)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(fa.backward_workspace_bytes(fa.problem(q, k, **kw)), dtype=torch.uint8, device=dev)

    run_fwd = fa.plan_forward(q, k, v, out, lse, **kw)
    run_bwd = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, **kw)
    run_q = fa.plan_backward(q, k, v, out, lse, do, grads[0], None, None, ws, **kw)

    def step(_i=0):
        run_fwd()
        run_bwd()

    # The GPU clock ramps up over the first few tens of milliseconds of load
    # (the first 100 steps run about a third slower than the rest), so steps
    # are run untimed for settle_s seconds before the W warmup steps.
    log(f"[bench] settle {args.settle_s} s, warmup {args.warmup}")
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(50):
            step()
        settle_steps += 50
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    fb_flops = w.fwd_flops() + w.bwd_flops()
    tflops = fb_flops / (ms_step * 1e-3) / 1e12

    log("[bench] per-pass timing")
    ms_fwd = time_calls(lambda i: run_fwd(), args.reps, torch)
    ms_q = time_calls(lambda i: run_q(), args.reps, torch)
    ms_bwd = time_calls(lambda i: run_bwd(), args.reps, torch)
    # A full 16-bit backward launches the query kernel (which also writes the
    # row statistics) and then the key/value kernel on one stream, so the
    # key/value kernel's time is the difference of the two timings.
    ms_kv = ms_bwd - ms_q
    pairs = w.pairs()
    D = w.head_dim
    # algorithmic flop per launch of each kernel
    kernels = {
        "fwd16_kernel": (4.0 * D * pairs, ms_fwd),
        "dkdv16_kernel": (8.0 * D * pairs, ms_kv),
        "dq16_kernel": (2.0 * D * pairs, ms_q),
    }
    dom = max(kernels, key=lambda n: kernels[n][1])
    dom_flops, dom_ms = kernels[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": measured_traffic(dom),
                "avg_ms": round(dom_ms, 4)}

    log("[bench] decode")
    decode = {}
    for wd in (W.DECODE_F16_2K, W.DECODE_F16_32K):
        per = 2 * wd.batch * wd.heads * wd.seq_kv * wd.head_dim * 2
        n_sets = max(2, -(-(1 << 30) // per))
        xd = wd.make()
        qd = xd["q"].to(dev)
        ks = [xd["k"].to(dev) for _ in range(n_sets)]
        vs = [xd["v"].to(dev) for _ in range(n_sets)]
        od = torch.empty_like(qd)
        ld = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        wsd = torch.empty(fa.decode_workspace_bytes(fa.problem(qd, ks[0], scale=wd.scale)), dtype=torch.uint8,
                          device=dev)
        plans = [fa.plan_decode(qd, ks[j], vs[j], od, ld, wsd, scale=wd.scale) for j in range(n_sets)]
        call = lambda i: plans[i % n_sets]()
        for i in range(3):
            call(i)
        ms = time_calls(call, max(args.reps, 2 * n_sets), torch)
        nbytes = per + wd.batch * wd.heads * wd.head_dim * 2 * 2 + wd.batch * wd.heads * 4
        gbps = nbytes / (ms * 1e-3) / 1e9
        decode[str(wd.seq_kv)] = {"GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                                  "us": round(ms * 1e3, 2), "bytes": nbytes, "kv_copies_rotated": n_sets}
        del ks, vs, plans
        torch.cuda.empty_cache()

    result = {
        "metric": "attention TFLOP/s fwd & fwd+bwd (% MFMA peak); decode GB/s (% HBM peak)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "prefill forward+backward, fp16, causal, ALiBi", "batch": w.batch,
                   "heads": w.heads, "seq": w.seq_q, "head_dim": w.head_dim, "scale": "1/sqrt(64)"},
        "fwd_bwd": {"TFLOP/s": round(tflops, 2), "frac_mfma_peak": round(tflops / PEAK_F16_TFLOPS, 4),
                    "ms": round(ms_step, 4), "flop": fb_flops, "wall_s": round(wall, 3)},
        "forward": {"TFLOP/s": round(w.fwd_flops() / (ms_fwd * 1e-3) / 1e12, 2),
                    "frac_mfma_peak": round(w.fwd_flops() / (ms_fwd * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
                    "ms": round(ms_fwd, 4)},
        "backward_ms": {"all": round(ms_bwd, 4), "dq16_kernel": round(ms_q, 4), "dkdv16_kernel": round(ms_kv, 4)},
        "decode": decode,
        "roofline": roofline,
    }
    if args.extra:
        result["extra"] = extra_workloads(fa, W, torch, args.reps)
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_heads} slices")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_heads)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
