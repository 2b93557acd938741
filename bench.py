#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

A step is one forward plus one full backward (dQ, dK, dV) of the prefill
workload: fp16 q, k, v ~ N(0, 1) of shape (8, 8, 2048, 64), causal, ALiBi
score_mod, dO ~ N(0, 1).  The headline value is forward+backward TFLOP/s on
the algorithmic flop count (causal pairs S(S+1)/2 per head; 4*D flop per pair
forward, 10*D backward).  The same JSON line also carries the other
workloads, each timed with HIP events on the library's stream:

* tiny fp32 (1, 2, 256, 64): forward and forward+backward (latency-bound);
* key-padding bf16 (4, 16, 4096, 128), Bernoulli(0.5) key mask and
  checkerboard: forward and forward+backward (all pairs evaluated);
* long-context fp32 (1, 1, 131072, 512), causal: forward and
  forward+backward against the fp32 matrix peak;
* split-KV decode, fp16 (8, 8, 1, 64) against 2048 and 32768 keys, GB/s of
  K + V + q + O + lse with K/V copies rotated so reads come from HBM;

plus the backward of both 16-bit workloads in each dQ mode (separate query
pass and atomics), the roofline of the headline's dominant kernel (with its
average duration from the committed rocprofv3 trace beside the event-derived
one), and the fp64 oracle timed on a bounded sample on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-s SECONDS]
"""
from __future__ import annotations

import argparse
import hashlib
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
    """Average milliseconds per call of fn(i) from HIP events on the current
    stream (the stream the library launches on)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def settle(fn, seconds: float, torch) -> int:
    """Calls fn(i) untimed for `seconds` (the GPU clock ramps up over the
    first tens of milliseconds of load); returns the number of calls."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


COMMON_HEADER = "tiled_online_softmax_flashattention_amd/csrc/fa_common.hpp"


def source_sha(path: str) -> str:
    """sha256 over a kernel's source file followed by the device header that
    every kernel file includes."""
    h = hashlib.sha256()
    for p in (path, COMMON_HEADER):
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


SOURCES = {"fwd16_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_fwd16.hip",
           "dq16_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_dq16.hip",
           "dkdv16_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_bwd16.hip",
           "bwd_pre_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_bwd16.hip",
           "dq_convert_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_bwd16.hip",
           "fwd32_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_fwd32.hip",
           "dq32_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_bwd32.hip",
           "dkdv32_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_bwd32.hip",
           "decode_split_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_decode.hip",
           "decode_merge_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_decode.hip",
           "fwd16_split_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_fwd16.hip",
           "fwd16_halves_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_fwd16.hip",
           "fwd32_short_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_fwd32.hip",
           "split_merge_kernel": "tiled_online_softmax_flashattention_amd/csrc/fa_decode.hip"}


def source_of(kernel_name: str):
    """Source file of a kernel from its (demangled) rocprof name."""
    for short, src in SOURCES.items():
        if f"::{short}<" in kernel_name or kernel_name.startswith(short):
            return src
    return None


# The headline's dominant kernel, as rocprofv3 names it.
DKDV_PREFILL = "void fa::dkdv16_kernel<fa::F16, 64, 1, true, false, false, false, false>(fa::AttnArgs)"
TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace_bench.json")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bench.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_bench.json")
COPY_BYTES = 256 * 1024 * 1024    # the calibration copy of --counters


# ------------------------------------------------------------------ profiles
#
# The summaries under profiles/ come from rocprofv3 runs of this script and
# are written by the summary modes below; each records the command that made
# it and the sha256 of every kernel's source (its file and the shared device
# header), and bench.py reports a figure from them only while that source is
# unchanged.


def counters_pass() -> int:
    """What the rocprofv3 --pmc runs profile: a device copy of COPY_BYTES (the
    counters' calibration), then two forward + backward steps of the prefill
    and of the key-padding workload and one of the long-context workload."""
    import torch

    import tiled_online_softmax_flashattention_amd as fa
    import workloads as W

    x = torch.ones(COPY_BYTES // 4, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    del x, y
    for w, kw, n in ((W.PREFILL_F16, dict(causal=True, score_mod="alibi"), 2),
                     (W.KEYPAD_BF16, dict(score_mod="checkerboard"), 2),
                     (W.LONG_F32, dict(causal=True), 1)):
        d = {k: (None if t is None else t.cuda()) for k, t in w.make().items()}
        kw = dict(kw, key_mask=d["key_mask"], scale=w.scale)
        q, k, v, do = d["q"], d["k"], d["v"], d["dout"]
        out, lse = fa.forward(q, k, v, **kw)
        for _ in range(n):
            fa.forward(q, k, v, out=out, lse=lse, **kw)
            fa.backward(q, k, v, out, lse, do, **kw)
        torch.cuda.synchronize()
        del d, q, k, v, do, out, lse
        torch.cuda.empty_cache()
    print("counters pass done", flush=True)
    return 0


def _per_dispatch(path: str):
    """{dispatch id: (kernel name, {counter: value summed over the device})}."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return {d: (names[d], vals[d]) for d in vals}


def traffic_summary(fetch_csv: str, write_csv: str, command: str) -> int:
    """Writes the HBM traffic summary from the counter_collection CSVs of the
    two rocprofv3 passes over --counters: per-dispatch FETCH_SIZE / WRITE_SIZE
    (KiB, summed over the device) of each kernel (median over its dispatches),
    scaled by what the same counters read for the calibration copy."""
    from collections import defaultdict
    fetch, write = _per_dispatch(fetch_csv), _per_dispatch(write_csv)

    def by_kernel(disp, counter):
        out = defaultdict(list)
        for name, c in disp.values():
            out[name].append(c[counter])
        return out

    fk, wk = by_kernel(fetch, "FETCH_SIZE"), by_kernel(write, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024
    cf = max(v for n, lst in fk.items() if "copyBuffer" in n or "elementwise" in n for v in lst)
    cw = max(v for n, lst in wk.items() if "copyBuffer" in n or "elementwise" in n for v in lst)
    out = {"command": command, "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                                                    "fetch_factor": round(copy_kib / cf, 4),
                                                    "write_factor": round(copy_kib / cw, 4)},
           "kernels": {}}
    for name in sorted(fk):
        src = source_of(name)
        if src is None or name not in wk:
            continue
        f = sorted(fk[name])[len(fk[name]) // 2]
        wv = sorted(wk[name])[len(wk[name]) // 2]
        out["kernels"][name] = {"fetch_kib": f, "write_kib": wv, "dispatches": len(fk[name]),
                                "hbm_bytes": int(round((f * copy_kib / cf + wv * copy_kib / cw) * 1024)),
                                "source": src, "source_sha256": source_sha(src)}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    rows = [(n, r["dispatches"], round(r["fetch_kib"] / 1024, 1), round(r["write_kib"] / 1024, 1),
             round(r["hbm_bytes"] / 1e6, 1)) for n, r in sorted(out["kernels"].items())]
    _write_md(TRAFFIC_FILE[:-5] + ".md", "traffic-summary", "L2-to-memory traffic per dispatch (rocprofv3 FETCH_SIZE, WRITE_SIZE)",
              command, ("kernel", "dispatches", "FETCH_SIZE MiB", "WRITE_SIZE MiB", "bytes (calibrated), MB"), rows,
              f"`bench.py --counters`: a {COPY_BYTES >> 20} MiB device copy, then untimed forward + backward steps of "
              f"the prefill, key-padding and long-context workloads; the median dispatch of each kernel. "
              f"Calibration on the copy: FETCH_SIZE reads {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB for "
              f"{copy_kib:.0f} KiB moved, so fetch counts are scaled by {copy_kib / cf:.4f} and write counts by "
              f"{copy_kib / cw:.4f}. These count bytes between L2 and the memory fabric (the on-package cache "
              f"included), an upper bound on HBM bytes.")
    print(json.dumps(out, indent=1))
    return 0


def _write_md(path: str, mode: str, title: str, command: str, header, rows, notes: str = "") -> None:
    """A short markdown table beside a JSON summary (same figures)."""
    lines = [f"# {title}", "", "Command (from the repository root on the GPU box, `R` = that root), then "
             f"`python bench.py --{mode} ...` on its CSVs:", "", "```",
             command, "```", ""]
    if notes:
        lines += [notes, ""]
    lines.append("| " + " | ".join(header) + " |")
    lines.append("|" + "---|" * len(header))
    lines += ["| " + " | ".join(str(c) for c in r) + " |" for r in rows]
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def trace_summary(stats_csv: str, command: str) -> int:
    """Writes the kernel-duration summary from rocprofv3's kernel_stats.csv."""
    import csv
    out = {"command": command, "kernels": {}}
    for r in csv.DictReader(open(stats_csv)):
        src = source_of(r["Name"])
        rec = {"calls": int(r["Calls"]), "average_ns": float(r["AverageNs"]), "min_ns": float(r["MinNs"]),
               "max_ns": float(r["MaxNs"]), "share_percent": float(r["Percentage"])}
        if src:
            rec.update(source=src, source_sha256=source_sha(src))
        out["kernels"][r["Name"]] = rec
    with open(TRACE_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    rows = [(n, r["calls"], round(r["average_ns"] / 1e3, 2), round(r["min_ns"] / 1e3, 2), round(r["max_ns"] / 1e3, 2),
             f'{r["share_percent"]:.2f} %')
            for n, r in sorted(out["kernels"].items(), key=lambda kv: -kv[1]["share_percent"])]
    _write_md(TRACE_FILE[:-5] + ".md", "trace-summary", "Kernel durations of bench.py (rocprofv3 kernel trace)", command,
              ("kernel", "calls", "average us", "min us", "max us", "share of traced time"), rows,
              "The traced run is the default bench without the CPU baseline: every workload of the JSON line, "
              "each timed loop after its clock settle.")
    print(json.dumps(out, indent=1))
    return 0


def counter_summary(csv1: str, csv2: str, csv3: str, command: str) -> int:
    """Shader-counter summary (last dispatch of each kernel) from the three
    rocprofv3 --pmc passes over --counters.  cycles = GRBM_GUI_ACTIVE / 8
    (summed over the 8 XCDs); SIMD-cycle shares divide by cycles x 1024 SIMDs:
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES, VALU busy = 4 SQ_ACTIVE_INST_VALU
    (quad-cycles), both in one cycle = SQ_VALU_MFMA_COEXEC_CYCLES; waves per
    CU = 4 SQ_WAVE_CYCLES / cycles / 256; VALU instructions per MFMA =
    (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA; exp per MFMA =
    SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_MFMA; s_waitcnt share =
    SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; LDS bank-conflict share =
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    merged = {}
    for path in (csv1, csv2, csv3):
        disp = _per_dispatch(path)
        last = {}
        for d, (name, c) in sorted(disp.items()):
            last[name] = c
        for name, c in last.items():
            merged.setdefault(name, {}).update(c)
    out = {"command": command, "kernels": {}}
    print("| kernel | cycles | MFMA busy | VALU busy | MFMA and VALU in one cycle | waves per CU | VALU instr "
          "per MFMA | exp per MFMA | wave time in s_waitcnt | LDS bank-conflict share |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for name, c in sorted(merged.items()):
        src = source_of(name)
        need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_WAVE_CYCLES")
        if src is None or any(k not in c for k in need) or c["SQ_INSTS_MFMA"] == 0:
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / 8
        simd = cyc * 1024
        rec = {"cycles": cyc, "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / simd,
               "valu_busy": 4 * c.get("SQ_ACTIVE_INST_VALU", 0) / simd,
               "coexec": c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0) / simd,
               "waves_per_cu": 4 * c["SQ_WAVE_CYCLES"] / cyc / 256,
               "valu_per_mfma": (c.get("SQ_INSTS_VALU", 0) - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"],
               "exp_per_mfma": c.get("SQ_INSTS_VALU_TRANS_F32", 0) / c["SQ_INSTS_MFMA"],
               "waitcnt_share": c.get("SQ_WAIT_INST_ANY", 0) / c["SQ_WAVE_CYCLES"],
               "lds_conflict_share": c.get("SQ_LDS_BANK_CONFLICT", 0) / max(1.0, c.get("SQ_LDS_IDX_ACTIVE", 0)),
               "source": src, "source_sha256": source_sha(src), "raw": dict(c)}
        out["kernels"][name] = rec
        print(f"| {name} | {cyc:.0f} | {100 * rec['mfma_busy']:.1f} % | {100 * rec['valu_busy']:.1f} % | "
              f"{100 * rec['coexec']:.1f} % | {rec['waves_per_cu']:.1f} | {rec['valu_per_mfma']:.1f} | "
              f"{rec['exp_per_mfma']:.2f} | {100 * rec['waitcnt_share']:.0f} % | "
              f"{100 * rec['lds_conflict_share']:.0f} % |")
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    rows = [(n, f'{r["cycles"]:.0f}', f'{100 * r["mfma_busy"]:.1f} %', f'{100 * r["valu_busy"]:.1f} %',
             f'{100 * r["coexec"]:.1f} %', f'{r["waves_per_cu"]:.1f}', f'{r["valu_per_mfma"]:.1f}',
             f'{r["exp_per_mfma"]:.2f}', f'{100 * r["waitcnt_share"]:.0f} %', f'{100 * r["lds_conflict_share"]:.0f} %')
            for n, r in sorted(out["kernels"].items())]
    _write_md(COUNTERS_FILE[:-5] + ".md", "counter-summary", "Shader counters per kernel (rocprofv3 --pmc, three passes)", command,
              ("kernel", "cycles", "MFMA busy", "VALU busy", "MFMA and VALU in one cycle", "waves per CU",
               "VALU instr per MFMA", "exp per MFMA", "wave time in s_waitcnt", "LDS bank-conflict share"), rows,
              "Last dispatch of each kernel in `bench.py --counters`. " + " ".join(counter_summary.__doc__.split()))
    return 0


def _from_summary(path: str, kernel: str, field: str):
    """A kernel's figure from a committed summary, or None when the file,
    the kernel or its unchanged source is missing."""
    try:
        rec = json.load(open(path))["kernels"][kernel]
        if rec["source_sha256"] != source_sha(rec["source"]):
            return None
        return rec[field]
    except (OSError, KeyError, ValueError):
        return None



# ------------------------------------------------------------------ workloads


def dense_workload(fa, W, torch, w, kw: dict, peak: float, reps: int, settle_s: float, dq_modes=("auto",)) -> dict:
    """Forward and forward+backward of one workload (inputs resident in HBM),
    and the backward alone in each dQ mode asked for."""
    d = {k: (None if t is None else t.cuda()) for k, t in w.make().items()}
    kw = dict(kw, key_mask=d["key_mask"], scale=w.scale)
    q, k, v, do = d["q"], d["k"], d["v"], d["dout"]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    run_fwd = fa.plan_forward(q, k, v, out, lse, **kw)
    bwd = {}
    for mode in dq_modes:
        ws = torch.empty(fa.backward_workspace_bytes(fa.problem(q, k, dq_mode=mode, **kw)), dtype=torch.uint8,
                         device=q.device)
        bwd[mode] = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, dq_mode=mode, **kw)
    run_bwd = bwd[dq_modes[0]]
    run_fwd()
    for f in bwd.values():
        f()
    settle(lambda i: (run_fwd(), run_bwd()), settle_s, torch)
    ms_f = time_calls(lambda i: run_fwd(), reps, torch)
    ms_fb = time_calls(lambda i: (run_fwd(), run_bwd()), reps, torch)
    ff, fb = w.fwd_flops(), w.fwd_flops() + w.bwd_flops()
    res = {"forward": {"ms": round(ms_f, 4), "TFLOP/s": round(ff / ms_f / 1e9, 2),
                       "frac_peak": round(ff / ms_f / 1e9 / peak, 4)},
           "fwd_bwd": {"ms": round(ms_fb, 4), "TFLOP/s": round(fb / ms_fb / 1e9, 2),
                       "frac_peak": round(fb / ms_fb / 1e9 / peak, 4)},
           "peak_TFLOP/s": peak, "calls_timed": reps,
           "flop_convention": "causal pairs" if w.causal else "all pairs evaluated"}
    if len(dq_modes) > 1:
        res["backward_ms_by_dq_mode"] = {m: round(time_calls(lambda i: f(), reps, torch), 4) for m, f in bwd.items()}
    del d, q, k, v, do, out, lse, grads, bwd, run_fwd, run_bwd
    torch.cuda.empty_cache()
    return res


def decode_workloads(fa, W, torch, reps: int, settle_s: float) -> dict:
    """Split-KV decode at 2048 and 32768 keys; K/V copies are rotated (>= 1
    GiB in all) so every call reads from HBM, after a clock settle."""
    res = {}
    for wd in (W.DECODE_F16_2K, W.DECODE_F16_32K):
        per = 2 * wd.batch * wd.heads * wd.seq_kv * wd.head_dim * 2
        n_sets = max(2, -(-(1 << 30) // per))
        xd = wd.make()
        qd = xd["q"].cuda()
        ks = [xd["k"].cuda() for _ in range(n_sets)]
        vs = [xd["v"].cuda() for _ in range(n_sets)]
        od = torch.empty_like(qd)
        ld = torch.empty(qd.shape[:3], dtype=torch.float32, device=qd.device)
        wsd = torch.empty(fa.decode_workspace_bytes(fa.problem(qd, ks[0], scale=wd.scale)), dtype=torch.uint8,
                          device=qd.device)
        plans = [fa.plan_decode(qd, ks[j], vs[j], od, ld, wsd, scale=wd.scale) for j in range(n_sets)]
        call = lambda i: plans[i % n_sets]()
        settled = settle(call, settle_s, torch)
        ms = time_calls(call, max(reps, 4 * n_sets), torch)
        nbytes = per + wd.batch * wd.heads * wd.head_dim * 2 * 2 + wd.batch * wd.heads * 4
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[str(wd.seq_kv)] = {"GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                               "us": round(ms * 1e3, 2), "bytes": nbytes, "kv_copies_rotated": n_sets,
                               "settle_calls": settled}
        del ks, vs, plans
        torch.cuda.empty_cache()
    return res

def extra_workloads(fa, W, torch, reps: int) -> dict:
    """A short query block against a long KV cache (split over keys vs. the
    plain forward) and a block-sparse prefill (sliding window of blocks)."""
    res = {}
    # A block of 16 new queries after a 32752-key cache (causal, ALiBi), fp16
    # and fp32: the key-split path of fa_decode against the plain forward on
    # the same problem; K/V copies are rotated so reads come from HBM.
    for dt, tdt, es in (("f16", torch.float16, 2), ("f32", torch.float32, 4)):
        B, H, Sq, Skv, D = 8, 8, 16, 32768, 64
        log(f"[bench] extra: short query block {dt} {B}x{H}x{Sq} against {Skv} keys")
        gen = torch.Generator(device="cuda").manual_seed(7)
        q = torch.randn(B, H, Sq, D, device="cuda", dtype=tdt, generator=gen)
        kvs = [(torch.randn(B, H, Skv, D, device="cuda", dtype=tdt, generator=gen),
                torch.randn(B, H, Skv, D, device="cuda", dtype=tdt, generator=gen)) for _ in range(2)]
        kw = dict(causal=True, score_mod="alibi", q_offset=Skv - Sq)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.decode_workspace_bytes(fa.problem(q, kvs[0][0], **kw)), dtype=torch.uint8, device="cuda")
        split = [fa.plan_decode(q, k, v, out, lse, ws, **kw) for k, v in kvs]
        plain = [fa.plan_forward(q, k, v, out, lse, kv_splits=1, **kw) for k, v in kvs]
        for f in split + plain:
            f()
        settle(lambda i: split[i % 2](), 0.2, torch)
        ms_s = time_calls(lambda i: split[i % 2](), max(reps, 4), torch)
        ms_p = time_calls(lambda i: plain[i % 2](), max(reps, 4), torch)
        nbytes = 2 * B * H * Skv * D * es + 2 * B * H * Sq * D * es + B * H * Sq * 4
        res[f"short query block {dt} causal ALiBi ({B},{H},{Sq},{D}) after {Skv - Sq} cached keys"] = {
            "split_us": round(ms_s * 1e3, 2), "split_GB/s": round(nbytes / (ms_s * 1e-3) / 1e9, 1),
            "split_frac_hbm_peak": round(nbytes / (ms_s * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "forward_unsplit_us": round(ms_p * 1e3, 2), "bytes": nbytes}
        del q, kvs, out, lse, ws, split, plain
        torch.cuda.empty_cache()

    # One long head: fp16 (1, 1, 32768, 128), causal, ALiBi.  Its 256 query
    # blocks alone leave the device idle (the last, longest ones finish
    # alone); forward() splits the key axis by the library's per-shape table
    # (fa_forward_split), timed against the unsplit fa_forward.
    B, H, S, D = 1, 1, 32768, 128
    log(f"[bench] extra: long single head {B}x{H}x{S}x{D} f16 causal ALiBi, split vs unsplit forward")
    gen = torch.Generator(device="cuda").manual_seed(11)
    q, k, v = (torch.randn(B, H, S, D, device="cuda", dtype=torch.float16, generator=gen) for _ in range(3))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    kw = dict(causal=True, score_mod="alibi")
    chunks = fa.forward_split_workspace_bytes(fa.problem(q, k, **kw)) // (B * H * S * (D + 2) * 4)
    run_split = fa.plan_forward(q, k, v, out, lse, **kw)
    run_whole = fa.plan_forward(q, k, v, out, lse, kv_splits=1, **kw)
    run_split(); run_whole()
    settle(lambda i: run_split(), 0.2, torch)
    ms_s = time_calls(lambda i: run_split(), reps, torch)
    ms_w = time_calls(lambda i: run_whole(), reps, torch)
    flop = 4.0 * D * B * H * S * (S + 1) / 2
    res[f"long single head f16 causal ALiBi ({B},{H},{S},{D}), forward split over keys"] = {
        "key_chunks": int(chunks), "split_ms": round(ms_s, 4), "split_TFLOP/s": round(flop / ms_s / 1e9, 1),
        "split_frac_peak": round(flop / ms_s / 1e9 / PEAK_F16_TFLOPS, 4),
        "unsplit_ms": round(ms_w, 4), "unsplit_TFLOP/s": round(flop / ms_w / 1e9, 1),
        "flop_convention": "causal pairs"}
    del q, k, v, out, lse, run_split, run_whole
    torch.cuda.empty_cache()

    # Caller-defined score_mods at the prefill shape, fp16 (8, 8, 2048, 64),
    # causal: ALiBi written as a caller mod (slopes from mod_params) against
    # the built-in ALiBi kernels, and a tanh soft cap (a score-dependent mod,
    # whose backward multiplies dS by its derivative).  The first call
    # compiles each configuration; it runs before the timed loops.
    B, H, S, D = 8, 8, 2048, 64
    log(f"[bench] extra: caller-defined score_mods {B}x{H}x{S}x{D} f16 causal")
    alibi_src = """
__device__ float fa_score_mod(float s, int b, int h, int q, int k, const float* p) { return s - p[h] * (float)(q - k); }
__device__ float fa_score_mod_grad(float s, int b, int h, int q, int k, const float* p) { return 1.0f; }
"""
    softcap_src = """
__device__ float fa_score_mod(float s, int b, int h, int q, int k, const float* p) { return p[0] * tanhf(s / p[0]); }
__device__ float fa_score_mod_grad(float s, int b, int h, int q, int k, const float* p) {
  const float t = tanhf(s / p[0]);
  return 1.0f - t * t;
}
"""
    gen = torch.Generator(device="cuda").manual_seed(13)
    q, k, v, do = (torch.randn(B, H, S, D, device="cuda", dtype=torch.float16, generator=gen) for _ in range(4))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32, device="cuda")
    cap = torch.tensor([20.0], dtype=torch.float32, device="cuda")
    flop_f = 4.0 * D * B * H * S * (S + 1) / 2
    mods = {"built-in ALiBi": (None, "alibi", None), "ALiBi as a caller mod": (alibi_src, None, slopes),
            "tanh soft cap (caller mod)": (softcap_src, None, cap)}
    row = {}
    for name, (src, builtin, params) in mods.items():
        mod = fa.ScoreMod(src) if src else builtin
        kw = dict(causal=True, score_mod=mod, mod_params=params)
        ws = torch.empty(fa.backward_workspace_bytes(fa.problem(q, k, **kw)), dtype=torch.uint8, device="cuda")
        run_fwd = fa.plan_forward(q, k, v, out, lse, kv_splits=1, **kw)
        run_bwd = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, **kw)
        run_fwd(); run_bwd()
        settle(lambda i: (run_fwd(), run_bwd()), 0.2, torch)
        ms_f = time_calls(lambda i: run_fwd(), reps, torch)
        ms_fb = time_calls(lambda i: (run_fwd(), run_bwd()), reps, torch)
        row[name] = {"forward_ms": round(ms_f, 4), "forward_TFLOP/s": round(flop_f / ms_f / 1e9, 1),
                     "fwd_bwd_ms": round(ms_fb, 4), "fwd_bwd_TFLOP/s": round(3.5 * flop_f / ms_fb / 1e9, 1)}
        torch.cuda.synchronize()
        del run_fwd, run_bwd, ws
        if src:
            mod.close()
    res[f"caller-defined score_mods f16 causal ({B},{H},{S},{D})"] = dict(row, flop_convention="causal pairs")
    del q, k, v, do, out, lse, grads
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
                    help="seconds of untimed calls before each timed loop, so the GPU clock has left its ramp")
    ap.add_argument("--reps", type=int, default=20, help="calls per per-kernel timing loop")
    ap.add_argument("--cpu-heads", type=int, default=64, help="(batch, head) slices in the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true",
                    help="also time a short query block against a KV cache and a block-sparse prefill")
    ap.add_argument("--counters", action="store_true",
                    help="only run the calibration copy and untimed steps (for rocprofv3 --pmc)")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write the HBM traffic summary from two rocprofv3 counter CSVs of --counters")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_STATS_CSV", "COMMAND"),
                    help="write the kernel-duration summary from a rocprofv3 kernel_stats.csv of this script")
    ap.add_argument("--counter-summary", nargs=4, metavar=("CSV1", "CSV2", "CSV3", "COMMAND"),
                    help="write the shader-counter summary from three rocprofv3 --pmc CSVs of --counters")
    args = ap.parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    if args.trace_summary:
        return trace_summary(*args.trace_summary)
    if args.counter_summary:
        return counter_summary(*args.counter_summary)
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
    ws = torch.empty(fa.backward_workspace_bytes(fa.problem(q, k, dq_mode="atomic", **kw)), dtype=torch.uint8,
                     device=dev)

    run_fwd = fa.plan_forward(q, k, v, out, lse, **kw)
    run_bwd = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, **kw)
    run_q = fa.plan_backward(q, k, v, out, lse, do, grads[0], None, None, ws, **kw)
    run_sep = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, dq_mode="separate", **kw)
    run_atomic = fa.plan_backward(q, k, v, out, lse, do, *grads, ws, dq_mode="atomic", **kw)

    def step(_i=0):
        run_fwd()
        run_bwd()

    log(f"[bench] settle {args.settle_s} s, warmup {args.warmup}")
    settle_steps = settle(step, args.settle_s, torch)
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
    ms_sep = time_calls(lambda i: run_sep(), args.reps, torch)
    ms_atomic = time_calls(lambda i: run_atomic(), args.reps, torch)
    # The backward (dQ mode "auto" = the separate query pass) launches the
    # query kernel, which also writes the row statistics, and then the
    # key/value kernel on one stream, so the key/value kernel's time is the
    # difference of the two timings.
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
    full = {"dkdv16_kernel": DKDV_PREFILL,
            "dq16_kernel": "void fa::dq16_kernel<fa::F16, 64, 1, true, false, false, false>(fa::AttnArgs)",
            "fwd16_kernel": "void fa::fwd16_kernel<fa::F16, 64, 1, true, false, false>(fa::AttnArgs)"}[dom]
    traced_ns = _from_summary(TRACE_FILE, full, "average_ns")
    roofline = {"bound": "mfma", "kernel": full, "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                "traffic": _from_summary(TRAFFIC_FILE, full, "hbm_bytes"),
                "algorithmic_flop_per_launch": dom_flops, "avg_ms": round(dom_ms, 4),
                "rocprof_avg_ms": None if traced_ns is None else round(traced_ns * 1e-6, 4)}
    if traced_ns is not None:
        roofline["frac_from_rocprof_avg"] = round(dom_flops / (traced_ns * 1e-9) / 1e12 / PEAK_F16_TFLOPS, 4)
    del q, k, v, do, out, lse, grads, ws, run_fwd, run_bwd, run_q, run_sep, run_atomic
    torch.cuda.empty_cache()

    log("[bench] decode")
    decode = decode_workloads(fa, W, torch, args.reps, args.settle_s)
    log("[bench] tiny fp32")
    tiny = dense_workload(fa, W, torch, W.TINY_F32, {}, PEAK_F32_TFLOPS, 200, 0.05)
    log("[bench] key-padding bf16")
    keypad = dense_workload(fa, W, torch, W.KEYPAD_BF16, dict(score_mod="checkerboard"), PEAK_F16_TFLOPS,
                            args.reps, args.settle_s, dq_modes=("auto", "atomic"))
    log("[bench] long-context fp32")
    long32 = dense_workload(fa, W, torch, W.LONG_F32, dict(causal=True), PEAK_F32_TFLOPS, 2, 0.0)

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
        "backward_ms": {"all": round(ms_bwd, 4), "dq16_kernel": round(ms_q, 4), "dkdv16_kernel": round(ms_kv, 4),
                        "by_dq_mode": {"separate": round(ms_sep, 4), "atomic": round(ms_atomic, 4)}},
        "decode": decode,
        "workloads": {W.TINY_F32.name: tiny, W.KEYPAD_BF16.name: keypad, W.LONG_F32.name: long32},
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
