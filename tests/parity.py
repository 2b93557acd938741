"""Helpers shared by the GPU parity tests: run the HIP library and the fp64
oracle on the same seeded inputs and measure the difference."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from bounds import kappa, within

MOD_NAME = {W.MOD_NONE: None, W.MOD_ALIBI: "alibi", W.MOD_CHECKERBOARD: "checkerboard"}

# Tolerances (fp32: max-abs-err; 16-bit: max-abs-err / max|ref|).
TOL_F32 = {"o": 1e-4, "grad": 1e-5}
TOL_16 = {"o": 2e-2, "grad": 5e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def err(gpu: torch.Tensor, ref: np.ndarray, dtype: str, strict: bool = True) -> float:
    """fp32: max-abs-err.  16-bit: max-abs-err / max|ref|.

    With strict=False (edge-case shapes only), a 16-bit reference that is
    identically zero up to rounding (max|ref| < 1e-3, e.g. dQ and dK with a
    single key) is compared in absolute terms."""
    g = gpu.detach().double().cpu().numpy()
    d = float(np.abs(g - ref).max()) if ref.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if dtype == "f32":
        return d
    if not strict and scale < 1e-3:
        return d
    return d / max(scale, 1e-30)


def check(name: str, gpu: torch.Tensor, ref: np.ndarray, dtype: str, kind: str, strict: bool = True,
          mag: np.ndarray = None, kap: float = None) -> float:
    """Error against the bar; returns the error (fp32: absolute).

    fp32 passes when the absolute error is within the bar.  Otherwise, with
    strict=False and the oracle's magnitudes ``mag`` given, every element must
    be within the per-element bound tol + kap u M derived from its
    accumulation (tests/bounds.py); the log says which held."""
    tol = (TOL_F32 if dtype == "f32" else TOL_16)[kind]
    g = gpu.detach().double().cpu().numpy()
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    e = err(gpu, ref, dtype, strict)
    if dtype == "f32":
        if e <= tol:
            say(f"[{name}] fp32 max-abs-err {e:.3e} <= {tol:.0e}")
            return e
        assert not strict and mag is not None, f"{name}: error {e:.3e} > {tol:.1e}"
        ok, ratio = within(np.abs(g - ref), tol, kap, mag)
        say(f"[{name}] fp32 max-abs-err {e:.3e} > {tol:.0e}: per-element bound tol + {kap:.1f} u M, "
            f"worst ratio {ratio:.3f}")
        assert ok, f"{name}: error above the derived bound (worst ratio {ratio:.3f})"
        return e
    say(f"[{name}] {dtype} max-abs-err / max|ref| {e:.3e} <= {tol:.0e}" if e <= tol else f"[{name}] {e:.3e}")
    assert e <= tol, f"{name}: error {e:.3e} > {tol:.1e}"
    return e


def check_lse(gpu: torch.Tensor, ref: np.ndarray) -> None:
    g = gpu.detach().double().cpu().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin), "lse: empty rows differ"
    assert np.all(g[~fin] == -np.inf)
    if fin.any():
        d = np.abs(g[fin] - ref[fin])
        assert (d <= 1e-3 + 1e-5 * np.abs(ref[fin])).all(), f"lse: max error {d.max():.3e}"


def kw_of(w: W.Workload) -> dict:
    return dict(causal=w.causal, score_mod=MOD_NAME[w.mod], scale=w.scale)


def oracle_kw(w: W.Workload, inputs: dict) -> dict:
    kw = dict(scale=w.scale, causal=w.causal, mod=w.mod,
              key_mask=None if inputs.get("key_mask") is None else inputs["key_mask"].numpy())
    if inputs.get("block_mask") is not None:
        kw["block_mask"] = inputs["block_mask"].numpy() != 0
    return kw


def to_dev(inputs: dict) -> dict:
    return {k: (None if v is None else v.cuda()) for k, v in inputs.items()}


def run_forward(w: W.Workload, dev: dict):
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], key_mask=dev.get("key_mask"),
                          block_mask=dev.get("block_mask"), **kw_of(w))
    torch.cuda.synchronize()
    return out, lse


def run_backward(w: W.Workload, dev: dict, out, lse, dout, dq_mode: str = "auto"):
    g = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dout, key_mask=dev.get("key_mask"),
                    block_mask=dev.get("block_mask"), dq_mode=dq_mode, **kw_of(w))
    torch.cuda.synchronize()
    return g


def oracle_refs(w: W.Workload, inputs: dict, okw: dict, backward: bool, strict: bool):
    """Oracle outputs, and for relaxed fp32 checks the error magnitudes."""
    o_ref, lse_ref = oracle.forward(inputs["q"], inputs["k"], inputs["v"], **okw)
    grads = oracle.backward(inputs["q"], inputs["k"], inputs["v"], inputs["dout"], **okw) if backward else None
    mags = None
    if w.dtype == "f32" and not strict:
        mags = oracle.magnitudes(inputs["q"], inputs["k"], inputs["v"],
                                 inputs["dout"] if backward else torch.zeros_like(inputs["q"]), **okw)
    return o_ref, lse_ref, grads, mags


def check_case(dtype: str, inputs: dict, okw: dict, out, lse, grads=None, strict: bool = True) -> dict:
    """O, lse (and dQ, dK, dV when grads is given) of one GPU run against the
    oracle with keyword arguments okw (the same inputs)."""
    q = inputs["q"]
    Sq, D, Skv = q.shape[2], q.shape[3], inputs["k"].shape[2]
    o_ref, lse_ref = oracle.forward(q, inputs["k"], inputs["v"], **okw)
    mags = None
    if dtype == "f32" and not strict:
        mags = oracle.magnitudes(q, inputs["k"], inputs["v"],
                                 inputs["dout"] if grads is not None else torch.zeros_like(q), **okw)
    kap = kappa(Sq, Skv, D)
    res = {"o": check("o", out, o_ref, dtype, "o", strict, None if mags is None else mags[0], kap)}
    check_lse(lse, lse_ref)
    if grads is not None:
        g_ref = oracle.backward(q, inputs["k"], inputs["v"], inputs["dout"], **okw)
        for i, name in enumerate(("dq", "dk", "dv")):
            res[name] = check(name, grads[i], g_ref[i], dtype, "grad", strict,
                              None if mags is None else mags[i + 1], kap)
    return res


def full_parity(w: W.Workload, backward: bool = True, inputs=None, strict: bool = True,
                dq_modes=("auto",)) -> dict:
    """Every output element against the oracle (sizes the oracle finishes
    quickly); the backward once per dQ mode in dq_modes, against one oracle run."""
    say(f"[parity] {w.name} B{w.batch} H{w.heads} Sq{w.seq_q} Skv{w.seq_kv} D{w.head_dim} {w.dtype} "
        f"causal={w.causal} mod={w.mod} mask={w.key_mask}")
    inputs = inputs or w.make(with_dout=backward)
    dev = to_dev(inputs)
    out, lse = run_forward(w, dev)
    okw = oracle_kw(w, inputs)
    o_ref, lse_ref, g_ref, mags = oracle_refs(w, inputs, okw, backward, strict)
    kap = kappa(w.seq_q, w.seq_kv, w.head_dim)
    res = {"o": check("o", out, o_ref, w.dtype, "o", strict, None if mags is None else mags[0], kap)}
    check_lse(lse, lse_ref)
    if backward:
        for mode in dq_modes:
            grads = run_backward(w, dev, out, lse, dev["dout"], dq_mode=mode)
            sfx = "" if mode == "auto" else f" ({mode} dQ)"
            for i, name in enumerate(("dq", "dk", "dv")):
                res[name + sfx] = check(name + sfx, grads[i], g_ref[i], w.dtype, "grad", strict,
                                        None if mags is None else mags[i + 1], kap)
            del grads
    say(f"[parity] ok {res}")
    return res


def sampled_parity(w: W.Workload, n_rows: int, backward: bool = True, block_mask=None) -> dict:
    """Large shapes: O, lse and dQ on sampled query rows; all dK, dV rows from
    a second backward whose dO is zero outside the sampled rows (exact, since
    the backward is linear in dO)."""
    say(f"[sampled] {w.name}: generating inputs")
    inputs = w.make(with_dout=backward)
    inputs["block_mask"] = block_mask
    rows = W.sample_rows(w.seq_q, n_rows, w.workload_id)
    dev = to_dev(inputs)
    say(f"[sampled] {w.name}: forward on GPU")
    out, lse = run_forward(w, dev)
    okw = oracle_kw(w, inputs)
    say(f"[sampled] {w.name}: oracle forward on {len(rows)} rows")
    o_ref, lse_ref = oracle.forward(inputs["q"], inputs["k"], inputs["v"], rows=rows, **okw)
    r = torch.from_numpy(rows).cuda()
    res = {"o": check("o", out[:, :, r], o_ref, w.dtype, "o")}
    check_lse(lse[:, :, r], lse_ref)
    if backward:
        say(f"[sampled] {w.name}: backward on GPU (dense dO)")
        dq, _, _ = run_backward(w, dev, out, lse, dev["dout"])
        dq_s = dq[:, :, r].cpu()
        del dq
        sparse = torch.zeros_like(dev["dout"])
        sparse[:, :, r] = dev["dout"][:, :, r]
        say(f"[sampled] {w.name}: backward on GPU (dO zero outside sampled rows)")
        _, dk, dv = run_backward(w, dev, out, lse, sparse)
        say(f"[sampled] {w.name}: oracle backward on {len(rows)} rows")
        dq_r, dk_r, dv_r = oracle.backward(inputs["q"], inputs["k"], inputs["v"], inputs["dout"], rows=rows, **okw)
        res["dq"] = check("dq", dq_s, dq_r, w.dtype, "grad")
        res["dk"] = check("dk", dk, dk_r, w.dtype, "grad")
        res["dv"] = check("dv", dv, dv_r, w.dtype, "grad")
    say(f"[sampled] ok {res}")
    return res
