"""Caller-defined score_mods (attnax pallas_flash_attention page: score_mod,
a callable applied to the scaled scores with global indices) compiled by the
library at run time, forward and backward against the fp64 oracle with the
same functions written in numpy.

Bars as for the built-in mods: 16-bit max-abs-err / max|ref| <= 2e-2 (O) and
5e-2 (gradients); fp32 max-abs-err <= 1e-4 (O) and 1e-5 (gradients); lse
within 1e-3 + 1e-5 |lse|.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from parity import check, check_lse, say, to_dev

pytestmark = pytest.mark.gpu

# tanh soft-cap of the scores, cap = params[0]: score-dependent, so the
# backward needs the derivative 1 - tanh^2
SOFTCAP = """
__device__ float fa_score_mod(float s, int b, int h, int q, int k, const float* p) {
  return p[0] * tanhf(s / p[0]);
}
__device__ float fa_score_mod_grad(float s, int b, int h, int q, int k, const float* p) {
  const float t = tanhf(s / p[0]);
  return 1.0f - t * t;
}
"""
# ALiBi written as a caller-defined mod, slopes = params[h]
ALIBI = """
__device__ float fa_score_mod(float s, int b, int h, int q, int k, const float* p) {
  return s - p[h] * (float)(q - k);
}
__device__ float fa_score_mod_grad(float s, int b, int h, int q, int k, const float* p) { return 1.0f; }
"""
CAP = 2.0


def softcap_np(s, b, h, qi, kj):
    return CAP * np.tanh(s / CAP)


def softcap_grad_np(s, b, h, qi, kj):
    return 1.0 - np.tanh(s / CAP) ** 2


@pytest.fixture(scope="module")
def mods(gpu_lib):
    m = {"softcap": fa.ScoreMod(SOFTCAP), "alibi": fa.ScoreMod(ALIBI)}
    yield m
    torch.cuda.synchronize()
    for x in m.values():
        x.close()


def run_custom(mod, params, w, inputs, *, q_offset=0, block_mask=None):
    dev = to_dev(inputs)
    kw = dict(causal=w.causal, score_mod=mod, mod_params=params, scale=w.scale, key_mask=dev.get("key_mask"),
              q_offset=q_offset, block_mask=None if block_mask is None else block_mask.cuda())
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    grads = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], **kw)
    torch.cuda.synchronize()
    return out, lse, grads


CASES = [("f16", 64, False, False, False, 0), ("f16", 64, True, False, False, 0), ("bf16", 64, True, True, False, 0),
         ("f16", 128, False, True, False, 0), ("bf16", 128, True, False, True, 0), ("f16", 64, True, True, True, 37),
         ("bf16", 64, False, False, True, 0), ("f16", 128, True, False, False, 90),
         ("f32", 64, True, False, False, 0), ("f32", 64, False, True, True, 0), ("f32", 128, True, True, False, 53),
         ("f32", 128, False, False, True, 0)]


@pytest.mark.parametrize("dtype,D,causal,mask,blk,off", CASES)
def test_custom_softcap(mods, dtype, D, causal, mask, blk, off):
    Sq, Skv = 300, 300 + off if causal else 413
    w = W.Workload("custom softcap", 400, 2, 2, Sq, Skv, D, dtype, causal=causal, key_mask=mask)
    x = w.make()
    x["q"], x["k"] = (2.0 * x["q"].float()).to(x["q"].dtype), (2.0 * x["k"].float()).to(x["k"].dtype)
    bm = W.bernoulli_block_mask(2, 2, Sq, Skv, 400, p_keep=0.7) if blk else None
    say(f"[custom softcap] {dtype} D{D} causal={causal} mask={mask} blk={blk} off={off}")
    params = torch.tensor([CAP], dtype=torch.float32, device="cuda")
    out, lse, (dq, dk, dv) = run_custom(mods["softcap"], params, w, x, q_offset=off, block_mask=bm)
    okw = dict(scale=w.scale, causal=causal, q_offset=off, mod=oracle.MOD_CUSTOM,
               custom=(softcap_np, softcap_grad_np),
               key_mask=None if x.get("key_mask") is None else x["key_mask"].numpy(),
               block_mask=None if bm is None else bm.numpy() != 0)
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], **okw)
    g_r = oracle.backward(x["q"], x["k"], x["v"], x["dout"], **okw)
    check("o", out, o_r, dtype, "o")
    check_lse(lse, lse_r)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_r):
        check(name, g, r, dtype, "grad")


@pytest.mark.parametrize("dtype,D,causal,mask", [("f16", 64, True, False), ("bf16", 128, False, True)])
def test_custom_alibi_matches_the_builtin_alibi(mods, dtype, D, causal, mask):
    """ALiBi written as a caller-defined mod gives what the built-in ALiBi
    kernels give (and the oracle's ALiBi)."""
    w = W.Workload("custom alibi", 401, 2, 4, 333, 333, D, dtype, causal=causal, mod=W.MOD_ALIBI, key_mask=mask)
    x = w.make()
    slopes = torch.from_numpy(oracle.default_alibi_slopes(4)).float().cuda()
    out, lse, grads = run_custom(mods["alibi"], slopes, w, x)
    dev = to_dev(x)
    kw = dict(causal=causal, score_mod="alibi", scale=w.scale, key_mask=dev.get("key_mask"))
    out_b, lse_b = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    grads_b = fa.backward(dev["q"], dev["k"], dev["v"], out_b, lse_b, dev["dout"], **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=causal, mod=W.MOD_ALIBI,
               key_mask=None if x.get("key_mask") is None else x["key_mask"].numpy())
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], **okw)
    g_r = oracle.backward(x["q"], x["k"], x["v"], x["dout"], **okw)
    check("o", out, o_r, dtype, "o")
    check_lse(lse, lse_r)
    assert (lse - lse_b).abs().max().item() < 1e-3
    for name, g, gb, r in zip(("dq", "dk", "dv"), grads, grads_b, g_r):
        check(name, g, r, dtype, "grad")
        check(name + " (custom vs built-in)", g, gb.double().cpu().numpy(), dtype, "grad")


@pytest.mark.timeout(600)
def test_custom_softcap_prefill_full_size(mods):
    """The prefill shape (8, 8, 2048, 64) fp16 causal with the soft-cap mod:
    every element of O, lse, dQ, dK, dV against the oracle."""
    w = W.Workload("custom softcap prefill", 402, 8, 8, 2048, 2048, 64, "f16", causal=True)
    x = w.make()
    params = torch.tensor([CAP], dtype=torch.float32, device="cuda")
    say("[custom softcap] prefill (8, 8, 2048, 64)")
    out, lse, grads = run_custom(mods["softcap"], params, w, x)
    okw = dict(scale=w.scale, causal=True, mod=oracle.MOD_CUSTOM, custom=(softcap_np, softcap_grad_np))
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], **okw)
    g_r = oracle.backward(x["q"], x["k"], x["v"], x["dout"], **okw)
    check("o", out, o_r, "f16", "o")
    check_lse(lse, lse_r)
    for name, g, r in zip(("dq", "dk", "dv"), grads, g_r):
        check(name, g, r, "f16", "grad")


def test_custom_mod_is_refused_where_it_is_not_built(mods):
    """fa_decode and the split forward stop at head_dim 128: an fp32
    head_dim 512 problem with a caller-defined mod is FA_ERR_UNSUPPORTED
    there, nothing launched."""
    q = torch.randn(1, 2, 1, 512, device="cuda", dtype=torch.float32)
    k = torch.randn(1, 2, 100, 512, device="cuda", dtype=torch.float32)
    p = torch.tensor([CAP], dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.decode(q, k, k, score_mod=mods["softcap"], mod_params=p)
    assert e.value.status == 2
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, k, k, score_mod=mods["softcap"], mod_params=p, kv_splits=2)
    assert e.value.status == 2


@pytest.mark.parametrize("causal,mask", [(True, False), (False, True)])
def test_custom_softcap_f32_d512(mods, causal, mask):
    """fp32 at head_dim 512 (the long-context kernels, dims split over four
    waves) with the soft cap, forward and backward against the oracle."""
    Sq, Skv = 80, 80 if causal else 130
    w = W.Workload("custom softcap d512", 405, 1, 2, Sq, Skv, 512, "f32", causal=causal, key_mask=mask)
    x = w.make()
    x["q"], x["k"] = 2.0 * x["q"], 2.0 * x["k"]
    say(f"[custom softcap] f32 D512 causal={causal} mask={mask}")
    params = torch.tensor([CAP], dtype=torch.float32, device="cuda")
    out, lse, (dq, dk, dv) = run_custom(mods["softcap"], params, w, x)
    okw = dict(scale=w.scale, causal=causal, mod=oracle.MOD_CUSTOM, custom=(softcap_np, softcap_grad_np),
               key_mask=None if x.get("key_mask") is None else x["key_mask"].numpy())
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], **okw)
    g_r = oracle.backward(x["q"], x["k"], x["v"], x["dout"], **okw)
    check("o", out, o_r, "f32", "o")
    check_lse(lse, lse_r)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_r):
        check(name, g, r, "f32", "grad")


@pytest.mark.parametrize("dtype,D,Sq,Skv,causal,mask,n", [
    ("f16", 64, 1, 5000, False, False, 0), ("bf16", 128, 1, 4100, True, True, 7), ("f16", 128, 16, 3000, True, False, 0),
    ("bf16", 64, 64, 2500, False, True, 5), ("f32", 64, 1, 3000, True, True, 0), ("f32", 128, 16, 2100, False, False, 3)])
def test_custom_softcap_decode(mods, dtype, D, Sq, Skv, causal, mask, n):
    """fa_decode (and fa_decode_noalloc) with a caller-defined mod: one query
    or a short block after a KV cache (query row i at key position
    Skv - Sq + i), split over the keys, against the oracle."""
    w = W.Workload("custom softcap decode", 403, 2, 3, Sq, Skv, D, dtype, causal=causal, key_mask=mask)
    x = w.make()
    x["q"] = (2.0 * x["q"].float()).to(x["q"].dtype)
    dev = to_dev(x)
    off = Skv - Sq
    params = torch.tensor([CAP], dtype=torch.float32, device="cuda")
    kw = dict(score_mod=mods["softcap"], mod_params=params, scale=w.scale, key_mask=dev.get("key_mask"),
              q_offset=off, causal=causal)
    say(f"[custom decode] {dtype} D{D} Sq={Sq} Skv={Skv} causal={causal} mask={mask} n={n}")
    out, lse = fa.decode(dev["q"], dev["k"], dev["v"], kv_splits=n, **kw)
    out2, lse2 = fa.decode_noalloc(dev["q"], dev["k"], dev["v"], **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=causal, q_offset=off, mod=oracle.MOD_CUSTOM,
               custom=(softcap_np, softcap_grad_np),
               key_mask=None if x.get("key_mask") is None else x["key_mask"].numpy())
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], **okw)
    check("o", out, o_r, dtype, "o")
    check_lse(lse, lse_r)
    check("o (no-allocation decode)", out2, o_r, dtype, "o")
    check_lse(lse2, lse_r)


@pytest.mark.parametrize("dtype,D,causal,blk,n", [("f16", 64, True, False, 3), ("bf16", 128, False, True, 5),
                                                  ("f32", 128, True, True, 4)])
def test_custom_softcap_forward_split(mods, dtype, D, causal, blk, n):
    """fa_forward_split with a caller-defined mod (an explicit chunk count:
    the table keeps caller mods whole) against the oracle, and the backward
    from its lse."""
    Sq = Skv = 700
    w = W.Workload("custom softcap split", 404, 2, 2, Sq, Skv, D, dtype, causal=causal)
    x = w.make()
    x["q"], x["k"] = (2.0 * x["q"].float()).to(x["q"].dtype), (2.0 * x["k"].float()).to(x["k"].dtype)
    bm = W.bernoulli_block_mask(2, 2, Sq, Skv, 404, p_keep=0.7) if blk else None
    dev = to_dev(x)
    params = torch.tensor([CAP], dtype=torch.float32, device="cuda")
    kw = dict(causal=causal, score_mod=mods["softcap"], mod_params=params, scale=w.scale,
              block_mask=None if bm is None else bm.cuda())
    say(f"[custom split] {dtype} D{D} causal={causal} blk={blk} n={n}")
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], kv_splits=n, **kw)
    grads = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=causal, mod=oracle.MOD_CUSTOM, custom=(softcap_np, softcap_grad_np),
               block_mask=None if bm is None else bm.numpy() != 0)
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], **okw)
    g_r = oracle.backward(x["q"], x["k"], x["v"], x["dout"], **okw)
    check("o", out, o_r, dtype, "o")
    check_lse(lse, lse_r)
    for name, g, r in zip(("dq", "dk", "dv"), grads, g_r):
        check(name, g, r, dtype, "grad")
