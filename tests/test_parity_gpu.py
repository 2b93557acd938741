"""GPU parity: the HIP library against the fp64 oracle on identical seeded inputs.

Bars: fp32 max-abs-err <= 1e-4 on O and <= 1e-5 on dQ/dK/dV; f16/bf16
max-abs-err / max|ref| <= 2e-2 on O and <= 5e-2 on each gradient; lse within
1e-3 + 1e-5 |lse|.  Small cases compare every element; the five workloads at
their full sizes compare sampled rows (and all dK/dV rows through a sparse dO).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from parity import (MOD_NAME, check, check_case, check_lse, full_parity, oracle_kw, run_backward, run_forward,
                    sampled_parity, say, to_dev)

pytestmark = pytest.mark.gpu

MODS = [W.MOD_NONE, W.MOD_ALIBI, W.MOD_CHECKERBOARD]


def small(dtype, D, causal, mod, mask, Sq=200, Skv=333, B=2, H=2, wid=100):
    if causal:
        Skv = Sq
    return W.Workload(f"small {dtype} D{D}", wid, B, H, Sq, Skv, D, dtype, causal=causal, mod=mod, key_mask=mask)


INSTANCES = [(dt, D, c, m, k) for dt, Ds in (("f16", (64, 128)), ("bf16", (64, 128)), ("f32", (64, 128)))
             for D in Ds for c in (False, True) for m in MODS for k in (False, True)]


@pytest.mark.parametrize("dtype,D,causal,mod,mask", INSTANCES)
def test_every_instance_small(gpu_lib, dtype, D, causal, mod, mask):
    full_parity(small(dtype, D, causal, mod, mask))


@pytest.mark.parametrize("dtype,D,causal,mod,mask", [x for x in INSTANCES if x[0] != "f32"])
def test_every_16bit_instance_both_dq_modes(gpu_lib, dtype, D, causal, mod, mask):
    """The backward with dQ from the separate query pass and from fp32
    atomics in the key/value pass, each against the oracle."""
    full_parity(small(dtype, D, causal, mod, mask, wid=109), dq_modes=("separate", "atomic"))


@pytest.mark.parametrize("causal,mod,mask", [(c, m, k) for c in (False, True) for m in MODS for k in (False, True)])
def test_f32_d512_small(gpu_lib, causal, mod, mask):
    full_parity(small("f32", 512, causal, mod, mask, Sq=80, Skv=130, B=1, H=2))


@pytest.mark.parametrize("Skv", [1, 31, 32, 33, 64, 65, 97])
@pytest.mark.parametrize("mask", [False, True])
def test_f32_d512_key_tile_edges(gpu_lib, Skv, mask):
    """head_dim 512 stages 32-key (and 32-query) tiles through two LDS buffers
    with the next tile's loads in flight: one, two and three tiles, full and
    ragged, with and without a key mask (the mask bytes load in the step)."""
    full_parity(small("f32", 512, False, W.MOD_ALIBI, mask, Sq=45, Skv=Skv, B=1, H=2, wid=108), strict=False)


@pytest.mark.parametrize("S", [1, 17, 63, 64, 65, 127, 129, 255, 257])
@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64), ("f32", 512)])
def test_ragged_causal_lengths(gpu_lib, S, dtype, D):
    full_parity(small(dtype, D, True, W.MOD_ALIBI, False, Sq=S, B=1, H=3, wid=101), strict=False)


def forward_halves(B, H, Sq, D, causal):
    """Whether a 16-bit forward runs on 64-query blocks with two waves per 32
    queries: with n 128-query blocks per slice and the device's forward slots
    (3 workgroups per CU at head_dim 64, 2 at 128), causal when B H (n + 1)
    is below the slots (1.2 times the slots at head_dim 128), otherwise when
    2 B H n is at most the slots."""
    n = (Sq + 127) // 128
    slots = (3 if D == 64 else 2) * torch.cuda.get_device_properties(0).multi_processor_count
    if not causal:
        return 2 * B * H * n <= slots
    return B * H * (n + 1) < slots if D == 64 else 5 * B * H * (n + 1) < 6 * slots


@pytest.mark.parametrize("B,H,Sq,Skv,off", [(2, 2, 200, 200, 0), (16, 16, 200, 200, 0), (1, 3, 700, 700, 0),
                                           (2, 3, 150, 301, 151), (16, 16, 150, 301, 151)])
@pytest.mark.parametrize("D,causal", [(64, True), (64, False), (128, True), (128, False)])
@pytest.mark.parametrize("dtype,mod,mask", [("f16", W.MOD_ALIBI, False), ("bf16", W.MOD_CHECKERBOARD, True)])
def test_forward_layouts(gpu_lib, B, H, Sq, Skv, off, D, causal, dtype, mod, mask):
    """With few blocks per workgroup slot the 16-bit forward takes 64-query
    blocks whose waves each cover one key half of every tile (the two waves
    of a query group merge their max, sum and accumulator at the end), with
    many the 128-query blocks.  On MI355X's 256 CUs the 2 x 2, 1 x 3 and
    2 x 3 shapes here take the first layout and the 16 x 16 shapes the
    second; every output element against the oracle, with ragged tails and a
    query offset on both sides."""
    w = small(dtype, D, False, mod, mask, Sq=Sq, Skv=Skv, B=B, H=H, wid=111)
    inputs = w.make(with_dout=False)
    say(f"[forward layout] {dtype} D{D} causal={causal} B{B} H{H} Sq{Sq} Skv{Skv} off{off} mod={mod} "
        f"mask={mask} halves={forward_halves(B, H, Sq, D, causal)}")
    dev = to_dev(inputs)
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal, score_mod=MOD_NAME[mod], scale=w.scale,
                          key_mask=dev.get("key_mask"), q_offset=off)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=causal, mod=mod, q_offset=off,
               key_mask=None if inputs.get("key_mask") is None else inputs["key_mask"].numpy())
    check_case(dtype, inputs, okw, out, lse)


def backward_halves(B, H, n, D, causal):
    """Whether a 16-bit dQ or dK/dV pass over n 128-row blocks per slice
    (queries for dQ, keys for dK/dV) runs on 64-row blocks with two waves per
    32 rows: with the passes' slots (2 workgroups per CU at head_dim 64, 1 at
    128), causal when 5 B H (n + 1) is below 6 slots, otherwise when 2 B H n
    is at most the slots."""
    slots = (2 if D == 64 else 1) * torch.cuda.get_device_properties(0).multi_processor_count
    return 5 * B * H * (n + 1) < 6 * slots if causal else 2 * B * H * n <= slots


@pytest.mark.parametrize("B,H,Sq,Skv,off", [(2, 2, 200, 200, 0), (16, 16, 200, 200, 0), (2, 3, 150, 301, 151),
                                           (16, 16, 150, 301, 151)])
@pytest.mark.parametrize("D,causal", [(64, True), (64, False), (128, True), (128, False)])
@pytest.mark.parametrize("dtype,mod,mask", [("f16", W.MOD_ALIBI, False), ("bf16", W.MOD_CHECKERBOARD, True)])
def test_backward_layouts(gpu_lib, B, H, Sq, Skv, off, D, causal, dtype, mod, mask):
    """With few blocks per workgroup slot the 16-bit dQ and dK/dV passes take
    64-row blocks whose waves each cover one half of every tile (the two
    waves of a row group add their sums at the end), with many the 128-row
    blocks.  On MI355X's 256 CUs the 2 x 2 and 2 x 3 shapes here take the
    first layout and the 16 x 16 shapes the second; forward and backward,
    every output element against the oracle, with ragged tails and a query
    offset on both sides."""
    w = small(dtype, D, False, mod, mask, Sq=Sq, Skv=Skv, B=B, H=H, wid=112)
    inputs = w.make()
    say(f"[backward layout] {dtype} D{D} causal={causal} B{B} H{H} Sq{Sq} Skv{Skv} off{off} mod={mod} mask={mask} "
        f"dq halves={backward_halves(B, H, (Sq + 127) // 128, D, causal)} "
        f"dk/dv halves={backward_halves(B, H, (Skv + 127) // 128, D, causal)}")
    dev = to_dev(inputs)
    kw = dict(causal=causal, score_mod=MOD_NAME[mod], scale=w.scale, key_mask=dev.get("key_mask"), q_offset=off)
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    grads = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], dq_mode="separate", **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=causal, mod=mod, q_offset=off,
               key_mask=None if inputs.get("key_mask") is None else inputs["key_mask"].numpy())
    check_case(dtype, inputs, okw, out, lse, grads)


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (1, 300), (300, 1), (5, 70), (129, 64), (64, 129)])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_ragged_noncausal_shapes(gpu_lib, Sq, Skv, dtype):
    full_parity(small(dtype, 64, False, W.MOD_CHECKERBOARD, True, Sq=Sq, Skv=Skv, B=2, H=1, wid=102), strict=False)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64), ("f32", 512)])
def test_fully_masked_rows_are_empty(gpu_lib, dtype, D):
    """Causal with the first keys masked: the first rows have no allowed key,
    so O = 0, lse = -inf and dQ = 0 there (the empty-sum reading)."""
    w = small(dtype, D, True, W.MOD_NONE, True, Sq=70, B=1, H=2, wid=103)
    inputs = w.make()
    km = torch.ones(1, 70, dtype=torch.uint8)
    km[0, :3] = 0
    inputs["key_mask"] = km
    res = full_parity(w, inputs=inputs)
    dev = to_dev(inputs)
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True, key_mask=dev["key_mask"])
    assert torch.all(out[:, :, :3] == 0) and torch.all(lse[:, :, :3] == float("-inf"))
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], causal=True, key_mask=dev["key_mask"])
    assert torch.all(dq[:, :, :3] == 0)
    assert res


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_masked_keys_with_garbage_are_ignored(gpu_lib, dtype):
    w = small(dtype, 64, False, W.MOD_NONE, True, Sq=90, Skv=150, B=2, H=2, wid=104)
    inputs = w.make()
    km = inputs["key_mask"]
    bad = (km == 0)
    for name in ("k", "v"):
        t = inputs[name].clone()
        t.permute(0, 2, 1, 3)[bad] = 300.0   # finite, huge values in masked rows
        inputs[name] = t
    full_parity(w, inputs=inputs)


def test_backward_is_deterministic(gpu_lib):
    """With the separate dQ pass (no atomics) repeated calls are bitwise equal."""
    for dtype, D, causal in (("f16", 64, True), ("bf16", 128, False), ("f32", 512, True)):
        w = small(dtype, D, causal, W.MOD_ALIBI, False, Sq=150, B=1, H=2, wid=105)
        say(f"[determinism] {dtype} D{D} causal={causal}")
        dev = to_dev(w.make())
        kw = dict(causal=causal, score_mod="alibi", dq_mode="separate")
        out, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal, score_mod="alibi")
        g1 = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], **kw)
        out2, lse2 = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal, score_mod="alibi")
        g2 = fa.backward(dev["q"], dev["k"], dev["v"], out2, lse2, dev["dout"], **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(lse, lse2)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("f32", 512)])
def test_backward_single_pass_matches_full(gpu_lib, dtype, D):
    w = small(dtype, D, True, W.MOD_ALIBI, False, Sq=140, B=1, H=2, wid=107)
    dev = to_dev(w.make())
    kw = dict(causal=True, score_mod="alibi")
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], dq_mode="separate", **kw)
    dq1, n1, n2 = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], which="dq", **kw)
    n3, dk1, dv1 = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], which="dkdv", **kw)
    torch.cuda.synchronize()
    assert n1 is None and n2 is None and n3 is None
    assert torch.equal(dq, dq1)
    if dtype == "f32":
        assert torch.equal(dk, dk1) and torch.equal(dv, dv1)
    else:
        # 16-bit: the full call takes delta = <dO, O> from the query pass, the
        # key/value-only call from the preprocess kernel (another fp32
        # summation order), so dK and dV may differ in the last bit
        for x, y in ((dk, dk1), (dv, dv1)):
            assert (x.float() - y.float()).abs().max().item() <= 1e-2 * x.float().abs().max().item()


def test_uniform_scores_full_shape_invariants(gpu_lib):
    """q = 0 at a long causal shape: O_i is the running mean of V and
    lse_i = log(i+1), checkable for every row without the oracle."""
    S, D = 4096, 64
    v = W.normal((1, 2, S, D), "f32", 106, W.V).cuda()
    q = torch.zeros_like(v)
    k = W.normal((1, 2, S, D), "f32", 106, W.K).cuda()
    out, lse = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    vd = v.double().cpu()
    cum = torch.cumsum(vd, dim=2) / torch.arange(1, S + 1, dtype=torch.float64)[None, None, :, None]
    assert (out.double().cpu() - cum).abs().max().item() < 3e-5
    ref = torch.log(torch.arange(1, S + 1, dtype=torch.float64))
    assert (lse.double().cpu() - ref).abs().max().item() < 3e-5


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("causal,mod,mask", [(True, W.MOD_ALIBI, False), (False, W.MOD_CHECKERBOARD, True),
                                             (False, W.MOD_NONE, False)])
def test_ones_v_gives_ones(gpu_lib, dtype, causal, mod, mask):
    """Rows of P sum to 1: with V = 1 every output is 1 (each row here has an
    allowed key).  The 16-bit bound is the rounding of P to the input type."""
    w = small(dtype, 64, causal, mod, mask, Sq=300, Skv=517)
    inputs = w.make(with_dout=False)
    inputs["v"] = torch.ones_like(inputs["v"])
    dev = to_dev(inputs)
    say(f"[ones] {dtype} causal={causal} mod={mod} mask={mask}")
    out, _ = run_forward(w, dev)
    tol = {"f32": 1e-5, "f16": 2e-3, "bf16": 8e-3}[dtype]
    assert (out.float() - 1.0).abs().max().item() <= tol


@pytest.mark.parametrize("w", [W.PREFILL_F16, W.KEYPAD_BF16], ids=["prefill", "keypad"])
def test_full_shape_hull_and_gradient_sums(gpu_lib, w):
    """At the full workload shape, for every row: the output lies in the box
    spanned by the head's V rows (per dim), sum_j dV_j = sum_i dO_i (rows of P
    sum to 1) and sum_j dK_j = 0 (rows of dS sum to 0)."""
    inputs = w.make()
    dev = to_dev(inputs)
    say(f"[invariants] {w.name}")
    out, lse = run_forward(w, dev)
    v = dev["v"].float()
    lo, hi = v.amin(dim=2, keepdim=True), v.amax(dim=2, keepdim=True)
    slack = 1e-2 * (hi - lo)   # P and O rounded to the 16-bit type
    o = out.float()
    assert bool(((o >= lo - slack) & (o <= hi + slack)).all())
    _, dk, dv = run_backward(w, dev, out, lse, dev["dout"])
    do = dev["dout"].double()
    sum_dv, sum_do, abs_do = dv.double().sum(dim=2), do.sum(dim=2), do.abs().sum(dim=2)
    assert bool(((sum_dv - sum_do).abs() <= 1e-2 * abs_do + 1e-3).all())
    sum_dk, abs_dk = dk.double().sum(dim=2), dk.double().abs().sum(dim=2)
    assert bool((sum_dk.abs() <= 2e-2 * abs_dk + 1e-3).all())


# ------------------------------------------------------------------ decode


def decode_case(dtype, D, Skv, mod, mask, B=3, H=2, wid=110):
    w = W.Workload(f"decode {dtype}", wid, B, H, 1, Skv, D, dtype, mod=mod, key_mask=mask, backward=False)
    say(f"[decode] {dtype} D{D} Skv{Skv} mod={mod} mask={mask}")
    inputs = w.make()
    dev = to_dev(inputs)
    out, lse = fa.decode(dev["q"], dev["k"], dev["v"], key_mask=dev.get("key_mask"),
                         score_mod={0: None, 1: "alibi", 2: "checkerboard"}[mod], scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(inputs["q"], inputs["k"], inputs["v"], **{k: v for k, v in oracle_kw(w, inputs).items() if k != "causal"})
    check("decode o", out, o_ref, dtype, "o")
    check_lse(lse, lse_ref)
    return dev, out, lse, w


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("f16", 128), ("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("Skv", [1, 77, 2053])
@pytest.mark.parametrize("mod,mask", [(W.MOD_NONE, False), (W.MOD_ALIBI, True), (W.MOD_CHECKERBOARD, False)])
def test_decode_small(gpu_lib, dtype, D, Skv, mod, mask):
    decode_case(dtype, D, Skv, mod, mask)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_decode_matches_forward_at_one_query(gpu_lib, dtype):
    dev, out, lse, w = decode_case(dtype, 64, 4100, W.MOD_CHECKERBOARD, True)
    out2, lse2 = fa.forward(dev["q"], dev["k"], dev["v"], key_mask=dev["key_mask"], score_mod="checkerboard")
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert (out.float() - out2.float()).abs().max().item() <= tol * max(1.0, out2.float().abs().max().item())
    assert (lse - lse2).abs().max().item() < 1e-4


def test_decode_independent_of_split(gpu_lib):
    """The number of key chunks depends on batch * heads: one head decoded
    alone (many chunks) and as head 0 of a 64-head batch (few chunks) agree,
    and both match the oracle."""
    Skv, D = 32768, 64
    w1 = W.Workload("decode one head", 120, 1, 1, 1, Skv, D, "f16", backward=False)
    one = w1.make()
    w64 = W.Workload("decode 64 heads", 121, 8, 8, 1, Skv, D, "f16", backward=False)
    many = w64.make()
    for k in ("q", "k", "v"):
        many[k][0, 0] = one[k][0, 0]
    d1, d64 = to_dev(one), to_dev(many)
    say("[decode split] one head vs 64 heads")
    o1, l1 = fa.decode(d1["q"], d1["k"], d1["v"])
    o64, l64 = fa.decode(d64["q"], d64["k"], d64["v"])
    torch.cuda.synchronize()
    assert (o1[0, 0].float() - o64[0, 0].float()).abs().max().item() <= 2e-3 * o1.float().abs().max().item()
    assert abs(l1[0, 0, 0].item() - l64[0, 0, 0].item()) < 1e-4
    o_ref, lse_ref = oracle.decode(one["q"], one["k"], one["v"], scale=w1.scale)
    check("decode o (one head)", o1, o_ref, "f16", "o")
    check_lse(l1, lse_ref)


@pytest.mark.parametrize("dtype,Sq", [("f16", 1), ("bf16", 1), ("f32", 1), ("f16", 16), ("bf16", 16), ("f32", 16)])
def test_decode_explicit_key_splits(gpu_lib, dtype, Sq):
    """The same decode split into 1, 2, 7 and the most (FA_MAX_KV_SPLITS
    requested) key chunks: every split against the oracle, and the splits
    against each other (they differ only in the order of the exact merge)."""
    Skv, D = 5000, 64
    w = W.Workload(f"decode splits {dtype}", 122, 2, 3, Sq, Skv, D, dtype, mod=W.MOD_ALIBI, key_mask=True,
                   backward=False)
    x = w.make()
    dev = to_dev(x)
    off = Skv - Sq
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], scale=w.scale, mod=W.MOD_ALIBI, q_offset=off, causal=True,
                                key_mask=x["key_mask"].numpy())
    outs = []
    for n in (1, 2, 7, 256):
        say(f"[decode splits] {dtype} Sq{Sq} kv_splits={n}")
        out, lse = fa.decode(dev["q"], dev["k"], dev["v"], key_mask=dev["key_mask"], score_mod="alibi",
                             scale=w.scale, q_offset=off, causal=True, kv_splits=n)
        torch.cuda.synchronize()
        check("o", out, o_r, dtype, "o")
        check_lse(lse, lse_r)
        outs.append((out.float(), lse))
    tol = 1e-5 if dtype == "f32" else 1e-2
    for o, l in outs[1:]:
        assert (o - outs[0][0]).abs().max().item() <= tol * max(1.0, outs[0][0].abs().max().item())
        assert (l - outs[0][1]).abs().max().item() < 1e-4


# ------------------------------------------------------------- the workloads


def test_workload_tiny_f32_exact(gpu_lib):
    full_parity(W.TINY_F32)


@pytest.mark.timeout(900)
def test_workload_prefill_f16_causal_alibi(gpu_lib):
    """The prefill workload at its full size (8, 8, 2048, 64), dense dO:
    every element of O, lse, dQ, dK and dV against the oracle (flash-attention-jax
    page, value_and_grad_difference: plain against flash on o, dq, dk, dv),
    with both dQ modes."""
    full_parity(W.PREFILL_F16, dq_modes=("separate", "atomic"))


@pytest.mark.timeout(900)
def test_workload_keypad_bf16_checkerboard(gpu_lib):
    """The key-padding workload at its full size (4, 16, 4096, 128), dense dO:
    every element against the oracle, with both dQ modes."""
    full_parity(W.KEYPAD_BF16, dq_modes=("separate", "atomic"))


@pytest.mark.parametrize("w", [W.DECODE_F16_2K, W.DECODE_F16_32K], ids=["2k", "32k"])
def test_workload_decode_f16(gpu_lib, w):
    inputs = w.make()
    dev = to_dev(inputs)
    say(f"[workload] {w.name}")
    out, lse = fa.decode(dev["q"], dev["k"], dev["v"], scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(inputs["q"], inputs["k"], inputs["v"], scale=w.scale)
    check("decode o", out, o_ref, "f16", "o")
    check_lse(lse, lse_ref)


def test_workload_long_f32_d512_causal(gpu_lib):
    sampled_parity(W.LONG_F32, 256)


@pytest.mark.timeout(600)
def test_long_f32_d512_uniform_scores_every_row(gpu_lib):
    """q = 0 at the long-context shape (1, 1, 131072, 512), causal: every score
    is 0, so O_i is the running mean of V[0..i] and lse_i = log(i + 1), for
    every one of the 131072 rows (closed form, no oracle needed)."""
    w = W.LONG_F32
    v = W.normal(w.kv_shape(), "f32", w.workload_id, W.V).cuda()
    k = W.normal(w.kv_shape(), "f32", w.workload_id, W.K).cuda()
    q = torch.zeros(w.q_shape(), dtype=torch.float32, device="cuda")
    say("[long q=0] forward at (1, 1, 131072, 512)")
    out, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    S = w.seq_q
    vd = v.double().cpu()
    cum = torch.cumsum(vd, dim=2) / torch.arange(1, S + 1, dtype=torch.float64)[None, None, :, None]
    e_o = (out.double().cpu() - cum).abs().max().item()
    ref = torch.log(torch.arange(1, S + 1, dtype=torch.float64))
    e_l = (lse.double().cpu() - ref).abs().max().item()
    say(f"[long q=0] O max-abs-err {e_o:.3e}, lse max-abs-err {e_l:.3e}")
    assert e_o <= 1e-4 and e_l <= 1e-4


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 64), ("f16", 128), ("f32", 64), ("f32", 512)])
@pytest.mark.parametrize("causal,mod,spike", [(False, W.MOD_NONE, "last"), (False, W.MOD_ALIBI, "first"),
                                              (True, W.MOD_NONE, "first"), (True, W.MOD_ALIBI, "first")])
def test_running_max_grows_on_the_last_visited_tile(gpu_lib, dtype, D, causal, mod, spike):
    """One key scores far above the rest (about 2^23 in P) and sits in the tile
    the forward visits last (key 0 for causal and for ALiBi, whose tiles are
    visited last key first; the last key otherwise), so the running max grows
    at the very end and the accumulator rescale runs on the final tile.

    Forward only: with attention this close to one-hot, dS = P (dP - D) is a
    difference of two nearly equal numbers (D = rowsum(dO * O) uses the
    stored 16-bit O), so the exact dQ and dK are near zero and an error
    relative to their maximum says nothing about the kernel."""
    S = 260
    w = small(dtype, D, causal, mod, False, Sq=S, Skv=S, B=1, H=8, wid=106)
    inputs = w.make()
    g = torch.Generator().manual_seed(106)
    q = 1.25 + 0.1 * torch.randn(1, 8, S, D, generator=g, dtype=torch.float64)
    k = inputs["k"].double().clone()
    k[:, :, 0 if spike == "first" else S - 1, :] = 2.0
    tdt = inputs["q"].dtype
    inputs["q"], inputs["k"] = q.to(tdt), k.to(tdt)
    full_parity(w, backward=False, inputs=inputs)


# ------------------------------------------------------------------ query offsets (KV cache)

OFFSET_SHAPES = [(70, 333, 263), (129, 300, 40), (1, 300, 299), (200, 150, 0), (33, 64, 7)]


def offset_parity(dtype, D, causal, mod, mask, Sq, Skv, off, wid):
    """Forward and backward with query row i at key position i + off, every
    output element against the oracle with the same offset."""
    w = small(dtype, D, False, mod, mask, Sq=Sq, Skv=Skv, B=1, H=2, wid=wid)
    inputs = w.make()
    say(f"[offset] {dtype} D{D} causal={causal} mod={mod} mask={mask} Sq{Sq} Skv{Skv} off{off}")
    dev = to_dev(inputs)
    kw = dict(causal=causal, score_mod={W.MOD_NONE: None, W.MOD_ALIBI: "alibi", W.MOD_CHECKERBOARD: "checkerboard"}[mod],
              scale=w.scale, key_mask=dev.get("key_mask"), q_offset=off)
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=causal, mod=mod, q_offset=off,
               key_mask=None if inputs.get("key_mask") is None else inputs["key_mask"].numpy())
    check_case(dtype, inputs, okw, out, lse, (dq, dk, dv), strict=False)


@pytest.mark.parametrize("Sq,Skv,off", OFFSET_SHAPES)
@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("causal,mod,mask", [(True, W.MOD_ALIBI, False), (True, W.MOD_CHECKERBOARD, True),
                                             (True, W.MOD_NONE, False), (False, W.MOD_ALIBI, True),
                                             (False, W.MOD_CHECKERBOARD, False)])
def test_query_offset(gpu_lib, dtype, D, causal, mod, mask, Sq, Skv, off):
    offset_parity(dtype, D, causal, mod, mask, Sq, Skv, off, wid=130)


@pytest.mark.parametrize("dtype,D", [("f16", 128), ("bf16", 64), ("f32", 128), ("f32", 512)])
def test_query_offset_other_instances(gpu_lib, dtype, D):
    offset_parity(dtype, D, True, W.MOD_CHECKERBOARD, False, 45, 190, 145, wid=131)
    offset_parity(dtype, D, True, W.MOD_ALIBI, True, 64, 129, 65, wid=132)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mod", [W.MOD_NONE, W.MOD_ALIBI, W.MOD_CHECKERBOARD])
@pytest.mark.parametrize("off", [0, 1000, 4099])
def test_decode_with_offset(gpu_lib, dtype, mod, off):
    """Decode of the query at position off: non-causal (score_mod at that
    position) and causal (keys 0 .. off only)."""
    Skv, D = 4100, 64
    w = W.Workload(f"decode offset {dtype}", 133, 2, 3, 1, Skv, D, dtype, mod=mod, backward=False)
    x = w.make()
    dev = to_dev(x)
    name = {W.MOD_NONE: None, W.MOD_ALIBI: "alibi", W.MOD_CHECKERBOARD: "checkerboard"}[mod]
    for causal in (False, True):
        say(f"[decode offset] {dtype} mod={mod} off={off} causal={causal}")
        out, lse = fa.decode(dev["q"], dev["k"], dev["v"], score_mod=name, scale=w.scale, q_offset=off, causal=causal)
        torch.cuda.synchronize()
        o_r, lse_r = oracle.decode(x["q"], x["k"], x["v"], scale=w.scale, mod=mod, q_offset=off, causal=causal)
        check("o", out, o_r, dtype, "o")
        check_lse(lse, lse_r)


# ------------------------------------------------------------------ short query blocks (split over keys)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("Sq,Skv", [(2, 300), (16, 5000), (32, 2100), (33, 4100), (64, 700)])
@pytest.mark.parametrize("causal,mod,mask", [(True, W.MOD_ALIBI, False), (True, W.MOD_NONE, True),
                                             (False, W.MOD_CHECKERBOARD, True), (False, W.MOD_NONE, False)])
def test_decode_short_query_block(gpu_lib, dtype, D, Sq, Skv, causal, mod, mask):
    """1 < seq_q <= 64 through fa_decode (the forward split over key chunks
    plus the exact merge), queries after a KV cache (q_offset = seq_kv -
    seq_q), against the oracle and against fa_forward."""
    off = Skv - Sq
    w = small(dtype, D, False, mod, mask, Sq=Sq, Skv=Skv, B=2, H=3, wid=140)
    x = w.make(with_dout=False)
    dev = to_dev(x)
    name = {W.MOD_NONE: None, W.MOD_ALIBI: "alibi", W.MOD_CHECKERBOARD: "checkerboard"}[mod]
    kw = dict(score_mod=name, scale=w.scale, key_mask=dev.get("key_mask"), q_offset=off, causal=causal)
    say(f"[short block] {dtype} D{D} Sq{Sq} Skv{Skv} causal={causal} mod={mod} mask={mask}")
    out, lse = fa.decode(dev["q"], dev["k"], dev["v"], **kw)
    out_f, lse_f = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    torch.cuda.synchronize()
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], scale=w.scale, causal=causal, mod=mod, q_offset=off,
                                key_mask=None if x.get("key_mask") is None else x["key_mask"].numpy())
    check("o", out, o_r, dtype, "o")
    check_lse(lse, lse_r)
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert (out.float() - out_f.float()).abs().max().item() <= tol * max(1.0, out_f.float().abs().max().item())
