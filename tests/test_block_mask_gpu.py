"""GPU parity of block-sparse attention (block mask over 128 x 128 blocks of
(query row, key)) against the fp64 oracle, on identical seeded inputs.

Same bars as the dense parity tests: fp32 max-abs-err <= 1e-4 on O and
<= 1e-5 on dQ/dK/dV; f16/bf16 max-abs-err / max|ref| <= 2e-2 on O and
<= 5e-2 on each gradient; lse within 1e-3 + 1e-5 |lse|.  Every mask carries an
empty block row (rows with no allowed key: O = 0, lse = -inf, dQ = 0) and an
empty block column (keys no query sees: dK = dV = 0).

Removing blocks (with a key mask on top) leaves each query few keys, so the
probabilities concentrate and dK, dV grow to about 10 (oracle: max|dV| = 10.3
for fp32 D = 128 with a key mask); a 300-term fp32 sum of that size resolves
to about 1e-6 of it, above the absolute 1e-5.  The fp32 small cases therefore
pass either within the absolute bars or within the per-element bound derived
from the accumulation (tests/bounds.py); the long sampled cases stay strict.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from parity import check, check_case, check_lse, full_parity, oracle_kw, sampled_parity, say, to_dev

pytestmark = pytest.mark.gpu

MODS = [W.MOD_NONE, W.MOD_ALIBI, W.MOD_CHECKERBOARD]


def block_case(dtype, D, causal, mod, mask, Sq=300, Skv=400, B=2, H=2, wid=200):
    """Inputs with a Bernoulli(0.5) block mask, block row 1 of (0, 0) and block
    column 0 of (0, 1) cleared."""
    if causal:
        Skv = Sq
    w = W.Workload(f"block-sparse {dtype} D{D}", wid, B, H, Sq, Skv, D, dtype, causal=causal, mod=mod,
                   key_mask=mask)
    inputs = w.make()
    bm = W.bernoulli_block_mask(B, H, Sq, Skv, wid)
    if bm.shape[2] > 1:
        bm[0, 0, 1, :] = 0
    bm[0, min(1, H - 1), :, 0] = 0
    inputs["block_mask"] = bm
    return w, inputs


INSTANCES = [(dt, D, c, m, k) for dt, Ds in (("f16", (64, 128)), ("bf16", (64, 128)), ("f32", (64, 128)))
             for D in Ds for c in (False, True) for m in MODS for k in (False, True)]


@pytest.mark.parametrize("dtype,D,causal,mod,mask", INSTANCES)
def test_block_mask_every_instance(gpu_lib, dtype, D, causal, mod, mask):
    w, inputs = block_case(dtype, D, causal, mod, mask)
    full_parity(w, inputs=inputs, strict=dtype != "f32")


@pytest.mark.parametrize("dtype,D,causal,mod,mask", [("f16", 64, True, W.MOD_ALIBI, False),
                                                     ("bf16", 128, False, W.MOD_CHECKERBOARD, True),
                                                     ("f16", 128, True, W.MOD_NONE, True),
                                                     ("bf16", 64, False, W.MOD_NONE, False)])
def test_block_mask_atomic_dq(gpu_lib, dtype, D, causal, mod, mask):
    """Block-sparse backward with dQ from atomics in the key/value pass."""
    w, inputs = block_case(dtype, D, causal, mod, mask, wid=209)
    full_parity(w, inputs=inputs, dq_modes=("atomic",))


@pytest.mark.parametrize("causal,mod,mask", [(False, W.MOD_NONE, False), (True, W.MOD_ALIBI, False),
                                             (False, W.MOD_CHECKERBOARD, True), (True, W.MOD_NONE, True)])
def test_block_mask_f32_d512(gpu_lib, causal, mod, mask):
    w, inputs = block_case("f32", 512, causal, mod, mask, Sq=280, Skv=390, B=1, H=2, wid=201)
    full_parity(w, inputs=inputs, strict=False)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64), ("f32", 512)])
def test_block_mask_empty_rows_and_columns(gpu_lib, dtype, D):
    """Cleared blocks give exact zeros: O = 0 and lse = -inf on rows whose
    block row is empty, dQ = 0 there, dK = dV = 0 on keys whose block column
    is empty."""
    w, inputs = block_case(dtype, D, False, W.MOD_ALIBI, False, Sq=300, Skv=400, B=1, H=2, wid=202)
    full_parity(w, inputs=inputs, strict=dtype != "f32")
    dev = to_dev(inputs)
    kw = dict(score_mod="alibi", block_mask=dev["block_mask"])
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], **kw)
    torch.cuda.synchronize()
    assert torch.all(out[0, 0, 128:256] == 0) and torch.all(lse[0, 0, 128:256] == float("-inf"))
    assert torch.all(dq[0, 0, 128:256] == 0)
    assert torch.all(dk[0, 1, :128] == 0) and torch.all(dv[0, 1, :128] == 0)


@pytest.mark.parametrize("dtype,D,causal", [("f16", 64, True), ("bf16", 128, False), ("f32", 64, True),
                                            ("f32", 512, False)])
def test_full_block_mask_is_the_dense_result(gpu_lib, dtype, D, causal):
    """A block mask with every block set visits the dense tiles in the dense
    order, so every output is bitwise equal to the call without one (dQ from
    the deterministic separate pass)."""
    Sq = 333 if D < 512 else 150
    w = W.Workload("full block mask", 203, 2, 2, Sq, Sq, D, dtype, causal=causal, mod=W.MOD_ALIBI)
    dev = to_dev(w.make())
    ones = torch.ones(fa.block_mask_shape(2, 2, Sq, Sq), dtype=torch.uint8, device="cuda")
    say(f"[full block mask] {dtype} D{D} causal={causal}")
    res = []
    for bm in (None, ones):
        kw = dict(causal=causal, score_mod="alibi", block_mask=bm)
        out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
        g = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], dq_mode="separate", **kw)
        res.append((out, lse) + tuple(g))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (129, 64), (64, 129), (257, 383), (128, 256)])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_block_mask_ragged_shapes(gpu_lib, Sq, Skv, dtype):
    w, inputs = block_case(dtype, 64, False, W.MOD_CHECKERBOARD, True, Sq=Sq, Skv=Skv, B=2, H=2, wid=204)
    full_parity(w, inputs=inputs, strict=False)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("Sq", [1, 16])
def test_block_mask_decode(gpu_lib, dtype, D, Sq):
    """fa_decode (one query: the streaming kernel; 16 queries: the forward
    split over key chunks) with a block mask, against the oracle."""
    Skv = 5000
    w = W.Workload("block-sparse decode", 205, 2, 3, Sq, Skv, D, dtype, mod=W.MOD_ALIBI, key_mask=True,
                   backward=False)
    inputs = w.make()
    bm = W.bernoulli_block_mask(2, 3, Sq, Skv, 205, p_keep=0.3)
    bm[0, 0] = 0                                       # one (batch, head) sees no key at all
    inputs["block_mask"] = bm
    dev = to_dev(inputs)
    off = 7
    say(f"[block decode] {dtype} D{D} Sq{Sq} Skv{Skv}")
    out, lse = fa.decode(dev["q"], dev["k"], dev["v"], key_mask=dev["key_mask"], score_mod="alibi", q_offset=off,
                         block_mask=dev["block_mask"])
    torch.cuda.synchronize()
    okw = oracle_kw(w, inputs)
    o_ref, lse_ref = oracle.forward(inputs["q"], inputs["k"], inputs["v"], q_offset=off, **okw)
    check("decode o", out, o_ref, dtype, "o")
    check_lse(lse, lse_ref)
    assert torch.all(out[0, 0] == 0) and torch.all(lse[0, 0] == float("-inf"))


def test_block_mask_sliding_window_long(gpu_lib):
    """Prefill-style f16 causal ALiBi at 8192 tokens with a sliding window of 4
    blocks (512 keys) as the block mask: sampled rows against the oracle."""
    w = W.Workload("sliding-window f16 causal ALiBi (2,4,8192,64)", 206, 2, 4, 8192, 8192, 64, "f16",
                   causal=True, mod=W.MOD_ALIBI)
    bm = W.window_block_mask(2, 4, 8192, 8192, 4)
    sampled_parity(w, 128, block_mask=bm)


def test_block_mask_long_fp32_d512(gpu_lib):
    """The long-context fp32 shape (1, 1, 131072, 512), causal, with a
    Bernoulli(0.5) block mask: tile lists of up to about 2000 of the 4096
    32-row tiles (the longest sequence a block mask takes), on sampled rows."""
    w = W.Workload("block-sparse fp32 causal (1,1,131072,512)", 207, 1, 1, 131072, 131072, 512, "f32",
                   causal=True)
    bm = W.bernoulli_block_mask(1, 1, 131072, 131072, 207)
    sampled_parity(w, 64, block_mask=bm)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64)])
def test_block_mask_with_query_offset(gpu_lib, dtype, D):
    """Block mask plus a KV-cache offset: 300 queries at positions 100..399
    against 400 keys, causal, ALiBi.  Block rows index query ROWS (0..2), not
    positions; forward and backward against the oracle."""
    Sq, Skv, off = 300, 400, 100
    w = W.Workload("block-sparse with offset", 208, 2, 2, Sq, Skv, D, dtype, causal=True, mod=W.MOD_ALIBI)
    inputs = w.make()
    bm = W.bernoulli_block_mask(2, 2, Sq, Skv, 208, p_keep=0.6)
    bm[..., 0] = 1   # key block 0 is allowed for every row (no query row is empty)
    inputs["block_mask"] = bm
    dev = to_dev(inputs)
    kw = dict(causal=True, score_mod="alibi", q_offset=off, block_mask=dev["block_mask"])
    say(f"[block offset] {dtype} D{D}")
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], **kw)
    torch.cuda.synchronize()
    okw = dict(oracle_kw(w, inputs), q_offset=off)
    check_case(dtype, inputs, okw, out, lse, (dq, dk, dv), strict=dtype != "f32")
