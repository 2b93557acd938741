"""The forward split over the key axis (fa_forward_split): every (query
block, key chunk) pair writes an unnormalised partial per row and a second
kernel merges a row's partials exactly.  Same bars as the forward: fp32
max-abs-err <= 1e-4 on O (the derived per-element bound on ragged shapes);
f16/bf16 max-abs-err / max|ref| <= 2e-2 on O and <= 5e-2 on each gradient of
the backward that uses the split forward's lse; lse within 1e-3 + 1e-5 |lse|.
"""
import pytest
import torch

import oracle
import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from parity import MOD_NAME, check, check_case, check_lse, sampled_parity, say, to_dev

pytestmark = pytest.mark.gpu

# dtype, D, causal, mod, key mask, block mask, Sq, Skv, q_offset, kv_splits
CASES = [
    ("f16", 64, True, W.MOD_ALIBI, False, False, 700, 700, 0, 3),
    ("bf16", 128, False, W.MOD_CHECKERBOARD, True, False, 300, 900, 0, 5),
    ("f16", 128, True, W.MOD_NONE, True, True, 333, 1000, 667, 4),
    ("bf16", 64, True, W.MOD_CHECKERBOARD, False, True, 520, 520, 0, 7),
    ("f16", 64, False, W.MOD_NONE, False, False, 129, 1300, 0, 16),
    ("f32", 64, True, W.MOD_ALIBI, False, False, 450, 450, 0, 3),
    ("f32", 128, False, W.MOD_NONE, True, True, 260, 700, 0, 4),
    ("f32", 64, True, W.MOD_CHECKERBOARD, True, False, 200, 900, 700, 6),
    # query blocks of <= 32 and 33..64 rows: the one- and two-wave fp32 workgroups
    ("f32", 64, False, W.MOD_ALIBI, True, False, 24, 3000, 0, 5),
    ("f32", 128, True, W.MOD_NONE, False, False, 40, 5000, 4960, 7),
    ("f32", 64, True, W.MOD_CHECKERBOARD, False, False, 64, 2000, 1936, 3),
]


def _kw(w, dev, off, bm):
    return dict(causal=w.causal, score_mod=MOD_NAME[w.mod], scale=w.scale, key_mask=dev.get("key_mask"),
                q_offset=off, block_mask=None if bm is None else bm.cuda())


@pytest.mark.parametrize("dtype,D,causal,mod,mask,blk,Sq,Skv,off,n", CASES)
def test_forward_split_matches_oracle(gpu_lib, dtype, D, causal, mod, mask, blk, Sq, Skv, off, n):
    """An explicit chunk count on ragged shapes spanning several query blocks
    and chunks: O and lse against the oracle, the backward from the split
    forward's lse against the oracle, and the split forward against the
    unsplit one."""
    w = W.Workload(f"split {dtype} D{D}", 140, 2, 2, Sq, Skv, D, dtype, causal=causal, mod=mod, key_mask=mask)
    x = w.make()
    bm = W.bernoulli_block_mask(2, 2, Sq, Skv, 140, p_keep=0.7) if blk else None
    dev = to_dev(x)
    kw = _kw(w, dev, off, bm)
    p = fa.problem(dev["q"], dev["k"], causal=causal, key_mask=kw["key_mask"], score_mod=kw["score_mod"],
                   scale=w.scale, q_offset=off, block_mask=kw["block_mask"], kv_splits=n)
    assert fa.forward_split_workspace_bytes(p) > 0, "the case must take the split path"
    say(f"[split] {dtype} D{D} causal={causal} mod={mod} mask={mask} blk={blk} Sq={Sq} Skv={Skv} off={off} n={n}")
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], kv_splits=n, **kw)
    grads = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], **kw)
    out_u, lse_u = fa.forward(dev["q"], dev["k"], dev["v"], kv_splits=1, **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=causal, mod=mod, q_offset=off,
               key_mask=None if x.get("key_mask") is None else x["key_mask"].numpy(),
               block_mask=None if bm is None else bm.numpy() != 0)
    check_case(dtype, x, okw, out, lse, grads, strict=dtype != "f32")
    fin = torch.isfinite(lse_u)
    assert torch.equal(torch.isfinite(lse), fin)
    assert (lse[fin] - lse_u[fin]).abs().max().item() <= 1e-4
    scale = out_u.float().abs().max().item() or 1.0
    assert (out.float() - out_u.float()).abs().max().item() / scale <= (1e-5 if dtype == "f32" else 1e-2)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,B,H,S,D,dtype,causal,mod,mask", [
    ("long causal", 1, 2, 16384, 128, "f16", True, W.MOD_ALIBI, False),
    ("long keys masked", 1, 1, 16384, 64, "bf16", False, W.MOD_CHECKERBOARD, True),
])
def test_forward_split_chosen_by_the_table(gpu_lib, name, B, H, S, D, dtype, causal, mod, mask):
    """Shapes whose query blocks alone leave the device idle: forward() takes
    the split path by itself (the library's per-shape choice); O, lse and dQ
    on sampled rows and every dK, dV row (sparse dO) against the oracle."""
    w = W.Workload(f"split table {name}", 141, B, H, S, S, D, dtype, causal=causal, mod=mod, key_mask=mask)
    q = torch.empty(w.q_shape(), dtype=W.torch_dtype(dtype), device="cuda")
    km = torch.ones((B, S), dtype=torch.uint8, device="cuda") if mask else None
    p = fa.problem(q, q, causal=causal, key_mask=km, score_mod=MOD_NAME[mod], scale=w.scale)
    assert fa.forward_split_workspace_bytes(p) > 0, "the table must split this shape"
    del q
    sampled_parity(w, 128)
