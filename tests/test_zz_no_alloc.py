"""fa_decode_noalloc (fixed per-device scratch, no workspace argument)
against fa_decode (caller workspace) on the same inputs: two calls in a row,
the second smaller than the first, each against the oracle too.  Runs last:
it leaves the scratch holding the partials of its last call."""
import pytest
import torch

import oracle
import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from parity import check, check_lse, say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, H, Sq, Skv, D, dtype, wid, mod, mask, causal):
    w = W.Workload("noalloc decode", wid, B, H, Sq, Skv, D, dtype, mod=mod, key_mask=mask, backward=False)
    x = w.make()
    dev = to_dev(x)
    name = {W.MOD_NONE: None, W.MOD_ALIBI: "alibi", W.MOD_CHECKERBOARD: "checkerboard"}[mod]
    off = Skv - Sq
    kw = dict(score_mod=name, scale=w.scale, key_mask=dev.get("key_mask"), q_offset=off, causal=causal)
    say(f"[noalloc] {dtype} B{B} H{H} Sq{Sq} Skv{Skv} D{D} mod={mod} mask={mask} causal={causal}")
    o_ws, l_ws = fa.decode(dev["q"], dev["k"], dev["v"], **kw)
    o_na, l_na = fa.decode_noalloc(dev["q"], dev["k"], dev["v"], **kw)
    torch.cuda.synchronize()
    o_r, lse_r = oracle.forward(x["q"], x["k"], x["v"], scale=w.scale, mod=mod, q_offset=off, causal=causal,
                                key_mask=None if x.get("key_mask") is None else x["key_mask"].numpy())
    check("noalloc o", o_na, o_r, dtype, "o")
    check_lse(l_na, lse_r)
    # same kernels, same key split, same inputs: the same bits as fa_decode
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128), ("f32", 64)])
def test_decode_noalloc_matches_decode_twice(gpu_lib, dtype, D):
    # a larger call, then a smaller one (fewer heads, keys and chunks): the
    # second must not see the first one's partials
    _case(4, 8, 1, 9000, D, dtype, 150, W.MOD_ALIBI, True, False)
    _case(2, 3, 1, 700, D, dtype, 151, W.MOD_CHECKERBOARD, False, False)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_noalloc_short_query_block_twice(gpu_lib, dtype):
    """Short query blocks (the key-split forward plus the merge), larger then smaller."""
    _case(2, 4, 32, 6000, 64, dtype, 152, W.MOD_ALIBI, False, True)
    _case(1, 2, 5, 900, 64, dtype, 153, W.MOD_NONE, True, True)
