"""GPU parity on a seeded random sample of the option space: dtype, head_dim,
ragged sequence lengths, causal with a query offset, score_mod, key mask and
block mask, forward and backward, each case against the fp64 oracle.

The cases are drawn once from a fixed seed (the list is the same on every
run).  Bars as elsewhere: 16-bit max-abs-err / max|ref| <= 2e-2 (O) and 5e-2
(gradients); fp32 1e-4 (O) and 1e-5 (gradients) absolute, or, where random
masks leave a row a handful of keys and dK, dV grow past 1, the per-element
bound derived from the accumulation (tests/bounds.py); lse within
1e-3 + 1e-5 |lse|.
"""
import numpy as np
import pytest
import torch

import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from parity import MOD_NAME, check_case, say, to_dev

pytestmark = pytest.mark.gpu


def draw_cases(n=28, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["f16", "bf16", "f32"][rng.integers(3)]
        D = int(rng.choice([64, 128] if dtype != "f32" else [64, 128, 512]))
        Sq = int(rng.integers(1, 300 if D < 512 else 140))
        causal = bool(rng.integers(2))
        off = int(rng.integers(0, 150)) if causal and rng.integers(2) else 0
        Skv = Sq + off if causal else int(rng.integers(1, 400 if D < 512 else 160))
        cases.append(dict(id=300 + i, dtype=dtype, D=D, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                          Sq=Sq, Skv=Skv, causal=causal, off=off, mod=int(rng.integers(3)),
                          mask=bool(rng.integers(2)), block=bool(rng.integers(2))))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c['dtype']}-D{c['D']}-{c['Sq']}x{c['Skv']}-c{int(c['causal'])}"
                                             f"o{c['off']}-m{c['mod']}-k{int(c['mask'])}-b{int(c['block'])}"
                                             for c in CASES])
def test_random_config(gpu_lib, case):
    c = case
    w = W.Workload("random", c["id"], c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"], causal=c["causal"],
                   mod=c["mod"], key_mask=c["mask"])
    inputs = w.make()
    if c["block"]:
        inputs["block_mask"] = W.bernoulli_block_mask(c["B"], c["H"], c["Sq"], c["Skv"], c["id"], p_keep=0.7)
    dev = to_dev(inputs)
    say(f"[random] {c}")
    kw = dict(causal=c["causal"], score_mod=MOD_NAME[c["mod"]], scale=w.scale, q_offset=c["off"],
              key_mask=dev.get("key_mask"), block_mask=dev.get("block_mask"))
    out, lse = fa.forward(dev["q"], dev["k"], dev["v"], **kw)
    # 16-bit cases alternate between the two dQ modes
    mode = "separate" if c["dtype"] == "f32" or c["id"] % 2 else "atomic"
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], out, lse, dev["dout"], dq_mode=mode, **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w.scale, causal=c["causal"], mod=c["mod"], q_offset=c["off"],
               key_mask=None if inputs.get("key_mask") is None else inputs["key_mask"].numpy(),
               block_mask=None if inputs.get("block_mask") is None else inputs["block_mask"].numpy() != 0)
    check_case(c["dtype"], inputs, okw, out, lse, (dq, dk, dv), strict=False)
