"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test checks the oracle against something the definition or mathematics
fixes: hand-worked values, closed forms (uniform scores, geometric series for
ALiBi, parity counts for the checkerboard), central finite differences of the
analytic backward, invariants, and an independent library attention routine
(torch's fp64 CPU ``scaled_dot_product_attention`` with autograd).
"""
import json
import sys
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import MOD_ALIBI, MOD_CHECKERBOARD, MOD_NONE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _eval_expr(s):
    env = {"e": math.e, "exp": math.exp, "log": math.log, "__builtins__": {}}
    return float(eval(str(s), env))  # expressions from the hand-worked fixture only


def _eval_tree(x):
    if isinstance(x, list):
        return [_eval_tree(y) for y in x]
    return _eval_expr(x)


# --------------------------------------------------------------------------- golden


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"][:40])
def test_hand_worked_examples(case):
    q, k, v = (np.array(case[n], dtype=np.float64) for n in ("q", "k", "v"))
    km = None if case["key_mask"] is None else np.array(case["key_mask"])
    kw = dict(scale=case["scale"], causal=case["causal"], key_mask=km, mod=case["mod"])
    o, lse = oracle.forward(q, k, v, **kw)
    np.testing.assert_allclose(o, np.array(_eval_tree(case["o"])), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(_eval_tree(case["lse"])), rtol=0, atol=1e-14)
    if "dout" in case:
        dq, dk, dv = oracle.backward(q, k, v, np.array(case["dout"], dtype=np.float64), **kw)
        np.testing.assert_allclose(dq, np.array(_eval_tree(case["dq"])), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dk, np.array(_eval_tree(case["dk"])), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dv, np.array(_eval_tree(case["dv"])), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- closed forms


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_uniform_scores_give_mean_of_v():
    B, H, Sq, Skv, D = 2, 3, 7, 11, 5
    q = np.zeros((B, H, Sq, D))
    k, v = _rand((B, H, Skv, D), 1), _rand((B, H, Skv, D), 2)
    o, lse = oracle.forward(q, k, v, scale=0.37)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(Skv), atol=1e-14)


def test_uniform_scores_with_key_mask_give_mean_of_kept_v():
    B, H, Sq, Skv, D = 2, 2, 4, 9, 3
    q = np.zeros((B, H, Sq, D))
    k, v = _rand((B, H, Skv, D), 3), _rand((B, H, Skv, D), 4)
    km = np.array([[1, 0, 1, 1, 0, 0, 1, 0, 1], [0, 0, 0, 1, 0, 0, 0, 0, 0]], dtype=np.uint8)
    o, lse = oracle.forward(q, k, v, scale=1.0, key_mask=km)
    for b in range(B):
        kept = km[b] != 0
        np.testing.assert_allclose(o[b], np.broadcast_to(v[b][:, kept].mean(axis=1, keepdims=True), o[b].shape), atol=1e-14)
        np.testing.assert_allclose(lse[b], math.log(kept.sum()), atol=1e-14)


def test_causal_uniform_scores_give_cumulative_mean():
    B, H, S, D = 1, 2, 13, 4
    q = np.zeros((B, H, S, D))
    k, v = _rand((B, H, S, D), 5), _rand((B, H, S, D), 6)
    o, lse = oracle.forward(q, k, v, scale=0.5, causal=True)
    cum = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    np.testing.assert_allclose(o, cum, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, S + 1))[None, None, :].repeat(H, 1), atol=1e-14)


def test_causal_row_zero_is_single_key():
    q, k, v = _rand((1, 1, 6, 4), 7), _rand((1, 1, 6, 4), 8), _rand((1, 1, 6, 4), 9)
    o, lse = oracle.forward(q, k, v, scale=0.3, causal=True)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 0.3 * q[0, 0, 0] @ k[0, 0, 0], atol=1e-15)


@pytest.mark.parametrize("mod", [MOD_NONE, MOD_ALIBI, MOD_CHECKERBOARD])
def test_single_kept_key(mod):
    B, H, Sq, Skv, D = 1, 2, 5, 8, 3
    q, k, v = _rand((B, H, Sq, D), 10), _rand((B, H, Skv, D), 11), _rand((B, H, Skv, D), 12)
    do = _rand((B, H, Sq, D), 13)
    j = 5
    km = np.zeros((B, Skv), dtype=np.uint8)
    km[0, j] = 1
    o, lse = oracle.forward(q, k, v, scale=0.4, key_mask=km, mod=mod)
    dq, dk, dv = oracle.backward(q, k, v, do, scale=0.4, key_mask=km, mod=mod)
    for h in range(H):
        np.testing.assert_allclose(o[0, h], np.broadcast_to(v[0, h, j], (Sq, D)), atol=1e-15)
        bias = oracle.score_bias(mod, h, np.arange(Sq), np.array([j]), H)[:, 0]
        np.testing.assert_allclose(lse[0, h], 0.4 * q[0, h] @ k[0, h, j] + bias, atol=1e-14)
    np.testing.assert_allclose(dq, 0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, atol=1e-15)
    exp_dv = np.zeros_like(dv)
    exp_dv[:, :, j] = do.sum(axis=2)
    np.testing.assert_allclose(dv, exp_dv, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_alibi_geometric_series(causal):
    """q = 0: s_ij = -slope (i - j); weights are powers of r = exp(-slope)."""
    H, S = 4, 37
    q = np.zeros((1, H, S, 2))
    k = _rand((1, H, S, 2), 14)
    j = np.arange(S, dtype=np.float64)
    v = np.zeros((1, H, S, 2))
    v[..., 0] = 1.0
    v[..., 1] = j
    o, lse = oracle.forward(q, k, v, scale=1.0, causal=causal, mod=MOD_ALIBI)
    for h in range(H):
        slope = 2.0 ** (-8.0 * (h + 1) / H)
        r = math.exp(-slope)
        for i in range(S):
            n_back = i + 1                      # keys j <= i: weights r^0 .. r^i
            z_back = (1 - r ** n_back) / (1 - r)
            m_back = r * (1 - n_back * r ** (n_back - 1) + (n_back - 1) * r ** n_back) / (1 - r) ** 2
            z, num = z_back, i * z_back - m_back  # sum_j j w_j with j = i - t
            if not causal:
                n_fwd = S - 1 - i               # keys j > i: weights (1/r)^1 .. (1/r)^n_fwd
                g = 1.0 / r
                z_fwd = g * (g ** n_fwd - 1) / (g - 1) if n_fwd else 0.0
                # sum_{t=1}^{n} t g^t = g (1 - (n+1) g^n + n g^(n+1)) / (1-g)^2
                m_fwd = g * (1 - (n_fwd + 1) * g ** n_fwd + n_fwd * g ** (n_fwd + 1)) / (1 - g) ** 2
                z += z_fwd
                num += i * z_fwd + m_fwd
            assert abs(lse[0, h, i] - math.log(z)) < 1e-12
            assert abs(o[0, h, i, 1] - num / z) < 1e-9 * max(1.0, abs(num / z))
            assert abs(o[0, h, i, 0] - 1.0) < 1e-14


def test_alibi_row_shift_invariance():
    """The -slope*q_idx part is constant along a row: O is unchanged and lse
    moves by exactly that constant when it is dropped."""
    B, H, S, D = 1, 3, 9, 4
    q, k, v = _rand((B, H, S, D), 15), _rand((B, H, S, D), 16), _rand((B, H, S, D), 17)
    o1, lse1 = oracle.forward(q, k, v, scale=0.5, mod=MOD_ALIBI)
    o0, lse0 = oracle.forward(q, k, v, scale=0.5)
    slopes = oracle.default_alibi_slopes(H)
    # reference: add slope*j through the key side by augmenting q, k with one extra dim
    qa = np.concatenate([q, np.ones((B, H, S, 1))], axis=-1)
    ka = np.concatenate([k, (slopes[None, :, None, None] / 0.5) * np.arange(S)[None, None, :, None]], axis=-1)
    o2, lse2 = oracle.forward(qa, ka, v, scale=0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    i = np.arange(S)
    np.testing.assert_allclose(lse1, lse2 - slopes[None, :, None] * i[None, None, :], atol=1e-12)
    assert np.abs(o1 - o0).max() > 1e-3  # the bias does change the result


@pytest.mark.parametrize("Skv", [10, 11])
def test_checkerboard_counts(Skv):
    """q = 0, non-causal: s_ij = +0.5 on even (i+j), -0.5 on odd."""
    Sq = 6
    q = np.zeros((1, 1, Sq, 1))
    k = _rand((1, 1, Skv, 1), 18)
    v = ((-1.0) ** np.arange(Skv)).reshape(1, 1, Skv, 1)
    o, lse = oracle.forward(q, k, v, scale=1.0, mod=MOD_CHECKERBOARD)
    n_even_j = (Skv + 1) // 2
    n_odd_j = Skv // 2
    for i in range(Sq):
        # keys with (i+j) even: j even when i is even, j odd when i is odd
        n_plus = n_even_j if i % 2 == 0 else n_odd_j
        n_minus = Skv - n_plus
        z = n_plus * math.exp(0.5) + n_minus * math.exp(-0.5)
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-14
        sign_plus = 1.0 if i % 2 == 0 else -1.0   # v_j = (-1)^j, and (-1)^j = (-1)^i on the + keys
        expect = sign_plus * (n_plus * math.exp(0.5) - n_minus * math.exp(-0.5)) / z
        assert abs(o[0, 0, i, 0] - expect) < 1e-14


# --------------------------------------------------------------------------- invariants


COMBOS = [(c, m, km) for c in (False, True) for m in (MOD_NONE, MOD_ALIBI, MOD_CHECKERBOARD)
          for km in (False, True)]


def _case(seed, B=2, H=2, Sq=6, Skv=6, D=3, key_mask=False, keep_all_first=True):
    q, k, v = _rand((B, H, Sq, D), seed), _rand((B, H, Skv, D), seed + 1), _rand((B, H, Skv, D), seed + 2)
    do = _rand((B, H, Sq, D), seed + 3)
    km = None
    if key_mask:
        km = (np.random.default_rng(seed + 4).random((B, Skv)) < 0.6).astype(np.uint8)
        km[:, 0] = 1 if keep_all_first else km[:, 0]
    return q, k, v, do, km


@pytest.mark.parametrize("causal,mod,use_mask", COMBOS)
def test_ones_v_gives_ones(causal, mod, use_mask):
    q, k, _, _, km = _case(20, key_mask=use_mask)
    v = np.ones((2, 2, 6, 3))
    o, _ = oracle.forward(q, k, v, scale=0.7, causal=causal, key_mask=km, mod=mod)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)


def test_masked_key_with_garbage_is_ignored():
    B, H, Sq, Skv, D = 1, 2, 5, 9, 4
    q, k, v = _rand((B, H, Sq, D), 21), _rand((B, H, Skv, D), 22), _rand((B, H, Skv, D), 23)
    km = np.ones((B, Skv), dtype=np.uint8)
    km[0, 3] = 0
    km[0, 7] = 0
    k2, v2 = k.copy(), v.copy()
    k2[:, :, [3, 7]] = 1e4
    v2[:, :, [3, 7]] = -3e5
    o, lse = oracle.forward(q, k2, v2, scale=0.5, key_mask=km)
    keep = [j for j in range(Skv) if km[0, j]]
    o_ref, lse_ref = oracle.forward(q, k[:, :, keep], v[:, :, keep], scale=0.5)
    np.testing.assert_allclose(o, o_ref, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-14)


@pytest.mark.parametrize("causal,mod,use_mask", COMBOS)
def test_backward_invariants(causal, mod, use_mask):
    q, k, v, do, km = _case(30, key_mask=use_mask)
    o, _ = oracle.forward(q, k, v, scale=0.6, causal=causal, key_mask=km, mod=mod)
    dq, dk, dv = oracle.backward(q, k, v, do, scale=0.6, causal=causal, key_mask=km, mod=mod)
    # every row keeps key 0 here, so every row has an allowed key
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-13)
    assert np.isfinite(o).all()


def test_fully_masked_row_is_empty_sum():
    B, H, S, D = 1, 1, 4, 3
    q, k, v, do = (_rand((B, H, S, D), 40 + i) for i in range(4))
    km = np.array([[0, 1, 1, 1]], dtype=np.uint8)   # row 0 (causal) sees only key 0, which is masked
    o, lse = oracle.forward(q, k, v, scale=1.0, causal=True, key_mask=km)
    assert np.all(o[0, 0, 0] == 0.0) and lse[0, 0, 0] == -np.inf
    dq, dk, dv = oracle.backward(q, k, v, do, scale=1.0, causal=True, key_mask=km)
    assert np.all(dq[0, 0, 0] == 0.0)
    # rows 1..3 are unaffected by row 0's empty sum: compare with the row subset
    o_r, lse_r = oracle.forward(q, k, v, scale=1.0, causal=True, key_mask=km, rows=[1, 2, 3])
    np.testing.assert_allclose(o[0, 0, 1:], o_r[0, 0], atol=0)
    assert np.isfinite(lse[0, 0, 1:]).all()


# --------------------------------------------------------------------------- calculus


def _loss(q, k, v, do, kw):
    o, _ = oracle.forward(q, k, v, **kw)
    return float((o * do).sum())


@pytest.mark.parametrize("causal,mod,use_mask", COMBOS)
def test_gradients_match_central_differences(causal, mod, use_mask):
    B, H, S, D = 1, 2, 5, 3
    q, k, v, do, km = _case(50, B=B, H=H, Sq=S, Skv=S, D=D, key_mask=use_mask)
    kw = dict(scale=0.8, causal=causal, key_mask=km, mod=mod)
    dq, dk, dv = oracle.backward(q, k, v, do, **kw)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, kw)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, kw)) / (2 * h)
        np.testing.assert_allclose(g, num, atol=1e-8, err_msg=f"d{name}")


def _torch_bias(mod, B, H, Sq, Skv, causal, km, q_offset=0):
    """Additive float mask for torch SDPA, written independently of the oracle
    (query row i at position i + q_offset)."""
    i = torch.arange(Sq, dtype=torch.float64)[:, None] + q_offset
    j = torch.arange(Skv, dtype=torch.float64)[None, :]
    bias = torch.zeros(B, H, Sq, Skv, dtype=torch.float64)
    if mod == MOD_ALIBI:
        slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float64)
        bias = bias + (slopes[:, None, None] * (j - i))[None]
    elif mod == MOD_CHECKERBOARD:
        bias = bias + torch.where(((i + j) % 2) == 0, 0.5, -0.5)[None, None]
    neg = torch.zeros(B, 1, Sq, Skv, dtype=torch.float64)
    if causal:
        neg = neg.masked_fill(j > i, float("-inf"))
    if km is not None:
        neg = neg.masked_fill(torch.from_numpy(km == 0)[:, None, None, :], float("-inf"))
    return bias + neg


@pytest.mark.parametrize("causal,mod,use_mask", COMBOS)
@pytest.mark.parametrize("shape", [(2, 3, 33, 33, 16, 0), (1, 2, 17, 40, 8, 0), (1, 2, 17, 40, 8, 23),
                                   (1, 2, 17, 40, 8, 9)])
def test_against_torch_sdpa_fp64(causal, mod, use_mask, shape):
    B, H, Sq, Skv, D, off = shape
    q, k, v, do, km = _case(60, B=B, H=H, Sq=Sq, Skv=Skv, D=D, key_mask=use_mask)
    scale = 1.0 / math.sqrt(D)
    kw = dict(scale=scale, causal=causal, key_mask=km, mod=mod, q_offset=off)
    o, lse = oracle.forward(q, k, v, **kw)
    dq, dk, dv = oracle.backward(q, k, v, do, **kw)

    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = _torch_bias(mod, B, H, Sq, Skv, causal, km, off)
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    # lse against torch's logsumexp of the masked, biased scores
    s = torch.matmul(torch.from_numpy(q), torch.from_numpy(k).transpose(-1, -2)) * scale + mask
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


# --------------------------------------------------------------------------- query offsets


@pytest.mark.parametrize("causal,mod,use_mask", COMBOS)
def test_offset_rows_are_the_tail_of_the_full_run(causal, mod, use_mask):
    """Query rows placed at positions q_offset.. of a key sequence give the
    same outputs as the same rows inside the full-length problem: the
    attention of a query depends only on its position, its vector and the
    keys (a KV cache of q_offset keys)."""
    S, Sq = 20, 7
    off = S - Sq
    q, k, v, do, km = _case(90, B=1, H=3, Sq=S, Skv=S, D=4, key_mask=use_mask)
    kw = dict(scale=0.6, causal=causal, key_mask=km, mod=mod)
    o, lse = oracle.forward(q, k, v, **kw)
    o_t, lse_t = oracle.forward(q[:, :, off:], k, v, q_offset=off, **kw)
    np.testing.assert_allclose(o_t, o[:, :, off:], atol=1e-14)
    np.testing.assert_allclose(lse_t, lse[:, :, off:], atol=1e-14)
    do_tail = np.zeros_like(do)
    do_tail[:, :, off:] = do[:, :, off:]
    dq, dk, dv = oracle.backward(q, k, v, do_tail, **kw)
    dq_t, dk_t, dv_t = oracle.backward(q[:, :, off:], k, v, do[:, :, off:], q_offset=off, **kw)
    np.testing.assert_allclose(dq_t, dq[:, :, off:], atol=1e-14)
    np.testing.assert_allclose(dk_t, dk, atol=1e-14)
    np.testing.assert_allclose(dv_t, dv, atol=1e-14)


@pytest.mark.parametrize("mod", [MOD_NONE, MOD_ALIBI, MOD_CHECKERBOARD])
def test_decode_with_offset_is_a_causal_row(mod):
    """Decoding the query at position p with causal masking equals row p of
    the full causal forward (keys after p ignored, score_mod at position p)."""
    q, k, v, _, _ = _case(95, B=2, H=2, Sq=12, Skv=12, D=5)
    o, lse = oracle.forward(q, k, v, scale=0.5, causal=True, mod=mod)
    for p in (0, 5, 11):
        od, lsed = oracle.decode(q[:, :, p:p + 1], k, v, scale=0.5, mod=mod, q_offset=p, causal=True)
        np.testing.assert_allclose(od[:, :, 0], o[:, :, p], atol=1e-14)
        np.testing.assert_allclose(lsed[:, :, 0], lse[:, :, p], atol=1e-14)


# --------------------------------------------------------------------------- block masks


def _block_mask(B, H, Sq, Skv, seed):
    """Random 128 x 128 block mask that keeps block (r, 0) for every row block."""
    nq, nk = -(-Sq // 128), -(-Skv // 128)
    bm = np.random.default_rng(seed).random((B, H, nq, nk)) < 0.5
    bm[..., 0] = True
    return bm


@pytest.mark.parametrize("causal,mod,use_mask", [(False, MOD_NONE, False), (True, MOD_ALIBI, False),
                                                 (False, MOD_CHECKERBOARD, True), (True, MOD_NONE, True)])
def test_block_mask_against_torch_sdpa(causal, mod, use_mask):
    """The block mask removes whole 128 x 128 (query row, key) blocks; checked
    against torch SDPA with the block mask expanded to elements."""
    B, H, Sq, Skv, D = 1, 2, 300, 400, 8
    q, k, v, do, km = _case(97, B=B, H=H, Sq=Sq, Skv=Skv, D=D, key_mask=use_mask)
    bm = _block_mask(B, H, Sq, Skv, 98)
    kw = dict(scale=0.35, causal=causal, key_mask=km, mod=mod, q_offset=Skv - Sq if causal else 0, block_mask=bm)
    o, lse = oracle.forward(q, k, v, **kw)
    dq, dk, dv = oracle.backward(q, k, v, do, **kw)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = _torch_bias(mod, B, H, Sq, Skv, causal, km, Skv - Sq if causal else 0)
    elem = torch.from_numpy(bm).repeat_interleave(128, dim=2)[:, :, :Sq].repeat_interleave(128, dim=3)[..., :Skv]
    mask = mask.masked_fill(~elem, float("-inf"))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.35)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    s_ = torch.matmul(torch.from_numpy(q), torch.from_numpy(k).transpose(-1, -2)) * 0.35 + mask
    np.testing.assert_allclose(lse, torch.logsumexp(s_, dim=-1).numpy(), atol=1e-12)


def test_full_block_mask_changes_nothing():
    q, k, v, do, _ = _case(99, B=1, H=2, Sq=200, Skv=260, D=4)
    bm = np.ones((1, 2, 2, 3), dtype=bool)
    for causal in (False, True):
        kw = dict(scale=0.5, causal=causal, mod=MOD_ALIBI, q_offset=60 if causal else 0)
        o, lse = oracle.forward(q, k, v, **kw)
        o2, lse2 = oracle.forward(q, k, v, block_mask=bm, **kw)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)


# --------------------------------------------------------------------------- row subsets


@pytest.mark.parametrize("causal,mod,use_mask", [(True, MOD_ALIBI, False), (False, MOD_CHECKERBOARD, True)])
def test_row_subset_matches_full_and_sparse_dout(causal, mod, use_mask):
    q, k, v, do, km = _case(70, B=1, H=2, Sq=24, Skv=24, D=4, key_mask=use_mask)
    kw = dict(scale=0.5, causal=causal, key_mask=km, mod=mod)
    rows = [0, 3, 11, 23]
    o, lse = oracle.forward(q, k, v, **kw)
    o_r, lse_r = oracle.forward(q, k, v, rows=rows, **kw)
    np.testing.assert_allclose(o_r, o[:, :, rows], atol=1e-15)
    np.testing.assert_allclose(lse_r, lse[:, :, rows], atol=1e-15)
    dq, _, _ = oracle.backward(q, k, v, do, **kw)
    do_sparse = np.zeros_like(do)
    do_sparse[:, :, rows] = do[:, :, rows]
    _, dk_s, dv_s = oracle.backward(q, k, v, do_sparse, **kw)
    dq_r, dk_r, dv_r = oracle.backward(q, k, v, do, rows=rows, **kw)
    np.testing.assert_allclose(dq_r, dq[:, :, rows], atol=1e-14)
    np.testing.assert_allclose(dk_r, dk_s, atol=1e-14)
    np.testing.assert_allclose(dv_r, dv_s, atol=1e-14)


def test_decode_is_forward_at_one_query():
    q, k, v = _rand((2, 3, 1, 8), 80), _rand((2, 3, 50, 8), 81), _rand((2, 3, 50, 8), 82)
    o, lse = oracle.decode(q, k, v, scale=0.25)
    qa = np.zeros((2, 3, 1, 8)) + q
    tq, tk, tv = (torch.from_numpy(x) for x in (qa, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.25)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-14)


# --------------------------------------------------------------------------- planted mistakes


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (on the CPU) and check that the
    pins above reject each of them."""
    import oracle.attention as A
    case = json.load(open(GOLDEN))["cases"]

    def run_golden():
        for c in case:
            test_hand_worked_examples(c)

    # 1) ALiBi sign flipped
    orig_bias = A.score_bias

    def flipped(mod, *a, **kw):
        b = orig_bias(mod, *a, **kw)
        return -b if mod == MOD_ALIBI else b
    monkeypatch.setattr(A, "score_bias", flipped)
    with pytest.raises(AssertionError):
        test_alibi_geometric_series(True)
    monkeypatch.setattr(A, "score_bias", orig_bias)

    # 2) scale applied to the bias as well as the dot product
    orig_probs = A._probabilities

    def scaled_bias(qb, kb, scale, bias, ok):
        return orig_probs(qb, kb, scale, scale * bias, ok)
    monkeypatch.setattr(A, "_probabilities", scaled_bias)
    with pytest.raises(AssertionError):
        run_golden()
    monkeypatch.setattr(A, "_probabilities", orig_probs)

    # 3) causal mask transposed (j >= i instead of j <= i)
    orig_allowed = A.allowed_pairs

    def transposed(q_idx, seq_kv, causal, km):
        ok = orig_allowed(q_idx, seq_kv, False, km)
        if causal:
            ok &= np.arange(seq_kv)[None, :] >= np.asarray(q_idx)[:, None]
        return ok
    monkeypatch.setattr(A, "allowed_pairs", transposed)
    with pytest.raises(AssertionError):
        test_causal_uniform_scores_give_cumulative_mean()
    monkeypatch.setattr(A, "allowed_pairs", orig_allowed)

    # 4) backward without the D_i term
    def bad_backward(q, k, v, dout, *, scale, causal=False, key_mask=None, mod=0,
                     alibi_slopes=None, checker=(0.5, -0.5), rows=None):
        q, k, v, rows, km = A._setup(q, k, v, rows, key_mask)
        do = A.as_f64(dout)
        B, H, _, D = q.shape
        dq = np.zeros((B, H, len(rows), D))
        dk, dv = np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            ok = A.allowed_pairs(rows, k.shape[2], causal, None if km is None else km[b])
            for h in range(H):
                bias = A.score_bias(mod, h, rows, np.arange(k.shape[2]), H, alibi_slopes, checker)
                _, _, p = A._probabilities(q[b, h, rows], k[b, h], scale, bias, ok)
                ds = p * (do[b, h, rows] @ v[b, h].T)
                dq[b, h] = scale * ds @ k[b, h]
                dk[b, h] = scale * ds.T @ q[b, h, rows]
                dv[b, h] = p.T @ do[b, h, rows]
        return dq, dk, dv
    monkeypatch.setattr(oracle, "backward", bad_backward)
    with pytest.raises(AssertionError):
        test_gradients_match_central_differences(False, MOD_NONE, False)


# --------------------------------------------------------------------------- error magnitudes

from bounds import U32, kappa, within  # noqa: E402


def _mag_case(causal, mod, use_mask, B=2, H=2, Sq=9, Skv=13, D=6, seed=70):
    q, k, v, do = (_rand((B, H, Sq if i in (0, 3) else Skv, D), seed + i) for i in range(4))
    km = None
    if use_mask:
        km = (np.random.default_rng(seed + 9).random((B, Skv)) < 0.6).astype(np.uint8)
        km[:, 0] = 1
    if causal:
        Skv = Sq
        k, v = k[:, :, :Sq], v[:, :, :Sq]
        km = None if km is None else km[:, :Sq]
    kw = dict(scale=0.4, causal=causal, mod=mod, key_mask=km)
    return q, k, v, do, kw


@pytest.mark.parametrize("causal,mod,use_mask", [(False, MOD_NONE, False), (True, MOD_ALIBI, False),
                                                 (False, MOD_CHECKERBOARD, True), (True, MOD_NONE, True)])
def test_magnitudes_bound_the_results(causal, mod, use_mask):
    """Every magnitude is at least the absolute value of the result it
    belongs to (triangle inequality on the same sums)."""
    q, k, v, do, kw = _mag_case(causal, mod, use_mask)
    o, _ = oracle.forward(q, k, v, **kw)
    g = oracle.backward(q, k, v, do, **kw)
    for m, r in zip(oracle.magnitudes(q, k, v, do, **kw), (o,) + tuple(g)):
        assert np.all(m >= np.abs(r) - 1e-12)


def test_magnitudes_closed_forms():
    """q = 0 and v >= 0 with no score_mod: every score is 0, so a_ij = 0,
    r_ij = 1 and M_o equals O = mean of V exactly; dO >= 0 makes M_dv = dV.
    A single kept key j*: P is one-hot, r = 1 + 2 a_ij*, so
    M_o,i = (1 + 2 scale sum_d |q_id| |k_j*d|) |v_j*|."""
    B, H, S, D = 1, 2, 7, 5
    v = np.abs(_rand((B, H, S, D), 80))
    k = _rand((B, H, S, D), 81)
    do = np.abs(_rand((B, H, S, D), 82))
    q0 = np.zeros((B, H, S, D))
    mo, _, _, mdv = oracle.magnitudes(q0, k, v, do, scale=0.3)
    o, _ = oracle.forward(q0, k, v, scale=0.3)
    _, _, dv = oracle.backward(q0, k, v, do, scale=0.3)
    np.testing.assert_allclose(mo, np.broadcast_to(v.mean(axis=2, keepdims=True), mo.shape), atol=1e-14)
    np.testing.assert_allclose(mo, o, atol=1e-14)
    np.testing.assert_allclose(mdv, dv, atol=1e-14)
    q = _rand((B, H, S, D), 83)
    km = np.zeros((B, S), dtype=np.uint8)
    km[0, 4] = 1
    mo1, _, _, _ = oracle.magnitudes(q, k, v, do, scale=0.3, key_mask=km)
    a = 0.3 * (np.abs(q) * np.abs(k[:, :, 4:5])).sum(axis=3, keepdims=True)
    np.testing.assert_allclose(mo1, (1 + 2 * a) * np.abs(v[:, :, 4:5]), rtol=1e-14)


@pytest.mark.parametrize("causal,mod,use_mask,D", [(False, MOD_CHECKERBOARD, True, 64), (True, MOD_ALIBI, False, 64),
                                                   (False, MOD_NONE, False, 128), (True, MOD_NONE, True, 32)])
def test_fp32_evaluation_stays_within_the_derived_bound(causal, mod, use_mask, D):
    """An independent fp32 evaluation of the definition (torch CPU float32:
    matmul, softmax and autograd) against the fp64 oracle: every element of O,
    dQ, dK and dV is within kappa u M of the exact value."""
    B, H, Sq, Skv = 1, 2, 150, 230
    if causal:
        Skv = Sq
    rng = np.random.default_rng(90)
    q, k, v, do = (rng.standard_normal((B, H, Sq if i in (0, 3) else Skv, D)).astype(np.float32) for i in range(4))
    km = (rng.random((B, Skv)) < 0.5).astype(np.uint8) if use_mask else None
    if km is not None:
        km[:, 0] = 1
    scale = 1.0 / math.sqrt(D)
    kw = dict(scale=scale, causal=causal, mod=mod, key_mask=km)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    pos, kj = np.arange(Sq), np.arange(Skv)
    bias = torch.from_numpy(np.stack([oracle.score_bias(mod, h, pos, kj, H) for h in range(H)])).float()
    s = scale * (tq @ tk.transpose(-1, -2)) + bias[None]
    ok = torch.ones(B, 1, Sq, Skv, dtype=torch.bool)
    if km is not None:
        ok &= torch.from_numpy(km != 0)[:, None, None, :]
    if causal:
        ok &= torch.from_numpy(kj[None, :] <= pos[:, None])[None, None]
    o32 = torch.softmax(s.masked_fill(~ok, float("-inf")), dim=-1) @ tv
    o32.backward(torch.from_numpy(do))
    o, _ = oracle.forward(q, k, v, **kw)
    g = oracle.backward(q, k, v, do, **kw)
    mags = oracle.magnitudes(q, k, v, do, **kw)
    kap = kappa(Sq, Skv, D)
    for name, got, ref, m in zip(("o", "dq", "dk", "dv"), (o32.detach(), tq.grad, tk.grad, tv.grad), (o,) + tuple(g),
                                 mags):
        ok_, ratio = within(np.abs(got.double().numpy() - ref), 0.0, kap, m)
        assert ok_, f"{name}: error / (kappa u M) = {ratio:.3f}"


# --------------------------------------------------------------------------- caller-defined score_mods

from oracle import MOD_CUSTOM  # noqa: E402

CAP = 1.5   # soft-cap of the tanh score_mod below


def softcap(s, b, h, qi, kj):
    return CAP * np.tanh(s / CAP)


def softcap_grad(s, b, h, qi, kj):
    return 1.0 - np.tanh(s / CAP) ** 2


@pytest.mark.parametrize("causal,use_mask", [(False, False), (True, False), (False, True), (True, True)])
def test_custom_identity_and_additive_alibi_are_the_builtin_mods(causal, use_mask):
    """A custom mod returning the score unchanged is MOD_NONE, and one adding
    -slope_h (q_idx - kv_idx) is MOD_ALIBI, for the output, lse and every
    gradient (the derivative of an additive mod is 1)."""
    B, H, Sq, Skv, D, off = 2, 3, 13, 21, 4, 8
    q, k, v, do, km = _case(75, B=B, H=H, Sq=Sq, Skv=Skv, D=D, key_mask=use_mask)
    slopes = 2.0 ** (-8.0 * (np.arange(H) + 1) / H)
    ident = (lambda s, b, h, qi, kj: s, lambda s, b, h, qi, kj: np.ones_like(s))
    alibi = (lambda s, b, h, qi, kj: s - slopes[h] * (qi - kj), lambda s, b, h, qi, kj: np.ones_like(s))
    for builtin, custom in ((MOD_NONE, ident), (MOD_ALIBI, alibi)):
        base = dict(scale=0.7, causal=causal, key_mask=km, q_offset=off)
        o0, l0 = oracle.forward(q, k, v, mod=builtin, **base)
        o1, l1 = oracle.forward(q, k, v, mod=MOD_CUSTOM, custom=custom, **base)
        np.testing.assert_allclose(o1, o0, atol=1e-14)
        np.testing.assert_allclose(l1, l0, atol=1e-13)
        for g0, g1 in zip(oracle.backward(q, k, v, do, mod=builtin, **base),
                          oracle.backward(q, k, v, do, mod=MOD_CUSTOM, custom=custom, **base)):
            np.testing.assert_allclose(g1, g0, atol=1e-13)


@pytest.mark.parametrize("causal,use_mask,off", [(False, False, 0), (True, False, 0), (True, True, 9),
                                                 (False, True, 5)])
def test_custom_softcap_against_torch_autograd(causal, use_mask, off):
    """A score-dependent mod (tanh soft-cap of the scaled scores) against an
    independent torch fp64 evaluation: scores, tanh, masks, softmax, P V, and
    torch's autograd for the gradients."""
    B, H, Sq, Skv, D = 2, 2, 17, 26, 8
    q, k, v, do, km = _case(76, B=B, H=H, Sq=Sq, Skv=Skv, D=D, key_mask=use_mask)
    q, k = 2.0 * q, 2.0 * k   # scores well into tanh's bend
    scale = 1.0 / math.sqrt(D)
    kw = dict(scale=scale, causal=causal, key_mask=km, q_offset=off, mod=MOD_CUSTOM, custom=(softcap, softcap_grad))
    o, lse = oracle.forward(q, k, v, **kw)
    dq, dk, dv = oracle.backward(q, k, v, do, **kw)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = CAP * torch.tanh(scale * (tq @ tk.transpose(-1, -2)) / CAP)
    s = s + _torch_bias(MOD_NONE, B, H, Sq, Skv, causal, km, off)
    to = torch.softmax(s, dim=-1) @ tv
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).detach().numpy(), atol=1e-12)
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12)


def test_custom_softcap_gradients_match_central_differences():
    B, H, S, D = 1, 2, 5, 3
    q, k, v, do, km = _case(77, B=B, H=H, Sq=S, Skv=S, D=D, key_mask=True)
    kw = dict(scale=2.0, causal=True, key_mask=km, mod=MOD_CUSTOM, custom=(softcap, softcap_grad))
    grads = oracle.backward(q, k, v, do, **kw)
    h = 1e-5
    for name, x, g in zip(("q", "k", "v"), (q, k, v), grads):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = [{"q": q, "k": k, "v": v}, {"q": q, "k": k, "v": v}]
            for sgn, a in zip((1, -1), args):
                xx = x.copy()
                xx[idx] += sgn * h
                a[name] = xx
            num[idx] = (_loss(args[0]["q"], args[0]["k"], args[0]["v"], do, kw)
                        - _loss(args[1]["q"], args[1]["k"], args[1]["v"], do, kw)) / (2 * h)
        np.testing.assert_allclose(g, num, atol=1e-8, err_msg=f"d{name}")


def test_custom_pins_catch_a_dropped_chain_rule_factor(monkeypatch):
    """Plant a mistake (the backward forgets the mod's derivative) and check
    that the autograd pin rejects it."""
    import oracle.attention as A
    real = softcap_grad
    monkeypatch.setattr(sys.modules[__name__], "softcap_grad", lambda s, b, h, qi, kj: np.ones_like(s))
    with pytest.raises(AssertionError):
        test_custom_softcap_against_torch_autograd(False, False, 0)
    monkeypatch.setattr(sys.modules[__name__], "softcap_grad", real)
    assert A.MOD_CUSTOM == MOD_CUSTOM
