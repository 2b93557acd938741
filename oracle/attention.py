"""fp64 CPU oracle for exact softmax attention, forward and analytic backward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the HIP library and
must never be used as a fallback for it.

What it computes (the definition the flash kernels reach up to rounding order):

* scores  s_ij = scale * <q_i, k_j> + bias_h(i, j).  The scale is applied to the
  dot product and the score_mod is added afterwards, without scaling
  (attnax ``pallas_flash_attention`` page, kernel body: scores are formed as
  ``q k^T * scale`` and then passed through ``score_mod`` with global query and
  key indices).
* a key (i, j) is *allowed* when the key-padding mask keeps key j of that batch
  row (flash-attention-jax page, "Use flash_attention": mask of shape
  (batch, seq); nonzero = keep, as in the attnax kernel body's
  ``where(mask, scores, min)``) and, for causal attention, j <= i
  (flash-attention-jax page, "Use causal_flash_attention").
* lse_i = log sum_{j allowed} exp(s_ij), P_ij = exp(s_ij - lse_i) on allowed
  pairs and 0 elsewhere, O_i = sum_j P_ij v_j.  This is the exact result the
  online softmax of the attnax kernel body (running max, running sum, rescaled
  accumulator, final division by the sum) arrives at.
* positions: query row i sits at position i + q_offset (q_offset = 0 by
  default; a KV cache of q_offset earlier keys otherwise: the flaxattention
  page's TODO list names decoding with a cache), and both the causal rule and
  the score_mod use that position.
* block sparsity (the flaxattention page's block mask): with a boolean
  block_mask (B, H, ceil(Sq/128), ceil(Skv/128)), pair (i, j) is also
  allowed only when block (i // 128, j // 128) is set (query ROW i, key j).
* a query row with no allowed key is an empty sum: O_i = 0, lse_i = -inf, and
  its gradients are zero.  (The pages leave this open; the attnax kernel's
  finite ``min`` fill would instead average V.)
* backward, by calculus on the definition (the bias does not depend on the
  scores, so it adds no term):
  dP = dO V^T, D_i = sum_j P_ij dP_ij (= <dO_i, O_i>), dS = P * (dP - D),
  dQ = scale * dS K, dK = scale * dS^T Q, dV = P^T dO.

A caller-defined score_mod (mod = MOD_CUSTOM, attnax pallas_flash_attention
page: score_mod is a callable applied to the scaled scores with global
indices, before the mask) is a pair custom = (fn, dfn) of numpy functions
fn(s, b, h, q_idx, kv_idx) -> modified scores and dfn(...) -> d fn / d s,
evaluated on the (rows, keys) matrix of s = scale <q_i, k_j> with q_idx a
column and kv_idx a row of global positions.  Then s'_ij = fn(s_ij, ...),
P = softmax of s' over the allowed keys, and by the chain rule
dS_ij = P_ij (dP_ij - D_i) dfn(s_ij, ...) in dQ = scale dS K and
dK = scale dS^T Q (the page obtains the same derivative by tracing).

score_mod kinds (the pages name them but do not define them; the readings
are the workloads' own definitions):

* ALiBi (flaxattention page, example: ``generate_alibi_bias(num_heads)``):
  bias = -slope_h * (q_idx - kv_idx) with slope_h = 2^(-8 (h+1) / H).
* checkerboard (flaxattention page, autograd example and benchmark):
  bias = +even when (q_idx + kv_idx) is even, +odd otherwise
  (defaults +0.5 / -0.5).

Query rows may be restricted to a subset ``rows`` (global indices).  Then the
forward returns those rows, and the backward returns dQ for those rows and the
dK, dV that a dO which is zero outside those rows produces (the backward is
linear in dO, so these are exact).

Every function here is pinned by tests that do not use this module's
arithmetic: closed forms, finite differences, hand-worked values and a
library attention routine.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

MOD_NONE, MOD_ALIBI, MOD_CHECKERBOARD, MOD_CUSTOM = 0, 1, 2, 3


def as_f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to fp64."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def default_alibi_slopes(num_heads: int) -> np.ndarray:
    """slope_h = 2^(-8 (h+1) / H), h = 0..H-1."""
    h = np.arange(num_heads, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / num_heads)


def score_bias(mod: int, h: int, q_idx: np.ndarray, kv_idx: np.ndarray, num_heads: int,
               alibi_slopes: Optional[Sequence[float]] = None,
               checker: Tuple[float, float] = (0.5, -0.5)) -> np.ndarray:
    """Additive bias of shape (len(q_idx), len(kv_idx)) for head h."""
    qi = np.asarray(q_idx, dtype=np.int64)[:, None]
    kj = np.asarray(kv_idx, dtype=np.int64)[None, :]
    if mod == MOD_NONE:
        return np.zeros((qi.shape[0], kj.shape[1]))
    if mod == MOD_ALIBI:
        slopes = default_alibi_slopes(num_heads) if alibi_slopes is None else np.asarray(
            alibi_slopes, dtype=np.float64)
        return -slopes[h] * (qi - kj).astype(np.float64)
    if mod == MOD_CHECKERBOARD:
        even = ((qi + kj) % 2) == 0
        return np.where(even, float(checker[0]), float(checker[1]))
    raise ValueError(f"unknown score_mod kind {mod}")


def allowed_pairs(q_idx: np.ndarray, seq_kv: int, causal: bool,
                  key_mask_row: Optional[np.ndarray]) -> np.ndarray:
    """Boolean (len(q_idx), seq_kv): key kept by the mask and, if causal, j <= i."""
    kj = np.arange(seq_kv)[None, :]
    ok = np.ones((len(q_idx), seq_kv), dtype=bool)
    if key_mask_row is not None:
        ok &= (np.asarray(key_mask_row) != 0)[None, :]
    if causal:
        ok &= kj <= np.asarray(q_idx)[:, None]
    return ok


def _block_allowed(block_mask, b: int, h: int, rows: np.ndarray, seq_kv: int) -> np.ndarray:
    """Boolean (len(rows), seq_kv): block (row // 128, key // 128) is set."""
    bm = np.asarray(block_mask, dtype=bool)[b, h]
    return bm[(np.asarray(rows) // 128)[:, None], (np.arange(seq_kv) // 128)[None, :]]


def _probabilities(qb: np.ndarray, kb: np.ndarray, scale: float, bias: np.ndarray,
                   ok: np.ndarray):
    """Scores, lse and P for one (batch, head) and a block of query rows."""
    return _softmax_rows(scale * (qb @ kb.T) + bias, ok)


def _custom_scores(qb, kb, scale, custom, b, h, pos, kv_idx):
    """(s, s') for a caller-defined score_mod: s = scale q.k, s' = fn(s, ...)."""
    s = scale * (qb @ kb.T)
    return s, np.asarray(custom[0](s, b, h, np.asarray(pos)[:, None], np.asarray(kv_idx)[None, :]),
                         dtype=np.float64) * np.ones_like(s)


def _softmax_rows(s: np.ndarray, ok: np.ndarray):
    """lse and P of the allowed entries of each row of s (empty rows: -inf, 0)."""
    s_allowed = np.where(ok, s, -np.inf)
    m = s_allowed.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    any_ok = np.isfinite(m)
    m_safe = np.where(any_ok, m, 0.0)
    e = np.where(ok, np.exp(s_allowed - m_safe[:, None]), 0.0)
    tot = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(any_ok, m_safe + np.log(tot), -np.inf)
    p = np.where(any_ok[:, None], e / np.where(any_ok, tot, 1.0)[:, None], 0.0)
    return s, lse, p


def _setup(q, k, v, rows, key_mask):
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    if (q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape[:3] != v.shape[:3]
            or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]):
        raise ValueError("q (B,H,Sq,D), k (B,H,Skv,D) and v (B,H,Skv,Dv) expected")
    seq_q = q.shape[2]
    rows = np.arange(seq_q) if rows is None else np.asarray(rows, dtype=np.int64)
    km = None if key_mask is None else as_f64(key_mask)
    return q, k, v, rows, km


def forward(q, k, v, *, scale: float, causal: bool = False, key_mask=None,
            mod: int = MOD_NONE, alibi_slopes=None, checker=(0.5, -0.5),
            rows: Optional[Sequence[int]] = None, q_offset: int = 0, block_mask=None, custom=None):
    """Exact attention output and log-sum-exp.

    Returns ``(o, lse)``: o (B, H, R, D), lse (B, H, R) in fp64, where R are the
    requested query rows (all rows by default).  Query row i sits at position
    i + q_offset of the key sequence (a KV cache holding q_offset earlier
    keys): the causal mask keeps keys j <= i + q_offset and the score_mod sees
    that position.
    """
    q, k, v, rows, km = _setup(q, k, v, rows, key_mask)
    B, H = q.shape[:2]
    seq_kv = k.shape[2]
    o = np.zeros((B, H, len(rows), v.shape[3]))
    lse = np.zeros((B, H, len(rows)))
    kv_idx = np.arange(seq_kv)
    pos = rows + int(q_offset)
    for b in range(B):
        ok = allowed_pairs(pos, seq_kv, causal, None if km is None else km[b])
        for h in range(H):
            okh = ok if block_mask is None else ok & _block_allowed(block_mask, b, h, rows, seq_kv)
            if mod == MOD_CUSTOM:
                _, s_mod = _custom_scores(q[b, h, rows], k[b, h], scale, custom, b, h, pos, kv_idx)
                _, lse[b, h], p = _softmax_rows(s_mod, okh)
            else:
                bias = score_bias(mod, h, pos, kv_idx, H, alibi_slopes, checker)
                _, lse[b, h], p = _probabilities(q[b, h, rows], k[b, h], scale, bias, okh)
            o[b, h] = p @ v[b, h]
    return o, lse


def backward(q, k, v, dout, *, scale: float, causal: bool = False, key_mask=None,
             mod: int = MOD_NONE, alibi_slopes=None, checker=(0.5, -0.5),
             rows: Optional[Sequence[int]] = None, q_offset: int = 0, block_mask=None, custom=None):
    """Analytic gradients of sum(dout * O) with respect to q, k and v.

    Returns ``(dq, dk, dv)``: dq (B, H, R, D) for the requested rows; dk and dv
    (B, H, Skv, D) are the gradients for a dout that is zero outside those rows
    (with all rows, the ordinary full gradient).  q_offset as in forward.
    """
    q, k, v, rows, km = _setup(q, k, v, rows, key_mask)
    do = as_f64(dout)
    if do.shape != q.shape[:3] + v.shape[3:]:
        raise ValueError("dout must have shape (B, H, Sq, Dv)")
    B, H, _, D = q.shape
    seq_kv = k.shape[2]
    dq = np.zeros((B, H, len(rows), D))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    kv_idx = np.arange(seq_kv)
    pos = rows + int(q_offset)
    for b in range(B):
        ok = allowed_pairs(pos, seq_kv, causal, None if km is None else km[b])
        for h in range(H):
            qb, dob = q[b, h, rows], do[b, h, rows]
            okh = ok if block_mask is None else ok & _block_allowed(block_mask, b, h, rows, seq_kv)
            if mod == MOD_CUSTOM:
                s_raw, s_mod = _custom_scores(qb, k[b, h], scale, custom, b, h, pos, kv_idx)
                _, _, p = _softmax_rows(s_mod, okh)
            else:
                bias = score_bias(mod, h, pos, kv_idx, H, alibi_slopes, checker)
                _, _, p = _probabilities(qb, k[b, h], scale, bias, okh)
            dp = dob @ v[b, h].T
            d_row = (p * dp).sum(axis=1)
            ds = p * (dp - d_row[:, None])
            if mod == MOD_CUSTOM:   # chain rule through the caller's mod (allowed pairs only)
                ds = np.where(okh, ds * (np.asarray(custom[1](s_raw, b, h, pos[:, None], kv_idx[None, :]),
                                                    dtype=np.float64) * np.ones_like(s_raw)), 0.0)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ qb)
            dv[b, h] = p.T @ dob
    return dq, dk, dv


def decode(q, k, v, *, scale: float, key_mask=None, mod: int = MOD_NONE, alibi_slopes=None,
           checker=(0.5, -0.5), q_offset: int = 0, causal: bool = False):
    """Single-query attention (seq_q = 1, query at position q_offset): the
    forward at Sq = 1."""
    q = as_f64(q)
    if q.shape[2] != 1:
        raise ValueError("decode takes seq_q = 1")
    return forward(q, k, v, scale=scale, causal=causal, key_mask=key_mask, mod=mod,
                   alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset)


def magnitudes(q, k, v, dout, *, scale: float, causal: bool = False, key_mask=None,
               mod: int = MOD_NONE, alibi_slopes=None, checker=(0.5, -0.5),
               rows: Optional[Sequence[int]] = None, q_offset: int = 0, block_mask=None):
    """Magnitudes that bound the rounding error of an fp32 evaluation of the
    forward and backward, per output element.

    An fp32 kernel forms every output as sums of products (dot products of
    length head_dim for the scores and dP, sums over keys or queries for O, dQ,
    dK, dV), and each rounding error is at most u = 2^-24 times the magnitude
    of the quantity it rounds.  Carrying absolute values through the same
    formulas gives, for every output element, the magnitude M that its
    accumulated rounding error is proportional to:

    * a_ij = scale * sum_d |q_id| |k_jd| + |bias_ij|: magnitude of the score,
      whose rounding moves P_ij by a relative amount proportional to a_ij, and
      lse_i by the P-weighted mean abar_i of a_ij; r_ij = 1 + a_ij + abar_i is
      the relative error weight of P_ij (the 1 for the exponential and the
      normalisation themselves);
    * M_o = (P o r) |V|,  M_dv = (P o r)^T |dO|;
    * the error of dS_ij = P_ij (dP_ij - D_i) is weighted by
      T_ij = P_ij (r_ij |dP_ij - D_i| + b_ij + c_i) with b_ij = sum_d |dO_id| |v_jd|
      (magnitude of dP_ij) and c_i = sum_d |dO_id| (M_o,id + |O_id|)
      (magnitude of D_i = <dO_i, O_i> including the error O carries);
    * M_dq = scale * T |K|,  M_dk = scale * T^T |Q|.

    Returns (M_o, M_dq, M_dk, M_dv) with the shapes of (o, dq, dk, dv) from
    forward/backward with the same ``rows``.  Every M is at least the absolute
    value of the corresponding result (r >= 1 and T_ij >= |dS_ij|).
    """
    if mod == MOD_CUSTOM:
        raise NotImplementedError("error magnitudes are defined for the built-in score_mods")
    q, k, v, rows, km = _setup(q, k, v, rows, key_mask)
    do = as_f64(dout)
    B, H, _, D = q.shape
    seq_kv = k.shape[2]
    m_o = np.zeros((B, H, len(rows), v.shape[3]))
    m_dq = np.zeros((B, H, len(rows), D))
    m_dk = np.zeros_like(k)
    m_dv = np.zeros_like(v)
    kv_idx = np.arange(seq_kv)
    pos = rows + int(q_offset)
    for b in range(B):
        ok = allowed_pairs(pos, seq_kv, causal, None if km is None else km[b])
        for h in range(H):
            bias = score_bias(mod, h, pos, kv_idx, H, alibi_slopes, checker)
            qb, dob = q[b, h, rows], do[b, h, rows]
            okh = ok if block_mask is None else ok & _block_allowed(block_mask, b, h, rows, seq_kv)
            _, _, p = _probabilities(qb, k[b, h], scale, bias, okh)
            a = scale * (np.abs(qb) @ np.abs(k[b, h]).T) + np.abs(bias)
            abar = (p * a).sum(axis=1)
            pr = p * (1.0 + a + abar[:, None])
            o = p @ v[b, h]
            m_o[b, h] = pr @ np.abs(v[b, h])
            dp = dob @ v[b, h].T
            d_row = (p * dp).sum(axis=1)
            bmag = np.abs(dob) @ np.abs(v[b, h]).T
            cmag = (np.abs(dob) * (m_o[b, h] + np.abs(o))).sum(axis=1)
            t = pr * np.abs(dp - d_row[:, None]) + p * (bmag + cmag[:, None])
            m_dq[b, h] = scale * (t @ np.abs(k[b, h]))
            m_dk[b, h] = scale * (t.T @ np.abs(qb))
            m_dv[b, h] = pr.T @ np.abs(dob)
    return m_o, m_dq, m_dk, m_dv
