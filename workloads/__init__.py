"""Seeded synthetic inputs for the attention workloads.

This module only draws numbers; it holds none of the attention arithmetic.
Both the fp64 oracle (through the tests) and the HIP library (through the
tests, ``bench.py`` and the smoke check) are fed from here, so that both
sides see bit-identical, dtype-rounded inputs.

Every tensor is drawn from its own stream,
``np.random.SeedSequence([seed, workload_id, tensor_id])``, in fp64 with
``standard_normal`` and then rounded to the storage dtype by torch's
round-to-nearest-even conversion.  The pages draw q, k and v from one
``PRNGKey(42)`` (flash-attention-jax page, "Use flash_attention" example),
which would make them identical; separate streams avoid that, and 42 is kept
as the default seed.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

SEED = 42

# tensor ids of the per-tensor streams
Q, K, V, DOUT, MASK, ROWS, BLOCKS = 0, 1, 2, 3, 4, 5, 6

# edge of a block-mask block (query rows and keys)
BLOCK = 128

# score_mod kinds; the numbering matches the C-ABI enum
MOD_NONE, MOD_ALIBI, MOD_CHECKERBOARD = 0, 1, 2

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def _rng(workload_id: int, tensor_id: int, seed: int = SEED) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, workload_id, tensor_id]))


def normal(shape, dtype: str, workload_id: int, tensor_id: int, seed: int = SEED) -> torch.Tensor:
    """N(0,1) draw in fp64, rounded to ``dtype`` (CPU tensor, contiguous)."""
    x = _rng(workload_id, tensor_id, seed).standard_normal(size=tuple(shape))
    return torch.from_numpy(x).to(_DTYPES[dtype]).contiguous()


def bernoulli_key_mask(batch: int, seq_kv: int, workload_id: int, p_keep: float = 0.5,
                       seed: int = SEED) -> torch.Tensor:
    """(batch, seq_kv) uint8 key-padding mask, 1 = keep, each entry Bernoulli(p_keep).

    A batch row that draws no kept key is drawn again from the same stream,
    so every batch row keeps at least one key.
    """
    rng = _rng(workload_id, MASK, seed)
    rows = []
    for _ in range(batch):
        while True:
            r = (rng.random(seq_kv) < p_keep).astype(np.uint8)
            if r.any():
                break
        rows.append(r)
    return torch.from_numpy(np.stack(rows)).contiguous()


def block_grid(seq_q: int, seq_kv: int) -> Tuple[int, int]:
    """Number of 128-row and 128-key blocks."""
    return -(-seq_q // BLOCK), -(-seq_kv // BLOCK)


def bernoulli_block_mask(batch: int, heads: int, seq_q: int, seq_kv: int, workload_id: int,
                         p_keep: float = 0.5, seed: int = SEED) -> torch.Tensor:
    """(batch, heads, ceil(seq_q/128), ceil(seq_kv/128)) uint8 block mask, 1 =
    the block's pairs may attend, each entry Bernoulli(p_keep)."""
    nq, nk = block_grid(seq_q, seq_kv)
    r = _rng(workload_id, BLOCKS, seed).random((batch, heads, nq, nk)) < p_keep
    return torch.from_numpy(r.astype(np.uint8)).contiguous()


def window_block_mask(batch: int, heads: int, seq_q: int, seq_kv: int, window: int) -> torch.Tensor:
    """Block mask of a sliding window of whole blocks: block (r, c) is set
    when r - window < c <= r (the diagonal block and the window - 1 before it)."""
    nq, nk = block_grid(seq_q, seq_kv)
    r = np.arange(nq)[:, None]
    c = np.arange(nk)[None, :]
    m = ((c <= r) & (c > r - window)).astype(np.uint8)
    return torch.from_numpy(np.broadcast_to(m, (batch, heads, nq, nk)).copy()).contiguous()


def sample_rows(seq: int, n: int, workload_id: int, seed: int = SEED) -> np.ndarray:
    """Sorted distinct row indices in [0, seq): always 0, 1, 127, 128 and seq-1
    (causal edge, tile boundary, last row) when they exist, the rest drawn
    without replacement from the workload's ROWS stream."""
    fixed = sorted({r for r in (0, 1, 127, 128, seq - 1) if 0 <= r < seq})
    n = min(n, seq)
    rng = _rng(workload_id, ROWS, seed)
    pool = np.setdiff1d(np.arange(seq), np.array(fixed, dtype=np.int64))
    extra = rng.choice(pool, size=max(0, n - len(fixed)), replace=False) if len(pool) else []
    return np.array(sorted(set(fixed) | set(int(x) for x in extra)), dtype=np.int64)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype, masking and score_mod."""
    name: str
    workload_id: int
    batch: int
    heads: int
    seq_q: int
    seq_kv: int
    head_dim: int
    dtype: str
    causal: bool = False
    mod: int = MOD_NONE
    key_mask: bool = False
    backward: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def q_shape(self) -> Tuple[int, int, int, int]:
        return (self.batch, self.heads, self.seq_q, self.head_dim)

    def kv_shape(self) -> Tuple[int, int, int, int]:
        return (self.batch, self.heads, self.seq_kv, self.head_dim)

    def make(self, seed: int = SEED, with_dout: Optional[bool] = None) -> dict:
        """CPU tensors q, k, v (+ dout, key_mask when the workload has them)."""
        wid = self.workload_id
        out = {
            "q": normal(self.q_shape(), self.dtype, wid, Q, seed),
            "k": normal(self.kv_shape(), self.dtype, wid, K, seed),
            "v": normal(self.kv_shape(), self.dtype, wid, V, seed),
            "key_mask": bernoulli_key_mask(self.batch, self.seq_kv, wid, seed=seed)
            if self.key_mask else None,
        }
        if self.backward if with_dout is None else with_dout:
            out["dout"] = normal(self.q_shape(), self.dtype, wid, DOUT, seed)
        return out

    def pairs(self) -> int:
        """Evaluated (query, key) pairs: the causal lower triangle, else all."""
        per = (self.seq_q * (self.seq_q + 1) // 2) if self.causal else self.seq_q * self.seq_kv
        return self.batch * self.heads * per

    def fwd_flops(self) -> float:
        return 4.0 * self.head_dim * self.pairs()

    def bwd_flops(self) -> float:
        return 10.0 * self.head_dim * self.pairs()


# The five workloads.  Ids 1..5 seed the streams.
TINY_F32 = Workload("tiny exact fp32 (1,2,256,64)", 1, 1, 2, 256, 256, 64, "f32")
PREFILL_F16 = Workload("prefill fp16 causal ALiBi (8,8,2048,64)", 2, 8, 8, 2048, 2048, 64, "f16",
                       causal=True, mod=MOD_ALIBI)
KEYPAD_BF16 = Workload("key-padding bf16 checkerboard (4,16,4096,128)", 3, 4, 16, 4096, 4096, 128,
                       "bf16", mod=MOD_CHECKERBOARD, key_mask=True)
DECODE_F16_2K = Workload("decode fp16 (8,8,1,64) x 2048 keys", 4, 8, 8, 1, 2048, 64, "f16",
                         backward=False)
DECODE_F16_32K = Workload("decode fp16 (8,8,1,64) x 32768 keys", 4, 8, 8, 1, 32768, 64, "f16",
                          backward=False)
LONG_F32 = Workload("long-context fp32 causal (1,1,131072,512)", 5, 1, 1, 131072, 131072, 512,
                    "f32", causal=True)

ALL = (TINY_F32, PREFILL_F16, KEYPAD_BF16, DECODE_F16_2K, DECODE_F16_32K, LONG_F32)


def scaled(w: Workload, *, batch=None, heads=None, seq_q=None, seq_kv=None, head_dim=None,
           workload_id=None, name=None) -> Workload:
    """The same workload kind at other sizes (for oracle-sized parity cases)."""
    return dataclasses.replace(
        w,
        name=name or w.name + " (scaled)",
        workload_id=w.workload_id if workload_id is None else workload_id,
        batch=batch or w.batch, heads=heads or w.heads, seq_q=seq_q or w.seq_q,
        seq_kv=seq_kv or w.seq_kv, head_dim=head_dim or w.head_dim)
