"""Tiled online-softmax attention for AMD Instinct MI355X (gfx950).

Thin binding over the C ABI in ``include/fa_mi355x.h``: it only marshals
torch tensors (device memory) and the current HIP stream into the library
calls.  Every step of the computation runs in the library's HIP kernels; there
is no CPU or PyTorch fallback, and a missing library raises.

    out, lse = forward(q, k, v, causal=..., key_mask=..., score_mod=...)
    dq, dk, dv = backward(q, k, v, out, lse, dout, ...)
    out, lse = decode(q, k, v, ...)              # seq_q == 1, split over keys

q, k, v: (batch, heads, seq, head_dim) contiguous cuda tensors of one dtype
(float32, float16 or bfloat16); key_mask: (batch, seq_kv) uint8/bool,
nonzero = keep; score_mod: None, "alibi", "checkerboard" or a ScoreMod (caller-defined, with
mod_params); block_mask:
(batch, heads, ceil(seq_q/128), ceil(seq_kv/128)) uint8/bool, zero removes a
128 x 128 block of (query row, key) pairs (``block_mask_shape`` gives the
shape).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import FaError

__all__ = ["forward", "backward", "decode", "decode_noalloc", "ScoreMod", "forward_split_workspace_bytes",
           "backward_workspace_bytes", "decode_workspace_bytes",
           "FaError", "problem", "plan_forward", "plan_backward", "plan_decode", "block_mask_shape"]

_DTYPE = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16, torch.bfloat16: _lib.FA_BF16}
_MOD = {None: _lib.FA_MOD_NONE, "none": _lib.FA_MOD_NONE, "alibi": _lib.FA_MOD_ALIBI,
        "checkerboard": _lib.FA_MOD_CHECKERBOARD}
_DQ_MODE = {"auto": _lib.FA_DQ_AUTO, "separate": _lib.FA_DQ_SEPARATE, "atomic": _lib.FA_DQ_ATOMIC}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


class ScoreMod:
    """A caller-defined score_mod, compiled by the library (hipRTC).

    ``source`` is HIP device code defining

        __device__ float fa_score_mod(float score, int b, int h, int q_idx, int kv_idx,
                                      const float* params);
        __device__ float fa_score_mod_grad(float score, int b, int h, int q_idx, int kv_idx,
                                           const float* params);

    (the modified score of score = scale * q.k at global positions, and its
    derivative with respect to score).  Pass the object as ``score_mod=`` and
    its parameters as ``mod_params=`` (a float32 cuda tensor) to forward and
    backward.  Compile errors raise FaError with the compiler's log."""

    def __init__(self, source: str):
        lib = _lib.load()
        handle = ctypes.c_void_p()
        log = ctypes.create_string_buffer(1 << 16)
        st = lib.fa_score_mod_create(source.encode(), ctypes.byref(handle), log, len(log))
        if st != _lib.FA_OK:
            raise FaError(st, "fa_score_mod_create", log.value.decode(errors="replace"))
        self.source = source
        self._handle = handle

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._handle is None:
            raise ValueError("ScoreMod has been closed")
        return self._handle

    def close(self) -> None:
        """Releases the compiled code (no call using it may be in flight)."""
        if getattr(self, "_handle", None) is not None:
            _lib.load().fa_score_mod_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def block_mask_shape(batch: int, heads: int, seq_q: int, seq_kv: int) -> Tuple[int, int, int, int]:
    """Shape of a block mask: one byte per 128 x 128 block of (query row, key)."""
    n = _lib.FA_BLOCK_MASK_BLOCK
    return (batch, heads, -(-seq_q // n), -(-seq_kv // n))


def problem(q: torch.Tensor, k: torch.Tensor, *, causal: bool = False,
            key_mask: Optional[torch.Tensor] = None, score_mod: Optional[str] = None,
            scale: Optional[float] = None, alibi_slopes: Optional[torch.Tensor] = None,
            checker: Tuple[float, float] = (0.5, -0.5), q_offset: int = 0,
            block_mask: Optional[torch.Tensor] = None, dq_mode: str = "auto",
            kv_splits: int = 0, mod_params: Optional[torch.Tensor] = None) -> _lib.FaProblem:
    """The C-ABI problem descriptor for these tensors.  q_offset is the
    position of query row 0 among the keys (0 for self-attention; the number
    of cached keys before the first query with a KV cache).  dq_mode ("auto",
    "separate" or "atomic") picks how the backward forms dQ; kv_splits (0 =
    the library's choice) the number of key chunks of fa_decode and
    fa_forward_split."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be (batch, heads, seq, head_dim)")
    if block_mask is not None:
        _expect(block_mask, "block_mask", block_mask_shape(q.shape[0], q.shape[1], q.shape[2], k.shape[2]),
                torch.uint8)
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if not isinstance(score_mod, ScoreMod) and score_mod not in _MOD:
        raise ValueError(f"unknown score_mod {score_mod!r}")
    B, H, Sq, D = q.shape
    p = _lib.FaProblem()
    p.batch, p.heads, p.seq_q, p.seq_kv, p.head_dim = B, H, Sq, k.shape[2], D
    p.dtype = _DTYPE[q.dtype]
    p.causal = int(bool(causal))
    p.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    if isinstance(score_mod, ScoreMod):
        p.mod_kind = _lib.FA_MOD_CUSTOM
        p.custom_mod = score_mod.handle
    else:
        p.mod_kind = _MOD[score_mod]
    if mod_params is not None:
        if mod_params.dtype != torch.float32 or not mod_params.is_contiguous():
            raise ValueError("mod_params must be a contiguous float32 tensor")
        p.mod_params = mod_params.data_ptr()
    p.alibi_slopes = None if alibi_slopes is None else alibi_slopes.data_ptr()
    p.checker_even, p.checker_odd = float(checker[0]), float(checker[1])
    p.key_mask = None if key_mask is None else key_mask.data_ptr()
    p.q_offset = int(q_offset)
    p.block_mask = None if block_mask is None else block_mask.data_ptr()
    if dq_mode not in _DQ_MODE:
        raise ValueError(f"dq_mode must be one of {sorted(_DQ_MODE)}, not {dq_mode!r}")
    p.dq_mode = _DQ_MODE[dq_mode]
    p.kv_splits = int(kv_splits)
    return p


def _check_tensors(*ts):
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or t.device != dev:
            raise ValueError("all tensors must be on the same cuda device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, name, shape, dtype):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")


def _validate(q, k, v, *, key_mask=None, alibi_slopes=None, block_mask=None, out=None, lse=None, dout=None,
              grads=(None, None, None), workspace=None):
    """Shapes and dtypes of every tensor against q and k, so that no
    mismatched tensor reaches the library as an out-of-bounds read or write.
    Pure metadata checks (they run on CPU tensors too)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None or t.dim() != 4:
            raise ValueError(f"{name} must be (batch, heads, seq, head_dim)")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    _expect(k, "k", (B, H, Skv, D), q.dtype)
    _expect(v, "v", (B, H, Skv, D), q.dtype)
    _expect(key_mask, "key_mask", (B, Skv), torch.uint8)
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.dim() != 1 or alibi_slopes.numel() < H:
            raise ValueError(f"alibi_slopes must be a float32 vector of at least {H} entries")
    _expect(block_mask, "block_mask", block_mask_shape(B, H, Sq, Skv), torch.uint8)
    _expect(out, "out", (B, H, Sq, D), q.dtype)
    _expect(lse, "lse", (B, H, Sq), torch.float32)
    _expect(dout, "dout", (B, H, Sq, D), q.dtype)
    dq, dk, dv = grads
    _expect(dq, "dq", (B, H, Sq, D), q.dtype)
    _expect(dk, "dk", (B, H, Skv, D), q.dtype)
    _expect(dv, "dv", (B, H, Skv, D), q.dtype)
    if workspace is not None and workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor (its numel is the byte count)")


def _mask_u8(key_mask):
    if key_mask is None:
        return None
    return key_mask.to(torch.uint8).contiguous() if key_mask.dtype != torch.uint8 else key_mask.contiguous()


def forward_split_workspace_bytes(p: _lib.FaProblem) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().fa_forward_split_workspace_size(ctypes.byref(p), ctypes.byref(n)),
               "fa_forward_split_workspace_size")
    return int(n.value)


def forward(q, k, v, *, causal=False, key_mask=None, score_mod=None, scale=None, alibi_slopes=None,
            checker=(0.5, -0.5), q_offset=0, block_mask=None, out=None, lse=None, mod_params=None, kv_splits=0,
            workspace=None):
    """Attention output (q's dtype) and log-sum-exp (float32, natural log).

    kv_splits: 0 = the library's per-shape choice (fa_forward_split: the key
    axis is split and merged where the query blocks alone leave the device
    idle), 1 = never split (fa_forward), n > 1 = about n key chunks."""
    key_mask, block_mask = _mask_u8(key_mask), _mask_u8(block_mask)
    _validate(q, k, v, key_mask=key_mask, alibi_slopes=alibi_slopes, block_mask=block_mask, out=out, lse=lse,
              workspace=workspace)
    _check_tensors(q, k, v, key_mask, alibi_slopes, block_mask, out, lse, mod_params, workspace)
    p = problem(q, k, causal=causal, key_mask=key_mask, score_mod=score_mod, scale=scale,
                alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset, block_mask=block_mask,
                mod_params=mod_params, kv_splits=kv_splits)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    lib = _lib.load()
    need = 0 if kv_splits == 1 else forward_split_workspace_bytes(p)
    if need == 0:
        _lib.check(lib.fa_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream(q)),
                   "fa_forward")
        return out, lse
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _lib.check(lib.fa_forward_split(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    _ptr(workspace), workspace.numel(), _stream(q)), "fa_forward_split")
    return out, lse


def backward_workspace_bytes(p: _lib.FaProblem) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().fa_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)), "fa_backward_workspace_size")
    return int(n.value)


def backward(q, k, v, out, lse, dout, *, causal=False, key_mask=None, score_mod=None, scale=None,
             alibi_slopes=None, checker=(0.5, -0.5), q_offset=0, block_mask=None, workspace=None, grads=None,
             which="all", dq_mode="auto", mod_params=None):
    """Gradients (dq, dk, dv) of sum(dout * out).

    which="dq" runs only the query pass (dk, dv come back as None), "dkdv"
    only the key/value pass (dq is None), "all" both.  dq_mode: "separate"
    (deterministic query pass), "atomic" (fp32 atomics in the key/value pass)
    or "auto" (the library's measured choice)."""
    if which not in ("all", "dq", "dkdv"):
        raise ValueError(f"which must be 'all', 'dq' or 'dkdv', not {which!r}")
    key_mask, block_mask = _mask_u8(key_mask), _mask_u8(block_mask)
    _validate(q, k, v, key_mask=key_mask, alibi_slopes=alibi_slopes, block_mask=block_mask, out=out, lse=lse,
              dout=dout, grads=grads if grads is not None else (None, None, None), workspace=workspace)
    _check_tensors(q, k, v, out, lse, dout, key_mask, alibi_slopes, block_mask, workspace, mod_params,
                   *(grads if grads is not None else ()))
    p = problem(q, k, causal=causal, key_mask=key_mask, score_mod=score_mod, scale=scale,
                alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset, block_mask=block_mask,
                dq_mode=dq_mode, mod_params=mod_params)
    need = backward_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    if which == "dq":
        dk = dv = None
    elif which == "dkdv":
        dq = None
    lib = _lib.load()
    _lib.check(lib.fa_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(q)),
               "fa_backward")
    return dq, dk, dv


def decode_workspace_bytes(p: _lib.FaProblem) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().fa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)), "fa_decode_workspace_size")
    return int(n.value)


def decode(q, k, v, *, key_mask=None, score_mod=None, scale=None, alibi_slopes=None, checker=(0.5, -0.5), q_offset=0,
           causal=False, block_mask=None, workspace=None, out=None, lse=None, kv_splits=0, mod_params=None):
    """Attention for a short query block (1 <= seq_q <= 64, row i at key
    position q_offset + i), split over the key axis (into about kv_splits
    chunks; 0 = the library's choice).  With causal=True a row sees keys up
    to its position only."""
    key_mask, block_mask = _mask_u8(key_mask), _mask_u8(block_mask)
    _validate(q, k, v, key_mask=key_mask, alibi_slopes=alibi_slopes, block_mask=block_mask, out=out, lse=lse,
              workspace=workspace)
    _check_tensors(q, k, v, key_mask, alibi_slopes, block_mask, out, lse, workspace)
    p = problem(q, k, causal=causal, key_mask=key_mask, score_mod=score_mod, scale=scale,
                alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset, block_mask=block_mask,
                kv_splits=kv_splits, mod_params=mod_params)
    need = decode_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    lib = _lib.load()
    _lib.check(lib.fa_decode(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace),
                             workspace.numel(), _stream(q)), "fa_decode")
    return out, lse


def decode_noalloc(q, k, v, *, key_mask=None, score_mod=None, scale=None, alibi_slopes=None, checker=(0.5, -0.5),
                   q_offset=0, causal=False, block_mask=None, out=None, lse=None, mod_params=None):
    """decode() through fa_decode_noalloc: no workspace, the library's fixed
    per-device scratch instead (for callers that cannot allocate at call time;
    pass out and lse to allocate nothing here either).  Calls that overlap on
    one device race on that scratch."""
    key_mask, block_mask = _mask_u8(key_mask), _mask_u8(block_mask)
    _validate(q, k, v, key_mask=key_mask, alibi_slopes=alibi_slopes, block_mask=block_mask, out=out, lse=lse)
    _check_tensors(q, k, v, key_mask, alibi_slopes, block_mask, out, lse, mod_params)
    p = problem(q, k, causal=causal, key_mask=key_mask, score_mod=score_mod, scale=scale,
                alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset, block_mask=block_mask,
                mod_params=mod_params)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    lib = _lib.load()
    _lib.check(lib.fa_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream(q)),
               "fa_decode_noalloc")
    return out, lse


# ---------------------------------------------------------------- prepared calls
#
# A plan marshals every argument once and returns a zero-argument callable
# that only enqueues the library call on the stream that was current when the
# plan was made.  The tensors are kept alive by the plan.


def _plan(fn, name, args, keep):
    def run():
        _lib.check(fn(*args), name)
    run.keep = keep
    return run


def plan_forward(q, k, v, out, lse, *, causal=False, key_mask=None, score_mod=None, scale=None,
                 alibi_slopes=None, checker=(0.5, -0.5), q_offset=0, block_mask=None, mod_params=None,
                 kv_splits=0, workspace=None):
    """kv_splits as in forward(); a split plan allocates its workspace now
    unless one is passed."""
    key_mask, block_mask = _mask_u8(key_mask), _mask_u8(block_mask)
    _validate(q, k, v, key_mask=key_mask, alibi_slopes=alibi_slopes, block_mask=block_mask, out=out, lse=lse,
              workspace=workspace)
    _check_tensors(q, k, v, out, lse, key_mask, alibi_slopes, block_mask, mod_params, workspace)
    p = problem(q, k, causal=causal, key_mask=key_mask, score_mod=score_mod, scale=scale,
                alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset, block_mask=block_mask,
                mod_params=mod_params, kv_splits=kv_splits)
    lib = _lib.load()
    keep = (p, q, k, v, out, lse, key_mask, alibi_slopes, block_mask, score_mod, mod_params)
    need = 0 if kv_splits == 1 else forward_split_workspace_bytes(p)
    if need == 0:
        args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream(q))
        return _plan(lib.fa_forward, "fa_forward", args, keep)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
            _stream(q))
    return _plan(lib.fa_forward_split, "fa_forward_split", args, keep + (workspace,))


def plan_backward(q, k, v, out, lse, dout, dq, dk, dv, workspace, *, causal=False, key_mask=None,
                  score_mod=None, scale=None, alibi_slopes=None, checker=(0.5, -0.5), q_offset=0, block_mask=None,
                  dq_mode="auto", mod_params=None):
    """dq may be None (key/value pass only); dk and dv may both be None (query pass only)."""
    key_mask, block_mask = _mask_u8(key_mask), _mask_u8(block_mask)
    _validate(q, k, v, key_mask=key_mask, alibi_slopes=alibi_slopes, block_mask=block_mask, out=out, lse=lse,
              dout=dout, grads=(dq, dk, dv), workspace=workspace)
    _check_tensors(q, k, v, out, lse, dout, dq, dk, dv, workspace, key_mask, alibi_slopes, block_mask, mod_params)
    p = problem(q, k, causal=causal, key_mask=key_mask, score_mod=score_mod, scale=scale,
                alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset, block_mask=block_mask,
                dq_mode=dq_mode, mod_params=mod_params)
    lib = _lib.load()
    args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace.numel(), _stream(q))
    return _plan(lib.fa_backward, "fa_backward", args,
                 (p, q, k, v, out, lse, dout, dq, dk, dv, workspace, key_mask, alibi_slopes, block_mask, score_mod,
                  mod_params))


def plan_decode(q, k, v, out, lse, workspace, *, key_mask=None, score_mod=None, scale=None, alibi_slopes=None,
                checker=(0.5, -0.5), q_offset=0, causal=False, block_mask=None, kv_splits=0, mod_params=None):
    key_mask, block_mask = _mask_u8(key_mask), _mask_u8(block_mask)
    _validate(q, k, v, key_mask=key_mask, alibi_slopes=alibi_slopes, block_mask=block_mask, out=out, lse=lse,
              workspace=workspace)
    _check_tensors(q, k, v, out, lse, workspace, key_mask, alibi_slopes, block_mask, mod_params)
    p = problem(q, k, causal=causal, key_mask=key_mask, score_mod=score_mod, scale=scale,
                alibi_slopes=alibi_slopes, checker=checker, q_offset=q_offset, block_mask=block_mask,
                kv_splits=kv_splits, mod_params=mod_params)
    lib = _lib.load()
    args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
            _stream(q))
    return _plan(lib.fa_decode, "fa_decode", args,
                 (p, q, k, v, out, lse, workspace, key_mask, alibi_slopes, block_mask, score_mod, mod_params))
