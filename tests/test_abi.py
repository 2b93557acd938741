"""The C ABI loads, exports every symbol the header declares, and rejects bad
arguments on the host before anything reaches the GPU (no compute calls here)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from tiled_online_softmax_flashattention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Fake, 256-byte aligned device addresses: validation must reject the call
# before any of them could be dereferenced.
A = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(12)]


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fa_[a-z0-9_]+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("fa_forward", "fa_backward", "fa_decode", "fa_backward_workspace_size",
               "fa_decode_workspace_size", "fa_status_string", "fa_abi_version"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(_lib.SIGNATURES) == declared_functions()
    # the race-check build (FA_DEBUG_BARRIERS) exports the same interface
    rc = ctypes.CDLL(os.path.join(os.path.dirname(_lib.LIB_PATH), "libfa_mi355x_racecheck.so"))
    for name in declared_functions():
        assert hasattr(rc, name), name
    rc.fa_abi_version.restype = ctypes.c_int
    assert rc.fa_abi_version() == _lib.FA_ABI_VERSION


def test_abi_version_and_status_strings():
    lib = _lib.load()
    assert lib.fa_abi_version() == _lib.FA_ABI_VERSION == 7
    for s in range(7):
        assert lib.fa_status_string(s)
    assert lib.fa_status_string(99) == b"unknown status"


def test_problem_struct_layout_matches_the_header(tmp_path):
    """The ctypes view of fa_problem has the size and field offsets that a C
    compiler gives the header's struct (and the header's constants agree)."""
    fields = [f for f, _ in _lib.FaProblem._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "fa_mi355x.h"\nint main(void) {\n'
        '  printf("%zu %d %d %d\\n", sizeof(fa_problem), FA_ABI_VERSION, FA_BLOCK_MASK_BLOCK, FA_BLOCK_MASK_MAX_SEQ);\n'
        + "".join(f'  printf("%zu\\n", offsetof(fa_problem, {f}));\n' for f in fields) + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    size, ver, blk, max_seq = (int(x) for x in out[:4])
    assert size == ctypes.sizeof(_lib.FaProblem)
    assert (ver, blk, max_seq) == (_lib.FA_ABI_VERSION, _lib.FA_BLOCK_MASK_BLOCK, _lib.FA_BLOCK_MASK_MAX_SEQ)
    for f, off in zip(fields, out[4:]):
        assert getattr(_lib.FaProblem, f).offset == int(off), f


def prob(**kw):
    p = _lib.FaProblem()
    p.batch, p.heads, p.seq_q, p.seq_kv, p.head_dim = 2, 4, 100, 100, 64
    p.dtype, p.causal, p.scale, p.mod_kind = _lib.FA_F16, 0, 0.125, 0
    p.checker_even, p.checker_odd = 0.5, -0.5
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def fwd(p, q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4]):
    return _lib.load().fa_forward(ctypes.byref(p) if p is not None else None, q, k, v, o, lse, None)


def bwd(p, ws_bytes=1 << 30, ws=A[11], **override):
    ptrs = dict(q=A[0], k=A[1], v=A[2], o=A[3], lse=A[4], do=A[5], dq=A[6], dk=A[7], dv=A[8])
    ptrs.update(override)
    return _lib.load().fa_backward(ctypes.byref(p), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["lse"],
                                   ptrs["do"], ptrs["dq"], ptrs["dk"], ptrs["dv"], ws, ws_bytes, None)


def dec(p, ws_bytes=1 << 30, ws=A[11]):
    return _lib.load().fa_decode(ctypes.byref(p), A[0], A[1], A[2], A[3], A[4], ws, ws_bytes, None)


INVALID, UNSUP, WS = _lib.FA_ERR_INVALID_ARGUMENT, _lib.FA_ERR_UNSUPPORTED, _lib.FA_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("field,value", [("batch", 0), ("heads", -1), ("seq_q", 0), ("seq_kv", 0),
                                         ("head_dim", 0), ("dtype", 7), ("causal", 2), ("mod_kind", 4),
                                         ("scale", float("nan")), ("scale", float("inf"))])
def test_invalid_problem_fields(field, value):
    assert fwd(prob(**{field: value})) == INVALID


def test_null_problem_and_pointers():
    assert fwd(None) == INVALID
    assert fwd(prob(), q=None) == INVALID
    assert fwd(prob(), o=None) == INVALID
    assert fwd(prob(), k=ctypes.c_void_p(0x10008)) == INVALID       # not 16-byte aligned
    assert fwd(prob(), lse=ctypes.c_void_p(0x10002)) == INVALID


def test_query_offset_rules():
    """Causal needs no square shape (query row i sits at key position i +
    q_offset); q_offset must be >= 0 and keep positions below 2^31."""
    assert fwd(prob(q_offset=-1)) == INVALID
    assert fwd(prob(causal=1, q_offset=-5)) == INVALID
    assert fwd(prob(seq_q=100, q_offset=(1 << 31) - 100)) == UNSUP
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    assert lib.fa_backward_workspace_size(ctypes.byref(prob(causal=1, seq_q=7, seq_kv=101, q_offset=94)),
                                          ctypes.byref(n)) == _lib.FA_OK
    assert lib.fa_decode_workspace_size(ctypes.byref(prob(causal=1, seq_q=1, seq_kv=4096, q_offset=100)),
                                        ctypes.byref(n)) == _lib.FA_OK
    assert lib.fa_decode_workspace_size(ctypes.byref(prob(causal=1, seq_q=1, seq_kv=4096, q_offset=-1)),
                                        ctypes.byref(n)) == INVALID


def test_unsupported_head_dims():
    assert fwd(prob(head_dim=96)) == UNSUP
    assert fwd(prob(head_dim=512)) == UNSUP                      # 512 is fp32-only
    assert fwd(prob(head_dim=256, dtype=_lib.FA_F32)) == UNSUP


def test_scale_must_be_positive():
    assert fwd(prob(scale=0.0)) == UNSUP
    assert fwd(prob(scale=-0.125)) == UNSUP
    assert bwd(prob(scale=-1.0)) == UNSUP
    assert dec(prob(seq_q=1, scale=0.0)) == UNSUP


def test_checkerboard_needs_finite_values():
    assert fwd(prob(mod_kind=2, checker_even=float("nan"))) == INVALID


def test_oversized_problem():
    assert fwd(prob(seq_q=1 << 26, seq_kv=1 << 26)) == UNSUP


def test_backward_workspace_rules():
    lib = _lib.load()
    p = prob(seq_q=300, seq_kv=300)
    n = ctypes.c_size_t(0)
    assert lib.fa_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.FA_OK
    rows = 2 * 4 * 300
    assert n.value >= 2 * rows * 4 and n.value % 256 == 0
    assert bwd(p, ws_bytes=n.value - 1) == WS
    assert bwd(p, ws=None) == INVALID
    assert bwd(p, ws=ctypes.c_void_p(0x10010)) == INVALID            # workspace must be 256-byte aligned
    assert bwd(p, lse=None) == INVALID
    assert bwd(p, dk=None) == INVALID                               # dk and dv go together
    assert bwd(p, dq=None, dk=None, dv=None) == INVALID              # nothing requested
    assert lib.fa_backward_workspace_size(ctypes.byref(p), None) == INVALID


def test_decode_rules():
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    assert lib.fa_decode_workspace_size(ctypes.byref(prob(seq_q=65, seq_kv=4096)), ctypes.byref(n)) == INVALID
    assert lib.fa_decode_workspace_size(ctypes.byref(prob(seq_q=64, seq_kv=4096)), ctypes.byref(n)) == _lib.FA_OK
    assert n.value >= 2 * 4 * 64 * (64 + 2) * 4   # a partial row per (batch, head, query) and key chunk
    p = prob(seq_q=1, seq_kv=32768)
    assert lib.fa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.FA_OK
    assert n.value > 0 and n.value % 256 == 0
    assert dec(p, ws_bytes=n.value - 1) == WS
    assert dec(prob(seq_q=65)) == INVALID
    assert dec(prob(seq_q=1, head_dim=512, dtype=_lib.FA_F32)) == UNSUP


def test_block_mask_length_limit():
    """A block mask takes sequences up to FA_BLOCK_MASK_MAX_SEQ (tile lists in
    LDS); without one the same lengths pass validation."""
    m = _lib.FA_BLOCK_MASK_MAX_SEQ
    bm = A[9]
    assert fwd(prob(seq_q=m + 1, seq_kv=64, block_mask=bm)) == UNSUP
    assert fwd(prob(seq_q=64, seq_kv=m + 1, block_mask=bm)) == UNSUP
    assert bwd(prob(seq_q=m + 1, seq_kv=m + 1, block_mask=bm)) == UNSUP
    assert dec(prob(seq_q=1, seq_kv=m + 1, block_mask=bm)) == UNSUP
    # at the limit validation passes and the next check (a null tensor) fails
    assert fwd(prob(seq_q=m, seq_kv=m, block_mask=bm), q=None) == INVALID
    assert fwd(prob(seq_q=m + 1, seq_kv=64), q=None) == INVALID


def test_binding_block_mask_shape_and_pointer():
    """The binding takes a (batch, heads, ceil(Sq/128), ceil(Skv/128)) uint8
    block mask, rejects any other shape or dtype, and passes its address."""
    import torch
    import tiled_online_softmax_flashattention_amd as fa
    q = torch.zeros(2, 3, 300, 64, dtype=torch.float16)
    k = torch.zeros(2, 3, 129, 64, dtype=torch.float16)
    assert fa.block_mask_shape(2, 3, 300, 129) == (2, 3, 3, 2)
    bm = torch.ones(2, 3, 3, 2, dtype=torch.uint8)
    p = fa.problem(q, k, block_mask=bm)
    assert p.block_mask == bm.data_ptr()
    assert fa.problem(q, k).block_mask is None
    for bad in (torch.ones(2, 3, 2, 2, dtype=torch.uint8), torch.ones(2, 3, 3, 3, dtype=torch.uint8),
                torch.ones(2, 3, 3, 2, dtype=torch.int32)):
        with pytest.raises(ValueError):
            fa.problem(q, k, block_mask=bad)


def _cpu_inputs(B=2, H=3, Sq=50, Skv=70, D=64, dtype=None):
    import torch
    dtype = dtype or torch.float16
    q = torch.zeros(B, H, Sq, D, dtype=dtype)
    k = torch.zeros(B, H, Skv, D, dtype=dtype)
    v = torch.zeros(B, H, Skv, D, dtype=dtype)
    return q, k, v


def _bad_cases():
    """(entry point, keyword overrides) pairs that the binding must reject
    with ValueError before anything reaches the library: every tensor's shape
    and dtype is checked against q and k."""
    import torch
    q, k, v = _cpu_inputs()
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    f16, f32, u8 = torch.float16, torch.float32, torch.uint8
    return [
        ("forward", dict(k=torch.zeros(B, H + 1, Skv, D, dtype=f16))),          # heads differ
        ("forward", dict(k=torch.zeros(B + 1, H, Skv, D, dtype=f16))),          # batch differs
        ("forward", dict(k=torch.zeros(B, H, Skv, 128, dtype=f16))),            # head_dim differs
        ("forward", dict(k=torch.zeros(B, H, Skv, D, dtype=torch.bfloat16))),   # dtype differs
        ("forward", dict(v=torch.zeros(B, H, Skv + 1, D, dtype=f16))),          # v.shape != k.shape
        ("forward", dict(v=torch.zeros(B, H, Skv, D, dtype=f32))),
        ("forward", dict(key_mask=torch.ones(B, Skv + 1, dtype=u8))),           # key mask (B, Skv)
        ("forward", dict(key_mask=torch.ones(B + 1, Skv, dtype=u8))),
        ("forward", dict(alibi_slopes=torch.ones(H - 1, dtype=f32), score_mod="alibi")),   # too few slopes
        ("forward", dict(alibi_slopes=torch.ones(H, dtype=torch.float64), score_mod="alibi")),
        ("forward", dict(out=torch.zeros(B, H, Sq - 1, D, dtype=f16))),         # caller's out too small
        ("forward", dict(out=torch.zeros(B, H, Sq, D, dtype=f32))),
        ("forward", dict(lse=torch.zeros(B, H, Sq - 1, dtype=f32))),            # caller's lse too small
        ("forward", dict(lse=torch.zeros(B, H, Sq, dtype=f16))),
        ("forward", dict(block_mask=torch.ones(B, H, 1, 2, dtype=u8))),
        ("backward", dict(dout=torch.zeros(B, H, Sq, D - 32, dtype=f16))),
        ("backward", dict(dout=torch.zeros(B, H, Sq, D, dtype=f32))),
        ("backward", dict(out=torch.zeros(B, H, Sq + 1, D, dtype=f16))),
        ("backward", dict(lse=torch.zeros(B, H, Sq + 1, dtype=f32))),
        ("backward", dict(grads=(torch.zeros(B, H, Sq - 1, D, dtype=f16), torch.zeros_like(k), torch.zeros_like(v)))),
        ("backward", dict(grads=(torch.zeros_like(q), torch.zeros(B, H, Skv - 1, D, dtype=f16), torch.zeros_like(v)))),
        ("backward", dict(grads=(torch.zeros_like(q), torch.zeros_like(k), torch.zeros(B, H, Skv, D, dtype=f32)))),
        ("backward", dict(workspace=torch.zeros(1024, dtype=f32))),            # bytes counted from numel
        ("decode", dict(out=torch.zeros(B, H, Sq, D + 64, dtype=f16))),
        ("decode", dict(lse=torch.zeros(B, H, 1, dtype=f32))),
        ("decode", dict(k=torch.zeros(B, H, Skv, D, dtype=f32))),
    ]


@pytest.mark.parametrize("case", range(26))
def test_binding_rejects_mismatched_tensors(case):
    """A mismatched k, v, key mask, slope vector, dout or caller-supplied out,
    lse, gradient or workspace tensor raises ValueError in the binding (it
    would otherwise reach the kernels as an out-of-bounds read or write)."""
    import torch
    import tiled_online_softmax_flashattention_amd as fa
    cases = _bad_cases()
    assert len(cases) == 26
    fn_name, over = cases[case]
    q, k, v = _cpu_inputs()
    B, H, Sq, D = q.shape
    args = dict(q=q, k=k, v=v)
    for name in ("q", "k", "v"):
        if name in over:
            args[name] = over.pop(name)
    if fn_name == "forward":
        call = lambda: fa.forward(args["q"], args["k"], args["v"], **over)
    elif fn_name == "backward":
        out = over.pop("out", torch.zeros_like(q))
        lse = over.pop("lse", torch.zeros(B, H, Sq, dtype=torch.float32))
        dout = over.pop("dout", torch.zeros_like(q))
        call = lambda: fa.backward(args["q"], args["k"], args["v"], out, lse, dout, **over)
    else:
        call = lambda: fa.decode(args["q"], args["k"], args["v"], **over)
    with pytest.raises(ValueError):
        call()


def test_binding_accepts_matching_cpu_tensors_until_the_device_check():
    """Well-formed tensors pass the shape checks and are then refused only
    because they are not on a GPU (the library is never called)."""
    import torch
    import tiled_online_softmax_flashattention_amd as fa
    q, k, v = _cpu_inputs()
    B, H, Sq, D = q.shape
    with pytest.raises(ValueError, match="cuda"):
        fa.forward(q, k, v, key_mask=torch.ones(B, k.shape[2], dtype=torch.uint8),
                   out=torch.zeros_like(q), lse=torch.zeros(B, H, Sq, dtype=torch.float32))


def test_decode_noalloc_rules():
    """fa_decode_noalloc validates like fa_decode (no workspace argument) and
    refuses a problem whose partials exceed its fixed scratch, before any
    HIP call."""
    lib = _lib.load()
    nd = lambda p: lib.fa_decode_noalloc(ctypes.byref(p), A[0], A[1], A[2], A[3], A[4], None)
    assert lib.fa_decode_noalloc(None, A[0], A[1], A[2], A[3], A[4], None) == INVALID
    assert nd(prob(seq_q=65)) == INVALID
    assert nd(prob(seq_q=1, head_dim=512, dtype=_lib.FA_F32)) == UNSUP
    assert nd(prob(seq_q=1, scale=0.0)) == UNSUP
    assert lib.fa_decode_noalloc(ctypes.byref(prob(seq_q=1)), None, A[1], A[2], A[3], A[4], None) == INVALID
    big = prob(batch=4, heads=32, seq_q=64, seq_kv=32768, head_dim=128)
    n = ctypes.c_size_t(0)
    assert lib.fa_decode_workspace_size(ctypes.byref(big), ctypes.byref(n)) == _lib.FA_OK
    assert n.value > _lib.FA_DECODE_SCRATCH_BYTES
    assert nd(big) == _lib.FA_ERR_SCRATCH_LIMIT
    assert b"scratch" in lib.fa_status_string(_lib.FA_ERR_SCRATCH_LIMIT)


def test_dq_mode_and_kv_splits_rules():
    """dq_mode must name a mode; the atomic mode is for 16-bit types and adds
    an fp32 accumulator to the workspace; kv_splits is 0 (automatic) or
    1 .. FA_MAX_KV_SPLITS."""
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    sizes = {}
    for mode in (_lib.FA_DQ_AUTO, _lib.FA_DQ_SEPARATE, _lib.FA_DQ_ATOMIC):
        assert lib.fa_backward_workspace_size(ctypes.byref(prob(dq_mode=mode)), ctypes.byref(n)) == _lib.FA_OK
        sizes[mode] = n.value
    assert sizes[_lib.FA_DQ_ATOMIC] >= sizes[_lib.FA_DQ_SEPARATE] + 2 * 4 * 100 * 64 * 4
    assert sizes[_lib.FA_DQ_AUTO] == sizes[_lib.FA_DQ_SEPARATE]
    assert lib.fa_backward_workspace_size(ctypes.byref(prob(dq_mode=3)), ctypes.byref(n)) == INVALID
    assert lib.fa_backward_workspace_size(ctypes.byref(prob(dq_mode=_lib.FA_DQ_ATOMIC, dtype=_lib.FA_F32)),
                                          ctypes.byref(n)) == UNSUP
    assert bwd(prob(dq_mode=_lib.FA_DQ_ATOMIC), ws_bytes=sizes[_lib.FA_DQ_SEPARATE]) == WS
    assert fwd(prob(kv_splits=-1)) == INVALID
    assert fwd(prob(kv_splits=_lib.FA_MAX_KV_SPLITS + 1)) == UNSUP
    one = prob(seq_q=1, seq_kv=4096, kv_splits=1)
    seven = prob(seq_q=1, seq_kv=4096, kv_splits=7)
    assert lib.fa_decode_workspace_size(ctypes.byref(one), ctypes.byref(n)) == _lib.FA_OK
    n1 = n.value
    assert lib.fa_decode_workspace_size(ctypes.byref(seven), ctypes.byref(n)) == _lib.FA_OK
    assert n.value >= 7 * 2 * 4 * (64 + 2) * 4 and n1 >= 2 * 4 * (64 + 2) * 4 and n.value > n1


def test_forward_split_table_and_rules():
    """fa_forward_split: the per-shape table keeps the forward whole where its
    query blocks fill the device (every workload shape) or where chunks would
    be short, and splits few long sequences; an explicit kv_splits sets the
    chunk count; every error is returned before any HIP call."""
    lib = _lib.load()
    n = ctypes.c_size_t(0)

    def ws(p):
        assert lib.fa_forward_split_workspace_size(ctypes.byref(p), ctypes.byref(n)) == _lib.FA_OK
        return n.value

    f16, bf16, f32 = _lib.FA_F16, _lib.FA_BF16, _lib.FA_F32
    assert ws(prob(batch=8, heads=8, seq_q=2048, seq_kv=2048, causal=1, mod_kind=1)) == 0      # prefill
    assert ws(prob(batch=4, heads=16, seq_q=4096, seq_kv=4096, head_dim=128, dtype=bf16)) == 0
    assert ws(prob(batch=1, heads=2, seq_q=256, seq_kv=256, dtype=f32)) == 0
    assert ws(prob(batch=1, heads=1, seq_q=131072, seq_kv=131072, head_dim=512, dtype=f32, causal=1)) == 0
    assert ws(prob(batch=1, heads=1, seq_q=1000, seq_kv=1000, causal=1)) == 0                 # short chunks
    long_row = 1 * 2 * 16384 * (128 + 2) * 4                                                   # one chunk's partials
    big = ws(prob(batch=1, heads=2, seq_q=16384, seq_kv=16384, head_dim=128, causal=1))
    assert big >= 2 * long_row and big % 256 == 0
    assert ws(prob(batch=1, heads=2, seq_q=16384, seq_kv=16384, head_dim=128, causal=1, kv_splits=1)) == 0
    # causal with 2 <= R < 4 (256 CUs without a GPU): at head_dim 64 the whole forward runs on 64-query halves
    # where they apply (B H (n + 1) below the 768 slots) and the table keeps it whole; where they do not, and
    # at head_dim 128, it splits in 5 chunks
    assert ws(prob(batch=2, heads=4, seq_q=8192, seq_kv=8192, causal=1, mod_kind=1)) == 0
    assert ws(prob(batch=1, heads=8, seq_q=8192, seq_kv=8192, causal=1, mod_kind=1)) == 0
    assert ws(prob(batch=1, heads=3, seq_q=32768, seq_kv=32768, causal=1)) == 1 * 3 * 32768 * 5 * (64 + 2) * 4
    assert ws(prob(batch=1, heads=4, seq_q=16384, seq_kv=16384, head_dim=128, causal=1)) == \
        1 * 4 * 16384 * 5 * (128 + 2) * 4
    assert ws(prob(batch=1, heads=2, seq_q=16384, seq_kv=16384, head_dim=128, causal=1, kv_splits=4)) == \
        4 * long_row
    # chunks are whole 64-key tiles: 5 chunks of 80 keys become 128-key chunks, 4 in all
    assert ws(prob(seq_q=100, seq_kv=400, kv_splits=5)) == 2 * 4 * 100 * 4 * (64 + 2) * 4
    assert lib.fa_forward_split_workspace_size(ctypes.byref(prob(head_dim=512, dtype=f32, kv_splits=4)),
                                               ctypes.byref(n)) == UNSUP
    # a caller-defined mod is split only on request: the table keeps it whole
    assert ws(prob(seq_q=4096, seq_kv=4096, batch=1, heads=1, mod_kind=_lib.FA_MOD_CUSTOM, custom_mod=A[10])) == 0
    assert ws(prob(mod_kind=_lib.FA_MOD_CUSTOM, custom_mod=A[10], kv_splits=2)) == 2 * 4 * 100 * 2 * (64 + 2) * 4
    assert lib.fa_forward_split_workspace_size(ctypes.byref(prob(mod_kind=_lib.FA_MOD_CUSTOM, custom_mod=A[10],
                                                                 dtype=f32, head_dim=512, kv_splits=4)),
                                               ctypes.byref(n)) == UNSUP
    assert lib.fa_forward_split_workspace_size(ctypes.byref(prob(kv_splits=-1)), ctypes.byref(n)) == INVALID
    assert lib.fa_forward_split_workspace_size(ctypes.byref(prob()), None) == INVALID

    def fs(p, ws_ptr=A[11], ws_bytes=1 << 30, q=A[0]):
        return lib.fa_forward_split(ctypes.byref(p), q, A[1], A[2], A[3], A[4], ws_ptr, ws_bytes, None)

    split = prob(seq_q=100, seq_kv=400, kv_splits=4)
    need = ws(split)
    assert fs(split, ws_bytes=need - 1) == WS
    assert fs(split, ws_ptr=None) == INVALID
    assert fs(split, ws_ptr=ctypes.c_void_p(0x10010)) == INVALID     # not 256-byte aligned
    assert fs(split, q=None) == INVALID
    assert fs(prob(seq_q=100, seq_kv=400, kv_splits=4, scale=0.0)) == UNSUP
    assert fs(prob(head_dim=512, dtype=f32, kv_splits=4)) == UNSUP


def test_score_mod_create_compiles_and_reports_errors():
    """fa_score_mod_create compiles the caller's functions into the generic
    kernels with the run-time compiler (no GPU needed for that) and returns
    FA_ERR_COMPILE with the compiler's log for a broken source."""
    lib = _lib.load()
    good = b"""
    __device__ float fa_score_mod(float s, int b, int h, int q, int k, const float* p) { return s * 0.5f + p[0]; }
    __device__ float fa_score_mod_grad(float s, int b, int h, int q, int k, const float* p) { return 0.5f; }
    """
    h = ctypes.c_void_p()
    log = ctypes.create_string_buffer(1 << 14)
    assert lib.fa_score_mod_create(good, ctypes.byref(h), log, len(log)) == _lib.FA_OK
    assert h.value
    assert lib.fa_score_mod_destroy(h) == _lib.FA_OK
    bad = b"__device__ float fa_score_mod(float s) { return s + ; }"
    h2 = ctypes.c_void_p()
    assert lib.fa_score_mod_create(bad, ctypes.byref(h2), log, len(log)) == _lib.FA_ERR_COMPILE
    assert not h2.value and b"error" in log.value
    assert lib.fa_score_mod_create(None, ctypes.byref(h2), None, 0) == INVALID
    assert lib.fa_score_mod_destroy(None) == INVALID
    # a custom mod needs its handle; fa_decode and 16-bit kernels stop at head_dim 128
    assert fwd(prob(mod_kind=_lib.FA_MOD_CUSTOM)) == INVALID
    assert fwd(prob(mod_kind=_lib.FA_MOD_CUSTOM, custom_mod=A[10], dtype=_lib.FA_F16, head_dim=512)) == UNSUP
    assert dec(prob(seq_q=1, mod_kind=_lib.FA_MOD_CUSTOM, custom_mod=A[10], dtype=_lib.FA_F32, head_dim=512)) == UNSUP
    # fa_decode takes a caller-defined mod in whole 64-key chunks (the forward's split kernel)
    n = ctypes.c_size_t(0)
    assert lib.fa_decode_workspace_size(ctypes.byref(prob(seq_q=1, seq_kv=1000, kv_splits=4, mod_kind=_lib.FA_MOD_CUSTOM,
                                                           custom_mod=A[10])), ctypes.byref(n)) == _lib.FA_OK
    assert n.value == 2 * 4 * 1 * 4 * (64 + 2) * 4   # ceil(1000 / 4) = 250 -> 256-key chunks, 4 of them
