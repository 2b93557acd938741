"""Race check: the library built with FA_DEBUG_BARRIERS (every workgroup
barrier and every wait for a wave's loads first drains all of the wave's
outstanding memory operations, so nothing is in flight across a barrier)
must give bitwise the results of the normal library.  The two builds do the
same arithmetic in the same order; a difference means a wave read LDS before
its writer had finished, which the drained build cannot do.

Every kernel family is covered: the 16-bit and fp32 forward and backward
(separate dQ pass, deterministic), the split forward, decode (one query and
a short block), and a caller-defined score_mod (compiled at run time by each
library with its own barriers).
"""
import ctypes
import os

import pytest
import torch

import tiled_online_softmax_flashattention_amd as fa
import workloads as W
from tiled_online_softmax_flashattention_amd import _lib
from parity import MOD_NAME, say, to_dev

pytestmark = pytest.mark.gpu

RACECHECK = os.path.join(os.path.dirname(_lib.__file__), "libfa_mi355x_racecheck.so")

SOFTCAP = """
__device__ float fa_score_mod(float s, int b, int h, int q, int k, const float* p) { return p[0] * tanhf(s / p[0]); }
__device__ float fa_score_mod_grad(float s, int b, int h, int q, int k, const float* p) {
  const float t = tanhf(s / p[0]);
  return 1.0f - t * t;
}
"""


@pytest.fixture(scope="module")
def libs(gpu_lib):
    if not os.path.exists(RACECHECK):
        raise RuntimeError(f"{RACECHECK} is not built (tiled_online_softmax_flashattention_amd.build)")
    rc = ctypes.CDLL(RACECHECK)
    for name, (res, args) in _lib.SIGNATURES.items():
        f = getattr(rc, name)
        f.restype, f.argtypes = res, args
    assert rc.fa_abi_version() == _lib.FA_ABI_VERSION
    return {"normal": _lib.load(), "racecheck": rc}


def P(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def run_all(lib, p, x, *, backward=True, split=0, decode=False):
    """Forward (or split forward / decode) and backward through one library's
    C ABI; returns the output tensors."""
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    q, k, v = x["q"], x["k"], x["v"]
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    n = ctypes.c_size_t(0)
    if decode:
        assert lib.fa_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
        ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device="cuda")
        assert lib.fa_decode(ctypes.byref(p), P(q), P(k), P(v), P(out), P(lse), P(ws), ws.numel(), st) == 0
    elif split:
        assert lib.fa_forward_split_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0 and n.value > 0
        ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
        assert lib.fa_forward_split(ctypes.byref(p), P(q), P(k), P(v), P(out), P(lse), P(ws), ws.numel(), st) == 0
    else:
        assert lib.fa_forward(ctypes.byref(p), P(q), P(k), P(v), P(out), P(lse), st) == 0
    res = {"o": out, "lse": lse}
    if backward:
        assert lib.fa_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
        ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device="cuda")
        g = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        assert lib.fa_backward(ctypes.byref(p), P(q), P(k), P(v), P(out), P(lse), P(x["dout"]), P(g[0]), P(g[1]),
                               P(g[2]), P(ws), ws.numel(), st) == 0
        res.update(dq=g[0], dk=g[1], dv=g[2])
    torch.cuda.synchronize()
    return res


def compare(a, b, label):
    for name in a:
        same = torch.equal(torch.nan_to_num(a[name], nan=7.0), torch.nan_to_num(b[name], nan=7.0)) and \
            torch.equal(torch.isnan(a[name]), torch.isnan(b[name]))
        assert same, f"{label}: {name} differs between the normal and the race-check build"


# name, dtype, D, causal, mod, key mask, block mask, Sq, Skv, q_offset
CASES = [
    ("f16 causal ALiBi", "f16", 64, True, W.MOD_ALIBI, False, False, 700, 700, 0),
    ("bf16 mask checker blocks", "bf16", 128, False, W.MOD_CHECKERBOARD, True, True, 333, 650, 0),
    ("f16 D128 causal offset", "f16", 128, True, W.MOD_NONE, False, False, 200, 520, 320),
    ("bf16 D64 blocks causal", "bf16", 64, True, W.MOD_NONE, True, True, 513, 513, 0),
    ("f32 D64 causal ALiBi", "f32", 64, True, W.MOD_ALIBI, False, False, 300, 300, 0),
    ("f32 D128 mask", "f32", 128, False, W.MOD_CHECKERBOARD, True, False, 260, 390, 0),
    ("f32 D512 causal", "f32", 512, True, W.MOD_NONE, False, False, 97, 97, 0),
    ("f32 D512 mask blocks", "f32", 512, False, W.MOD_ALIBI, True, True, 80, 200, 0),
]


def _inputs(dtype, D, causal, mod, mask, blk, Sq, Skv, wid=150):
    w = W.Workload("race check", wid, 2, 3, Sq, Skv, D, dtype, causal=causal, mod=mod, key_mask=mask)
    x = to_dev(w.make())
    if blk:
        x["block_mask"] = W.bernoulli_block_mask(2, 3, Sq, Skv, wid, p_keep=0.7).cuda()
    return w, x


@pytest.mark.parametrize("name,dtype,D,causal,mod,mask,blk,Sq,Skv,off", CASES)
def test_race_check_forward_backward(libs, name, dtype, D, causal, mod, mask, blk, Sq, Skv, off):
    w, x = _inputs(dtype, D, causal, mod, mask, blk, Sq, Skv)
    p = fa.problem(x["q"], x["k"], causal=causal, key_mask=x.get("key_mask"), score_mod=MOD_NAME[mod],
                   scale=w.scale, q_offset=off, block_mask=x.get("block_mask"), dq_mode="separate")
    say(f"[race check] {name}")
    a = run_all(libs["normal"], p, x)
    b = run_all(libs["racecheck"], p, x)
    compare(a, b, name)


@pytest.mark.parametrize("dtype,D,Sq,Skv,causal,n", [("f16", 64, 1, 5000, False, 0), ("bf16", 128, 16, 3000, True, 0),
                                                     ("f32", 64, 16, 2100, True, 0), ("f16", 128, 600, 1500, True, 3),
                                                     ("f32", 128, 300, 900, False, 4)])
def test_race_check_decode_and_split(libs, dtype, D, Sq, Skv, causal, n):
    """Decode (one query, a short block after a cache) and the forward split
    over keys (with its merge)."""
    w, x = _inputs(dtype, D, causal, W.MOD_ALIBI, False, False, Sq, Skv, wid=151)
    decode = Sq <= 64
    p = fa.problem(x["q"], x["k"], causal=causal, score_mod="alibi", scale=w.scale, q_offset=Skv - Sq, kv_splits=n)
    say(f"[race check] {'decode' if decode else 'split forward'} {dtype} D{D} Sq={Sq} Skv={Skv} n={n}")
    a = run_all(libs["normal"], p, x, backward=False, decode=decode, split=0 if decode else n)
    b = run_all(libs["racecheck"], p, x, backward=False, decode=decode, split=0 if decode else n)
    compare(a, b, "decode/split")


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("f32", 128)])
def test_race_check_caller_mod(libs, dtype, D):
    """A caller-defined score_mod: each library compiles it with its own
    barriers (run time), forward and backward."""
    w, x = _inputs(dtype, D, True, W.MOD_NONE, True, False, 400, 400, wid=152)
    params = torch.tensor([2.0], dtype=torch.float32, device="cuda")
    res = {}
    for name, lib in libs.items():
        h = ctypes.c_void_p()
        log = ctypes.create_string_buffer(1 << 14)
        assert lib.fa_score_mod_create(SOFTCAP.encode(), ctypes.byref(h), log, len(log)) == 0, log.value
        p = fa.problem(x["q"], x["k"], causal=True, key_mask=x["key_mask"], scale=w.scale, dq_mode="separate")
        p.mod_kind, p.custom_mod, p.mod_params = _lib.FA_MOD_CUSTOM, h.value, params.data_ptr()
        say(f"[race check] caller mod {dtype} D{D} ({name})")
        res[name] = run_all(lib, p, x)
        assert lib.fa_score_mod_destroy(h) == 0
    compare(res["normal"], res["racecheck"], "caller mod")
