// C ABI of the attention library: argument validation on the host, choice of
// kernel instance, workspace sizing and launches on the caller's stream.
//
// Validation touches no HIP API, so every error path can be exercised on a
// machine without a GPU.  Nothing here allocates device memory.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa_mi355x.h"
#include "fa_launch.hpp"
#include "fa_rtc.hpp"

namespace {

constexpr int64_t kMaxI32 = 2147483647;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device (MI355X: 256; fewer in a partitioned
// mode), read once per device; 256 when no device answers (host-only use of
// the workspace queries).
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cus[dev] = n;
  }
  return cus[dev];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool head_dim_supported(int32_t dtype, int64_t d) {
  if (dtype == FA_F32) return d == 64 || d == 128 || d == 512;
  return d == 64 || d == 128;
}

// Checks shared by every entry point.  Pure host logic.
fa_status validate_problem(const fa_problem* p) {
  if (!p) return FA_ERR_INVALID_ARGUMENT;
  if (p->batch <= 0 || p->heads <= 0 || p->seq_q <= 0 || p->seq_kv <= 0 || p->head_dim <= 0)
    return FA_ERR_INVALID_ARGUMENT;
  if (p->dtype != FA_F32 && p->dtype != FA_F16 && p->dtype != FA_BF16) return FA_ERR_INVALID_ARGUMENT;
  if (p->causal != 0 && p->causal != 1) return FA_ERR_INVALID_ARGUMENT;
  if (p->mod_kind != FA_MOD_NONE && p->mod_kind != FA_MOD_ALIBI && p->mod_kind != FA_MOD_CHECKERBOARD &&
      p->mod_kind != FA_MOD_CUSTOM)
    return FA_ERR_INVALID_ARGUMENT;
  if (p->mod_kind == FA_MOD_CUSTOM && !p->custom_mod) return FA_ERR_INVALID_ARGUMENT;
  if (p->mod_params && ((uintptr_t)p->mod_params & 3u)) return FA_ERR_INVALID_ARGUMENT;
  if (!isfinite(p->scale)) return FA_ERR_INVALID_ARGUMENT;
  // the kernels mask scores as -inf before multiplying by scale and keep the
  // backward's log-sum-exp in units of scale * q.k: scale must be positive
  if (!(p->scale > 0.f)) return FA_ERR_UNSUPPORTED;
  if (p->mod_kind == FA_MOD_CHECKERBOARD && (!isfinite(p->checker_even) || !isfinite(p->checker_odd)))
    return FA_ERR_INVALID_ARGUMENT;
  if (p->q_offset < 0) return FA_ERR_INVALID_ARGUMENT;
  if (p->alibi_slopes && ((uintptr_t)p->alibi_slopes & 3u)) return FA_ERR_INVALID_ARGUMENT;
  if (!head_dim_supported(p->dtype, p->head_dim)) return FA_ERR_UNSUPPORTED;
  // index arithmetic inside the kernels is 32-bit per (batch, head) slice
  if (p->batch * p->heads > kMaxI32 / 8) return FA_ERR_UNSUPPORTED;
  if (p->seq_q > kMaxI32 / p->head_dim || p->seq_kv > kMaxI32 / p->head_dim) return FA_ERR_UNSUPPORTED;
  if (p->q_offset > kMaxI32 - p->seq_q) return FA_ERR_UNSUPPORTED;
  if (p->batch > kMaxI32 / p->seq_kv) return FA_ERR_UNSUPPORTED;
  // block-sparse loops keep their tile lists in LDS, sized for this length
  if (p->block_mask && (p->seq_q > FA_BLOCK_MASK_MAX_SEQ || p->seq_kv > FA_BLOCK_MASK_MAX_SEQ))
    return FA_ERR_UNSUPPORTED;
  if (p->dq_mode != FA_DQ_AUTO && p->dq_mode != FA_DQ_SEPARATE && p->dq_mode != FA_DQ_ATOMIC)
    return FA_ERR_INVALID_ARGUMENT;
  if (p->kv_splits < 0) return FA_ERR_INVALID_ARGUMENT;
  if (p->kv_splits > FA_MAX_KV_SPLITS) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// The atomic dQ mode's buffer descriptors bound a (batch, head) slice of the
// fp32 accumulator by a 32-bit byte count.
bool dq_atomic_fits(const fa_problem* p) {
  return p->dtype != FA_F32 && p->seq_q * p->head_dim < ((int64_t)1 << 28);
}

// Measured choice of FA_DQ_AUTO per (dtype, head_dim): true = atomic.  The
// atomic key/value pass loses at both 16-bit head dims on MI355X: its fp32
// atomics (B*H*Sq*D per 128-key block) run at about 2 TB/s of L2 atomic
// throughput, so the pass takes 233 vs 80 us (prefill f16 8x8x2048x64,
// causal) and 3.28 vs 1.40 ms (key-padding bf16 4x16x4096x128), more than the
// separate query pass it replaces (63 us, 0.99 ms).
bool dq_atomic_by_default(const fa_problem* p) {
  (void)p;
  return false;
}

// Whether fa_backward forms dQ with atomics for this problem (when both
// passes run).  FA_ERR_UNSUPPORTED for an explicit atomic request it cannot
// serve.
fa_status resolve_dq_atomic(const fa_problem* p, bool* atomic) {
  if (p->mod_kind == FA_MOD_CUSTOM) {   // the caller-defined score_mod kernels have the separate passes only
    if (p->dq_mode == FA_DQ_ATOMIC) return FA_ERR_UNSUPPORTED;
    *atomic = false;
    return FA_OK;
  }
  if (p->dq_mode == FA_DQ_ATOMIC) {
    if (!dq_atomic_fits(p)) return FA_ERR_UNSUPPORTED;
    *atomic = true;
  } else {
    *atomic = p->dq_mode == FA_DQ_AUTO && dq_atomic_fits(p) && dq_atomic_by_default(p);
  }
  return FA_OK;
}

bool tensors_ok(std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (!x || !aligned16(x)) return false;
  return true;
}

int block_q_fwd(const fa_problem* p) {
  return p->dtype == FA_F32 ? fa::fwd32_block_q((int)p->head_dim) : fa::fwd16_block_q((int)p->head_dim);
}

fa::AttnArgs make_args(const fa_problem* p) {
  fa::AttnArgs a = {};
  a.B = (int)p->batch;
  a.H = (int)p->heads;
  a.Sq = (int)p->seq_q;
  a.Skv = (int)p->seq_kv;
  a.scale = p->scale;
  a.scale_log2 = p->scale * fa::kLog2e;
  a.key_mask = p->key_mask;
  a.alibi_slopes = p->mod_kind == FA_MOD_ALIBI ? p->alibi_slopes : nullptr;
  a.even_nat = p->checker_even;
  a.odd_nat = p->checker_odd;
  a.even_log2 = p->checker_even * fa::kLog2e;
  a.odd_log2 = p->checker_odd * fa::kLog2e;
  a.causal = p->causal;
  a.q_off = (int)p->q_offset;
  a.block_mask = p->block_mask;
  a.bm_rows = (int)((p->seq_q + FA_BLOCK_MASK_BLOCK - 1) / FA_BLOCK_MASK_BLOCK);
  a.bm_cols = (int)((p->seq_kv + FA_BLOCK_MASK_BLOCK - 1) / FA_BLOCK_MASK_BLOCK);
  a.mod_params = p->mod_params;
  return a;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct BwdLayout {
  size_t delta_off, lse2_off, dq_acc_off, total;
};

// Workspace: delta and lse2 rows, and in the atomic dQ mode the fp32 dQ
// accumulator (B, H, Sq, D).
BwdLayout bwd_layout(const fa_problem* p, bool dq_atomic) {
  const size_t rows = (size_t)p->batch * p->heads * p->seq_q;
  BwdLayout l;
  l.delta_off = 0;
  l.lse2_off = round_up(rows * sizeof(float), 256);
  l.dq_acc_off = l.lse2_off + round_up(rows * sizeof(float), 256);
  l.total = l.dq_acc_off + (dq_atomic ? round_up(rows * (size_t)p->head_dim * sizeof(float), 256) : 0);
  return l;
}

constexpr int64_t kMaxDecodeQ = 64;   // longest query block fa_decode takes

// Keys the decode queries see: all of them, or with causal only keys up to
// the last query's position.
int decode_kv_len(const fa_problem* p) {
  const int64_t last = p->q_offset + p->seq_q;   // last query position + 1
  const int64_t n = p->causal ? (last < p->seq_kv ? last : p->seq_kv) : p->seq_kv;
  return (int)n;
}

// Split of the key axis and workspace bytes (one (D + 2)-float partial per
// query row and chunk).
// fp32 query blocks of at most 64 rows split over keys run one wave per 32
// rows in a workgroup (the launcher's choice, mirrored here for the split
// sizes): 8 one-wave workgroups per CU at head_dim 64, 4 at 128 (their LDS),
// 4 two-wave workgroups (registers at 64, LDS at 128).  Returns the
// workgroups per CU, 0 outside that case.
int f32_short(const fa_problem* p) {
  if (p->dtype != FA_F32 || p->head_dim > 128 || p->seq_q > 64 || p->block_mask || p->mod_kind == FA_MOD_CUSTOM)
    return 0;
  return p->seq_q <= 32 && p->head_dim == 64 ? 8 : 4;
}

size_t decode_ws(const fa_problem* p, int* n_split, int* chunk) {
  const int BH = (int)(p->batch * p->heads);
  if (p->kv_splits > 0) {   // the caller's split: about kv_splits chunks
    const int len = decode_kv_len(p);
    *chunk = (len + p->kv_splits - 1) / p->kv_splits;
  } else {
    // the chooser aims at two workgroups per CU; of the small fp32 ones
    // f32_short(p) fit a CU
    const int scale = f32_short(p) ? f32_short(p) / 2 : 1;
    *n_split = fa::decode_choose_split(BH, decode_kv_len(p), chunk, device_cus() * scale);
  }
  if (p->seq_q > 1 || p->mod_kind == FA_MOD_CUSTOM) *chunk = (*chunk + 63) / 64 * 64;   // whole 64-key tiles of the forward
  *n_split = (decode_kv_len(p) + *chunk - 1) / *chunk;
  return round_up((size_t)BH * (size_t)p->seq_q * (size_t)(*n_split) * (size_t)(p->head_dim + 2) * sizeof(float),
                  256);
}

// Workgroups of the forward resident on the device at once: its CUs times
// the workgroups per CU that the kernel's registers allow.
int64_t forward_slots(const fa_problem* p) {
  const int64_t cus = device_cus();
  if (f32_short(p)) return f32_short(p) * cus;
  if (p->dtype == FA_F32) return cus;
  return p->head_dim == 64 ? 3 * cus : 2 * cus;
}

// 16-bit forward with 64-query blocks and two waves per 32 queries (each one
// key half of every tile, merged at the end) when the 128-query blocks use
// the device's workgroup slots badly.  Causal: block b of a slice visits
// b + 1 key tiles of 128, so the longest block outlasts a slot's share of
// the work when r = B H (nqb + 1) / (2 slots) < 1.  Not causal: the blocks
// fill u = B H nqb / slots of the device.  The halves pay from r < 1/2 at
// head_dim 64, r < 0.6 at 128 and u <= 1/2 (MI355X, same box, us):
//  * causal f16 ALiBi, head_dim 64: r = 0.08 1x1x16384 231 -> 130; 0.34
//    1x8x8192 126 -> 91; 0.35 4x8x2048 36.8 -> 28.1; 0.44 5x8x2048 39.1 ->
//    36.5; 0.52 3x8x4096 78.3 -> 75.0; 0.53 6x8x2048 42.2 both; 0.54
//    8x8x1536 33.4 -> 33.8; 0.71 8x8x2048 50.7 -> 53.7.
//  * causal, head_dim 128: 0.13 1x1x16384 326 -> 201; 0.26 1x8x4096 88.1 ->
//    61.9; 0.51 1x8x8192 200 -> 163; 0.53 4x8x2048 58.4 -> 52.6; 0.66
//    5x8x2048 63.9 -> 68.1; 0.76 1x12x8192 238 -> 240; 1.06 8x8x2048 90.7 ->
//    101.4.
//  * not causal, head_dim 64 (f16 ALiBi): u = 0.17 1x1x16384 213 -> 129;
//    0.33 1x8x4096 56.9 -> 48.9; 0.5 3x8x2048 41.6 -> 37.3; 0.67 2x8x4096
//    86.2 -> 93.9; 0.83 5x8x2048 60.8 -> 61.0.  head_dim 128 (bf16
//    checkerboard, key mask): 0.25 1x4x4096 94.1 -> 63.0; 0.5 1x8x4096 94.9
//    -> 86.9; 0.75 3x8x2048 68.2 -> 74.8; 1.0 2x8x4096 141 -> 170.
// A block mask takes the same layout, so a mask with every block set gives
// the dense result bit for bit.
bool forward_halves(const fa_problem* p, int64_t nqb) {
  if (p->dtype == FA_F32) return false;
  const int64_t bh = p->batch * p->heads, slots = forward_slots(p);
  if (!p->causal) return 2 * bh * nqb <= slots;
  return p->head_dim == 64 ? bh * (nqb + 1) < slots : 5 * bh * (nqb + 1) < 6 * slots;
}

// The 16-bit dQ and dK/dV passes on 64-row blocks (two waves per 32 rows,
// each over one half of every tile, their sums added at the end) when the
// 128-row blocks use the passes' workgroup slots badly: 2 per CU at head_dim
// 64, 1 at 128; n = the pass's own 128-row blocks (queries for dQ, keys for
// dK/dV).  Causal when r = B H (n + 1) / (2 slots) < 0.6, otherwise when
// 2 B H n <= slots.  Measured on MI355X (both passes, f16 causal ALiBi or
// bf16 checkerboard with a key mask, same box, us):
//  * head_dim 64: r = 0.13 1x1x16384 517 -> 316; 0.27 2x8x2048 74.4 -> 55.0;
//    0.51 1x8x8192 314 -> 276; 0.53 4x8x2048 89.4 -> 84.0; 1.06 8x8x2048
//    145.6 -> 158.4.  Not causal: u = 0.5 1x8x4096 137.7 -> 131.5; 1.0
//    2x8x4096 235.6 -> 257.1.
//  * head_dim 128: r = 0.25 1x1x16384 912 -> 598; 0.52 1x8x4096 244 -> 188;
//    1.03 2x8x4096 283 -> 356; 2.1 8x8x2048 324 -> 412.  Not causal: 0.5
//    1x4x4096 220 -> 166; 1.0 1x8x4096 236 -> 305.
bool backward_halves(const fa_problem* p, int64_t n) {
  const int64_t bh = p->batch * p->heads, slots = (p->head_dim == 64 ? 2 : 1) * device_cus();
  return p->causal ? 5 * bh * (n + 1) < 6 * slots : 2 * bh * n <= slots;
}

// Per-shape table of fa_forward_split (kv_splits = 0): how many key chunks,
// from sweeps of the chunk count on MI355X over 16-bit and fp32 shapes with
// 64 .. 1024 query blocks and 4096 .. 32768 keys.  R is the ratio of the
// device's workgroup slots to the query blocks (with causal twice that: a
// causal block averages half the keys), i.e. about how many times the
// longest block's work exceeds one slot's fair share.
//  * 16-bit, causal, R >= 4: R - 1 chunks.  The non-empty (block, chunk)
//    pairs, about blocks (n + 1) / 2, then just fit in the slots and start
//    together; one more chunk starts the last full chunks in a second round
//    (1 x 1 x 32768 x 128: 421 us at 3 chunks, 588 at 4, 700 unsplit).
//  * 16-bit, causal, 2 <= R < 4, long sequences (>= 16384 keys at head_dim
//    128, >= 8192 at 64): 5 chunks, fine grains over several rounds
//    (1 x 4 x 16384 x 128: 351 us vs 404 unsplit with 128-query blocks);
//    shorter sequences stay whole (2 x 8 x 4096 x 128: 110 us unsplit, 117
//    at 2 chunks).  At head_dim 64 the whole forward on 64-query halves
//    (forward_halves) beats the 5 chunks where it applies: 2 x 4 x 8192: 93
//    vs 114 us, 1 x 8 x 8192: 94 vs 115, 1 x 4 x 16384: 177 vs 198, 1 x 2 x
//    32768: 389 vs 390; where it does not (1 x 3 x 32768, r = 0.50) the
//    chunks stay (554 vs 588).  At head_dim 128 the chunks mostly still win
//    over the halves (1 x 2 x 32768: 623 vs 703 us, 1 x 2 x 24576: 390 vs
//    486, 1 x 3 x 16384: 284 vs 415; 1 x 4 x 16384: 332 vs 293).
//  * 16-bit, not causal: R chunks when R >= 2 (1 x 2 x 8192 x 128: 90 us at
//    4 chunks vs 169 unsplit).
//  * fp32 (one workgroup per CU, 4x the time per key): 2R chunks with causal,
//    R without, when R >= 2 (1 x 1 x 8192 x 64 causal: 128 us at 16 chunks
//    vs 816 unsplit).  fp32 blocks of at most 64 rows run in small
//    workgroups, several per CU: one chunk per slot, R without the causal
//    factor (8 x 8 x 16 x 64 after 32752 cached keys: 32 chunks).
//  * Chunks of at least kMinSplitChunk keys (fp32: a quarter), so that the
//    partials' write and merge stay small against the chunk's arithmetic.
// Everything else (R < 2: the query blocks already fill the device, e.g.
// 8 x 8 x 2048 x 64, where 2 chunks cost 83 us against 54) stays whole, and
// so do sequences shorter than the sweeps went (kMinSplitKeys).
constexpr int kMinSplitChunk = 512;
constexpr int kMinSplitKeys = 4096;

int forward_choose_split(const fa_problem* p, int len) {
  if (p->mod_kind == FA_MOD_CUSTOM || p->head_dim > 128 || len < kMinSplitKeys) return 1;
  const int64_t blocks = p->batch * p->heads * ceil_div(p->seq_q, block_q_fwd(p));
  // fp32 blocks of at most 64 rows (small workgroups, usually after a KV
  // cache, where the causal rule does not halve a block's keys): one chunk
  // per free slot
  const int64_t R = (p->causal && !f32_short(p) ? 2 : 1) * forward_slots(p) / blocks;
  if (R < 2) return 1;
  int64_t n;
  if (f32_short(p)) n = R;
  else if (p->dtype == FA_F32) n = p->causal ? 2 * R : R;
  else if (!p->causal) n = R;
  else if (R >= 4) n = R - 1;
  else if (p->head_dim == 64 && forward_halves(p, ceil_div(p->seq_q, block_q_fwd(p)))) n = 1;
  else n = len >= (p->head_dim == 128 ? 16384 : 8192) ? 5 : 1;
  const int64_t most = len / (p->dtype == FA_F32 ? kMinSplitChunk / 4 : kMinSplitChunk);
  if (n > most) n = most;
  if (n > FA_MAX_KV_SPLITS) n = FA_MAX_KV_SPLITS;
  return n < 2 ? 1 : (int)n;
}

// Key split of fa_forward_split and its workspace bytes: one (D + 2)-float
// partial per query row and chunk; 0 bytes when the forward stays whole.
size_t forward_split_ws(const fa_problem* p, int* n_split, int* chunk) {
  const int len = decode_kv_len(p);   // keys the last query row sees
  const int n = p->kv_splits > 0 ? p->kv_splits : forward_choose_split(p, len);
  int c = (len + n - 1) / n;
  c = (c + 63) / 64 * 64;   // whole 64-key tiles
  *chunk = c;
  *n_split = (len + c - 1) / c;
  if (*n_split <= 1) return 0;
  return round_up((size_t)(p->batch * p->heads) * (size_t)p->seq_q * (size_t)(*n_split) *
                      (size_t)(p->head_dim + 2) * sizeof(float),
                  256);
}

// The forward over key chunks, then the merge of each row's partials, on a
// validated problem with `ws` holding n_split partials per row (many_rows:
// the forward's merge with several rows per workgroup; else the decode's).
fa_status split_forward_launch(const fa_problem* p, fa::AttnArgs a, int n_split, int chunk, void* ws, hipStream_t st,
                               bool many_rows) {
  const int D = (int)p->head_dim;
  const bool mask = p->key_mask != nullptr, causal = p->causal != 0;
  a.partial = (float*)ws;
  a.n_split = n_split;
  a.chunk = chunk;
  a.n_qblocks = (int)ceil_div(p->seq_q, block_q_fwd(p));
  if (p->mod_kind == FA_MOD_CUSTOM) {
    const unsigned grid = (unsigned)(a.n_qblocks * p->batch * p->heads * n_split);
    const bool blk = p->block_mask != nullptr;
    const fa_status s = fa::custom_launch(p->custom_mod, 3, p->dtype, D, causal, mask, blk, a, grid,
                                          p->dtype == FA_F32 ? fa::fwd32_lds_bytes(D, blk) : 0, st);
    if (s != FA_OK) return s;
  } else {
    const hipError_t err = p->dtype == FA_F32 ? fa::launch_fwd32(a, D, p->mod_kind, causal, mask, st, true)
                                              : fa::launch_fwd16(a, p->dtype == FA_BF16, D, p->mod_kind, causal,
                                                                 mask, st, true);
    if (err != hipSuccess) return FA_ERR_HIP;
  }
  const int rows = (int)(p->batch * p->heads * p->seq_q);
  const hipError_t err = many_rows ? fa::launch_split_merge(a, p->dtype, D, rows, st)
                                   : fa::launch_decode_merge(a, p->dtype, D, rows, st);
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_forward(const fa_problem* p, const void* q, const void* k, const void* v, void* out,
                     float* lse, void* stream) {
  fa_status s = validate_problem(p);
  if (s != FA_OK) return s;
  if (!tensors_ok({q, k, v, out})) return FA_ERR_INVALID_ARGUMENT;
  if (lse && ((uintptr_t)lse & 3u)) return FA_ERR_INVALID_ARGUMENT;
  const int64_t nqb = ceil_div(p->seq_q, block_q_fwd(p));
  if (nqb * p->batch * p->heads > kMaxI32) return FA_ERR_UNSUPPORTED;

  fa::AttnArgs a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.n_qblocks = (int)nqb;
  hipStream_t st = (hipStream_t)stream;
  if (p->mod_kind == FA_MOD_CUSTOM) {
    const bool blk = p->block_mask != nullptr;
    return fa::custom_launch(p->custom_mod, 0, p->dtype, (int)p->head_dim, p->causal != 0, p->key_mask != nullptr,
                             blk, a, (unsigned)(nqb * p->batch * p->heads),
                             p->dtype == FA_F32 ? fa::fwd32_lds_bytes((int)p->head_dim, blk) : 0, st);
  }
  hipError_t err;
  if (p->dtype == FA_F32)
    err = fa::launch_fwd32(a, (int)p->head_dim, p->mod_kind, p->causal != 0, p->key_mask != nullptr, st);
  else
    err = fa::launch_fwd16(a, p->dtype == FA_BF16, (int)p->head_dim, p->mod_kind, p->causal != 0,
                           p->key_mask != nullptr, st, false, forward_halves(p, nqb));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_forward_split_workspace_size(const fa_problem* p, size_t* bytes) {
  fa_status s = validate_problem(p);
  if (s != FA_OK) return s;
  if (!bytes) return FA_ERR_INVALID_ARGUMENT;
  if (p->kv_splits > 1 && p->head_dim > 128) return FA_ERR_UNSUPPORTED;
  int n_split, chunk;
  *bytes = forward_split_ws(p, &n_split, &chunk);
  return FA_OK;
}

fa_status fa_forward_split(const fa_problem* p, const void* q, const void* k, const void* v, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  fa_status s = validate_problem(p);
  if (s != FA_OK) return s;
  if (p->kv_splits > 1 && p->head_dim > 128) return FA_ERR_UNSUPPORTED;
  int n_split, chunk;
  const size_t need = forward_split_ws(p, &n_split, &chunk);
  if (need == 0) return fa_forward(p, q, k, v, out, lse, stream);
  if (!tensors_ok({q, k, v, out})) return FA_ERR_INVALID_ARGUMENT;
  if (lse && ((uintptr_t)lse & 3u)) return FA_ERR_INVALID_ARGUMENT;
  if (!workspace || ((uintptr_t)workspace & 255u)) return FA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
  if (ceil_div(p->seq_q, block_q_fwd(p)) * p->batch * p->heads * n_split > kMaxI32) return FA_ERR_UNSUPPORTED;
  if (p->batch * p->heads * p->seq_q > kMaxI32) return FA_ERR_UNSUPPORTED;   // merge grid
  fa::AttnArgs a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  return split_forward_launch(p, a, n_split, chunk, workspace, (hipStream_t)stream, true);
}

fa_status fa_backward_workspace_size(const fa_problem* p, size_t* bytes) {
  fa_status s = validate_problem(p);
  if (s != FA_OK) return s;
  if (!bytes) return FA_ERR_INVALID_ARGUMENT;
  bool atomic = false;
  s = resolve_dq_atomic(p, &atomic);
  if (s != FA_OK) return s;
  *bytes = bwd_layout(p, atomic).total;
  return FA_OK;
}

fa_status fa_backward(const fa_problem* p, const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, void* stream) {
  fa_status s = validate_problem(p);
  if (s != FA_OK) return s;
  if (!tensors_ok({q, k, v, out, dout})) return FA_ERR_INVALID_ARGUMENT;
  // dq == NULL skips the query pass; dk and dv both NULL skip the key/value pass
  const bool want_q = dq != nullptr, want_kv = dk != nullptr || dv != nullptr;
  if (!want_q && !want_kv) return FA_ERR_INVALID_ARGUMENT;
  if (want_q && !tensors_ok({dq})) return FA_ERR_INVALID_ARGUMENT;
  if (want_kv && !tensors_ok({dk, dv})) return FA_ERR_INVALID_ARGUMENT;
  if (!lse || ((uintptr_t)lse & 3u)) return FA_ERR_INVALID_ARGUMENT;
  if (!workspace || ((uintptr_t)workspace & 255u)) return FA_ERR_INVALID_ARGUMENT;
  bool atomic = false;
  s = resolve_dq_atomic(p, &atomic);
  if (s != FA_OK) return s;
  atomic = atomic && want_q && want_kv;   // a single pass has no dQ to share
  const BwdLayout lay = bwd_layout(p, atomic);
  if (workspace_bytes < lay.total) return FA_ERR_WORKSPACE_TOO_SMALL;
  const int D = (int)p->head_dim;
  const bool f32 = p->dtype == FA_F32;
  const int64_t nkb = ceil_div(p->seq_kv, f32 ? fa::bwd32_block_kv(D) : fa::bwd16_block_kv());
  const int64_t nqb = ceil_div(p->seq_q, f32 ? fa::bwd32_block_q(D) : fa::bwd16_block_q());
  if ((nkb > nqb ? nkb : nqb) * p->batch * p->heads > kMaxI32) return FA_ERR_UNSUPPORTED;

  fa::AttnArgs a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = const_cast<void*>(out);
  a.lse = const_cast<float*>(lse);
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = (float*)((char*)workspace + lay.delta_off);
  a.lse2 = (float*)((char*)workspace + lay.lse2_off);
  a.dq_acc = atomic ? (float*)((char*)workspace + lay.dq_acc_off) : nullptr;
  a.n_qblocks = (int)nqb;
  if (!f32 && p->mod_kind != FA_MOD_CUSTOM) {
    a.dq_halves = backward_halves(p, ceil_div(p->seq_q, 128)) ? 1 : 0;
    a.kv_halves = !atomic && backward_halves(p, ceil_div(p->seq_kv, 128)) ? 1 : 0;
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  if (p->mod_kind == FA_MOD_CUSTOM) {   // preprocess (plain rows), then the run-time compiled passes
    err = fa::launch_bwd_pre(a, p->dtype, D, st, 0);
    if (err != hipSuccess) return FA_ERR_HIP;
    const bool causal = p->causal != 0, mask = p->key_mask != nullptr, blk = p->block_mask != nullptr;
    const unsigned bh = (unsigned)(p->batch * p->heads);
    const size_t lds = f32 ? fa::bwd32_lds_bytes(D, blk) : 0;
    if (want_q) {
      s = fa::custom_launch(p->custom_mod, 1, p->dtype, D, causal, mask, blk, a, (unsigned)nqb * bh, lds, st);
      if (s != FA_OK) return s;
    }
    if (want_kv)
      s = fa::custom_launch(p->custom_mod, 2, p->dtype, D, causal, mask, blk, a, (unsigned)nkb * bh, lds, st);
    return s;
  }
  if (f32) {   // fp32: preprocess kernel, then the passes
    err = fa::launch_bwd_pre(a, p->dtype, D, st);
    if (err != hipSuccess) return FA_ERR_HIP;
    err = fa::launch_bwd32(a, D, p->mod_kind, p->causal != 0, p->key_mask != nullptr, want_kv, want_q, st);
  } else {     // 16-bit: the query pass computes the preprocess itself
    err = fa::launch_bwd16(a, p->dtype == FA_BF16, D, p->mod_kind, p->causal != 0, p->key_mask != nullptr,
                           want_kv, want_q, atomic, st);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_decode_workspace_size(const fa_problem* p, size_t* bytes) {
  fa_status s = validate_problem(p);
  if (s != FA_OK) return s;
  if (!bytes) return FA_ERR_INVALID_ARGUMENT;
  if (p->seq_q > kMaxDecodeQ) return FA_ERR_INVALID_ARGUMENT;
  if (p->head_dim > 128) return FA_ERR_UNSUPPORTED;
  int n_split, chunk;
  *bytes = decode_ws(p, &n_split, &chunk);
  return FA_OK;
}

}  // extern "C"

namespace {

// Checks shared by both decode entry points (pure host logic).
fa_status validate_decode(const fa_problem* p, const void* q, const void* k, const void* v, void* out,
                          float* lse) {
  fa_status s = validate_problem(p);
  if (s != FA_OK) return s;
  if (p->seq_q > kMaxDecodeQ) return FA_ERR_INVALID_ARGUMENT;
  if (p->head_dim > 128) return FA_ERR_UNSUPPORTED;
  if (!tensors_ok({q, k, v, out})) return FA_ERR_INVALID_ARGUMENT;
  if (lse && ((uintptr_t)lse & 3u)) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

// The decode launches on a validated problem with `ws` holding at least
// decode_ws(p) bytes.
fa_status decode_launch(const fa_problem* p, const void* q, const void* k, const void* v, void* out, float* lse,
                        void* ws, void* stream) {
  int n_split, chunk;
  decode_ws(p, &n_split, &chunk);
  fa::AttnArgs a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.partial = (float*)ws;
  a.n_split = n_split;
  a.chunk = chunk;
  hipStream_t st = (hipStream_t)stream;
  const int D = (int)p->head_dim;
  const bool mask = p->key_mask != nullptr;
  if (p->seq_q == 1 && p->mod_kind != FA_MOD_CUSTOM)
    return fa::launch_decode(a, p->dtype, D, p->mod_kind, mask, st) == hipSuccess ? FA_OK : FA_ERR_HIP;
  // a short query block, or a caller-defined score_mod (whose only key-split
  // kernel is the forward's): the forward split over the keys, then the merge
  return split_forward_launch(p, a, n_split, chunk, ws, st, false);
}

// Fixed device scratch of fa_decode_noalloc: the per-chunk partials live in
// this array instead of a caller workspace.  Every device the library runs
// on holds its own copy (module-scope device memory) until the process ends.
// Host code never uses the array's name as an address: its device address
// is taken once per device with hipGetSymbolAddress and kept below.
static __device__ __attribute__((aligned(256))) unsigned char scratch[FA_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first
// call on that device (with that device current).
fa_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_decode(const fa_problem* p, const void* q, const void* k, const void* v, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  fa_status s = validate_decode(p, q, k, v, out, lse);
  if (s != FA_OK) return s;
  if (!workspace || ((uintptr_t)workspace & 255u)) return FA_ERR_INVALID_ARGUMENT;
  int n_split, chunk;
  if (workspace_bytes < decode_ws(p, &n_split, &chunk)) return FA_ERR_WORKSPACE_TOO_SMALL;
  return decode_launch(p, q, k, v, out, lse, workspace, stream);
}

fa_status fa_decode_noalloc(const fa_problem* p, const void* q, const void* k, const void* v, void* out,
                            float* lse, void* stream) {
  fa_status s = validate_decode(p, q, k, v, out, lse);
  if (s != FA_OK) return s;
  int n_split, chunk;
  if (decode_ws(p, &n_split, &chunk) > (size_t)FA_DECODE_SCRATCH_BYTES) return FA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != FA_OK) return s;
  return decode_launch(p, q, k, v, out, lse, ws, stream);
}

fa_status fa_score_mod_create(const char* source, fa_score_mod* mod, char* log, size_t log_bytes) {
  return fa::custom_create(source, mod, log, log_bytes);
}

fa_status fa_score_mod_destroy(fa_score_mod mod) { return fa::custom_destroy(mod); }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported problem (dtype, head_dim or size)";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_SCRATCH_LIMIT: return "problem needs more than the fixed scratch of the allocation-free entry point";
    case FA_ERR_COMPILE: return "the caller-defined score_mod failed to compile";
  }
  return "unknown status";
}

int fa_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
