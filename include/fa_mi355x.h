/*
 * fa_mi355x.h - C ABI of the tiled online-softmax attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes exact attention
 *
 *     O = softmax(scale * Q K^T + score_mod + mask) V
 *
 * tile by tile with an online softmax (running row max m, running row sum l,
 * accumulator rescaled by exp(m_old - m_new)), so the seq_q x seq_kv score
 * matrix is never written to memory.  This is the computation of the attnax
 * ``pallas_flash_attention`` page (kernel body: per query block, a loop over
 * key/value blocks that forms scores, applies score_mod with global indices,
 * applies the mask, then updates max, sum and accumulator and divides at the
 * end), with the input layout of the flash-attention-jax page ("Use
 * flash_attention": q, k, v as (batch, heads, seq, dim), key mask as
 * (batch, seq)), its causal variant ("Use causal_flash_attention"), and the
 * score_mods named on the flaxattention page (ALiBi in the example,
 * checkerboard in the autograd example and benchmark).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, contiguous, row-major:
 *     q, out, dout, dq          (batch, heads, seq_q,  head_dim)
 *     k, v, dk, dv              (batch, heads, seq_kv, head_dim)
 *     lse                       (batch, heads, seq_q)  float32, natural log
 *     key_mask                  (batch, seq_kv) uint8, nonzero = keep the key
 *     block_mask                (batch, heads, ceil(seq_q/128), ceil(seq_kv/128)) uint8
 *   q, k, v, out, dout, dq, dk, dv all have the element type ``dtype``.
 * - Every pointer named as a tensor is a DEVICE pointer on the current HIP
 *   device, 16-byte aligned.  The ``fa_problem`` struct itself is a host
 *   pointer read only during the call.
 * - The caller owns all memory.  The library allocates nothing, keeps no
 *   state between calls and only enqueues work on ``stream`` (a hipStream_t;
 *   NULL means the legacy default stream).  Results are ready when the stream
 *   reaches them; device faults surface at the caller's synchronisation.
 * - Outputs must not alias inputs.  Calls on different streams may run
 *   concurrently when their outputs and workspaces are disjoint.
 * - Arguments are validated on the host before anything is enqueued; a
 *   non-zero fa_status means nothing was launched (except FA_ERR_HIP, which
 *   reports a failed launch).  There is no fallback path.
 *
 * Semantics
 * ---------
 * s_ij = scale * <q_i, k_j> + bias_h(pos_i, j), where pos_i = i + q_offset is
 * the position of query row i in the key sequence (q_offset = 0 for
 * self-attention; the number of cached keys before the first query when
 * decoding or prefilling against a KV cache), j is the 0-based key position,
 * and the bias is NOT multiplied by scale.  Key j is allowed for query i when
 * key_mask[b][j] != 0 (or key_mask == NULL), if causal, j <= pos_i, and, with
 * a block mask, block_mask[b][h][i / 128][j / 128] != 0 (query ROW i, not its
 * position).
 * lse_i = log sum_{allowed j} exp(s_ij); out_i =
 * sum_{allowed j} exp(s_ij - lse_i) v_j.  A row with no allowed key gets
 * out_i = 0, lse_i = -inf and zero gradients.  Score, softmax and
 * accumulation arithmetic is float32; probabilities are rounded to ``dtype``
 * before the probability-times-V product for the 16-bit types.
 */
#ifndef FA_MI355X_H_
#define FA_MI355X_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 7

/* Edge of the blocks of a block mask (query rows and keys), and the longest
 * seq_q / seq_kv a call with a block mask takes. */
#define FA_BLOCK_MASK_BLOCK 128
#define FA_BLOCK_MASK_MAX_SEQ 131072

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, bad enum, bad shape */
  FA_ERR_UNSUPPORTED = 2,        /* valid request outside what the kernels implement */
  FA_ERR_WORKSPACE_TOO_SMALL = 3,
  FA_ERR_HIP = 4,                /* a HIP runtime call or kernel launch failed */
  FA_ERR_SCRATCH_LIMIT = 5,      /* fa_decode_noalloc: the problem needs more than FA_DECODE_SCRATCH_BYTES */
  FA_ERR_COMPILE = 6             /* a caller-defined score_mod failed to compile */
} fa_status;

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* score_mod kinds (flaxattention page: example and benchmark; attnax
 * pallas_flash_attention page: score_mod, a callable on the scaled scores with
 * global indices).
 *  FA_MOD_ALIBI:        bias = -slope_h * (pos_i - j).  slope_h comes from
 *                       alibi_slopes[h] (device float[heads]) or, when that is
 *                       NULL, slope_h = 2^(-8 (h + 1) / heads).
 *  FA_MOD_CHECKERBOARD: bias = checker_even when (pos_i + j) is even, otherwise
 *                       checker_odd (the workloads use +0.5 / -0.5).
 *  FA_MOD_CUSTOM:       s_ij = mod(scale * <q_i, k_j>, b, h, pos_i, j) with the
 *                       caller's device function (fa_score_mod_create); every
 *                       dtype and head_dim, every entry point (fa_decode and
 *                       the key split stop at head_dim 128 as for the
 *                       built-in mods). */
typedef enum { FA_MOD_NONE = 0, FA_MOD_ALIBI = 1, FA_MOD_CHECKERBOARD = 2, FA_MOD_CUSTOM = 3 } fa_mod_kind;

/* A caller-defined score_mod compiled for the device (fa_score_mod_create). */
typedef struct fa_score_mod_s* fa_score_mod;

/* dQ formation of the backward (fa_problem.dq_mode). */
typedef enum { FA_DQ_AUTO = 0, FA_DQ_SEPARATE = 1, FA_DQ_ATOMIC = 2 } fa_dq_mode;

/* Most key chunks fa_decode and fa_forward_split split into (fa_problem.kv_splits). */
#define FA_MAX_KV_SPLITS 256

typedef struct {
  int64_t batch, heads, seq_q, seq_kv, head_dim;
  int32_t dtype;             /* fa_dtype */
  int32_t causal;            /* 0 or 1: key j allowed only when j <= i + q_offset */
  float scale;               /* multiplies q.k, > 0 (else FA_ERR_UNSUPPORTED); 1/sqrt(head_dim) usually */
  int32_t mod_kind;          /* fa_mod_kind */
  const float* alibi_slopes; /* device float[heads] or NULL (FA_MOD_ALIBI only) */
  float checker_even;        /* FA_MOD_CHECKERBOARD only */
  float checker_odd;
  const uint8_t* key_mask;   /* device uint8 (batch, seq_kv), nonzero = keep; NULL = keep all */
  int64_t q_offset;          /* >= 0: position of query row 0 among the keys (0 = self-attention) */
  /* Block sparsity (flaxattention page, "Example usage": create_block_mask
   * over 128 x 128 blocks).  Device uint8 (batch, heads, ceil(seq_q / 128),
   * ceil(seq_kv / 128)); byte (b, h, r, c) == 0 removes every pair of query
   * rows 128r .. 128r+127 and keys 128c .. 128c+127, nonzero leaves the
   * block's pairs to the other rules.  The kernels never load or compute a
   * removed block.  NULL = no block mask.  Requires seq_q and seq_kv
   * <= FA_BLOCK_MASK_MAX_SEQ (else FA_ERR_UNSUPPORTED). */
  const uint8_t* block_mask;
  /* How fa_backward forms dQ when dq, dk and dv are all requested (fa_dq_mode).
   * FA_DQ_AUTO: the library's measured choice for the dtype and head_dim.
   * FA_DQ_SEPARATE: a query-stationary pass that recomputes the scores and
   *   dP; no atomics, bitwise-repeatable.
   * FA_DQ_ATOMIC: the key/value pass also adds scale * dS K into an fp32
   *   workspace with atomics, then a conversion kernel writes dq; saves the
   *   recomputation, but the order of the additions (and so the last bits of
   *   dq) varies between calls.  f16 and bf16 only, and seq_q * head_dim
   *   below 2^28 (else FA_ERR_UNSUPPORTED).
   * A call that skips the query or the key/value pass ignores the mode. */
  int32_t dq_mode;
  /* fa_decode and fa_forward_split: 0 = the library's split of the key axis;
   * n > 0 = about n key chunks (1 <= n <= FA_MAX_KV_SPLITS; query blocks of
   * more than one row round chunks up to whole 64-key tiles).  The results do
   * not depend on it beyond rounding.  Other calls ignore it. */
  int32_t kv_splits;
  /* FA_MOD_CUSTOM: the compiled score_mod and its parameter array (device
   * floats handed to the caller's functions as `params`, or NULL). */
  fa_score_mod custom_mod;
  const float* mod_params;
} fa_problem;

/* Supported: dtype f16 or bf16 with head_dim 64 or 128; dtype f32 with
 * head_dim 64, 128 or 512.  Any seq_q, seq_kv >= 1 (ragged tails are masked
 * inside the kernels).  Sizes must keep every tensor under 2^31 elements per
 * (batch, head) slice, batch * heads under 2^31 and q_offset + seq_q under
 * 2^31.  A query whose position is past the last key (causal or not) sees
 * every key. */

/* Forward (attnax kernel body: online-softmax loop, final acc / l).
 * Writes out (dtype) and, when lse != NULL, lse (float32, natural log).  The
 * backward needs lse. */
fa_status fa_forward(const fa_problem* p, const void* q, const void* k, const void* v,
                     void* out, float* lse, void* stream);

/* Bytes of device workspace fa_forward_split needs for problem p (written to
 * *bytes); 0 when the call runs unsplit. */
fa_status fa_forward_split_workspace_size(const fa_problem* p, size_t* bytes);

/* Forward with the key axis split into chunks, for shapes whose query blocks
 * alone do not fill the device (few (batch, head) slices of long sequences;
 * with causal the last query blocks are the longest and would finish alone).
 * Every (query block, key chunk) pair is a workgroup that runs the forward's
 * online-softmax loop over its chunk and stores the unnormalised partial
 * (running max, sum, accumulator) of each row in the workspace; a second
 * kernel merges a row's partials exactly, rescaling each to the common max
 * as the loop itself does from tile to tile (attnax pallas_flash_attention
 * page, kernel body).  The flaxattention page's TODO list asks for default
 * configurations per input shape: with p->kv_splits == 0 the library's
 * per-shape table picks the chunk count, and where it keeps the forward
 * whole (enough query blocks, or too few keys per chunk to pay for the merge)
 * the call is exactly fa_forward.  Same outputs as fa_forward up to rounding.
 * The workspace (>= fa_forward_split_workspace_size bytes, 256-byte aligned)
 * is scratch; it may be NULL when that size is 0.  head_dim 512 is never
 * split (kv_splits > 1 gives FA_ERR_UNSUPPORTED); with FA_MOD_CUSTOM the
 * table keeps the forward whole and an explicit kv_splits > 1 splits it. */
fa_status fa_forward_split(const fa_problem* p, const void* q, const void* k, const void* v,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of device workspace fa_backward needs for problem p (written to *bytes). */
fa_status fa_backward_workspace_size(const fa_problem* p, size_t* bytes);

/* Backward: gradients of sum(dout * out) with respect to q, k and v, with the
 * probabilities recomputed from the saved lse (no score matrix is stored).
 * out and lse must be the values fa_forward produced for the same inputs.
 * Two passes: a key/value pass writing dk and dv, and a query pass writing
 * dq.  dq == NULL skips the query pass; dk == dv == NULL skips the key/value
 * pass (the flaxattention autograd example asks for the query gradient only);
 * at least one pass must be requested, and dk, dv are NULL together or not
 * at all.
 * The workspace (>= fa_backward_workspace_size bytes, 256-byte aligned) is
 * scratch: its contents on entry are ignored and on exit undefined.  Its size
 * depends on p->dq_mode (the atomic mode adds seq_q * head_dim floats per
 * (batch, head)).  With dq_mode FA_DQ_SEPARATE every kernel is deterministic:
 * repeated calls give bitwise-equal results; FA_DQ_ATOMIC (or FA_DQ_AUTO
 * where it picks the atomic mode) gives bitwise-equal dk, dv and a dq that
 * varies in its last bits. */
fa_status fa_backward(const fa_problem* p, const void* q, const void* k, const void* v,
                      const void* out, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Bytes of device workspace fa_decode needs for problem p (1 <= seq_q <= 64). */
fa_status fa_decode_workspace_size(const fa_problem* p, size_t* bytes);

/* Decode: a short block of queries (1 <= seq_q <= 64, query row i at key
 * position q_offset + i; with causal only keys up to that position count)
 * against seq_kv keys, split over the key axis into chunks whose partial
 * (max, sum, accumulator) are merged exactly.  The flaxattention page
 * (decoding benchmark and TODO list) singles this case out.  seq_q == 1 runs a
 * streaming kernel (one group of lanes per key); seq_q > 1, and any seq_q
 * with FA_MOD_CUSTOM, runs the forward kernel of the dtype (or of the
 * caller's mod) on each key chunk, whose chunks are then whole 64-key tiles.
 * f16, bf16 and f32 with head_dim 64 or 128.  Same outputs as fa_forward. */
fa_status fa_decode(const fa_problem* p, const void* q, const void* k, const void* v,
                    void* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Caller-defined score_mod (attnax pallas_flash_attention page: score_mod is
 * a callable traced into the inner loop, applied to the scaled scores with
 * global indices; its gradient there comes from tracing).  `source` is HIP
 * device code defining
 *
 *   __device__ float fa_score_mod(float score, int b, int h, int q_idx, int kv_idx,
 *                                 const float* params);
 *   __device__ float fa_score_mod_grad(float score, int b, int h, int q_idx, int kv_idx,
 *                                      const float* params);
 *
 * score = scale * <q_i, k_j> (natural units), b and h the batch and head,
 * q_idx = i + q_offset and kv_idx = j the global positions, params the
 * problem's mod_params; fa_score_mod returns the modified score (before any
 * mask: masked pairs are dropped whatever it returns) and fa_score_mod_grad
 * its derivative with respect to score, which the backward multiplies into dS.
 * The library compiles the source with hipRTC into its generic attention
 * kernels: once here for the target, to report errors (FA_ERR_COMPILE, with
 * the compiler's log in `log` (log_bytes, NUL-terminated) when log != NULL),
 * and again for each (device, dtype, head_dim, causal, key mask, block mask)
 * configuration on its first use (seconds; cached in the handle).  The handle
 * is freed with fa_score_mod_destroy once no call using it is in flight;
 * concurrent calls may share it. */
fa_status fa_score_mod_create(const char* source, fa_score_mod* mod, char* log, size_t log_bytes);
fa_status fa_score_mod_destroy(fa_score_mod mod);

/* Bytes of the fixed device scratch behind fa_decode_noalloc (per device). */
#define FA_DECODE_SCRATCH_BYTES (16u << 20)

/* fa_decode without a workspace argument, for callers that cannot allocate
 * device memory at call time (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same problems, arguments and
 * results as fa_decode; the per-chunk partials go to a fixed scratch array
 * of FA_DECODE_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends.  A problem whose fa_decode_workspace_size
 * exceeds that returns FA_ERR_SCRATCH_LIMIT (nothing launched).  The call
 * allocates nothing.  Every call on one device shares that device's scratch
 * (the last call's partials stay in it): calls that overlap on one device,
 * e.g. on two streams, race and give undefined results; calls on one stream
 * are ordered and safe.  Nothing in the scratch needs to start at zero. */
fa_status fa_decode_noalloc(const fa_problem* p, const void* q, const void* k, const void* v,
                            void* out, float* lse, void* stream);

/* Static description of a status code (never NULL). */
const char* fa_status_string(fa_status s);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H_ */
