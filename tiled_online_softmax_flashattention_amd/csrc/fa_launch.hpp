// Host-side launchers of the attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "fa_common.hpp"

namespace fa {

// 16-bit forward (f16 / bf16, head_dim 64 or 128).  With split, each query
// block is split over a.n_split key chunks of a.chunk keys whose partials go
// to a.partial (rows (bh, query) x chunks x (D + 2) floats) for
// launch_decode_merge.  halves (not split): 64-query blocks with two waves
// per 32 queries, one key half each.
int fwd16_block_q(int D);
hipError_t launch_fwd16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask,
                        hipStream_t st, bool split = false, bool halves = false);

// fp32 forward (head_dim 64, 128 or 512).  With split (head_dim <= 128), each
// query block is split over a.n_split key chunks of a.chunk keys (a multiple
// of 32) whose partials go to a.partial, as launch_fwd16 does.
int fwd32_block_q(int D);
size_t fwd32_lds_bytes(int D, bool blk);   // dynamic LDS of a forward launch (with a block mask: blk)
hipError_t launch_fwd32(const AttnArgs& a, int D, int mod, bool causal, bool mask, hipStream_t st,
                        bool split = false);

// Backward: preprocess (delta = rowsum(dO * O), lse in base 2), then the
// key-stationary dK/dV pass and the query-stationary dQ pass.  kv16 = 0: the
// rows as the fp32 passes read them; 1: as the 16-bit key/value pass reads
// them (-delta, -lse2 / c); 2: the same with the ALiBi query share folded in.
hipError_t launch_bwd_pre(const AttnArgs& a, int dtype, int D, hipStream_t st, int kv16 = 0);
int bwd16_block_kv();
int bwd16_block_q();
// dq_atomic (with both passes wanted): dQ from fp32 atomics in the key/value
// pass (a.dq_acc, B*H*Sq*D floats) instead of the query pass.
hipError_t launch_bwd16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask,
                        bool want_kv, bool want_q, bool dq_atomic, hipStream_t st);
// The 16-bit dQ pass alone (separate mode; it also writes delta and lse2 for
// the key/value pass).
hipError_t launch_dq16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask, hipStream_t st);
int bwd32_block_kv(int D);
size_t bwd32_lds_bytes(int D, bool blk);   // dynamic LDS of either fp32 backward pass
int bwd32_block_q(int D);
hipError_t launch_bwd32(const AttnArgs& a, int D, int mod, bool causal, bool mask, bool want_kv, bool want_q,
                        hipStream_t st);

// Split-KV decode and the merge of the partial (max, sum, accumulator).
int decode_choose_split(int BH, int Skv, int* chunk, int cus);   // cus: the device's compute units
hipError_t launch_decode(const AttnArgs& a, int dtype, int D, int mod, bool mask, hipStream_t st);
// Merge of `rows` partial rows (a.n_split chunks each) into O and lse rows.
hipError_t launch_decode_merge(const AttnArgs& a, int dtype, int D, int rows, hipStream_t st);
// The same merge for the forward split over keys (many rows; several rows
// per workgroup).
hipError_t launch_split_merge(const AttnArgs& a, int dtype, int D, int rows, hipStream_t st);

}  // namespace fa
