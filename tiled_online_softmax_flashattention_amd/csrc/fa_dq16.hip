// dQ pass of the 16-bit backward (f16, bf16; head_dim 64 or 128), in a
// translation unit of its own so that it can be compiled with its own
// instruction-scheduling options.
//
// Gradient of sum(dO * O) with respect to Q by calculus on the attention
// definition (the pages trace their kernel for it: attnax
// pallas_flash_attention docstring; flaxattention benchmark table):
//   dQ = scale * dS K,  dS = P * (dP - delta),  dP = dO V^T,
// with P = exp(S - lse) recomputed from the forward's saved log-sum-exp and
// delta_i = <dO_i, O_i>.  Query-stationary, like the forward: each wave keeps
// 32 queries' Q and dO rows in registers; K and V tiles go straight into
// LDS; S^T and dP^T are formed with keys as rows so the lane holds one query,
// and dQ^T = K^T dS^T accumulates in registers (K^T fragments through the
// transposing LDS read).  The pass also writes each row's delta and lse2 for
// the key/value pass, which runs after it.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// Query-stationary dQ pass, structured like the forward kernel: the score_mod
// bias (and the key mask row) start the S^T accumulator, masking runs only on
// diagonal and tail halves, K/V tiles go straight into double-buffered LDS
// (K permuted for both of its reads: row fragments for S^T, transposed for
// dQ), and per score one FMA and one exp give P = 2^(S' c + b - lse2).  With
// BLK only the key tiles whose block (this workgroup's 128 queries, tile / 2)
// is set in the block mask are visited.  With HALVES the block has 64
// queries and two waves share each 32 of them: wave w takes queries
// 32 (w & 1) .. +31 and key half w >> 1 of every tile, and the pair's dQ
// sums are added through LDS at the end (a.n_qblocks counts 64-query
// blocks then).
template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool BLK, bool HALVES = false>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void dq16_kernel(const AttnArgs a) {
  constexpr int BM = HALVES ? 64 : 128;   // queries per workgroup
  constexpr int BN = 64;    // keys per tile
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int TILE = BN * D;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];
  __shared__ __attribute__((aligned(16))) float sB0[MASK ? 2 * BN + 4 : 4];   // q parity 0 / 1
  __shared__ __attribute__((aligned(16))) float sB1[MASK ? 2 * BN + 4 : 4];
  __shared__ uint16_t sList[BLK ? kBlkMaxSeq / BN : 1];   // visited key tiles (block-sparse)
  __shared__ int sCnt[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const BlockCoord bc = block_coord(blockIdx.x, BH, a.n_qblocks, CAUSAL);
  const int bh = bc.bh;
  const int qb = CAUSAL ? a.n_qblocks - 1 - bc.blk : bc.blk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM;
  const int qw = q0 + 32 * (HALVES ? wave & 1 : wave);
  const int qi = qw + l32;
  const int qwp = qw + a.q_off, qpos = qi + a.q_off;   // positions among the keys
  const float c = a.scale_log2;
  const float inv_scale = 1.0f / a.scale;

  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * Sq * D;
  const uint16_t* dOg = (const uint16_t*)a.dout + (size_t)bh * Sq * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * Skv * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * Skv * D;

  // This lane's query: Q and dO rows as B operands, and the row's delta =
  // <dO, O> and lse * log2(e), which this pass also writes to the workspace
  // for the key/value pass that runs after it (lse2 with the query's ALiBi
  // share folded in, as bwd_pre_kernel does).
  const uint16_t* Og = (const uint16_t*)a.o + (size_t)bh * Sq * D;
  u32x4 qf[KS], of[KS];
  float lse2, delta;
  {
    const bool ok = qi < Sq;
    const size_t off = (size_t)min(qi, Sq - 1) * D + 8 * hi;
    float dsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const u32x4 x = *(const u32x4*)(Qg + off + 16 * kk);
      const u32x4 y = *(const u32x4*)(dOg + off + 16 * kk);
      const u32x4 z = *(const u32x4*)(Og + off + 16 * kk);
      qf[kk] = ok ? x : u32x4{0u, 0u, 0u, 0u};
      of[kk] = ok ? y : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        dsum += to_f32<T>((uint16_t)(y[cc] & 0xffffu)) * to_f32<T>((uint16_t)(z[cc] & 0xffffu));
        dsum += to_f32<T>((uint16_t)(y[cc] >> 16)) * to_f32<T>((uint16_t)(z[cc] >> 16));
      }
    }
    dsum += xor32(dsum);   // the partner lane holds the other half of the dims
    const float lse = a.lse[(size_t)bh * Sq + min(qi, Sq - 1)];
    lse2 = (ok && lse != kNegInf) ? lse * kLog2e : __builtin_inff();   // empty rows and rows past seq_q: P = 0
    delta = ok ? dsum : 0.f;
    if (ok && hi == 0 && (!HALVES || wave < 2)) {
      // for the key/value pass, as it consumes them (see bwd_pre_kernel):
      // -delta, and -lse2 / c with the query's ALiBi share folded in
      float l2 = lse2;
      if constexpr (MOD == MOD_ALIBI)
        l2 += alibi_slope(a.alibi_slopes, h, a.H) * kLog2e * (float)(qi & (kDkdvBQ - 1));
      a.delta[(size_t)bh * Sq + qi] = -delta;
      a.lse2[(size_t)bh * Sq + qi] = -l2 / a.scale_log2;
    }
  }

  if constexpr (D == 128) {   // one wave per SIMD: Q and dO fragments in AGPRs
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      keep_in_agprs(qf[kk]);
      keep_in_agprs(of[kk]);
    }
  }

  float slope2 = 0.f;
  f32x16 cinit = zero16();
  if constexpr (MOD == MOD_ALIBI) {
    const float slope = alibi_slope(a.alibi_slopes, h, a.H);
    slope2 = slope * kLog2e;
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = slope * inv_scale * (float)acc_row(r, hi);
  }
  if constexpr (MOD == MOD_CHECKERBOARD && !MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = (((qpos + r) & 1) == 0 ? a.even_nat : a.odd_nat) * inv_scale;
  }

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = zero16();
  // initial value of the dP^T accumulator: -delta in every register, so the
  // MFMAs produce dP - delta directly
  f32x16 dneg;
#pragma unroll
  for (int r = 0; r < 16; ++r) dneg[r] = -delta;

  const int kv_end = CAUSAL ? min(Skv, q0 + a.q_off + BM) : Skv;
  int ntiles = (kv_end + BN - 1) / BN;
  if constexpr (BLK) {
    const uint8_t* brow = a.block_mask + ((size_t)bh * a.bm_rows + (q0 >> 7)) * a.bm_cols;   // one block row
    ntiles = compact_tiles(brow, 1, 1, 0, ntiles, sList, sCnt);   // 64-key tile t lies in block t / 2
  }
  auto kv_of = [&](int n) __attribute__((always_inline)) {
    if constexpr (BLK) return list_at(sList, n) * BN;
    else return n * BN;
  };

  // Key-mask row: one byte per key, converted to an additive row in LDS.
  uint32_t mreg = 0;
  int mkv = 0;
  auto load_m = [&](int kv0) __attribute__((always_inline)) {
    if constexpr (MASK) {
      mkv = kv0 + (tid & (BN - 1));
      mreg = a.key_mask[(size_t)b * Skv + min(mkv, Skv - 1)];
    }
  };
  auto store_m = [&](float* sB) __attribute__((always_inline)) {
    if constexpr (MASK) {
      if (tid < BN) {
        const bool keep = mkv < Skv && mreg != 0;
        float e0 = 0.f, e1 = 0.f;
        if constexpr (MOD == MOD_CHECKERBOARD) {
          const bool kev = (mkv & 1) == 0;
          e0 = (kev ? a.even_nat : a.odd_nat) * inv_scale;
          e1 = (kev ? a.odd_nat : a.even_nat) * inv_scale;
        }
        sB[tid] = keep ? e0 : kNegInf;
        sB[parity_row_off<BN>() + tid] = keep ? e1 : kNegInf;
      }
    }
  };

  // Keys 32t .. 32t+31 of tile n, in two steps: the score products, then the
  // probabilities, dS and the dQ products.
  auto half_runs = [&](int n, int t) __attribute__((always_inline)) {
    return !CAUSAL || kv_of(n) + 32 * t <= qwp + 31;
  };
  // S'^T = K Q^T + C and dP'^T = V dO^T - delta, keys as rows
  auto scores = [&](int t, const uint16_t* sK, const uint16_t* sV, const float* sB, f32x16& s, f32x16& dp)
                    __attribute__((always_inline)) {
    s = cinit;
    dp = dneg;
    if constexpr (MASK) {   // the row starts the accumulator (cinit is nonzero only for ALiBi)
      const float* row = sB + ((qpos & 1) ? parity_row_off<BN>() : 0) + 32 * t + 4 * hi;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 m4 = *(const f32x4*)(row + 8 * u);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) s[4 * u + cc] = MOD == MOD_ALIBI ? cinit[4 * u + cc] + m4[cc] : m4[cc];
      }
    }
    // every K and V fragment is requested before the first MFMA
    const int kr = 32 * t + l32;
    u32x4 kfr[KS], vfr[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int off = tile_off<D, SW_BOTH>(kr, 16 * kk + 8 * hi);
      kfr[kk] = lds_read16(sK + off);
      vfr[kk] = lds_read16(sV + off);
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      s = mma16<T>(kfr[kk], qf[kk], s);
      dp = mma16<T>(vfr[kk], of[kk], dp);
    }
    // DS reads, then the MFMAs.  At head_dim 128 (one wave per SIMD) the
    // group also takes the four mask-row reads, so every read is in flight
    // before the first MFMA; at 64 the second wave covers the later ones.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * KS + (MASK && D == 128 ? 4 : 0), 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * KS, 0);
  };
  auto finish = [&](int n, int t, f32x16& s, f32x16& dp, const uint16_t* sK) __attribute__((always_inline)) {
    const int k0 = kv_of(n) + 32 * t;   // first key of the half
    // scores past the diagonal or past seq_kv: -inf (only on such halves)
    {
      int lim = 1 << 30;
      if (CAUSAL && k0 + 31 > qwp) lim = qpos - k0;
      if (!MASK && k0 + 32 > Skv) lim = min(lim, Skv - 1 - k0);
      if (__builtin_amdgcn_ballot_w64(lim < 31) != 0) {
        const int lim_l = lim - 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pos = 8 * (r >> 2) + (r & 3);
          if (pos > lim_l) s[r] = kNegInf;
        }
      }
    }

    float nb = -lse2;
    if constexpr (MOD == MOD_ALIBI) nb = slope2 * (float)(k0 - qpos) - lse2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_hw(fmaf(s[r], c, nb));
      dp[r] *= p;
    }

    // dQ^T += K^T dS^T over the half's 32 keys (K^T fragments requested first)
    u32x4 kt[2][DT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) kt[u][dt] = read_a_tr_tile<D, SW_BOTH>(sK, 32 * t + 16 * u, 32 * dt, lane);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 db = pack8<T>(dp, u);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dq[dt] = mma16<T>(kt[u][dt], db, dq[dt]);
    }
  };
  auto half = [&](int n, int t, const uint16_t* sK, const uint16_t* sV, const float* sB) __attribute__((always_inline)) {
    if (!half_runs(n, t)) return;
    f32x16 s, dp;
    scores(t, sK, sV, sB, s, dp);
    finish(n, t, s, dp, sK);
  };
  // head_dim 128 runs one wave per SIMD: both halves' score products first,
  // so the second half's products run while the first half's probabilities
  // are computed (as in the key/value pass).
  constexpr bool PAIRED = D == 128 && !HALVES;

  // Both halves of a causal tile at head_dim 128, scheduled by hand (the
  // non-causal instances measured 2 % faster with the compiler's schedule
  // of the plain sequence below, which has no per-half branch for them).
  // Scheduling barriers fix the order; each MFMA's operands are requested AHEAD steps
  // before it (a wait for LDS reads drains all of them while the tile loads
  // are in flight, so the reads of later steps are issued after the MFMAs
  // whose operands have arrived), and the VALU work of the other half sits
  // between the MFMAs: the second half's score products beside the first
  // half's probabilities, the first half's dQ products beside the second
  // half's.  Every half runs (a half wholly after the wave's queries is
  // masked to P = 0): a per-wave exit costs registers this schedule lacks.
  auto paired = [&](int n, const uint16_t* sK, const uint16_t* sV, const float* sB) __attribute__((always_inline)) {
    constexpr int AHEAD = 4;
    f32x16 s0, dp0, s1, dp1;
    auto start = [&](int t, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
      s = cinit;
      dp = dneg;
      if constexpr (MASK) {
        const float* row = sB + ((qpos & 1) ? parity_row_off<BN>() : 0) + 32 * t + 4 * hi;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 m4 = *(const f32x4*)(row + 8 * u);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) s[4 * u + cc] = MOD == MOD_ALIBI ? cinit[4 * u + cc] + m4[cc] : m4[cc];
        }
      }
    };
    auto frag = [&](const uint16_t* tile, int t, int kk) __attribute__((always_inline)) {
      return lds_read16(tile + tile_off<D, SW_BOTH>(32 * t + l32, 16 * kk + 8 * hi));
    };
    auto mask_half = [&](int t, f32x16& s) __attribute__((always_inline)) {
      const int k0 = kv_of(n) + 32 * t;
      int lim = 1 << 30;
      if (CAUSAL && k0 + 31 > qwp) lim = qpos - k0;
      if (!MASK && k0 + 32 > Skv) lim = min(lim, Skv - 1 - k0);
      if (__builtin_amdgcn_ballot_w64(lim < 31) != 0) {
        const int lim_l = lim - 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pos = 8 * (r >> 2) + (r & 3);
          if (pos > lim_l) s[r] = kNegInf;
        }
      }
    };
    auto nb_of = [&](int t) __attribute__((always_inline)) {
      if constexpr (MOD == MOD_ALIBI) return slope2 * (float)(kv_of(n) + 32 * t - qpos) - lse2;
      else return -lse2;
    };
    auto prob = [&](f32x16& s, f32x16& dp, float nb, int r) __attribute__((always_inline)) {
      dp[r] *= exp2_hw(fmaf(s[r], c, nb));
    };

    // first half's score products
    {
      start(0, s0, dp0);
      u32x4 kf[KS], vf[KS];
#pragma unroll
      for (int kk = 0; kk < AHEAD; ++kk) {
        kf[kk] = frag(sK, 0, kk);
        vf[kk] = frag(sV, 0, kk);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        s0 = mma16<T>(kf[kk], qf[kk], s0);
        dp0 = mma16<T>(vf[kk], of[kk], dp0);
        if (kk + AHEAD < KS) {
          kf[kk + AHEAD] = frag(sK, 0, kk + AHEAD);
          vf[kk + AHEAD] = frag(sV, 0, kk + AHEAD);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mask_half(0, s0);
    __builtin_amdgcn_sched_barrier(0);
    // second half's score products, first half's probabilities between them
    {
      const float nb0 = nb_of(0);
      start(1, s1, dp1);
      u32x4 kf[KS], vf[KS];
#pragma unroll
      for (int kk = 0; kk < AHEAD; ++kk) {
        kf[kk] = frag(sK, 1, kk);
        vf[kk] = frag(sV, 1, kk);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        s1 = mma16<T>(kf[kk], qf[kk], s1);
        dp1 = mma16<T>(vf[kk], of[kk], dp1);
        if (kk + AHEAD < KS) {
          kf[kk + AHEAD] = frag(sK, 1, kk + AHEAD);
          vf[kk + AHEAD] = frag(sV, 1, kk + AHEAD);
        }
        prob(s0, dp0, nb0, 2 * kk);
        prob(s0, dp0, nb0, 2 * kk + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mask_half(1, s1);
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T += K^T dS^T: product i of a half uses key step u = i / DT and
    // dims 32 (i % DT)
    constexpr int NP = 2 * DT;
    auto ktf = [&](int t, int i) __attribute__((always_inline)) {
      return read_a_tr_tile<D, SW_BOTH>(sK, 32 * t + 16 * (i / DT), 32 * (i % DT), lane);
    };
    // first half's products, second half's probabilities between them
    {
      const float nb1 = nb_of(1);
      const u32x4 db[2] = {pack8<T>(dp0, 0), pack8<T>(dp0, 1)};
      u32x4 kt[NP];
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) kt[i] = ktf(0, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        dq[i % DT] = mma16<T>(kt[i], db[i / DT], dq[i % DT]);
        if (i + AHEAD < NP) kt[i + AHEAD] = ktf(0, i + AHEAD);
        prob(s1, dp1, nb1, 2 * i);
        prob(s1, dp1, nb1, 2 * i + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // second half's products
    {
      const u32x4 db[2] = {pack8<T>(dp1, 0), pack8<T>(dp1, 1)};
      u32x4 kt[NP];
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) kt[i] = ktf(1, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        dq[i % DT] = mma16<T>(kt[i], db[i / DT], dq[i % DT]);
        if (i + AHEAD < NP) kt[i + AHEAD] = ktf(1, i + AHEAD);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto tile = [&](int n, const uint16_t* sK, const uint16_t* sV, const float* sB, uint16_t* sKn, uint16_t* sVn,
                  float* sBn) __attribute__((always_inline)) {
    wait_direct_loads();   // this wave's loads of tile n are in LDS
    sync_wg();       // ... and every other wave's; tile n-1 is retired
    if (n + 1 < ntiles) {
      load_tile_lds<D, BN, SW_BOTH>(Kg, kv_of(n + 1), Skv, sKn, wave, lane);
      load_tile_lds<D, BN, SW_BOTH>(Vg, kv_of(n + 1), Skv, sVn, wave, lane);
      store_m(sBn);
      load_m(kv_of(min(n + 2, ntiles - 1)));
    }
    if constexpr (HALVES) {
      half(n, wave >> 1, sK, sV, sB);
    } else if constexpr (PAIRED && CAUSAL) {
      paired(n, sK, sV, sB);
    } else if constexpr (PAIRED) {   // both halves always run without the causal rule
      f32x16 s0, dp0, s1, dp1;
      scores(0, sK, sV, sB, s0, dp0);
      scores(1, sK, sV, sB, s1, dp1);
      finish(n, 0, s0, dp0, sK);
      finish(n, 1, s1, dp1, sK);
    } else {
      half(n, 0, sK, sV, sB);
      __builtin_amdgcn_sched_barrier(0);   // the halves share registers
      half(n, 1, sK, sV, sB);
    }
  };

  if (!BLK || ntiles > 0) {   // without a block mask there is always a tile
    load_tile_lds<D, BN, SW_BOTH>(Kg, kv_of(0), Skv, sK0, wave, lane);
    load_tile_lds<D, BN, SW_BOTH>(Vg, kv_of(0), Skv, sV0, wave, lane);
    load_m(kv_of(0));
    store_m(sB0);
    load_m(kv_of(min(1, ntiles - 1)));
  }
  int n = 0;
  for (; n + 1 < ntiles; n += 2) {
    tile(n, sK0, sV0, sB0, sK1, sV1, sB1);
    tile(n + 1, sK1, sV1, sB1, sK0, sV0, sB0);
  }
  if (n < ntiles) tile(n, sK0, sV0, sB0, sK1, sV1, sB1);

  if constexpr (HALVES) {
    // the wave of key half 1 hands its dQ sums to the wave of half 0 through
    // the tile buffers (free once every wave is past its last tile)
    static_assert(TILE * sizeof(uint16_t) >= 16 * DT * 64 * sizeof(float), "merge buffer");
    sync_wg();
    float* xq = (float*)((wave & 1) ? sK1 : sK0);
    if (wave >> 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xq[(16 * dt + r) * 64 + lane] = dq[dt][r];
    }
    sync_wg();
    if (wave >> 1) return;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[dt][r] += xq[(16 * dt + r) * 64 + lane];
  }

  if (qi < Sq) {
    uint16_t* dQg = (uint16_t*)a.dq + ((size_t)bh * Sq + qi) * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        *(u32x2*)(dQg + 32 * dt + 8 * u + 4 * hi) =
            u32x2{pack2<T>(dq[dt][4 * u] * sc, dq[dt][4 * u + 1] * sc), pack2<T>(dq[dt][4 * u + 2] * sc, dq[dt][4 * u + 3] * sc)};
      }
    }
  }
}

// ----------------------------------------------------------------- launchers

template <class T, int D, int MOD, bool CAUSAL, bool MASK>
static hipError_t launch_dq16_inst(const AttnArgs& a, hipStream_t st) {
  if (a.dq_halves) {
    AttnArgs h = a;
    h.n_qblocks = (a.Sq + 63) / 64;
    const dim3 grid((unsigned)h.n_qblocks * (unsigned)(a.B * a.H));
    if (a.block_mask)
      hipLaunchKernelGGL((dq16_kernel<T, D, MOD, CAUSAL, MASK, true, true>), grid, dim3(256), 0, st, h);
    else
      hipLaunchKernelGGL((dq16_kernel<T, D, MOD, CAUSAL, MASK, false, true>), grid, dim3(256), 0, st, h);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)a.n_qblocks * (unsigned)(a.B * a.H);
  if (a.block_mask)
    hipLaunchKernelGGL((dq16_kernel<T, D, MOD, CAUSAL, MASK, true>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dq16_kernel<T, D, MOD, CAUSAL, MASK, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class T, int D, int MOD>
static hipError_t launch_dq16_mod(const AttnArgs& a, bool causal, bool mask, hipStream_t st) {
  if (causal)
    return mask ? launch_dq16_inst<T, D, MOD, true, true>(a, st) : launch_dq16_inst<T, D, MOD, true, false>(a, st);
  return mask ? launch_dq16_inst<T, D, MOD, false, true>(a, st) : launch_dq16_inst<T, D, MOD, false, false>(a, st);
}

template <class T, int D>
static hipError_t launch_dq16_d(const AttnArgs& a, int mod, bool causal, bool mask, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return launch_dq16_mod<T, D, MOD_ALIBI>(a, causal, mask, st);
    case MOD_CHECKERBOARD: return launch_dq16_mod<T, D, MOD_CHECKERBOARD>(a, causal, mask, st);
    default: return launch_dq16_mod<T, D, MOD_NONE>(a, causal, mask, st);
  }
}

hipError_t launch_dq16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask, hipStream_t st) {
  if (bf16)
    return D == 64 ? launch_dq16_d<BF16, 64>(a, mod, causal, mask, st) : launch_dq16_d<BF16, 128>(a, mod, causal, mask, st);
  return D == 64 ? launch_dq16_d<F16, 64>(a, mod, causal, mask, st) : launch_dq16_d<F16, 128>(a, mod, causal, mask, st);
}

}  // namespace fa
