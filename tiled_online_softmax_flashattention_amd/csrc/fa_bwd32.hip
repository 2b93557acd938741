// Backward attention for fp32 inputs, head_dim 64, 128 or 512.
//
// Same gradients as the 16-bit backward (P recomputed from the saved
// log-sum-exp; dV = P^T dO, dS = P (dP - delta), dK = scale dS^T Q,
// dQ = scale dS K) on the fp32 matrix cores.  With one operand value per lane
// no transposed LDS copy is needed.  Heads of 512 dims are split over the 4
// waves of a workgroup: each wave owns 128 dims of the register-resident rows
// and accumulators, and the partial S and dP products are summed through LDS.
#include "fa_common.hpp"
#ifndef __HIPCC_RTC__
#include "fa_launch.hpp"
#endif

// A caller-defined score_mod (the modified score of score = scale * q.k, and
// its derivative in score), used by the MOD_CUSTOM instances below.  Defined
// only in the units the library compiles at run time with the caller's
// source, which are the only units that instantiate MOD_CUSTOM.
__device__ float fa_score_mod(float score, int b, int h, int q_idx, int kv_idx, const float* params);
__device__ float fa_score_mod_grad(float score, int b, int h, int q_idx, int kv_idx, const float* params);

namespace fa {

template <int D>
struct B32Cfg {
  static constexpr int DS = D >= 512 ? 4 : 1;   // dim slices
  static constexpr int NG = 4 / DS;             // 32-row groups per workgroup
  static constexpr int P = D + 4;               // LDS pitch (floats)
  // two 32-row tiles + partial-sum exchange + two 32-float row vectors / mask
  static constexpr size_t lds = (size_t)2 * 32 * P * 4 + (DS > 1 ? 4 * 16 * 64 * 4 : 0) + 2 * 32 * 4 + 64;
  // block-sparse: the list of visited 32-row tiles and 4 counters after everything else
  static constexpr size_t lds_blk = lds + (size_t)kBlkMaxSeq / 32 * 2 + 16;
};

// Sum the DS partial accumulators of a row group through LDS (every wave calls
// it; 16-byte swizzled chunks).  TRAIL: end with a barrier (sS is reused at
// once); without it the caller guarantees a barrier before the next write to sS.
template <int DS, bool TRAIL = true>
__device__ __forceinline__ f32x16 slice_sum(f32x16 x, float* sS, int wave, int g, int lane) {
  slice_put(sS, x, wave, lane);
  sync_wg();
  const f32x16 s = slice_gather<DS>(sS, g, lane);
  if constexpr (TRAIL) sync_wg();
  return s;
}

// Stage a 32-row fp32 tile (rows row0.., natural layout, pitch D + 4).
template <int D>
__device__ __forceinline__ void stage32(float* dst, const float* g, int row0, int nrows, int tid) {
  constexpr int N = 32 * D / 4 / 256;
#pragma unroll 4
  for (int i = 0; i < N; ++i) {
    const int c = tid + 256 * i, row = c / (D / 4), ch = c % (D / 4);
    // rows past nrows: the last row (finite; the kernels mask it out)
    const f32x4 x = *(const f32x4*)(g + (size_t)min(row0 + row, nrows - 1) * D + 4 * ch);
    *(f32x4*)&dst[row * (D + 4) + 4 * ch] = x;
  }
}

// ------------------------------------------------------------- dK / dV pass

// With BLK only the query tiles whose 128 x 128 block is set in the block
// mask are visited (a workgroup's keys lie in one block column).
// MOD_CUSTOM: P from the caller's fa_score_mod of the scaled score and dS
// times its derivative fa_score_mod_grad (at head_dim 512 after the partial
// products are summed); compiled only at run time with the caller's source.
template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
__device__ __forceinline__ void dkdv32_body(const AttnArgs& a) {
  using C = B32Cfg<D>;
  constexpr int DS = C::DS, NG = C::NG, P = C::P;
  constexpr int DSL = D / DS, HS = DSL / 2, DT = DSL / 32;
  constexpr int BKV = 32 * NG, BQ = 32;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* sQ = smem;
  float* sO = sQ + 32 * P;
  float* sS = sO + 32 * P;
  float* sL = sS + (DS > 1 ? 4 * 16 * 64 : 0);
  float* sDl = sL + 32;
  uint16_t* sList = (uint16_t*)((char*)smem + C::lds);
  int* sCnt = (int*)(sList + kBlkMaxSeq / 32);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = wave / DS, e = wave % DS;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int kb = blockIdx.x / BH;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int k0 = kb * BKV;
  const int kw = k0 + 32 * g;
  const int kj = kw + l32;

  const float* Qg = (const float*)a.q + (size_t)bh * Sq * D;
  const float* dOg = (const float*)a.dout + (size_t)bh * Sq * D;
  const float* Kg = (const float*)a.k + (size_t)bh * Skv * D;
  const float* Vg = (const float*)a.v + (size_t)bh * Skv * D;

  float kf[HS], vf[HS];
  {
    const bool ok = kj < Skv;
    const size_t off = (size_t)(ok ? kj : 0) * D + e * DSL + hi * HS;
#pragma unroll
    for (int kk = 0; kk < HS; kk += 4) {
      const f32x4 x = *(const f32x4*)(Kg + off + kk);
      const f32x4 y = *(const f32x4*)(Vg + off + kk);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kf[kk + c] = ok ? x[c] : 0.f;
        vf[kk + c] = ok ? y[c] : 0.f;
      }
    }
  }
  bool key_ok = kj < Skv;
  if constexpr (MASK) key_ok = key_ok && a.key_mask[(size_t)b * Skv + (key_ok ? kj : 0)] != 0;

  float slope2 = 0.f, cbe = 0.f, cbo = 0.f;
  if constexpr (MOD == MOD_ALIBI) slope2 = alibi_slope(a.alibi_slopes, h, a.H) * kLog2e;
  if constexpr (MOD == MOD_CHECKERBOARD) {
    const bool keven = (kj & 1) == 0;
    cbe = keven ? a.even_log2 : a.odd_log2;
    cbo = keven ? a.odd_log2 : a.even_log2;
  }

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  const int off = a.q_off;   // query row q sits at key position q + off
  const int qt0 = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int nqt = (Sq + BQ - 1) / BQ;
  int nvis = nqt - qt0;
  if constexpr (BLK) {
    const uint8_t* bcol = a.block_mask + (size_t)bh * a.bm_rows * a.bm_cols + (k0 >> 7);
    nvis = compact_tiles(bcol, a.bm_cols, 2, qt0, nqt, sList, sCnt);   // 32-query tile t lies in block row t / 4
  }
  for (int n = 0; n < nvis; ++n) {
    const int q0 = (BLK ? list_at(sList, n) : qt0 + n) * BQ;
    sync_wg();
    if constexpr (D * 4 % 1024 == 0) {   // head_dim 512: direct loads, one wait
      stage32_direct<D>(sQ, Qg, q0, Sq, wave, lane);
      stage32_direct<D>(sO, dOg, q0, Sq, wave, lane);
      wait_direct_loads();
    } else {
      stage32<D>(sQ, Qg, q0, Sq, tid);
      stage32<D>(sO, dOg, q0, Sq, tid);
    }
    if (tid < 32) {
      const bool ok = q0 + tid < Sq;
      sL[tid] = ok ? a.lse2[(size_t)bh * Sq + q0 + tid] : __builtin_inff();
      sDl[tid] = ok ? a.delta[(size_t)bh * Sq + q0 + tid] : 0.f;
    }
    sync_wg();
    if (DS == 1 && CAUSAL && q0 + off + BQ - 1 < kw) continue;

    f32x16 s0 = zero16(), s1 = zero16(), p0 = zero16(), p1 = zero16();
    const float* qrow = sQ + l32 * P + e * DSL + hi * HS;
    const float* orow = sO + l32 * P + e * DSL + hi * HS;
#pragma unroll
    for (int kk = 0; kk < HS; kk += 4) {
      const f32x4 x = *(const f32x4*)(qrow + kk);
      const f32x4 y = *(const f32x4*)(orow + kk);
      s0 = mma_f32(x[0], kf[kk + 0], s0);
      s1 = mma_f32(x[1], kf[kk + 1], s1);
      p0 = mma_f32(y[0], vf[kk + 0], p0);
      p1 = mma_f32(y[1], vf[kk + 1], p1);
      s0 = mma_f32(x[2], kf[kk + 2], s0);
      s1 = mma_f32(x[3], kf[kk + 3], s1);
      p0 = mma_f32(y[2], vf[kk + 2], p0);
      p1 = mma_f32(y[3], vf[kk + 3], p1);
    }
    f32x16 s = s0 + s1, dp = p0 + p1;
    if constexpr (DS > 1) {   // the two barriers around the next tile's staging order the next exchange
      s = slice_sum<DS>(s, sS, wave, g, lane);
      dp = slice_sum<DS, false>(dp, sS, wave, g, lane);
    }

    const bool diag = CAUSAL && (q0 + off < kw + 31);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 l4 = *(const f32x4*)&sL[8 * u + 4 * hi];
      const f32x4 d4 = *(const f32x4*)&sDl[8 * u + 4 * hi];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * u + c;
        const int qi = q0 + acc_row(r, hi);
        float x = s[r] * a.scale_log2;
        if constexpr (MOD == MOD_ALIBI) x += slope2 * (float)(kj - qi - off);
        if constexpr (MOD == MOD_CHECKERBOARD) x += ((r + off) & 1) ? cbo : cbe;
        if constexpr (MOD == MOD_CUSTOM) x = fa_score_mod(s[r] * a.scale, b, h, qi + off, kj, a.mod_params) * kLog2e;
        float p = exp2_hw(x - l4[c]);
        if (!key_ok) p = 0.f;
        if (diag && kj > qi + off) p = 0.f;
        if constexpr (MOD == MOD_CUSTOM) {
          dp[r] = p != 0.f ? p * (dp[r] - d4[c]) * fa_score_mod_grad(s[r] * a.scale, b, h, qi + off, kj, a.mod_params)
                           : 0.f;
        } else {
          dp[r] = p * (dp[r] - d4[c]);
        }
        s[r] = p;
      }
    }

    // dV^T += dO^T P, dK^T += Q^T dS: step t pairs register t (query acc_row(t, hi)).
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int qr = acc_row(t, hi);
      const float* orw = sO + qr * P + e * DSL + l32;
      const float* qrw = sQ + qr * P + e * DSL + l32;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dv[dt] = mma_f32(orw[32 * dt], s[t], dv[dt]);
        dk[dt] = mma_f32(qrw[32 * dt], dp[t], dk[dt]);
      }
    }
  }

  if (kj < Skv) {
    float* dKg = (float*)a.dk + ((size_t)bh * Skv + kj) * D + e * DSL;
    float* dVg = (float*)a.dv + ((size_t)bh * Skv + kj) * D + e * DSL;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int col = 32 * dt + 8 * u + 4 * hi;
        *(f32x4*)(dKg + col) = f32x4{dk[dt][4 * u] * sc, dk[dt][4 * u + 1] * sc, dk[dt][4 * u + 2] * sc, dk[dt][4 * u + 3] * sc};
        *(f32x4*)(dVg + col) = f32x4{dv[dt][4 * u], dv[dt][4 * u + 1], dv[dt][4 * u + 2], dv[dt][4 * u + 3]};
      }
    }
  }
}

// ----------------------------------------------------------------- dQ pass

// With BLK only the key tiles whose 128 x 128 block is set are visited.
template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
__device__ __forceinline__ void dq32_body(const AttnArgs& a) {
  using C = B32Cfg<D>;
  constexpr int DS = C::DS, NG = C::NG, P = C::P;
  constexpr int DSL = D / DS, HS = DSL / 2, DT = DSL / 32;
  constexpr int BM = 32 * NG, BN = 32;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* sK = smem;
  float* sV = sK + 32 * P;
  float* sS = sV + 32 * P;
  uint8_t* sM = (uint8_t*)(sS + (DS > 1 ? 4 * 16 * 64 : 0) + 64);
  uint16_t* sList = (uint16_t*)((char*)smem + C::lds);
  int* sCnt = (int*)(sList + kBlkMaxSeq / 32);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = wave / DS, e = wave % DS;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (CAUSAL) qb = a.n_qblocks - 1 - qb;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM;
  const int qw = q0 + 32 * g;
  const int qi = qw + l32;
  const int qwp = qw + a.q_off, qpos = qi + a.q_off;   // positions among the keys

  const float* Qg = (const float*)a.q + (size_t)bh * Sq * D;
  const float* dOg = (const float*)a.dout + (size_t)bh * Sq * D;
  const float* Kg = (const float*)a.k + (size_t)bh * Skv * D;
  const float* Vg = (const float*)a.v + (size_t)bh * Skv * D;

  float qf[HS], of[HS];
  float lse2 = __builtin_inff(), delta = 0.f;
  {
    const bool ok = qi < Sq;
    const size_t off = (size_t)(ok ? qi : 0) * D + e * DSL + hi * HS;
#pragma unroll
    for (int kk = 0; kk < HS; kk += 4) {
      const f32x4 x = *(const f32x4*)(Qg + off + kk);
      const f32x4 y = *(const f32x4*)(dOg + off + kk);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qf[kk + c] = ok ? x[c] : 0.f;
        of[kk + c] = ok ? y[c] : 0.f;
      }
    }
    if (ok) {
      lse2 = a.lse2[(size_t)bh * Sq + qi];
      delta = a.delta[(size_t)bh * Sq + qi];
    }
  }

  float slope2 = 0.f, cb0 = 0.f, cb1 = 0.f;
  if constexpr (MOD == MOD_ALIBI) slope2 = alibi_slope(a.alibi_slopes, h, a.H) * kLog2e;
  if constexpr (MOD == MOD_CHECKERBOARD) {
    const bool qeven = (qpos & 1) == 0;
    cb0 = qeven ? a.even_log2 : a.odd_log2;
    cb1 = qeven ? a.odd_log2 : a.even_log2;
  }

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = zero16();

  const int kv_end = CAUSAL ? min(Skv, q0 + a.q_off + BM) : Skv;
  int ntiles = (kv_end + BN - 1) / BN;
  if constexpr (BLK) {
    const uint8_t* brow = a.block_mask + ((size_t)bh * a.bm_rows + (q0 >> 7)) * a.bm_cols;
    ntiles = compact_tiles(brow, 1, 2, 0, ntiles, sList, sCnt);   // 32-key tile t lies in block t / 4
  }
  // head_dim 512: K and V tiles arrive by direct loads (16 per wave and
  // tensor) issued from inline assembly and waited with per-wave counts: V of
  // tile j+1 is requested as soon as K of tile j has landed (every wave has
  // then read V_j for dP), K of tile j+1 once the dQ products of tile j are
  // issued; each step computes dP = dO V^T first, while its K lands.
  // Otherwise K, V tile j+1 (and its key-mask bytes) are loaded into
  // registers while tile j computes and stored to LDS after the barrier that
  // retires tile j (long fp32 workload at head_dim 512: dQ pass 408 -> 342 ms
  // before the direct loads).
  constexpr bool PIPE = D * 4 % 1024 == 0;
  auto tile_kv = [&](int j) __attribute__((always_inline)) { return (BLK ? list_at(sList, j) : j) * BN; };
  Rows32<D> rk, rv;
  uint8_t mnext = 0;
  auto fetch = [&](int kv0) __attribute__((always_inline)) {
    if constexpr (!PIPE) {
      rk.load(Kg, kv0, Skv, tid);
      rv.load(Vg, kv0, Skv, tid);
      if constexpr (MASK) {
        if (tid < BN) mnext = (kv0 + tid < Skv) ? a.key_mask[(size_t)b * Skv + kv0 + tid] : 0;
      }
    }
  };
  if (ntiles > 0) {
    if constexpr (PIPE) {
      stage32_direct<D, true>(sV, Vg, tile_kv(0), Skv, wave, lane);
      stage32_direct<D, true>(sK, Kg, tile_kv(0), Skv, wave, lane);
    } else {
      fetch(tile_kv(0));
    }
  }
  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = tile_kv(j);
    f32x16 s0 = zero16(), s1 = zero16(), p0 = zero16(), p1 = zero16();
    const float* krow = sK + l32 * P + e * DSL + hi * HS;
    const float* vrow = sV + l32 * P + e * DSL + hi * HS;
    if constexpr (PIPE) {
      uint8_t mb = 0;
      if constexpr (MASK) {   // the compiler waits for this load (and so for K_j) before the store
        if (tid < BN) mb = (kv0 + tid < Skv) ? a.key_mask[(size_t)b * Skv + kv0 + tid] : 0;
      }
      wait_vmcnt_le16();   // V_j landed; K_j may be in flight
      if constexpr (MASK) {
        if (tid < BN) sM[tid] = mb;
      }
      sync_wg();
#pragma unroll
      for (int kk = 0; kk < HS; kk += 4) {
        const f32x4 y = *(const f32x4*)(vrow + kk);
        p0 = mma_f32(y[0], of[kk + 0], p0);
        p1 = mma_f32(y[1], of[kk + 1], p1);
        p0 = mma_f32(y[2], of[kk + 2], p0);
        p1 = mma_f32(y[3], of[kk + 3], p1);
      }
      wait_direct_loads();   // K_j landed
      sync_wg();       // and V_j is dead in every wave
      if (j + 1 < ntiles) stage32_direct<D, true>(sV, Vg, tile_kv(j + 1), Skv, wave, lane);
#pragma unroll
      for (int kk = 0; kk < HS; kk += 4) {
        const f32x4 x = *(const f32x4*)(krow + kk);
        s0 = mma_f32(x[0], qf[kk + 0], s0);
        s1 = mma_f32(x[1], qf[kk + 1], s1);
        s0 = mma_f32(x[2], qf[kk + 2], s0);
        s1 = mma_f32(x[3], qf[kk + 3], s1);
      }
    } else {
      sync_wg();
      rk.store(sK, tid);
      rv.store(sV, tid);
      if constexpr (MASK) {
        if (tid < BN) sM[tid] = mnext;
      }
      if (j + 1 < ntiles) fetch(tile_kv(j + 1));
      sync_wg();
      if (DS == 1 && CAUSAL && kv0 > qwp + 31) continue;
#pragma unroll
      for (int kk = 0; kk < HS; kk += 4) {
        const f32x4 x = *(const f32x4*)(krow + kk);
        const f32x4 y = *(const f32x4*)(vrow + kk);
        s0 = mma_f32(x[0], qf[kk + 0], s0);
        s1 = mma_f32(x[1], qf[kk + 1], s1);
        p0 = mma_f32(y[0], of[kk + 0], p0);
        p1 = mma_f32(y[1], of[kk + 1], p1);
        s0 = mma_f32(x[2], qf[kk + 2], s0);
        s1 = mma_f32(x[3], qf[kk + 3], s1);
        p0 = mma_f32(y[2], of[kk + 2], p0);
        p1 = mma_f32(y[3], of[kk + 3], p1);
      }
    }
    f32x16 s = s0 + s1, dp = p0 + p1;
    if constexpr (DS > 1) {   // with PIPE the barrier before K_{j+1} orders the next exchange
      s = slice_sum<DS>(s, sS, wave, g, lane);
      dp = slice_sum<DS, !PIPE>(dp, sS, wave, g, lane);
    }

    const bool diag = CAUSAL && (kv0 + BN - 1 > qwp);
    const bool tail = kv0 + BN > Skv;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t mw = 0xffffffffu;
      if constexpr (MASK) mw = *(const uint32_t*)&sM[8 * u + 4 * hi];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * u + c;
        const int kv = kv0 + acc_row(r, hi);
        float x = s[r] * a.scale_log2;
        if constexpr (MOD == MOD_ALIBI) x += slope2 * (float)(kv - qpos);
        if constexpr (MOD == MOD_CHECKERBOARD) x += (r & 1) ? cb1 : cb0;
        if constexpr (MOD == MOD_CUSTOM) x = fa_score_mod(s[r] * a.scale, b, h, qpos, kv, a.mod_params) * kLog2e;
        float p = exp2_hw(x - lse2);
        if constexpr (MASK) {
          if (((mw >> (8 * c)) & 0xffu) == 0u) p = 0.f;
        } else {
          if (tail && kv >= Skv) p = 0.f;
        }
        if (diag && kv > qpos) p = 0.f;
        if constexpr (MOD == MOD_CUSTOM) {
          dp[r] = p != 0.f ? p * (dp[r] - delta) * fa_score_mod_grad(s[r] * a.scale, b, h, qpos, kv, a.mod_params)
                           : 0.f;
        } else {
          dp[r] = p * (dp[r] - delta);
        }
      }
    }

    // dQ^T += K^T dS^T: step t pairs register t (key acc_row(t, hi)) with that key's K row.
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float* krw = sK + acc_row(t, hi) * P + e * DSL + l32;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dq[dt] = mma_f32(krw[32 * dt], dp[t], dq[dt]);
    }
    if constexpr (PIPE) {
      sync_wg();   // K_j is dead in every wave
      if (j + 1 < ntiles) stage32_direct<D, true>(sK, Kg, tile_kv(j + 1), Skv, wave, lane);
    }
  }

  if (qi < Sq) {
    float* dQg = (float*)a.dq + ((size_t)bh * Sq + qi) * D + e * DSL;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *(f32x4*)(dQg + 32 * dt + 8 * u + 4 * hi) =
            f32x4{dq[dt][4 * u] * sc, dq[dt][4 * u + 1] * sc, dq[dt][4 * u + 2] * sc, dq[dt][4 * u + 3] * sc};
    }
  }
}

#ifndef __HIPCC_RTC__
template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
__global__ __launch_bounds__(256, 1) void dkdv32_kernel(const AttnArgs a) {
  dkdv32_body<D, MOD, CAUSAL, MASK, BLK>(a);
}

template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
__global__ __launch_bounds__(256, 1) void dq32_kernel(const AttnArgs a) {
  dq32_body<D, MOD, CAUSAL, MASK, BLK>(a);
}

template <class K>
static hipError_t launch_dyn32(K kern, unsigned grid, size_t lds, hipStream_t st, const AttnArgs& a) {
  if (lds > 65536) {
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
static hipError_t launch_bwd32_blk(const AttnArgs& a, bool want_kv, bool want_q, hipStream_t st) {
  using C = B32Cfg<D>;
  const int BH = a.B * a.H;
  const unsigned nkb = (unsigned)((a.Skv + 32 * C::NG - 1) / (32 * C::NG));
  const size_t lds = BLK ? C::lds_blk : C::lds;
  if (want_kv) {
    hipError_t err = launch_dyn32(dkdv32_kernel<D, MOD, CAUSAL, MASK, BLK>, nkb * BH, lds, st, a);
    if (err != hipSuccess) return err;
  }
  if (!want_q) return hipSuccess;
  return launch_dyn32(dq32_kernel<D, MOD, CAUSAL, MASK, BLK>, (unsigned)a.n_qblocks * BH, lds, st, a);
}

template <int D, int MOD, bool CAUSAL, bool MASK>
static hipError_t launch_bwd32_inst(const AttnArgs& a, bool want_kv, bool want_q, hipStream_t st) {
  return a.block_mask ? launch_bwd32_blk<D, MOD, CAUSAL, MASK, true>(a, want_kv, want_q, st)
                      : launch_bwd32_blk<D, MOD, CAUSAL, MASK, false>(a, want_kv, want_q, st);
}

template <int D, int MOD>
static hipError_t launch_bwd32_mod(const AttnArgs& a, bool causal, bool mask, bool kv, bool qq, hipStream_t st) {
  if (causal) return mask ? launch_bwd32_inst<D, MOD, true, true>(a, kv, qq, st) : launch_bwd32_inst<D, MOD, true, false>(a, kv, qq, st);
  return mask ? launch_bwd32_inst<D, MOD, false, true>(a, kv, qq, st) : launch_bwd32_inst<D, MOD, false, false>(a, kv, qq, st);
}

template <int D>
static hipError_t launch_bwd32_d(const AttnArgs& a, int mod, bool causal, bool mask, bool kv, bool qq, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return launch_bwd32_mod<D, MOD_ALIBI>(a, causal, mask, kv, qq, st);
    case MOD_CHECKERBOARD: return launch_bwd32_mod<D, MOD_CHECKERBOARD>(a, causal, mask, kv, qq, st);
    default: return launch_bwd32_mod<D, MOD_NONE>(a, causal, mask, kv, qq, st);
  }
}

size_t bwd32_lds_bytes(int D, bool blk) {
  if (blk) return D == 512 ? B32Cfg<512>::lds_blk : D == 128 ? B32Cfg<128>::lds_blk : B32Cfg<64>::lds_blk;
  return D == 512 ? B32Cfg<512>::lds : D == 128 ? B32Cfg<128>::lds : B32Cfg<64>::lds;
}

int bwd32_block_kv(int D) { return D >= 512 ? 32 : 128; }
int bwd32_block_q(int D) { return D >= 512 ? 32 : 128; }

hipError_t launch_bwd32(const AttnArgs& a, int D, int mod, bool causal, bool mask, bool kv, bool qq, hipStream_t st) {
  if (D == 64) return launch_bwd32_d<64>(a, mod, causal, mask, kv, qq, st);
  if (D == 128) return launch_bwd32_d<128>(a, mod, causal, mask, kv, qq, st);
  return launch_bwd32_d<512>(a, mod, causal, mask, kv, qq, st);
}

#endif  // !__HIPCC_RTC__

}  // namespace fa
