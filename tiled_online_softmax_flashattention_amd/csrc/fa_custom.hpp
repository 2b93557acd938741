// Attention kernels for a caller-defined score_mod, compiled at run time
// (hipRTC) around the caller's device functions
//
//   float fa_score_mod(float score, int b, int h, int q_idx, int kv_idx, const float* params);
//   float fa_score_mod_grad(float score, int b, int h, int q_idx, int kv_idx, const float* params);
//
// where score = scale * <q_i, k_j> in natural units, q_idx the query's
// position among the keys (row + q_offset), kv_idx the key index, and the
// second function is d fa_score_mod / d score.  This is the attnax
// pallas_flash_attention page's score_mod: a callable applied to the scaled
// scores inside the loop with global indices, before the mask; its gradient
// there comes from tracing the kernel, here from the caller's derivative:
//   s'_ij = mod(s_ij),  P = softmax(s'),  dS'_ij = P_ij (dP_ij - D_i),
//   dS_ij = dS'_ij * mod'(s_ij),  dQ = scale dS K,  dK = scale dS^T Q.
//
// The masks (causal, key mask, ragged tails) are applied after the mod, since
// a mod need not keep -inf at -inf.  Layouts and tile machinery are those of
// the 16-bit kernels (fa_common.hpp): S^T = K Q^T with one query per lane in
// the forward and the query pass, S = Q K^T with one key per lane in the
// key/value pass; K/V (or Q/dO) tiles staged by direct loads into
// double-buffered LDS; block-sparse tile lists.  The forward keeps an exact
// running maximum (one max per 32-key half), since the mod's range is unknown.
#pragma once

#include "fa_common.hpp"

namespace fa {

// ------------------------------------------------------------------ forward

// With SPLIT the workgroup covers one key chunk of its query block (the
// order and chunking of the built-in split forward: split_coord, a.chunk
// keys) and writes each row's unnormalised (accumulator, running max, sum)
// to a.partial for the merge kernels.
template <class T, int D, bool CAUSAL, bool MASK, bool BLK, bool SPLIT = false>
__device__ __forceinline__ void fwd_custom(const AttnArgs& a) {
  constexpr int BM = 128, BN = 64;
  constexpr int QS = D / 16, DT = D / 32, TILE = BN * D;
  constexpr int VSW = D == 64 ? SW_NONE : SW_TR;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];
  __shared__ uint8_t sM0[MASK ? BN : 4];
  __shared__ uint8_t sM1[MASK ? BN : 4];
  __shared__ uint16_t sList[BLK ? kBlkMaxSeq / BN : 1];
  __shared__ int sCnt[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  int bh, qb, split = 0;
  if constexpr (SPLIT) {
    const SplitCoord c = split_coord(blockIdx.x, a.B * a.H, a.n_qblocks, a.n_split, CAUSAL);
    bh = c.bh;
    qb = c.qb;
    split = c.split;
  } else {
    const BlockCoord bc = block_coord(blockIdx.x, a.B * a.H, a.n_qblocks, CAUSAL);
    bh = bc.bh;
    qb = CAUSAL ? a.n_qblocks - 1 - bc.blk : bc.blk;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM, qw = q0 + 32 * wave, qi = qw + l32;
  const int qwp = qw + a.q_off, qpos = qi + a.q_off;
  const float scale = a.scale;

  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * Sq * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * Skv * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * Skv * D;

  const int kv_end = CAUSAL ? min(Skv, min(q0 + BM, Sq) + a.q_off) : Skv;
  const int ntiles_all = (kv_end + BN - 1) / BN;
  int t_lo = 0, t_hi = ntiles_all;
  if constexpr (SPLIT) {
    const int ct = a.chunk / BN;
    t_lo = min(split * ct, ntiles_all);
    t_hi = min(t_lo + ct, ntiles_all);
    if (t_lo >= ntiles_all) return;   // past the block's last key: no row reads this partial
  }

  u32x4 qf[QS];
  {
    const bool ok = qi < Sq;
    const uint16_t* src = Qg + (size_t)(ok ? qi : 0) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < QS; ++kk) {
      const u32x4 v = *(const u32x4*)(src + 16 * kk);
      qf[kk] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  int ntiles = t_hi - t_lo;
  if constexpr (BLK) {
    const uint8_t* brow = a.block_mask + ((size_t)bh * a.bm_rows + (q0 >> 7)) * a.bm_cols;
    ntiles = compact_tiles(brow, 1, 1, t_lo, t_hi, sList, sCnt);
  }
  auto kv_of = [&](int n) __attribute__((always_inline)) { return (BLK ? list_at(sList, n) : t_lo + n) * BN; };
  auto load_tile = [&](int kv0, uint16_t* sK, uint16_t* sV, uint8_t* sM) __attribute__((always_inline)) {
    load_tile_lds<D, BN, SW_BOTH>(Kg, kv0, Skv, sK, wave, lane);
    load_tile_lds<D, BN, VSW>(Vg, kv0, Skv, sV, wave, lane);
    if constexpr (MASK) {
      if (tid < BN) sM[tid] = a.key_mask[(size_t)b * Skv + min(kv0 + tid, Skv - 1)];
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero16();

  auto half = [&](int kv0, int t, const uint16_t* sK, const uint16_t* sV, const uint8_t* sM)
                  __attribute__((always_inline)) {
    const int k0 = kv0 + 32 * t;
    if (CAUSAL && k0 > qwp + 31) return;
    f32x16 s = zero16();
    {
      const int kr = 32 * t + l32;
      u32x4 kfr[QS];
#pragma unroll
      for (int kk = 0; kk < QS; ++kk) kfr[kk] = lds_read16(sK + tile_off<D, SW_BOTH>(kr, 16 * kk + 8 * hi));
#pragma unroll
      for (int kk = 0; kk < QS; ++kk) s = mma16<T>(kfr[kk], qf[kk], s);
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = k0 + acc_row(r, hi);
      bool ok = kv < Skv && (!CAUSAL || kv <= qpos);
      if constexpr (MASK) ok = ok && sM[32 * t + acc_row(r, hi)] != 0;
      const float x = fa_score_mod(s[r] * scale, b, h, qpos, kv, a.mod_params) * kLog2e;
      s[r] = ok ? x : kNegInf;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_hw(s[r] - m_use);
      ls += s[r];
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 pb = u32x4{pack2<T>(s[8 * u + 0], s[8 * u + 1]), pack2<T>(s[8 * u + 2], s[8 * u + 3]),
                             pack2<T>(s[8 * u + 4], s[8 * u + 5]), pack2<T>(s[8 * u + 6], s[8 * u + 7])};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = mma16<T>(read_a_tr_tile<D, VSW>(sV, 32 * t + 16 * u, 32 * dt, lane), pb, o[dt]);
    }
  };

  auto tile = [&](int n, const uint16_t* sK, const uint16_t* sV, const uint8_t* sM, uint16_t* sKn, uint16_t* sVn,
                  uint8_t* sMn) __attribute__((always_inline)) {
    wait_direct_loads();
    sync_wg();
    if (n + 1 < ntiles) load_tile(kv_of(n + 1), sKn, sVn, sMn);
    if (qw < Sq) {
      const int kv0 = kv_of(n);
      half(kv0, 0, sK, sV, sM);
      half(kv0, 1, sK, sV, sM);
    }
  };
  if (ntiles > 0) load_tile(kv_of(0), sK0, sV0, sM0);
  int n = 0;
  for (; n + 1 < ntiles; n += 2) {
    tile(n, sK0, sV0, sM0, sK1, sV1, sM1);
    tile(n + 1, sK1, sV1, sM1, sK0, sV0, sM0);
  }
  if (n < ntiles) tile(n, sK0, sV0, sM0, sK1, sV1, sM1);

  const float l_tot = l_run + xor32(l_run);
  if constexpr (SPLIT) {
    if (qi < Sq) {
      float* P = a.partial + (((size_t)bh * Sq + qi) * a.n_split + split) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) P[32 * dt + 8 * (r >> 2) + 4 * hi + (r & 3)] = o[dt][r];
      }
      if (hi == 0) {
        P[D] = l_tot > 0.f ? m_run : kNegInf;
        P[D + 1] = l_tot;
      }
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < Sq) {
    uint16_t* Og = (uint16_t*)a.o + ((size_t)bh * Sq + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x2 w = {pack2<T>(o[dt][4 * u] * inv, o[dt][4 * u + 1] * inv),
                         pack2<T>(o[dt][4 * u + 2] * inv, o[dt][4 * u + 3] * inv)};
        *(u32x2*)(Og + 32 * dt + 8 * u + 4 * hi) = w;
      }
    }
    if (hi == 0 && a.lse) a.lse[(size_t)bh * Sq + qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
  }
}

// ------------------------------------------------------------- query pass

// delta (plain rowsum(dO o O)) and lse2 = lse log2(e) (+inf for an empty
// row) come from the preprocess kernel.  Per score: P = 2^(mod(s) log2 e -
// lse2), dS = P (dP - delta) mod'(s); dQ^T += K^T dS^T.
template <class T, int D, bool CAUSAL, bool MASK, bool BLK>
__device__ __forceinline__ void dq_custom(const AttnArgs& a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16, DT = D / 32, TILE = BN * D;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];
  __shared__ uint8_t sM0[MASK ? BN : 4];
  __shared__ uint8_t sM1[MASK ? BN : 4];
  __shared__ uint16_t sList[BLK ? kBlkMaxSeq / BN : 1];
  __shared__ int sCnt[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const BlockCoord bc = block_coord(blockIdx.x, a.B * a.H, a.n_qblocks, CAUSAL);
  const int bh = bc.bh, qb = CAUSAL ? a.n_qblocks - 1 - bc.blk : bc.blk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM, qw = q0 + 32 * wave, qi = qw + l32;
  const int qwp = qw + a.q_off, qpos = qi + a.q_off;
  const float scale = a.scale;

  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * Sq * D;
  const uint16_t* dOg = (const uint16_t*)a.dout + (size_t)bh * Sq * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * Skv * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * Skv * D;

  u32x4 qf[KS], of[KS];
  {
    const bool ok = qi < Sq;
    const size_t off = (size_t)min(qi, Sq - 1) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const u32x4 x = *(const u32x4*)(Qg + off + 16 * kk);
      const u32x4 y = *(const u32x4*)(dOg + off + 16 * kk);
      qf[kk] = ok ? x : u32x4{0u, 0u, 0u, 0u};
      of[kk] = ok ? y : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const size_t row = (size_t)bh * Sq + min(qi, Sq - 1);
  const float lse2 = qi < Sq ? a.lse2[row] : __builtin_inff();
  const float delta = qi < Sq ? a.delta[row] : 0.f;

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = zero16();

  const int kv_end = CAUSAL ? min(Skv, q0 + a.q_off + BM) : Skv;
  int ntiles = (kv_end + BN - 1) / BN;
  if constexpr (BLK) {
    const uint8_t* brow = a.block_mask + ((size_t)bh * a.bm_rows + qb) * a.bm_cols;
    ntiles = compact_tiles(brow, 1, 1, 0, ntiles, sList, sCnt);
  }
  auto kv_of = [&](int n) __attribute__((always_inline)) { return (BLK ? list_at(sList, n) : n) * BN; };
  auto load_tile = [&](int kv0, uint16_t* sK, uint16_t* sV, uint8_t* sM) __attribute__((always_inline)) {
    load_tile_lds<D, BN, SW_BOTH>(Kg, kv0, Skv, sK, wave, lane);
    load_tile_lds<D, BN, SW_BOTH>(Vg, kv0, Skv, sV, wave, lane);
    if constexpr (MASK) {
      if (tid < BN) sM[tid] = a.key_mask[(size_t)b * Skv + min(kv0 + tid, Skv - 1)];
    }
  };

  auto half = [&](int kv0, int t, const uint16_t* sK, const uint16_t* sV, const uint8_t* sM)
                  __attribute__((always_inline)) {
    const int k0 = kv0 + 32 * t;
    if (CAUSAL && k0 > qwp + 31) return;
    f32x16 s = zero16(), dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = -delta;
    {
      const int kr = 32 * t + l32;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int off = tile_off<D, SW_BOTH>(kr, 16 * kk + 8 * hi);
        s = mma16<T>(lds_read16(sK + off), qf[kk], s);
        dp = mma16<T>(lds_read16(sV + off), of[kk], dp);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = k0 + acc_row(r, hi);
      bool ok = kv < Skv && (!CAUSAL || kv <= qpos);
      if constexpr (MASK) ok = ok && sM[32 * t + acc_row(r, hi)] != 0;
      const float sr = s[r] * scale;
      const float x = fa_score_mod(sr, b, h, qpos, kv, a.mod_params) * kLog2e;
      const float p = ok ? exp2_hw(x - lse2) : 0.f;
      dp[r] = ok ? p * dp[r] * fa_score_mod_grad(sr, b, h, qpos, kv, a.mod_params) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 db = u32x4{pack2<T>(dp[8 * u + 0], dp[8 * u + 1]), pack2<T>(dp[8 * u + 2], dp[8 * u + 3]),
                             pack2<T>(dp[8 * u + 4], dp[8 * u + 5]), pack2<T>(dp[8 * u + 6], dp[8 * u + 7])};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        dq[dt] = mma16<T>(read_a_tr_tile<D, SW_BOTH>(sK, 32 * t + 16 * u, 32 * dt, lane), db, dq[dt]);
    }
  };

  auto tile = [&](int n, const uint16_t* sK, const uint16_t* sV, const uint8_t* sM, uint16_t* sKn, uint16_t* sVn,
                  uint8_t* sMn) __attribute__((always_inline)) {
    wait_direct_loads();
    sync_wg();
    if (n + 1 < ntiles) load_tile(kv_of(n + 1), sKn, sVn, sMn);
    const int kv0 = kv_of(n);
    half(kv0, 0, sK, sV, sM);
    half(kv0, 1, sK, sV, sM);
  };
  if (ntiles > 0) load_tile(kv_of(0), sK0, sV0, sM0);
  int n = 0;
  for (; n + 1 < ntiles; n += 2) {
    tile(n, sK0, sV0, sM0, sK1, sV1, sM1);
    tile(n + 1, sK1, sV1, sM1, sK0, sV0, sM0);
  }
  if (n < ntiles) tile(n, sK0, sV0, sM0, sK1, sV1, sM1);

  if (qi < Sq) {
    uint16_t* dQg = (uint16_t*)a.dq + ((size_t)bh * Sq + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *(u32x2*)(dQg + 32 * dt + 8 * u + 4 * hi) =
            u32x2{pack2<T>(dq[dt][4 * u] * scale, dq[dt][4 * u + 1] * scale),
                  pack2<T>(dq[dt][4 * u + 2] * scale, dq[dt][4 * u + 3] * scale)};
    }
  }
}

// --------------------------------------------------------- key/value pass

// One key per lane (S = Q K^T, queries as rows).  Q and dO tiles of 64
// queries with their lse2 and delta rows go by direct loads into
// double-buffered LDS.  dV^T += dO^T P, dK^T += Q^T dS.
template <class T, int D, bool CAUSAL, bool MASK, bool BLK>
__device__ __forceinline__ void dkdv_custom(const AttnArgs& a) {
  constexpr int BKV = 128, BQ = 64;
  constexpr int KS = D / 16, DT = D / 32, TILE = BQ * D;
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sO0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sO1[TILE];
  __shared__ __attribute__((aligned(16))) float sL0[BQ];
  __shared__ __attribute__((aligned(16))) float sL1[BQ];
  __shared__ __attribute__((aligned(16))) float sD0[BQ];
  __shared__ __attribute__((aligned(16))) float sD1[BQ];
  __shared__ uint16_t sList[BLK ? kBlkMaxSeq / BQ : 1];
  __shared__ int sCnt[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const BlockCoord bc = block_coord(blockIdx.x, BH, (a.Skv + BKV - 1) / BKV, CAUSAL);
  const int bh = bc.bh, kb = bc.blk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int k0 = kb * BKV, kw = k0 + 32 * wave, kj = kw + l32;
  const int off = a.q_off;
  const float scale = a.scale;

  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * Sq * D;
  const uint16_t* dOg = (const uint16_t*)a.dout + (size_t)bh * Sq * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * Skv * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * Skv * D;
  const float* lse2g = a.lse2 + (size_t)bh * Sq;
  const float* deltag = a.delta + (size_t)bh * Sq;

  u32x4 kf[KS], vf[KS];
  {
    const size_t o2 = (size_t)min(kj, Skv - 1) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      kf[kk] = *(const u32x4*)(Kg + o2 + 16 * kk);
      vf[kk] = *(const u32x4*)(Vg + o2 + 16 * kk);
    }
  }
  bool key_ok = kj < Skv;
  if constexpr (MASK) key_ok = key_ok && a.key_mask[(size_t)b * Skv + min(kj, Skv - 1)] != 0;

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  const int qt0 = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int nqt = (Sq + BQ - 1) / BQ;
  int n0 = qt0, n_end = nqt;
  if constexpr (BLK) {
    const uint8_t* bcol = a.block_mask + (size_t)bh * a.bm_rows * a.bm_cols + kb;
    n0 = 0;
    n_end = compact_tiles(bcol, a.bm_cols, 1, qt0, nqt, sList, sCnt);
  }
  auto it_of = [&](int n) __attribute__((always_inline)) { return BLK ? list_at(sList, n) : n; };
  auto load_tile = [&](int it, uint16_t* sQ, uint16_t* sO, float* sL, float* sD) __attribute__((always_inline)) {
    const int q0 = it * BQ;
    load_tile_lds<D, BQ, SW_BOTH>(Qg, q0, Sq, sQ, wave, lane);
    load_tile_lds<D, BQ, SW_BOTH>(dOg, q0, Sq, sO, wave, lane);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((const void*)(lse2g + min(q0 + lane, Sq - 1)), (lds_void_ptr)sL, 4, 0, 0);
    if (wave == 1)
      __builtin_amdgcn_global_load_lds((const void*)(deltag + min(q0 + lane, Sq - 1)), (lds_void_ptr)sD, 4, 0, 0);
  };

  auto half = [&](int it, int mt, const uint16_t* sQ, const uint16_t* sO, const float* sL, const float* sD)
                  __attribute__((always_inline)) {
    const int qs = it * BQ + 32 * mt;
    if (CAUSAL && qs + off + 31 < kw) return;
    const float* lrow = sL + 32 * mt + 4 * hi;
    const float* drow = sD + 32 * mt + 4 * hi;
    f32x16 sv = zero16(), dpv, l2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 l4 = *(const f32x4*)(lrow + 8 * u);
      const f32x4 d4 = *(const f32x4*)(drow + 8 * u);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        l2[4 * u + cc] = l4[cc];
        dpv[4 * u + cc] = -d4[cc];
      }
    }
    {
      const int qr = 32 * mt + l32;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int o2 = tile_off<D, SW_BOTH>(qr, 16 * kk + 8 * hi);
        sv = mma16<T>(lds_read16(sQ + o2), kf[kk], sv);
        dpv = mma16<T>(lds_read16(sO + o2), vf[kk], dpv);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = qs + acc_row(r, hi);
      const bool ok = key_ok && q < Sq && (!CAUSAL || kj <= q + off);
      const float sr = sv[r] * scale;
      const float x = fa_score_mod(sr, b, h, q + off, kj, a.mod_params) * kLog2e;
      const float p = ok ? exp2_hw(x - l2[r]) : 0.f;
      sv[r] = p;
      dpv[r] = ok ? p * dpv[r] * fa_score_mod_grad(sr, b, h, q + off, kj, a.mod_params) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p0 = 32 * mt + 16 * u;
      const u32x4 pb = u32x4{pack2<T>(sv[8 * u + 0], sv[8 * u + 1]), pack2<T>(sv[8 * u + 2], sv[8 * u + 3]),
                             pack2<T>(sv[8 * u + 4], sv[8 * u + 5]), pack2<T>(sv[8 * u + 6], sv[8 * u + 7])};
      const u32x4 db = u32x4{pack2<T>(dpv[8 * u + 0], dpv[8 * u + 1]), pack2<T>(dpv[8 * u + 2], dpv[8 * u + 3]),
                             pack2<T>(dpv[8 * u + 4], dpv[8 * u + 5]), pack2<T>(dpv[8 * u + 6], dpv[8 * u + 7])};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dv[dt] = mma16<T>(read_a_tr_tile<D, SW_BOTH>(sO, p0, 32 * dt, lane), pb, dv[dt]);
        dk[dt] = mma16<T>(read_a_tr_tile<D, SW_BOTH>(sQ, p0, 32 * dt, lane), db, dk[dt]);
      }
    }
  };

  auto tile = [&](int n, const uint16_t* sQ, const uint16_t* sO, const float* sL, const float* sD, uint16_t* sQn,
                  uint16_t* sOn, float* sLn, float* sDn) __attribute__((always_inline)) {
    wait_direct_loads();
    sync_wg();
    if (n + 1 < n_end) load_tile(it_of(n + 1), sQn, sOn, sLn, sDn);
    const int it = it_of(n);
    half(it, 0, sQ, sO, sL, sD);
    half(it, 1, sQ, sO, sL, sD);
  };
  if (n0 < n_end) load_tile(it_of(n0), sQ0, sO0, sL0, sD0);
  int n = n0;
  for (; n + 1 < n_end; n += 2) {
    tile(n, sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1);
    tile(n + 1, sQ1, sO1, sL1, sD1, sQ0, sO0, sL0, sD0);
  }
  if (n < n_end) tile(n, sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1);

  if (kj < Skv) {
    uint16_t* dKg = (uint16_t*)a.dk + ((size_t)bh * Skv + kj) * D;
    uint16_t* dVg = (uint16_t*)a.dv + ((size_t)bh * Skv + kj) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int col = 32 * dt + 8 * u + 4 * hi;
        *(u32x2*)(dKg + col) = u32x2{pack2<T>(dk[dt][4 * u] * scale, dk[dt][4 * u + 1] * scale),
                                     pack2<T>(dk[dt][4 * u + 2] * scale, dk[dt][4 * u + 3] * scale)};
        *(u32x2*)(dVg + col) = u32x2{pack2<T>(dv[dt][4 * u], dv[dt][4 * u + 1]),
                                     pack2<T>(dv[dt][4 * u + 2], dv[dt][4 * u + 3])};
      }
    }
  }
}

}  // namespace fa
