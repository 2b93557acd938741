// Forward attention for fp32 inputs, head_dim 64, 128 or 512.
//
// Same online-softmax recurrence as the 16-bit kernel (attnax
// pallas_flash_attention page, kernel body; base-2 exponentials), on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32: one operand value per lane, so V is
// read in its natural layout and no transposed copy is needed).
//
// Large heads are split over waves: with DS slices, each of the DS waves of a
// 32-query group holds Q and the O accumulator for D/DS dims only, computes a
// partial S^T over those dims, and the DS partials are summed through LDS
// before the (redundant, bit-identical) softmax in each wave.  At D = 512 this
// keeps Q (64 values) and the accumulator (64 values) per lane in registers
// while a 32-key K tile and V tile (128 KiB together) sit in LDS.
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
struct F32Cfg {
  static constexpr int DS = D >= 512 ? 4 : 1;   // dim slices per query group
  static constexpr int NQ = 4 / DS;             // 32-query groups per workgroup
  static constexpr int BM = 32 * NQ;
  static constexpr int BN = 32;
  static constexpr int P = D + 4;               // LDS pitch of the K and V tiles (floats)
  static constexpr size_t lds = (size_t)2 * BN * P * 4 + (DS > 1 ? 4 * 16 * 64 * 4 : 0) + 64;
  // block-sparse: the list of visited 32-key tiles and 4 counters after the tiles
  static constexpr size_t lds_blk = lds + (size_t)kBlkMaxSeq / BN * 2 + 16;
};

// With BLK only the key tiles whose 128 x 128 block is set in the block mask
// are visited (a workgroup's queries lie in one block row).  With SPLIT
// (head_dim <= 128; a short query block against a long key sequence) the
// grid is (batch * heads) x query blocks x a.n_split key chunks of a.chunk
// keys, and each workgroup writes its rows' unnormalised partial
// (accumulator, running max, sum) to a.partial for the decode merge.
// MOD_CUSTOM: the caller's fa_score_mod on the scaled score (at head_dim 512
// after the partial scores are summed), before the masks; compiled only at
// run time with the caller's source.  WQ < 4 (split, head_dim <= 128, no
// block mask): a workgroup of WQ waves and 32 WQ queries, for query blocks
// of at most that many rows, whose other waves would have no query; the
// device then holds several such workgroups per CU.
template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK, bool SPLIT = false, int WQ = 4>
__device__ __forceinline__ void fwd32_body(const AttnArgs& a) {
  using C = F32Cfg<D>;
  constexpr int DS = C::DS, BN = C::BN, P = C::P;
  constexpr int BM = WQ < 4 ? 32 * WQ : C::BM;
  constexpr int NT = WQ < 4 ? 64 * WQ : 256;   // threads of the workgroup
  constexpr int DSL = D / DS;          // dims per slice
  constexpr int HS = DSL / 2;          // operand values per lane per product
  constexpr int DT = DSL / 32;         // 32-row tiles of the O^T slice
  constexpr int NCH = BN * D / 4 / NT;
  static_assert(WQ == 4 || (SPLIT && DS == 1 && !BLK), "small workgroups: split, head_dim <= 128, dense");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* sK = smem;
  float* sV = sK + BN * P;
  float* sS = sV + BN * P;
  uint8_t* sM = (uint8_t*)(sS + (DS > 1 ? 4 * 16 * 64 : 0));
  uint16_t* sList = (uint16_t*)((char*)smem + C::lds);
  int* sCnt = (int*)(sList + kBlkMaxSeq / BN);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = wave / DS, e = wave % DS;
  static_assert(!SPLIT || DS == 1, "the key split is built for head_dim <= 128");
  const int BH = a.B * a.H;
  int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH, split = 0;
  if constexpr (SPLIT) {
    const SplitCoord c = split_coord(blockIdx.x, BH, a.n_qblocks, a.n_split, CAUSAL);
    bh = c.bh;
    qb = c.qb;
    split = c.split;
  } else if (CAUSAL) {
    qb = a.n_qblocks - 1 - qb;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM;
  const int qw = q0 + 32 * g;
  const int qi = qw + l32;
  const int qwp = qw + a.q_off, qpos = qi + a.q_off;   // positions among the keys

  const float* Qg = (const float*)a.q + (size_t)bh * Sq * D;
  const float* Kg = (const float*)a.k + (size_t)bh * Skv * D;
  const float* Vg = (const float*)a.v + (size_t)bh * Skv * D;

  // Q as the B operand: lane (query l32, group hi) holds dims e*DSL + hi*HS + kk.
  float qf[HS];
  {
    const bool ok = qi < Sq;
    const float* src = Qg + (size_t)(ok ? qi : 0) * D + e * DSL + hi * HS;
#pragma unroll
    for (int kk = 0; kk < HS; kk += 4) {
      const f32x4 v = *(const f32x4*)(src + kk);
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[kk + c] = ok ? v[c] : 0.f;
    }
  }

  float slope2 = 0.f, cb0 = 0.f, cb1 = 0.f;
  if constexpr (MOD == MOD_ALIBI) slope2 = alibi_slope(a.alibi_slopes, h, a.H) * kLog2e;
  if constexpr (MOD == MOD_CHECKERBOARD) {
    const bool qeven = (qpos & 1) == 0;
    cb0 = qeven ? a.even_log2 : a.odd_log2;
    cb1 = qeven ? a.odd_log2 : a.even_log2;
  }

  const int kv_end = CAUSAL ? min(Skv, q0 + a.q_off + BM) : Skv;
  const int ntiles_all = (kv_end + BN - 1) / BN;
  int t_lo = 0, t_hi = ntiles_all;   // the 32-key tiles this workgroup visits
  if constexpr (SPLIT) {
    const int ct = a.chunk / BN;
    t_lo = min(split * ct, ntiles_all);
    t_hi = min(t_lo + ct, ntiles_all);
    if (t_lo >= ntiles_all) return;   // past the block's last key: no row reads this partial
  }
  int ntiles = t_hi - t_lo;
  if constexpr (BLK) {
    const uint8_t* brow = a.block_mask + ((size_t)bh * a.bm_rows + (q0 >> 7)) * a.bm_cols;
    ntiles = compact_tiles(brow, 1, 2, t_lo, t_hi, sList, sCnt);   // 32-key tile t lies in block t / 4
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero16();

  // head_dim 512: K and V tiles arrive by direct loads (16 per wave and
  // tensor), pipelined over the two LDS buffers: K of tile j+1 is requested
  // once the partial scores of tile j are exchanged (K_j is then dead) and
  // lands during the softmax and P V of tile j; V of tile j+1 is requested
  // when P V of tile j is done and lands during the scores of tile j+1.  Each
  // wait counts the wave's own direct loads still allowed in flight.
  constexpr bool PIPE = D * 4 % 1024 == 0;
  auto tile_kv = [&](int j) __attribute__((always_inline)) { return (BLK ? list_at(sList, j) : t_lo + j) * BN; };
  if constexpr (PIPE) {
    if (ntiles > 0) stage32_direct<D, true>(sK, Kg, tile_kv(0), Skv, wave, lane);
  }
  // head_dim <= 128 with four waves: tile j+1 is read into registers while
  // tile j is computed, and stored to LDS after the next barrier
  constexpr bool PREF = !PIPE && WQ == 4;
  f32x4 pk[PREF ? NCH : 1], pv[PREF ? NCH : 1];
  uint8_t pmb = 0;
  auto fetch = [&](int kv0) __attribute__((always_inline)) {
    if constexpr (PREF) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        // rows past seq_kv: the last row (finite; its scores are masked to -inf)
        const int c = tid + NT * i, row = c / (D / 4), ch = c % (D / 4), kv = min(kv0 + row, Skv - 1);
        pk[i] = *(const f32x4*)(Kg + (size_t)kv * D + 4 * ch);
        pv[i] = *(const f32x4*)(Vg + (size_t)kv * D + 4 * ch);
      }
      if constexpr (MASK) {
        if (tid < BN) pmb = (kv0 + tid < Skv) ? a.key_mask[(size_t)b * Skv + kv0 + tid] : 0;
      }
    }
  };
  if (PREF && ntiles > 0) fetch(tile_kv(0));
  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = tile_kv(j);
    sync_wg();   // every wave is done with tile j-1 (its P V read V)
    if constexpr (PREF) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = tid + NT * i, row = c / (D / 4), ch = c % (D / 4);
        *(f32x4*)&sK[row * P + 4 * ch] = pk[i];
        *(f32x4*)&sV[row * P + 4 * ch] = pv[i];
      }
      if constexpr (MASK) {
        if (tid < BN) sM[tid] = pmb;
      }
      if (j + 1 < ntiles) fetch(tile_kv(j + 1));
    } else if constexpr (PIPE) {
      uint8_t mb = 0;
      if constexpr (MASK) {   // issued before V_j, so the wait below covers it
        if (tid < BN) mb = (kv0 + tid < Skv) ? a.key_mask[(size_t)b * Skv + kv0 + tid] : 0;
      }
      stage32_direct<D, true>(sV, Vg, kv0, Skv, wave, lane);
      wait_vmcnt_le16();   // K_j (and the mask bytes) landed; V_j may be in flight
      if constexpr (MASK) {
        if (tid < BN) sM[tid] = mb;
      }
    } else {
#pragma unroll 4
      for (int i = 0; i < NCH; ++i) {
        // rows past seq_kv: the last row (finite; its scores are masked to -inf)
        const int c = tid + NT * i, row = c / (D / 4), ch = c % (D / 4), kv = min(kv0 + row, Skv - 1);
        const f32x4 kx = *(const f32x4*)(Kg + (size_t)kv * D + 4 * ch);
        const f32x4 vx = *(const f32x4*)(Vg + (size_t)kv * D + 4 * ch);
        *(f32x4*)&sK[row * P + 4 * ch] = kx;
        *(f32x4*)&sV[row * P + 4 * ch] = vx;
      }
    }
    if constexpr (MASK && !PIPE && !PREF) {
      if (tid < BN) sM[tid] = (kv0 + tid < Skv) ? a.key_mask[(size_t)b * Skv + kv0 + tid] : 0;
    }
    sync_wg();
    if (DS == 1 && CAUSAL && kv0 > qwp + 31) continue;

    f32x16 s0 = zero16(), s1 = zero16();
    const float* krow = sK + l32 * P + e * DSL + hi * HS;
#pragma unroll
    for (int kk = 0; kk < HS; kk += 4) {
      const f32x4 kx = *(const f32x4*)(krow + kk);
      s0 = mma_f32(kx[0], qf[kk + 0], s0);
      s1 = mma_f32(kx[1], qf[kk + 1], s1);
      s0 = mma_f32(kx[2], qf[kk + 2], s0);
      s1 = mma_f32(kx[3], qf[kk + 3], s1);
    }
    f32x16 s = s0 + s1;
    if constexpr (DS > 1) {
      slice_put(sS, s, wave, lane);
      sync_wg();   // every wave's partial scores are in: K_j is dead
      if constexpr (PIPE) {
        if (j + 1 < ntiles) stage32_direct<D, true>(sK, Kg, tile_kv(j + 1), Skv, wave, lane);
      }
      s = slice_gather<DS>(sS, g, lane);
    }

    const bool diag = CAUSAL && (kv0 + BN - 1 > qwp);
    const bool tail = kv0 + BN > Skv;
    float mx = kNegInf;
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
        if constexpr (MASK) {
          if (((mw >> (8 * c)) & 0xffu) == 0u) x = kNegInf;
        } else {
          if (tail && kv >= Skv) x = kNegInf;
        }
        if (diag && kv > qpos) x = kNegInf;
        s[r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_hw(s[r] - m_use);
      s[r] = p;
      ls += p;
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // alpha is exactly 1 wherever the running max did not move: skip the
    // rescale when that holds for the whole wave (the usual case once a
    // row's largest scores are in)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }

    if constexpr (PIPE) {   // V_j landed (K_{j+1} may be in flight) in every wave
      if (j + 1 < ntiles) wait_vmcnt_le16();
      else wait_direct_loads();
      sync_wg();
    }

    // O^T += V^T P^T: step t pairs register t of the probabilities (key
    // acc_row(t, hi)) with that key's V row, one key per lane group.
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float* vrow = sV + acc_row(t, hi) * P + e * DSL + l32;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = mma_f32(vrow[32 * dt], s[t], o[dt]);
    }
  }

  const float l_tot = l_run + xor32(l_run);
  if constexpr (SPLIT) {
    if (qi < Sq) {
      float* Pp = a.partial + (((size_t)bh * Sq + qi) * a.n_split + split) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Pp[32 * dt + 8 * (r >> 2) + 4 * hi + (r & 3)] = o[dt][r];
      }
      if (hi == 0) {
        Pp[D] = l_tot > 0.f ? m_run : kNegInf;
        Pp[D + 1] = l_tot;
      }
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < Sq) {
    float* Og = (float*)a.o + ((size_t)bh * Sq + qi) * D + e * DSL;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 w = {o[dt][4 * u] * inv, o[dt][4 * u + 1] * inv, o[dt][4 * u + 2] * inv, o[dt][4 * u + 3] * inv};
        *(f32x4*)(Og + 32 * dt + 8 * u + 4 * hi) = w;
      }
    }
    if (e == 0 && hi == 0 && a.lse) a.lse[(size_t)bh * Sq + qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
  }
}

#ifndef __HIPCC_RTC__
template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK, bool SPLIT = false>
__global__ __launch_bounds__(256, 1) void fwd32_kernel(const AttnArgs a) {
  fwd32_body<D, MOD, CAUSAL, MASK, BLK, SPLIT>(a);
}

// Split forward of a query block of at most 32 WQ rows: WQ waves per
// workgroup (the second bound: waves per SIMD; 8 such workgroups fit a CU's
// LDS at head_dim 64, 4 at 128).
template <int D, int MOD, bool CAUSAL, bool MASK, int WQ>
__global__ __launch_bounds__(64 * WQ, D == 64 ? 2 : 1) void fwd32_short_kernel(const AttnArgs a) {
  fwd32_body<D, MOD, CAUSAL, MASK, false, true, WQ>(a);
}

template <int D, int MOD, bool CAUSAL, bool MASK, bool BLK, bool SPLIT>
static hipError_t launch_one_blk(const AttnArgs& a, hipStream_t st) {
  auto kern = fwd32_kernel<D, MOD, CAUSAL, MASK, BLK, SPLIT>;
  const size_t lds = BLK ? F32Cfg<D>::lds_blk : F32Cfg<D>::lds;
  if (lds > 65536) {
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  const unsigned blocks = (unsigned)(a.n_qblocks * a.B * a.H) * (SPLIT ? (unsigned)a.n_split : 1u);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int D, int MOD, bool CAUSAL, bool MASK, bool SPLIT>
static hipError_t launch_one(const AttnArgs& a, hipStream_t st) {
  if constexpr (SPLIT && D <= 128) {
    if (!a.block_mask && a.Sq <= 64) {
      const unsigned blocks = (unsigned)(a.n_qblocks * a.B * a.H) * (unsigned)a.n_split;
      if (a.Sq <= 32)
        hipLaunchKernelGGL((fwd32_short_kernel<D, MOD, CAUSAL, MASK, 1>), dim3(blocks), dim3(64), F32Cfg<D>::lds, st, a);
      else
        hipLaunchKernelGGL((fwd32_short_kernel<D, MOD, CAUSAL, MASK, 2>), dim3(blocks), dim3(128), F32Cfg<D>::lds, st, a);
      return hipGetLastError();
    }
  }
  return a.block_mask ? launch_one_blk<D, MOD, CAUSAL, MASK, true, SPLIT>(a, st)
                      : launch_one_blk<D, MOD, CAUSAL, MASK, false, SPLIT>(a, st);
}

template <int D, int MOD, bool SPLIT>
static hipError_t launch_fwd32_mod(const AttnArgs& a, bool causal, bool mask, hipStream_t st) {
  if (causal)
    return mask ? launch_one<D, MOD, true, true, SPLIT>(a, st) : launch_one<D, MOD, true, false, SPLIT>(a, st);
  return mask ? launch_one<D, MOD, false, true, SPLIT>(a, st) : launch_one<D, MOD, false, false, SPLIT>(a, st);
}

template <int D, bool SPLIT>
static hipError_t launch_fwd32_d(const AttnArgs& a, int mod, bool causal, bool mask, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return launch_fwd32_mod<D, MOD_ALIBI, SPLIT>(a, causal, mask, st);
    case MOD_CHECKERBOARD: return launch_fwd32_mod<D, MOD_CHECKERBOARD, SPLIT>(a, causal, mask, st);
    default: return launch_fwd32_mod<D, MOD_NONE, SPLIT>(a, causal, mask, st);
  }
}

int fwd32_block_q(int D) {
  return D == 512 ? F32Cfg<512>::BM : D == 128 ? F32Cfg<128>::BM : F32Cfg<64>::BM;
}

size_t fwd32_lds_bytes(int D, bool blk) {
  if (blk) return D == 512 ? F32Cfg<512>::lds_blk : D == 128 ? F32Cfg<128>::lds_blk : F32Cfg<64>::lds_blk;
  return D == 512 ? F32Cfg<512>::lds : D == 128 ? F32Cfg<128>::lds : F32Cfg<64>::lds;
}

hipError_t launch_fwd32(const AttnArgs& a, int D, int mod, bool causal, bool mask, hipStream_t st, bool split) {
  if (split) return D == 64 ? launch_fwd32_d<64, true>(a, mod, causal, mask, st)
                            : launch_fwd32_d<128, true>(a, mod, causal, mask, st);
  if (D == 64) return launch_fwd32_d<64, false>(a, mod, causal, mask, st);
  if (D == 128) return launch_fwd32_d<128, false>(a, mod, causal, mask, st);
  return launch_fwd32_d<512, false>(a, mod, causal, mask, st);
}

#endif  // !__HIPCC_RTC__

}  // namespace fa
