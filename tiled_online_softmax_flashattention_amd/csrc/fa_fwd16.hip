// Forward attention for 16-bit inputs (f16, bf16) with head_dim 64 or 128.
//
// Computes the online-softmax recurrence of the attnax pallas_flash_attention
// page (kernel body: per query block, loop over key blocks; scores, score_mod
// with global positions, mask, then running max / running sum / rescaled
// accumulator, and acc / l at the end), in base 2 (the flaxattention page's
// "log2 trick": scale * log2(e) folded into the score so every exponential is
// a native v_exp_f32).
//
// Work decomposition: one workgroup of 4 waves per 128-query block; each wave
// owns 32 queries.  Key/value tiles of 64 keys go from HBM straight into LDS
// (global_load_lds_dwordx4: no staging registers, no LDS write instructions)
// and are double buffered: while tile n is used, tile n+1 is in flight, so
// one barrier per tile suffices.  Each tile is processed as two 32-key halves
// in sequence, which keeps a wave's registers small enough for three waves
// per SIMD at head_dim 64 (two at 128): the matrix cores of a SIMD are kept
// busy by the other waves while one wave works through its softmax (a wave's
// own vector instructions overlap its MFMAs poorly on this chip).
// With few query blocks per workgroup slot the forward uses 64-query blocks
// instead, two waves per 32 queries, each over one 32-key half of every
// tile, merged through LDS at the end (fwd16_halves_kernel): a causal
// sequence's longest block then takes half as long, so the slots finish
// together, and a device the 128-query blocks would leave half idle gets
// twice the workgroups.
//
// LDS layout: tiles are unpadded (key, dim) rows, because a direct load
// writes 64 consecutive 16-byte chunks; the chunks of each K row are permuted
// (tswz) so the score MFMA's fragment reads are free of bank conflicts, and
// at head_dim 128 so are V's for the transposing reads (ds_read_b64_tr_b16)
// of the P V product.
//
// Per half tile and wave: S'^T = K Q^T + C (MFMA 32x32x16, Q resident in
// registers as the B operand).  The accumulator starts from C = bias / scale,
// so the score_mod costs no per-score instruction: for ALiBi C holds the bias
// of the key's offset inside the half (the half's own offset is a per-lane
// scalar folded into the exponent), for the checkerboard the two parity
// values, and with a key mask C is read from an LDS row that holds 0 or -inf
// per key.  Then one FMA and one v_exp_f32 per score give P = 2^(S' c + b - m).
// The running max is updated lazily and without a per-half maximum: the
// exponentials are taken against the max as it stands, and only when some
// query's sum over the half exceeds 2^15 (or the query has no max yet) does
// the wave recompute the half's scores, update the max and rescale its
// accumulator.  P stays below 2^15 (inside fp16 range; the final division by l
// cancels the scale), and the common path needs no row maximum and no
// cross-lane exchange.
// Causal: key tiles past the block's last query are never visited, tiles are
// visited diagonal first (so the largest ALiBi scores set the maximum early;
// non-causal ALiBi also visits the tiles from the last one down),
// at head_dim 64 waves skip halves entirely past their own queries (at 128
// such halves run masked to P = 0, which needs fewer registers than the
// exit), and the per-score comparison happens only on diagonal and
// ragged-tail halves.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kSumLimit = 32768.0f;   // a half's row sum above this forces a max update

// One 128-query block (qb) of one (batch, head) slice (bh).  With SPLIT the
// block covers only key chunk `split` (a.chunk keys) and writes its
// unnormalised partial (accumulator, running max, sum) to a.partial for the
// exact merge of the decode path; otherwise it writes O and lse.  With BLK
// only the key tiles whose 128 x 128 block is set in a.block_mask are visited
// (the 128-query block is exactly one block row).  With HALVES the block
// has 64 queries and two waves share each 32 of them: wave w takes queries
// 32 (w & 1) .. +31 and key half w >> 1 of every tile, and the pair's
// (max, sum, accumulator) are merged through LDS at the end.
template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool SPLIT, bool BLK, bool HALVES = false>
__device__ __forceinline__ void fwd16_block(const AttnArgs& a, const int bh, const int qb, const int split) {
  constexpr int BM = HALVES ? 64 : 128;   // queries per workgroup
  constexpr int BN = 64;           // keys per tile
  constexpr int QS = D / 16;       // MFMA steps of the q.k product
  constexpr int DT = D / 32;       // 32-row tiles of O^T
  constexpr int TILE = BN * D;     // elements per K or V tile
  constexpr int VSW = D == 64 ? SW_NONE : SW_TR;   // V is read only transposed

  // Separate arrays per buffer: the compiler then sees that a direct load
  // into one buffer cannot alias reads of the other, and does not wait for it.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];
  __shared__ __attribute__((aligned(16))) float sB0[MASK ? 2 * BN + 4 : 4];  // per-key additive row (q parity 0 / 1)
  __shared__ __attribute__((aligned(16))) float sB1[MASK ? 2 * BN + 4 : 4];
  __shared__ uint16_t sList[BLK ? kBlkMaxSeq / BN : 1];   // visited key tiles (block-sparse)
  __shared__ int sCnt[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM;
  const int qw = q0 + (HALVES ? wave & 1 : wave) * 32;
  const int qi = qw + l32;
  // positions among the keys (query row 0 sits at key position q_off)
  const int qwp = qw + a.q_off, qpos = qi + a.q_off;
  const float c = a.scale_log2;
  const float inv_scale = 1.0f / a.scale;

  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * Sq * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * Skv * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * Skv * D;

  // Q as the B operand: lane (query l32, group hi) holds dims 16kk + 8hi .. +7.
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

  // Accumulator initial value, in units of q.k (bias / scale), per register.
  float slope2 = 0.f;
  f32x16 cinit = zero16();
  if constexpr (MOD == MOD_ALIBI) {
    const float slope = alibi_slope(a.alibi_slopes, h, a.H);
    slope2 = slope * kLog2e;
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = slope * inv_scale * (float)acc_row(r, hi);
  }
  if constexpr (MOD == MOD_CHECKERBOARD && !MASK) {
    // register r holds a key of parity (r & 1); (qpos + kv) is even when the parities agree
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = (((qpos + r) & 1) == 0 ? a.even_nat : a.odd_nat) * inv_scale;
  }

  // causal: keys up to the block's last query position
  const int kv_end = CAUSAL ? min(Skv, min(q0 + BM, Sq) + a.q_off) : Skv;
  const int ntiles_all = (kv_end + BN - 1) / BN;
  int t_lo = 0, t_hi = ntiles_all;   // tiles this workgroup visits
  if constexpr (SPLIT) {
    const int ct = a.chunk / BN;
    t_lo = min(split * ct, ntiles_all);
    t_hi = min(t_lo + ct, ntiles_all);
    // a chunk past the block's last key (causal): no row of the block reads
    // its partial, so none is written
    if (t_lo >= ntiles_all) return;
  }
  int ntiles = t_hi - t_lo;
  if constexpr (BLK) {
    const uint8_t* brow = a.block_mask + ((size_t)bh * a.bm_rows + (q0 >> 7)) * a.bm_cols;
    ntiles = compact_tiles(brow, 1, 1, t_lo, t_hi, sList, sCnt);   // 64-key tile t lies in block t / 2
  }
  // Causal: the diagonal tile first, then towards key 0.  ALiBi grows with the
  // key index, so its largest scores also come first when the tiles are
  // visited from the last one down, and the running max rarely moves.
  constexpr bool REV = CAUSAL || MOD == MOD_ALIBI;
  auto kv_of = [&](int n) __attribute__((always_inline)) {
    if constexpr (BLK) return list_at(sList, REV ? ntiles - 1 - n : n) * BN;
    else return (REV ? t_hi - 1 - n : t_lo + n) * BN;
  };

  // Direct loads of tile kv0 into (sK, sV).  Rows past seq_kv are clamped to
  // the last row (finite values whose scores are masked to -inf).  The split
  // workgroups of a short query block (the only query block) are the only
  // readers of their key chunks, so those loads carry the non-temporal hint;
  // the query blocks of a longer split sequence share each chunk through L2.
  const bool nt = SPLIT && a.n_qblocks == 1;
  auto load_tile = [&](int kv0, uint16_t* sK, uint16_t* sV) __attribute__((always_inline)) {
    if (nt) {
      if (kv0 + BN <= Skv) {
        load_full_tile_lds<D, BN, SW_BOTH, 4, kCpolNT>(Kg + (size_t)kv0 * D, sK, wave, lane);
        load_full_tile_lds<D, BN, VSW, 4, kCpolNT>(Vg + (size_t)kv0 * D, sV, wave, lane);
      } else {
        load_tile_lds<D, BN, SW_BOTH, 4, kCpolNT>(Kg, kv0, Skv, sK, wave, lane);
        load_tile_lds<D, BN, VSW, 4, kCpolNT>(Vg, kv0, Skv, sV, wave, lane);
      }
    } else if (kv0 + BN <= Skv) {
      load_full_tile_lds<D, BN, SW_BOTH, 4, kCpolNone>(Kg + (size_t)kv0 * D, sK, wave, lane);
      load_full_tile_lds<D, BN, VSW, 4, kCpolNone>(Vg + (size_t)kv0 * D, sV, wave, lane);
    } else {
      load_tile_lds<D, BN, SW_BOTH, 4, kCpolNone>(Kg, kv0, Skv, sK, wave, lane);
      load_tile_lds<D, BN, VSW, 4, kCpolNone>(Vg, kv0, Skv, sV, wave, lane);
    }
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
        float e0 = 0.f, e1 = 0.f;   // additive bias for queries of parity 0 / 1
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

  float m_run = kNegInf, l_run = 0.f;
  float neg_m = 0.f;         // -m_run (read only once have_max holds)
  bool have_max = false;     // every lane of the wave has a finite m_run
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero16();

  // S'^T = K Q^T + C for keys 32t .. 32t+31 (first key k0) of the tile in
  // (sK, sB), with scores past the diagonal or past seq_kv set to -inf (the
  // comparison runs only on such halves).
  auto scores = [&](int t, int k0, const uint16_t* sK, const float* sB) __attribute__((always_inline)) {
    f32x16 s = cinit;
    if constexpr (MASK) {
      // the row starts the accumulator (plus the ALiBi offsets, the only
      // nonzero cinit with a mask: the checkerboard values are in the row)
      const float* row = sB + ((qpos & 1) ? parity_row_off<BN>() : 0) + 32 * t + 4 * hi;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 m4 = *(const f32x4*)(row + 8 * u);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) s[4 * u + cc] = MOD == MOD_ALIBI ? cinit[4 * u + cc] + m4[cc] : m4[cc];
      }
    }
    if constexpr (D == 128) {
      // software-pipelined by hand: 4 fragments up front, then each MFMA
      // followed by the read 4 steps ahead (scheduling barriers keep the
      // order)
      constexpr int AHEAD = 4;
      const int kr = 32 * t + l32;
      u32x4 kfr[QS];
#pragma unroll
      for (int kk = 0; kk < AHEAD; ++kk) kfr[kk] = lds_read16(sK + tile_off<D, SW_BOTH>(kr, 16 * kk + 8 * hi));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < QS; ++kk) {
        s = mma16<T>(kfr[kk], qf[kk], s);
        if (kk + AHEAD < QS) kfr[kk + AHEAD] = lds_read16(sK + tile_off<D, SW_BOTH>(kr, 16 * (kk + AHEAD) + 8 * hi));
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // every K fragment is requested (into its own registers) before the
      // first MFMA, so the LDS latency is paid once per half, not per MFMA
      const int kr = 32 * t + l32;
      u32x4 kfr[QS];
#pragma unroll
      for (int kk = 0; kk < QS; ++kk) kfr[kk] = lds_read16(sK + tile_off<D, SW_BOTH>(kr, 16 * kk + 8 * hi));
#pragma unroll
      for (int kk = 0; kk < QS; ++kk) s = mma16<T>(kfr[kk], qf[kk], s);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, QS, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, QS, 0);
    }
    // the diagonal and ragged-tail conditions are uniform over the wave
    const bool diag = CAUSAL && k0 + 31 > qwp;
    const bool tail = !MASK && k0 + 32 > Skv;
    if (diag || tail) {
      int lim = diag ? qpos - k0 : (1 << 30);   // last allowed key position inside the half
      if (tail) lim = min(lim, Skv - 1 - k0);
      const int lim_l = lim - 4 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = 8 * (r >> 2) + (r & 3);   // acc_row(r, hi) - 4 hi
        if (pos > lim_l) s[r] = kNegInf;
      }
    }
    return s;
  };

  // Keys 32t .. 32t+31 of tile n, held in (sK, sV, sB).
  auto half = [&](int n, int t, const uint16_t* sK, const uint16_t* sV, const float* sB) __attribute__((always_inline)) {
    const int k0 = kv_of(n) + 32 * t;   // first key of the half
    // every key follows every query of this wave: nothing to add (at head_dim
    // 128 the half still runs, masked to P = 0: the early exit costs the
    // causal instances more registers than they have)
    if (CAUSAL && D == 64 && k0 > qwp + 31) return;

    f32x16 s = scores(t, k0, sK, sB);
    // per-lane exponent offset (ALiBi: bias of the half's first key)
    float add = 0.f;
    if constexpr (MOD == MOD_ALIBI) add = slope2 * (float)(k0 - qpos);

    // P rounded to the 16-bit type and packed in pairs (the B operand of the
    // P V product), packed right after the exponentials so that the fp32
    // values are dead before the V fragments are read, and its fp32 row sum
    // over the half.  (Summing the packed fp16 pairs with v_dot2 measured
    // slower, and bf16's 2^-9 rounding would be too coarse for lse.)
    u32x4 pb[2];
    auto pack_sum = [&]() __attribute__((always_inline)) {
      float l4[4];
#pragma unroll
      for (int r = 0; r < 16; ++r) l4[r & 3] = r < 4 ? s[r] : l4[r & 3] + s[r];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        pb[u] = u32x4{pack2<T>(s[8 * u + 0], s[8 * u + 1]), pack2<T>(s[8 * u + 2], s[8 * u + 3]),
                      pack2<T>(s[8 * u + 4], s[8 * u + 5]), pack2<T>(s[8 * u + 6], s[8 * u + 7])};
      return (l4[0] + l4[1]) + (l4[2] + l4[3]);
    };

    // Fast path: exponentials against the running max as it stands, valid
    // when every lane has one (have_max, uniform) and no lane's sum over the
    // half exceeds 2^15 (so every P fits fp16).  Otherwise (a row's first
    // visible keys, or a max that grew) the scores are recomputed from LDS,
    // the max updated and the accumulator rescaled.
    float ls = 0.f;
    bool ok = have_max;
    if (ok) {
      const float nb = MOD == MOD_ALIBI ? add - m_run : neg_m;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = exp2_hw(fmaf(s[r], c, nb));
      ls = pack_sum();
      ok = __builtin_amdgcn_ballot_w64(!(ls <= kSumLimit)) == 0;
    }
    if (!ok) {
      s = scores(t, k0, sK, sB);
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaf(mx, c, add);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_hw(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m_run = m_new;
      neg_m = -m_run;
      have_max = __builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0;
      const float nb = add - m_use;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = exp2_hw(fmaf(s[r], c, nb));
      ls = pack_sum();
    }
    l_run += ls;

    // O^T += V^T P^T over the two 16-key steps of the half (all V fragments
    // requested before the first MFMA)
    u32x4 vfr[2][DT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vfr[u][dt] = read_a_tr_tile<D, VSW>(sV, 32 * t + 16 * u, 32 * dt, lane);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = mma16<T>(vfr[u][dt], pb[u], o[dt]);
    }
  };

  // Prologue: tile 0 (and its mask row) requested.
  if (ntiles > 0) {
    load_tile(kv_of(0), sK0, sV0);
    load_m(kv_of(0));
    store_m(sB0);
    load_m(kv_of(min(1, ntiles - 1)));
  }

  // Tile n in buffers (n & 1); tile n+1 is requested into the other buffers
  // right after the barrier that retires tile n-1.
  auto tile = [&](int n, const uint16_t* sK, const uint16_t* sV, const float* sB,
                  uint16_t* sKn, uint16_t* sVn, float* sBn) __attribute__((always_inline)) {
    wait_direct_loads();                   // this wave's loads of tile n are in LDS
    sync_wg();                       // ... and every other wave's; tile n-1 is retired
    if (n + 1 < ntiles) {
      load_tile(kv_of(n + 1), sKn, sVn);
      store_m(sBn);
      load_m(kv_of(min(n + 2, ntiles - 1)));
    }
    if (qw < Sq) {   // a wave past the last query only loads its share of the tiles
      if constexpr (HALVES) {
        half(n, wave >> 1, sK, sV, sB);
      } else {
        half(n, 0, sK, sV, sB);
        __builtin_amdgcn_sched_barrier(0);   // keep the halves apart: their registers are shared
        half(n, 1, sK, sV, sB);
      }
    }
  };

  int n = 0;
  for (; n + 1 < ntiles; n += 2) {
    tile(n, sK0, sV0, sB0, sK1, sV1, sB1);
    tile(n + 1, sK1, sV1, sB1, sK0, sV0, sB0);
  }
  if (n < ntiles) tile(n, sK0, sV0, sB0, sK1, sV1, sB1);

  if constexpr (HALVES) {
    // The wave of key half 1 hands its (max, sum, accumulator) to the wave of
    // half 0 through the tile buffers (free once every wave is past its last
    // tile); that wave rescales both to the larger max and adds them.
    static_assert(TILE * sizeof(uint16_t) >= 16 * DT * 64 * sizeof(float), "merge buffer");
    sync_wg();
    float* xo = (float*)((wave & 1) ? sK1 : sK0);
    float* xm = (float*)sV0 + 128 * (wave & 1);
    if (wave >> 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(16 * dt + r) * 64 + lane] = o[dt][r];
      xm[lane] = m_run;
      xm[64 + lane] = l_run;
    }
    sync_wg();
    if (wave >> 1) return;
    const float mb = xm[lane], lb = xm[64 + lane];
    const float m_new = fmaxf(m_run, mb);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float wa = exp2_hw(m_run - m_use), wb = exp2_hw(mb - m_use);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * wa + xo[(16 * dt + r) * 64 + lane] * wb;
    l_run = l_run * wa + lb * wb;
    m_run = m_new;
  }

  const float l_tot = l_run + xor32(l_run);
  if constexpr (SPLIT) {
    if (qi < Sq) {
      float* P = a.partial + (((size_t)bh * Sq + qi) * a.n_split + split) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) P[32 * dt + 8 * (r >> 2) + 4 * hi + (r & 3)] = o[dt][r];   // rows are only 8-byte aligned
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

// Workgroup order: block_coord (each head's blocks on one XCD, non-causal
// heads one after the other per XCD).  Causal query blocks are dispatched
// longest first.
template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void fwd16_kernel(const AttnArgs a) {
  const BlockCoord c = block_coord(blockIdx.x, a.B * a.H, a.n_qblocks, CAUSAL);
  fwd16_block<T, D, MOD, CAUSAL, MASK, false, BLK>(a, c.bh, CAUSAL ? a.n_qblocks - 1 - c.blk : c.blk, 0);
}

// Split over the key axis (short query blocks against a long key sequence,
// and sequences whose query blocks alone leave the device idle): workgroup
// (bh, query block, key chunk) in the order of split_coord (longest blocks
// first, chunks rotated over the XCDs).
template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void fwd16_split_kernel(const AttnArgs a) {
  const SplitCoord c = split_coord(blockIdx.x, a.B * a.H, a.n_qblocks, a.n_split, CAUSAL);
  fwd16_block<T, D, MOD, CAUSAL, MASK, true, BLK>(a, c.bh, c.qb, c.split);
}

// Few query blocks per workgroup slot: 64-query blocks, two waves per 32
// queries (one key half each).  Causal: longest first; the longest block
// then takes half the time while the total stays the same, so the slots
// finish closer together.  Not causal: twice the workgroups on a device the
// 128-query blocks leave half idle.  a.n_qblocks counts 64-query blocks.
template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void fwd16_halves_kernel(const AttnArgs a) {
  const BlockCoord c = block_coord(blockIdx.x, a.B * a.H, a.n_qblocks, CAUSAL);
  fwd16_block<T, D, MOD, CAUSAL, MASK, false, BLK, true>(a, c.bh, CAUSAL ? a.n_qblocks - 1 - c.blk : c.blk, 0);
}

template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
static void launch_fwd16_inst(const AttnArgs& a, bool split, hipStream_t st, bool halves) {
  if (halves && !split) {
    AttnArgs h = a;
    h.n_qblocks = (a.Sq + 63) / 64;
    hipLaunchKernelGGL((fwd16_halves_kernel<T, D, MOD, CAUSAL, MASK, BLK>), dim3((unsigned)(h.n_qblocks * a.B * a.H)),
                       dim3(256), 0, st, h);
    return;
  }
  const unsigned blocks = (unsigned)(a.n_qblocks * a.B * a.H);
  if (split)
    hipLaunchKernelGGL((fwd16_split_kernel<T, D, MOD, CAUSAL, MASK, BLK>), dim3(blocks * (unsigned)a.n_split),
                       dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((fwd16_kernel<T, D, MOD, CAUSAL, MASK, BLK>), dim3(blocks), dim3(256), 0, st, a);
}

template <class T, int D, int MOD, bool CAUSAL, bool MASK>
static void launch_fwd16_blk(const AttnArgs& a, bool split, hipStream_t st, bool halves) {
  if (a.block_mask) launch_fwd16_inst<T, D, MOD, CAUSAL, MASK, true>(a, split, st, halves);
  else launch_fwd16_inst<T, D, MOD, CAUSAL, MASK, false>(a, split, st, halves);
}

template <class T, int D, int MOD>
static hipError_t launch_fwd16_mod(const AttnArgs& a, bool causal, bool mask, bool split, hipStream_t st,
                                   bool halves) {
  if (causal) {
    if (mask) launch_fwd16_blk<T, D, MOD, true, true>(a, split, st, halves);
    else launch_fwd16_blk<T, D, MOD, true, false>(a, split, st, halves);
  } else {
    if (mask) launch_fwd16_blk<T, D, MOD, false, true>(a, split, st, halves);
    else launch_fwd16_blk<T, D, MOD, false, false>(a, split, st, halves);
  }
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fwd16_d(const AttnArgs& a, int mod, bool causal, bool mask, bool split, hipStream_t st,
                                 bool halves) {
  switch (mod) {
    case MOD_ALIBI: return launch_fwd16_mod<T, D, MOD_ALIBI>(a, causal, mask, split, st, halves);
    case MOD_CHECKERBOARD: return launch_fwd16_mod<T, D, MOD_CHECKERBOARD>(a, causal, mask, split, st, halves);
    default: return launch_fwd16_mod<T, D, MOD_NONE>(a, causal, mask, split, st, halves);
  }
}

int fwd16_block_q(int) { return 128; }

hipError_t launch_fwd16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask, hipStream_t st,
                        bool split, bool halves) {
  if (bf16) {
    return D == 64 ? launch_fwd16_d<BF16, 64>(a, mod, causal, mask, split, st, halves)
                   : launch_fwd16_d<BF16, 128>(a, mod, causal, mask, split, st, halves);
  }
  return D == 64 ? launch_fwd16_d<F16, 64>(a, mod, causal, mask, split, st, halves)
                 : launch_fwd16_d<F16, 128>(a, mod, causal, mask, split, st, halves);
}

}  // namespace fa
