// Backward attention for 16-bit inputs (f16, bf16), head_dim 64 or 128.
//
// Gradients of sum(dO * O) by calculus on the attention definition:
//   P = exp(S - lse) recomputed from the forward's saved log-sum-exp,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta) with delta_i = <dO_i, O_i>,
//   dK = scale * dS^T Q,  dQ = scale * dS K.
// The pages obtain their gradient by tracing the kernel (attnax
// pallas_flash_attention docstring) and time it (flaxattention benchmark
// table); this is the hand-written counterpart.
//
// Two modes for dQ.  Separate (deterministic, no atomics): two passes,
//  * dkdv16_kernel: key-stationary.  Each wave keeps 32 keys' K and V rows in
//    registers and their dK^T, dV^T accumulators, and loops over 64-query
//    tiles whose Q and dO go straight from HBM into LDS.  S and dP are formed
//    with queries as rows, so the lane holds one key and the probabilities
//    feed dV^T = dO^T P and dK^T = Q^T dS directly as MFMA B operands; the
//    dO^T and Q^T fragments come from the tiles through the transposing LDS
//    read.
//  * dq16_kernel (fa_dq16.hip): query-stationary, like the forward.  Each
//    wave keeps 32 queries' Q and dO rows in registers; K and V tiles go
//    straight into LDS; S^T and dP^T are formed with keys as rows so the
//    lane holds one query, and dQ^T = K^T dS^T accumulates in registers (K^T
//    fragments through the transposing LDS read).
// Atomic: the preprocess kernel writes the row statistics and zeroes an fp32
// dQ accumulator; the key/value pass (DQA) also stores each query tile's dS^T
// in LDS and adds dS K over its 128 keys into the accumulator with fp32
// atomics; a convert kernel scales and rounds it to dQ.  This removes the
// query pass's recomputation of S and dP (4 D of its 6 D flop per pair); the
// order of the atomic additions varies, so dQ is not bitwise repeatable.
// The LDS tiles are unpadded rows with permuted 16-byte chunks (tswz), which
// keeps both the row-fragment and the transposing reads free of bank
// conflicts.  With few blocks per workgroup slot both passes run on 64-row
// blocks instead, two waves per 32 rows, each over one half of every tile,
// their sums added through LDS at the end (HALVES instances).
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// ---------------------------------------------------------------- preprocess

// delta_i = sum_d dO_id * O_id; lse2_i = lse_i * log2(e), +inf for an empty
// row (so that exp2(s - lse2) = 0 there).  For the 16-bit key/value pass
// (kv16) the rows are stored as that pass consumes them: -delta_i, and
// -lse2_i / c in units of q.k (c = scale * log2(e) > 0), with lse2_i carrying
// the query's share of the ALiBi bias relative to its 64-query tile,
// slope * log2(e) * (i mod 64).  Both then serve as the initial values of
// the dP and S accumulators.
template <int ES, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const AttnArgs a, int dtype, int kv16) {
  constexpr int EPL = 16 / ES;                        // elements per 16-byte load
  constexpr int LPR = (D * ES / 16) < 64 ? (D * ES / 16) : 64;  // lanes per row
  constexpr int IT = D * ES / 16 / LPR;               // loads per lane
  constexpr int RPB = 256 / LPR;                      // rows per block
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const int64_t rows = (int64_t)a.B * a.H * a.Sq;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  float acc = 0.f;
  if (row < rows) {
    const char* O = (const char*)a.o + row * D * ES;
    const char* dO = (const char*)a.dout + row * D * ES;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int off = (it * LPR + sub) * 16;
      const u32x4 x = *(const u32x4*)(O + off);
      const u32x4 y = *(const u32x4*)(dO + off);
      if constexpr (ES == 4) {
        // bit-cast whole vectors: a bit_cast of a single vector element is
        // miscompiled (every element reads as element 0)
        const f32x4 xf = __builtin_bit_cast(f32x4, x), yf = __builtin_bit_cast(f32x4, y);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc += xf[c] * yf[c];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint16_t x0 = x[c] & 0xffffu, x1 = x[c] >> 16, y0 = y[c] & 0xffffu, y1 = y[c] >> 16;
          if (dtype == 2) acc += to_f32<BF16>(x0) * to_f32<BF16>(y0) + to_f32<BF16>(x1) * to_f32<BF16>(y1);
          else acc += to_f32<F16>(x0) * to_f32<F16>(y0) + to_f32<F16>(x1) * to_f32<F16>(y1);
        }
      }
    }
  }
#pragma unroll
  for (int w = 1; w < LPR; w <<= 1) acc += __shfl_xor(acc, w);
  if (a.dq_acc && row < rows) {   // atomic dQ mode: the key/value pass adds into these rows
    float* z = a.dq_acc + row * D;
#pragma unroll
    for (int c = sub; c < D / 4; c += LPR) *(f32x4*)(z + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (row < rows && sub == 0) {
    const float l = a.lse[row];
    float l2 = (l == kNegInf) ? __builtin_inff() : l * kLog2e;
    if (kv16) {
      if (kv16 == 2) {   // ALiBi
        const int64_t bhr = row / a.Sq;
        const int qrow = (int)(row - bhr * a.Sq);
        l2 += alibi_slope(a.alibi_slopes, (int)(bhr % a.H), a.H) * kLog2e * (float)(qrow & (kDkdvBQ - 1));
      }
      a.delta[row] = -acc;
      a.lse2[row] = -l2 / a.scale_log2;
    } else {
      a.delta[row] = acc;
      a.lse2[row] = l2;
    }
  }
  (void)EPL;
}

hipError_t launch_bwd_pre(const AttnArgs& a, int dtype, int D, hipStream_t st, int kv16) {
  const int64_t rows = (int64_t)a.B * a.H * a.Sq;
  const int es = dtype == 0 ? 4 : 2;
  const int lpr = (D * es / 16) < 64 ? (D * es / 16) : 64;
  const int rpb = 256 / lpr;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(256);
  if (es == 4) {
    if (D == 64) hipLaunchKernelGGL((bwd_pre_kernel<4, 64>), grid, block, 0, st, a, dtype, kv16);
    else if (D == 128) hipLaunchKernelGGL((bwd_pre_kernel<4, 128>), grid, block, 0, st, a, dtype, kv16);
    else hipLaunchKernelGGL((bwd_pre_kernel<4, 512>), grid, block, 0, st, a, dtype, kv16);
  } else {
    if (D == 64) hipLaunchKernelGGL((bwd_pre_kernel<2, 64>), grid, block, 0, st, a, dtype, kv16);
    else hipLaunchKernelGGL((bwd_pre_kernel<2, 128>), grid, block, 0, st, a, dtype, kv16);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- dK / dV pass

// Key-stationary dK/dV pass.  The S accumulator starts from the query row's
// -lse2 / c and the dP accumulator from -delta (rows stored that way by the
// query pass or the preprocess), so the MFMAs produce S - lse2 / c and
// dP - delta directly.  The ALiBi bias slope (k - q) splits into the query's
// part relative to its tile start, which arrives folded into the lse2 row,
// and a per-lane term slope (k - tile start) that joins the key mask (-inf)
// and the checkerboard bias (two per-lane values by register parity) in one
// exponent offset.  Per score the work is one FMA and one exp for P and one
// multiply for dS.  Query tiles (Q, dO and their
// lse2 and delta rows) go from HBM straight into double-buffered LDS; both
// 16-bit tiles are read as row fragments (S, dP) and transposed (dV, dK), so
// their chunks carry the permutation that serves both reads.  Each 64-query
// tile is processed as two 32-query halves, which keeps the live registers
// (K, V, dK, dV and two score blocks) within the 256 of two waves per SIMD
// at head_dim 64.  With BLK only the query tiles whose 128 x 128 block (row
// tile / 2, this workgroup's 128 keys) is set in the block mask are visited.
// With HALVES (not with DQA) the block has 64 keys and two waves share each
// 32 of them: wave w takes keys 32 (w & 1) .. +31 and query half w >> 1 of
// every tile, and the pair's dK, dV sums are added through LDS at the end.
template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool BLK, bool DQA, bool HALVES = false>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void dkdv16_kernel(const AttnArgs a) {
  static_assert(!(HALVES && DQA), "the atomic dQ mode keeps 128-key blocks");
  constexpr int BKV = HALVES ? 64 : 128;   // keys per workgroup (4 waves x 32, or 2 x 32 twice)
  constexpr int BQ = kDkdvBQ;   // queries per tile
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int TILE = BQ * D;
  // atomic dQ mode: the workgroup's K rows and each query tile's dS^T (128
  // keys x 64 queries, 16-bit) in LDS, read transposed by the dQ products
  __shared__ __attribute__((aligned(16))) uint16_t sKd[DQA ? BKV * D : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sDS[DQA ? BKV * BQ : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sO0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sO1[TILE];
  __shared__ __attribute__((aligned(16))) float sL0[BQ];
  __shared__ __attribute__((aligned(16))) float sL1[BQ];
  __shared__ __attribute__((aligned(16))) float sD0[BQ];
  __shared__ __attribute__((aligned(16))) float sD1[BQ];
  __shared__ uint16_t sList[BLK ? kBlkMaxSeq / BQ : 1];   // visited query tiles (block-sparse)
  __shared__ int sCnt[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  // low kb = most query tiles under causal: dispatched first
  const BlockCoord bc = block_coord(blockIdx.x, BH, (a.Skv + BKV - 1) / BKV, CAUSAL);
  const int bh = bc.bh, kb = bc.blk;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int k0 = kb * BKV;
  const int kw = k0 + 32 * (HALVES ? wave & 1 : wave);
  const int kj = kw + l32;            // this lane's key
  const float c = a.scale_log2;

  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * Sq * D;
  const uint16_t* dOg = (const uint16_t*)a.dout + (size_t)bh * Sq * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * Skv * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * Skv * D;
  const float* lse2g = a.lse2 + (size_t)bh * Sq;
  const float* deltag = a.delta + (size_t)bh * Sq;

  // K and V rows of this lane's key as B operands (dims 16kk + 8hi .. +7).
  u32x4 kf[KS], vf[KS];
  {
    const size_t off = (size_t)min(kj, Skv - 1) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      kf[kk] = *(const u32x4*)(Kg + off + 16 * kk);
      vf[kk] = *(const u32x4*)(Vg + off + 16 * kk);
    }
  }
  if constexpr (D == 128 && !DQA) {   // one wave per SIMD: K and V fragments in AGPRs
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      keep_in_agprs(kf[kk]);
      keep_in_agprs(vf[kk]);
    }
  }
  if constexpr (DQA) {   // K rows of the workgroup for the dQ products (visible after the first barrier)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) lds_write16(sKd + tile_off<D, SW_TR>(32 * wave + l32, 16 * kk + 8 * hi), kf[kk]);
  }
  // per-lane exponent term: the key's share of the bias, or -inf for a
  // masked key or a key past seq_kv (its dK, dV rows are not stored)
  bool key_ok = kj < Skv;
  if constexpr (MASK) key_ok = key_ok && a.key_mask[(size_t)b * Skv + min(kj, Skv - 1)] != 0;
  float slope2 = 0.f;
  if constexpr (MOD == MOD_ALIBI) slope2 = alibi_slope(a.alibi_slopes, h, a.H) * kLog2e;
  // checkerboard bias (log2 units) of registers r even / odd: query tiles
  // start at even rows, so register r holds a query at a position of parity
  // ((r + q_off) & 1)
  float cb0 = 0.f, cb1 = 0.f;
  if constexpr (MOD == MOD_CHECKERBOARD) {
    const bool kev = ((kj + a.q_off) & 1) == 0;
    cb0 = kev ? a.even_log2 : a.odd_log2;
    cb1 = kev ? a.odd_log2 : a.even_log2;
  }

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  const int off = a.q_off;            // query row q sits at key position q + off
  const int qt0 = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int nqt = (Sq + BQ - 1) / BQ;
  // Visit n = n0 .. n_end-1 is query tile it_of(n): the tile itself, or
  // entry n of the list of tiles whose block is set.
  int n0 = qt0, n_end = nqt;
  if constexpr (BLK) {
    const uint8_t* bcol = a.block_mask + (size_t)bh * a.bm_rows * a.bm_cols + (k0 >> 7);   // one block column
    n0 = 0;
    n_end = compact_tiles(bcol, a.bm_cols, 1, qt0, nqt, sList, sCnt);   // 64-query tile t lies in block row t / 2
  }
  auto it_of = [&](int n) __attribute__((always_inline)) {
    if constexpr (BLK) return list_at(sList, n);
    else return n;
  };

  // Direct loads of query tile it.  Rows past seq_q are clamped to the last
  // row; their scores are masked below.
  auto load_tile = [&](int it, uint16_t* sQ, uint16_t* sO, float* sL, float* sD) __attribute__((always_inline)) {
    const int q0 = it * BQ;
    load_tile_lds<D, BQ, SW_BOTH>(Qg, q0, Sq, sQ, wave, lane);
    load_tile_lds<D, BQ, SW_BOTH>(dOg, q0, Sq, sO, wave, lane);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((const void*)(lse2g + min(q0 + lane, Sq - 1)), (lds_void_ptr)sL, 4, 0, 0);
    if (wave == 1)
      __builtin_amdgcn_global_load_lds((const void*)(deltag + min(q0 + lane, Sq - 1)), (lds_void_ptr)sD, 4, 0, 0);
  };

  // dS^T of queries 32mt + 16u .. +15 held by this lane (its key, 8 queries
  // in accumulator order) into the LDS tile of the dQ products: row = key,
  // position p = 32mt + 16u + 8hi + j for register 8u + j, i.e. query
  // swap23(p) of the tile (bits 2 and 3 of the position exchanged).
  auto put_ds = [&](int mt, int u, u32x4 db) __attribute__((always_inline)) {
    if constexpr (DQA) lds_write16(sDS + tile_off<64, SW_BOTH>(32 * wave + l32, 32 * mt + 16 * u + 8 * hi), db);
  };

  // Queries 32mt .. 32mt+31 of tile it, in two steps: the score products,
  // then the probabilities, dS and the dV, dK products.
  // every query precedes every key of this wave: nothing to add (in the
  // atomic dQ mode the half still runs, masked to P = 0, so its dS^T rows
  // of the LDS tile are zeros; such halves occur only in a key block's
  // first query tile)
  // (at head_dim 128 every half runs: the paired schedule below has no room
  // for a per-wave exit, whose registers spilled; the skipped halves are a
  // few per key block)
  auto half_runs = [&](int it, int mt) __attribute__((always_inline)) {
    return DQA || !CAUSAL || D == 128 || it * BQ + 32 * mt + off + 31 >= kw;
  };
  // S' = Q K^T - lse2 / c and dP' = dO V^T - delta, queries as rows: the
  // accumulators start from the rows' stored values
  auto scores = [&](int mt, const uint16_t* sQ, const uint16_t* sO, const float* sL, const float* sD, f32x16& sv,
                    f32x16& dpv) __attribute__((always_inline)) {
    const float* lrow = sL + 32 * mt + 4 * hi;
    const float* drow = sD + 32 * mt + 4 * hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 l4 = *(const f32x4*)(lrow + 8 * u);
      const f32x4 d4 = *(const f32x4*)(drow + 8 * u);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        sv[4 * u + cc] = l4[cc];
        dpv[4 * u + cc] = d4[cc];
      }
    }
    const int qr = 32 * mt + l32;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int off = tile_off<D, SW_BOTH>(qr, 16 * kk + 8 * hi);
      sv = mma16<T>(lds_read16(sQ + off), kf[kk], sv);
      dpv = mma16<T>(lds_read16(sO + off), vf[kk], dpv);
    }
  };
  // The same products with the fragment reads software-pipelined by hand:
  // the rows and the first AHEAD fragment pairs are requested up front, then
  // each step's two MFMAs are followed by the reads of the pair AHEAD steps
  // later (scheduling barriers keep the order, so AHEAD pairs stay in
  // flight in registers of their own).
  auto scores_pipelined = [&](int mt, const uint16_t* sQ, const uint16_t* sO, const float* sL, const float* sD,
                              f32x16& sv, f32x16& dpv) __attribute__((always_inline)) {
    constexpr int AHEAD = 4;
    const float* lrow = sL + 32 * mt + 4 * hi;
    const float* drow = sD + 32 * mt + 4 * hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 l4 = *(const f32x4*)(lrow + 8 * u);
      const f32x4 d4 = *(const f32x4*)(drow + 8 * u);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        sv[4 * u + cc] = l4[cc];
        dpv[4 * u + cc] = d4[cc];
      }
    }
    const int qr = 32 * mt + l32;
    u32x4 fq[KS], fo[KS];
#pragma unroll
    for (int kk = 0; kk < AHEAD; ++kk) {
      const int o = tile_off<D, SW_BOTH>(qr, 16 * kk + 8 * hi);
      fq[kk] = lds_read16(sQ + o);
      fo[kk] = lds_read16(sO + o);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      sv = mma16<T>(fq[kk], kf[kk], sv);
      dpv = mma16<T>(fo[kk], vf[kk], dpv);
      if (kk + AHEAD < KS) {
        const int o = tile_off<D, SW_BOTH>(qr, 16 * (kk + AHEAD) + 8 * hi);
        fq[kk + AHEAD] = lds_read16(sQ + o);
        fo[kk + AHEAD] = lds_read16(sO + o);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P = 0 for queries before the key (causal), only on such halves.  Rows
  // past seq_q need nothing here: their lse2 row entries are -inf (below).
  auto mask_scores = [&](int it, int mt, f32x16& sv) __attribute__((always_inline)) {
    if constexpr (CAUSAL) {
      const int qs = it * BQ + 32 * mt;   // first query of the half
      if (__builtin_amdgcn_ballot_w64(qs + off < kj) != 0) {
        const int ql = qs + 4 * hi;   // query of register r: ql + 8 (r / 4) + r % 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = ql + 8 * (r >> 2) + (r & 3);
          if (q + off < kj) sv[r] = kNegInf;
        }
      }
    }
  };
  // P and dS = P (dP - delta), rounded and packed as MFMA B operands
  auto probs = [&](int it, f32x16& sv, f32x16& dpv, u32x4* pb, u32x4* db) __attribute__((always_inline)) {
    float lb = key_ok ? 0.f : kNegInf;
    if constexpr (MOD == MOD_ALIBI) lb = key_ok ? slope2 * (float)(kj - it * BQ - off) : kNegInf;
    const float lb0 = lb + cb0, lb1 = lb + cb1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_hw(fmaf(sv[r], c, (r & 1) ? lb1 : lb0));
      sv[r] = p;
      dpv[r] *= p;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb[u] = pack8<T>(sv, u);
      db[u] = pack8<T>(dpv, u);
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries
  auto products = [&](int mt, const u32x4* pb, const u32x4* db, const uint16_t* sQ, const uint16_t* sO)
                      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p0 = 32 * mt + 16 * u;
      put_ds(mt, u, db[u]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dv[dt] = mma16<T>(read_a_tr_tile<D, SW_BOTH>(sO, p0, 32 * dt, lane), pb[u], dv[dt]);
        dk[dt] = mma16<T>(read_a_tr_tile<D, SW_BOTH>(sQ, p0, 32 * dt, lane), db[u], dk[dt]);
      }
    }
  };
  auto finish = [&](int it, int mt, f32x16& sv, f32x16& dpv, const uint16_t* sQ, const uint16_t* sO)
                    __attribute__((always_inline)) {
    mask_scores(it, mt, sv);
    u32x4 pb[2], db[2];
    probs(it, sv, dpv, pb, db);
    products(mt, pb, db, sQ, sO);
  };
  auto half = [&](int it, int mt, const uint16_t* sQ, const uint16_t* sO, const float* sL, const float* sD) __attribute__((always_inline)) {
    if (!half_runs(it, mt)) return;
    f32x16 sv, dpv;
    scores(mt, sQ, sO, sL, sD, sv, dpv);
    finish(it, mt, sv, dpv, sQ, sO);
  };
  // head_dim 128 runs one wave per SIMD, so no other wave fills the matrix
  // cores while a wave works through its exponentials: both halves' score
  // products are issued first, and the first half's probabilities are
  // computed while the second half's products run (and its dV, dK products
  // while the second half's probabilities are computed).
  constexpr bool PAIRED = D == 128 && !DQA && !HALVES;

  // Atomic dQ mode, after every wave has stored its dS^T of query tile it:
  // dQ_tile += dS K over the workgroup's 128 keys, as (64 queries x D) / 4
  // waves of 32 x 32 MFMA tiles (wave w: queries 32 (w >> 1) .., dims
  // 32 ((w & 1) NT + t) ..), both operands through the transposing LDS read,
  // then added into the fp32 accumulator rows with buffer atomics whose
  // descriptor bounds the slice (lanes past seq_q are dropped by the
  // hardware, so every wave issues exactly NA atomics per tile).
  constexpr int NT = DQA ? D / 64 : 1;
  __amdgpu_buffer_rsrc_t dq_rsrc;
  if constexpr (DQA)
    dq_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.dq_acc + (size_t)bh * Sq * D, 0, Sq * D * 4, 0x00020000);
  auto dq_tile = [&](int it) __attribute__((always_inline)) {
    if constexpr (DQA) {
      const int qh = wave >> 1;
      f32x16 cq[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) cq[t] = zero16();
#pragma unroll
      for (int ks = 0; ks < BKV / 16; ++ks) {
        const u32x4 af = read_a_tr_tile<64, SW_BOTH>(sDS, 16 * ks, 32 * qh, lane);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          cq[t] = mma16<T>(af, read_a_tr_tile<D, SW_TR>(sKd, 16 * ks, 32 * ((wave & 1) * NT + t), lane), cq[t]);
      }
      // register r holds position 32qh + 8(r/4) + 4hi + r%4, i.e. query
      // 32qh + 16(r/8) + 8hi + 4((r/4)%2) + r%4 of the tile
      const int qb = it * BQ + 32 * qh + 8 * hi;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int dcol = 32 * ((wave & 1) * NT + t) + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(cq[t][r], dq_rsrc, (q * D + dcol) * 4, 0, 0);
        }
      }
    }
  };

  // Both halves of a tile at head_dim 128, scheduled by hand.  Scheduling
  // barriers fix the order; each MFMA's operands are requested AHEAD steps
  // before it (a wait for LDS reads drains all of them while the tile loads
  // are in flight, so the reads of later steps are issued after the MFMAs
  // whose operands have arrived), and the VALU work of the other half sits
  // between the MFMAs: the second half's score products beside the first
  // half's probabilities, the first half's dV, dK products beside the
  // second half's.  The causal masking runs between the regions (rows past
  // seq_q arrive masked in their lse2 row).
  auto paired = [&](int it, const uint16_t* sQ, const uint16_t* sO, const float* sL, const float* sD)
                       __attribute__((always_inline)) {
    constexpr int AHEAD = 4;
    f32x16 sv0, dp0, sv1, dp1;
    u32x4 pb0[2], db0[2], pb1[2], db1[2];
    scores_pipelined(0, sQ, sO, sL, sD, sv0, dp0);
    mask_scores(it, 0, sv0);
    __builtin_amdgcn_sched_barrier(0);

    float lb = key_ok ? 0.f : kNegInf;
    if constexpr (MOD == MOD_ALIBI) lb = key_ok ? slope2 * (float)(kj - it * BQ - off) : kNegInf;
    const float lb0 = lb + cb0, lb1 = lb + cb1;
    auto prob = [&](f32x16& sv, f32x16& dpv, int r) __attribute__((always_inline)) {
      const float p = exp2_hw(fmaf(sv[r], c, (r & 1) ? lb1 : lb0));
      sv[r] = p;
      dpv[r] *= p;
    };

    // second half's score products, first half's probabilities between them
    {
      const float* lrow = sL + 32 + 4 * hi;
      const float* drow = sD + 32 + 4 * hi;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 l4 = *(const f32x4*)(lrow + 8 * u);
        const f32x4 d4 = *(const f32x4*)(drow + 8 * u);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          sv1[4 * u + cc] = l4[cc];
          dp1[4 * u + cc] = d4[cc];
        }
      }
      const int qr = 32 + l32;
      u32x4 fq[KS], fo[KS];
#pragma unroll
      for (int kk = 0; kk < AHEAD; ++kk) {
        const int o = tile_off<D, SW_BOTH>(qr, 16 * kk + 8 * hi);
        fq[kk] = lds_read16(sQ + o);
        fo[kk] = lds_read16(sO + o);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        sv1 = mma16<T>(fq[kk], kf[kk], sv1);
        dp1 = mma16<T>(fo[kk], vf[kk], dp1);
        if (kk + AHEAD < KS) {
          const int o = tile_off<D, SW_BOTH>(qr, 16 * (kk + AHEAD) + 8 * hi);
          fq[kk + AHEAD] = lds_read16(sQ + o);
          fo[kk + AHEAD] = lds_read16(sO + o);
        }
        prob(sv0, dp0, 2 * kk);
        prob(sv0, dp0, 2 * kk + 1);
        if (kk == 3 || kk == 7) {
          pb0[kk >> 2] = pack8<T>(sv0, kk >> 2);
          db0[kk >> 2] = pack8<T>(dp0, kk >> 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    mask_scores(it, 1, sv1);
    __builtin_amdgcn_sched_barrier(0);

    // dV^T += dO^T P and dK^T += Q^T dS: MFMA i of a half uses the
    // transposed fragment of query step u = i / (2 DT), dims 32 dt (dt =
    // (i / 2) % DT), of dO (i even, for dV) or Q (i odd, for dK)
    constexpr int NP = 4 * DT;
    auto pfrag = [&](int mt, int i) __attribute__((always_inline)) {
      const int u = i / (2 * DT), dt = (i / 2) % DT;
      return read_a_tr_tile<D, SW_BOTH>((i & 1) ? sQ : sO, 32 * mt + 16 * u, 32 * dt, lane);
    };
    auto pmma = [&](int i, u32x4 af, const u32x4* pb, const u32x4* db) __attribute__((always_inline)) {
      const int u = i / (2 * DT), dt = (i / 2) % DT;
      if (i & 1) dk[dt] = mma16<T>(af, db[u], dk[dt]);
      else dv[dt] = mma16<T>(af, pb[u], dv[dt]);
    };
    // first half's products, second half's probabilities between them
    {
      u32x4 af[NP];
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) af[i] = pfrag(0, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        pmma(i, af[i], pb0, db0);
        if (i + AHEAD < NP) af[i + AHEAD] = pfrag(0, i + AHEAD);
        prob(sv1, dp1, i);
        if (i == 7 || i == 15) {
          pb1[i >> 3] = pack8<T>(sv1, i >> 3);
          db1[i >> 3] = pack8<T>(dp1, i >> 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // second half's products
    {
      u32x4 af[NP];
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) af[i] = pfrag(1, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        pmma(i, af[i], pb1, db1);
        if (i + AHEAD < NP) af[i + AHEAD] = pfrag(1, i + AHEAD);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // Visit n in the buffers of its parity; visit n+1 is requested into the
  // other buffers right after the barrier that retires visit n-1.
  auto tile = [&](int n, const uint16_t* sQ, const uint16_t* sO, float* sL, const float* sD, uint16_t* sQn,
                  uint16_t* sOn, float* sLn, float* sDn) __attribute__((always_inline)) {
    const int it = it_of(n);
    // this wave's loads of tile n are in LDS; in the atomic dQ mode the NA
    // atomics of tile n-1, issued after those loads, may still be in flight
    // (vector memory operations complete in issue order)
    if constexpr (DQA) {
      if (n == n0) wait_direct_loads();
      else wait_vmcnt_le<16 * NT>();
    } else {
      wait_direct_loads();
    }
    // Rows past seq_q (clamped copies of the last row) get -inf in place of
    // -lse2 / c, so their P and dS are 0 without a per-score mask; wave 0,
    // which loaded the row, writes it before the barrier publishes it.
    if (wave == 0 && it * BQ + BQ > Sq && it * BQ + lane >= Sq) sL[lane] = kNegInf;
    if constexpr (DQA) barrier_lds();   // ... and every other wave's; tile n-1 is retired
    else sync_wg();
    if (n + 1 < n_end) load_tile(it_of(n + 1), sQn, sOn, sLn, sDn);
    if constexpr (HALVES) {
      half(it, wave >> 1, sQ, sO, sL, sD);
    } else if (PAIRED) {
      paired(it, sQ, sO, sL, sD);
    } else {
      half(it, 0, sQ, sO, sL, sD);
      __builtin_amdgcn_sched_barrier(0);   // the halves share registers
      half(it, 1, sQ, sO, sL, sD);
    }
    if constexpr (DQA) {
      barrier_lds_loads_in_flight();   // every wave's dS^T of tile n is in sDS; tile n+1's loads stay in flight
      dq_tile(it);
    }
  };

  if (n0 < n_end) load_tile(it_of(n0), sQ0, sO0, sL0, sD0);
  int n = n0;
  for (; n + 1 < n_end; n += 2) {
    tile(n, sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1);
    tile(n + 1, sQ1, sO1, sL1, sD1, sQ0, sO0, sL0, sD0);
  }
  if (n < n_end) tile(n, sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1);

  if constexpr (HALVES) {
    // the wave of query half 1 hands its dK, dV sums to the wave of half 0
    // through the tile buffers (free once every wave is past its last tile)
    static_assert(TILE * sizeof(uint16_t) >= 16 * DT * 64 * sizeof(float), "merge buffer");
    sync_wg();
    float* xk = (float*)((wave & 1) ? sQ1 : sQ0);
    float* xv = (float*)((wave & 1) ? sO1 : sO0);
    if (wave >> 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xk[(16 * dt + r) * 64 + lane] = dk[dt][r];
          xv[(16 * dt + r) * 64 + lane] = dv[dt][r];
        }
    }
    sync_wg();
    if (wave >> 1) return;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[dt][r] += xk[(16 * dt + r) * 64 + lane];
        dv[dt][r] += xv[(16 * dt + r) * 64 + lane];
      }
  }

  if (kj < Skv) {
    uint16_t* dKg = (uint16_t*)a.dk + ((size_t)bh * Skv + kj) * D;
    uint16_t* dVg = (uint16_t*)a.dv + ((size_t)bh * Skv + kj) * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int col = 32 * dt + 8 * u + 4 * hi;
        *(u32x2*)(dKg + col) = u32x2{pack2<T>(dk[dt][4 * u] * sc, dk[dt][4 * u + 1] * sc),
                                     pack2<T>(dk[dt][4 * u + 2] * sc, dk[dt][4 * u + 3] * sc)};
        *(u32x2*)(dVg + col) = u32x2{pack2<T>(dv[dt][4 * u], dv[dt][4 * u + 1]),
                                     pack2<T>(dv[dt][4 * u + 2], dv[dt][4 * u + 3])};
      }
    }
  }
}

// ----------------------------------------------------------- dQ conversion

// Atomic dQ mode: dQ = scale * dQacc rounded to the 16-bit type, 8 elements
// per thread (two 16-byte loads, one 16-byte store).
template <class T>
__global__ __launch_bounds__(256) void dq_convert_kernel(const AttnArgs a, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x = *(const f32x4*)(a.dq_acc + 8 * i);
  const f32x4 y = *(const f32x4*)(a.dq_acc + 8 * i + 4);
  const float sc = a.scale;
  *(u32x4*)((uint16_t*)a.dq + 8 * i) = u32x4{pack2<T>(x[0] * sc, x[1] * sc), pack2<T>(x[2] * sc, x[3] * sc),
                                             pack2<T>(y[0] * sc, y[1] * sc), pack2<T>(y[2] * sc, y[3] * sc)};
}

// ----------------------------------------------------------------- launchers

int bwd16_block_kv() { return 128; }
int bwd16_block_q() { return 128; }

// Separate mode: the query pass runs first and writes delta and lse2 for the
// key/value pass; without it, the preprocess kernel provides them.  Atomic
// mode (dq_atomic, both passes wanted): preprocess (row statistics, zeroed
// accumulator), the key/value pass with the dQ products, the conversion.
template <class T, int D, int MOD, bool CAUSAL, bool MASK, bool BLK>
static hipError_t launch_bwd16_inst(const AttnArgs& a, bool want_kv, bool want_q, bool dq_atomic, hipStream_t st) {
  const int BH = a.B * a.H;
  const unsigned nkb = (unsigned)((a.Skv + bwd16_block_kv() - 1) / bwd16_block_kv());
  hipError_t err;
  if (dq_atomic && want_q && want_kv) {
    err = launch_bwd_pre(a, __is_same(T, BF16) ? 2 : 1, D, st, MOD == MOD_ALIBI ? 2 : 1);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((dkdv16_kernel<T, D, MOD, CAUSAL, MASK, BLK, true>), dim3(nkb * BH), dim3(256), 0, st, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t n8 = (int64_t)BH * a.Sq * D / 8;
    hipLaunchKernelGGL((dq_convert_kernel<T>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, a, n8);
    return hipGetLastError();
  }
  if (want_q) {
    err = launch_dq16(a, __is_same(T, BF16), D, MOD, CAUSAL, MASK, st);
  } else {
    err = launch_bwd_pre(a, __is_same(T, BF16) ? 2 : 1, D, st, MOD == MOD_ALIBI ? 2 : 1);
  }
  if (err != hipSuccess || !want_kv) return err;
  if (a.kv_halves)
    hipLaunchKernelGGL((dkdv16_kernel<T, D, MOD, CAUSAL, MASK, BLK, false, true>), dim3((unsigned)((a.Skv + 63) / 64) * BH),
                       dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dkdv16_kernel<T, D, MOD, CAUSAL, MASK, BLK, false>), dim3(nkb * BH), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class T, int D, int MOD, bool CAUSAL, bool MASK>
static hipError_t launch_bwd16_blk(const AttnArgs& a, bool kv, bool qq, bool at, hipStream_t st) {
  return a.block_mask ? launch_bwd16_inst<T, D, MOD, CAUSAL, MASK, true>(a, kv, qq, at, st)
                      : launch_bwd16_inst<T, D, MOD, CAUSAL, MASK, false>(a, kv, qq, at, st);
}

template <class T, int D, int MOD>
static hipError_t launch_bwd16_mod(const AttnArgs& a, bool causal, bool mask, bool kv, bool qq, bool at,
                                   hipStream_t st) {
  if (causal)
    return mask ? launch_bwd16_blk<T, D, MOD, true, true>(a, kv, qq, at, st)
                : launch_bwd16_blk<T, D, MOD, true, false>(a, kv, qq, at, st);
  return mask ? launch_bwd16_blk<T, D, MOD, false, true>(a, kv, qq, at, st)
              : launch_bwd16_blk<T, D, MOD, false, false>(a, kv, qq, at, st);
}

template <class T, int D>
static hipError_t launch_bwd16_d(const AttnArgs& a, int mod, bool causal, bool mask, bool kv, bool qq, bool at,
                                 hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return launch_bwd16_mod<T, D, MOD_ALIBI>(a, causal, mask, kv, qq, at, st);
    case MOD_CHECKERBOARD: return launch_bwd16_mod<T, D, MOD_CHECKERBOARD>(a, causal, mask, kv, qq, at, st);
    default: return launch_bwd16_mod<T, D, MOD_NONE>(a, causal, mask, kv, qq, at, st);
  }
}

hipError_t launch_bwd16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask, bool kv, bool qq,
                        bool dq_atomic, hipStream_t st) {
  if (bf16)
    return D == 64 ? launch_bwd16_d<BF16, 64>(a, mod, causal, mask, kv, qq, dq_atomic, st)
                   : launch_bwd16_d<BF16, 128>(a, mod, causal, mask, kv, qq, dq_atomic, st);
  return D == 64 ? launch_bwd16_d<F16, 64>(a, mod, causal, mask, kv, qq, dq_atomic, st)
                 : launch_bwd16_d<F16, 128>(a, mod, causal, mask, kv, qq, dq_atomic, st);
}

}  // namespace fa
