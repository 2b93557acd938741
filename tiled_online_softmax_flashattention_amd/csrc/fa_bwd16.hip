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
// Two deterministic passes, no atomics:
//  * dkdv16_kernel: key-stationary.  Each wave keeps 32 keys' K and V rows in
//    registers and their dK^T, dV^T accumulators, and loops over 64-query
//    tiles whose Q and dO are staged through LDS.  S and dP are formed with
//    queries as rows, so the lane holds one key and the probabilities feed
//    dV^T = dO^T P and dK^T = Q^T dS directly as MFMA B operands; the dO^T
//    and Q^T fragments come from the natural tiles through the transposing
//    LDS read.
//  * dq16_kernel: query-stationary, like the forward.  Each wave keeps 32
//    queries' Q and dO rows in registers; K and V tiles are staged natural;
//    S^T and dP^T are formed with keys as rows so the lane holds one query,
//    and dQ^T = K^T dS^T accumulates in registers (K^T fragments through the
//    transposing LDS read).
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// ---------------------------------------------------------------- preprocess

// delta_i = sum_d dO_id * O_id; lse2_i = lse_i * log2(e), +inf for an empty
// row (so that exp2(s - lse2) = 0 there).
template <int ES, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const AttnArgs a, int dtype) {
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
  if (row < rows && sub == 0) {
    a.delta[row] = acc;
    const float l = a.lse[row];
    a.lse2[row] = (l == kNegInf) ? __builtin_inff() : l * kLog2e;
  }
  (void)EPL;
}

hipError_t launch_bwd_pre(const AttnArgs& a, int dtype, int D, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.H * a.Sq;
  const int es = dtype == 0 ? 4 : 2;
  const int lpr = (D * es / 16) < 64 ? (D * es / 16) : 64;
  const int rpb = 256 / lpr;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(256);
  if (es == 4) {
    if (D == 64) hipLaunchKernelGGL((bwd_pre_kernel<4, 64>), grid, block, 0, st, a, dtype);
    else if (D == 128) hipLaunchKernelGGL((bwd_pre_kernel<4, 128>), grid, block, 0, st, a, dtype);
    else hipLaunchKernelGGL((bwd_pre_kernel<4, 512>), grid, block, 0, st, a, dtype);
  } else {
    if (D == 64) hipLaunchKernelGGL((bwd_pre_kernel<2, 64>), grid, block, 0, st, a, dtype);
    else hipLaunchKernelGGL((bwd_pre_kernel<2, 128>), grid, block, 0, st, a, dtype);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ shared helpers

// Natural-layout staging of a ROWS-row tile of a (rows, D) 16-bit tensor
// (pitch D + 8).  Rows past nrows are clamped to the last row (finite values
// that the kernels mask out), so the loads carry no branch.
template <int D, int ROWS>
struct Stage1 {
  static constexpr int N = ROWS * D / 8 / 256;   // 16-byte chunks per thread
  u32x4 r[N];
  __device__ __forceinline__ void load(const uint16_t* g, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + 256 * i, row = c / (D / 8), ch = c % (D / 8);
      r[i] = *(const u32x4*)(g + (size_t)min(row0 + row, nrows - 1) * D + 8 * ch);
    }
  }
  __device__ __forceinline__ void store(uint16_t* nat, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + 256 * i, row = c / (D / 8), ch = c % (D / 8);
      lds_write16(&nat[row * (D + 8) + 8 * ch], r[i]);
    }
  }
};

template <class T>
__device__ __forceinline__ u32x4 pack8(const f32x16& x, int u) {
  return u32x4{pack2<T>(x[8 * u + 0], x[8 * u + 1]), pack2<T>(x[8 * u + 2], x[8 * u + 3]),
               pack2<T>(x[8 * u + 4], x[8 * u + 5]), pack2<T>(x[8 * u + 6], x[8 * u + 7])};
}

// ------------------------------------------------------------- dK / dV pass

template <int D>
struct DkdvCfg {
  static constexpr int BKV = 128;   // keys per workgroup (4 waves x 32)
  static constexpr int BQ = 64;     // queries per tile
  static constexpr int QP = D + 8;
  // one buffer: Q and dO (natural, 16-bit), then the lse2 and delta rows
  static constexpr size_t buf_elems = (size_t)2 * BQ * QP + 2 * BQ * 2;
  static constexpr size_t lds = 2 * buf_elems * 2;
};

// Key-stationary dK/dV pass.  The ALiBi and checkerboard bias start the S
// accumulator (the per-query part, per register) with the per-key part and
// the key mask (-inf) folded into one per-lane exponent term, so per score
// the work is one subtraction of the row's lse, one FMA and one exp for P
// and a subtraction and a multiply for dS.  Query tiles are double buffered.
template <class T, int D, int MOD, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void dkdv16_kernel(const AttnArgs a) {
  using C = DkdvCfg<D>;
  constexpr int BKV = C::BKV, BQ = C::BQ, QP = C::QP;
  constexpr int KS = D / 16, DT = D / 32;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem16[];
  auto sQ = [&](int buf) { return smem16 + buf * C::buf_elems; };
  auto sO = [&](int buf) { return sQ(buf) + BQ * QP; };
  auto sL = [&](int buf) { return (float*)(sO(buf) + BQ * QP); };
  auto sDl = [&](int buf) { return sL(buf) + BQ; };

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int kb = blockIdx.x / BH;     // low kb = most query tiles under causal: dispatched first
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int k0 = kb * BKV;
  const int kw = k0 + 32 * wave;
  const int kj = kw + l32;            // this lane's key
  const float c = a.scale_log2;
  const float inv_scale = 1.0f / a.scale;

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
  // per-lane exponent term: the key's share of the bias, or -inf for a
  // masked key or a key past seq_kv (its dK, dV rows are not stored)
  bool key_ok = kj < Skv;
  if constexpr (MASK) key_ok = key_ok && a.key_mask[(size_t)b * Skv + min(kj, Skv - 1)] != 0;
  float slope2 = 0.f;
  f32x16 cinit = zero16();
  if constexpr (MOD == MOD_ALIBI) {
    // bias = slope (kj - q); per register: -slope * acc_row / scale
    const float slope = alibi_slope(a.alibi_slopes, h, a.H);
    slope2 = slope * kLog2e;
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = -slope * inv_scale * (float)acc_row(r, hi);
  }
  if constexpr (MOD == MOD_CHECKERBOARD) {
    // query tiles start at even positions, so register r holds a query of parity (r & 1)
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = (((kj + r) & 1) == 0 ? a.even_nat : a.odd_nat) * inv_scale;
  }

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  const int qt0 = CAUSAL ? k0 / BQ : 0;
  const int nqt = (Sq + BQ - 1) / BQ;
  Stage1<D, BQ> stq, sto;
  float lreg = 0.f, dreg = 0.f;
  int lq = 0;
  auto load_tile = [&](int it) {
    const int q0 = min(it, nqt - 1) * BQ;   // clamped: no branch next to the loads
    stq.load(Qg, q0, Sq, tid);
    sto.load(dOg, q0, Sq, tid);
    lq = q0 + (tid & (BQ - 1));
    lreg = lse2g[min(lq, Sq - 1)];
    dreg = deltag[min(lq, Sq - 1)];
  };
  auto store_tile = [&](int buf) {
    stq.store(sQ(buf), tid);
    sto.store(sO(buf), tid);
    if (tid < BQ) {   // rows past seq_q: P = 0 (lse2 = +inf) and delta = 0
      sL(buf)[tid] = lq < Sq ? lreg : __builtin_inff();
      sDl(buf)[tid] = lq < Sq ? dreg : 0.f;
    }
  };

  if (qt0 < nqt) {
    load_tile(qt0);
    store_tile(qt0 & 1);
    __syncthreads();
    load_tile(qt0 + 1);
  }
  for (int it = qt0; it < nqt; ++it) {
    const int q0 = it * BQ;
    __syncthreads();   // everyone is past tile it-1, whose buffer ((it+1)&1) is free
    store_tile((it + 1) & 1);
    load_tile(it + 2);
    if (CAUSAL && q0 + BQ - 1 < kw) continue;  // every query of the tile precedes every key of this wave
    const int buf = it & 1;
    const uint16_t* qb = sQ(buf);
    const uint16_t* ob = sO(buf);

    // one 32-query half at a time keeps S and dP to 32 registers
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      // S' = Q K^T + C and dP = dO V^T, queries as rows
      f32x16 sv = cinit, dpv = zero16();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int off = (32 * mt + l32) * QP + 16 * kk + 8 * hi;
        sv = mma16<T>(lds_read16(&qb[off]), kf[kk], sv);
        dpv = mma16<T>(lds_read16(&ob[off]), vf[kk], dpv);
      }
      // queries before the key (causal): P = 0, only on diagonal tiles
      if (CAUSAL && __builtin_amdgcn_ballot_w64(q0 + 32 * mt < kj) != 0) {
        const int lim_l = kj - q0 - 32 * mt - 4 * hi;   // rows with acc_row < kj - q0 - 32 mt are masked
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pos = 8 * (r >> 2) + (r & 3);
          if (pos < lim_l) sv[r] = kNegInf;
        }
      }
      float lb = key_ok ? 0.f : kNegInf;
      if constexpr (MOD == MOD_ALIBI) lb = key_ok ? slope2 * (float)(kj - q0 - 32 * mt) : kNegInf;
      const float* lrow = sL(buf) + 32 * mt + 4 * hi;
      const float* drow = sDl(buf) + 32 * mt + 4 * hi;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 l4 = *(const f32x4*)(lrow + 8 * u);
        const f32x4 d4 = *(const f32x4*)(drow + 8 * u);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int r = 4 * u + cc;
          const float p = exp2_hw(fmaf(sv[r], c, lb - l4[cc]));
          sv[r] = p;
          dpv[r] = p * (dpv[r] - d4[cc]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int st = 2 * mt + u;
        const u32x4 pb = pack8<T>(sv, u);
        const u32x4 db = pack8<T>(dpv, u);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dv[dt] = mma16<T>(read_a_tr(ob, QP, 16 * st, 32 * dt, lane), pb, dv[dt]);
          dk[dt] = mma16<T>(read_a_tr(qb, QP, 16 * st, 32 * dt, lane), db, dk[dt]);
        }
      }
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

// ----------------------------------------------------------------- dQ pass

template <int D>
struct Dq16Cfg {
  static constexpr int BM = 128;   // queries per workgroup
  static constexpr int BN = 64;    // keys per tile
  static constexpr int KP = D + 8;
  // one buffer: K and V natural (16-bit) and the key row
  static constexpr size_t buf_elems = (size_t)2 * BN * KP + 2 * BN * 2;
  static constexpr size_t lds = 2 * buf_elems * 2;
};

// Query-stationary dQ pass, structured like the forward kernel: the score_mod
// bias (and the key mask row) start the S^T accumulator, masking runs only on
// diagonal and tail tiles, tiles are double buffered with branch-free staging,
// and per score one FMA and one exp give P = 2^(S' c + b - lse2).
template <class T, int D, int MOD, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void dq16_kernel(const AttnArgs a) {
  using C = Dq16Cfg<D>;
  constexpr int BM = C::BM, BN = C::BN, KP = C::KP;
  constexpr int KS = D / 16, DT = D / 32;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem16[];
  auto sK = [&](int buf) { return smem16 + buf * C::buf_elems; };
  auto sV = [&](int buf) { return sK(buf) + BN * KP; };
  auto sB = [&](int buf) { return (float*)(sV(buf) + BN * KP); };   // 2 x BN floats: q parity 0 / 1

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (CAUSAL) qb = a.n_qblocks - 1 - qb;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM;
  const int qw = q0 + 32 * wave;
  const int qi = qw + l32;
  const float c = a.scale_log2;
  const float inv_scale = 1.0f / a.scale;

  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)bh * Sq * D;
  const uint16_t* dOg = (const uint16_t*)a.dout + (size_t)bh * Sq * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)bh * Skv * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)bh * Skv * D;

  // This lane's query: Q and dO rows as B operands, and the row's delta =
  // <dO, O> and lse * log2(e), which this pass also writes to the workspace
  // for the key/value pass that runs after it.
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
    if (ok && hi == 0) {
      a.delta[(size_t)bh * Sq + qi] = delta;
      a.lse2[(size_t)bh * Sq + qi] = lse2;
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
    for (int r = 0; r < 16; ++r) cinit[r] = (((qi + r) & 1) == 0 ? a.even_nat : a.odd_nat) * inv_scale;
  }

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = zero16();

  const int kv_end = CAUSAL ? min(Skv, q0 + BM) : Skv;
  const int ntiles = (kv_end + BN - 1) / BN;
  Stage1<D, BN> stk, stv;
  uint32_t mreg = 0;
  int mkv = 0;
  auto load_tile = [&](int n) {
    const int kv0 = min(n, ntiles - 1) * BN;   // clamped: no branch next to the loads
    stk.load(Kg, kv0, Skv, tid);
    stv.load(Vg, kv0, Skv, tid);
    if constexpr (MASK) {
      mkv = kv0 + (tid & (BN - 1));
      mreg = a.key_mask[(size_t)b * Skv + min(mkv, Skv - 1)];
    }
  };
  auto store_tile = [&](int buf) {
    stk.store(sK(buf), tid);
    stv.store(sV(buf), tid);
    if constexpr (MASK) {
      if (tid < BN) {
        const bool keep = mkv < Skv && mreg != 0;
        float e0 = 0.f, e1 = 0.f;
        if constexpr (MOD == MOD_CHECKERBOARD) {
          const bool kev = (mkv & 1) == 0;
          e0 = (kev ? a.even_nat : a.odd_nat) * inv_scale;
          e1 = (kev ? a.odd_nat : a.even_nat) * inv_scale;
        }
        sB(buf)[tid] = keep ? e0 : kNegInf;
        sB(buf)[BN + tid] = keep ? e1 : kNegInf;
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  load_tile(1);
  for (int n = 0; n < ntiles; ++n) {
    const int kv0 = n * BN;
    __syncthreads();   // everyone is past tile n-1, whose buffer ((n+1)&1) is free
    store_tile((n + 1) & 1);
    load_tile(n + 2);
    if (CAUSAL && kv0 > qw + 31) continue;
    const uint16_t* kb = sK(n & 1);
    const uint16_t* vb = sV(n & 1);

    // S'^T = K Q^T + C and dP^T = V dO^T, keys as rows
    f32x16 s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 acc = cinit;
      if constexpr (MASK) {
        const float* row = sB(n & 1) + ((qi & 1) ? BN : 0) + 32 * t + 4 * hi;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 m4 = *(const f32x4*)(row + 8 * u);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) acc[4 * u + cc] += m4[cc];
        }
      }
      f32x16 pacc = zero16();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int off = (32 * t + l32) * KP + 16 * kk + 8 * hi;
        acc = mma16<T>(lds_read16(&kb[off]), qf[kk], acc);
        pacc = mma16<T>(lds_read16(&vb[off]), of[kk], pacc);
      }
      s[t] = acc;
      dp[t] = pacc;
    }

    // scores past the diagonal or past seq_kv: -inf (only on such tiles)
    {
      int lim = 1 << 30;
      if (CAUSAL && kv0 + BN - 1 > qw) lim = qi - kv0;
      if (!MASK && kv0 + BN > Skv) lim = min(lim, Skv - 1 - kv0);
      if (__builtin_amdgcn_ballot_w64(lim < BN - 1) != 0) {
        const int lim_l = lim - 4 * hi;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pos = 32 * t + 8 * (r >> 2) + (r & 3);
            if (pos > lim_l) s[t][r] = kNegInf;
          }
        }
      }
    }

    float nb0 = -lse2, nb1 = -lse2;
    if constexpr (MOD == MOD_ALIBI) {
      const float add0 = slope2 * (float)(kv0 - qi);
      nb0 = add0 - lse2;
      nb1 = add0 + slope2 * 32.0f - lse2;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = exp2_hw(fmaf(s[0][r], c, nb0));
      const float p1 = exp2_hw(fmaf(s[1][r], c, nb1));
      dp[0][r] = p0 * (dp[0][r] - delta);
      dp[1][r] = p1 * (dp[1][r] - delta);
    }

    // dQ^T += K^T dS^T over the tile's 64 keys
#pragma unroll
    for (int st = 0; st < BN / 16; ++st) {
      const int t = st >> 1, u = st & 1;
      const u32x4 db = pack8<T>(dp[t], u);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dq[dt] = mma16<T>(read_a_tr(kb, KP, 16 * st, 32 * dt, lane), db, dq[dt]);
    }
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

template <class K>
static hipError_t launch_dyn(K kern, unsigned grid, size_t lds, hipStream_t st, const AttnArgs& a) {
  if (lds > 65536) {
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

// The query pass runs first and writes delta and lse2 for the key/value
// pass; without it, the preprocess kernel provides them.
template <class T, int D, int MOD, bool CAUSAL, bool MASK>
static hipError_t launch_bwd16_inst(const AttnArgs& a, bool want_kv, bool want_q, hipStream_t st) {
  const int BH = a.B * a.H;
  const unsigned nkb = (unsigned)((a.Skv + DkdvCfg<D>::BKV - 1) / DkdvCfg<D>::BKV);
  hipError_t err;
  if (want_q) {
    err = launch_dyn(dq16_kernel<T, D, MOD, CAUSAL, MASK>, (unsigned)a.n_qblocks * BH, Dq16Cfg<D>::lds, st, a);
  } else {
    err = launch_bwd_pre(a, __is_same(T, BF16) ? 2 : 1, D, st);
  }
  if (err != hipSuccess || !want_kv) return err;
  return launch_dyn(dkdv16_kernel<T, D, MOD, CAUSAL, MASK>, nkb * BH, DkdvCfg<D>::lds, st, a);
}

template <class T, int D, int MOD>
static hipError_t launch_bwd16_mod(const AttnArgs& a, bool causal, bool mask, bool kv, bool qq, hipStream_t st) {
  if (causal) return mask ? launch_bwd16_inst<T, D, MOD, true, true>(a, kv, qq, st) : launch_bwd16_inst<T, D, MOD, true, false>(a, kv, qq, st);
  return mask ? launch_bwd16_inst<T, D, MOD, false, true>(a, kv, qq, st) : launch_bwd16_inst<T, D, MOD, false, false>(a, kv, qq, st);
}

template <class T, int D>
static hipError_t launch_bwd16_d(const AttnArgs& a, int mod, bool causal, bool mask, bool kv, bool qq, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return launch_bwd16_mod<T, D, MOD_ALIBI>(a, causal, mask, kv, qq, st);
    case MOD_CHECKERBOARD: return launch_bwd16_mod<T, D, MOD_CHECKERBOARD>(a, causal, mask, kv, qq, st);
    default: return launch_bwd16_mod<T, D, MOD_NONE>(a, causal, mask, kv, qq, st);
  }
}

int bwd16_block_kv() { return 128; }
int bwd16_block_q() { return 128; }

hipError_t launch_bwd16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask, bool kv, bool qq,
                        hipStream_t st) {
  if (bf16)
    return D == 64 ? launch_bwd16_d<BF16, 64>(a, mod, causal, mask, kv, qq, st) : launch_bwd16_d<BF16, 128>(a, mod, causal, mask, kv, qq, st);
  return D == 64 ? launch_bwd16_d<F16, 64>(a, mod, causal, mask, kv, qq, st) : launch_bwd16_d<F16, 128>(a, mod, causal, mask, kv, qq, st);
}

}  // namespace fa
