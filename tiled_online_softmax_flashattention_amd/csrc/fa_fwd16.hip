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
// owns 32 queries.  Key/value tiles of 64 keys are staged through LDS in their
// natural (key, dim) layout; the P V product reads its V fragments with the
// transposing LDS read (ds_read_b64_tr_b16), so no transpose is done in
// registers.  K and V are double
// buffered: while tile n is used, tile n+1 is written to the other buffers
// and tile n+2 is in flight from HBM into registers, so one barrier per tile
// suffices.  At head_dim 64 the kernel fits 3 waves per SIMD; issuing the
// next tile's scores before the current softmax was measured slower here
// because its extra registers cost a wave of occupancy.
//
// Per tile and wave: S'^T = K Q^T + C (MFMA 32x32x16, Q resident in registers
// as the B operand).  The accumulator starts from C = bias / scale, so the
// score_mod costs no per-score instruction: for ALiBi C holds the bias of the
// key's offset inside the tile (the tile's own offset is a per-lane scalar
// folded into the exponent), for the checkerboard the two parity values, and
// with a key mask C is read from an LDS row that holds 0 or -inf per key.
// Then one FMA and one v_exp_f32 per score give P = 2^(S' c + b - m).  The
// running max is updated lazily: only when some query's maximum grows by more
// than 2^8 does the wave rescale its accumulator, otherwise P stays below 2^8
// (exact in fp16/bf16 range; the final division by l cancels the scale).
// Causal: key tiles past the block's last query are never visited, tiles are
// visited diagonal first (so the largest ALiBi scores set the maximum early),
// waves skip tiles entirely past their own queries, and the per-score
// comparison happens only on diagonal and ragged-tail tiles.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr float kLazyRescale = 8.0f;   // log2 units: P is kept below 2^8

template <class T, int D, int MOD, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, D == 64 ? 3 : 1) void fwd16_kernel(const AttnArgs a) {
  constexpr int BM = 128;          // queries per workgroup
  constexpr int BN = 64;           // keys per tile
  constexpr int KP = D + 8;        // K tile pitch in elements (16-byte pad)
  constexpr int NK = D / 32;       // 16-byte K (and V) chunks per thread per tile
  constexpr int QS = D / 16;       // MFMA steps of the q.k product
  constexpr int DT = D / 32;       // 32-row tiles of O^T

  // Double buffers: tile n+1 is written while tile n is read.
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * KP];      // V natural, read transposed
  __shared__ __attribute__((aligned(16))) float sB[2][MASK ? 2 * BN : 4];  // per-key additive row (q parity 0 / 1)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (CAUSAL) qb = a.n_qblocks - 1 - qb;  // longest query blocks are dispatched first
  const int b = bh / a.H, h = bh - b * a.H;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
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
    // register r holds a key of parity (r & 1); (qi + kv) is even when the parities agree
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[r] = (((qi + r) & 1) == 0 ? a.even_nat : a.odd_nat) * inv_scale;
  }

  const int kv_end = CAUSAL ? min(Skv, q0 + BM) : Skv;
  const int ntiles = (kv_end + BN - 1) / BN;
  // causal: the diagonal tile first, then towards key 0
  auto kv_of = [&](int n) { return (CAUSAL ? ntiles - 1 - n : n) * BN; };
  // every key of the tile follows every query of this wave
  auto skipped = [&](int n) { return CAUSAL && kv_of(n) > qw + 31; };

  // Staging loads are unconditional: rows past seq_kv are clamped to the last
  // row (finite values whose scores are masked to -inf), so no branch (and no
  // wait for outstanding loads at a branch merge) sits next to a load.
  u32x4 kreg[NK], vreg[NK];
  uint32_t mreg = 0;
  int mkv = 0;

  auto load_k = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int cc = tid + 256 * i, row = cc / (D / 8), ch = cc % (D / 8);
      kreg[i] = *(const u32x4*)(Kg + (size_t)min(kv0 + row, Skv - 1) * D + 8 * ch);
    }
    if constexpr (MASK) {
      mkv = kv0 + (tid & (BN - 1));
      mreg = a.key_mask[(size_t)b * Skv + min(mkv, Skv - 1)];
    }
  };
  auto load_v = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int cc = tid + 256 * i, row = cc / (D / 8), ch = cc % (D / 8);
      vreg[i] = *(const u32x4*)(Vg + (size_t)min(kv0 + row, Skv - 1) * D + 8 * ch);
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int cc = tid + 256 * i, row = cc / (D / 8), ch = cc % (D / 8);
      lds_write16(&sK[buf][row * KP + 8 * ch], kreg[i]);
    }
    if constexpr (MASK) {
      if (tid < BN) {
        const bool keep = mkv < Skv && mreg != 0;
        float e0 = 0.f, e1 = 0.f;   // additive bias for queries of parity 0 / 1
        if constexpr (MOD == MOD_CHECKERBOARD) {
          const bool kev = (mkv & 1) == 0;
          e0 = (kev ? a.even_nat : a.odd_nat) * inv_scale;
          e1 = (kev ? a.odd_nat : a.even_nat) * inv_scale;
        }
        sB[buf][tid] = keep ? e0 : kNegInf;
        sB[buf][BN + tid] = keep ? e1 : kNegInf;
      }
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int cc = tid + 256 * i, row = cc / (D / 8), ch = cc % (D / 8);
      lds_write16(&sV[buf][row * KP + 8 * ch], vreg[i]);
    }
  };
  // S'^T = K Q^T + C for the tile held in K buffer `buf`
  auto scores = [&](int buf, f32x16* s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 acc = cinit;
      if constexpr (MASK) {
        const float* row = sB[buf] + ((qi & 1) ? BN : 0) + 32 * t + 4 * hi;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 m4 = *(const f32x4*)(row + 8 * u);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) acc[4 * u + cc] += m4[cc];
        }
      }
#pragma unroll
      for (int kk = 0; kk < QS; ++kk)
        acc = mma16<T>(lds_read16(&sK[buf][(32 * t + l32) * KP + 16 * kk + 8 * hi]), qf[kk], acc);
      s[t] = acc;
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero16();

  // Staging is unconditional (tile indices past the end are clamped to the
  // last tile): the buffers written near the end are never read again, and
  // straight-line staging keeps the load waits exact.
  auto kv_c = [&](int n) { return kv_of(min(n, ntiles - 1)); };

  load_k(kv_c(0));
  load_v(kv_c(0));
  store_k(0);
  store_v(0);
  __syncthreads();
  load_k(kv_c(1));
  load_v(kv_c(1));
  f32x16 sa[2], sb[2];

  // one tile (n): stage tile n+1, then scores, softmax and P V of tile n
  auto tile = [&](int n, f32x16* s) {
    const int kv0 = kv_of(n);
    __syncthreads();   // everyone is past tile n-1, whose buffers ((n+1)&1) are now free
    store_k((n + 1) & 1);    // K of tile n+1
    store_v((n + 1) & 1);    // V of tile n+1
    load_k(kv_c(n + 2));
    load_v(kv_c(n + 2));
    if (skipped(n)) return;
    scores(n & 1, s);

    // scores past the diagonal or past seq_kv: -inf (only on such tiles)
    {
      int lim = 1 << 30;   // last allowed key position inside the tile, for this lane
      if (CAUSAL && kv0 + BN - 1 > qw) lim = qi - kv0;
      if (!MASK && kv0 + BN > Skv) lim = min(lim, Skv - 1 - kv0);
      if (__builtin_amdgcn_ballot_w64(lim < BN - 1) != 0) {
        const int lim_l = lim - 4 * hi;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pos = 32 * t + 8 * (r >> 2) + (r & 3);   // acc_row(r, hi) - 4 hi
            if (pos > lim_l) s[t][r] = kNegInf;
          }
        }
      }
    }

    // per-lane exponent offsets of the two 32-key halves (ALiBi: bias of the half's first key)
    float add0 = 0.f, add1 = 0.f;
    if constexpr (MOD == MOD_ALIBI) {
      add0 = slope2 * (float)(kv0 - qi);
      add1 = add0 + slope2 * 32.0f;
    }
    float mx0 = s[0][0], mx1 = s[1][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      mx0 = fmaxf(mx0, s[0][r]);
      mx1 = fmaxf(mx1, s[1][r]);
    }
    float mx = fmaxf(fmaf(mx0, c, add0), fmaf(mx1, c, add1));
    mx = fmaxf(mx, xor32(mx));
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_hw(m_run - ((m_new == kNegInf) ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    const float nb0 = add0 - m_use, nb1 = add1 - m_use;
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = exp2_hw(fmaf(s[0][r], c, nb0));
      const float p1 = exp2_hw(fmaf(s[1][r], c, nb1));
      s[0][r] = p0;
      s[1][r] = p1;
      ls += p0 + p1;
    }
    l_run += ls;

    // O^T += V^T P^T
    const uint16_t* vb = sV[n & 1];
#pragma unroll
    for (int st = 0; st < BN / 16; ++st) {
      const int t = st >> 1, u = st & 1;
      const u32x4 pb = {pack2<T>(s[t][8 * u + 0], s[t][8 * u + 1]), pack2<T>(s[t][8 * u + 2], s[t][8 * u + 3]),
                        pack2<T>(s[t][8 * u + 4], s[t][8 * u + 5]), pack2<T>(s[t][8 * u + 6], s[t][8 * u + 7])};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = mma16<T>(read_a_tr(vb, KP, 16 * st, 32 * dt, lane), pb, o[dt]);
    }
  };

  for (int n = 0; n < ntiles; n += 2) {
    tile(n, sa);
    if (n + 1 < ntiles) tile(n + 1, sb);
  }

  const float l_tot = l_run + xor32(l_run);
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

template <class T, int D, int MOD>
static hipError_t launch_fwd16_mod(const AttnArgs& a, bool causal, bool mask, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_qblocks * a.B * a.H)), block(256);
  if (causal) {
    if (mask) hipLaunchKernelGGL((fwd16_kernel<T, D, MOD, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd16_kernel<T, D, MOD, true, false>), grid, block, 0, st, a);
  } else {
    if (mask) hipLaunchKernelGGL((fwd16_kernel<T, D, MOD, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd16_kernel<T, D, MOD, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fwd16_d(const AttnArgs& a, int mod, bool causal, bool mask, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return launch_fwd16_mod<T, D, MOD_ALIBI>(a, causal, mask, st);
    case MOD_CHECKERBOARD: return launch_fwd16_mod<T, D, MOD_CHECKERBOARD>(a, causal, mask, st);
    default: return launch_fwd16_mod<T, D, MOD_NONE>(a, causal, mask, st);
  }
}

int fwd16_block_q() { return 128; }

hipError_t launch_fwd16(const AttnArgs& a, bool bf16, int D, int mod, bool causal, bool mask, hipStream_t st) {
  if (bf16) {
    return D == 64 ? launch_fwd16_d<BF16, 64>(a, mod, causal, mask, st)
                   : launch_fwd16_d<BF16, 128>(a, mod, causal, mask, st);
  }
  return D == 64 ? launch_fwd16_d<F16, 64>(a, mod, causal, mask, st)
                 : launch_fwd16_d<F16, 128>(a, mod, causal, mask, st);
}

}  // namespace fa
