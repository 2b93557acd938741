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
// owns 32 queries.  Key/value tiles of 64 keys are staged through LDS: K in
// its natural (key, dim) layout, V transposed to (dim, key) so both products
// read operand fragments with single 16-byte LDS reads.  The next tile is
// fetched from HBM into registers while the current one is being used.
//
// Per tile and wave: S^T = K Q^T (MFMA 32x32x16, Q resident in registers as
// the B operand), then scale / bias / mask in fp32, row max and sum (inside
// the lane plus one exchange with lane ^ 32), then O^T += V^T P^T with P
// rounded to the input type.  Causal: key tiles past the block's last query
// are never visited, waves skip tiles entirely past their own queries, and
// per-element masking happens only on diagonal tiles.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

template <class T, int D, int MOD, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, 2) void fwd16_kernel(const AttnArgs a) {
  constexpr int BM = 128;          // queries per workgroup
  constexpr int BN = 64;           // keys per tile
  constexpr int KP = D + 8;        // K tile pitch in elements (16-byte pad)
  constexpr int NK = D / 32;       // 16-byte K chunks per thread per tile
  constexpr int NV = D / 64;       // 4x4 V blocks per thread per tile
  constexpr int QS = D / 16;       // MFMA steps of the q.k product
  constexpr int DT = D / 32;       // 32-row tiles of O^T

  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * BN];  // V^T, 16-byte chunks XOR-swizzled by row
  __shared__ __attribute__((aligned(16))) uint8_t sM[BN];

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

  float slope2 = 0.f, cb0 = 0.f, cb1 = 0.f;
  if constexpr (MOD == MOD_ALIBI) slope2 = alibi_slope(a.alibi_slopes, h, a.H) * kLog2e;
  if constexpr (MOD == MOD_CHECKERBOARD) {
    // register r holds a key of parity (r & 1); (qi + kv) is even when the parities agree
    const bool qeven = (qi & 1) == 0;
    cb0 = qeven ? a.even_log2 : a.odd_log2;
    cb1 = qeven ? a.odd_log2 : a.even_log2;
  }

  const int kv_end = CAUSAL ? min(Skv, q0 + BM) : Skv;
  const int ntiles = (kv_end + BN - 1) / BN;

  u32x4 kreg[NK];
  u32x2 vreg[NV][4];
  uint8_t mreg = 0;

  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int c = tid + 256 * i, row = c / (D / 8), ch = c % (D / 8), kv = kv0 + row;
      kreg[i] = kv < Skv ? *(const u32x4*)(Kg + (size_t)kv * D + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, db = e % (D / 4), kvb = e / (D / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kv = kv0 + 4 * kvb + r;
        vreg[i][r] = kv < Skv ? *(const u32x2*)(Vg + (size_t)kv * D + 4 * db) : u32x2{0u, 0u};
      }
    }
    if constexpr (MASK) {
      if (tid < BN) mreg = (kv0 + tid < Skv) ? a.key_mask[(size_t)b * Skv + kv0 + tid] : 0;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int c = tid + 256 * i, row = c / (D / 8), ch = c % (D / 8);
      lds_write16(&sK[row * KP + 8 * ch], kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, db = e % (D / 4), kvb = e / (D / 4);
      const int col = swap23(4 * kvb);  // logical column of keys 4kvb .. 4kvb+3
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int d = 4 * db + c4, word = c4 >> 1, sh = (c4 & 1) * 16;
        const uint32_t e0 = (vreg[i][0][word] >> sh) & 0xffffu, e1 = (vreg[i][1][word] >> sh) & 0xffffu;
        const uint32_t e2 = (vreg[i][2][word] >> sh) & 0xffffu, e3 = (vreg[i][3][word] >> sh) & 0xffffu;
        const int phys = (((col >> 3) ^ (d & 7)) << 3) + (col & 7);
        lds_write8(&sV[d * BN + phys], u32x2{e0 | (e1 << 16), e2 | (e3 << 16)});
      }
    }
    if constexpr (MASK) {
      if (tid < BN) sM[tid] = mreg;
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero16();

  load_tile(0);
  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * BN;
    if (j > 0) __syncthreads();
    store_tile();
    __syncthreads();
    if (j + 1 < ntiles) load_tile(kv0 + BN);
    if (CAUSAL && kv0 > qw + 31) continue;  // every key of the tile follows every query of this wave

    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
#pragma unroll
      for (int kk = 0; kk < QS; ++kk)
        s[t] = mma16<T>(lds_read16(&sK[(32 * t + l32) * KP + 16 * kk + 8 * hi]), qf[kk], s[t]);
    }

    const bool diag = CAUSAL && (kv0 + BN - 1 > qw);
    const bool tail = kv0 + BN > Skv;
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t mw = 0xffffffffu;
        if constexpr (MASK) mw = *(const uint32_t*)&sM[32 * t + 8 * u + 4 * hi];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * u + c;
          const int kv = kv0 + 32 * t + acc_row(r, hi);
          float x = s[t][r] * a.scale_log2;
          if constexpr (MOD == MOD_ALIBI) x += slope2 * (float)(kv - qi);
          if constexpr (MOD == MOD_CHECKERBOARD) x += (r & 1) ? cb1 : cb0;
          if constexpr (MASK) {
            if (((mw >> (8 * c)) & 0xffu) == 0u) x = kNegInf;
          } else {
            if (tail && kv >= Skv) x = kNegInf;
          }
          if (diag && kv > qi) x = kNegInf;
          s[t][r] = x;
          mx = fmaxf(mx, x);
        }
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(s[t][r] - m_use);
        s[t][r] = p;
        ls += p;
      }
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

#pragma unroll
    for (int st = 0; st < BN / 16; ++st) {
      const int t = st >> 1, u = st & 1;
      const u32x4 pb = {pack2<T>(s[t][8 * u + 0], s[t][8 * u + 1]), pack2<T>(s[t][8 * u + 2], s[t][8 * u + 3]),
                        pack2<T>(s[t][8 * u + 4], s[t][8 * u + 5]), pack2<T>(s[t][8 * u + 6], s[t][8 * u + 7])};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + l32;
        const int phys = ((2 * st + hi) ^ (d & 7)) << 3;
        o[dt] = mma16<T>(lds_read16(&sV[d * BN + phys]), pb, o[dt]);
      }
    }
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
