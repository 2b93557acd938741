// Split-KV decode: one query per (batch, head) against seq_kv keys.
//
// The flaxattention page times single-query decoding separately and lists
// faster decoding as open work; with one query the problem is a pair of
// matrix-vector products bound by streaming K and V from HBM, so it gets its
// own kernels instead of the 128-query tiles of the forward.
//
// decode_split_kernel: workgroup (b, h, chunk) streams its chunk of keys.
// Each key is handled by a group of lanes that each own 16 bytes of the head
// (8 halves or 4 floats), so a wave reads whole rows with fully coalesced
// 16-byte loads; the group reduces the dot product with lane shuffles and
// keeps its own online-softmax state (max, sum, accumulator slice).  Groups,
// then waves, are merged exactly, and the chunk's (max, sum, accumulator) go
// to the workspace.
// decode_merge_kernel: combines the chunks of each (b, h):
//   M = max_s m_s, w_s = 2^(m_s - M), O = sum w_s acc_s / sum w_s l_s,
//   lse = (M + log2 sum w_s l_s) ln 2.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

struct F32 {};

template <class T>
struct Elem {
  static constexpr int size = 2;
};
template <>
struct Elem<F32> {
  static constexpr int size = 4;
};

template <class T>
__device__ __forceinline__ void unpack16(const u32x4 x, float* out) {
  if constexpr (__is_same(T, F32)) {
    const f32x4 xf = __builtin_bit_cast(f32x4, x);  // whole-vector cast (see bwd_pre_kernel)
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = xf[c];
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      out[2 * c] = to_f32<T>((uint16_t)(x[c] & 0xffffu));
      out[2 * c + 1] = to_f32<T>((uint16_t)(x[c] >> 16));
    }
  }
}

// Online-softmax state of a group; all values in log2 units.
template <int EPL>
struct State {
  float m, l, acc[EPL];
};

template <int EPL>
__device__ __forceinline__ void merge_into(State<EPL>& s, float m2, float l2, const float* acc2) {
  const float M = fmaxf(s.m, m2);
  const float Mu = (M == kNegInf) ? 0.f : M;
  const float w1 = exp2_hw(s.m - Mu), w2 = exp2_hw(m2 - Mu);
  s.l = s.l * w1 + l2 * w2;
#pragma unroll
  for (int c = 0; c < EPL; ++c) s.acc[c] = s.acc[c] * w1 + acc2[c] * w2;
  s.m = M;
}

// Keys per lane group per step (U), chosen per launch by the chunk length:
// with non-temporal loads, 4096-key chunks (32768 keys, 8 x 8 heads) measured
// U = 1: 104.5, 2: 85.7, 3: 86.4, 4: 82.2 us, and 256-key chunks (2048 keys)
// U = 1: 12.7, 2: 11.5, 3: 12.0, 4: 12.5 us.
constexpr int kDecodeLongChunk = 2048;   // chunks this long use U = 4, shorter ones U = 2

// With BLK, keys whose 128-key block is unset in block row 0 of the block
// mask are neither loaded nor counted.
template <class T, int D, int MOD, bool MASK, bool BLK, int U>
__global__ __launch_bounds__(256) void decode_split_kernel(const AttnArgs a) {
  constexpr int ES = Elem<T>::size;
  constexpr int EPL = 16 / ES;           // elements per lane
  constexpr int LPK = D / EPL;           // lanes per key
  constexpr int KPW = 64 / LPK;          // keys per wave per step
  constexpr int KPB = 4 * KPW;           // keys per workgroup per step
  __shared__ float sPart[4][D + 2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane / LPK, sub = lane % LPK;
  const int split = blockIdx.x % a.n_split;
  const int bh = blockIdx.x / a.n_split;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Skv = a.Skv;
  // causal: only keys 0 .. q_off exist for the query (the split covers just those)
  const int kv_len = a.causal ? min(Skv, a.q_off + 1) : Skv;
  const int c0 = split * a.chunk;
  const int c1 = min(kv_len, c0 + a.chunk);

  const char* Kg = (const char*)a.k + ((size_t)bh * Skv * D) * ES + sub * 16;
  const char* Vg = (const char*)a.v + ((size_t)bh * Skv * D) * ES + sub * 16;
  float qv[EPL];
  unpack16<T>(*(const u32x4*)((const char*)a.q + (size_t)bh * D * ES + sub * 16), qv);
#pragma unroll
  for (int c = 0; c < EPL; ++c) qv[c] *= a.scale_log2;

  float slope2 = 0.f;
  if constexpr (MOD == MOD_ALIBI) slope2 = alibi_slope(a.alibi_slopes, h, a.H) * kLog2e;
  const uint8_t* mrow = MASK ? a.key_mask + (size_t)b * Skv : nullptr;
  const uint8_t* brow = BLK ? a.block_mask + (size_t)bh * a.bm_rows * a.bm_cols : nullptr;

  State<EPL> st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < EPL; ++c) st.acc[c] = 0.f;

  // Software prefetch: the next batch of U keys per group is requested before
  // the current one is used (rows past the chunk are clamped to its last key
  // and masked), so two batches are in flight per lane.  K and V are read
  // exactly once, so the loads carry the non-temporal hint (measured at 32768
  // keys: 95 -> 86 us).
  u32x4 kx[U], vx[U], kn[U], vn[U];
  auto load_batch = [&](int base, u32x4* kk, u32x4* vv) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kv = min(base + u * KPB, c1 - 1);
      if (!BLK || brow[kv >> 7] != 0) {
        kk[u] = __builtin_nontemporal_load((const u32x4*)(Kg + (size_t)kv * D * ES));
        vv[u] = __builtin_nontemporal_load((const u32x4*)(Vg + (size_t)kv * D * ES));
      } else {
        kk[u] = u32x4{0u, 0u, 0u, 0u};
        vv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  const int base0 = c0 + wave * KPW + grp;
  load_batch(base0, kx, vx);
  for (int base = base0; base < c1; base += U * KPB) {
    load_batch(base + U * KPB, kn, vn);
    float t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      unpack16<T>(kx[u], kf);
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < EPL; ++c) d += qv[c] * kf[c];
#pragma unroll
      for (int w = 1; w < LPK; w <<= 1) d += __shfl_xor(d, w);
      const int kv = base + u * KPB;
      if constexpr (MOD == MOD_ALIBI) d += slope2 * (float)(kv - a.q_off);  // -slope * (q_off - kv)
      if constexpr (MOD == MOD_CHECKERBOARD) d += ((kv + a.q_off) & 1) ? a.odd_log2 : a.even_log2;
      bool ok = kv < c1;
      if constexpr (MASK) ok = ok && mrow[min(kv, c1 - 1)] != 0;
      if constexpr (BLK) ok = ok && brow[min(kv, c1 - 1) >> 7] != 0;
      t[u] = ok ? d : kNegInf;
    }
    float mx = st.m;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, t[u]);
    const float mu = (mx == kNegInf) ? 0.f : mx;
    const float alpha = exp2_hw(st.m - mu);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < EPL; ++c) st.acc[c] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = exp2_hw(t[u] - mu);
      float vf[EPL];
      unpack16<T>(vx[u], vf);
      st.l += p;
#pragma unroll
      for (int c = 0; c < EPL; ++c) st.acc[c] += p * vf[c];
    }
    st.m = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kx[u] = kn[u];
      vx[u] = vn[u];
    }
  }

  // merge the groups of the wave (lanes with equal sub)
#pragma unroll
  for (int w = LPK; w < 64; w <<= 1) {
    float acc2[EPL];
#pragma unroll
    for (int c = 0; c < EPL; ++c) acc2[c] = __shfl_xor(st.acc[c], w);
    const float m2 = __shfl_xor(st.m, w), l2 = __shfl_xor(st.l, w);
    merge_into<EPL>(st, m2, l2, acc2);
  }
  if (grp == 0) {
#pragma unroll
    for (int c = 0; c < EPL; ++c) sPart[wave][sub * EPL + c] = st.acc[c];
    if (sub == 0) {
      sPart[wave][D] = st.m;
      sPart[wave][D + 1] = st.l;
    }
  }
  sync_wg();
  if (wave == 0 && grp == 0) {
    for (int w2 = 1; w2 < 4; ++w2) {
      float acc2[EPL];
#pragma unroll
      for (int c = 0; c < EPL; ++c) acc2[c] = sPart[w2][sub * EPL + c];
      merge_into<EPL>(st, sPart[w2][D], sPart[w2][D + 1], acc2);
    }
    float* out = a.partial + ((size_t)bh * a.n_split + split) * (D + 2);
#pragma unroll
    for (int c = 0; c < EPL; ++c) out[sub * EPL + c] = st.acc[c];
    if (sub == 0) {
      out[D] = st.m;
      out[D + 1] = st.l;
    }
  }
}

constexpr int kMaxSplit = 256;

// One workgroup of D threads per output row: (b, h) for decode, (b, h, query)
// for a query block split over the key axis.  Thread d reads, for 8 chunks at
// a time, each chunk's (max, sum) and its own accumulator element together
// (the max and sum addresses are the same for every thread: one broadcast),
// so a batch of chunks costs one round of independent loads; batches merge
// online, rescaled to the running max.  No LDS, no barrier.  With causal a
// row reads only the chunks that hold keys up to its position (the split
// forward writes no partial for a chunk past its query block's last key).
constexpr int kMergeBatch = 8;

template <class T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const AttnArgs a) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  int ns = a.n_split;
  if (a.causal) {
    const int qpos = bh % a.Sq + a.q_off;
    const int kv_end = min(a.Skv, qpos + 1);
    ns = min(ns, (kv_end + a.chunk - 1) / a.chunk);
  }
  const float* part = a.partial + (size_t)bh * a.n_split * (D + 2);
  float M = kNegInf, L = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch], av[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool ok = s0 + j < ns;
      const float* pj = part + (size_t)(ok ? s0 + j : s0) * (D + 2);
      mv[j] = ok ? pj[D] : kNegInf;
      lv[j] = ok ? pj[D + 1] : 0.f;
      av[j] = ok ? pj[d] : 0.f;
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) mb = fmaxf(mb, mv[j]);
    const float mu = (mb == kNegInf) ? 0.f : mb;
    const float sc = exp2_hw(M - mu);
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float w = exp2_hw(mv[j] - mu);
      L += w * lv[j];
      acc += w * av[j];
    }
    M = mb;
  }
  const float o = L > 0.f ? acc / L : 0.f;
  if constexpr (__is_same(T, F32)) {
    ((float*)a.o)[(size_t)bh * D + d] = o;
  } else if constexpr (__is_same(T, F16)) {
    ((_Float16*)a.o)[(size_t)bh * D + d] = (_Float16)o;
  } else {
    ((__bf16*)a.o)[(size_t)bh * D + d] = (__bf16)o;
  }
  if (d == 0 && a.lse) a.lse[bh] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

// Merge for the forward split over keys (many rows): D / 2 threads per row,
// two dims per thread with 8-byte loads (a partial row of D + 2 floats is
// 8-byte aligned), 256 / (D / 2) rows per workgroup; otherwise the same
// batched online merge as decode_merge_kernel.
template <class T, int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const AttnArgs a, int rows) {
  constexpr int TPR = D / 2, RPW = 256 / TPR;
  const int t = threadIdx.x % TPR;
  const int row = blockIdx.x * RPW + threadIdx.x / TPR;
  if (row >= rows) return;
  int ns = a.n_split;
  if (a.causal) {   // chunks holding keys up to the row's position
    const int kv_end = min(a.Skv, row % a.Sq + a.q_off + 1);
    ns = min(ns, (kv_end + a.chunk - 1) / a.chunk);
  }
  const float* part = a.partial + (size_t)row * a.n_split * (D + 2);
  float M = kNegInf, L = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    float2 av[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool ok = s0 + j < ns;
      const float* pj = part + (size_t)(ok ? s0 + j : s0) * (D + 2);
      mv[j] = ok ? pj[D] : kNegInf;
      lv[j] = ok ? pj[D + 1] : 0.f;
      const float2 x = *(const float2*)(pj + 2 * t);
      av[j] = ok ? x : float2{0.f, 0.f};
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) mb = fmaxf(mb, mv[j]);
    const float mu = (mb == kNegInf) ? 0.f : mb;
    const float sc = exp2_hw(M - mu);
    L *= sc;
    acc0 *= sc;
    acc1 *= sc;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float w = exp2_hw(mv[j] - mu);
      L += w * lv[j];
      acc0 += w * av[j].x;
      acc1 += w * av[j].y;
    }
    M = mb;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t o = (size_t)row * D + 2 * t;
  if constexpr (__is_same(T, F32)) {
    *(float2*)((float*)a.o + o) = float2{acc0 * inv, acc1 * inv};
  } else {
    *(uint32_t*)((uint16_t*)a.o + o) = pack2<T>(acc0 * inv, acc1 * inv);
  }
  if (t == 0 && a.lse) a.lse[row] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

template <class T>
static hipError_t launch_split_merge_t(const AttnArgs& a, int D, int rows, hipStream_t st) {
  const unsigned rpw = 256u / (unsigned)(D / 2);
  const dim3 grid(((unsigned)rows + rpw - 1) / rpw);
  if (D == 64) hipLaunchKernelGGL((split_merge_kernel<T, 64>), grid, dim3(256), 0, st, a, rows);
  else hipLaunchKernelGGL((split_merge_kernel<T, 128>), grid, dim3(256), 0, st, a, rows);
  return hipGetLastError();
}

hipError_t launch_split_merge(const AttnArgs& a, int dtype, int D, int rows, hipStream_t st) {
  if (dtype == 0) return launch_split_merge_t<F32>(a, D, rows, st);
  if (dtype == 2) return launch_split_merge_t<BF16>(a, D, rows, st);
  return launch_split_merge_t<F16>(a, D, rows, st);
}

int decode_choose_split(int BH, int Skv, int* chunk, int cus) {
  // Aim for about two workgroups per CU in total (512 on MI355X; longer
  // streams per workgroup measured faster than more, shorter chunks), with
  // chunks of 256 .. 4096 keys (a multiple of 64 keys).
  const long long wgs = 2LL * (cus > 0 ? cus : 256);
  long long c = ((long long)Skv * BH + wgs - 1) / wgs;
  c = (c + 63) / 64 * 64;
  if (c < 256) c = 256;
  if (c > 4096) c = 4096;
  if (c > Skv) c = (Skv + 63) / 64 * 64;
  if ((Skv + c - 1) / c > kMaxSplit) c = (Skv + kMaxSplit - 1) / kMaxSplit;  // bounds the merge's serial batches
  *chunk = (int)c;
  return (int)((Skv + c - 1) / c);
}

template <class T, int D, int MOD, bool MASK, bool BLK>
static void launch_decode_split(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H * a.n_split));
  if (a.chunk >= kDecodeLongChunk)
    hipLaunchKernelGGL((decode_split_kernel<T, D, MOD, MASK, BLK, 4>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, MOD, MASK, BLK, 2>), grid, dim3(256), 0, st, a);
}

template <class T, int D, int MOD, bool MASK>
static hipError_t launch_decode_inst(const AttnArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  if (a.block_mask) launch_decode_split<T, D, MOD, MASK, true>(a, st);
  else launch_decode_split<T, D, MOD, MASK, false>(a, st);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)BH), dim3(D), 0, st, a);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_decode_d(const AttnArgs& a, int mod, bool mask, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return mask ? launch_decode_inst<T, D, MOD_ALIBI, true>(a, st) : launch_decode_inst<T, D, MOD_ALIBI, false>(a, st);
    case MOD_CHECKERBOARD:
      return mask ? launch_decode_inst<T, D, MOD_CHECKERBOARD, true>(a, st) : launch_decode_inst<T, D, MOD_CHECKERBOARD, false>(a, st);
    default: return mask ? launch_decode_inst<T, D, MOD_NONE, true>(a, st) : launch_decode_inst<T, D, MOD_NONE, false>(a, st);
  }
}

template <class T>
static hipError_t launch_merge_t(const AttnArgs& a, int D, int rows, hipStream_t st) {
  if (D == 64) hipLaunchKernelGGL((decode_merge_kernel<T, 64>), dim3((unsigned)rows), dim3(64), 0, st, a);
  else hipLaunchKernelGGL((decode_merge_kernel<T, 128>), dim3((unsigned)rows), dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const AttnArgs& a, int dtype, int D, int rows, hipStream_t st) {
  if (dtype == 0) return launch_merge_t<F32>(a, D, rows, st);
  if (dtype == 2) return launch_merge_t<BF16>(a, D, rows, st);
  return launch_merge_t<F16>(a, D, rows, st);
}

template <class T>
static hipError_t launch_decode_t(const AttnArgs& a, int D, int mod, bool mask, hipStream_t st) {
  return D == 64 ? launch_decode_d<T, 64>(a, mod, mask, st) : launch_decode_d<T, 128>(a, mod, mask, st);
}

hipError_t launch_decode(const AttnArgs& a, int dtype, int D, int mod, bool mask, hipStream_t st) {
  if (dtype == 0) return launch_decode_t<F32>(a, D, mod, mask, st);
  if (dtype == 2) return launch_decode_t<BF16>(a, D, mod, mask, st);
  return launch_decode_t<F16>(a, D, mod, mask, st);
}

}  // namespace fa
