// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Orientation used throughout: a wave computes S^T = K Q^T with one 32x32
// MFMA tile per 32 keys x 32 queries.  In the 32x32 accumulator layout lane l
// owns column n = l % 32 and rows m = 8*(r/4) + 4*(l/32) + (r%4) of register
// r, so every lane holds a single query (or, in the key-stationary backward
// pass, a single key) and the softmax row statistics stay inside one lane
// plus its partner lane l ^ 32.
#pragma once

#ifdef __HIPCC_RTC__
// Compiled at run time (hipRTC, the caller-defined score_mod kernels): the
// runtime header is implicit and the fixed-width types live in its namespace.
typedef __hip_internal::uint8_t uint8_t;
typedef __hip_internal::uint16_t uint16_t;
typedef __hip_internal::uint32_t uint32_t;
typedef __hip_internal::uint64_t uint64_t;
typedef __hip_internal::int64_t int64_t;
typedef __UINTPTR_TYPE__ uintptr_t;
#else
#include <hip/hip_runtime.h>
#include <stdint.h>
#endif

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

enum Mod { MOD_NONE = 0, MOD_ALIBI = 1, MOD_CHECKERBOARD = 2, MOD_CUSTOM = 3 };

// Element tags for the 16-bit storage types.
struct F16 {};
struct BF16 {};

// v_mfma_f32_32x32x16_{f16,bf16}: 8 operand values per lane, fp32 accumulate.
template <class T>
__device__ __forceinline__ f32x16 mma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (__is_same(T, F16)) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// v_mfma_f32_32x32x2_f32: one operand value per lane.
__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Round two floats to the 16-bit type (round to nearest even) and pack them,
// the first value in the low half.
template <class T>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  if constexpr (__is_same(T, F16)) {
    f16x2 v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Registers 8u .. 8u+7 of a 32 x 32 accumulator rounded and packed: the
// 16-bit operand fragment for keys (or queries) 16u .. 16u+15 of the block.
template <class T>
__device__ __forceinline__ u32x4 pack8(const f32x16& x, int u) {
  return u32x4{pack2<T>(x[8 * u + 0], x[8 * u + 1]), pack2<T>(x[8 * u + 2], x[8 * u + 3]),
               pack2<T>(x[8 * u + 4], x[8 * u + 5]), pack2<T>(x[8 * u + 6], x[8 * u + 7])};
}

// Place a loop-invariant MFMA operand in the accumulation registers (AGPRs).
// MFMA reads its A and B operands from either register file; at one wave per
// SIMD the accumulation file has room that the architectural one, holding
// the addresses and the softmax arithmetic, lacks.  (An empty asm statement
// with an AGPR operand: no instruction of its own.)
__device__ __forceinline__ void keep_in_agprs(u32x4& x) { asm volatile("" : "+a"(x)); }

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Query tile of the 16-bit key/value pass.  The query pass, which runs
// first, stores each row's lse2 with the query's ALiBi share relative to
// this tile's start folded in.
constexpr int kDkdvBQ = 64;

template <class T>
__device__ __forceinline__ float to_f32(uint16_t bits) {
  if constexpr (__is_same(T, F16)) {
    return (float)__builtin_bit_cast(_Float16, bits);
  } else {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  }
}

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (l ^ 32): one ds_bpermute with a loop-invariant address.
__device__ __forceinline__ float xor32(float x) {
  const int addr = (int)(((threadIdx.x & 63u) ^ 32u) << 2);
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row of the 32x32 accumulator held in register r by lane group hi.
__device__ __forceinline__ constexpr int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// Column order of the transposed (key- or query-major) LDS tiles.  A 16-wide
// MFMA step over keys takes, in lane group hi, the eight accumulator rows
// {8u + 4hi + c} (u = 0,1; c = 0..3) of one 32x32 tile; swapping bits 2 and 3
// of the position puts exactly those eight positions in one contiguous
// 16-byte run, so each operand fragment is a single ds_read_b128.
__device__ __forceinline__ constexpr int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Row swizzle of the 16-byte chunks of a transposed (dim-major) LDS tile.
// Readers take 8 consecutive rows at once (conflict-free when the 8 rows map
// to 8 distinct chunks); writers take rows 8 apart (Stage2) or 4 apart (the
// forward's V tile), which the d >> 3 term spreads over distinct chunks too.
__device__ __forceinline__ constexpr int tr_swz(int d) { return (d ^ (d >> 3)) & 7; }

// ALiBi slope for head h of H: slope_h = 2^(-8 (h+1) / H), or the caller's.
__device__ __forceinline__ float alibi_slope(const float* slopes, int h, int H) {
  return slopes ? slopes[h] : exp2f(-8.0f * (float)(h + 1) / (float)H);
}

__device__ __forceinline__ u32x4 lds_read16(const void* p) { return *(const u32x4*)p; }

// ds_read_b64_tr_b16: within each group of 16 lanes, output lane i receives,
// as element j, element (i & 3) of the four 16-bit values that lane
// 4j + (i >> 2) of the group addressed (measured on gfx950).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
  return __builtin_bit_cast(u32x2, r);
}

// A operand (M = 32 rows of dim d, K = 16 positions) of a product whose
// 16-bit tile is stored natural, position-major: tile[pos * pitch + d].
// Lane L gets dim d0 + (L & 31) and, in slots 0..3 / 4..7, positions
// p0 + 4 hi + 0..3 / p0 + 8 + 4 hi + 0..3 (hi = L >> 5): the positions an
// accumulator-layout B operand holds in its registers 8u .. 8u+7.  Each
// group of 16 lanes addresses 4 positions x 16 dims (8 bytes per lane).
__device__ __forceinline__ u32x4 read_a_tr(const uint16_t* tile, int pitch, int p0, int d0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int row = p0 + 4 * (g >> 1) + (s >> 2);
  const int col = d0 + 16 * (g & 1) + 4 * (s & 3);
  const u32x2 lo = lds_read_tr(tile + row * pitch + col);
  const u32x2 hi = lds_read_tr(tile + (row + 8) * pitch + col);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
// Unpadded (position, dim) 16-bit LDS tiles filled by direct loads store the
// 16-byte chunk c of row r at chunk c ^ tswz(r).  LDS has 64 banks of 4 bytes;
// a 16-byte read serves 16 lanes per pass and an 8-byte transposing read 32
// lanes (measured).  The row-fragment read (16 lanes: 16 consecutive rows, one
// chunk) and the transposing read (32 lanes: 4 consecutive rows, 4 adjacent
// chunks) are then both conflict-free: at 128-byte rows the two row parities
// use different bank halves, so bit 2 of the permutation (flipping every two
// rows) separates rows r and r+2 and bits 0-1 spread 8 rows of one parity; at
// 256-byte rows bits 2-3 separate the 4 rows of a transposing read and all 16
// rows of a fragment read get distinct chunks.
template <int D>
__device__ __forceinline__ constexpr int tswz(int r) {
  return D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
}

// Chunk permutation by tile mode: SW_BOTH uses tswz (tiles read both ways);
// SW_TR, for tiles read only by transposing reads, depends on r mod 4 alone
// (0, 6, 12, 10 at 256-byte rows: the 4 rows of one read get disjoint 4-chunk
// blocks), so rows r and r+8 share it and a lane's addresses differ by
// constant offsets; SW_NONE is plain rows.  Every permutation costs address
// registers where a lane's offsets stop being constants.
enum { SW_NONE = 0, SW_BOTH = 1, SW_TR = 2 };
template <int D, int SW>
__device__ __forceinline__ constexpr int chunk_perm(int r) {
  return SW == SW_BOTH ? tswz<D>(r) : SW == SW_TR ? (D == 64 ? 2 * (r & 3) : (0xAC60 >> (4 * (r & 3))) & 15) : 0;
}

// Element offset of (row, col) in a tile of D-element rows.
template <int D, int SW>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ chunk_perm<D, SW>(row)) << 3)) + (col & 7);
}

// A operand read from a tile (see read_a_tr for the lane layout).
template <int D, int SW>
__device__ __forceinline__ u32x4 read_a_tr_tile(const uint16_t* tile, int p0, int d0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int row = p0 + 4 * (g >> 1) + (s >> 2);
  const int col = d0 + 16 * (g & 1) + 4 * (s & 3);
  const u32x2 lo = lds_read_tr(tile + tile_off<D, SW>(row, col));
  const u32x2 hi = lds_read_tr(tile + tile_off<D, SW>(row + 8, col));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Cache-policy bits of a direct load: 0, or the non-temporal hint for data
// read exactly once (a key chunk of the split decode path).
constexpr int kCpolNone = 0;
constexpr int kCpolNT = 2;

// Direct load (global_load_lds_dwordx4) of a ROWS x D 16-bit tile into an LDS
// tile by the NW waves of a workgroup: wave w issues the 1 KiB blocks
// w*NJ .. w*NJ+NJ-1, each lane fetching the global chunk that belongs at its
// LDS slot.  Rows past nrows are clamped to the last row.
template <int D, int ROWS, int SW, int NW = 4, int CPOL = kCpolNone>
__device__ __forceinline__ void load_tile_lds(const uint16_t* g, int row0, int nrows, uint16_t* tile, int wave,
                                              int lane) {
  constexpr int NJ = ROWS * D * 2 / 1024 / NW;
  static_assert(NJ * NW * 1024 == ROWS * D * 2, "tile must split into 1 KiB blocks per wave");
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int blk = wave * NJ + j;
    const int e = blk * 512 + lane * 8;
    const int row = e / D, pch = (e % D) >> 3;
    const int lch = pch ^ chunk_perm<D, SW>(row);
    __builtin_amdgcn_global_load_lds((const void*)(g + (size_t)min(row0 + row, nrows - 1) * D + (lch << 3)),
                                     (lds_void_ptr)(tile + blk * 512), 16, 0, CPOL);
  }
}

// The same load for a tile whose rows all exist (row0 + ROWS <= nrows): a
// uniform base address plus a per-lane 32-bit byte offset, so the address
// arithmetic per tile is scalar.
template <int D, int ROWS, int SW, int NW = 4, int CPOL = kCpolNone>
__device__ __forceinline__ void load_full_tile_lds(const uint16_t* g_row0, uint16_t* tile, int wave, int lane) {
  constexpr int NJ = ROWS * D * 2 / 1024 / NW;
  static_assert(NJ * NW * 1024 == ROWS * D * 2, "tile must split into 1 KiB blocks per wave");
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int blk = wave * NJ + j;
    const int e = blk * 512 + lane * 8;
    const int row = e / D, pch = (e % D) >> 3;
    const uint32_t off = (uint32_t)(row * D + ((pch ^ chunk_perm<D, SW>(row)) << 3)) * 2u;
    __builtin_amdgcn_global_load_lds((const void*)((const char*)g_row0 + off), (lds_void_ptr)(tile + blk * 512), 16,
                                     0, CPOL);
  }
}

// Race-check build (FA_DEBUG_BARRIERS): every workgroup barrier and every
// wait for a wave's loads first drains all of the wave's outstanding memory
// operations (vector loads and stores, direct loads into LDS, LDS accesses),
// so nothing is in flight across a barrier.  The arithmetic is unchanged, so
// results that differ from the normal build's mean that some wave reads LDS
// before its writer (another wave, or its own load in flight) has finished.
#ifdef FA_DEBUG_BARRIERS
__device__ __forceinline__ void debug_drain() { __builtin_amdgcn_s_waitcnt(0); }
#else
__device__ __forceinline__ void debug_drain() {}
#endif

// Workgroup barrier with the release and acquire fences of __syncthreads.
__device__ __forceinline__ void sync_wg() {
  debug_drain();
  __syncthreads();
}

// Wait until this wave's direct loads have landed (vmcnt(0)).
__device__ __forceinline__ void wait_direct_loads() {
  debug_drain();
  __builtin_amdgcn_s_waitcnt(0x3f70);
}
// Wait until at most N (<= 63) of this wave's vector memory operations are in
// flight (they complete in issue order, so the older ones have).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  debug_drain();
  __builtin_amdgcn_s_waitcnt(0x3f70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vmcnt_le16() { wait_vmcnt_le<16>(); }

// Workgroup barrier ordering LDS only: each wave's LDS operations complete,
// then all waves meet.  Unlike __syncthreads() (a release fence on all of
// memory), it does not wait for the wave's global stores, atomics or direct
// loads still in flight; a caller that needs its direct loads in LDS waits
// for them (vmcnt) first.
__device__ __forceinline__ void barrier_lds() {
  debug_drain();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same barrier while this wave's direct loads into other LDS buffers are
// in flight: the fence of barrier_lds makes the compiler complete every
// pending direct load first, so this form waits for the wave's own LDS
// instructions (lgkmcnt) in the same asm block as the barrier, whose memory
// clobber keeps the compiler from moving memory accesses across it.  The
// caller must not read the buffers those loads write before waiting for them.
__device__ __forceinline__ void barrier_lds_loads_in_flight() {
  debug_drain();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void lds_write16(void* p, u32x4 v) { *(u32x4*)p = v; }
__device__ __forceinline__ void lds_write8(void* p, u32x2 v) { *(u32x2*)p = v; }

// A 32-row fp32 tile (rows row0 .., D floats each) held in registers by the
// 256 threads of a workgroup (thread tid holds the 16-byte chunks tid + 256 i),
// so the next tile of an fp32 loop can be loaded while the current one
// computes and stored to LDS (pitch D + 4) after the barrier that frees it.
// Rows past nrows are clamped to the last row (finite; the kernels mask them).
template <int D>
struct Rows32 {
  static constexpr int N = 32 * D / 4 / 256;
  f32x4 x[N];
  __device__ __forceinline__ void load(const float* g, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + 256 * i, row = c / (D / 4), ch = c % (D / 4);
      x[i] = *(const f32x4*)(g + (size_t)min(row0 + row, nrows - 1) * D + 4 * ch);
    }
  }
  __device__ __forceinline__ void store(float* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + 256 * i, row = c / (D / 4), ch = c % (D / 4);
      *(f32x4*)&dst[row * (D + 4) + 4 * ch] = x[i];
    }
  }
};

// The same 32-row fp32 tile (pitch D + 4 floats) staged with direct loads
// (global_load_lds_dwordx4), for rows of a whole number of 1 KiB blocks
// (head_dim 512: two per row): each instruction fills one block of one row,
// wave w the rows 8w .. 8w+7, no registers held and every load of the tile in
// flight at once.  The caller waits (wait_direct_loads) and synchronises the
// workgroup before reading the tile.
// One direct load (global_load_lds_dwordx4: lane i's 16 bytes from g land at
// lds_blk + 16 i) issued from inline assembly, so the compiler does not track
// it: a pipelined loop then waits with its own vmcnt counts instead of the
// compiler draining every load in flight before each LDS read.  The
// instruction has no register result (its address registers are read at
// issue); the caller's waits and barriers order it.  It writes M0 and says so
// (an m0 clobber), so the compiler re-establishes any other value it keeps in
// M0 after it.  Users: the head_dim 512 fp32 forward and dQ pass.
__device__ __forceinline__ void direct_load16_untracked(const void* g, const void* lds_blk) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(lds_void_ptr)lds_blk;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0v), "v"(g) : "memory", "m0");
}

template <int D, bool UNTRACKED = false>
__device__ __forceinline__ void stage32_direct(float* dst, const float* g, int row0, int nrows, int wave, int lane) {
  static_assert(D * 4 % 1024 == 0, "rows must be whole 1 KiB blocks");
  constexpr int BPR = D * 4 / 1024;   // blocks per row
  const int w = __builtin_amdgcn_readfirstlane(wave);   // the LDS address (M0) is uniform
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int row = w * 8 + r;
    const float* src = g + (size_t)min(row0 + row, nrows - 1) * D + lane * 4;
#pragma unroll
    for (int hb = 0; hb < BPR; ++hb) {
      if constexpr (UNTRACKED)
        direct_load16_untracked(src + hb * 256, dst + row * (D + 4) + hb * 256);
      else
        __builtin_amdgcn_global_load_lds((const void*)(src + hb * 256),
                                         (lds_void_ptr)(dst + row * (D + 4) + hb * 256), 16, 0, 0);
    }
  }
}

// Exchange of partial 32x32 accumulators between the waves that split a
// head's dims (fp32 head_dim 512): wave w stores its 16 values per lane at
// sS[w * 1024 + lane * 16 ..] as four 16-byte chunks, chunk c at position
// c ^ ((lane >> 2) & 3), so a 16-lane pass of 16-byte accesses touches 16
// distinct 4-bank groups; after a barrier every wave of group g sums the DS
// partials of waves g*DS .. g*DS+DS-1.
__device__ __forceinline__ void slice_put(float* sS, const f32x16& x, int wave, int lane) {
  float* base = sS + wave * 1024 + lane * 16;
  const int sw = (lane >> 2) & 3;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    *(f32x4*)(base + 4 * (c ^ sw)) = f32x4{x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]};
}

template <int DS>
__device__ __forceinline__ f32x16 slice_gather(const float* sS, int g, int lane) {
  f32x16 s;
  const int sw = (lane >> 2) & 3;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int e2 = 0; e2 < DS; ++e2) {
      const f32x4 v = *(const f32x4*)(sS + (g * DS + e2) * 1024 + lane * 16 + 4 * (c ^ sw));
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * c + i] = e2 == 0 ? v[i] : s[4 * c + i] + v[i];
    }
  }
  return s;
}

// Workgroup order.  Workgroups are dealt to the 8 XCDs round robin (block i
// runs on XCD i mod 8), each XCD with its own 4 MB L2.  Block i of a grid of
// BH * nblk blocks gets (bh, blk):
//  * causal (blocks of unequal length): bh = i mod BH, blk = i / BH, so with
//    BH a multiple of 8 each head stays on one XCD and the blocks of every
//    head are dealt in the same order (the kernels turn blk into
//    longest-first);
//  * otherwise, with BH a multiple of 8: XCD x = i mod 8 takes heads
//    x, x + 8, ... one after the other, blk = (i / 8) mod nblk, so the blocks
//    resident on an XCD span one or two heads and share their K/V (or Q/dO)
//    in its L2 (8 heads at once would not fit at 4096 x 128);
//  * otherwise the first rule.
struct BlockCoord {
  int bh, blk;
};
__device__ __forceinline__ BlockCoord block_coord(int i, int BH, int nblk, bool causal) {
  if (causal || (BH & 7) != 0) return BlockCoord{i % BH, i / BH};
  const int x = i & 7, j = i >> 3;
  return BlockCoord{x + 8 * (j / nblk), j % nblk};
}

// Per-key additive rows for queries of even and odd position (key mask and
// checkerboard) share one LDS array: the odd row starts one row plus 16 bytes
// in, so that in a 16-byte read, whose lanes hold queries of both parities,
// the two rows' chunks fall in different banks (one row apart they would
// share every bank).
template <int BN>
__device__ __forceinline__ constexpr int parity_row_off() {
  return BN + 4;
}

// Order of a forward split over the key axis: query blocks longest first
// (with causal, the last blocks: their chunks are full), the chunks of one
// block next to each other, so that the longest pieces of work start first
// and the short ones (diagonal chunks; chunks past the diagonal, which exit at
// once) fill in at the end.  bh is the fastest index, as in block_coord.
// Workgroup i runs on XCD i mod 8; with chunk j of every block's group on the
// same XCD, the XCDs holding the first chunks would get most of the causal
// work.  So the chunk also turns with the block: the (j, k) pairs of one XCD
// recur every g = 8 / gcd(BH * n_split, 8) blocks, and chunk
// (j + k / g) mod n_split runs through every chunk on every XCD.
struct SplitCoord {
  int bh, qb, split;
};
__device__ __forceinline__ SplitCoord split_coord(int i, int BH, int nq, int n_split, bool causal) {
  const int bh = i % BH, r = i / BH;
  const int k = r / n_split, j = r - k * n_split;   // k-th longest block
  const int m = (BH * n_split) & 7;                   // BH n_split mod 8
  const int g = m == 0 ? 1 : (m & 1) ? 8 : (m & 3) ? 4 : 2;
  return SplitCoord{bh, causal ? nq - 1 - k : k, (j + k / g) % n_split};
}

// Launch arguments of every attention kernel (tensors contiguous BHSD).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;     // backward workspace: rowsum(dO * O), (B, H, Sq)
  float* lse2;      // backward workspace: lse * log2(e), +inf for empty rows (16-bit ALiBi: plus the
                    // query's bias share within its 64-query tile)
  float* dq_acc;    // backward workspace of the atomic dQ mode: fp32 (B, H, Sq, D) sums of dS K
  const uint8_t* key_mask;
  const float* alibi_slopes;
  float* partial;   // decode workspace
  int B, H, Sq, Skv;
  float scale;         // natural-log scale applied to q.k
  float scale_log2;    // scale * log2(e)
  float even_log2;     // checkerboard bias * log2(e) for even (i + j)
  float odd_log2;      // ... for odd (i + j)
  float even_nat;      // checkerboard bias, natural units
  float odd_nat;
  int causal;
  int q_off;           // position of query row 0 among the keys
  int n_qblocks;
  int n_split;         // decode: number of key chunks
  int chunk;           // decode: keys per chunk
  const uint8_t* block_mask;   // (B, H, bm_rows, bm_cols) bytes, 0 = block skipped; NULL = dense
  int bm_rows, bm_cols;        // ceil(Sq / kBlk), ceil(Skv / kBlk)
  const float* mod_params;     // caller-defined score_mod: its parameter array (device), or NULL
  int dq_halves;               // 16-bit dQ pass: 64-query blocks, two waves per query group (host choice)
  int kv_halves;               // 16-bit dK/dV pass: 64-key blocks, two waves per key group (host choice)
};

// ------------------------------------------------------------ block sparsity
//
// A block mask (the flaxattention page's create_block_mask over 128 x 128
// blocks) removes whole blocks of (query row, key) pairs: block (r, c) covers
// query rows 128r .. 128r+127 and keys 128c .. 128c+127.  A workgroup first
// lists the tiles of its loop whose block is set, in ascending order, in LDS,
// and then runs its usual double-buffered loop over that list, so a skipped
// block costs neither loads nor arithmetic.

constexpr int kBlk = 128;             // block edge of the block mask (rows and keys)
constexpr int kBlkMaxSeq = 131072;    // longest seq_q / seq_kv with a block mask (bounds the LDS lists)

// Writes, in ascending order, the tiles t in [t_lo, t_hi) whose block byte
// bytes[(t >> shift) * stride] is nonzero to list, and returns their number
// (uniform).  Every thread of the 4-wave workgroup calls it; cnt4 is 4 ints of
// LDS.  Ends with a barrier, so the list is visible to all waves on return.
__device__ __forceinline__ int compact_tiles(const uint8_t* bytes, int stride, int shift, int t_lo, int t_hi,
                                             uint16_t* list, int* cnt4) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int total = 0;
  for (int base = t_lo; base < t_hi; base += 256) {
    const int t = base + tid;
    const bool vis = t < t_hi && bytes[(size_t)(t >> shift) * stride] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(vis);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (lane == 0) cnt4[wave] = __builtin_popcountll(bal);
    sync_wg();
    int before = total, sum = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int cw = cnt4[w];
      sum += cw;
      if (w < wave) before += cw;
    }
    if (vis) list[before + below] = (uint16_t)t;
    total = __builtin_amdgcn_readfirstlane(total + sum);
    sync_wg();
  }
  return total;
}

// Entry n of an LDS tile list, as a uniform value.
__device__ __forceinline__ int list_at(const uint16_t* list, int n) {
  return __builtin_amdgcn_readfirstlane((int)list[n]);
}

}  // namespace fa
