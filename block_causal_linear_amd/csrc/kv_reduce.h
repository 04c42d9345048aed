// KV reduction of one block: per token split s of every (b, h),
//   P_s = phi(K_s)^T V_s  (d x d)   and   p_s = phi(K_s)^T 1  (d).
// The computation splits along token order with identical results
// ("Nvidia, MIT ve diğerleri video yapay zeka devrimini başlattı", section
// "Sabit Bellekli KV önbelleğe alma mekanizması"), which is what lets many
// workgroups share one head's tokens.
//
// A sequence may be cut into several blocks (the whole-sequence block-causal
// call); every (block, split) pair gets its own partial in a buffer
// [B][H][blocks][splits][d*d + d] that state_reduce / state_scan sum in a
// fixed order.  With one block and one split the kernel writes
// S_out = S_in + P and z_out = z_in + p straight into the state.
#pragma once

#include "la_common.h"
#include "row_tiles.h"

namespace la {

// ---------------------------------------------------------------------------
// bfloat16 inputs: MFMA 16x16x32 over token tiles staged through LDS.
//
// The contraction runs over tokens, but K and V are token-major in HBM, so
// an MFMA operand (8 consecutive tokens of one feature per lane) is a column
// of the tile.  Each 64-token tile of K and V is loaded with coalesced 16-B
// loads (two tiles ahead, in registers), phi is applied to K in registers
// (v_pk_max_i16), and the tile is written to LDS token-major.  Operands are
// read back with the gfx950 transposing LDS read ds_read_b64_tr_b16: within
// each 16-lane group, lane i receives element (i mod 4) of the 8-byte chunks
// that lanes 4k + i/4 (k = 0..3) point at.  When lane j of the group points
// at features f0 + 4 (j mod 4) .. +3 of token t0 + j/4, lane i receives
// tokens t0 .. t0 + 3 of feature f0 + i; two such reads give the eight
// consecutive tokens of an operand.  The 16-byte unit index inside a token
// row is XOR-swizzled by 2 (t mod 4), so the four token rows one read
// touches fall on different LDS banks.
//
// Work split in a workgroup of WR x WC waves: wave (wi, wj) owns the output
// block rows [wi d/WR, +d/WR) x cols [wj d/WC, +d/WC); waves with wj == 0
// also accumulate z with a second MFMA against an all-ones B operand.

template <int D, int WR, int WC>
struct KvTile {
  static constexpr int NT = kWave * WR * WC;  // threads per workgroup
  static constexpr int TT = 64;               // tokens per tile
  static constexpr int UPR = D / 8;           // 16-byte units per token row
  static constexpr int UNITS = TT * UPR;      // units per tensor per tile
  static constexpr int CPT = UNITS / NT;      // units per thread per tensor
  static_assert(UNITS % NT == 0, "tile must split evenly over the workgroup");
};

// Wave layouts: 2 x 2 at d <= 64, 4 x 4 (1024 threads) at d = 128.
template <int D>
struct KvWaves {
  static constexpr int WR = D == 128 ? 4 : 2;
  static constexpr int WC = D == 128 ? 4 : 2;
};

template <int D>
constexpr int kv_threads() {
  return KvTile<D, KvWaves<D>::WR, KvWaves<D>::WC>::NT;
}

// Waves per SIMD kv_partial_bf16 is built for (its launch bound).  Without a
// bound the compiler kept the MFMA accumulators in AGPRs at d <= 64 and moved
// them every tile (32 v_accvgpr moves per loop iteration at d = 64, whose
// loop body has 118 VALU instructions); with it they stay in VGPRs (88 at
// d = 64, five waves per SIMD instead of four).
template <int D>
constexpr int kv_min_waves() {
  return D == 128 ? 1 : D == 64 ? 4 : 8;
}

template <int UPR>
__device__ __forceinline__ int unit_swizzle(int t) {
  return ((t & 3) * 2) & (UPR - 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Lane's MFMA operand: feature f0 + (lane % 16) of tokens ks + 8g .. +7,
// g = lane / 16, from a token-major tile whose 16-byte unit index is XORed
// with SWZ(t) in token row t (SWZ keeps the 4 rows one read touches on
// distinct 32-byte bank groups).
template <int UPR, int (*SWZ)(int) = unit_swizzle<UPR>>
__device__ __forceinline__ uint4 tile_column8(const uint16_t* tile, int ks, int f0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int f = f0 + 4 * (j & 3);  // this lane's 4-feature chunk
  uint4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = ks + 8 * g + 4 * h + (j >> 2);
    const int unit = (f >> 3) ^ SWZ(t);
    const uint16_t* p = tile + (t * UPR + unit) * 8 + (f & 7);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    const uint2 w = __builtin_bit_cast(uint2, v);
    if (h == 0) {
      r.x = w.x;
      r.y = w.y;
    } else {
      r.z = w.x;
      r.w = w.y;
    }
  }
  return r;
}

// Grid: (blocks x splits, H, B).  Block c covers tokens [c T, min((c+1) T, N))
// of every (b, h) sequence of N tokens; split s of it covers tps tokens.  The
// result for (b, h, c, s) goes to dst[((b H + h) C + c) splits + s]; with a
// single block and a single split, dst is the state itself and state_in (if
// any) is added.
template <int D>
__global__ __launch_bounds__(kv_threads<D>(), kv_min_waves<D>()) void kv_partial_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int TB, int splits,
    int tps, const float* state_in, float* dst) {
  constexpr int WR = KvWaves<D>::WR, WC = KvWaves<D>::WC;
  using T = KvTile<D, WR, WC>;
  constexpr int BR = D / WR, BC = D / WC;  // output block of one wave
  constexpr int NR = BR / 16, NC = BC / 16;
  constexpr int E = D * D + D;
  __shared__ uint4 lds[2][2][T::UNITS];  // [buffer][K, V][unit]

  const int nblk = gridDim.x / splits;
  const int blk = blockIdx.x / splits;
  const int split = blockIdx.x - blk * splits;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int c0 = blk * TB;
  const int c1 = min(N, c0 + TB);
  const int t0 = c0 + split * tps;
  const int t1 = min(c1, t0 + tps);
  const uint4* kb = reinterpret_cast<const uint4*>(k + bh * static_cast<size_t>(N) * D);
  const uint4* vb = reinterpret_cast<const uint4*>(v + bh * static_cast<size_t>(N) * D);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wi = wave / WC, wj = wave % WC;
  const int n = lane & 15, g = lane >> 4;

  f32x4 acc[NR][NC];
  f32x4 accz[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    accz[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);

  // Two register stages: while tile i is in LDS and being multiplied, the
  // loads of tiles i + 1 and i + 2 are in flight.
  uint4 rk0[T::CPT], rv0[T::CPT], rk1[T::CPT], rv1[T::CPT];
  // K and V through descriptors that cover the tile's rows inside the split:
  // rows past t1 read as zero in hardware, so no load needs a branch.
  auto gload = [&](uint4 (&rk)[T::CPT], uint4 (&rv)[T::CPT], int tile) {
    const int base = t0 + tile * T::TT;
    const int bytes = (min(t1, base + T::TT) - base) * T::UPR * 16;
    const size_t first = static_cast<size_t>(base) * T::UPR;
    const rsrc_t ksrc = tile_rsrc(kb, first, 16, bytes);
    const rsrc_t vsrc = tile_rsrc(vb, first, 16, bytes);
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int off = (tid + T::NT * i) * 16;
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(ksrc, off, 0, kBufNt);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(vsrc, off, 0, kBufNt);
      rk[i] = make_uint4(a.x, a.y, a.z, a.w);
      rv[i] = make_uint4(b.x, b.y, b.z, b.w);
    }
  };
  auto lstore = [&](const uint4 (&rk)[T::CPT], const uint4 (&rv)[T::CPT], int buf) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int u = tid + T::NT * i;
      const int t = u / T::UPR;
      const int c = u % T::UPR;
      const int s = t * T::UPR + (c ^ unit_swizzle<T::UPR>(t));
      lds[buf][0][s] = relu_bf16x8(rk[i]);
      lds[buf][1][s] = rv[i];
    }
  };
  auto compute = [&](int buf) {
    const uint16_t* lk = reinterpret_cast<const uint16_t*>(lds[buf][0]);
    const uint16_t* lv = reinterpret_cast<const uint16_t*>(lds[buf][1]);
#pragma unroll
    for (int ks = 0; ks < T::TT; ks += 32) {
      uint4 a[NR], b[NC];
#pragma unroll
      for (int r = 0; r < NR; ++r) a[r] = tile_column8<T::UPR>(lk, ks, wi * BR + r * 16, lane);
#pragma unroll
      for (int c = 0; c < NC; ++c) b[c] = tile_column8<T::UPR>(lv, ks, wj * BC + c * 16, lane);
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[r][c] = mfma_16x16x32(a[r], b[c], acc[r][c]);
      if (wj == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) accz[r] = mfma_16x16x32(a[r], ones, accz[r]);
      }
    }
  };

  // LDS buffer reuse: tile i + 2 overwrites the buffer tile i was read
  // from; every thread has passed tile i + 1's barrier, which follows its
  // own reads of tile i, before any thread writes tile i + 2.
  const int ntiles = t1 > t0 ? (t1 - t0 + T::TT - 1) / T::TT : 0;
  if (ntiles > 0) gload(rk0, rv0, 0);
  if (ntiles > 1) gload(rk1, rv1, 1);
  for (int it = 0; it < ntiles; it += 2) {
    lstore(rk0, rv0, 0);
    __syncthreads();
    if (it + 2 < ntiles) gload(rk0, rv0, it + 2);
    compute(0);
    if (it + 1 < ntiles) {
      lstore(rk1, rv1, 1);
      __syncthreads();
      if (it + 3 < ntiles) gload(rk1, rv1, it + 3);
      compute(1);
    }
  }

  const bool direct = nblk == 1 && splits == 1;
  float* o = dst + ((bh * nblk + blk) * splits + split) * static_cast<size_t>(E);
  const float* si = (direct && state_in != nullptr) ? state_in + bh * E : nullptr;
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wi * BR + r * 16 + 4 * g + i;
        const int cc = wj * BC + c * 16 + n;
        float x = acc[r][c][i];
        if (si) x = si[ra * D + cc] + x;
        o[ra * D + cc] = x;
      }
  if (wj == 0 && n == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wi * BR + r * 16 + 4 * g + i;
        float x = accz[r][i];
        if (si) x = si[D * D + ra] + x;
        o[D * D + ra] = x;
      }
  }
}

// ---------------------------------------------------------------------------
// One block at d = 128 with enough heads to fill the GPU: quadrants instead of
// token splits.  Workgroup (pair, quadrant) computes the 64 x 64 quadrant
// rows [a0, a0 + 64) x columns [c0, c0 + 64) of phi(K)^T V over every token
// of the block, from the 64-feature halves K[:, a0:] and V[:, c0:] of each
// token row (one 128-byte cache line each), and writes S_in + that quadrant
// straight into the state: no partial sums and no reduce launch.  The
// quadrants with c0 = 0 also write z_out[a0 .. a0 + 63].  Each element of the
// state is read and written by the same thread, so state_out may be state_in.
//
// The four quadrants of a head read the same halves twice over (K[:, a0:] by
// the two quadrants of row half a0, V[:, c0:] by those of column half c0):
// workgroups are numbered so that a head's four land on one XCD (workgroups
// are dealt to the eight XCDs round robin), where the second read of a line
// hits that XCD's L2.  With one four-wave workgroup per CU, the loads run
// KvQuad::PF tiles ahead.
#ifndef LA_KV_QUAD_PF
#define LA_KV_QUAD_PF 4
#endif
// 1: number the quadrant workgroups so that a head's four share an XCD.
#ifndef LA_KV_QUAD_XCD
#define LA_KV_QUAD_XCD 1
#endif
struct KvQuad {
  static constexpr int D = 128;
  static constexpr int F = 64;            // features of a half row
  static constexpr int TT = 64;           // tokens per tile
  static constexpr int UPR = F / 8;       // 16-byte units per half row
  static constexpr int RS = D / 8;        // 16-byte units per whole row
  static constexpr int NT = 4 * kWave;    // 2 x 2 waves, 32 x 32 outputs each
  static constexpr int UNITS = TT * UPR;
  static constexpr int CPT = UNITS / NT;
  static constexpr int PF = LA_KV_QUAD_PF;  // tiles in flight (registers)
  static constexpr int XCD = 8;
  // launch bound: waves per SIMD the registers must allow (keeps the MFMA
  // accumulators in VGPRs instead of moving them through AGPRs every tile)
  static constexpr int MIN_WAVES = 2;
  static_assert(UNITS % NT == 0, "tile must split evenly over the workgroup");
};

// Workgroups in the grid for BH (b, h) pairs: four per pair, rounded up to
// whole groups of eight pairs (the extra workgroups return at once).
__host__ __device__ constexpr long long kv_quad_workgroups(long long bh) {
  return 4 * KvQuad::XCD * ((bh + KvQuad::XCD - 1) / KvQuad::XCD);
}

__global__ __launch_bounds__(KvQuad::NT, KvQuad::MIN_WAVES) void kv_quad_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int BH,
    const float* state_in, float* state_out) {
  using Q = KvQuad;
  constexpr int D = Q::D, E = D * D + D;
  constexpr int NR = 2, NC = 2;  // 16 x 16 blocks per wave (32 x 32)
  __shared__ uint4 lds[2][2][Q::UNITS];  // [buffer][K, V][unit]

  // workgroup w -> XCD w % 8; the four quadrants of a pair share an XCD
  const int w = blockIdx.x;
  const int xcd = w % Q::XCD, r = w / Q::XCD;
  const int quad = LA_KV_QUAD_XCD ? r % 4 : w % 4;
  const int pair = LA_KV_QUAD_XCD ? (r / 4) * Q::XCD + xcd : w / 4;
  if (pair >= BH) return;
  const int a0 = (quad >> 1) * Q::F, c0 = (quad & 1) * Q::F;
  const size_t bh = static_cast<size_t>(pair);
  const uint4* kb = reinterpret_cast<const uint4*>(k + bh * static_cast<size_t>(N) * D) + a0 / 8;
  const uint4* vb = reinterpret_cast<const uint4*>(v + bh * static_cast<size_t>(N) * D) + c0 / 8;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wi = wave / 2, wj = wave % 2;
  const int n = lane & 15, g = lane >> 4;

  f32x4 acc[NR][NC];
  f32x4 accz[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    accz[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
  const bool zcols = c0 == 0 && wj == 0;

  uint4 rk[Q::PF][Q::CPT], rv[Q::PF][Q::CPT];
  // half rows of tile `tile` through descriptors that end at the last token:
  // rows past N read as zero
  auto gload = [&](uint4 (&ck)[Q::CPT], uint4 (&cv)[Q::CPT], int tile) {
    const int base = tile * Q::TT;
    const int rows = max(0, min(N, base + Q::TT) - base);
    const size_t first = static_cast<size_t>(base) * Q::RS;
    const rsrc_t ksrc = tile_rsrc(kb, first, 16, rows * Q::RS * 16);
    const rsrc_t vsrc = tile_rsrc(vb, first, 16, rows * Q::RS * 16);
#pragma unroll
    for (int i = 0; i < Q::CPT; ++i) {
      const int u = tid + Q::NT * i;
      const int off = ((u / Q::UPR) * Q::RS + u % Q::UPR) * 16;
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(ksrc, off, 0, kBufNt);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(vsrc, off, 0, kBufNt);
      ck[i] = make_uint4(a.x, a.y, a.z, a.w);
      cv[i] = make_uint4(b.x, b.y, b.z, b.w);
    }
  };
  auto lstore = [&](const uint4 (&ck)[Q::CPT], const uint4 (&cv)[Q::CPT], int buf) {
#pragma unroll
    for (int i = 0; i < Q::CPT; ++i) {
      const int u = tid + Q::NT * i;
      const int t = u / Q::UPR;
      const int c = u % Q::UPR;
      const int sl = t * Q::UPR + (c ^ unit_swizzle<Q::UPR>(t));
      lds[buf][0][sl] = relu_bf16x8(ck[i]);
      lds[buf][1][sl] = cv[i];
    }
  };
  auto compute = [&](int buf) {
    const uint16_t* lk = reinterpret_cast<const uint16_t*>(lds[buf][0]);
    const uint16_t* lv = reinterpret_cast<const uint16_t*>(lds[buf][1]);
#pragma unroll
    for (int ks = 0; ks < Q::TT; ks += 32) {
      uint4 a[NR], b[NC];
#pragma unroll
      for (int i = 0; i < NR; ++i) a[i] = tile_column8<Q::UPR>(lk, ks, wi * 32 + i * 16, lane);
#pragma unroll
      for (int j = 0; j < NC; ++j) b[j] = tile_column8<Q::UPR>(lv, ks, wj * 32 + j * 16, lane);
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int j = 0; j < NC; ++j) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
      if (zcols) {
#pragma unroll
        for (int i = 0; i < NR; ++i) accz[i] = mfma_16x16x32(a[i], ones, accz[i]);
      }
    }
  };

  // PF register stages, two LDS buffers, one barrier per tile: tile i + 2
  // overwrites the LDS buffer tile i was read from only after every thread
  // has passed tile i + 1's barrier, which follows its reads of tile i.
  // Stages run unconditionally in groups of PF: tiles past the last read
  // zeros through their empty descriptors and add exactly nothing, and no
  // load is conditional (a conditional load would make the compiler wait
  // for every load in flight before the barrier).
  const int ntiles = (N + Q::TT - 1) / Q::TT;
  // issued in tile order (the scheduler may not reorder them): the first
  // stage then waits for the oldest loads only
#pragma unroll
  for (int st = 0; st < Q::PF; ++st) {
    gload(rk[st], rv[st], st);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int it = 0; it < ntiles; it += Q::PF) {
#pragma unroll
    for (int st = 0; st < Q::PF; ++st) {
      lstore(rk[st], rv[st], st & 1);
      lds_barrier();
      gload(rk[st], rv[st], it + st + Q::PF);
      compute(st & 1);
    }
  }

  float* o = state_out + bh * E;
  const float* si = state_in != nullptr ? state_in + bh * E : nullptr;
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ra = a0 + wi * 32 + i * 16 + 4 * g + e;
        const int cc = c0 + wj * 32 + j * 16 + n;
        float x = acc[i][j][e];
        if (si) x = si[ra * D + cc] + x;
        o[ra * D + cc] = x;
      }
  if (zcols && n == 0) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ra = a0 + wi * 32 + i * 16 + 4 * g + e;
        float x = accz[i][e];
        if (si) x = si[D * D + ra] + x;
        o[D * D + ra] = x;
      }
  }
}

// ---------------------------------------------------------------------------
// float32 inputs: plain VALU outer-product accumulation (the float32 path is
// for exactness checks and small problems; bfloat16 is the bandwidth path).
template <int D>
__global__ __launch_bounds__(kBlock) void kv_partial_f32(const float* __restrict__ k,
                                                         const float* __restrict__ v, int N, int T,
                                                         int splits, int tps,
                                                         const float* state_in, float* dst) {
  constexpr int TT = 16;
  constexpr int E = D * D + D;
  constexpr int PER = D * D / kBlock;
  static_assert(D * D % kBlock == 0 && D <= kBlock, "shape");
  __shared__ float sk[TT * D];
  __shared__ float sv[TT * D];

  const int nblk = gridDim.x / splits;
  const int blk = blockIdx.x / splits;
  const int split = blockIdx.x - blk * splits;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int c0 = blk * T;
  const int c1 = min(N, c0 + T);
  const int t0 = c0 + split * tps;
  const int t1 = min(c1, t0 + tps);
  const float* kb = k + bh * static_cast<size_t>(N) * D;
  const float* vb = v + bh * static_cast<size_t>(N) * D;
  const int tid = threadIdx.x;

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float accz = 0.f;

  for (int base = t0; base < t1; base += TT) {
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D;
      float x = 0.f, y = 0.f;
      if (base + t < t1) {
        x = kb[static_cast<size_t>(base) * D + e];
        y = vb[static_cast<size_t>(base) * D + e];
      }
      sk[e] = x > 0.f ? x : 0.f;
      sv[e] = y;
    }
    __syncthreads();
    for (int t = 0; t < TT; ++t) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid + kBlock * i;
        acc[i] = fmaf(sk[t * D + e / D], sv[t * D + e % D], acc[i]);
      }
      if (tid < D) accz += sk[t * D + tid];
    }
    __syncthreads();
  }

  const bool direct = nblk == 1 && splits == 1;
  float* o = dst + ((bh * nblk + blk) * splits + split) * static_cast<size_t>(E);
  const float* si = (direct && state_in != nullptr) ? state_in + bh * E : nullptr;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + kBlock * i;
    o[e] = si ? si[e] + acc[i] : acc[i];
  }
  if (tid < D) o[D * D + tid] = si ? si[D * D + tid] + accz : accz;
}

}  // namespace la
