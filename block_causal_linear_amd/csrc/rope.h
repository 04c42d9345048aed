// Linear attention with rotary position embedding (RoPE) over the latent
// token grid.  The Linear DiT adds rotary position encoding so attention
// sees relative positions in space and time (sd114.wiki article on
// SANA-Video, section "1. 线性 DiT").  Placement and layout are this
// library's reading; the pages give none:
//   * 3-D positions: token i of a (b, h) sequence sits at frame
//     frame0 + i / (gh gw), row (i / gw) % gh, column i % gw;
//   * features (2m, 2m + 1) form pair m; the first d_t / 2 pairs turn with
//     the frame, the next d_h / 2 with the row, the last d_w / 2 with the
//     column (d_h = d_w = 2 floor(d / 6), d_t = d - d_h - d_w); pair j of a
//     group of size d_a turns by p theta^(-2 j / d_a);
//   * RoFormer's linear-attention form (Su et al. 2021, section 3.4.3): the
//     rotation acts on phi(q) and phi(k) in the numerator only, so
//       S = sum_j R_j phi(k_j) v_j^T,  z = sum_j phi(k_j),
//       o_i = (R_i phi(q_i))^T S / (phi(q_i) . z + eps).
// The state keeps the (d*d + d) layout; its S holds keys rotated by their
// absolute positions, so a stream carries it across blocks when every call
// passes the absolute frame of its first token.
//
// Precision.  A rotated bfloat16 feature is no longer a bfloat16 value: it
// is formed in float32 and carried as a bfloat16 hi/lo pair (16 significant
// bits).  The KV kernel multiplies both halves with V (exact in bf16); the
// readout multiplies the rotated query's hi/lo against S's hi/lo (three
// products, the lo x lo term dropped).  Angles are formed in turns with the
// product's rounding error folded back in (fmaf), so the turn count keeps
// float resolution at any position; the bfloat16 kernels take sin and cos
// from v_sin_f32 / v_cos_f32, the float32 kernels from sincospif.
#pragma once

#include "la_common.h"
#include "kv_reduce.h"
#include "row_tiles.h"
#include "rope_math.h"

namespace la {

// Waves per SIMD kv_partial_rope_bf16 is built for.  Its LDS (48 KB a
// workgroup at d = 64, 24 KB at d = 32) allows three (six) workgroups per
// CU, and the bound says so: without it the compiler kept the accumulators
// in AGPRs and moved them every tile (32 v_accvgpr moves per two tiles at
// d = 64).
template <int D>
constexpr int kv_rope_min_waves() {
  return D == 128 ? 1 : D == 64 ? 3 : 6;
}

// ---------------------------------------------------------------------------
// KV reduction with rotated keys (bfloat16 inputs).  The tiling, grid and
// partial layout are those of kv_partial_bf16; what changes is the staging
// of K: phi(K) is turned by the token's angles in float32 and written to
// LDS as a hi and a lo tile, and z is summed from the unrotated phi(K) on
// the VALU (each thread keeps one 16-byte column of the token rows, so it
// sums eight features; the partial sums meet in LDS at the end and are
// added in a fixed order).
template <int D>
__global__ __launch_bounds__(kv_threads<D>(), kv_rope_min_waves<D>()) void kv_partial_rope_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int TB, int splits,
    int tps, const float* state_in, float* dst, RopeGrid rg) {
  constexpr int WR = KvWaves<D>::WR, WC = KvWaves<D>::WC;
  using T = KvTile<D, WR, WC>;
  constexpr int BR = D / WR, BC = D / WC;
  constexpr int NR = BR / 16, NC = BC / 16;
  constexpr int E = D * D + D;
  static_assert(T::NT % T::UPR == 0, "a thread keeps one unit column");
  static_assert(T::NT * 8 <= 3 * T::UNITS * 4, "z partial sums fit one LDS buffer");
  __shared__ uint4 lds[2][3][T::UNITS];  // [buffer][K hi, K lo, V][unit]

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
  const int cu = tid % T::UPR;  // this thread's 16-byte column: pairs 4 cu .. 4 cu + 3

  float2 fq[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) fq[e] = rope_freq<D>(4 * cu + e, rg.theta);
  // positions of this thread's token rows, tile after tile
  const RopeStep tstep = rope_step(rg, T::TT);
  RopeTrack trk[T::CPT];
#pragma unroll
  for (int i = 0; i < T::CPT; ++i) trk[i].init(rg, t0 + (tid + T::NT * i) / T::UPR);
  float zacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zacc[j] = 0.f;

  f32x4 acc[NR][NC];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 rk0[T::CPT], rv0[T::CPT], rk1[T::CPT], rv1[T::CPT];
  // Raw buffer loads through descriptors that cover the tile's rows inside
  // the split: the hardware returns zero for rows past t1, so the last tile
  // needs no branch (a branch costs a zero fill and an exec-mask switch per
  // load, and this loop is bound by instruction issue).
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
  // called for tiles 0, 1, 2, ... in order: the trackers advance one tile per call
  auto lstore = [&](const uint4 (&rk)[T::CPT], const uint4 (&rv)[T::CPT], int buf) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int u = tid + T::NT * i;
      const int t = u / T::UPR;
      const int s = t * T::UPR + (cu ^ unit_swizzle<T::UPR>(t));
      float f[8];
      unpack_bf16x8(relu_bf16x8(rk[i]), f);
#pragma unroll
      for (int j = 0; j < 8; ++j) zacc[j] += f[j];
      // rows past the split are zero and stay zero
      const RopePos p = trk[i].pos();
      trk[i].advance(rg, tstep);
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rope_turn<false>(rope_turns(rope_axis_pos<D>(p, 4 * cu + e), fq[e]), f[2 * e],
                         f[2 * e + 1]);
        split_bf16x2(f[2 * e], f[2 * e + 1], &h[e], &l[e]);
      }
      lds[buf][0][s] = make_uint4(h[0], h[1], h[2], h[3]);
      lds[buf][1][s] = make_uint4(l[0], l[1], l[2], l[3]);
      lds[buf][2][s] = rv[i];
    }
  };
  auto compute = [&](int buf) {
    const uint16_t* lh = reinterpret_cast<const uint16_t*>(lds[buf][0]);
    const uint16_t* ll = reinterpret_cast<const uint16_t*>(lds[buf][1]);
    const uint16_t* lv = reinterpret_cast<const uint16_t*>(lds[buf][2]);
#pragma unroll
    for (int ks = 0; ks < T::TT; ks += 32) {
      uint4 ah[NR], al[NR], b[NC];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        ah[r] = tile_column8<T::UPR>(lh, ks, wi * BR + r * 16, lane);
        al[r] = tile_column8<T::UPR>(ll, ks, wi * BR + r * 16, lane);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) b[c] = tile_column8<T::UPR>(lv, ks, wj * BC + c * 16, lane);
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          acc[r][c] = mfma_16x16x32(ah[r], b[c], acc[r][c]);
          acc[r][c] = mfma_16x16x32(al[r], b[c], acc[r][c]);
        }
    }
  };

  // the buffer schedule of kv_partial_bf16
  const int ntiles = t1 > t0 ? (t1 - t0 + T::TT - 1) / T::TT : 0;
  if (ntiles > 0) gload(rk0, rv0, 0);
  if (ntiles > 1) gload(rk1, rv1, 1);
  for (int it = 0; it < ntiles; it += 2) {
    lstore(rk0, rv0, 0);
    lds_barrier();
    if (it + 2 < ntiles) gload(rk0, rv0, it + 2);
    compute(0);
    if (it + 1 < ntiles) {
      lstore(rk1, rv1, 1);
      lds_barrier();
      if (it + 3 < ntiles) gload(rk1, rv1, it + 3);
      compute(1);
    }
  }

  // z: the threads of one column hold disjoint token rows
  lds_barrier();  // every wave is past its last LDS read
  float* zl = reinterpret_cast<float*>(&lds[0][0][0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) zl[tid * 8 + j] = zacc[j];
  lds_barrier();

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
  if (tid < D) {
    const int c = tid / 8, e = tid % 8;
    float zs = 0.f;
    for (int r = 0; r < T::NT / T::UPR; ++r) zs += zl[(r * T::UPR + c) * 8 + e];
    if (si) zs = si[D * D + tid] + zs;
    o[D * D + tid] = zs;
  }
}

// ---------------------------------------------------------------------------
// Readout with rotated queries (bfloat16 inputs) over the persistent work
// items of readout_items_bf16, at every d.  Per tile each lane turns its
// row's eight features per k-step (four pairs) by the token's angles and
// splits them into bf16 hi/lo; the numerator takes three MFMAs per operand
// (hi x S_hi, hi x S_lo, lo x S_hi) and the denominator the unrotated
// phi(q) against z as before.  The pair frequencies sit in LDS.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256, readout_items_min_waves<D>()) void readout_rope_bf16(
    const uint16_t* __restrict__ q, const float* __restrict__ states, void* __restrict__ out,
    int N, int TB, int nblk, int S, int items, float eps, RopeGrid rg) {
  using Sh = RowTile<D>;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, GRP = Sh::GRP, UPR = Sh::UPR;
  constexpr int TT = Sh::TT;
  constexpr int E = D * D + D;
  constexpr int OE = OUT_BF16 ? 2 : 4;
  __shared__ uint4 scol[Sh::NF][kWave];   // columns of S, hi/lo
  __shared__ uint4 zfrag[KS * 2][kWave];  // z in every column, hi/lo
  __shared__ float2 ftab[D / 2];          // pair frequencies, hi/lo

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);
  // read only after the first item's barriers
  if (tid < D / 2) ftab[tid] = rope_freq<D>(tid, rg.theta);
  // a lane's token moves S tiles per step of an item
  const RopeStep tstep = rope_step(rg, S * TT);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const RowItem w = row_item(item, S, nblk, N, TB, TT);
    const size_t bh = w.pair / nblk;
    const float* st = states + w.pair * E;
    const size_t row0 = bh * static_cast<size_t>(N);
    const uint4* qb = reinterpret_cast<const uint4*>(q + row0 * D);
    auto tile_base = [&](int j) { return w.c0 + (w.split + j * S) * TT; };
    auto row_token = [&](int j) { return min(tile_base(j) + 16 * wave + sig, w.c1 - 1); };

    uint4 qa0[KS], qa1[KS];
    // rows past the block (and prefetches past the item) load its last row
    auto gload = [&](int j, uint4 (&qa)[KS]) {
      const int tc = row_token(j);
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[s] = qb[static_cast<size_t>(tc) * UPR + 4 * s + g];
    };
    // the lane's row position for tiles 0, 1, 2, ... of the item (unclamped:
    // rows past the block are never stored)
    RopeTrack trk;
    trk.init(rg, tile_base(0) + 16 * wave + sig);
    if (w.mine > 0) {
      gload(0, qa0);
      gload(1, qa1);
    }

    lds_barrier();  // the previous item's LDS readers are done
    build_col_frags<D>(st, scol, wave, lane);
    if (wave < KS) {
      const float* zp = st + D * D + 32 * wave + 8 * g;
      uint32_t h[4], l[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) split_bf16x2(zp[j], zp[j + 1], &h[j / 2], &l[j / 2]);
      zfrag[2 * wave][lane] = make_uint4(h[0], h[1], h[2], h[3]);
      zfrag[2 * wave + 1][lane] = make_uint4(l[0], l[1], l[2], l[3]);
    }
    lds_barrier();

    auto tile = [&](int j, uint4 (&qa)[KS]) {
      asm volatile("" ::: "memory");
      const int tb = tile_base(j);
      const rsrc_t ro = tile_rsrc(out, (row0 + tb) * D, OE, max(0, min(TT, w.c1 - tb)) * D * OE);
      const RopePos pp = trk.pos();
      trk.advance(rg, tstep);
      uint4 qp[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) qp[s] = relu_bf16x8(qa[s]);
      gload(j + 2, qa);
      uint4 rh[KS], rl[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float f[8];
        unpack_bf16x8(qp[s], f);
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * s + 4 * g + e;
          rope_turn<false>(rope_turns(rope_axis_pos<D>(pp, m), ftab[m]), f[2 * e], f[2 * e + 1]);
          split_bf16x2(f[2 * e], f[2 * e + 1], &h[e], &l[e]);
        }
        rh[s] = make_uint4(h[0], h[1], h[2], h[3]);
        rl[s] = make_uint4(l[0], l[1], l[2], l[3]);
      }
      f32x4 accz = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 acc[NBK];
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        accz = mfma_16x16x32(qp[s], zfrag[2 * s][lane], accz);
        accz = mfma_16x16x32(qp[s], zfrag[2 * s + 1][lane], accz);
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) {
          const int f = 2 * (s * NBK + nb);
          const uint4 sh = scol[f][lane];
          acc[nb] = mfma_16x16x32(rh[s], sh, acc[nb]);
          acc[nb] = mfma_16x16x32(rh[s], scol[f + 1][lane], acc[nb]);
          acc[nb] = mfma_16x16x32(rl[s], sh, acc[nb]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float inv = fast_rcp(accz[i] + eps);
        const int tt = 16 * wave + 4 * i + g;  // row within the tile
#pragma unroll
        for (int gr = 0; gr < GRP; ++gr) {
          float x[W];
#pragma unroll
          for (int e = 0; e < W; ++e) x[e] = acc[gr * W + e][i] * inv;
          store_row_buf<W, OUT_BF16, true>(ro, (tt * D + 16 * W * gr + W * n) * OE, x);
        }
      }
    };
    for (int j = 0; j < w.mine; j += 2) {
      tile(j, qa0);
      tile(j + 1, qa1);
    }
  }
}

// ---------------------------------------------------------------------------
// float32 inputs: the VALU kernels of the plain path with the rotation in
// their staging (sincospif).  Grids and partial layout as kv_partial_f32
// and readout_f32.
template <int D>
__global__ __launch_bounds__(kBlock) void kv_partial_rope_f32(const float* __restrict__ k,
                                                              const float* __restrict__ v, int N,
                                                              int T, int splits, int tps,
                                                              const float* state_in, float* dst,
                                                              RopeGrid rg) {
  constexpr int TT = 16;
  constexpr int E = D * D + D;
  constexpr int PER = D * D / kBlock;
  static_assert(D * D % kBlock == 0 && D <= kBlock, "shape");
  __shared__ float sk[TT * D];  // rotated phi(k)
  __shared__ float su[TT * D];  // phi(k)
  __shared__ float sv[TT * D];
  __shared__ float2 ftab[D / 2];

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
  if (tid < D / 2) ftab[tid] = rope_freq<D>(tid, rg.theta);

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float accz = 0.f;

  for (int base = t0; base < t1; base += TT) {
    __syncthreads();  // ftab written; the previous tile's readers are done
    for (int e2 = tid; e2 < TT * D / 2; e2 += kBlock) {
      const int t = e2 / (D / 2), m = e2 % (D / 2);
      float x = 0.f, y = 0.f, vx = 0.f, vy = 0.f;
      if (base + t < t1) {
        const size_t idx = static_cast<size_t>(base) * D + 2 * e2;
        x = kb[idx];
        y = kb[idx + 1];
        vx = vb[idx];
        vy = vb[idx + 1];
      }
      x = x > 0.f ? x : 0.f;
      y = y > 0.f ? y : 0.f;
      su[2 * e2] = x;
      su[2 * e2 + 1] = y;
      rope_turn<true>(rope_turns(rope_axis_pos<D>(rope_pos(rg, base + t), m), ftab[m]), x, y);
      sk[2 * e2] = x;
      sk[2 * e2 + 1] = y;
      sv[2 * e2] = vx;
      sv[2 * e2 + 1] = vy;
    }
    __syncthreads();
    for (int t = 0; t < TT; ++t) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid + kBlock * i;
        acc[i] = fmaf(sk[t * D + e / D], sv[t * D + e % D], acc[i]);
      }
      if (tid < D) accz += su[t * D + tid];
    }
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

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kBlock) void readout_rope_f32(const float* __restrict__ q,
                                                           const float* __restrict__ state,
                                                           void* __restrict__ out, int N, int T,
                                                           int nblk, int tpw, float eps,
                                                           RopeGrid rg) {
  constexpr int TT = 32;
  constexpr int E = D * D + D;
  extern __shared__ float smem[];
  float* sS = smem;                                     // E
  float* sq = smem + E;                                 // TT * D, rotated phi(q)
  float* su = sq + TT * D;                              // TT * D, phi(q)
  float* sden = su + TT * D;                            // TT
  float2* ftab = reinterpret_cast<float2*>(sden + TT);  // D / 2

  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int per = gridDim.x / nblk;
  const int blk = blockIdx.x / per;
  const int tb = blk * T + (blockIdx.x - blk * per) * tpw;
  const int te = min(min(N, (blk + 1) * T), tb + tpw);
  const int tid = threadIdx.x;
  const float* st = state + (bh * nblk + blk) * E;
  for (int e = tid; e < E; e += kBlock) sS[e] = st[e];
  if (tid < D / 2) ftab[tid] = rope_freq<D>(tid, rg.theta);
  const float* qb = q + bh * static_cast<size_t>(N) * D;

  for (int base = tb; base < te; base += TT) {
    __syncthreads();
    for (int e2 = tid; e2 < TT * D / 2; e2 += kBlock) {
      const int t = e2 / (D / 2), m = e2 % (D / 2);
      float x = 0.f, y = 0.f;
      if (base + t < te) {
        x = qb[static_cast<size_t>(base) * D + 2 * e2];
        y = qb[static_cast<size_t>(base) * D + 2 * e2 + 1];
      }
      x = x > 0.f ? x : 0.f;
      y = y > 0.f ? y : 0.f;
      su[2 * e2] = x;
      su[2 * e2 + 1] = y;
      rope_turn<true>(rope_turns(rope_axis_pos<D>(rope_pos(rg, base + t), m), ftab[m]), x, y);
      sq[2 * e2] = x;
      sq[2 * e2 + 1] = y;
    }
    __syncthreads();
    if (tid < TT) {
      float den = 0.f;
      for (int a = 0; a < D; ++a) den = fmaf(su[tid * D + a], sS[D * D + a], den);
      sden[tid] = den + eps;
    }
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D, c = e % D;
      if (base + t >= te) continue;
      float num = 0.f;
      for (int a = 0; a < D; ++a) num = fmaf(sq[t * D + a], sS[a * D + c], num);
      const float o = num / sden[t];
      const size_t idx = (bh * N + base + t) * static_cast<size_t>(D) + c;
      if constexpr (OUT_BF16)
        static_cast<uint16_t*>(out)[idx] = to_bf16(o);
      else
        static_cast<float*>(out)[idx] = o;
    }
  }
}

template <int D>
constexpr size_t readout_rope_f32_smem() {
  return sizeof(float) * (D * D + D + 2 * 32 * D + 32 + D);
}

}  // namespace la
