// Gradients of the RoPE'd block-causal form (rope.h states the forward and
// the reading behind it).  With q~ = R phi(q), k~ = R phi(k), R a token's
// rotation and R^T the turn by the opposite angles, the chain rule gives,
// for block n (state S_n, z_n; den_i = phi(q_i) . z_n + eps):
//   u_i = R_i^T (S_n do_i),  t_i = phi(q_i) . u_i  (= do_i . num_i)
//   dq_i = (u_i - (t_i / den_i) z_n) / den_i * [q_i > 0]
//   dS_n += sum_i q~_i (do_i / den_i)^T,  dz_n += sum_i (-t_i / den_i^2) phi(q_i)
// and for block m with the suffix sums G_m, g_m of those (plus the caller's
// state gradients):
//   dk_j = (R_j^T (G_m v_j) + g_m) * [k_j > 0],  dv_j = G_m^T k~_j.
// The kernels follow the plain backward's (backward.h) grids, item split and
// partial layout; the suffix over blocks (state_suffix_scan) is shared.
#pragma once

#include "la_common.h"
#include "kv_reduce.h"
#include "row_tiles.h"
#include "rope_math.h"
#include "backward.h"

namespace la {

// Pair (x, y) turned back by 2 pi t (the transpose of rope_turn's rotation).
template <bool PRECISE>
__device__ __forceinline__ void rope_turn_back(float t, float& x, float& y) {
  float s, c;
  rope_sincos<PRECISE>(t, s, c);
  const float x1 = x * c + y * s;
  y = y * c - x * s;
  x = x1;
}

// ---------------------------------------------------------------------------
// float32 inputs: the plain float32 kernels with rotations in their staging.
// Grids and partial layout as bwd_query_f32 / bwd_key_f32.
template <int D, bool GO_BF16>
__global__ __launch_bounds__(kBlock) void bwd_query_rope_f32(const float* __restrict__ q,
                                                             const void* __restrict__ dout,
                                                             const float* __restrict__ states,
                                                             void* __restrict__ dq, int N, int TB,
                                                             int splits, int tps, float eps,
                                                             float* __restrict__ dst,
                                                             RopeGrid rg) {
  constexpr int TT = 16;
  constexpr int E = D * D + D;
  constexpr int PER = D * D / kBlock;
  static_assert(D * D % kBlock == 0 && D <= kBlock, "shape");
  extern __shared__ float smem[];
  float* sS = smem;                                     // E
  float* sq = sS + E;                                   // TT x D: phi(q)
  float* sr = sq + TT * D;                              // TT x D: R phi(q)
  float* sd = sr + TT * D;                              // TT x D: dO, then dnum
  float* sw = sd + TT * D;                              // TT x D: S dO, then u = R^T S dO
  float* srd = sw + TT * D;                             // TT: 1/den
  float* sc = srd + TT;                                 // TT: t / den
  float2* ftab = reinterpret_cast<float2*>(sc + TT);    // D / 2

  const int nblk = gridDim.x / splits;
  const int blk = blockIdx.x / splits;
  const int split = blockIdx.x - blk * splits;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int c0 = blk * TB;
  const int c1 = min(N, c0 + TB);
  const int t0 = c0 + split * tps;
  const int t1 = min(c1, t0 + tps);
  const int tid = threadIdx.x;
  const float* st = states + (bh * nblk + blk) * E;
  for (int e = tid; e < E; e += kBlock) sS[e] = st[e];
  if (tid < D / 2) ftab[tid] = rope_freq<D>(tid, rg.theta);
  const size_t row0 = bh * static_cast<size_t>(N);

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float accz = 0.f;

  for (int base = t0; base < t1; base += TT) {
    __syncthreads();
    for (int e2 = tid; e2 < TT * D / 2; e2 += kBlock) {
      const int t = e2 / (D / 2), m = e2 % (D / 2);
      float x = 0.f, y = 0.f, dx = 0.f, dy = 0.f;
      if (base + t < t1) {
        const size_t idx = (row0 + base) * D + 2 * e2;
        x = q[idx];
        y = q[idx + 1];
        dx = GO_BF16 ? from_bf16(static_cast<const uint16_t*>(dout)[idx])
                     : static_cast<const float*>(dout)[idx];
        dy = GO_BF16 ? from_bf16(static_cast<const uint16_t*>(dout)[idx + 1])
                     : static_cast<const float*>(dout)[idx + 1];
      }
      x = x > 0.f ? x : 0.f;
      y = y > 0.f ? y : 0.f;
      sq[2 * e2] = x;
      sq[2 * e2 + 1] = y;
      rope_turn<true>(rope_turns(rope_axis_pos<D>(rope_pos(rg, base + t), m), ftab[m]), x, y);
      sr[2 * e2] = x;
      sr[2 * e2 + 1] = y;
      sd[2 * e2] = dx;
      sd[2 * e2 + 1] = dy;
    }
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D, a = e % D;
      float w = 0.f;
      for (int c = 0; c < D; ++c) w = fmaf(sS[a * D + c], sd[t * D + c], w);
      sw[e] = w;
    }
    __syncthreads();
    for (int e2 = tid; e2 < TT * D / 2; e2 += kBlock) {
      const int t = e2 / (D / 2), m = e2 % (D / 2);
      float x = sw[2 * e2], y = sw[2 * e2 + 1];
      rope_turn_back<true>(rope_turns(rope_axis_pos<D>(rope_pos(rg, base + t), m), ftab[m]), x,
                           y);
      sw[2 * e2] = x;
      sw[2 * e2 + 1] = y;
    }
    __syncthreads();
    if (tid < TT) {
      float den = 0.f, t = 0.f;
      for (int a = 0; a < D; ++a) {
        den = fmaf(sq[tid * D + a], sS[D * D + a], den);
        t = fmaf(sq[tid * D + a], sw[tid * D + a], t);
      }
      const float rd = base + tid < t1 ? 1.f / (den + eps) : 0.f;
      srd[tid] = rd;
      sc[tid] = t * rd;
    }
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D, a = e % D;
      const float rd = srd[t];
      if (base + t < t1) {
        const float gq = sq[e] > 0.f ? (sw[e] - sc[t] * sS[D * D + a]) * rd : 0.f;
        const size_t idx = (row0 + base) * D + e;
        if constexpr (GO_BF16)
          static_cast<uint16_t*>(dq)[idx] = to_bf16(gq);
        else
          static_cast<float*>(dq)[idx] = gq;
      }
      sd[e] *= rd;  // dnum
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + kBlock * i;
      const int a = e / D, c = e % D;
      float x = acc[i];
      for (int t = 0; t < TT; ++t) x = fmaf(sr[t * D + a], sd[t * D + c], x);
      acc[i] = x;
    }
    if (tid < D)
      for (int t = 0; t < TT; ++t) accz = fmaf(-sc[t] * srd[t], sq[t * D + tid], accz);
  }

  float* o = dst + ((bh * nblk + blk) * splits + split) * static_cast<size_t>(E);
#pragma unroll
  for (int i = 0; i < PER; ++i) o[tid + kBlock * i] = acc[i];
  if (tid < D) o[D * D + tid] = accz;
}

template <int D>
constexpr size_t bwd_query_rope_f32_smem() {
  return sizeof(float) * (D * D + D + 4 * 16 * D + 2 * 16 + D);
}

template <int D, bool GO_BF16>
__global__ __launch_bounds__(kBlock) void bwd_key_rope_f32(const float* __restrict__ k,
                                                           const float* __restrict__ v,
                                                           const float* __restrict__ R,
                                                           void* __restrict__ dk,
                                                           void* __restrict__ dv, int N, int TB,
                                                           int splits, int tps, RopeGrid rg) {
  constexpr int TT = 16;
  constexpr int E = D * D + D;
  extern __shared__ float smem[];
  float* sR = smem;                                     // E
  float* sk = sR + E;                                   // TT x D: k (raw)
  float* skr = sk + TT * D;                             // TT x D: R phi(k)
  float* sv = skr + TT * D;                             // TT x D: v
  float* sg = sv + TT * D;                              // TT x D: G v, then R^T G v
  float2* ftab = reinterpret_cast<float2*>(sg + TT * D);  // D / 2

  const int nblk = gridDim.x / splits;
  const int blk = blockIdx.x / splits;
  const int split = blockIdx.x - blk * splits;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int c0 = blk * TB;
  const int c1 = min(N, c0 + TB);
  const int t0 = c0 + split * tps;
  const int t1 = min(c1, t0 + tps);
  const int tid = threadIdx.x;
  const float* rs = R + (bh * nblk + blk) * E;
  for (int e = tid; e < E; e += kBlock) sR[e] = rs[e];
  if (tid < D / 2) ftab[tid] = rope_freq<D>(tid, rg.theta);
  const size_t row0 = bh * static_cast<size_t>(N);

  for (int base = t0; base < t1; base += TT) {
    __syncthreads();
    for (int e2 = tid; e2 < TT * D / 2; e2 += kBlock) {
      const int t = e2 / (D / 2), m = e2 % (D / 2);
      float x = 0.f, y = 0.f, vx = 0.f, vy = 0.f;
      if (base + t < t1) {
        const size_t idx = (row0 + base) * D + 2 * e2;
        x = k[idx];
        y = k[idx + 1];
        vx = v[idx];
        vy = v[idx + 1];
      }
      sk[2 * e2] = x;
      sk[2 * e2 + 1] = y;
      sv[2 * e2] = vx;
      sv[2 * e2 + 1] = vy;
      x = x > 0.f ? x : 0.f;
      y = y > 0.f ? y : 0.f;
      rope_turn<true>(rope_turns(rope_axis_pos<D>(rope_pos(rg, base + t), m), ftab[m]), x, y);
      skr[2 * e2] = x;
      skr[2 * e2 + 1] = y;
    }
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D, a = e % D;
      float gk = 0.f;
      for (int c = 0; c < D; ++c) gk = fmaf(sR[a * D + c], sv[t * D + c], gk);
      sg[e] = gk;
    }
    __syncthreads();
    for (int e2 = tid; e2 < TT * D / 2; e2 += kBlock) {
      const int t = e2 / (D / 2), m = e2 % (D / 2);
      float x = sg[2 * e2], y = sg[2 * e2 + 1];
      rope_turn_back<true>(rope_turns(rope_axis_pos<D>(rope_pos(rg, base + t), m), ftab[m]), x,
                           y);
      sg[2 * e2] = x;
      sg[2 * e2 + 1] = y;
    }
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D, a = e % D;
      if (base + t >= t1) continue;
      float gv = 0.f;
      for (int b = 0; b < D; ++b) gv = fmaf(skr[t * D + b], sR[b * D + a], gv);
      const float gk = sk[e] > 0.f ? sg[e] + sR[D * D + a] : 0.f;
      const size_t idx = (row0 + base) * D + e;
      if constexpr (GO_BF16) {
        static_cast<uint16_t*>(dk)[idx] = to_bf16(gk);
        static_cast<uint16_t*>(dv)[idx] = to_bf16(gv);
      } else {
        static_cast<float*>(dk)[idx] = gk;
        static_cast<float*>(dv)[idx] = gv;
      }
    }
  }
}

template <int D>
constexpr size_t bwd_key_rope_f32_smem() {
  return sizeof(float) * (D * D + D + 4 * 16 * D + D);
}

// Waves per SIMD of the rotary key kernel (its launch bound, and with
// four-wave workgroups its workgroups per CU).  Below the plain kernel's
// bound at d <= 64: the rotation's extra registers would spill, and the
// spill slots of every resident wave together exceed L2, so their reloads
// in the tile loop would go to HBM.
#ifndef LA_ROPE_BWDK_WAVES64
#define LA_ROPE_BWDK_WAVES64 3
#endif
#ifndef LA_ROPE_BWDK_WAVES32
#define LA_ROPE_BWDK_WAVES32 5
#endif
template <int D>
constexpr int bwd_key_rope_min_waves() {
  return D == 128 ? 1 : D == 64 ? LA_ROPE_BWDK_WAVES64 : LA_ROPE_BWDK_WAVES32;
}

// ---------------------------------------------------------------------------
// bwd_key_rope_bf16: dK and dV with rotated keys (bf16 keys and values), the
// structure of bwd_key_bf16.  Per tile each wave takes 16 tokens as MFMA rows:
//   G v_j       = v x (rows of G), turned back per feature pair in the
//                 accumulator layout (a lane holds whole pairs), plus g, and
//                 masked by phi(k) (one-hot MFMAs, exact): dk;
//   G^T k~_j    = k~ x (columns of G), k~ the turned phi(k) as a bf16 hi/lo
//                 A operand (three products): dv.
// Token positions are carried from tile to tile (S tiles per step).
template <int D, bool GO_BF16>
__global__ __launch_bounds__(256, bwd_key_rope_min_waves<D>()) void bwd_key_rope_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ R,
    void* __restrict__ dk, void* __restrict__ dv, int N, int TB, int nblk, int S, int items,
    RopeGrid rg) {
  using Sh = RowTile<D>;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, GRP = Sh::GRP, UPR = Sh::UPR;
  constexpr int TT = Sh::TT;
  constexpr int E = D * D + D;
  static_assert(W % 2 == 0, "a lane holds whole feature pairs");
  __shared__ uint4 rrow[Sh::NF][kWave];
  __shared__ uint4 rcol[Sh::NF][kWave];
  __shared__ float rsh[D];         // g, for the epilogue
  __shared__ float2 ftab[D / 2];   // pair frequencies

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);
  // read only after the first item's barriers
  if (tid < D / 2) ftab[tid] = rope_freq<D>(tid, rg.theta);
  const RopeStep tstep = rope_step(rg, S * TT);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const RowItem w = row_item(item, S, nblk, N, TB, TT);
    const size_t bh = w.pair / nblk;
    const float* rs = R + w.pair * E;
    const size_t row0 = bh * static_cast<size_t>(N);
    const uint4* kb = reinterpret_cast<const uint4*>(k + row0 * D);
    const uint4* vb = reinterpret_cast<const uint4*>(v + row0 * D);
    auto wave_base = [&](int j) { return w.c0 + (w.split + j * S) * TT + 16 * wave; };
    uint4 ka0[KS], va0[KS];
    auto gload = [&](int j, uint4 (&ka)[KS], uint4 (&va)[KS]) {
      const int tc = min(wave_base(j) + sig, w.c1 - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[s] = kb[static_cast<size_t>(tc) * UPR + 4 * s + g];
        va[s] = vb[static_cast<size_t>(tc) * UPR + 4 * s + g];
      }
    };
    if (w.mine > 0) gload(0, ka0, va0);
    // positions of the lane's A row and of its four accumulator rows
    // (unclamped: rows past the block are never stored)
    RopeTrack tra, trc[4];
    tra.init(rg, wave_base(0) + sig);
#pragma unroll
    for (int i = 0; i < 4; ++i) trc[i].init(rg, wave_base(0) + 4 * i + g);

    lds_barrier();  // the previous item's LDS readers are done
    build_row_frags<D>(rs, rrow, wave, lane);
    build_col_frags_scalar<D>(rs, rcol, wave, lane);
    if (tid < D) rsh[tid] = rs[D * D + tid];
    lds_barrier();

    auto step = [&](int j, uint4 (&ka)[KS], uint4 (&va)[KS]) {
      asm volatile("" ::: "memory");
      constexpr int GE = GO_BF16 ? 2 : 4;
      const int tb = w.c0 + (w.split + j * S) * TT;
      const int bytes = max(0, min(TT, w.c1 - tb)) * D * GE;
      const rsrc_t rdk = tile_rsrc(dk, (row0 + tb) * D, GE, bytes);
      const rsrc_t rdv = tile_rsrc(dv, (row0 + tb) * D, GE, bytes);
      uint4 kp[KS], vv[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kp[s] = relu_bf16x8(ka[s]);
        vv[s] = va[s];
      }
      gload(j + 1, ka, va);
      // k~ as hi/lo, from the A row's position
      uint4 rkh[KS], rkl[KS];
      {
        const RopePos pa = tra.pos();
        tra.advance(rg, tstep);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          float f[8];
          unpack_bf16x8(kp[s], f);
          uint32_t h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 16 * s + 4 * g + e;
            rope_turn<false>(rope_turns(rope_axis_pos<D>(pa, m), ftab[m]), f[2 * e],
                             f[2 * e + 1]);
            split_bf16x2(f[2 * e], f[2 * e + 1], &h[e], &l[e]);
          }
          rkh[s] = make_uint4(h[0], h[1], h[2], h[3]);
          rkl[s] = make_uint4(l[0], l[1], l[2], l[3]);
        }
      }
      f32x4 acck[NBK], accv[NBK];
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) {
        acck[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        accv[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) {
          const int f = 2 * (s * NBK + nb);
          acck[nb] = mfma_16x16x32(vv[s], rrow[f][lane], acck[nb]);
          acck[nb] = mfma_16x16x32(vv[s], rrow[f + 1][lane], acck[nb]);
          const uint4 ch = rcol[f][lane];
          accv[nb] = mfma_16x16x32(rkh[s], ch, accv[nb]);
          accv[nb] = mfma_16x16x32(rkh[s], rcol[f + 1][lane], accv[nb]);
          accv[nb] = mfma_16x16x32(rkl[s], ch, accv[nb]);
        }
      // phi(K) in the accumulator layout (exact): its sign is the mask
      f32x4 kacc[NBK];
      rows_to_acc<D>(kp, kacc, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const RopePos pc = trc[i].pos();
        trc[i].advance(rg, tstep);
        const int tt = 16 * wave + 4 * i + g;  // row within the tile
#pragma unroll
        for (int gr = 0; gr < GRP; ++gr) {
          float xk[W], xv[W];
          const int col = 16 * W * gr + W * n;
#pragma unroll
          for (int e = 0; e < W; e += 2) {
            const int nb = gr * W + e;
            const int m = (col + e) / 2;  // the feature pair (col + e, col + e + 1)
            float x = acck[nb][i], y = acck[nb + 1][i];
            rope_turn_back<false>(rope_turns(rope_axis_pos<D>(pc, m), ftab[m]), x, y);
            // the LDS reads outside the selects (inside, the compiler
            // branched around them)
            const float gx = x + rsh[col + e], gy = y + rsh[col + e + 1];
            xk[e] = kacc[nb][i] > 0.f ? gx : 0.f;
            xk[e + 1] = kacc[nb + 1][i] > 0.f ? gy : 0.f;
            xv[e] = accv[nb][i];
            xv[e + 1] = accv[nb + 1][i];
          }
          store_row_buf<W, GO_BF16, true>(rdk, (tt * D + col) * GE, xk);
          store_row_buf<W, GO_BF16, true>(rdv, (tt * D + col) * GE, xv);
        }
      }
    };
    for (int j = 0; j < w.mine; ++j) step(j, ka0, va0);
  }
}

// ---------------------------------------------------------------------------
// bwd_query_rope_bf16: dQ and the per-item partial state gradients with
// rotated queries (bf16 queries), the structure of bwd_query_bf16 with:
//   * the denominators and w = S dO on MFMA as before (unrotated phi(q)
//     against z; dO hi/lo against rows of S);
//   * u = R^T w turned back per feature pair in the accumulator layout, so
//     t_i = phi(q_i) . u_i and dq use the unrotated phi(q), which one-hot
//     MFMAs place in that layout;
//   * dS += q~^T dnum with q~ = R phi(q) as bf16 hi/lo token-major tiles
//     (three products per operand), written after the epilogue's barrier
//     together with the dnum tiles (one buffer each, two barriers a tile);
//   * dz += sum_i dden_i phi(q_i) on the VALU in the accumulator layout,
//     summed over the lane groups and the four waves in a fixed order.
template <int D, bool GO_BF16>
__global__ __launch_bounds__(256, bwd_query_min_waves<D>()) void bwd_query_rope_bf16(
    const uint16_t* __restrict__ q, const void* __restrict__ dout,
    const float* __restrict__ states, void* __restrict__ dq, int N, int TB, int nblk, int S,
    int items, float eps, float* __restrict__ dst, RopeGrid rg) {
  using Sh = RowTile<D>;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, GRP = Sh::GRP, UPR = Sh::UPR;
  constexpr int TT = Sh::TT, BR = Sh::BR, NR = Sh::NR;
  constexpr int E = D * D + D;
  constexpr int UNITS = TT * UPR;
  static_assert(W % 2 == 0, "a lane holds whole feature pairs");
  __shared__ uint4 sfrag[Sh::NF][kWave];  // rows of S, hi/lo
  __shared__ uint4 zfrag[KS * 2][kWave];  // z in every column, hi/lo
  __shared__ uint4 qth[UNITS], qtl[UNITS];  // q~ tile, hi/lo
  __shared__ uint4 dnh[UNITS], dnl[UNITS];  // dnum tile, hi/lo
  __shared__ float zsh[D];                // z, for the epilogue
  __shared__ float gred[4][D];            // per-wave dz sums
  __shared__ float2 ftab[D / 2];          // pair frequencies

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);
  const int wi = wave >> 1, wj = wave & 1;
  const int ta = 16 * wave + sig;  // this lane's A row within a tile
  // read only after the first item's barriers
  if (tid < D / 2) ftab[tid] = rope_freq<D>(tid, rg.theta);
  const RopeStep tstep = rope_step(rg, S * TT);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const RowItem w = row_item(item, S, nblk, N, TB, TT);
    const size_t bh = w.pair / nblk;
    const float* st = states + w.pair * E;
    const uint4* qb = reinterpret_cast<const uint4*>(q + bh * static_cast<size_t>(N) * D);
    const size_t row0 = bh * static_cast<size_t>(N);
    auto tile_base = [&](int kk) { return w.c0 + (w.split + kk * S) * TT; };

    // one register stage; rows past the block load its last row again and
    // get 1/den = 0, so they add nothing and their stores are dropped
    uint4 qa0[KS];
    DoRow<GO_BF16> da0[KS];
    auto gload = [&](int kk, uint4 (&qa)[KS], DoRow<GO_BF16> (&da)[KS]) {
      const int tc = min(tile_base(kk) + ta, w.c1 - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qa[s] = qb[static_cast<size_t>(tc) * UPR + 4 * s + g];
        da[s].load(dout, (row0 + tc) * D + 32 * s + 8 * g);
      }
    };
    if (w.mine > 0) gload(0, qa0, da0);
    // positions of the lane's A row and of its four accumulator rows
    RopeTrack tra, trc[4];
    tra.init(rg, tile_base(0) + ta);
#pragma unroll
    for (int i = 0; i < 4; ++i) trc[i].init(rg, tile_base(0) + 16 * wave + 4 * i + g);

    lds_barrier();  // the previous item's LDS readers are done
    build_row_frags<D>(st, sfrag, wave, lane);
    if (wave < KS) {
      const float* zp = st + D * D + 32 * wave + 8 * g;
      uint32_t h[4], l[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) split_bf16x2(zp[j], zp[j + 1], &h[j / 2], &l[j / 2]);
      zfrag[2 * wave][lane] = make_uint4(h[0], h[1], h[2], h[3]);
      zfrag[2 * wave + 1][lane] = make_uint4(l[0], l[1], l[2], l[3]);
    }
    if (tid < D) zsh[tid] = st[D * D + tid];

    f32x4 accG[NR][NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NR; ++c) accG[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float gacc[NBK];  // dz over this lane's rows, per accumulator column
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) gacc[nb] = 0.f;
    lds_barrier();

    auto tile = [&](int kk, uint4 (&qa)[KS], DoRow<GO_BF16> (&da)[KS]) {
      const int base = tile_base(kk);
      constexpr int GE = GO_BF16 ? 2 : 4;  // gradient element bytes
      const rsrc_t rdq =
          tile_rsrc(dq, (row0 + base) * D, GE, max(0, min(TT, w.c1 - base)) * D * GE);
      uint4 qp[KS];
      float dv[KS][8];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qp[s] = relu_bf16x8(qa[s]);
        da[s].get(dv[s]);
      }
      gload(kk + 1, qa, da);

      // q~ of the A row as hi/lo (stored to the tile after the barrier)
      uint4 rqh[KS], rql[KS];
      {
        const RopePos pa = tra.pos();
        tra.advance(rg, tstep);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          float f[8];
          unpack_bf16x8(qp[s], f);
          uint32_t h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 16 * s + 4 * g + e;
            rope_turn<false>(rope_turns(rope_axis_pos<D>(pa, m), ftab[m]), f[2 * e],
                             f[2 * e + 1]);
            split_bf16x2(f[2 * e], f[2 * e + 1], &h[e], &l[e]);
          }
          rqh[s] = make_uint4(h[0], h[1], h[2], h[3]);
          rql[s] = make_uint4(l[0], l[1], l[2], l[3]);
        }
      }

      // 1. den and w = S dO on MFMA
      f32x4 accz = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 accw[NBK];
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) accw[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        accz = mfma_16x16x32(qp[s], zfrag[2 * s][lane], accz);
        accz = mfma_16x16x32(qp[s], zfrag[2 * s + 1][lane], accz);
        uint32_t h[4], l[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) split_bf16x2(dv[s][j], dv[s][j + 1], &h[j / 2], &l[j / 2]);
        const uint4 ah = make_uint4(h[0], h[1], h[2], h[3]);
        const uint4 al = make_uint4(l[0], l[1], l[2], l[3]);
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) {
          const uint4 bh16 = sfrag[2 * (s * NBK + nb)][lane];
          const uint4 bl16 = sfrag[2 * (s * NBK + nb) + 1][lane];
          accw[nb] = mfma_16x16x32(ah, bh16, accw[nb]);
          accw[nb] = mfma_16x16x32(ah, bl16, accw[nb]);
          if constexpr (!GO_BF16) accw[nb] = mfma_16x16x32(al, bh16, accw[nb]);
        }
      }
      // phi(Q) in the accumulator layout (exact)
      f32x4 qacc[NBK];
      rows_to_acc<D>(qp, qacc, lane);

      // 2. epilogue: u = R^T w, t, dq, and dz on the VALU
      float rdv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const RopePos pc = trc[i].pos();
        trc[i].advance(rg, tstep);
        const int tt = 16 * wave + 4 * i + g;
        const int tok = base + tt;  // rows past the block are dropped by rdq
#pragma unroll
        for (int gr = 0; gr < GRP; ++gr)
#pragma unroll
          for (int e = 0; e < W; e += 2) {
            const int nb = gr * W + e;
            const int m = (16 * W * gr + W * n + e) / 2;
            float x = accw[nb][i], y = accw[nb + 1][i];
            rope_turn_back<false>(rope_turns(rope_axis_pos<D>(pc, m), ftab[m]), x, y);
            accw[nb][i] = x;
            accw[nb + 1][i] = y;
          }
        float t = 0.f;
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) t = fmaf(qacc[nb][i], accw[nb][i], t);
        t = row16_sum(t);
        const float rd = tok < w.c1 ? fast_rcp(accz[i] + eps) : 0.f;
        rdv[i] = rd;
        const float c = t * rd;
#pragma unroll
        for (int gr = 0; gr < GRP; ++gr) {
          float x[W];
#pragma unroll
          for (int e = 0; e < W; ++e) {
            const int nb = gr * W + e;
            const float gq = (accw[nb][i] - c * zsh[acc_col<D>(nb, n)]) * rd;
            x[e] = qacc[nb][i] > 0.f ? gq : 0.f;
          }
          store_row_buf<W, GO_BF16, true>(rdq, (tt * D + 16 * W * gr + W * n) * GE, x);
        }
        const float dden = -c * rd;
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) gacc[nb] = fmaf(qacc[nb][i], dden, gacc[nb]);
      }
      lds_barrier();  // every wave is done with the previous tile's LDS tiles

      // 3. q~ and dnum = dO / den as bf16 hi/lo, token-major.  This lane's A
      // row, token 4 (n % 4) + n / 4, is row n % 4 of lane group n / 4.
      {
        const int src = 16 * (n >> 2) + n;
        const float r0 = __shfl(rdv[0], src), r1 = __shfl(rdv[1], src);
        const float r2 = __shfl(rdv[2], src), r3 = __shfl(rdv[3], src);
        const int ri = n & 3;
        const float rd = ri == 0 ? r0 : ri == 1 ? r1 : ri == 2 ? r2 : r3;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          uint32_t h[4], l[4];
#pragma unroll
          for (int j = 0; j < 8; j += 2)
            split_bf16x2(dv[s][j] * rd, dv[s][j + 1] * rd, &h[j / 2], &l[j / 2]);
          const int u = ta * UPR + ((4 * s + g) ^ bwd_swizzle<UPR>(ta));
          dnh[u] = make_uint4(h[0], h[1], h[2], h[3]);
          dnl[u] = make_uint4(l[0], l[1], l[2], l[3]);
          qth[u] = rqh[s];
          qtl[u] = rql[s];
        }
      }
      lds_barrier();

      // 4. dS += q~^T dnum over the tile's tokens
      const uint16_t* lqh = reinterpret_cast<const uint16_t*>(qth);
      const uint16_t* lql = reinterpret_cast<const uint16_t*>(qtl);
      const uint16_t* lh = reinterpret_cast<const uint16_t*>(dnh);
      const uint16_t* ll = reinterpret_cast<const uint16_t*>(dnl);
#pragma unroll
      for (int ks = 0; ks < TT; ks += 32) {
        uint4 ah[NR], al[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          ah[r] = tile_column8<UPR, bwd_swizzle<UPR>>(lqh, ks, wi * BR + 16 * r, lane);
          al[r] = tile_column8<UPR, bwd_swizzle<UPR>>(lql, ks, wi * BR + 16 * r, lane);
        }
#pragma unroll
        for (int c = 0; c < NR; ++c) {
          const uint4 bh16 = tile_column8<UPR, bwd_swizzle<UPR>>(lh, ks, wj * BR + 16 * c, lane);
          const uint4 bl16 = tile_column8<UPR, bwd_swizzle<UPR>>(ll, ks, wj * BR + 16 * c, lane);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            accG[r][c] = mfma_16x16x32(ah[r], bh16, accG[r][c]);
            accG[r][c] = mfma_16x16x32(ah[r], bl16, accG[r][c]);
            accG[r][c] = mfma_16x16x32(al[r], bh16, accG[r][c]);
          }
        }
      }
    };
    for (int kk = 0; kk < w.mine; ++kk) tile(kk, qa0, da0);

    float* o = dst + static_cast<size_t>(item) * E;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NR; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[(wi * BR + 16 * r + 4 * g + i) * D + wj * BR + 16 * c + n] = accG[r][c][i];
    // dz: the lane groups of a wave, then the four waves, in a fixed order
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
      float x = gacc[nb];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (g == 0) gred[wave][acc_col<D>(nb, n)] = x;
    }
    lds_barrier();
    if (tid < D) o[D * D + tid] = ((gred[0][tid] + gred[1][tid]) + gred[2][tid]) + gred[3][tid];
  }
}

}  // namespace la
