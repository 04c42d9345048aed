// Gradients of the block-causal form (the global form is one block), for
// training with the same attention the model samples with ("SANA-Video:
// Efficient Video Generation with Block Linear Diffusion Transformer",
// abstract; "Nvidia, MIT ve diğerleri video yapay zeka devrimini
// başlattı", section "Sabit Bellekli KV önbelleğe alma mekanizması").
//
// The forward, per (b, h): S_n = S_0 + KV_1 + ... + KV_n (z_n likewise) and
// o_i = phi(q_i)^T S_n / (phi(q_i) . z_n + eps) for the queries of block n.
// For an upstream gradient dO (and optionally dS_n, dz_n on every block's
// state) the chain rule gives, with den_i = phi(q_i) . z_n + eps:
//   w_i    = S_n do_i                      (d)
//   t_i    = phi(q_i) . w_i                (= do_i . num_i)
//   dq_i   = (w_i - (t_i / den_i) z_n) / den_i * [q_i > 0]
//   G_n    = sum_i phi(q_i) (do_i / den_i)^T,  g_n = sum_i (-t_i / den_i^2) phi(q_i)
//   R_m    = sum_{n >= m} (G_n + dS_n),        r_m likewise (suffix over blocks)
//   dk_j   = (R_m v_j + r_m) * [k_j > 0],      dv_j = R_m^T phi(k_j)
//   dS_0   = R_1,  dz_0 = r_1.
// The derivative of max(x, 0) is taken as 0 at x = 0.
//
// Three launches: bwd_query (dQ and the per-split partials of (G_n, g_n)),
// state_suffix_scan (R_m from the partials), bwd_key (dK, dV).
#pragma once

#include "la_common.h"
#include "kv_reduce.h"
#include "row_tiles.h"

namespace la {

// Unit swizzle of the query kernel's token-major LDS tiles.  Its writes come
// from the MFMA A layout: the eight lanes of a 16-byte store instruction
// hold tokens 4 r + m' of the wave's sixteen (r = lane / 4 in {0, 1},
// m' = lane % 4), i.e. rows t = 4 m + r with four values of m and two of r.
// XORing the unit of row t = 4 m + r with 2 (r ^ 2 ((m >> 1) & 1)) + (m & 1)
// sends those eight rows to eight different 16-byte columns, and keeps the
// four consecutive rows of a transposing read (one m, r = 0..3) on four
// different 32-byte column pairs.
template <int UPR>
__device__ __forceinline__ int bwd_swizzle(int t) {
  const int r = t & 3, m = t >> 2;
  return (2 * (r ^ (2 * ((m >> 1) & 1))) + (m & 1)) & (UPR - 1);
}

// ---------------------------------------------------------------------------
// bwd_query_bf16: dQ and the partials of (G_n, g_n), bfloat16 queries.  Item
// (b, h, c, s) writes its partial to dst[item] (d*d floats of G, then d of g).
//
// Per 64-token tile, four waves:
//  1. wave w takes tokens 16 w .. 16 w + 15 as MFMA rows (A row m holds token
//     4 (m % 4) + m / 4, so each store instruction writes 4 consecutive
//     token rows): den from phi(Q) against z, w_i from dO (bf16 hi/lo) against
//     S (hi/lo, "rows of S"); phi(Q) rows go to an LDS tile (token-major,
//     swizzled) and come back in the accumulator layout; in the epilogue
//     t_i is a 16-lane DPP sum, dq is formed and stored, and dden goes to
//     LDS;
//  2. each lane fetches 1/den of its own A row from the lanes that formed
//     it (wave shuffles), scales its dO and writes dnum as a bf16 hi/lo
//     pair into two more LDS tiles;
//  3. after a barrier the waves accumulate G (2 x 2 blocks of d/2 x d/2) over
//     the tile's tokens with transposing LDS reads, as the KV reduction
//     does; waves in block column 0 also accumulate g against dden.
// The LDS tiles and dden are double-buffered, so one barrier per tile
// suffices: a wave writes tile i + 1's buffers only after the barrier of
// tile i, which every wave reaches after its step 3 of tile i - 1, the last
// reader of those buffers.  At d = 128 (LDS too small for two dnum tiles)
// the dnum tiles are single and a second barrier before step 2 keeps tile
// i + 1's writes behind every wave's step 3 of tile i.  A barrier at the
// start of every item separates it from the previous item's LDS use.
// Waves per SIMD each kernel is compiled for (its launch bound); with four
// waves per workgroup this is also the number of resident workgroups per CU
// (LDS permitting: 23 / 53 / 137 KB per workgroup at d = 32 / 64 / 128),
// which sizes the persistent grid.
#ifndef LA_BWDQ_WAVES64
#define LA_BWDQ_WAVES64 2  // query kernel waves per SIMD at d = 64
#endif
#ifndef LA_BWDQ_PF64
#define LA_BWDQ_PF64 2     // query kernel prefetch stages at d = 64
#endif
#ifndef LA_BWDQ_DNB64
#define LA_BWDQ_DNB64 2    // query kernel dnum tile buffers at d = 64
#endif
#ifndef LA_BWDQ_WAVES32
// query kernel waves per SIMD at d = 32: at four it spills 100 B per lane,
// ~26 MB over the resident waves; three need no spill slots
#define LA_BWDQ_WAVES32 3
#endif
template <int D>
constexpr int bwd_query_min_waves() {
  return D == 128 ? 1 : D == 64 ? LA_BWDQ_WAVES64 : LA_BWDQ_WAVES32;
}

template <int D, bool GO_BF16>
__global__ __launch_bounds__(256, bwd_query_min_waves<D>()) void bwd_query_bf16(
    const uint16_t* __restrict__ q, const void* __restrict__ dout,
    const float* __restrict__ states, void* __restrict__ dq, int N, int TB, int nblk, int S,
    int items, float eps, float* __restrict__ dst) {
  using Sh = RowTile<D>;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, GRP = Sh::GRP, UPR = Sh::UPR;
  constexpr int TT = Sh::TT, BR = Sh::BR, NR = Sh::NR;
  constexpr int E = D * D + D;
  constexpr int UNITS = TT * UPR;
  __shared__ uint4 sfrag[Sh::NF][kWave];  // rows of S, hi/lo
  __shared__ uint4 zfrag[KS * 2][kWave];  // z in every column, hi/lo
  constexpr int DNB = D == 128 ? 1 : D == 64 ? LA_BWDQ_DNB64 : 2;  // dnum tile buffers
  __shared__ uint4 qt[2][UNITS];          // phi(Q) tile, two buffers
  __shared__ uint4 dnh[DNB][UNITS], dnl[DNB][UNITS];
  __shared__ float sdd[2][TT];
  __shared__ float zsh[D];                // z, for the epilogue

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);
  const int wi = wave >> 1, wj = wave & 1;
  const int ta = 16 * wave + sig;  // this lane's A row within a tile

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const RowItem w = row_item(item, S, nblk, N, TB, TT);
    const size_t bh = w.pair / nblk;
    const float* st = states + w.pair * E;
    const uint4* qb = reinterpret_cast<const uint4*>(q + bh * static_cast<size_t>(N) * D);
    const size_t row0 = bh * static_cast<size_t>(N);
    auto tile_base = [&](int k) { return w.c0 + (w.split + k * S) * TT; };

    // PF register stages: while tile k is processed, the loads of tiles
    // k + 1 .. k + PF are in flight (one stage at d = 128, where registers
    // are short).  Rows past the block load its last row again; their
    // 1/den is set to 0 in the epilogue, which makes their dnum and dden
    // exactly 0 (no contribution to G or g), and their dq stores fall
    // outside the tile's descriptor.  (Zeroing them in registers instead
    // would put a divergent branch, and the waits it brings, in the loop.)
    constexpr int PF = D == 128 ? 1 : D == 64 ? LA_BWDQ_PF64 : 2;
    uint4 qa0[KS], qa1[KS];
    DoRow<GO_BF16> da0[KS], da1[KS];
    auto gload = [&](int k, uint4 (&qa)[KS], DoRow<GO_BF16> (&da)[KS]) {
      const int tc = min(tile_base(k) + ta, w.c1 - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qa[s] = qb[static_cast<size_t>(tc) * UPR + 4 * s + g];
        da[s].load(dout, (row0 + tc) * D + 32 * s + 8 * g);
      }
    };
    if (w.mine > 0) {
      gload(0, qa0, da0);
      if (PF == 2) gload(1, qa1, da1);
    }

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

    f32x4 accG[NR][NR], accg[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      accg[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NR; ++c) accG[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    lds_barrier();

    auto tile = [&](int k, uint4 (&qa)[KS], DoRow<GO_BF16> (&da)[KS]) {
      const int buf = k & 1;
      const int base = tile_base(k);
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
      gload(k + PF, qa, da);

      // 1. phi(Q) rows to the tile; den and w on MFMA
#pragma unroll
      for (int s = 0; s < KS; ++s) qt[buf][ta * UPR + ((4 * s + g) ^ bwd_swizzle<UPR>(ta))] = qp[s];
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
      // phi(Q) in the accumulator layout, for t_i and the mask: read back
      // from the tile rows this wave has just written (its own rows only;
      // a wavefront's LDS operations complete in order, the fences keep the
      // compiler from moving the reads above the writes)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      f32x4 qacc[NBK];
      {
        const uint16_t* lq = reinterpret_cast<const uint16_t*>(qt[buf]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 16 * wave + 4 * i + g;
#pragma unroll
          for (int gr = 0; gr < GRP; ++gr) {
            const int f = 16 * W * gr + W * n;
            const uint16_t* pq =
                lq + (tt * UPR + ((f >> 3) ^ bwd_swizzle<UPR>(tt))) * 8 + (f & 7);
            float x[W];
            if constexpr (W == 4) {
              const uint2 u = *reinterpret_cast<const uint2*>(pq);
              x[0] = __uint_as_float(u.x << 16);
              x[1] = __uint_as_float(u.x & 0xFFFF0000u);
              x[2] = __uint_as_float(u.y << 16);
              x[3] = __uint_as_float(u.y & 0xFFFF0000u);
            } else {
              const uint32_t u = *reinterpret_cast<const uint32_t*>(pq);
              x[0] = __uint_as_float(u << 16);
              x[1] = __uint_as_float(u & 0xFFFF0000u);
            }
#pragma unroll
            for (int e = 0; e < W; ++e) qacc[gr * W + e][i] = x[e];
          }
        }
      }
      // epilogue: rows 4 g + i hold tokens 4 i + g of the wave's sixteen
      float rdv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 16 * wave + 4 * i + g;
        const int tok = base + tt;  // rows past the block are dropped by rdq
        float t = 0.f;
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) t = fmaf(qacc[nb][i], accw[nb][i], t);
        t = row16_sum(t);
        // rows past the block: rd = 0 (see the loads above)
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
          // non-temporal (see the key kernel's stores)
          store_row_buf<W, GO_BF16, true>(rdq, (tt * D + 16 * W * gr + W * n) * GE, x);
        }
        if (n == 0) sdd[buf][tt] = -c * rd;
      }
      if constexpr (DNB == 1) lds_barrier();

      // 2. dnum = dO / den as a bf16 hi/lo pair, token-major.  This lane's
      // A row, token 4 (n % 4) + n / 4, is row n % 4 of lane group n / 4.
      {
        const int src = 16 * (n >> 2) + n;
        const float r0 = __shfl(rdv[0], src), r1 = __shfl(rdv[1], src);
        const float r2 = __shfl(rdv[2], src), r3 = __shfl(rdv[3], src);
        const int ri = n & 3;
        const float rd = ri == 0 ? r0 : ri == 1 ? r1 : ri == 2 ? r2 : r3;
        const int db = DNB == 2 ? buf : 0;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          uint32_t h[4], l[4];
#pragma unroll
          for (int j = 0; j < 8; j += 2)
            split_bf16x2(dv[s][j] * rd, dv[s][j + 1] * rd, &h[j / 2], &l[j / 2]);
          const int u = ta * UPR + ((4 * s + g) ^ bwd_swizzle<UPR>(ta));
          dnh[db][u] = make_uint4(h[0], h[1], h[2], h[3]);
          dnl[db][u] = make_uint4(l[0], l[1], l[2], l[3]);
        }
      }
      lds_barrier();

      // 3. G += phi(Q)^T dnum, g += phi(Q)^T dden over the tile's tokens
      const uint16_t* lq = reinterpret_cast<const uint16_t*>(qt[buf]);
      const uint16_t* lh = reinterpret_cast<const uint16_t*>(dnh[DNB == 2 ? buf : 0]);
      const uint16_t* ll = reinterpret_cast<const uint16_t*>(dnl[DNB == 2 ? buf : 0]);
#pragma unroll
      for (int ks = 0; ks < TT; ks += 32) {
        uint4 a[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) a[r] = tile_column8<UPR, bwd_swizzle<UPR>>(lq, ks, wi * BR + 16 * r, lane);
#pragma unroll
        for (int c = 0; c < NR; ++c) {
          const uint4 bh16 = tile_column8<UPR, bwd_swizzle<UPR>>(lh, ks, wj * BR + 16 * c, lane);
          const uint4 bl16 = tile_column8<UPR, bwd_swizzle<UPR>>(ll, ks, wj * BR + 16 * c, lane);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            accG[r][c] = mfma_16x16x32(a[r], bh16, accG[r][c]);
            accG[r][c] = mfma_16x16x32(a[r], bl16, accG[r][c]);
          }
        }
        if (wj == 0) {
          uint4 ddh = make_uint4(0, 0, 0, 0), ddl = make_uint4(0, 0, 0, 0);
          if (n == 0) {
            const float* pp = &sdd[buf][ks + 8 * g];
            uint32_t h[4], l[4];
#pragma unroll
            for (int j = 0; j < 8; j += 2) split_bf16x2(pp[j], pp[j + 1], &h[j / 2], &l[j / 2]);
            ddh = make_uint4(h[0], h[1], h[2], h[3]);
            ddl = make_uint4(l[0], l[1], l[2], l[3]);
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            accg[r] = mfma_16x16x32(a[r], ddh, accg[r]);
            accg[r] = mfma_16x16x32(a[r], ddl, accg[r]);
          }
        }
      }
    };
    // Every call and every prefetch is unconditional, so the two register
    // stages stay in fixed registers (conditional ones make the compiler
    // shuffle registers that are still being loaded, and wait for them).
    // With an odd tile count the last call is a tile past the block: all
    // its rows have rd = 0, so it adds exactly zero to G and g, and its
    // descriptor covers no bytes.  Its loads (and the prefetches past the
    // end) read the block's last row.
    for (int k = 0; k < w.mine; k += PF) {
      tile(k, qa0, da0);
      if constexpr (PF == 2) tile(k + 1, qa1, da1);
    }

    float* o = dst + static_cast<size_t>(item) * E;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NR; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[(wi * BR + 16 * r + 4 * g + i) * D + wj * BR + 16 * c + n] = accG[r][c][i];
    if (wj == 0 && n == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[D * D + wi * BR + 16 * r + 4 * g + i] = accg[r][i];
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_key_bf16: dK and dV, bfloat16 keys and values.  For each item the
// workgroup builds two operand sets of R_c in LDS ("rows of R" and "columns
// of R"); each wave takes 16 tokens of every tile as MFMA rows:
//   dphi(k) = v R^T + r  (A = v, B = rows of R),
//   dv      = phi(k) R   (A = phi(k), B = columns of R),
// masks dphi(k) with phi(k) moved to the accumulator layout by one-hot
// MFMAs, and stores both with the readout's 4-token-row store pattern.  No
// barrier inside an item.
// (LDS: 8 / 32 / 128 KB per workgroup at d = 32 / 64 / 128)
#ifndef LA_BWDK_WAVES64
#define LA_BWDK_WAVES64 4  // key kernel waves per SIMD at d = 64
#endif
#ifndef LA_BWDK_PF
#define LA_BWDK_PF 1       // key kernel prefetch stages
#endif
template <int D>
constexpr int bwd_key_min_waves() {
  return D == 128 ? 1 : D == 64 ? LA_BWDK_WAVES64 : 6;
}

template <int D, bool GO_BF16>
__global__ __launch_bounds__(256, bwd_key_min_waves<D>()) void bwd_key_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ R,
    void* __restrict__ dk, void* __restrict__ dv, int N, int TB, int nblk, int S, int items) {
  using Sh = RowTile<D>;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, GRP = Sh::GRP, UPR = Sh::UPR;
  constexpr int TT = Sh::TT;
  constexpr int E = D * D + D;
  __shared__ uint4 rrow[Sh::NF][kWave];
  __shared__ uint4 rcol[Sh::NF][kWave];
  __shared__ float rsh[D];  // r, for the epilogue

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const RowItem w = row_item(item, S, nblk, N, TB, TT);
    const size_t bh = w.pair / nblk;
    const float* rs = R + w.pair * E;
    const size_t row0 = bh * static_cast<size_t>(N);
    const uint4* kb = reinterpret_cast<const uint4*>(k + row0 * D);
    const uint4* vb = reinterpret_cast<const uint4*>(v + row0 * D);
    // this wave's 16 tokens of tile j of the item
    auto wave_base = [&](int j) { return w.c0 + (w.split + j * S) * TT + 16 * wave; };
    // PF register stages of the wave's next tiles; loads past the item read
    // the block's last row (unused)
    constexpr int PF = LA_BWDK_PF;
    uint4 ka0[KS], va0[KS], ka1[KS], va1[KS];
    auto gload = [&](int j, uint4 (&ka)[KS], uint4 (&va)[KS]) {
      const int tc = min(wave_base(j) + sig, w.c1 - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[s] = kb[static_cast<size_t>(tc) * UPR + 4 * s + g];
        va[s] = vb[static_cast<size_t>(tc) * UPR + 4 * s + g];
      }
    };
    if (w.mine > 0) {
      gload(0, ka0, va0);
      if (PF == 2) gload(1, ka1, va1);
    }

    lds_barrier();  // the previous item's LDS readers are done
    build_row_frags<D>(rs, rrow, wave, lane);
    build_col_frags_scalar<D>(rs, rcol, wave, lane);
    if (tid < D) rsh[tid] = rs[D * D + tid];
    lds_barrier();

    auto step = [&](int j, uint4 (&ka)[KS], uint4 (&va)[KS]) {
      // read the operand fragments from LDS where they are used instead of
      // holding all of them in registers across the loop
      asm volatile("" ::: "memory");
      // the tile's valid rows; stores past them are dropped (rows past the
      // block hold copies of its last row: every row is independent here)
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
      gload(j + PF, ka, va);
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
          accv[nb] = mfma_16x16x32(kp[s], rcol[f][lane], accv[nb]);
          accv[nb] = mfma_16x16x32(kp[s], rcol[f + 1][lane], accv[nb]);
        }
      // phi(K) in the accumulator layout (exact): its sign is the mask
      f32x4 kacc[NBK];
      rows_to_acc<D>(kp, kacc, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 16 * wave + 4 * i + g;  // row within the tile
#pragma unroll
        for (int gr = 0; gr < GRP; ++gr) {
          float xk[W], xv[W];
          const int col = 16 * W * gr + W * n;
#pragma unroll
          for (int e = 0; e < W; ++e) {
            const int nb = gr * W + e;
            // r read outside the select: with the LDS read inside one arm
            // the compiler branched around it (an exec-mask switch per value)
            const float r = rsh[col + e];
            const float gk = acck[nb][i] + r;
            xk[e] = kacc[nb][i] > 0.f ? gk : 0.f;
            xv[e] = accv[nb][i];
          }
          // non-temporal: by itself this kernel measures slower with it at
          // d = 64 (378 -> 390 us), but its write-back lines otherwise drain
          // during the next kernel on the stream; per backward call at the
          // 720p chunk: 726 us with non-temporal stores in both kernels,
          // 733 us with plain stores here
          store_row_buf<W, GO_BF16, true>(rdk, (tt * D + col) * GE, xk);
          store_row_buf<W, GO_BF16, true>(rdv, (tt * D + col) * GE, xv);
        }
      }
    };
    // unconditional pairs when PF = 2 (a step past the item stores nothing)
    for (int j = 0; j < w.mine; j += PF) {
      step(j, ka0, va0);
      if constexpr (PF == 2) step(j + 1, ka1, va1);
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_key_sweep_bf16: the same dK and dV on the forward readout's sweep
// schedule (bf16 keys and values, d <= 64).  A unit is four wave tiles of RB
// 16-token row blocks inside one block; step j of workgroup w takes unit
// w + j G, so the whole grid moves through the (b, h, block, token) space
// together, one narrow window of keys, values and gradients at a time (runs
// of two consecutive units per step, which the forward readout takes on
// short blocks, measured slower here: 1,782 against 1,693 us per call on the
// 480p stream in one call).  The two operand
// sets of R (rows and columns, bf16 hi/lo) and r are rebuilt only when a
// step's block differs from the last one, from slices of R that each wave
// loads one step ahead into registers, into one of two LDS buffers; a
// barrier at every step keeps the workgroup's four waves on one unit.  Per
// token the arithmetic, down to the order of the MFMAs into each
// accumulator, is that of bwd_key_bf16: the results are bitwise equal.
// (LDS: 16 / 64 KB per workgroup at d = 32 / 64.)
#ifndef LA_BWDK_SWEEP_ROWS
#define LA_BWDK_SWEEP_ROWS 2  // 16-token row blocks per wave tile
#endif
template <int D>
struct KeySweep {
  static constexpr int RB = LA_BWDK_SWEEP_ROWS;
  static constexpr int TILE = 16 * RB;   // tokens per wave tile
  static constexpr int UNIT = 4 * TILE;  // tokens per unit
  static constexpr int MIN_WAVES = 2;    // waves per SIMD = workgroups per CU
};

template <int D, bool GO_BF16>
__global__ __launch_bounds__(256, KeySweep<D>::MIN_WAVES) void bwd_key_sweep_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ R,
    void* __restrict__ dk, void* __restrict__ dv, int N, int T, int nblk, int units_per_block,
    int total_units) {
  static_assert(D <= 64, "the key sweep is built for d <= 64");
  using Sh = RowTile<D>;
  using Kw = KeySweep<D>;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, GRP = Sh::GRP, UPR = Sh::UPR;
  constexpr int RB = Kw::RB, TILE = Kw::TILE;
  constexpr int E = D * D + D;
  constexpr int NF = Sh::NF;
  constexpr int GE = GO_BF16 ? 2 : 4;
  constexpr int PAIRS = KS * NBK;                  // (k-step, column block) pairs
  constexpr int PW = PAIRS >= 4 ? PAIRS / 4 : 1;   // pairs per producer wave
  static_assert(PAIRS % PW == 0 && NBK % PW == 0 && W % PW == 0, "pair split");
  using vecP = float __attribute__((ext_vector_type(PW)));
  __shared__ uint4 rrow[2][NF][kWave];  // rows of R, hi/lo
  __shared__ uint4 rcol[2][NF][kWave];  // columns of R, hi/lo
  __shared__ float rsh[2][D];           // r

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);

  // this wave's pairs: k-step ps, column blocks pc0 .. pc0 + PW - 1 (adjacent
  // columns of one store group, acc_col)
  const bool producer = wave * PW < PAIRS;
  const int p0 = producer ? wave * PW : 0;
  const int ps = p0 / NBK, pc0 = p0 % NBK;

  float4 rraw[PW][2];  // rows of R: 8 consecutive values of row acc_col(nb, n)
  vecP craw[8];        // columns of R: rows 32 ps + 8 g + j, PW adjacent columns
  float rval = 0.f;
  auto load_r = [&](int sb) {  // sb = (b H + h) nblk + block
    const float* rs = R + static_cast<size_t>(sb) * E;
    if (producer) {
#pragma unroll
      for (int c = 0; c < PW; ++c) {
        const float* src = rs + acc_col<D>(pc0 + c, n) * D + 32 * ps + 8 * g;
        rraw[c][0] = *reinterpret_cast<const float4*>(src);
        rraw[c][1] = *reinterpret_cast<const float4*>(src + 4);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        craw[j] = *reinterpret_cast<const vecP*>(rs + (32 * ps + 8 * g + j) * D +
                                                 acc_col<D>(pc0, n));
    }
    if (tid < D) rval = rs[D * D + tid];
  };
  auto build = [&](int buf) {
    if (producer) {
#pragma unroll
      for (int c = 0; c < PW; ++c) {
        const int p = ps * NBK + pc0 + c;
        uint32_t h[4], l[4];
        split_bf16x2(rraw[c][0].x, rraw[c][0].y, &h[0], &l[0]);
        split_bf16x2(rraw[c][0].z, rraw[c][0].w, &h[1], &l[1]);
        split_bf16x2(rraw[c][1].x, rraw[c][1].y, &h[2], &l[2]);
        split_bf16x2(rraw[c][1].z, rraw[c][1].w, &h[3], &l[3]);
        rrow[buf][2 * p][lane] = make_uint4(h[0], h[1], h[2], h[3]);
        rrow[buf][2 * p + 1][lane] = make_uint4(l[0], l[1], l[2], l[3]);
#pragma unroll
        for (int j = 0; j < 8; j += 2) split_bf16x2(craw[j][c], craw[j + 1][c], &h[j / 2], &l[j / 2]);
        rcol[buf][2 * p][lane] = make_uint4(h[0], h[1], h[2], h[3]);
        rcol[buf][2 * p + 1][lane] = make_uint4(l[0], l[1], l[2], l[3]);
      }
    }
    if (tid < D) rsh[buf][tid] = rval;
  };
  // Rows past the end of the block load its last row (their outputs are never
  // stored: every output row depends on its own input row only).
  auto load_kv = [&](uint4 (&ka)[RB][KS], uint4 (&va)[RB][KS], int bh, int t0, int te) {
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint4* kb = reinterpret_cast<const uint4*>(k + row0 * D);
    const uint4* vb = reinterpret_cast<const uint4*>(v + row0 * D);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int tok = min(t0 + 16 * r + sig, te - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[r][s] = kb[static_cast<size_t>(tok) * UPR + 4 * s + g];
        va[r][s] = vb[static_cast<size_t>(tok) * UPR + 4 * s + g];
      }
    }
  };
  auto consume = [&](int buf, const uint4 (&ka)[RB][KS], const uint4 (&va)[RB][KS], int bh,
                     int t0, int te) {
    // the wave tile's rows inside the block; stores past them are dropped
    const int valid = max(0, min(TILE, te - t0));
    const size_t e0 = (static_cast<size_t>(bh) * N + t0) * D;
    const rsrc_t rdk = tile_rsrc(dk, e0, GE, valid * D * GE);
    const rsrc_t rdv = tile_rsrc(dv, e0, GE, valid * D * GE);
    // each operand fragment read from LDS serves the RB row blocks
    uint4 kp[RB][KS];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int s = 0; s < KS; ++s) kp[r][s] = relu_bf16x8(ka[r][s]);
    f32x4 acck[RB][NBK], accv[RB][NBK];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) {
        acck[r][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        accv[r][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) {
        const int f = 2 * (s * NBK + nb);
        const uint4 rh = rrow[buf][f][lane], rl = rrow[buf][f + 1][lane];
        const uint4 ch = rcol[buf][f][lane], cl = rcol[buf][f + 1][lane];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          acck[r][nb] = mfma_16x16x32(va[r][s], rh, acck[r][nb]);
          acck[r][nb] = mfma_16x16x32(va[r][s], rl, acck[r][nb]);
          accv[r][nb] = mfma_16x16x32(kp[r][s], ch, accv[r][nb]);
          accv[r][nb] = mfma_16x16x32(kp[r][s], cl, accv[r][nb]);
        }
      }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      f32x4 kacc[NBK];
      rows_to_acc<D>(kp[r], kacc, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 16 * r + 4 * i + g;  // row within the wave tile
#pragma unroll
        for (int gr = 0; gr < GRP; ++gr) {
          float xk[W], xv[W];
          const int col = 16 * W * gr + W * n;
#pragma unroll
          for (int e = 0; e < W; ++e) {
            const int nb = gr * W + e;
            const float rr = rsh[buf][col + e];
            const float gk = acck[r][nb][i] + rr;
            xk[e] = kacc[nb][i] > 0.f ? gk : 0.f;
            xv[e] = accv[r][nb][i];
          }
          store_row_buf<W, GO_BF16, true>(rdk, (tt * D + col) * GE, xk);
          store_row_buf<W, GO_BF16, true>(rdv, (tt * D + col) * GE, xv);
        }
      }
    }
  };

  // unit -> (b, h), block, this wave's tile, end of the block
  auto locate = [&](int u, int& bh, int& sb, int& t0, int& te) {
    const int upb = units_per_block;
    bh = u / (nblk * upb);
    const int rem = u - bh * nblk * upb;
    const int blk = rem / upb;
    sb = bh * nblk + blk;
    t0 = blk * T + ((rem - blk * upb) * 4 + wave) * TILE;
    te = min(N, (blk + 1) * T);
  };
  // The unit index is uniform across the workgroup: every wave takes the
  // same barriers, and waves whose tile lies past the block store nothing.
  int unit = blockIdx.x;
  if (unit >= total_units) return;
  int bh, sb, t0, te;
  locate(unit, bh, sb, t0, te);
  uint4 ka[RB][KS], va[RB][KS];
  load_r(sb);
  load_kv(ka, va, bh, t0, te);
  int built = -1;  // the block whose operands the current buffer holds
  int buf = 1;
  for (;;) {
    // buffer buf ^ 1 was last read before the previous build's barrier,
    // which every wave has passed
    if (sb != built) {
      buf ^= 1;
      build(buf);
      built = sb;
    }
    lds_barrier();
    const int next = unit + static_cast<int>(gridDim.x);
    const bool more = next < total_units;
    const int nu = more ? next : unit;
    int nbh, nsb, nt0, nte;
    locate(nu, nbh, nsb, nt0, nte);
    uint4 kn[RB][KS], vn[RB][KS];
    if (nsb != sb) load_r(nsb);
    load_kv(kn, vn, nbh, nt0, nte);
    consume(buf, ka, va, bh, t0, te);
    if (!more) break;
    unit = next;
    bh = nbh;
    sb = nsb;
    t0 = nt0;
    te = nte;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[r][s] = kn[r][s];
        va[r][s] = vn[r][s];
      }
  }
}

// ---------------------------------------------------------------------------
// float32 inputs: plain VALU versions of the two kernels above (the float32
// path is for exactness checks and small problems).  Same grids and outputs.
template <int D, bool GO_BF16>
__global__ __launch_bounds__(kBlock) void bwd_query_f32(const float* __restrict__ q,
                                                        const void* __restrict__ dout,
                                                        const float* __restrict__ states,
                                                        void* __restrict__ dq, int N, int TB,
                                                        int splits, int tps, float eps,
                                                        float* __restrict__ dst) {
  constexpr int TT = 16;
  constexpr int E = D * D + D;
  constexpr int PER = D * D / kBlock;
  static_assert(D * D % kBlock == 0 && D <= kBlock, "shape");
  extern __shared__ float smem[];
  float* sS = smem;              // E
  float* sq = sS + E;            // TT x D: phi(q)
  float* sd = sq + TT * D;       // TT x D: dO, then dnum
  float* sw = sd + TT * D;       // TT x D: w
  float* srd = sw + TT * D;      // TT: 1/den
  float* sc = srd + TT;          // TT: t / den

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
  const size_t row0 = bh * static_cast<size_t>(N);

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float accz = 0.f;

  for (int base = t0; base < t1; base += TT) {
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D;
      float x = 0.f, y = 0.f;
      if (base + t < t1) {
        const size_t idx = (row0 + base) * D + e;
        x = q[idx];
        y = GO_BF16 ? from_bf16(static_cast<const uint16_t*>(dout)[idx])
                    : static_cast<const float*>(dout)[idx];
      }
      sq[e] = x > 0.f ? x : 0.f;
      sd[e] = y;
    }
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D, a = e % D;
      float w = 0.f;
      for (int c = 0; c < D; ++c) w = fmaf(sS[a * D + c], sd[t * D + c], w);
      sw[e] = w;
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
      for (int t = 0; t < TT; ++t) x = fmaf(sq[t * D + a], sd[t * D + c], x);
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
constexpr size_t bwd_query_f32_smem() {
  return sizeof(float) * (D * D + D + 3 * 16 * D + 2 * 16);
}

template <int D, bool GO_BF16>
__global__ __launch_bounds__(kBlock) void bwd_key_f32(const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      const float* __restrict__ R,
                                                      void* __restrict__ dk, void* __restrict__ dv,
                                                      int N, int TB, int splits, int tps) {
  constexpr int TT = 16;
  constexpr int E = D * D + D;
  extern __shared__ float smem[];
  float* sR = smem;            // E
  float* sk = sR + E;          // TT x D: k (raw)
  float* sv = sk + TT * D;     // TT x D: v

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
  const size_t row0 = bh * static_cast<size_t>(N);

  for (int base = t0; base < t1; base += TT) {
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D;
      float x = 0.f, y = 0.f;
      if (base + t < t1) {
        x = k[(row0 + base) * D + e];
        y = v[(row0 + base) * D + e];
      }
      sk[e] = x;
      sv[e] = y;
    }
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D, a = e % D;
      if (base + t >= t1) continue;
      float gk = sR[D * D + a], gv = 0.f;
      for (int c = 0; c < D; ++c) gk = fmaf(sR[a * D + c], sv[t * D + c], gk);
      for (int b = 0; b < D; ++b) gv = fmaf(fmaxf(sk[t * D + b], 0.f), sR[b * D + a], gv);
      gk = sk[e] > 0.f ? gk : 0.f;
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
constexpr size_t bwd_key_f32_smem() {
  return sizeof(float) * (D * D + D + 2 * 16 * D);
}

}  // namespace la
