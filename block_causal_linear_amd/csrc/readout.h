// Readout of a block's queries against the updated state:
//   o_i = phi(q_i)^T S / (phi(q_i) . z + eps)
// (sd114.wiki article on SANA-Video, section "1. 线性 DiT": a kernel
// mapping followed by a global aggregation, no N x N matrix; the block reads
// KVsum plus its own KV, "Nvidia, MIT ve diğerleri video yapay zeka devrimini
// başlattı", section "Sabit Bellekli KV önbelleğe alma mekanizması").
#pragma once

#include "la_common.h"
#include "row_tiles.h"

// (Measured at the 720p chunk: non-temporal stores of the output beat plain
// ones, 171-172 us against 174-176 us per readout; plain loads beat
// non-temporal ones; two 16-token row blocks per wave tile beat one or four.)
#ifndef LA_READOUT_STREAM_STORES
#define LA_READOUT_STREAM_STORES 1
#endif
#ifndef LA_READOUT_STREAM_LOADS
#define LA_READOUT_STREAM_LOADS 0
#endif
// 16-token row blocks per wave tile at d <= 64.
#ifndef LA_READOUT_ROWS
#define LA_READOUT_ROWS 2
#endif

namespace la {

// ---------------------------------------------------------------------------
// bfloat16 queries on MFMA 16x16x32.
//
// phi(q) is exact in bfloat16.  The float32 state is split into a pair of
// bfloat16 values S = S_hi + S_lo (S_lo rounds S - S_hi), which carries 16
// significant bits; bf16 x bf16 products are exact in float32, so two MFMAs
// per operand give phi(q)^T S with float32 accumulation and a representation
// error of about 2^-17 relative per state entry.  The denominator phi(q).z
// is a fifth column block whose B operand holds z (hi and lo) in every
// column, so each lane's accumulator already holds the denominator of the
// rows it owns: no cross-lane traffic.
//
// Row and column placement.  A row block is 16 tokens; MFMA row m holds
// token sigma(m) = 4 (m % 4) + m / 4 of the block, so accumulator element i
// of lane l (row 4 (l / 16) + i) is token 4 i + l / 16.  Column n of column
// block nb holds state column pi(nb, n) = 16 W (nb / W) + W n + nb % W, where
// W (4, or 2 when d = 32) values make one vector store.  Together these make
// every store instruction of a wavefront write 4 consecutive tokens' rows
// (1 KB at d = 64, float32) contiguously.

template <int D>
struct ReadoutShape {
  static constexpr int KS = D / 32;              // k-steps of 32 features
  static constexpr int NBK = D / 16;             // 16-column blocks of S
  static constexpr int W = (D == 32) ? 2 : 4;    // values per vector store
  static constexpr int GRP = NBK / W;            // vector stores per token row
  static constexpr int R = (D == 128) ? 2 : LA_READOUT_ROWS;  // 16-token row blocks per wave tile
  static constexpr int TILE = 16 * R;            // tokens per wave tile
  static constexpr int UPR = D / 8;              // 16-byte units per query row
};

__device__ __forceinline__ uint4 load_q(const uint4* p) {
#if LA_READOUT_STREAM_LOADS
  return load_stream(p);
#else
  return *p;
#endif
}

// Sweep readout shape (built for d <= 64 only: at d = 128 the per-unit
// rebuild of a 66 KB state's operands dominated, and readout_items_bf16 reads
// out there).  The NCH = 2 column split below is the layout the sweep had at
// d = 128 and is kept only as the generic form of the template.
template <int D>
struct SweepShape {
  static constexpr int NCH = D == 128 ? 2 : 1;          // column halves
  static constexpr int NW = 4 * NCH;                    // waves per workgroup
  static constexpr int NT = kWave * NW;                 // threads per workgroup
  static constexpr int CB = ReadoutShape<D>::NBK / NCH;  // column blocks per half
  static constexpr int MIN_WAVES = D == 128 ? 2 : 3;
  // Operand buffers in LDS (two: one barrier per unit).
  static constexpr int NBUF = 2;
};

template <int D>
constexpr int sweep_threads() {
  return SweepShape<D>::NT;
}

template <int D>
constexpr int sweep_min_waves() {
  return SweepShape<D>::MIN_WAVES;
}

// A sequence of N tokens per (b, h) may be cut into blocks of T tokens, each
// read against its own state states[(b H + h) nblk + c] (the whole-sequence
// block-causal call); units never straddle a block.  One block: T = N.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(sweep_threads<D>(), sweep_min_waves<D>()) void readout_sweep_bf16(
    const uint16_t* __restrict__ q, const float* __restrict__ state, void* __restrict__ out, int N,
    int T, int nblk, int units_per_block, int total_units, int run_log2, float eps) {
  using Sh = ReadoutShape<D>;
  using Sw = SweepShape<D>;
  constexpr int E = D * D + D;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, R = Sh::R;
  constexpr int NW = Sw::NW, CB = Sw::CB;
  static_assert(CB == W, "a lane stores W consecutive columns, one from each column block");
  constexpr int NF = KS * (NBK + 1) * 2;  // operands: [k-step][column block, z last][hi, lo]
  constexpr int PAIRS = KS * NBK;         // (k-step, column block) pairs
  constexpr int PW = PAIRS >= NW ? PAIRS / NW : 1;  // pairs per wave
  static_assert(PAIRS % PW == 0 && NBK % PW == 0 && PW <= W && CB % W == 0, "pair split");
  using vecP = float __attribute__((ext_vector_type(PW)));
  constexpr int NBUF = Sw::NBUF;
  __shared__ uint4 frag[NBUF][NF][kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int tw = wave % 4;   // tile of the unit
  const int ch = wave / 4;   // column half
  const int n = lane & 15, g = lane >> 4;
  const int tok_a = 4 * (n & 3) + (n >> 2);
  auto fi = [](int s, int c, int p) { return (s * (NBK + 1) + c) * 2 + p; };

  // this wave's pairs: k-step ps, column blocks pc0 .. pc0 + PW - 1
  const bool producer = wave * PW < PAIRS;
  const int p0 = producer ? wave * PW : 0;
  const int ps = p0 / NBK, pc0 = p0 % NBK;

  vecP sraw[8];
  f32x4 zraw[2];
  auto load_state = [&](int sb) {  // sb = (b H + h) nblk + block
    const float* st = state + static_cast<size_t>(sb) * E;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sraw[j] = *reinterpret_cast<const vecP*>(st + (32 * ps + 8 * g + j) * D + 16 * W * (pc0 / W) +
                                                 W * n + pc0 % W);
    zraw[0] = *reinterpret_cast<const f32x4*>(st + D * D + 32 * ps + 8 * g);
    zraw[1] = *reinterpret_cast<const f32x4*>(st + D * D + 32 * ps + 8 * g + 4);
  };
  auto build = [&](int buf) {
    if (!producer) return;
#pragma unroll
    for (int c = 0; c < PW; ++c) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) split_bf16x2(sraw[j][c], sraw[j + 1][c], &h[j / 2], &l[j / 2]);
      frag[buf][fi(ps, pc0 + c, 0)][lane] = make_uint4(h[0], h[1], h[2], h[3]);
      frag[buf][fi(ps, pc0 + c, 1)][lane] = make_uint4(l[0], l[1], l[2], l[3]);
    }
    if (pc0 == 0) {
      uint32_t h[4], l[4];
      split_bf16x2(zraw[0][0], zraw[0][1], &h[0], &l[0]);
      split_bf16x2(zraw[0][2], zraw[0][3], &h[1], &l[1]);
      split_bf16x2(zraw[1][0], zraw[1][1], &h[2], &l[2]);
      split_bf16x2(zraw[1][2], zraw[1][3], &h[3], &l[3]);
      frag[buf][fi(ps, NBK, 0)][lane] = make_uint4(h[0], h[1], h[2], h[3]);
      frag[buf][fi(ps, NBK, 1)][lane] = make_uint4(l[0], l[1], l[2], l[3]);
    }
  };
  // Query rows past the end of the block load its last row instead: an MFMA
  // output row depends only on its own A row, and those rows are never
  // stored.  phi is applied where the operand is used.
  auto load_a = [&](uint4 (&a)[R][KS], int bh, int t0, int te) {
    const uint4* qb = reinterpret_cast<const uint4*>(q + static_cast<size_t>(bh) * N * D);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int tok = min(t0 + 16 * r + tok_a, te - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) a[r][s] = load_q(qb + static_cast<size_t>(tok) * Sh::UPR + 4 * s + g);
    }
  };
  auto consume = [&](int buf, const uint4 (&qraw)[R][KS], int bh, int t0, int te) {
    uint4 a[R][KS];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int s = 0; s < KS; ++s) a[r][s] = relu_bf16x8(qraw[r][s]);
    f32x4 acc[R][CB];
    f32x4 accz[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      accz[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 zh = frag[buf][fi(s, NBK, 0)][lane], zl = frag[buf][fi(s, NBK, 1)][lane];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        accz[r] = mfma_16x16x32(a[r][s], zh, accz[r]);
        accz[r] = mfma_16x16x32(a[r][s], zl, accz[r]);
      }
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int cg = ch * CB + c;
        const uint4 bh16 = frag[buf][fi(s, cg, 0)][lane], bl16 = frag[buf][fi(s, cg, 1)][lane];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r][c] = mfma_16x16x32(a[r][s], bh16, acc[r][c]);
          acc[r][c] = mfma_16x16x32(a[r][s], bl16, acc[r][c]);
        }
      }
    }
    // Rows go out through a descriptor that covers the tile's rows inside the
    // block: the hardware drops the stores past te, so no lane branches (a
    // per-row branch cost an exec-mask switch around every store).
    constexpr int OE = OUT_BF16 ? 2 : 4;
    const int valid = max(0, min(Sh::TILE, te - t0));
    const rsrc_t ro = tile_rsrc(out, (static_cast<size_t>(bh) * N + t0) * D, OE, valid * D * OE);
    const int col = 16 * W * (ch * CB / W) + W * n;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = 16 * r + 4 * i + g;  // row within the wave's tile
        const float inv = fast_rcp(accz[r][i] + eps);
        float o[W];
#pragma unroll
        for (int e = 0; e < W; ++e) o[e] = acc[r][e][i] * inv;
        store_row_buf<W, OUT_BF16, LA_READOUT_STREAM_STORES != 0>(ro, (tt * D + col) * OE, o);
      }
  };

  // The unit index is uniform across the workgroup, so every wave takes the
  // same number of barriers; waves whose tile lies past the end of a head
  // compute on clamped rows and store nothing.
  // unit -> (b, h), block, tile of this wave, end of the block
  auto locate = [&](int u, int& bh, int& sb, int& t0, int& te) {
    const int upb = units_per_block;
    bh = u / (nblk * upb);
    const int rem = u - bh * nblk * upb;
    const int blk = rem / upb;
    sb = bh * nblk + blk;
    t0 = blk * T + ((rem - blk * upb) * 4 + tw) * Sh::TILE;
    te = min(N, (blk + 1) * T);
  };
  // Step j of workgroup w takes unit (w + (j / M) G) M + j % M with
  // M = 2^run_log2: runs of M consecutive units, the runs of all workgroups
  // sweeping together (the planner picks M).  When the next unit reads the
  // same state its operands are neither reloaded nor rebuilt; the workgroup
  // still takes a barrier at every unit, which keeps its four waves on the
  // same unit and so keeps the swept window narrow (without it the waves
  // drift apart and the readout is slower).
  auto unit_of = [&](int j) {
    return ((static_cast<int>(blockIdx.x) + (j >> run_log2) * static_cast<int>(gridDim.x))
            << run_log2) + (j & ((1 << run_log2) - 1));
  };
  int unit = unit_of(0);
  if (unit >= total_units) return;
  int bh, sb, t0, te;
  locate(unit, bh, sb, t0, te);
  uint4 a[R][KS];
  load_state(sb);
  load_a(a, bh, t0, te);
  int built = -1;  // the state whose operands the current buffer holds
  int buf = 1;
  for (int j = 0;; ++j) {
    if (sb != built) {
      buf = NBUF == 2 ? buf ^ 1 : 0;
      // With two buffers, buf was last read before the previous build's
      // barrier; with one, wait until every wave has consumed the last unit.
      if (NBUF == 1 && built >= 0) lds_barrier();
      build(buf);
      lds_barrier();
      built = sb;
    } else {
      lds_barrier();  // the waves stay on one unit (see above)
    }
    const int next = unit_of(j + 1);
    const bool more = next < total_units;
    const int nu = more ? next : unit;
    int nbh, nsb, nt0, nte;
    locate(nu, nbh, nsb, nt0, nte);
    uint4 an[R][KS];
    if (nsb != sb) load_state(nsb);
    load_a(an, nbh, nt0, nte);
    consume(buf, a, bh, t0, te);
    if (!more) break;
    unit = next;
    bh = nbh;
    sb = nsb;
    t0 = nt0;
    te = nte;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int s = 0; s < KS; ++s) a[r][s] = an[r][s];
  }
}

// ---------------------------------------------------------------------------
// Readout over persistent work items (bf16 queries; used at d = 128, where
// the sweep's per-unit rebuild of a 66 KB state's operands costs more than
// it saves).  Block c of (b, h) is cut into S items; a persistent grid
// takes items blockIdx.x, + gridDim.x, ... (row_item).  Per item the
// workgroup builds the state's operands once in LDS, "columns of S" as bf16
// hi/lo pairs and z in every column; each wave then takes 16 tokens of each
// of the item's tiles as MFMA rows (A = phi(Q), loaded two tiles ahead),
// and stores o = num / (den + eps) with the row-bounded buffer stores of the
// backward kernels (rows past the block hold copies of its last row and are
// dropped by the descriptor), so the loop has no branch.
#ifndef LA_READOUT_ITEMS_MIN_D
#define LA_READOUT_ITEMS_MIN_D 128  // smallest d that leaves the sweep readout
#endif

// Waves per SIMD the kernel is compiled for; with four waves per workgroup
// also its resident workgroups per CU (LDS: 72 KB at d = 128, 20 KB at 64).
template <int D>
constexpr int readout_items_min_waves() {
  return D == 128 ? 2 : 4;
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256, readout_items_min_waves<D>()) void readout_items_bf16(
    const uint16_t* __restrict__ q, const float* __restrict__ states, void* __restrict__ out,
    int N, int TB, int nblk, int S, int items, float eps) {
  using Sh = RowTile<D>;
  constexpr int KS = Sh::KS, NBK = Sh::NBK, W = Sh::W, GRP = Sh::GRP, UPR = Sh::UPR;
  constexpr int TT = Sh::TT;
  constexpr int E = D * D + D;
  constexpr int OE = OUT_BF16 ? 2 : 4;
  __shared__ uint4 scol[Sh::NF][kWave];   // columns of S, hi/lo
  __shared__ uint4 zfrag[KS * 2][kWave];  // z in every column, hi/lo

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g = lane >> 4;
  const int sig = 4 * (n & 3) + (n >> 2);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const RowItem w = row_item(item, S, nblk, N, TB, TT);
    const size_t bh = w.pair / nblk;
    const float* st = states + w.pair * E;
    const size_t row0 = bh * static_cast<size_t>(N);
    const uint4* qb = reinterpret_cast<const uint4*>(q + row0 * D);
    auto tile_base = [&](int j) { return w.c0 + (w.split + j * S) * TT; };

    uint4 qa0[KS], qa1[KS];
    // rows past the block (and prefetches past the item) load its last row
    auto gload = [&](int j, uint4 (&qa)[KS]) {
      const int tc = min(tile_base(j) + 16 * wave + sig, w.c1 - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[s] = qb[static_cast<size_t>(tc) * UPR + 4 * s + g];
    };
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
      // read the operands from LDS where they are used instead of holding
      // them in registers across the loop
      asm volatile("" ::: "memory");
      const int tb = tile_base(j);
      const rsrc_t ro = tile_rsrc(out, (row0 + tb) * D, OE, max(0, min(TT, w.c1 - tb)) * D * OE);
      uint4 qp[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) qp[s] = relu_bf16x8(qa[s]);
      gload(j + 2, qa);
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
          acc[nb] = mfma_16x16x32(qp[s], scol[f][lane], acc[nb]);
          acc[nb] = mfma_16x16x32(qp[s], scol[f + 1][lane], acc[nb]);
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
          // non-temporal: 52.5 -> 46.4 us per long-horizon chunk readout
          store_row_buf<W, OUT_BF16, true>(ro, (tt * D + 16 * W * gr + W * n) * OE, x);
        }
      }
    };
    // unconditional pairs: with an odd tile count the last call is a tile
    // past the block, whose stores all fall outside its descriptor
    for (int j = 0; j < w.mine; j += 2) {
      tile(j, qa0);
      tile(j + 1, qa1);
    }
  }
}

// ---------------------------------------------------------------------------
// float32 queries: plain VALU.  The state sits in LDS; each thread owns
// (token, column) outputs of a 32-token tile; the denominators are formed
// once per token.
// Grid: (blocks x workgroups per block, H, B); workgroup x of block c reads
// tokens [c T + x tpw, ...) of the block against states[(b H + h) nblk + c].
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kBlock) void readout_f32(const float* __restrict__ q,
                                                      const float* __restrict__ state,
                                                      void* __restrict__ out, int N, int T,
                                                      int nblk, int tpw, float eps) {
  constexpr int TT = 32;
  constexpr int E = D * D + D;
  extern __shared__ float smem[];
  float* sS = smem;             // E
  float* sq = smem + E;         // TT * D
  float* sden = sq + TT * D;    // TT

  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int per = gridDim.x / nblk;
  const int blk = blockIdx.x / per;
  const int tb = blk * T + (blockIdx.x - blk * per) * tpw;
  const int te = min(min(N, (blk + 1) * T), tb + tpw);
  const int tid = threadIdx.x;
  const float* st = state + (bh * nblk + blk) * E;
  for (int e = tid; e < E; e += kBlock) sS[e] = st[e];
  const float* qb = q + bh * static_cast<size_t>(N) * D;

  for (int base = tb; base < te; base += TT) {
    __syncthreads();
    for (int e = tid; e < TT * D; e += kBlock) {
      const int t = e / D;
      const float x = (base + t < te) ? qb[static_cast<size_t>(base) * D + e] : 0.f;
      sq[e] = x > 0.f ? x : 0.f;
    }
    __syncthreads();
    if (tid < TT) {
      float den = 0.f;
      for (int a = 0; a < D; ++a) den = fmaf(sq[tid * D + a], sS[D * D + a], den);
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
constexpr size_t readout_f32_smem() {
  return sizeof(float) * (D * D + D + 32 * D + 32);
}

}  // namespace la
