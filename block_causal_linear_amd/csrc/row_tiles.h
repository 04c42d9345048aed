// Row-tile building blocks shared by the kernels that take 16 tokens per
// wavefront as MFMA rows (v_mfma_f32_16x16x32_bf16, lane l holding row l % 16
// and k-range 8 (l / 16) .. + 7 of a 32-feature step): the accumulator column
// placement, operand fragments of a d x d float32 matrix as bf16 hi/lo pairs,
// row-bounded buffer stores, and the persistent work-item split.
#pragma once

#include "la_common.h"

namespace la {

template <int D>
struct RowTile {
  static constexpr int KS = D / 32;            // 32-feature k-steps
  static constexpr int NBK = D / 16;           // 16-column accumulator blocks
  static constexpr int W = D == 32 ? 2 : 4;    // values per vector store
  static constexpr int GRP = NBK / W;          // vector stores per token row
  static constexpr int UPR = D / 8;            // 16-byte units per bf16 token row
  static constexpr int TT = 64;                // tokens per tile: 16 per wave
  static constexpr int NT = 4 * kWave;         // four waves
  static constexpr int BR = D / 2;             // d x d block of one wave in a 2 x 2 grid
  static constexpr int NR = BR / 16;
  static constexpr int NF = KS * NBK * 2;      // operand fragments of one d x d matrix
};

// Accumulator column n of block nb holds feature 16 W (nb / W) + W n + nb % W
// (the readout's placement): each lane owns W consecutive features per
// group, so one vector store per (token, group) writes them, and the 16
// lanes of a row group cover 16 W consecutive features.
template <int D>
__device__ __forceinline__ int acc_col(int nb, int n) {
  constexpr int W = RowTile<D>::W;
  return 16 * W * (nb / W) + W * n + nb % W;
}

// MFMA B operand "rows of X": B[k = c][n] = X[acc_col(nb, n)][32 s + c] for
// the products sum_c X[a][c] y[c] with y in the A operand (tokens x c).
// frag[(s NBK + nb) 2 + {hi, lo}][lane]; the four waves share the work.
template <int D>
__device__ void build_row_frags(const float* X, uint4 (*frag)[kWave], int wave, int lane) {
  using Sh = RowTile<D>;
  const int n = lane & 15, g = lane >> 4;
  for (int p = wave; p < Sh::KS * Sh::NBK; p += 4) {
    const int s = p / Sh::NBK, nb = p % Sh::NBK;
    const float* src = X + acc_col<D>(nb, n) * D + 32 * s + 8 * g;
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    uint32_t h[4], l[4];
    split_bf16x2(x0.x, x0.y, &h[0], &l[0]);
    split_bf16x2(x0.z, x0.w, &h[1], &l[1]);
    split_bf16x2(x1.x, x1.y, &h[2], &l[2]);
    split_bf16x2(x1.z, x1.w, &h[3], &l[3]);
    frag[2 * p][lane] = make_uint4(h[0], h[1], h[2], h[3]);
    frag[2 * p + 1][lane] = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

// MFMA B operand "columns of X": B[k = a][n] = X[32 s + a][acc_col(nb, n)]
// for the products sum_a x[a] X[a][c] with x in the A operand (tokens x a).
// A lane needs eight rows of one column per fragment, but the W column
// blocks nb = W q .. W q + W - 1 place lane n's columns side by side
// (acc_col = 16 W q + W n + nb % W), so one W-float vector load per row
// serves W fragments: the waves take (k-step, group) units and issue 8
// vector loads per unit instead of 8 scalar loads per fragment.
template <int D>
__device__ void build_col_frags(const float* X, uint4 (*frag)[kWave], int wave, int lane) {
  using Sh = RowTile<D>;
  constexpr int W = Sh::W;
  typedef float vecW __attribute__((ext_vector_type(W)));
  const int n = lane & 15, g = lane >> 4;
  for (int u = wave; u < Sh::KS * Sh::GRP; u += 4) {
    const int s = u / Sh::GRP, q = u % Sh::GRP;
    const float* src = X + (32 * s + 8 * g) * D + 16 * W * q + W * n;
    vecW x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const vecW*>(src + j * D);
#pragma unroll
    for (int e = 0; e < W; ++e) {
      const int p = s * Sh::NBK + W * q + e;
      uint32_t h[4], l[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) split_bf16x2(x[j][e], x[j + 1][e], &h[j / 2], &l[j / 2]);
      frag[2 * p][lane] = make_uint4(h[0], h[1], h[2], h[3]);
      frag[2 * p + 1][lane] = make_uint4(l[0], l[1], l[2], l[3]);
    }
  }
}

// The same fragments with one scalar load per value: fewer live registers
// during the build.  The key-gradient kernels, which build two operand sets
// per item at four waves per SIMD, spill less with it (372 against 374 us
// per key kernel at the 720p chunk); the readouts gain from the vector loads.
template <int D>
__device__ void build_col_frags_scalar(const float* X, uint4 (*frag)[kWave], int wave, int lane) {
  using Sh = RowTile<D>;
  const int n = lane & 15, g = lane >> 4;
  for (int p = wave; p < Sh::KS * Sh::NBK; p += 4) {
    const int s = p / Sh::NBK, nb = p % Sh::NBK;
    const float* src = X + (32 * s + 8 * g) * D + acc_col<D>(nb, n);
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = src[j * D];
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) split_bf16x2(x[j], x[j + 1], &h[j / 2], &l[j / 2]);
    frag[2 * p][lane] = make_uint4(h[0], h[1], h[2], h[3]);
    frag[2 * p + 1][lane] = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

// Eight bfloat16 values, all zero except element c (0 <= c < 8), which is
// 1.0; all zero for any other c.
__device__ __forceinline__ uint4 onehot_bf16x8(int c) {
  const uint32_t one = (c & 1) ? 0x3F800000u : 0x00003F80u;
  const int w = c >> 1;
  return make_uint4(w == 0 ? one : 0u, w == 1 ? one : 0u, w == 2 ? one : 0u, w == 3 ? one : 0u);
}

// The wave's A-operand rows (16 tokens x d features, bf16, lane (n, g) holding
// row n, features 32 s + 8 g .. + 7) re-expressed in the accumulator layout:
// x[nb][i] = A[4 g + i][acc_col(nb, n)].  Each is an MFMA against a one-hot
// B operand, so every output is one product with 1.0 plus zeros: exact.
// This gives the epilogue the inputs' values where it needs them without
// reading them from memory a second time.
template <int D>
__device__ __forceinline__ void rows_to_acc(const uint4 (&a)[RowTile<D>::KS],
                                            f32x4 (&x)[RowTile<D>::NBK], int lane) {
  using Sh = RowTile<D>;
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nb = 0; nb < Sh::NBK; ++nb) {
    x[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int f = acc_col<D>(nb, n);
    // features of block nb: 16 W (nb / W) + [0, 16 W), i.e. k-steps s0 .. s1
    constexpr int SPAN = 16 * Sh::W / 32;
    const int s0 = (16 * Sh::W * (nb / Sh::W)) / 32;
#pragma unroll
    for (int e = 0; e < SPAN; ++e) {
      const int s = s0 + e;
      x[nb] = mfma_16x16x32(a[s], onehot_bf16x8(f - 32 * s - 8 * g), x[nb]);
    }
  }
}

// Sum over the 16 lanes of each row of a wavefront (lanes 16 g .. 16 g + 15),
// every lane receiving its row's sum: DPP quad permutations (xor 1, xor 2),
// then the half-row mirror (lane i <- 7 - i) and the row mirror
// (i <- 15 - i), each adding the other half of what is summed so far.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float t) {
  t += dpp_f32<0xB1>(t);   // quad_perm [1, 0, 3, 2]
  t += dpp_f32<0x4E>(t);   // quad_perm [2, 3, 0, 1]
  t += dpp_f32<0x141>(t);  // row_half_mirror
  t += dpp_f32<0x140>(t);  // row_mirror
  return t;
}

// Rows of a tile are stored (and, where a kernel says so, loaded) through a
// raw buffer descriptor that covers the tile's valid rows only: the hardware
// drops stores past num_records and returns zero for loads past it, so the
// rows past the end of a block need no branch (a branch around stores makes
// the compiler wait for every outstanding load, prefetches included).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Cache-policy bit 1 of a buffer access: non-temporal (data used once).
constexpr int kBufNt = 2;

// The descriptor of `bytes` bytes from element `elem_off` of `base`.  The
// base, offset and size must be the same in every lane of the wave: they are
// taken through readfirstlane so that the descriptor stays in scalar
// registers.  Built inside a loop without it, the compiler could carry the
// descriptor in vector registers and wrap every access in a loop over its
// distinct values (four readfirstlanes, two compares and two exec-mask
// switches per access, even when all lanes agree).
__device__ __forceinline__ rsrc_t tile_rsrc(const void* base, size_t elem_off, int elem_size,
                                            int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base) + elem_off * elem_size;
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  // word 3: 32-bit data format, as raw (untyped) buffer accesses expect
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// W values at byte offset `off` of a tile descriptor (float32 or bfloat16).
// NT: the non-temporal cache policy (the kernel never reads the rows back).
// Time it by whole calls, not one kernel's time: plain stores leave dirty
// lines that drain during whatever kernel runs next.
template <int W, bool BF16, bool NT>
__device__ __forceinline__ void store_row_buf(rsrc_t r, int off, const float (&x)[W]) {
  constexpr int AUX = NT ? kBufNt : 0;
  if constexpr (BF16) {
    if constexpr (W == 4) {
      __builtin_amdgcn_raw_buffer_store_b64(
          u32x2{pack2(to_bf16(x[0]), to_bf16(x[1])), pack2(to_bf16(x[2]), to_bf16(x[3]))}, r,
          off, 0, AUX);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(pack2(to_bf16(x[0]), to_bf16(x[1])), r, off, 0, AUX);
    }
  } else {
    if constexpr (W == 4) {
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                __float_as_uint(x[3])},
          r, off, 0, AUX);
    } else {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(x[0]), __float_as_uint(x[1])},
                                            r, off, 0, AUX);
    }
  }
}

// Eight consecutive dO values of one token (float32 or bfloat16 in HBM).
template <bool BF16>
struct DoRow;
template <>
struct DoRow<false> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};
template <>
struct DoRow<true> {
  uint4 u;
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
};

// ---------------------------------------------------------------------------
// Work items of the persistent row-tile kernels.  Block c of (b, h) is cut into S
// items; item (b, h, c, s) takes the block's 64-token tiles s, s + S,
// s + 2 S, ...  A persistent grid takes items blockIdx.x, + gridDim.x, ...
// (items are numbered ((b H + h) C + c) S + s): at any moment the running
// items cover whole groups of S items of a few heads, so the workgroups of a
// head sweep adjacent tiles together, and the host picks S so that the item
// count is a multiple of the grid where it can.
struct RowItem {
  size_t pair;  // (b H + h) C + c
  int split;
  int c0, c1;   // the block's token range
  int mine;     // tiles of this item
};

__device__ __forceinline__ RowItem row_item(int item, int S, int nblk, int N, int TB, int TT) {
  RowItem w;
  w.pair = static_cast<size_t>(item / S);
  w.split = item - static_cast<int>(w.pair) * S;
  const int blk = static_cast<int>(w.pair % nblk);
  w.c0 = blk * TB;
  w.c1 = min(N, w.c0 + TB);
  const int ntb = w.c1 > w.c0 ? (w.c1 - w.c0 + TT - 1) / TT : 0;
  w.mine = w.split < ntb ? (ntb - w.split + S - 1) / S : 0;
  return w;
}

}  // namespace la
