// KV reduction of one block: per token split s of every (b, h),
//   P_s = phi(K_s)^T V_s  (d x d)   and   p_s = phi(K_s)^T 1  (d).
// The computation splits along token order with identical results
// ("Nvidia, MIT ve diğerleri video yapay zeka devrimini başlattı", section
// "Sabit Bellekli KV önbelleğe alma mekanizması"), which is what lets many
// workgroups share one head's tokens.
//
// With one split the kernel writes S_out = S_in + P and z_out = z_in + p
// straight into the state; with more, it writes P_s, p_s to a partials
// buffer [B][H][splits][d*d + d] that state_reduce sums in a fixed order.
#pragma once

#include "la_common.h"

namespace la {

// ---------------------------------------------------------------------------
// bfloat16 inputs: MFMA 16x16x32 over token tiles staged through LDS.
//
// The contraction runs over tokens, but K and V are token-major in HBM, so
// an MFMA operand (8 consecutive tokens of one feature per lane) is a column
// of the tile.  Each 64-token tile of K and V is loaded with coalesced 16-B
// loads, phi is applied to K in registers (v_pk_max_i16), and the tile is
// written to LDS token-major; operands are then gathered with 16-bit LDS
// reads.  The 16-B unit index inside a token row is XOR-swizzled by the
// row's 8-token group so the four lane groups of a wavefront (which read
// rows 8 apart) land on different LDS banks.
//
// Work split in a workgroup: wave (wi, wj) owns the output quadrant
// rows [wi*d/2, +d/2) x cols [wj*d/2, +d/2); waves with wj == 0 also
// accumulate z with a second MFMA against an all-ones B operand.

template <int D>
struct KvTile {
  static constexpr int TT = 64;               // tokens per tile
  static constexpr int UPR = D / 8;           // 16-byte units per token row
  static constexpr int UNITS = TT * UPR;      // units per tensor per tile
  static constexpr int CPT = UNITS / kBlock;  // units per thread per tensor
  static_assert(UNITS % kBlock == 0, "tile must split evenly over the workgroup");
};

template <int UPR>
__device__ __forceinline__ int unit_swizzle(int t) {
  return (((t >> 3) & 3) * 2) & (UPR - 1);
}

// Lane's MFMA operand: feature f of tokens ks + 8g + j, j = 0..7.
template <int UPR>
__device__ __forceinline__ uint4 tile_column8(const uint16_t* tile, int ks, int f, int g) {
  const int t = ks + 8 * g;
  const int unit = (f >> 3) ^ unit_swizzle<UPR>(t);
  const uint16_t* p = tile + (t * UPR + unit) * 8 + (f & 7);
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = p[j * UPR * 8];
  return make_uint4(pack2(w[0], w[1]), pack2(w[2], w[3]), pack2(w[4], w[5]), pack2(w[6], w[7]));
}

template <int D>
__global__ __launch_bounds__(kBlock) void kv_partial_bf16(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, int L,
                                                          int tps, const float* state_in,
                                                          float* dst) {
  using T = KvTile<D>;
  constexpr int QD = D / 2;    // quadrant side
  constexpr int NB = QD / 16;  // 16x16 blocks per quadrant side
  constexpr int E = D * D + D;
  __shared__ uint4 lds[2][2][T::UNITS];  // [buffer][K, V][unit]

  const int split = blockIdx.x;
  const int splits = gridDim.x;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int t0 = split * tps;
  const int t1 = min(L, t0 + tps);
  const uint4* kb = reinterpret_cast<const uint4*>(k + bh * static_cast<size_t>(L) * D);
  const uint4* vb = reinterpret_cast<const uint4*>(v + bh * static_cast<size_t>(L) * D);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wi = wave >> 1, wj = wave & 1;
  const int n = lane & 15, g = lane >> 4;

  f32x4 acc[NB][NB];
  f32x4 accz[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    accz[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);

  // Two register stages: while tile i is in LDS and being multiplied, the
  // loads of tiles i + 1 and i + 2 are in flight.
  uint4 rk0[T::CPT], rv0[T::CPT], rk1[T::CPT], rv1[T::CPT];
  auto gload = [&](uint4 (&rk)[T::CPT], uint4 (&rv)[T::CPT], int tile) {
    const int base = t0 + tile * T::TT;
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int u = tid + kBlock * i;
      const int t = u / T::UPR;
      if (base + t < t1) {
        const size_t idx = static_cast<size_t>(base) * T::UPR + u;
        rk[i] = load_stream(kb + idx);
        rv[i] = load_stream(vb + idx);
      } else {
        rk[i] = make_uint4(0, 0, 0, 0);
        rv[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](const uint4 (&rk)[T::CPT], const uint4 (&rv)[T::CPT], int buf) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int u = tid + kBlock * i;
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
      uint4 a[NB], b[NB];
#pragma unroll
      for (int r = 0; r < NB; ++r) a[r] = tile_column8<T::UPR>(lk, ks, wi * QD + r * 16 + n, g);
#pragma unroll
      for (int c = 0; c < NB; ++c) b[c] = tile_column8<T::UPR>(lv, ks, wj * QD + c * 16 + n, g);
#pragma unroll
      for (int r = 0; r < NB; ++r)
#pragma unroll
        for (int c = 0; c < NB; ++c) acc[r][c] = mfma_16x16x32(a[r], b[c], acc[r][c]);
      if (wj == 0) {
#pragma unroll
        for (int r = 0; r < NB; ++r) accz[r] = mfma_16x16x32(a[r], ones, accz[r]);
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

  float* o = dst + (splits > 1 ? bh * splits + split : bh) * static_cast<size_t>(E);
  const float* si = (splits == 1 && state_in != nullptr) ? state_in + bh * E : nullptr;
#pragma unroll
  for (int r = 0; r < NB; ++r)
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wi * QD + r * 16 + 4 * g + i;
        const int cc = wj * QD + c * 16 + n;
        float x = acc[r][c][i];
        if (si) x = si[ra * D + cc] + x;
        o[ra * D + cc] = x;
      }
  if (wj == 0 && n == 0) {
#pragma unroll
    for (int r = 0; r < NB; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wi * QD + r * 16 + 4 * g + i;
        float x = accz[r][i];
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
                                                         const float* __restrict__ v, int L, int tps,
                                                         const float* state_in,
                                                         float* dst) {
  constexpr int TT = 16;
  constexpr int E = D * D + D;
  constexpr int PER = D * D / kBlock;
  static_assert(D * D % kBlock == 0 && D <= kBlock, "shape");
  __shared__ float sk[TT * D];
  __shared__ float sv[TT * D];

  const int split = blockIdx.x;
  const int splits = gridDim.x;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int t0 = split * tps;
  const int t1 = min(L, t0 + tps);
  const float* kb = k + bh * static_cast<size_t>(L) * D;
  const float* vb = v + bh * static_cast<size_t>(L) * D;
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

  float* o = dst + (splits > 1 ? bh * splits + split : bh) * static_cast<size_t>(E);
  const float* si = (splits == 1 && state_in != nullptr) ? state_in + bh * E : nullptr;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + kBlock * i;
    o[e] = si ? si[e] + acc[i] : acc[i];
  }
  if (tid < D) o[D * D + tid] = si ? si[D * D + tid] + accz : accz;
}

}  // namespace la
