// Depthwise 3x1x1 temporal convolution over latent frames with a one-frame
// chunk-boundary cache: the temporal convolution of the Spatial-Temporal
// Mix-FFN ("Nvidia, MIT ve diğerleri video yapay zeka devrimini başlattı",
// section "Verimli doğrusal DiT": the MLP alternates 1x3x3 spatial and 3x1x1
// temporal convolutions; sd114.wiki article, section "1. 线性 DiT": a temporal
// convolution module models motion between frames), streamed block by block
// with the visibility rule of the block-causal attention (same page, section
// "Sabit Bellekli KV önbelleğe alma mekanizması": a block reads earlier
// blocks, never later ones).
//
// Per batch b, frame f, position p and channel c, for the frames of one chunk
// (or of every chunk of a sequence cut into chunks of Tf frames):
//   y[f] = w[c][0] x[f-1] + w[c][1] x[f] + w[c][2] x[f+1] + bias[c]
// where x[f+1] is zero when frame f + 1 lies in a later chunk or past the
// sequence, and x[-1] is the cache (the last frame of the previous chunk;
// zero at the start of a video).  The cache out is the sequence's last frame.
#pragma once

#include "la_common.h"

namespace la {

// Eight consecutive channels of one (frame, position) row as floats.  Stores
// carry the non-temporal hint (the rows are written once and never read
// back here: 127 -> 121 us at the 720p chunk).
template <bool BF16>
struct Row8;
template <>
struct Row8<true> {
  __device__ __forceinline__ static void load(const void* base, size_t elem, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static void store(void* base, size_t elem, const float (&v)[8]) {
    const u32x4 u = {pack2(to_bf16(v[0]), to_bf16(v[1])), pack2(to_bf16(v[2]), to_bf16(v[3])),
                     pack2(to_bf16(v[4]), to_bf16(v[5])), pack2(to_bf16(v[6]), to_bf16(v[7]))};
    __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + elem));
  }
};
template <>
struct Row8<false> {
  __device__ __forceinline__ static void load(const void* base, size_t elem, float (&v)[8]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(void* base, size_t elem, const float (&v)[8]) {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + elem);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p + 1);
  }
};

// Grid: (ceil(B P C/8 / 256), chunks).  Thread (column, chunk): eight
// channels of one (b, p) over the frames of one chunk, with the previous,
// current and next frame in registers and the loads of the next four frames
// issued together.  The chunk index is uniform in a workgroup, so every
// frame-bound test below is a uniform branch.  x, cache_in: x_dt; y: y_dt;
// cache_out (x_dt) is written by the threads of the last chunk and may be
// cache_in when there is one chunk (each element is read, by the same
// thread, before it is written).
template <bool X_BF16, bool Y_BF16>
__global__ __launch_bounds__(kBlock) void temporal_conv(const void* __restrict__ x,
                                                        const void* cache_in,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        void* __restrict__ y, void* cache_out,
                                                        int F, int Tf, int P, int C8,
                                                        long long cols) {
  const long long col = static_cast<long long>(blockIdx.x) * kBlock + threadIdx.x;
  if (col >= cols) return;
  const int chunk = blockIdx.y;
  const int nchunks = gridDim.y;
  const long long pc = static_cast<long long>(P) * C8;
  const long long b = col / pc;
  const long long rem = col - b * pc;
  const int p = static_cast<int>(rem / C8);
  const int c8 = static_cast<int>(rem - static_cast<long long>(p) * C8);
  const int C = 8 * C8;
  const size_t frame = static_cast<size_t>(P) * C;                     // elements per frame
  const size_t base = static_cast<size_t>(b) * F * frame + static_cast<size_t>(p) * C + 8 * c8;
  const size_t cbase = (static_cast<size_t>(b) * P + p) * C + 8 * c8;  // cache row

  float w0[8], w1[8], w2[8], bs[8];
  {
    const float4* wp = reinterpret_cast<const float4*>(w + 24 * static_cast<size_t>(c8));
    float t[24];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const float4 q = wp[i];
      t[4 * i] = q.x;
      t[4 * i + 1] = q.y;
      t[4 * i + 2] = q.z;
      t[4 * i + 3] = q.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w0[j] = t[3 * j];
      w1[j] = t[3 * j + 1];
      w2[j] = t[3 * j + 2];
    }
    if (bias != nullptr) {
      const float4 a = reinterpret_cast<const float4*>(bias + 8 * c8)[0];
      const float4 c = reinterpret_cast<const float4*>(bias + 8 * c8)[1];
      bs[0] = a.x; bs[1] = a.y; bs[2] = a.z; bs[3] = a.w;
      bs[4] = c.x; bs[5] = c.y; bs[6] = c.z; bs[7] = c.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) bs[j] = 0.f;
    }
  }

  const int f0 = chunk * Tf;
  const int f1 = min(F, f0 + Tf);
  float prev[8], cur[8];
  if (f0 > 0) {
    Row8<X_BF16>::load(x, base + (f0 - 1) * frame, prev);
  } else if (cache_in != nullptr) {
    Row8<X_BF16>::load(cache_in, cbase, prev);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) prev[j] = 0.f;
  }
  if (f0 < f1) Row8<X_BF16>::load(x, base + f0 * frame, cur);

  for (int f = f0; f < f1; f += 4) {
    float nx[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (f + 1 + u < f1) {
        Row8<X_BF16>::load(x, base + (f + 1 + u) * frame, nx[u]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) nx[u][j] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (f + u >= f1) break;
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        o[j] = fmaf(w2[j], nx[u][j], fmaf(w1[j], cur[j], fmaf(w0[j], prev[j], bs[j])));
      Row8<Y_BF16>::store(y, base + (f + u) * frame, o);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        prev[j] = cur[j];
        cur[j] = nx[u][j];
      }
    }
  }
  // the sequence's last frame (prev after the loop), or the cache passed
  // through when there are no frames
  if (cache_out != nullptr && chunk == nchunks - 1) Row8<X_BF16>::store(cache_out, cbase, prev);
}

}  // namespace la
