// State update of the block-causal form: S_out = S_in + sum_s P_s and
// z_out = z_in + sum_s p_s ("Nvidia, MIT ve diğerleri video yapay zeka
// devrimini başlattı", section "Sabit Bellekli KV önbelleğe alma
// mekanizması": KV1 is cached, the next block's KV is added to it, and the
// last block's addition yields the global KV matrix).
#pragma once

#include "la_common.h"

namespace la {

// One workgroup per 64 float4 of the (d*d + d) state of one (b, h): its
// four wavefronts each sum one contiguous quarter of the splits (in split
// order, loads in batches of eight and four), then wave 0 adds the four quarters in
// order and adds the result to S_in.  The order is fixed, so repeated runs
// are bitwise identical.  splits == 0 copies state_in (or writes zeros when
// state_in is null).  state_in may equal state_out: each element is read
// before it is written, by the same thread.  Wave 0 issues its S_in load
// with the partial loads, so the kernel waits on memory once, not twice.
__global__ __launch_bounds__(kBlock) void state_reduce(const float4* __restrict__ partials,
                                                       int splits, int n4,
                                                       const float4* state_in,
                                                       float4* state_out) {
  __shared__ float4 part[kBlock / kWave][kWave];
  const int j = threadIdx.x / kWave;
  const int el = threadIdx.x % kWave;
  const int e = blockIdx.x * kWave + el;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  const int per = (splits + 3) / 4;
  const int s0 = min(splits, j * per);
  const int s1 = min(splits, s0 + per);
  float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [](float4& a, const float4& x) {
    a.x += x.x;
    a.y += x.y;
    a.z += x.z;
    a.w += x.w;
  };
  const size_t idx = bh * n4 + e;
  float4 si = make_float4(0.f, 0.f, 0.f, 0.f);
  if (j == 0 && e < n4 && state_in != nullptr) si = state_in[idx];
  if (e < n4) {
    const float4* p = partials + bh * static_cast<size_t>(splits) * n4 + e;
    // batches of 8 independent loads, then the adds in split order: a
    // quarter of up to 8 splits (32 splits per block) waits on memory once
    int s = s0;
    for (; s + 8 <= s1; s += 8) {
      float4 x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = p[static_cast<size_t>(s + i) * n4];
#pragma unroll
      for (int i = 0; i < 8; ++i) add(kv, x[i]);
    }
    for (; s + 4 <= s1; s += 4) {
      const float4 x0 = p[static_cast<size_t>(s) * n4];
      const float4 x1 = p[static_cast<size_t>(s + 1) * n4];
      const float4 x2 = p[static_cast<size_t>(s + 2) * n4];
      const float4 x3 = p[static_cast<size_t>(s + 3) * n4];
      add(kv, x0);
      add(kv, x1);
      add(kv, x2);
      add(kv, x3);
    }
    for (; s < s1; ++s) add(kv, p[static_cast<size_t>(s) * n4]);
  }
  part[j][el] = kv;
  __syncthreads();
  if (j != 0 || e >= n4) return;
  float4 t = part[0][el];
  add(t, part[1][el]);
  add(t, part[2][el]);
  add(t, part[3][el]);
  if (state_in != nullptr) {
    t.x = si.x + t.x;
    t.y = si.y + t.y;
    t.z = si.z + t.z;
    t.w = si.w + t.w;
  }
  state_out[idx] = t;
}

// Inclusive prefix over the blocks of a whole sequence: for block c,
//   S_c = S_{c-1} + sum_s P_{c,s},  S_{-1} = S_in (or 0),
// written to states[B][H][blocks][d*d + d].  One thread per float4 of one
// (b, h) state walks the blocks in order; the loads of four blocks' splits
// are issued together.  Each block's partials are summed in split order and
// then added to the running state (a fixed order: repeated runs are bitwise
// identical; against one la_chunk_forward per block only the float32
// summation order differs).  state_in must not overlap states; partials may
// be states itself (one split per block: each element is read before the
// same thread writes it).
__global__ __launch_bounds__(kBlock) void state_scan(const float4* partials,
                                                     int nblk, int splits, int n4,
                                                     const float4* __restrict__ state_in,
                                                     float4* states) {
  const int e = blockIdx.x * kBlock + threadIdx.x;
  if (e >= n4) return;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  auto add = [](float4& a, const float4& x) {
    a.x += x.x;
    a.y += x.y;
    a.z += x.z;
    a.w += x.w;
  };
  float4 run = state_in != nullptr ? state_in[bh * n4 + e] : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* p = partials + bh * static_cast<size_t>(nblk) * splits * n4 + e;
  float4* out = states + bh * static_cast<size_t>(nblk) * n4 + e;
  // The (block, split) partials of this element, block-major: taken in
  // batches of Q independent loads (latency, not bandwidth, bounds this
  // kernel), then added in order; a block's sum joins the running state
  // after its last split.  Every load of a batch precedes the stores of the
  // batch (partials may be states itself).
  constexpr int Q = 16;
  const int total = nblk * splits;
  float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
  int sc = 0, c = 0;
  for (int t0 = 0; t0 < total; t0 += Q) {
    float4 x[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j)
      x[j] = t0 + j < total ? p[static_cast<size_t>(t0 + j) * n4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      if (t0 + j < total) {
        add(kv, x[j]);
        if (++sc == splits) {
          run.x = run.x + kv.x;
          run.y = run.y + kv.y;
          run.z = run.z + kv.z;
          run.w = run.w + kv.w;
          out[static_cast<size_t>(c) * n4] = run;
          kv = make_float4(0.f, 0.f, 0.f, 0.f);
          sc = 0;
          ++c;
        }
      }
    }
  }
}

// Suffix over the blocks of a sequence, for the gradients:
//   R_c = R_{c+1} + sum_s P_{c,s} + dS_c,  c = C-1 .. 0,  R_C = 0,
// written to R[B][H][blocks][d*d + d]; dS (the gradients of the states
// after every block) may be null; d_in, if not null, receives R_0 (the
// gradient of the state before the first block).  One thread per float4 of
// one (b, h) walks the blocks backwards; splits are summed in order, so
// repeated runs are bitwise identical.  partials may be R itself (one split
// per block): each element is read before the same thread writes it.
__global__ __launch_bounds__(kBlock) void state_suffix_scan(const float4* partials, int nblk,
                                                            int splits, int n4,
                                                            const float4* __restrict__ dS,
                                                            float4* R,
                                                            float4* __restrict__ d_in) {
  const int e = blockIdx.x * kBlock + threadIdx.x;
  if (e >= n4) return;
  const size_t bh = static_cast<size_t>(blockIdx.z) * gridDim.y + blockIdx.y;
  auto add = [](float4& a, const float4& x) {
    a.x += x.x;
    a.y += x.y;
    a.z += x.z;
    a.w += x.w;
  };
  const float4* p = partials + bh * static_cast<size_t>(nblk) * splits * n4 + e;
  const float4* ds = dS != nullptr ? dS + bh * static_cast<size_t>(nblk) * n4 + e : nullptr;
  float4* out = R + bh * static_cast<size_t>(nblk) * n4 + e;
  // Blocks from the last to the first, each block's splits in order: taken
  // in batches of Q independent loads (with the state gradient of every
  // block a batch closes), then added in that order.  Every load of a batch
  // precedes the stores of the batch (partials may be R itself).
  constexpr int Q = 16;
  const int total = nblk * splits;
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 run = zero, x = zero;
  int sc = 0, c = nblk - 1;
  for (int k0 = 0; k0 < total; k0 += Q) {
    float4 v[Q], g[Q];
    // k = k0 + j is split (k mod splits) of block nblk - 1 - k / splits
    int cj = c, sj = sc;
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      const bool in = k0 + j < total;
      // (a temporary, not `zero`, on the right: a conditional of two lvalues
      // would select between a global and a private address)
      v[j] = in ? p[(static_cast<size_t>(cj) * splits + sj) * n4]
                : make_float4(0.f, 0.f, 0.f, 0.f);
      g[j] = in && ds != nullptr && sj == splits - 1 ? ds[static_cast<size_t>(cj) * n4]
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
      if (++sj == splits) {
        sj = 0;
        --cj;
      }
    }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      if (k0 + j < total) {
        add(x, v[j]);
        if (++sc == splits) {
          if (ds != nullptr) add(x, g[j]);
          add(run, x);
          out[static_cast<size_t>(c) * n4] = run;
          x = zero;
          sc = 0;
          --c;
        }
      }
    }
  }
  if (d_in != nullptr) d_in[bh * n4 + e] = run;
}

// Zero fill (used instead of a memset so that callers may graph-capture it).
__global__ __launch_bounds__(kBlock) void fill_zero(float4* __restrict__ p, size_t n4) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kBlock;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace la
