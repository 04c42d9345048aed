// Rotary-position arithmetic shared by the RoPE kernels: the token grid,
// positions (by division once, then carried in fixed steps), pair
// frequencies and angles, and the turn of a feature pair.  The reading it
// implements (3-D positions over frames, rows and columns; interleaved
// feature pairs in frame, row, column groups; rotation of phi(q) and phi(k)
// in the numerator only) is stated in rope.h.
#pragma once

#include <math.h>

#include "la_common.h"

namespace la {

// Token grid of the sequences of one call (positions as rope.h states
// them).  rcp_hw, rcp_gw: 1 / (gh gw) and 1 / gw rounded to float by the
// host.  Token indices stay below 2^22 (host check), where rope_div is exact.
struct RopeGrid {
  int frame0;
  int gh, gw, hw;
  float rcp_hw, rcp_gw;
  float theta;
};

template <int D>
struct RopeAxes {
  static constexpr int DH = 2 * (D / 6);      // row group size (= column group size)
  static constexpr int DT = D - 2 * DH;       // frame group size
  static constexpr int B1 = DT / 2;           // first row pair
  static constexpr int B2 = DT / 2 + DH / 2;  // first column pair
};

// n / d for 0 <= n < 2^22 and d >= 1: the float estimate is within one of
// the quotient, and one correction step makes it exact.
__device__ __forceinline__ int rope_div(int n, int d, float rcp) {
  int q = static_cast<int>(static_cast<float>(n) * rcp);
  const int r = n - q * d;
  q += r < 0 ? -1 : (r >= d ? 1 : 0);
  return q;
}

struct RopePos {
  float f, r, c;  // frame, row, column
};

__device__ __forceinline__ RopePos rope_pos(const RopeGrid& g, int tok) {
  const int fr = rope_div(tok, g.hw, g.rcp_hw);
  const int rem = tok - fr * g.hw;
  const int row = rope_div(rem, g.gw, g.rcp_gw);
  return {static_cast<float>(g.frame0 + fr), static_cast<float>(row),
          static_cast<float>(rem - row * g.gw)};
}

// A token's grid position carried along a sequence in fixed steps of `step`
// tokens: the step splits once into whole frames, rows and columns, and each
// advance adds them with at most one carry per axis (no division).
struct RopeStep {
  int f, r, c;
};

__device__ __forceinline__ RopeStep rope_step(const RopeGrid& g, int step) {
  const int f = step / g.hw;
  const int rem = step - f * g.hw;
  const int r = rem / g.gw;
  return {f, r, rem - r * g.gw};
}

struct RopeTrack {
  int f, r, c;  // frame (frame0 included), row, column
  __device__ __forceinline__ void init(const RopeGrid& g, int tok) {
    const int fr = rope_div(tok, g.hw, g.rcp_hw);
    const int rem = tok - fr * g.hw;
    r = rope_div(rem, g.gw, g.rcp_gw);
    c = rem - r * g.gw;
    f = g.frame0 + fr;
  }
  __device__ __forceinline__ void advance(const RopeGrid& g, const RopeStep& s) {
    c += s.c;
    r += s.r;
    f += s.f;
    if (c >= g.gw) {
      c -= g.gw;
      ++r;
    }
    if (r >= g.gh) {
      r -= g.gh;
      ++f;
    }
  }
  __device__ __forceinline__ RopePos pos() const {
    return {static_cast<float>(f), static_cast<float>(r), static_cast<float>(c)};
  }
};

// The position pair m turns with.
template <int D>
__device__ __forceinline__ float rope_axis_pos(const RopePos& p, int m) {
  using A = RopeAxes<D>;
  return m < A::B1 ? p.f : (m < A::B2 ? p.r : p.c);
}

// Frequency of pair m in turns per unit of position, theta^(-2 j / d_a) /
// (2 pi), evaluated in double and returned as float hi + lo.
template <int D>
__device__ float2 rope_freq(int m, float theta) {
  using A = RopeAxes<D>;
  const int j = m < A::B1 ? m : (m < A::B2 ? m - A::B1 : m - A::B2);
  const int da = m < A::B1 ? A::DT : A::DH;
  const double f = pow(static_cast<double>(theta), -2.0 * j / da) * (0.5 / M_PI);
  const float hi = static_cast<float>(f);
  return make_float2(hi, static_cast<float>(f - static_cast<double>(hi)));
}

// p * f in turns reduced to [0, 1) (plus a correction of a few ulp of the
// product): the fractional part of the rounded product is exact
// (`v_fract_f32`: h - floor(h), one instruction, clamped below 1.0), and the
// product's rounding error and the lo part are added after it.  Contraction
// is off here: fusing p * f.x into the reduction would add the rounding error
// twice (0.03 turns at frame 4,000,000).
__device__ __forceinline__ float rope_turns(float p, float2 f) {
#pragma clang fp contract(off)
  const float h = p * f.x;
  const float e = fmaf(p, f.x, -h);
  return __builtin_amdgcn_fractf(h) + fmaf(p, f.y, e);
}

template <bool PRECISE>
__device__ __forceinline__ void rope_sincos(float t, float& s, float& c) {
  if constexpr (PRECISE) {
    sincospif(2.0f * t, &s, &c);
  } else {
    s = __builtin_amdgcn_sinf(t);  // sin(2 pi t)
    c = __builtin_amdgcn_cosf(t);
  }
}

// Pair (x, y) turned by 2 pi t.
template <bool PRECISE>
__device__ __forceinline__ void rope_turn(float t, float& x, float& y) {
  float s, c;
  rope_sincos<PRECISE>(t, s, c);
  const float x1 = x * c - y * s;
  y = x * s + y * c;
  x = x1;
}

__device__ __forceinline__ void unpack_bf16x8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

}  // namespace la
