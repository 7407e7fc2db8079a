// Context Cache token score (rMuscle §4.1, Eq. 2) in exact fixed point, shared
// by the standalone score kernel and the finish kernel that scores the next
// layer's input as it writes it.
//
// Per element (float64, every operation separately rounded: these sources are
// compiled with -ffp-contract=off), each term is rounded half-even to an
// int64 at 2^-24 and summed as an integer, so a token's sums do not depend on
// how the row is split over lanes, waves or kernels:
//   rel-RMS : Sd = sum rint(2^24 (x - xr)^2), Sx = sum rint(2^24 x^2),
//             key = fl64(Sd) / fl64(max(Sx, E)),  E = max(1, ceil(d 2^24 / 10^12))
//             (d eps^2 in the same fixed point, eps = 1e-6): the square of Eq. 2.
//   cosine  : Sx, Sy = sum rint(2^24 xr^2), Sxy = sum rint(2^24 x xr),
//             key = 1 - fl64(q |q|) / fl64(fl64(Sx) fl64(Sy)), q = fl64(Sxy)
//             (1 if Sx Sy = 0): decreasing in cos(x, xr).
#pragma once

#include "common.hpp"

namespace cgs {

constexpr double kScoreScale = 16777216.0;  // 2^24

__device__ __forceinline__ long long score_term(double t) {
  return static_cast<long long>(rint(t * kScoreScale));
}

// Fixed-point sums of one token (partial over the elements a thread sees).
struct ScoreSums {
  long long sd = 0, sx = 0, sy = 0, sxy = 0;
  template <bool kCosine>
  __device__ __forceinline__ void add(double a, double b) {
    if (kCosine) {
      sx += score_term(a * a);
      sy += score_term(b * b);
      sxy += score_term(a * b);
    } else {
      const double df = a - b;
      sd += score_term(df * df);
      sx += score_term(a * a);
    }
  }
};

// d eps^2 in the 2^-24 fixed point, rounded up, at least 1 (eps = 1e-6).
inline long long score_floor(int d) {
  const long long v = (static_cast<long long>(d) * (1ll << 24) + 999999999999ll) / 1000000000000ll;
  return v > 1 ? v : 1;
}

// Key of a token from its complete sums.
template <bool kCosine>
__device__ __forceinline__ double score_key(const ScoreSums& s, long long floor_e) {
  if (kCosine) {
    const double q = static_cast<double>(s.sxy);
    const double den = static_cast<double>(s.sx) * static_cast<double>(s.sy);
    return (den == 0.0) ? 1.0 : 1.0 - (q * fabs(q)) / den;
  }
  const long long den = s.sx > floor_e ? s.sx : floor_e;
  return static_cast<double>(s.sd) / static_cast<double>(den);
}

}  // namespace cgs
