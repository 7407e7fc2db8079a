// MFMA fragments for the 16x16 output tiles used by every GEMM in libcgs.
//
// A fragment is 8 consecutive K elements of one row (A operand) or one column
// (B operand).  For bf16 one v_mfma_f32_16x16x32_bf16 consumes it; for fp32
// it feeds eight v_mfma_f32_16x16x4_f32, the i-th taking element i of every
// lane, which contracts the same 32 K values in a different grouping.  Lane
// l supplies row (A) or column (B) l % 16 and K elements 8*(l/16) .. +7 of the
// current 32-wide K step; the 16x16 fp32 result sits in lane l as rows
// 4*(l/16) + v (v = 0..3) of column l % 16.
#pragma once

#include "common.hpp"

namespace cgs {

template <typename T> struct Frag;

template <> struct Frag<uint16_t> {
  u32x4_t u;
  static constexpr int kBytes = 16;
  __device__ __forceinline__ void load(const void* p) { u = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ void zero() { u = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ u32x4_t& chunk(int) { return u; }
};

template <> struct Frag<float> {
  u32x4_t lo, hi;
  static constexpr int kBytes = 32;
  __device__ __forceinline__ void load(const void* p) {
    lo = reinterpret_cast<const u32x4_t*>(p)[0];
    hi = reinterpret_cast<const u32x4_t*>(p)[1];
  }
  __device__ __forceinline__ void zero() { lo = hi = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ u32x4_t& chunk(int q) { return q ? hi : lo; }
};

__device__ __forceinline__ f32x4_t mma(const Frag<uint16_t>& a, const Frag<uint16_t>& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.u),
                                                 __builtin_bit_cast(bf16x8_t, b.u), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mma(const Frag<float>& a, const Frag<float>& b, f32x4_t c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.lo[i]), __uint_as_float(b.lo[i]), c, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.hi[i]), __uint_as_float(b.hi[i]), c, 0, 0, 0);
  return c;
}

// GELU, tanh form (Hendrycks & Gimpel): 0.5 g (1 + tanh(z)), z = sqrt(2/pi)(g +
// 0.044715 g^3), evaluated as g / (1 + exp(-2z)) with the hardware exp2 and
// reciprocal (relative error ~1e-6; saturates correctly for large |g|).
__device__ __forceinline__ float gelu_tanh(float g) {
  const float m2z = -1.5957691216057308f * (g + 0.044715f * g * g * g);  // -2z
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(m2z));
}

}  // namespace cgs
