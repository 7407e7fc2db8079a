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

// Two fp32 values rounded to bf16 (to nearest, ties to even) in one word,
// `lo` in the low half: gfx950's packed conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Quad transpose of a 16 x 16 result tile's bf16 values for row-wise stores.
// Lane l holds rows 4 (l / 16) + v (v = 0..3) of column l % 16, packed as
// p0 = (row 0, row 1), p1 = (row 2, row 3) of its four.  Within each quad of
// lanes (columns 4 j .. 4 j + 3) the 4 x 4 block is transposed in two
// exchanges: lanes l, l ^ 1 swap half-words (v_perm_b32 + DPP), then lanes
// l, l ^ 2 swap words.  Lane l then holds row 4 (l / 16) + (l & 3), columns
// 4 ((l % 16) / 4) .. + 3, as 8 bytes.
struct QuadTranspose {
  uint32_t sel_send, sel_q0, sel_q1;
  bool hi2;
  __device__ __forceinline__ explicit QuadTranspose(int lane) {
    const bool odd = lane & 1;
    // v_perm_b32 (S0, S1, sel): byte i of the result is byte sel[i] of
    // {S0 : S1}, bytes 0..3 from S1 and 4..7 from S0.
    sel_send = odd ? 0x05040100u : 0x07060302u;  // odd: low halves of (p0, p1); even: high halves
    sel_q0 = odd ? 0x03020504u : 0x05040100u;
    sel_q1 = odd ? 0x03020706u : 0x07060100u;
    hi2 = lane & 2;
  }
  __device__ __forceinline__ uint2 operator()(uint32_t p0, uint32_t p1) const {
    // lanes l, l ^ 1: an even lane keeps rows 0, 2 of columns (c, c + 1), an
    // odd lane rows 1, 3 of (c - 1, c)
    const uint32_t send = __builtin_amdgcn_perm(p1, p0, sel_send);
    const uint32_t recv = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(send), 0xB1, 0xF, 0xF, false));
    const uint32_t q0 = __builtin_amdgcn_perm(recv, p0, sel_q0);
    const uint32_t q1 = __builtin_amdgcn_perm(recv, p1, sel_q1);
    // lanes l, l ^ 2: lanes 0, 1 of the quad keep their first word and take
    // the partner's, lanes 2, 3 keep their second
    const uint32_t send2 = hi2 ? q0 : q1;
    const uint32_t recv2 = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(send2), 0x4E, 0xF, 0xF, false));
    return hi2 ? uint2{recv2, q1} : uint2{q0, recv2};
  }
};

// GELU, tanh form (Hendrycks & Gimpel): 0.5 g (1 + tanh(z)), z = sqrt(2/pi)(g +
// 0.044715 g^3), evaluated as g / (1 + exp(-2z)) with the hardware exp2 and
// reciprocal: exp(-2z) = exp2(g (a + b g^2)), a = -2 sqrt(2/pi) / ln 2,
// b = 0.044715 a (relative error ~1e-6; saturates correctly for large |g|).
__device__ __forceinline__ float gelu_tanh(float g) {
  constexpr float a = -2.302208198144325f;
  constexpr float b = -0.1029432395800235f;
  const float t = g * __builtin_fmaf(b, g * g, a);  // -2z / ln 2
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

}  // namespace cgs
