// Device and host helpers shared by the HIP translation units of libcgs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cgs.h"

namespace cgs {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // 16 raw bytes
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;  // 8 raw bytes

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 is carried as its uint16 bit pattern)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element traits: bf16 (uint16_t storage) and fp32.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};

// ---------------------------------------------------------------------------
// Order-preserving 64-bit image of a double: a > b  <=>  okey(a) > okey(b)
// (for non-NaN values; -0.0 is folded onto +0.0 first).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ordered_key(double v) {
  if (v == 0.0) v = 0.0;
  uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// ---------------------------------------------------------------------------
// Wave / block reductions and scans
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    T u = __shfl_xor(v, o, kWave);
    v = u > v ? u : v;
  }
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    T u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// DPP (gfx9 data-parallel primitives) wave scans: row_shr 1/2/4/8 within rows
// of 16 lanes, then row_bcast 15 / 31 across rows.  Lanes without a source
// add 0.  Much cheaper than cross-lane shuffles through LDS permutes.
#define CGS_DPP(v, ctrl, rmask) \
  static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), ctrl, rmask, 0xf, false))

// Inclusive prefix sum of a 32-bit value across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += CGS_DPP(v, 0x111, 0xf);  // row_shr:1
  v += CGS_DPP(v, 0x112, 0xf);  // row_shr:2
  v += CGS_DPP(v, 0x114, 0xf);  // row_shr:4
  v += CGS_DPP(v, 0x118, 0xf);  // row_shr:8
  v += CGS_DPP(v, 0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  v += CGS_DPP(v, 0x143, 0xc);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Same for a 64-bit value, carried through two 32-bit halves.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
#define CGS_DPP64_STEP(ctrl, rmask)                \
  {                                                \
    const uint32_t l2 = CGS_DPP(lo, ctrl, rmask);  \
    const uint32_t h2 = CGS_DPP(hi, ctrl, rmask);  \
    const uint32_t nl = lo + l2;                   \
    hi = hi + h2 + (nl < lo ? 1u : 0u);            \
    lo = nl;                                       \
  }
  CGS_DPP64_STEP(0x111, 0xf)
  CGS_DPP64_STEP(0x112, 0xf)
  CGS_DPP64_STEP(0x114, 0xf)
  CGS_DPP64_STEP(0x118, 0xf)
  CGS_DPP64_STEP(0x142, 0xa)
  CGS_DPP64_STEP(0x143, 0xc)
#undef CGS_DPP64_STEP
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_last_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ uint64_t wave_last_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 63));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Sum of a 64-bit integer over the 64 lanes (two's complement, exact), every
// lane receives it.
__device__ __forceinline__ long long wave_sum_i64(long long v) {
  return static_cast<long long>(wave_last_u64(wave_incl_scan_u64(static_cast<uint64_t>(v))));
}

// Exclusive prefix sum of a 32-bit value over all threads of a block
// (blockDim.x a multiple of 64, at most 1024) with DPP wave scans; `scratch`
// holds >= 16 values in LDS.  Also returns the block total.  Contains
// barriers: call from every thread.
__device__ __forceinline__ uint32_t block_exclusive_scan_u32(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const uint32_t s = scratch[w];
    if (w < wid) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Exclusive prefix sum over all threads of a block (blockDim.x a multiple of
// 64, at most 1024).  `scratch` holds >= 16 values of T in LDS.  Also
// returns the block total.  Contains barriers: call from every thread.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* scratch, T* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  T inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  T off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    T s = scratch[w];
    if (w < wid) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
inline bool launch_ok() { return hipGetLastError() == hipSuccess; }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Carve consecutive 256-byte aligned sub-buffers out of a workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <typename T> T* take(size_t count) {
    off = align_up(off, 256);
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return align_up(off, 256); }
};

inline int elem_bytes(int dtype) { return dtype == CGS_BF16 ? 2 : 4; }
inline bool valid_dtype(int dtype) { return dtype == CGS_BF16 || dtype == CGS_F32; }

// LDS-DMA transfers (global_load_lds) address their source with a 32-bit
// per-lane byte offset from a 64-bit base, so an operand that the GEMM cores
// or the action down projection read that way must span fewer than 2^32
// bytes: rows * cols elements of esize bytes.
constexpr long long kDmaSpan = 1ll << 32;
inline bool dma_span_ok(long long rows, long long cols, int esize) {
  return rows >= 0 && cols >= 0 && rows * cols * esize < kDmaSpan;
}

}  // namespace cgs
