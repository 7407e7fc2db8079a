// Context Cache token selection (rMuscle §4.1, Eq. 2 and the top ceil(rho_p P) set).
//
// score_kernel: one wavefront per token.  Each lane takes 8-element vectors of
// the token's row of x and x_ref, forms the float64 per-element terms
// (x - xbar)^2 and x^2 (plus xbar^2 and x*xbar for the cosine kind), rounds
// each to an int64 at 2^-24 and sums them; integer sums are exact, so the
// key does not depend on the reduction order.  Lane 0 forms the float64 key.
//
// topk_kernel: one workgroup of 1024 threads runs an exact radix select over
// the 64-bit order-preserving image of the keys (ties to the lower index) and
// writes the chosen token indices in ascending order.
//
// This translation unit is compiled with -ffp-contract=off: every float64
// operation below is a separate, correctly rounded IEEE operation.
#include "block_select.hpp"
#include "common.hpp"
#include "profile.hpp"
#include "score.hpp"
#include "validate.hpp"

namespace cgs {
namespace {

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, double* out) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu)));
      out[2 * i + 1] = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(w[i] >> 16)));
    }
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, double* out) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};

template <typename T, bool kCosine>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ x,
                                                    const T* __restrict__ xr, int P, int d,
                                                    long long floor_e,
                                                    uint64_t* __restrict__ okeys,
                                                    double* __restrict__ key_out, bool vec) {
  const int lane = threadIdx.x & (kWave - 1);
  const int p = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (p >= P) return;
  const T* xp = x + static_cast<size_t>(p) * d;
  const T* rp = xr + static_cast<size_t>(p) * d;
  ScoreSums acc;
  auto accum = [&](double a, double b) { acc.add<kCosine>(a, b); };
  if (vec) {
    // four 8-element runs per lane in flight at once (d = 2048 bf16: one batch)
    for (int j0 = lane * 8; j0 < d; j0 += 4 * kWave * 8) {
      double a[4][8], b[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + q * kWave * 8;
        if (j < d) { Vec8<T>::load(xp + j, a[q]); Vec8<T>::load(rp + j, b[q]); }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j0 + q * kWave * 8 < d) {
#pragma unroll
          for (int i = 0; i < 8; ++i) accum(a[q][i], b[q][i]);
        }
      }
    }
  } else {
    for (int j = lane; j < d; j += kWave)
      accum(static_cast<double>(Elem<T>::to_f32(xp[j])), static_cast<double>(Elem<T>::to_f32(rp[j])));
  }
  acc.sx = wave_sum_i64(acc.sx);
  if (kCosine) {
    acc.sy = wave_sum_i64(acc.sy);
    acc.sxy = wave_sum_i64(acc.sxy);
  } else {
    acc.sd = wave_sum_i64(acc.sd);
  }
  const double key = score_key<kCosine>(acc, floor_e);
  if (lane == 0) {
    okeys[p] = ordered_key(key);
    if (key_out) key_out[p] = key;
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_kernel(const uint64_t* __restrict__ okeys,
                                                           int P, int k,
                                                           int32_t* __restrict__ idx_out) {
  __shared__ SelShared sm;
  __shared__ SelShared2 sm2;
  if (P <= 4 * kSelThreads) {  // keys cached in registers, 4 per thread
    SelChunk<4> c;
    chunk_load(c, P, [&](int i) { return okeys[i]; });
    chunk_topk(c, P, k, [&](int i, int pos, int) { idx_out[pos] = i; }, sm2);
    return;
  }
  block_topk([&](int i) { return okeys[i]; }, P, k,
             [&](int i, int pos) { idx_out[pos] = i; }, sm);
}

// Top k of precomputed float64 keys (the scores a finish kernel wrote).
__global__ __launch_bounds__(kSelThreads) void topk_values_kernel(const double* __restrict__ keys,
                                                                  int P, int k,
                                                                  int32_t* __restrict__ idx_out) {
  __shared__ SelShared sm;
  __shared__ SelShared2 sm2;
  if (P <= 4 * kSelThreads) {
    SelChunk<4> c;
    chunk_load(c, P, [&](int i) { return ordered_key(keys[i]); });
    chunk_topk(c, P, k, [&](int i, int pos, int) { idx_out[pos] = i; }, sm2);
    return;
  }
  block_topk([&](int i) { return ordered_key(keys[i]); }, P, k,
             [&](int i, int pos) { idx_out[pos] = i; }, sm);
}

}  // namespace
}  // namespace cgs

using namespace cgs;

extern "C" int ctx_select_from_keys(const double* keys, int P, int k, int32_t* idx_out, void* stream) {
  if (P < 0 || k < 0 || k > P || P > 65536) return CGS_ERR_SHAPE;
  if (P == 0 || k == 0) return CGS_OK;
  if (!keys || !idx_out) return CGS_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int st = validate_finite_f64(keys, P, s)) return st;
  ProfScope ps("ctx.topk", s);
  hipLaunchKernelGGL(topk_values_kernel, dim3(1), dim3(kSelThreads), 0, s, keys, P, k, idx_out);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}

extern "C" size_t cgs_ctx_select_workspace(int P, int d) {
  (void)d;
  if (P < 0) return 0;
  return align_up(static_cast<size_t>(P) * sizeof(uint64_t), 256) + 256;
}

extern "C" int ctx_select(const void* x, const void* x_ref, int P, int d, int dtype, int k,
                          int kind, int32_t* idx_out, double* key_out, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!valid_dtype(dtype) || (kind != CGS_SCORE_REL_RMS && kind != CGS_SCORE_COSINE))
    return CGS_ERR_ARG;
  if (P < 0 || d <= 0 || d > 4096 || k < 0 || k > P || P > 65536) return CGS_ERR_SHAPE;
  if (P == 0) return CGS_OK;
  if (!x || !x_ref || (k > 0 && !idx_out)) return CGS_ERR_ARG;
  if (!ws || ws_bytes < cgs_ctx_select_workspace(P, d)) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_on()) {  // fixed-point range of the score sums: |x|, |x_ref| <= 2^12
    int st = validate_abs(x, static_cast<size_t>(P) * d, dtype, 4096.0f, s);
    if (st == CGS_OK) st = validate_abs(x_ref, static_cast<size_t>(P) * d, dtype, 4096.0f, s);
    if (st != CGS_OK) return st;
  }
  uint64_t* okeys = static_cast<uint64_t*>(ws);
  // d * eps^2 in the 2^-24 fixed point, rounded up, at least 1 (eps = 1e-6)
  const long long floor_e = score_floor(d);
  const int eb = elem_bytes(dtype);
  const bool vec = (d % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(x_ref) % 16 == 0) && ((static_cast<size_t>(d) * eb) % 16 == 0);
  const dim3 grid((P + 3) / 4), block(256);
  {
  ProfScope ps("ctx.score", s);
  if (dtype == CGS_BF16) {
    auto* a = static_cast<const uint16_t*>(x);
    auto* b = static_cast<const uint16_t*>(x_ref);
    if (kind == CGS_SCORE_COSINE)
      hipLaunchKernelGGL((score_kernel<uint16_t, true>), grid, block, 0, s, a, b, P, d, floor_e, okeys, key_out, vec);
    else
      hipLaunchKernelGGL((score_kernel<uint16_t, false>), grid, block, 0, s, a, b, P, d, floor_e, okeys, key_out, vec);
  } else {
    auto* a = static_cast<const float*>(x);
    auto* b = static_cast<const float*>(x_ref);
    if (kind == CGS_SCORE_COSINE)
      hipLaunchKernelGGL((score_kernel<float, true>), grid, block, 0, s, a, b, P, d, floor_e, okeys, key_out, vec);
    else
      hipLaunchKernelGGL((score_kernel<float, false>), grid, block, 0, s, a, b, P, d, floor_e, okeys, key_out, vec);
  }
  }
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  if (k > 0) {
    ProfScope ps("ctx.topk", s);
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(kSelThreads), 0, s, okeys, P, k, idx_out);
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  return CGS_OK;
}
