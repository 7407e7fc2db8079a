// Action Cache group-shared neuron mask (rMuscle §3.4 Eq. 1 and §5).
//
// contrib_kernel: one wavefront per neuron n.  In fixed point
//   A[t,n] = sum_r rint(2^24 |h_ref[t,n,r]|),  B[n] = sum_j rint(2^40 w_nj^2)
// are exact int64 sums (order-free), nrm = sqrt(fl64(B)) is correctly
// rounded, c[t,n] = fl64(A) nrm and s[n] = fl64(sum_t A) nrm.  The kernel
// stores the 64-bit order-preserving images of c and s and the value of s.
//
// mask_select_kernel: one workgroup of 1024 threads.
//   TOPK      (§5) for every reference step t, the top K of c[t,:] joins a
//             union; the mask is the top K of the union by s.
//   COVERAGE  (§3.4 coverage) z_n = rint(s_n 2^-e) with e = ilogb(max s) - Q,
//             Q = 61 - ceil(log2 ff); the mask is the shortest prefix of the
//             (s desc, n asc) order with fl64(sum z) >= fl64(tau fl64(sum_all z)).
// Selections are exact radix selects; ties go to the lower neuron index.
//
// Compiled with -ffp-contract=off: every float64 operation is separately
// rounded.
#include <algorithm>

#include "block_select.hpp"
#include "common.hpp"
#include "profile.hpp"
#include "validate.hpp"

namespace cgs {
namespace {

constexpr double kTwo24 = 16777216.0;      // 2^24
constexpr double kTwo40 = 1099511627776.0; // 2^40

// Eight consecutive weights of a row as float (exact; widened to float64 at use).
template <typename T> struct W8;
template <> struct W8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};
template <> struct W8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0], b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
};

constexpr int kContribT = 8;  // reference steps whose activations are loaded up front

// The W_down of every layer of a batched build (one kernel argument).
constexpr int kMaxMaskLayers = 64;
struct LayerPtrs {
  const void* p[kMaxMaskLayers];
};

// The wave's share of B[n] = sum_j rint(2^40 w_nj^2) for the row wr (lane-strided).
template <typename T>
__device__ __forceinline__ long long row_b(const T* __restrict__ wr, int d, int lane, bool vec) {
  long long b = 0;
  if (vec) {
    for (int j0 = lane * 8; j0 < d; j0 += 4 * kWave * 8) {
      float w[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j0 + q * kWave * 8 < d) W8<T>::load(wr + j0 + q * kWave * 8, w[q]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j0 + q * kWave * 8 >= d) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double wv = static_cast<double>(w[q][i]);
          b += static_cast<long long>(rint((wv * wv) * kTwo40));
        }
      }
    }
  } else {
    for (int j = lane; j < d; j += kWave) {
      const double w = static_cast<double>(Elem<T>::to_f32(wr[j]));
      b += static_cast<long long>(rint((w * w) * kTwo40));
    }
  }
  return b;
}

// nrm[n] = sqrt(fl64(B[n])) (correctly rounded) of every neuron of every
// layer; one wavefront per neuron, blockIdx.y = layer.
template <typename T>
__global__ __launch_bounds__(256) void down_norm_kernel(LayerPtrs wdp, int d, int ff,
                                                        double* __restrict__ nrm_out, bool vec) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= ff) return;
  const T* wr = static_cast<const T*>(wdp.p[blockIdx.y]) + static_cast<size_t>(n) * d;
  const long long b = wave_sum_i64(row_b<T>(wr, d, lane, vec));
  if (lane == 0) nrm_out[static_cast<size_t>(blockIdx.y) * ff + n] = __dsqrt_rn(static_cast<double>(b));
}

// blockIdx.y = layer: its h_ref block [T][ff][S], W_down and key slices.
// pre (NULL: computed from W_down): nrm[layer][n] from down_norm_kernel.
template <typename T>
__global__ __launch_bounds__(256) void contrib_kernel(const float* __restrict__ h, int T_steps,
                                                      int S, LayerPtrs wdp, const double* __restrict__ pre,
                                                      int d, int ff, uint64_t* __restrict__ ckey,
                                                      uint64_t* __restrict__ skey,
                                                      double* __restrict__ sval, bool vec) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= ff) return;
  const int layer = blockIdx.y;
  h += static_cast<size_t>(layer) * T_steps * ff * S;
  ckey += static_cast<size_t>(layer) * T_steps * ff;
  skey += static_cast<size_t>(layer) * ff;
  sval += static_cast<size_t>(layer) * ff;
  // The activations of up to kContribT steps (S <= 64: one per lane) are
  // fetched before the weight row (or the stored norm), so both loads are in
  // flight together.
  const bool fast_h = T_steps <= kContribT && S <= kWave;
  float hv[kContribT];
#pragma unroll
  for (int t = 0; t < kContribT; ++t)
    hv[t] = (fast_h && t < T_steps && lane < S) ? h[(static_cast<size_t>(t) * ff + n) * S + lane] : 0.f;
  double nrm;
  if (pre) {
    nrm = pre[static_cast<size_t>(layer) * ff + n];
  } else {
    const T* wr = static_cast<const T*>(wdp.p[layer]) + static_cast<size_t>(n) * d;
    nrm = __dsqrt_rn(static_cast<double>(wave_sum_i64(row_b<T>(wr, d, lane, vec))));
  }
  long long atot = 0;
  for (int t = 0; t < T_steps; ++t) {
    long long a = 0;
    if (fast_h) {
      float hvt = 0.f;
#pragma unroll
      for (int q = 0; q < kContribT; ++q)
        if (q == t) hvt = hv[q];
      a = static_cast<long long>(rint(fabs(static_cast<double>(hvt)) * kTwo24));
    } else {
      const float* hr = h + (static_cast<size_t>(t) * ff + n) * S;
      for (int r = lane; r < S; r += kWave)
        a += static_cast<long long>(rint(fabs(static_cast<double>(hr[r])) * kTwo24));
    }
    a = wave_sum_i64(a);
    atot += a;
    if (lane == 0) ckey[static_cast<size_t>(t) * ff + n] = ordered_key(static_cast<double>(a) * nrm);
  }
  if (lane == 0) {
    const double sv = static_cast<double>(atot) * nrm;
    sval[n] = sv;
    skey[n] = ordered_key(sv);
  }
}

struct MaskShared {
  SelShared sel;
  SelShared2 sel2;
  double dred[kSelThreads / kWave];
  long long lred[kSelThreads / kWave];
};

constexpr int kChunkR = 4;  // neurons per thread in the register-cached path (ff <= 4096)

// Largest sval over the block (sval >= 0), then the coverage threshold pieces:
// e = ilogb(max) - q_bits, z_n = rint(sval_n 2^-e), Z = sum z.
__device__ __forceinline__ double block_max_d(double m, MaskShared& sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  m = wave_max(m);
  if (lane == 0) sm.dred[wid] = m;
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < static_cast<int>(blockDim.x / kWave); ++w) r = fmax(r, sm.dred[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ long long block_sum_ll(long long v, MaskShared& sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) sm.lred[wid] = v;
  __syncthreads();
  long long r = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x / kWave); ++w) r += sm.lred[w];
  __syncthreads();
  return r;
}

// One workgroup per layer (blockIdx.x): its key slices, scratch and outputs.
__global__ __launch_bounds__(kSelThreads) void mask_select_kernel(
    const uint64_t* __restrict__ ckey, const uint64_t* __restrict__ skey,
    const double* __restrict__ sval, int T_steps, int ff, int mode, int K, double coverage,
    int q_bits, uint32_t* __restrict__ uni, uint32_t* __restrict__ flag,
    uint64_t* __restrict__ mask_out, int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out) {
  {
    const size_t layer = blockIdx.x;
    ckey += layer * T_steps * ff;
    skey += layer * ff;
    sval += layer * ff;
    uni += layer * ff;
    flag += layer * ff;
    mask_out += layer * ((ff + 63) / 64);
    idx_out += layer * ff;
    count_out += layer;
  }
  __shared__ MaskShared sm;
  __shared__ uint32_t bm[kSelThreads * kChunkR / 32];  // mask bits of the cached path
  const int tid = threadIdx.x;
  int count = 0;
  const bool cached = ff <= kSelThreads * kChunkR;
  if (cached) {
    // Register-cached path: every thread owns a contiguous chunk of <= 4 neurons.
    for (int q = tid; q < kSelThreads * kChunkR / 32; q += blockDim.x) bm[q] = 0;
    __syncthreads();
    SelChunk<kChunkR> c;
    auto emit = [&](int i, int pos, int) {
      idx_out[pos] = i;
      atomicOr(&bm[i >> 5], 1u << (i & 31));
    };
    if (mode == CGS_MASK_TOPK) {
      if (K > 0) {
        uint32_t in_union = 0;
        for (int t = 0; t < T_steps; ++t) {
          const uint64_t* ck = ckey + static_cast<size_t>(t) * ff;
          chunk_load(c, ff, [&](int i) { return ck[i]; });
          chunk_topk(c, ff, K, [&](int, int, int j) { in_union |= 1u << j; }, sm.sel2);
          __syncthreads();
        }
        chunk_load(c, ff, [&](int i) { return skey[i]; });
#pragma unroll
        for (int j = 0; j < kChunkR; ++j)
          if (!((in_union >> j) & 1u)) c.key[j] = 0ull;
        count = chunk_topk(c, ff, K, emit, sm.sel2);
      }
    } else {
      chunk_load(c, ff, [&](int i) { return skey[i]; });
      double sv[kChunkR];
      double m = 0.0;
#pragma unroll
      for (int j = 0; j < kChunkR; ++j) {
        sv[j] = (j < c.cnt) ? sval[c.lo + j] : 0.0;
        m = fmax(m, sv[j]);
      }
      const double smax = block_max_d(m, sm);
      if (smax > 0.0) {
        const int e = ilogb(smax) - q_bits;
        long long zs = 0;
#pragma unroll
        for (int j = 0; j < kChunkR; ++j) {
          c.z[j] = (j < c.cnt) ? static_cast<long long>(rint(ldexp(sv[j], -e))) : 0;
          zs += c.z[j];
        }
        const long long Z = block_sum_ll(zs, sm);
        const double thr = coverage * static_cast<double>(Z);
        count = chunk_coverage_cut(c, ff, thr, emit, sm.sel2);
      }
    }
    __syncthreads();
    for (int i = count + tid; i < ff; i += blockDim.x) idx_out[i] = -1;
    const int words = (ff + 63) / 64;
    for (int wdx = tid; wdx < words; wdx += blockDim.x)
      mask_out[wdx] = static_cast<uint64_t>(bm[2 * wdx]) | (static_cast<uint64_t>(bm[2 * wdx + 1]) << 32);
    if (tid == 0) *count_out = count;
    return;
  }

  // General path (ff > 4096): keys re-read from global memory on every pass.
  const int lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < ff; i += blockDim.x) { uni[i] = 0; flag[i] = 0; }
  __syncthreads();
  auto emit = [&](int i, int pos) { idx_out[pos] = i; flag[i] = 1; };
  if (mode == CGS_MASK_TOPK) {
    if (K > 0) {
      for (int t = 0; t < T_steps; ++t) {
        const uint64_t* ck = ckey + static_cast<size_t>(t) * ff;
        block_topk([&](int i) { return ck[i]; }, ff, K, [&](int i, int) { uni[i] = 1; }, sm.sel);
        __syncthreads();
      }
      count = block_topk([&](int i) { return uni[i] ? skey[i] : 0ull; }, ff, K, emit, sm.sel);
    }
  } else {
    double m = 0.0;
    for (int i = tid; i < ff; i += blockDim.x) m = fmax(m, sval[i]);
    m = wave_max(m);
    if (lane == 0) sm.dred[wid] = m;
    __syncthreads();
    double smax = 0.0;
    for (int w = 0; w < static_cast<int>(blockDim.x / kWave); ++w) smax = fmax(smax, sm.dred[w]);
    if (smax > 0.0) {
      const int e = ilogb(smax) - q_bits;
      auto z_of = [&](int i) { return static_cast<long long>(rint(ldexp(sval[i], -e))); };
      long long zs = 0;
      for (int i = tid; i < ff; i += blockDim.x) zs += z_of(i);
      zs = wave_sum(zs);
      if (lane == 0) sm.lred[wid] = zs;
      __syncthreads();
      long long Z = 0;
      for (int w = 0; w < static_cast<int>(blockDim.x / kWave); ++w) Z += sm.lred[w];
      const double thr = coverage * static_cast<double>(Z);
      count = block_coverage_cut([&](int i) { return skey[i]; }, z_of, ff, thr, emit, sm.sel);
    }
  }
  __syncthreads();
  for (int i = count + tid; i < ff; i += blockDim.x) idx_out[i] = -1;
  const int words = (ff + 63) / 64;
  for (int wdx = tid; wdx < words; wdx += blockDim.x) {
    uint64_t bits = 0;
    for (int b = 0; b < 64 && wdx * 64 + b < ff; ++b)
      if (flag[wdx * 64 + b]) bits |= 1ull << b;
    mask_out[wdx] = bits;
  }
  if (tid == 0) *count_out = count;
}

struct MaskWs {
  uint64_t* ckey;
  uint64_t* skey;
  double* sval;
  uint32_t* uni;
  uint32_t* flag;
  size_t bytes;
};

MaskWs carve_mask(void* ws, int layers, int T, int ff) {
  Carve cv(ws);
  MaskWs m{};
  const size_t lf = static_cast<size_t>(layers) * ff;
  m.ckey = cv.take<uint64_t>(lf * T);
  m.skey = cv.take<uint64_t>(lf);
  m.sval = cv.take<double>(lf);
  m.uni = cv.take<uint32_t>(lf);
  m.flag = cv.take<uint32_t>(lf);
  m.bytes = cv.bytes();
  return m;
}

// Stored masks back to index lists: one workgroup per mask; thread t takes
// kIdxWords consecutive 64-bit words, the block's exclusive prefix sum of the
// words' populations places each thread's neurons, and positions past the
// count are filled with -1.  Bits at positions >= ff are ignored.
constexpr int kIdxThreads = 256;
constexpr int kIdxWords = 4;  // ff <= 65536: at most 1024 words per mask

__global__ __launch_bounds__(kIdxThreads) void mask_indices_kernel(const uint64_t* __restrict__ masks, int ff,
                                                                  int32_t* __restrict__ idx_out,
                                                                  int32_t* __restrict__ count_out) {
  __shared__ int scan[kIdxThreads];
  const int tid = threadIdx.x;
  const int nw = (ff + 63) / 64;
  const size_t m = blockIdx.x;
  const uint64_t* w = masks + m * nw;
  int32_t* out = idx_out + m * ff;
  uint64_t v[kIdxWords];
  int pop = 0;
#pragma unroll
  for (int j = 0; j < kIdxWords; ++j) {
    const int wi = tid * kIdxWords + j;
    uint64_t x = wi < nw ? w[wi] : 0ull;
    const int valid = ff - wi * 64;  // bits of this word inside [0, ff)
    if (valid < 64) x &= valid > 0 ? (~0ull >> (64 - valid)) : 0ull;
    v[j] = x;
    pop += __popcll(x);
  }
  scan[tid] = pop;
  __syncthreads();
  // inclusive Hillis-Steele scan over the block
  for (int off = 1; off < kIdxThreads; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  const int total = scan[kIdxThreads - 1];
  int pos = scan[tid] - pop;
#pragma unroll
  for (int j = 0; j < kIdxWords; ++j) {
    uint64_t x = v[j];
    const int base = (tid * kIdxWords + j) * 64;
    while (x) {
      const int b = __builtin_ctzll(x);
      out[pos++] = base + b;
      x &= x - 1;
    }
  }
  for (int i = total + tid; i < ff; i += kIdxThreads) out[i] = -1;
  if (tid == 0 && count_out) count_out[m] = total;
}

int bit_length(unsigned v) {
  int b = 0;
  while (v) { ++b; v >>= 1; }
  return b;
}

}  // namespace
}  // namespace cgs

using namespace cgs;

extern "C" size_t cgs_act_build_masks_workspace(int layers, int T, int S, int ff, int d) {
  (void)S; (void)d;
  if (layers <= 0 || layers > kMaxMaskLayers || T <= 0 || ff <= 0) return 0;
  return carve_mask(nullptr, layers, T, ff).bytes;
}

extern "C" size_t cgs_act_build_mask_workspace(int T, int S, int ff, int d) {
  return cgs_act_build_masks_workspace(1, T, S, ff, d);
}

namespace {

// Shape checks shared by the weight-based and the norm-based builds.
int mask_shape_status(int layers, int T, int S, int ff, int mode, int K, double coverage) {
  if (layers <= 0 || layers > kMaxMaskLayers) return CGS_ERR_SHAPE;
  if (mode != CGS_MASK_TOPK && mode != CGS_MASK_COVERAGE) return CGS_ERR_ARG;
  if (T <= 0 || S <= 0 || ff <= 0 || ff > 65536 || static_cast<long long>(S) * T > (1 << 14))
    return CGS_ERR_SHAPE;
  if (mode == CGS_MASK_TOPK && (K < 0 || K > ff)) return CGS_ERR_SHAPE;
  if (mode == CGS_MASK_COVERAGE && !(coverage >= 0.0 && coverage <= 1.0)) return CGS_ERR_SHAPE;
  return CGS_OK;
}

// W_down of every layer (FD layout, one shape and dtype); sets *vec when
// 16-byte row loads are possible.
int down_layers(const cgs_ffn* w, int layers, LayerPtrs* wdp, bool* vec) {
  for (int l = 0; l < layers; ++l)
    if (!w[l].w_down || !valid_dtype(w[l].dtype) || w[l].down_layout != CGS_DOWN_FD) return CGS_ERR_ARG;
  const int ff = w[0].ff, d = w[0].d, dt = w[0].dtype;
  for (int l = 1; l < layers; ++l)
    if (w[l].ff != ff || w[l].d != d || w[l].dtype != dt) return CGS_ERR_SHAPE;
  if (d <= 0 || d > 4096 || ff <= 0 || ff > 65536) return CGS_ERR_SHAPE;
  *vec = d % 8 == 0 && (static_cast<size_t>(d) * elem_bytes(dt)) % 16 == 0;
  for (int l = 0; l < layers; ++l) {
    wdp->p[l] = w[l].w_down;
    *vec = *vec && reinterpret_cast<uintptr_t>(w[l].w_down) % 16 == 0;
  }
  return CGS_OK;
}

int validate_down(const cgs_ffn* w, int layers, hipStream_t s) {
  // fixed-point range of the weight norms: |w| < 2^5
  int st = CGS_OK;
  for (int l = 0; l < layers && st == CGS_OK; ++l)
    st = validate_abs(w[l].w_down, static_cast<size_t>(w[l].ff) * w[l].d, w[l].dtype, 31.999998f, s);
  return st;
}

// Contribution keys (from W_down, or from stored norms when pre is given),
// then the per-layer selection.
int build_masks(const float* h_ref, int layers, int T, int S, const LayerPtrs& wdp, const double* pre, int d,
                int ff, int dt, bool vec, int mode, int K, double coverage, uint64_t* mask_out, int32_t* idx_out,
                int32_t* count_out, void* ws, hipStream_t s) {
  const MaskWs m = carve_mask(ws, layers, T, ff);
  const dim3 grid((ff + 3) / 4, layers), block(256);
  {
    ProfScope ps("mask.contrib", s);
    if (dt == CGS_F32)
      hipLaunchKernelGGL((contrib_kernel<float>), grid, block, 0, s, h_ref, T, S, wdp, pre, d, ff, m.ckey,
                         m.skey, m.sval, vec);
    else
      hipLaunchKernelGGL((contrib_kernel<uint16_t>), grid, block, 0, s, h_ref, T, S, wdp, pre, d, ff, m.ckey,
                         m.skey, m.sval, vec);
  }
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  const int q_bits = 61 - bit_length(static_cast<unsigned>(ff - 1));
  ProfScope ps("mask.select", s);
  hipLaunchKernelGGL(mask_select_kernel, dim3(layers), dim3(kSelThreads), 0, s, m.ckey, m.skey, m.sval,
                     T, ff, mode, K, coverage, q_bits, m.uni, m.flag, mask_out, idx_out, count_out);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}

}  // namespace

extern "C" int act_build_masks(const float* h_ref, int layers, int T, int S, const cgs_ffn* w, int mode,
                               int K, double coverage, uint64_t* mask_out, int32_t* idx_out,
                               int32_t* count_out, void* ws, size_t ws_bytes, void* stream) {
  if (!h_ref || !w || !mask_out || !idx_out || !count_out) return CGS_ERR_ARG;
  if (layers <= 0 || layers > kMaxMaskLayers) return CGS_ERR_SHAPE;
  LayerPtrs wdp{};
  bool vec = false;
  if (const int st = down_layers(w, layers, &wdp, &vec)) return st;
  const int ff = w[0].ff, d = w[0].d;
  if (const int st = mask_shape_status(layers, T, S, ff, mode, K, coverage)) return st;
  if (!ws || ws_bytes < cgs_act_build_masks_workspace(layers, T, S, ff, d)) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_on()) {
    // fixed-point range of the activation sums: |h| < 2^24
    int st = validate_abs(h_ref, static_cast<size_t>(layers) * T * ff * S, CGS_F32, 16777215.0f, s);
    if (st == CGS_OK) st = validate_down(w, layers, s);
    if (st != CGS_OK) return st;
  }
  return build_masks(h_ref, layers, T, S, wdp, nullptr, d, ff, w[0].dtype, vec, mode, K, coverage, mask_out,
                     idx_out, count_out, ws, s);
}

extern "C" int act_down_norms(const cgs_ffn* w, int layers, double* nrm_out, void* stream) {
  if (!w || !nrm_out) return CGS_ERR_ARG;
  if (layers <= 0 || layers > kMaxMaskLayers) return CGS_ERR_SHAPE;
  LayerPtrs wdp{};
  bool vec = false;
  if (const int st = down_layers(w, layers, &wdp, &vec)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_on())
    if (const int st = validate_down(w, layers, s)) return st;
  const int ff = w[0].ff, d = w[0].d;
  const dim3 grid((ff + 3) / 4, layers), block(256);
  ProfScope ps("mask.norms", s);
  if (w[0].dtype == CGS_F32)
    hipLaunchKernelGGL((down_norm_kernel<float>), grid, block, 0, s, wdp, d, ff, nrm_out, vec);
  else
    hipLaunchKernelGGL((down_norm_kernel<uint16_t>), grid, block, 0, s, wdp, d, ff, nrm_out, vec);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}

extern "C" int act_build_masks_normed(const float* h_ref, int layers, int T, int S, const double* nrm, int ff,
                                      int mode, int K, double coverage, uint64_t* mask_out, int32_t* idx_out,
                                      int32_t* count_out, void* ws, size_t ws_bytes, void* stream) {
  if (!h_ref || !nrm || !mask_out || !idx_out || !count_out) return CGS_ERR_ARG;
  if (const int st = mask_shape_status(layers, T, S, ff, mode, K, coverage)) return st;
  if (!ws || ws_bytes < cgs_act_build_masks_workspace(layers, T, S, ff, 1)) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_on()) {
    int st = validate_abs(h_ref, static_cast<size_t>(layers) * T * ff * S, CGS_F32, 16777215.0f, s);
    if (st == CGS_OK) st = validate_finite_f64(nrm, layers * ff, s, true);
    if (st != CGS_OK) return st;
  }
  return build_masks(h_ref, layers, T, S, LayerPtrs{}, nrm, 0, ff, CGS_BF16, false, mode, K, coverage,
                     mask_out, idx_out, count_out, ws, s);
}

extern "C" int act_build_mask(const float* h_ref, int T, int S, const cgs_ffn* w, int mode, int K,
                              double coverage, uint64_t* mask_out, int32_t* idx_out,
                              int32_t* count_out, void* ws, size_t ws_bytes, void* stream) {
  return act_build_masks(h_ref, 1, T, S, w, mode, K, coverage, mask_out, idx_out, count_out, ws, ws_bytes,
                         stream);
}

extern "C" int act_mask_indices(const uint64_t* masks, int n, int ff, int32_t* idx_out, int32_t* count_out,
                                void* stream) {
  if (n < 0 || ff <= 0 || ff > kIdxThreads * kIdxWords * 64) return CGS_ERR_SHAPE;
  if (n == 0) return CGS_OK;
  if (!masks || !idx_out) return CGS_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ProfScope ps("mask.indices", s);
  hipLaunchKernelGGL(mask_indices_kernel, dim3(n), dim3(kIdxThreads), 0, s, masks, ff, idx_out, count_out);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}
