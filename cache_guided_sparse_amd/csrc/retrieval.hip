// Reference retrieval over the prepared working set (rMuscle §4.2 "Retrieving
// a Relevant Reference" and §5 "Joint-History Retrieval" / "Fallback policy"):
//   1. visual match: cosine similarity between the flattened query features
//      and every prepared entry's features, keep the top T;
//   2. rerank those T by the RMS joint-angle difference of the aligned robot
//      state histories ([L][J], two arms of J/2 joints; a dual-arm task takes
//      the larger arm distance, a single-arm task its active arm);
//   3. fallback: if the best cosine is below the threshold, no reference is
//      used (dense execution).
//
// The cosine uses the same exact fixed point as the token score's cosine kind
// (score.hpp): every product of two features is an exact float64, rounded
// half-even to an int64 at 2^-24, and the sums are integers, so the result
// does not depend on how the feature vector is split over workgroups.
//   ret_dot_kernel     grid (chunks, N + 1): workgroup (c, n) sums chunk c of
//                      the query against entry n (Sqq only for n = N) and
//                      writes its integer partials (no atomics, no zeroing);
//   ret_select_kernel  one workgroup: sums the partials (a wave per row), forms
//                      the keys, the top T (key desc, index asc), the rerank
//                      distances (one thread per candidate, fixed order, no
//                      contraction: this file is compiled with
//                      -ffp-contract=off) and the choice.
#include "../../include/cgs.h"
#include "common.hpp"
#include "profile.hpp"
#include "score.hpp"

namespace cgs {
namespace {

constexpr int kRetThreads = 256;
constexpr int kRetChunks = 64;
constexpr int kRetMaxN = 256;
// Features per entry, at most: with |feature| <= 2^7 every rounded product is
// <= 2^38 and a sum of 2^24 of them stays below 2^63.
constexpr long long kRetMaxF = 1ll << 24;

template <typename T> struct Feat8;
template <> struct Feat8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, double* v) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = static_cast<double>(__uint_as_float(u[i] << 16));
      v[2 * i + 1] = static_cast<double>(__uint_as_float(u[i] & 0xffff0000u));
    }
  }
};
template <> struct Feat8<float> {
  static __device__ __forceinline__ void load(const float* p, double* v) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0], b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
};

template <int NT>
__device__ __forceinline__ long long block_sum_ll(long long v, long long* red) {
  v = wave_sum_i64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// part layout: [(N + 1)][kRetChunks][2] int64; entry n: (Srr, Sqr); row N: (Sqq, 0).
template <typename T>
__global__ __launch_bounds__(kRetThreads) void ret_dot_kernel(const T* __restrict__ q, const T* __restrict__ refs,
                                                            int N, long long F, long long* __restrict__ part) {
  __shared__ long long red[kRetThreads / 64];
  const int c = blockIdx.x, n = blockIdx.y;
  const long long per = (F / 8 + kRetChunks - 1) / kRetChunks * 8;  // elements per chunk, multiple of 8
  const long long b = c * per, e = min(F, b + per);
  const T* r = refs + static_cast<size_t>(n < N ? n : 0) * F;
  long long s_rr = 0, s_qr = 0;
  for (long long i = b + threadIdx.x * 8; i < e; i += kRetThreads * 8) {
    double qv[8], rv[8];
    Feat8<T>::load(q + i, qv);
    if (n < N) Feat8<T>::load(r + i, rv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (n < N) {
        s_rr += score_term(rv[j] * rv[j]);
        s_qr += score_term(qv[j] * rv[j]);
      } else {
        s_rr += score_term(qv[j] * qv[j]);
      }
    }
  }
  s_rr = block_sum_ll<kRetThreads>(s_rr, red);
  s_qr = block_sum_ll<kRetThreads>(s_qr, red);
  if (threadIdx.x == 0) {
    long long* o = part + (static_cast<size_t>(n) * kRetChunks + c) * 2;
    o[0] = s_rr;
    o[1] = s_qr;
  }
}

__global__ __launch_bounds__(kRetThreads) void ret_select_kernel(
    const long long* __restrict__ part, int N, int T, const float* __restrict__ q_hist,
    const float* __restrict__ r_hist, int L, int J, int arm, double min_cos, double* __restrict__ cos_out,
    int32_t* __restrict__ top_out, double* __restrict__ dist_out, int32_t* __restrict__ choice_out) {
  __shared__ double key[kRetMaxN];
  __shared__ int32_t top[kRetMaxN];
  __shared__ double dist[kRetMaxN];
  __shared__ long long srr[kRetMaxN + 1], sqr[kRetMaxN + 1];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // row n of the partials (n = N: the query's Sqq): lane c holds chunk c, a
  // wave sums the 64 chunks (integers: order-free); waves take rows in turn
  static_assert(kRetChunks == 64, "one chunk per lane");
  for (int n = wave; n <= N; n += kRetThreads / 64) {
    const long long* pr = part + (static_cast<size_t>(n) * kRetChunks + lane) * 2;
    const long long a = wave_sum_i64(pr[0]);
    const long long b = wave_sum_i64(pr[1]);
    if (lane == 0) { srr[n] = a; sqr[n] = b; }
  }
  __syncthreads();
  if (t < N) {
    const double den = static_cast<double>(srr[N]) * static_cast<double>(srr[t]);
    const double k = den > 0.0 ? static_cast<double>(sqr[t]) / __dsqrt_rn(den) : 0.0;
    key[t] = k;
    cos_out[t] = k;
  }
  __syncthreads();
  // rank of entry t: entries before it in (key desc, index asc) order
  if (t < N) {
    int rank = 0;
    for (int u = 0; u < N; ++u) rank += (key[u] > key[t]) || (key[u] == key[t] && u < t);
    if (rank < T) top[rank] = t;
  }
  __syncthreads();
  // rerank distance of the candidate at rank t
  if (t < T) {
    const int n = top[t];
    const int half = J / 2;
    double best = 0.0;
    for (int a = 0; a < 2; ++a) {
      if (arm >= 0 && a != arm) continue;
      double s = 0.0;
      for (int l = 0; l < L; ++l)
        for (int j = a * half; j < (a + 1) * half; ++j) {
          const double df = static_cast<double>(q_hist[l * J + j]) -
                            static_cast<double>(r_hist[(static_cast<size_t>(n) * L + l) * J + j]);
          s += df * df;
        }
      const double rms = __dsqrt_rn(s / static_cast<double>(L * half));
      best = fmax(best, rms);
    }
    dist[t] = best;
    top_out[t] = n;
    dist_out[t] = best;
  }
  __syncthreads();
  if (t == 0) {
    int choice = -1;
    if (T > 0 && key[top[0]] >= min_cos) {
      int bi = 0;
      for (int r = 1; r < T; ++r)
        if (dist[r] < dist[bi]) bi = r;
      choice = top[bi];
    }
    *choice_out = choice;
  }
}

}  // namespace
}  // namespace cgs

using namespace cgs;

extern "C" size_t cgs_ret_select_workspace(int N, long long F) {
  if (N <= 0 || N > kRetMaxN || F <= 0 || F > kRetMaxF) return 0;
  return static_cast<size_t>(N + 1) * kRetChunks * 2 * sizeof(long long);
}

extern "C" int ret_select(const void* query, const void* refs, int N, long long F, int dtype, int T,
                          const float* q_hist, const float* r_hist, const cgs_rerank* rr, double* cos_out,
                          int32_t* top_out, double* dist_out, int32_t* choice_out, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!query || !refs || !rr || !q_hist || !r_hist || !cos_out || !top_out || !dist_out || !choice_out ||
      !valid_dtype(dtype))
    return CGS_ERR_ARG;
  if (N <= 0 || N > kRetMaxN || F <= 0 || F > kRetMaxF || F % 8 != 0 || T <= 0 || T > N || rr->hist_len <= 0 ||
      rr->joints <= 0 || rr->joints % 2 != 0 || rr->arm < -1 || rr->arm > 1 ||
      static_cast<long long>(rr->hist_len) * rr->joints > (1 << 16))
    return CGS_ERR_SHAPE;
  if (!ws || ws_bytes < cgs_ret_select_workspace(N, F)) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  long long* part = static_cast<long long*>(ws);
  {
    ProfScope ps("ret.dot", s);
    const dim3 grid(kRetChunks, N + 1);
    if (dtype == CGS_BF16)
      hipLaunchKernelGGL((ret_dot_kernel<uint16_t>), grid, dim3(kRetThreads), 0, s,
                         static_cast<const uint16_t*>(query), static_cast<const uint16_t*>(refs), N, F, part);
    else
      hipLaunchKernelGGL((ret_dot_kernel<float>), grid, dim3(kRetThreads), 0, s, static_cast<const float*>(query),
                         static_cast<const float*>(refs), N, F, part);
  }
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  ProfScope ps("ret.select", s);
  hipLaunchKernelGGL(ret_select_kernel, dim3(1), dim3(kRetThreads), 0, s, part, N, T, q_hist, r_hist,
                     rr->hist_len, rr->joints, rr->arm, rr->min_cos, cos_out, top_out, dist_out, choice_out);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}
