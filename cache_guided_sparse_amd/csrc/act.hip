// Action Cache masked FFN with a dense anchor (rMuscle §4.1, Eq. 4):
//   y = y_a + (h^M - h_a^M) W_down[M],   h^M = gelu_tanh(x W_gate[M]^T) * (x W_up[M]^T).
//
// Only the mask's rows of W_gate, W_up and the neuron-major W_down are read;
// each is a contiguous d-element row, so every weight access is a coalesced
// row segment.
//
//   masked_glu_kernel  (phase 1) a workgroup owns 16 mask positions and 64
//       tokens; its four waves split d into quarters and each computes the
//       gate and up products of its quarter with MFMA, fragments loaded
//       straight from global memory (x rows and gathered weight rows); the
//       quarters are summed in LDS in a fixed order.  Fused epilogue: h, the
//       optional h_out rows, and the anchor delta rounded to the activation
//       type, stored token-major [S_pad][K_pad] as the next GEMM's A operand.
//   masked_down_kernel (phase 2) a workgroup owns 64 output columns, 64
//       tokens and a contiguous range of mask positions (split-K); it gathers
//       32 down rows x 64 columns per step into LDS and reads them transposed
//       as MFMA B fragments.  fp32 partials per split.
//   masked_finish_kernel sums the partials in split order and adds y_a.
#include <algorithm>

#include "common.hpp"
#include "mfma.hpp"
#include "profile.hpp"

namespace cgs {
namespace {

constexpr int kThreads = 256;
constexpr int kNB = 16;      // mask positions per phase-1 workgroup
constexpr int kTok = 64;     // tokens per workgroup (4 waves x 16)
constexpr int kStep = 32;    // mask positions per phase-2 K step
constexpr int kCols = 64;    // output columns per phase-2 workgroup

template <typename T>
__global__ __launch_bounds__(kThreads) void masked_glu_kernel(
    const T* __restrict__ x, int S, int d, const int32_t* __restrict__ idx, int K, int K_pad,
    const T* __restrict__ wg, const T* __restrict__ wu, const float* __restrict__ h_anchor,
    float* __restrict__ h_out, T* __restrict__ D) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = blockIdx.x * kNB;
  const int s0 = blockIdx.y * kTok;
  const int r = lane & 15, grp = lane >> 4;
  const int dq = d / 4;

  const int i_lane = i0 + r;
  const bool nvalid = i_lane < K;
  const size_t wrow = nvalid ? static_cast<size_t>(idx[i_lane]) * d : 0;
  const T* xrow[4];
  bool tvalid[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int s = s0 + mt * 16 + r;
    tvalid[mt] = s < S;
    xrow[mt] = x + static_cast<size_t>(tvalid[mt] ? s : 0) * d;
  }

  f32x4_t ag[4], au[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) ag[mt] = au[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = wave * dq; k < (wave + 1) * dq; k += 32) {
    const int kk = k + grp * 8;
    Frag<T> bg, bu;
    if (nvalid) { bg.load(wg + wrow + kk); bu.load(wu + wrow + kk); } else { bg.zero(); bu.zero(); }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Frag<T> a;
      if (tvalid[mt]) a.load(xrow[mt] + kk); else a.zero();
      ag[mt] = mma(a, bg, ag[mt]);
      au[mt] = mma(a, bu, au[mt]);
    }
  }
  // Lane holds rows (tokens) mt*16 + 4*grp + v of column (mask position) r.
  __shared__ float part[4][2][kTok][kNB];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      part[wave][0][mt * 16 + 4 * grp + v][r] = ag[mt][v];
      part[wave][1][mt * 16 + 4 * grp + v][r] = au[mt][v];
    }
  __syncthreads();
  for (int e = tid; e < kTok * kNB; e += kThreads) {
    const int s = e / kNB, c = e % kNB;
    const float gsum = part[0][0][s][c] + part[1][0][s][c] + part[2][0][s][c] + part[3][0][s][c];
    const float usum = part[0][1][s][c] + part[1][1][s][c] + part[2][1][s][c] + part[3][1][s][c];
    const int i = i0 + c, sg = s0 + s;
    float delta = 0.f;
    if (i < K && sg < S) {
      const size_t hn = static_cast<size_t>(idx[i]) * S + sg;
      const float h = gelu_tanh(gsum) * usum;
      if (h_out) h_out[hn] = h;
      delta = h_anchor ? h - h_anchor[hn] : h;
    }
    if (i < K_pad) D[static_cast<size_t>(sg) * K_pad + i] = Elem<T>::from_f32(delta);
  }
}

template <typename T>
__device__ __forceinline__ void gather_b_frag(const char* tile, int pitch, int col, int grp, Frag<T>& f);

template <>
__device__ __forceinline__ void gather_b_frag<uint16_t>(const char* tile, int pitch, int col, int grp,
                                                       Frag<uint16_t>& f) {
  uint32_t w[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint16_t lo = *reinterpret_cast<const uint16_t*>(tile + (grp * 8 + 2 * v) * pitch + col * 2);
    const uint16_t hi = *reinterpret_cast<const uint16_t*>(tile + (grp * 8 + 2 * v + 1) * pitch + col * 2);
    w[v] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
  }
  f.u = u32x4_t{w[0], w[1], w[2], w[3]};
}

template <>
__device__ __forceinline__ void gather_b_frag<float>(const char* tile, int pitch, int col, int grp,
                                                    Frag<float>& f) {
  uint32_t w[8];
#pragma unroll
  for (int v = 0; v < 8; ++v)
    w[v] = *reinterpret_cast<const uint32_t*>(tile + (grp * 8 + v) * pitch + col * 4);
  f.lo = u32x4_t{w[0], w[1], w[2], w[3]};
  f.hi = u32x4_t{w[4], w[5], w[6], w[7]};
}

template <typename T>
__global__ __launch_bounds__(kThreads) void masked_down_kernel(
    const T* __restrict__ D, int S, int K_pad, const int32_t* __restrict__ idx, int K,
    const T* __restrict__ wd, int d, int steps_per_split, float* __restrict__ part) {
  constexpr int RB = kCols * sizeof(T);          // bytes of a row segment
  constexpr int PITCH = RB + 8;                  // padded LDS pitch
  constexpr int CH = RB / 8;                     // 8-byte chunks per row segment
  __shared__ __attribute__((aligned(16))) char tile[kStep * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int j0 = blockIdx.x * kCols;
  const int split = blockIdx.y;
  const int s0 = blockIdx.z * kTok;
  const int st_begin = split * steps_per_split;
  const int st_end = min(K_pad / kStep, st_begin + steps_per_split);
  const int srow = s0 + wave * 16 + r;           // token row of this lane's A fragment

  f32x4_t acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int st = st_begin; st < st_end; ++st) {
    const int i0 = st * kStep;
    for (int q = tid; q < kStep * CH; q += kThreads) {
      const int rr = q / CH, c = q % CH;
      u32x2_t v = u32x2_t{0u, 0u};
      if (i0 + rr < K) {
        const char* src = reinterpret_cast<const char*>(wd + static_cast<size_t>(idx[i0 + rr]) * d + j0);
        v = *reinterpret_cast<const u32x2_t*>(src + c * 8);
      }
      *reinterpret_cast<u32x2_t*>(tile + rr * PITCH + c * 8) = v;
    }
    __syncthreads();
    Frag<T> a;
    a.load(D + static_cast<size_t>(srow) * K_pad + i0 + grp * 8);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      Frag<T> b;
      gather_b_frag<T>(tile, PITCH, nt * 16 + r, grp, b);
      acc[nt] = mma(a, b, acc[nt]);
    }
    __syncthreads();
  }
  const size_t so = static_cast<size_t>(split) * S * d;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int s = s0 + wave * 16 + 4 * grp + v;
      if (s < S) part[so + static_cast<size_t>(s) * d + j0 + nt * 16 + r] = acc[nt][v];
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void masked_finish_kernel(
    const float* __restrict__ part, int splits, int S, int d, const float* __restrict__ y_anchor,
    T* __restrict__ y_out, float* __restrict__ y_f32) {
  const size_t n = static_cast<size_t>(S) * d;
  for (size_t e = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; e < n;
       e += static_cast<size_t>(gridDim.x) * kThreads) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += part[s * n + e];
    if (y_anchor) v = y_anchor[e] + v;
    if (y_f32) y_f32[e] = v;
    y_out[e] = Elem<T>::from_f32(v);
  }
}

struct ActPlan {
  int K_pad, S_pad, splits, steps_per_split;
  size_t d_elems, part_elems;
};

ActPlan plan_act(int S, int K, int d) {
  ActPlan p{};
  p.K_pad = (K + kStep - 1) / kStep * kStep;
  p.S_pad = (S + kTok - 1) / kTok * kTok;
  const int steps = p.K_pad / kStep;
  const int base = (d / kCols) * (p.S_pad / kTok);
  int splits = std::max(1, std::min(std::max(steps, 1), (256 + base - 1) / std::max(base, 1)));
  p.steps_per_split = std::max(1, (steps + splits - 1) / splits);
  p.splits = steps > 0 ? (steps + p.steps_per_split - 1) / p.steps_per_split : 0;
  p.d_elems = static_cast<size_t>(p.S_pad) * p.K_pad;
  p.part_elems = static_cast<size_t>(p.splits) * S * d;
  return p;
}

bool act_shape_ok(int d, int ff) { return d > 0 && ff > 0 && d % 128 == 0; }

template <typename T>
int act_t(const cgs_ffn& w, const T* x, int S, const int32_t* idx, int K, const float* ya,
          const float* ha, T* y_out, float* y_f32, float* h_out, void* ws, hipStream_t s) {
  const ActPlan p = plan_act(S, K, w.d);
  Carve cv(ws);
  T* D = cv.take<T>(p.d_elems);
  float* part = cv.take<float>(std::max<size_t>(p.part_elems, 1));
  if (K > 0) {
    {
    ProfScope ps(K == w.ff ? "act.glu.dense" : "act.glu.masked", s);
    hipLaunchKernelGGL((masked_glu_kernel<T>), dim3(p.K_pad / kNB, p.S_pad / kTok), dim3(kThreads), 0, s,
                       x, S, w.d, idx, K, p.K_pad, static_cast<const T*>(w.w_gate),
                       static_cast<const T*>(w.w_up), ha, h_out, D);
    }
    if (!launch_ok()) return CGS_ERR_LAUNCH;
    ProfScope ps(K == w.ff ? "act.down.dense" : "act.down.masked", s);
    hipLaunchKernelGGL((masked_down_kernel<T>), dim3(w.d / kCols, p.splits, p.S_pad / kTok), dim3(kThreads),
                       0, s, D, S, p.K_pad, idx, K, static_cast<const T*>(w.w_down), w.d,
                       p.steps_per_split, part);
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  const size_t n = static_cast<size_t>(S) * w.d;
  const int blocks = static_cast<int>(std::min<size_t>((n + kThreads - 1) / kThreads, 1024));
  ProfScope ps("act.finish", s);
  hipLaunchKernelGGL((masked_finish_kernel<T>), dim3(blocks), dim3(kThreads), 0, s, part,
                     K > 0 ? p.splits : 0, S, w.d, ya, y_out, y_f32);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}

}  // namespace
}  // namespace cgs

using namespace cgs;

extern "C" size_t cgs_act_ffn_masked_workspace(int S, int K, int d, int ff) {
  if (S <= 0 || K < 0 || K > ff || !act_shape_ok(d, ff)) return 0;
  const ActPlan p = plan_act(S, K, d);
  Carve cv(nullptr);
  cv.take<float>(p.d_elems);  // sized for the wider element type
  cv.take<float>(std::max<size_t>(p.part_elems, 1));
  return cv.bytes();
}

extern "C" int act_ffn_masked(const cgs_ffn* w, const void* x, int S, const int32_t* idx, int K,
                              const float* y_anchor, const float* h_anchor, void* y_out,
                              float* y_f32_out, float* h_out, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down || !valid_dtype(w->dtype) ||
      w->down_layout != CGS_DOWN_FD || !x || !y_out || (K > 0 && !idx))
    return CGS_ERR_ARG;
  if (!act_shape_ok(w->d, w->ff)) return CGS_ERR_UNSUPPORTED;
  if (S < 0 || K < 0 || K > w->ff) return CGS_ERR_SHAPE;
  if (S == 0) return CGS_OK;
  if (!ws || ws_bytes < cgs_act_ffn_masked_workspace(S, K, w->d, w->ff)) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w->dtype == CGS_BF16)
    return act_t<uint16_t>(*w, static_cast<const uint16_t*>(x), S, idx, K, y_anchor, h_anchor,
                           static_cast<uint16_t*>(y_out), y_f32_out, h_out, ws, s);
  return act_t<float>(*w, static_cast<const float*>(x), S, idx, K, y_anchor, h_anchor,
                      static_cast<float*>(y_out), y_f32_out, h_out, ws, s);
}
