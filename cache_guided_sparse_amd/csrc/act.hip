// Action Cache masked FFN with a dense anchor (rMuscle §4.1, Eq. 4):
//   y = y_a + (h^M - h_a^M) W_down[M],   h^M = gelu_tanh(x W_gate[M]^T) * (x W_up[M]^T).
//
// Only the mask's rows of W_gate, W_up and the neuron-major W_down are read;
// each is a contiguous d-element row, so every weight access is a coalesced
// row segment.  The path is memory- and latency-bound (a masked layer of the
// 18-layer expert moves ~7.5 MB), so every kernel puts all of its weight
// loads in flight before it computes:
//
//   act_glu_kernel    a workgroup owns 16 (32 for large masks) mask positions and TT tokens (64
//       for dense-size masks of at most 64 tokens); its waves split d into slices.  Each wave issues all of its
//       gathered gate/up fragments and its x fragments of a chunk at once,
//       then runs the MFMAs; the quarters are summed in LDS in a fixed order.
//       Epilogue: h (optionally stored to the neuron-major h_out rows) and the
//       anchor delta h - h_a rounded to the activation type, stored
//       token-major [S_pad][K_pad] as the next GEMM's A operand (zero past K).
//   act_down_kernel   a workgroup owns 64 output columns, 64 tokens and a
//       contiguous range of at most kMaxSteps x 32 mask positions (split-K).
//       All of its gathered W_down row segments go global -> LDS by LDS DMA
//       up front; B fragments are read transposed (column-major) out of LDS.
//       fp32 partials per split.
//   act_finish_kernel sums the partials in split order, adds y_a, stores y
//       (and its fp32 value), and optionally applies the residual/RMSNorm glue.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "gemm.hpp"
#include "glue.hpp"
#include "profile.hpp"
#include "validate.hpp"

namespace cgs {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4;      // 32-wide K steps per load batch of a GLU wave (any NTW)
constexpr int kStep = 32;      // mask positions per down K step
constexpr int kCols = 32;      // output columns per down workgroup
constexpr int kTokDown = 64;   // tokens per down workgroup (4 waves x 16)
constexpr int kMaxSteps = 8;   // K steps per down workgroup (LDS: 8 x 32 rows)
constexpr int kDownSplits = 8; // preferred K splits of the down projection
constexpr int kWideGluK = 2048;  // masks of at least this many positions use 32-position GLU workgroups
constexpr int kGluWaves = 8;     // waves (d slices) of a gate/up workgroup when d allows (else 4)
constexpr bool kXcdMap = true;   // XCD-aware workgroup numbering (xcd_tile)

// COMPACT: the weights hold the mask's rows only (row i is mask position i);
// idx then only addresses h_anchor / h_out rows and may be NULL without them.
// tok (NULL = identity): the S computed rows are rows tok[0..S) of x, of
// S_all rows in all (the row index of h_anchor / h_out columns).
// NTW: 16-wide tiles of mask positions per workgroup (NB = 16 NTW positions).
// NW waves split d into NW slices.
// Workgroups are dealt round-robin over the 8 XCDs.  With kXcdMap, the
// linear workgroup id is renumbered so that each XCD runs a contiguous range
// of logical (x fastest) tiles: tiles that share operand rows then share that
// XCD's L2.  Returns the logical (x, y) of this workgroup.
// lx: the logical x extent (lx * ly = gridDim.x * gridDim.y).
__device__ __forceinline__ int2 xcd_tile(int lx) {
  const int b = blockIdx.x + gridDim.x * blockIdx.y;
  const int n = gridDim.x * gridDim.y;
  const int l = (kXcdMap && n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
  return make_int2(l % lx, l / lx);
}

template <typename T, int MTW, int NTW, bool COMPACT, int NW = 4>
__global__ __launch_bounds__(64 * NW) void act_glu_kernel(
    const T* __restrict__ x, int S, int d, const int32_t* __restrict__ idx, int K, int K_pad,
    const T* __restrict__ wg, const T* __restrict__ wu, const float* __restrict__ h_anchor,
    float* __restrict__ h_out, T* __restrict__ D, const int32_t* __restrict__ tok, int S_all) {
  constexpr int TT = 16 * MTW;  // tokens per workgroup
  constexpr int NB = 16 * NTW;  // mask positions per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // logical tile: token block fastest, so both token blocks of a neuron
  // block (the same weight rows) run on one XCD
  const int2 tl = xcd_tile(gridDim.y);
  const int i0 = tl.y * NB;
  const int s0 = tl.x * TT;
  const int r = lane & 15, grp = lane >> 4;
  constexpr int NTH = 64 * NW;
  const int dq = d / NW;

  bool nvalid[NTW];
  size_t wrow[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int i_lane = i0 + nt * 16 + r;
    nvalid[nt] = i_lane < K;
    wrow[nt] = nvalid[nt] ? static_cast<size_t>(COMPACT ? i_lane : idx[i_lane]) * d : 0;
  }

  // Epilogue elements of this thread: e = tid + NTH j -> (token e / NB, mask
  // position e % NB).  Their neuron rows and anchor activations are fetched
  // now, so that the wait for them overlaps the weight loads below.
  constexpr int NE = TT * NB;                 // epilogue elements of the workgroup
  constexpr int EPT = (NE + NTH - 1) / NTH;
  size_t hn[EPT];
  bool ev[EPT];
  float ha[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + NTH * j;
    const int i = i0 + e % NB, sg = s0 + e / NB;
    ev[j] = e < NE && i < K && sg < S;
    hn[j] = (ev[j] && idx) ? static_cast<size_t>(idx[i]) * S_all + (tok ? tok[sg] : sg) : 0;
    ha[j] = (ev[j] && h_anchor) ? h_anchor[hn[j]] : 0.f;
  }
  const T* xrow[MTW];
  bool tvalid[MTW];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
    const int s = s0 + mt * 16 + r;
    tvalid[mt] = s < S;
    xrow[mt] = x + static_cast<size_t>(tvalid[mt] ? (tok ? tok[s] : s) : 0) * d;
  }

  f32x4_t ag[MTW][NTW], au[MTW][NTW];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) ag[mt][nt] = au[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int CH = kChunk;  // 32-wide K steps per load batch
  const int kb = wave * dq, ke = kb + dq;
  for (int k0 = kb; k0 < ke; k0 += CH * 32) {
    Frag<T> bg[CH][NTW], bu[CH][NTW], a[CH][MTW];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int kk = k0 + c * 32 + grp * 8;
      const bool kv = k0 + c * 32 < ke;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (nvalid[nt] && kv) { bg[c][nt].load(wg + wrow[nt] + kk); bu[c][nt].load(wu + wrow[nt] + kk); }
        else { bg[c][nt].zero(); bu[c][nt].zero(); }
      }
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        if (tvalid[mt] && kv) a[c][mt].load(xrow[mt] + kk); else a[c][mt].zero();
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          ag[mt][nt] = mma(a[c][mt], bg[c][nt], ag[mt][nt]);
          au[mt][nt] = mma(a[c][mt], bu[c][nt], au[mt][nt]);
        }
  }
  // Lane holds rows (tokens) mt*16 + 4*grp + v of column (mask position) nt*16 + r.
  __shared__ float part[NW][2][TT][NB];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        part[wave][0][mt * 16 + 4 * grp + v][nt * 16 + r] = ag[mt][nt][v];
        part[wave][1][mt * 16 + 4 * grp + v][nt * 16 + r] = au[mt][nt][v];
      }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + NTH * j;
    if (NE % NTH != 0 && e >= NE) break;
    const int s = e / NB, c = e % NB;
    float gsum = part[0][0][s][c], usum = part[0][1][s][c];
#pragma unroll
    for (int q = 1; q < NW; ++q) {
      gsum += part[q][0][s][c];
      usum += part[q][1][s][c];
    }
    const int i = i0 + c, sg = s0 + s;
    float delta = 0.f;
    if (ev[j]) {
      const float h = gelu_tanh(gsum) * usum;
      if (h_out) h_out[hn[j]] = h;
      delta = h - ha[j];
    }
    if (i < K_pad) D[static_cast<size_t>(sg) * K_pad + i] = Elem<T>::from_f32(delta);
  }
}

// B fragment of a 16x16x32 MFMA read column-major out of a [32 rows][pitch]
// LDS tile: lane (col, grp) takes the 8 rows grp*8 .. grp*8+7 of its column.
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

template <typename T, bool COMPACT>
__global__ __launch_bounds__(kThreads) void act_down_kernel(
    const T* __restrict__ D, int S, int K_pad, const int32_t* __restrict__ idx, int K,
    const T* __restrict__ wd, int d, int steps_per_split, float* __restrict__ part) {
  constexpr int RB = kCols * static_cast<int>(sizeof(T));  // bytes of a row segment
  constexpr int RPD = 1024 / RB;                           // rows per 1 KB DMA transfer
  constexpr int DPS = kStep / RPD;                         // transfers per K step
  __shared__ __attribute__((aligned(1024))) char tile[kMaxSteps * kStep * RB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, grp = lane >> 4;
  // logical tile: column block fastest, so the column blocks of one split
  // (the same delta rows, neighbouring 64-byte halves of W_down lines) run on
  // one XCD
  const int2 tl = xcd_tile(gridDim.x);
  const int j0 = tl.x * kCols;
  const int split = tl.y;
  const int s0 = blockIdx.z * kTokDown;
  const int st_begin = split * steps_per_split;
  const int nst = min(K_pad / kStep, st_begin + steps_per_split) - st_begin;

  // Every row segment of this workgroup's mask range, global -> LDS.  Rows
  // past K read the last mask row (their D entries are zero).  All index
  // loads are issued before the first transfer, so no wait for an index
  // also waits for an earlier transfer.
  constexpr int QMAX = kMaxSteps * DPS / 4;  // transfers per wave, at most
  const uint32_t lds0 = lds_addr(tile);
  const int lrow = lane / (RB / 16), lchunk = lane % (RB / 16);
  const int nq = nst * DPS;
  int src[QMAX];
#pragma unroll
  for (int t = 0; t < QMAX; ++t) {
    const int q = wave + 4 * t;
    const int i = min(st_begin * kStep + q * RPD + lrow, K - 1);
    src[t] = (q < nq) ? (COMPACT ? i : idx[i]) : 0;
  }
#pragma unroll
  for (int t = 0; t < QMAX; ++t) {
    const int q = wave + 4 * t;
    if (q < nq)
      dma_1k(lds0 + q * 1024, wd,
             static_cast<uint32_t>(src[t]) * static_cast<uint32_t>(d) * sizeof(T) +
                 static_cast<uint32_t>(j0) * sizeof(T) + lchunk * 16);
  }
  // A fragments (the deltas of this lane's token row) of every K step.
  const int srow = s0 + wave * 16 + r;  // token row of this lane's A fragment
  Frag<T> a[kMaxSteps];
#pragma unroll
  for (int st = 0; st < kMaxSteps; ++st) {
    if (st < nst) a[st].load(D + static_cast<size_t>(srow) * K_pad + (st_begin + st) * kStep + grp * 8);
    else a[st].zero();
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  constexpr int NTD = kCols / 16;  // 16-column MFMA tiles per wave
  f32x4_t acc[NTD];
#pragma unroll
  for (int nt = 0; nt < NTD; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < kMaxSteps; ++st) {
    if (st >= nst) break;
    const char* tl = tile + st * kStep * RB;
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt) {
      Frag<T> b;
      gather_b_frag<T>(tl, RB, nt * 16 + r, grp, b);
      acc[nt] = mma(a[st], b, acc[nt]);
    }
  }
  const size_t so = static_cast<size_t>(split) * S * d;
#pragma unroll
  for (int nt = 0; nt < NTD; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int s = s0 + wave * 16 + 4 * grp + v;
      if (s < S) part[so + static_cast<size_t>(s) * d + j0 + nt * 16 + r] = acc[nt][v];
    }
}

// One workgroup per token row: y = y_a + sum over splits (split order), then
// the optional residual/RMSNorm glue on the rounded y.
// Output row s = blockIdx.x of S_all.  With tok (ascending, S entries), the
// partials hold only the rows tok[i]: row s takes partial row i if tok[i] = s
// and none otherwise (y = y_a).
template <typename T>
__global__ __launch_bounds__(kThreads) void act_finish_kernel(
    const float* __restrict__ part, int splits, int S, int d, const float* __restrict__ y_anchor,
    T* __restrict__ y_out, float* __restrict__ y_f32, GlueArgs<T> glue, const int32_t* __restrict__ tok) {
  __shared__ float red[kThreads / 64];
  const int s = blockIdx.x;
  const size_t ro = static_cast<size_t>(s) * d;
  const size_t n = static_cast<size_t>(S) * d;
  size_t po = ro;  // this row's partials
  if (tok) {
    int lo = 0, hi = S;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(tok[mid]) < s) lo = mid + 1; else hi = mid;
    }
    if (lo < S && tok[lo] == s) po = static_cast<size_t>(lo) * d;
    else splits = 0;
  }
  float ss = 0.f;
  float keep[kGlueKeep][8];
  int j = 0;
  for (int c = threadIdx.x * 8; c < d; c += kThreads * 8, ++j) {
    float v[8], rr[8], b[8];
    if (glue.r) glue_prefetch(glue, ro, c, rr, b);
    if (y_anchor) Row8<float>::load(y_anchor + ro + c, v);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    add_splits(part + po + c, n, splits, v);
    if (y_f32) Row8<float>::store(y_f32 + ro + c, v);
    Row8<T>::store(y_out + ro + c, v);
    if (glue.r) {
      ss += glue_add(glue, ro, c, v, rr, b);
      if (j < kGlueKeep) {
#pragma unroll
        for (int e = 0; e < 8; ++e) keep[j][e] = rr[e];
      }
    }
  }
  if (glue.r && glue.x_next) glue_norm(glue, ro, d, ss, red, keep);
}

// Rows idx[0..K-1] of three [ff][d] matrices into compact [K][d] buffers:
// one wavefront per row, 16 bytes per lane per access.
template <typename T>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const T* __restrict__ a, const T* __restrict__ b,
                                                               const T* __restrict__ c,
                                                               const int32_t* __restrict__ idx, int K, int d,
                                                               T* __restrict__ ao, T* __restrict__ bo,
                                                               T* __restrict__ co) {
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= 3 * K) return;
  const int m = row / K, i = row - m * K;
  const T* src = (m == 0 ? a : m == 1 ? b : c) + static_cast<size_t>(idx[i]) * d;
  T* dst = (m == 0 ? ao : m == 1 ? bo : co) + static_cast<size_t>(i) * d;
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  for (int e = (threadIdx.x & 63) * V; e < d; e += 64 * V)
    *reinterpret_cast<u32x4_t*>(dst + e) = *reinterpret_cast<const u32x4_t*>(src + e);
}

// act_gather_rows over several layers in one launch: global row r of the
// launch is row (r - first[l]) of layer l's three matrices, one wavefront
// per row (matrix-major within a layer, as gather_rows_kernel).
constexpr int kGatherMaxLayers = 32;  // the table travels as a kernel argument (about 2 KB)
template <typename T> struct GatherTable {
  const T* src[kGatherMaxLayers][3];
  T* dst[kGatherMaxLayers][3];
  const int32_t* idx[kGatherMaxLayers];
  int first[kGatherMaxLayers + 1];  // prefix of 3 K per layer
  int K[kGatherMaxLayers];
  int n, d;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void gather_layers_kernel(GatherTable<T> tab) {
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= tab.first[tab.n]) return;
  int l = 0;
  while (l + 1 < tab.n && row >= tab.first[l + 1]) ++l;
  const int r = row - tab.first[l];
  const int K = tab.K[l];
  const int m = r / K, i = r - m * K;
  const T* src = tab.src[l][m] + static_cast<size_t>(tab.idx[l][i]) * tab.d;
  T* dst = tab.dst[l][m] + static_cast<size_t>(i) * tab.d;
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  for (int e = (threadIdx.x & 63) * V; e < tab.d; e += 64 * V)
    *reinterpret_cast<u32x4_t*>(dst + e) = *reinterpret_cast<const u32x4_t*>(src + e);
}

struct ActPlan {
  int K_pad, S_pad, tt, splits, steps_per_split;
  size_t d_elems, part_elems;
};

ActPlan plan_act(int S, int K, int d) {
  ActPlan p{};
  p.K_pad = (K + kStep - 1) / kStep * kStep;
  p.tt = S <= 16 ? 16 : 32;  // tokens per GLU workgroup
  p.S_pad = (S + kTokDown - 1) / kTokDown * kTokDown;
  const int steps = p.K_pad / kStep;
  // up to kDownSplits K splits (fewer partials for the finish kernel; measured
  // best for the 18-layer expert's ~1250-row masks), more only when a split
  // would exceed the kMaxSteps rows of W_down that fit in LDS
  int splits = std::max(1, std::min(std::max(steps, 1), kDownSplits));
  splits = std::max(splits, (steps + kMaxSteps - 1) / kMaxSteps);
  p.steps_per_split = std::max(1, (steps + splits - 1) / splits);
  p.splits = steps > 0 ? (steps + p.steps_per_split - 1) / p.steps_per_split : 0;
  p.d_elems = static_cast<size_t>(p.S_pad) * p.K_pad;
  p.part_elems = static_cast<size_t>(p.splits) * S * d;
  return p;
}

// The down projection reads W_down rows by LDS DMA (32-bit byte offsets):
// the [ff][d] matrix it addresses spans < 2^32 bytes (4-byte elements, the
// wider type).
bool act_shape_ok(int d, int ff) { return d > 0 && ff > 0 && d % 128 == 0 && dma_span_ok(ff, d, 4); }

// S rows computed (rows tok[0..S) of S_all when tok is given, else all).
// dense: the mask takes every neuron (profiling site names only).
template <typename T, bool COMPACT>
int act_t(const cgs_ffn& w, const T* x, int S, const int32_t* idx, int K, const float* ya,
          const float* ha, T* y_out, float* y_f32, float* h_out, const cgs_glue* gl, void* ws,
          hipStream_t s, bool dense, const int32_t* tok = nullptr, int S_all = -1) {
  if (S_all < 0) S_all = S;
  const ActPlan p = plan_act(S, K, w.d);
  Carve cv(ws);
  T* D = cv.take<T>(p.d_elems);
  float* part = cv.take<float>(std::max<size_t>(p.part_elems, 1));
  if (K > 0 && S > 0) {
    {
      ProfScope ps(dense ? "act.glu.dense" : "act.glu.masked", s);
      const T* wgp = static_cast<const T*>(w.w_gate);
      const T* wup = static_cast<const T*>(w.w_up);
      // Masks of dense size with at most 64 tokens: one 64-token workgroup per
      // 16 positions, so every weight row is read once and the grid keeps
      // K/16 workgroups.  Otherwise two 16-wide position tiles per workgroup
      // for large masks (x is then read once per 32 positions) and one for
      // small ones (more workgroups).
      const bool dense64 = sizeof(T) == 2 && K >= kWideGluK && p.S_pad <= 64;
      const int tt = dense64 ? 64 : p.tt;
      const int ntw = (K >= kWideGluK && !dense64) ? 2 : 1;
      const dim3 grid((p.K_pad + 16 * ntw - 1) / (16 * ntw), (p.S_pad + tt - 1) / tt);
      // NW waves split d (8 when d allows: more loads in flight per workgroup)
      const bool w8 = w.d % (kGluWaves * 32) == 0;
      const dim3 blk(w8 ? 64 * kGluWaves : kThreads);
#define CGS_GLU(MTW_, NTW_)                                                                              \
  do {                                                                                                   \
    if (w8)                                                                                              \
      hipLaunchKernelGGL((act_glu_kernel<T, MTW_, NTW_, COMPACT, kGluWaves>), grid, blk, 0, s, x, S, w.d, idx, K, \
                         p.K_pad, wgp, wup, ha, h_out, D, tok, S_all);                                   \
    else                                                                                                 \
      hipLaunchKernelGGL((act_glu_kernel<T, MTW_, NTW_, COMPACT, 4>), grid, blk, 0, s, x, S, w.d, idx, K, \
                         p.K_pad, wgp, wup, ha, h_out, D, tok, S_all);                                   \
  } while (0)
      if (tt == 64) {
        if constexpr (sizeof(T) == 2) CGS_GLU(4, 1);
      } else if (tt == 16 && ntw == 1) CGS_GLU(1, 1);
      else if (tt == 16) CGS_GLU(1, 2);
      else if (ntw == 1) CGS_GLU(2, 1);
      else CGS_GLU(2, 2);
#undef CGS_GLU
    }
    if (!launch_ok()) return CGS_ERR_LAUNCH;
    ProfScope ps(dense ? "act.down.dense" : "act.down.masked", s);
    hipLaunchKernelGGL((act_down_kernel<T, COMPACT>), dim3(w.d / kCols, p.splits, p.S_pad / kTokDown), dim3(kThreads),
                       0, s, D, S, p.K_pad, idx, K, static_cast<const T*>(w.w_down), w.d,
                       p.steps_per_split, part);
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  ProfScope ps("act.finish", s);
  hipLaunchKernelGGL((act_finish_kernel<T>), dim3(S_all), dim3(kThreads), 0, s, part,
                     (K > 0 && S > 0) ? p.splits : 0, S, w.d, ya, y_out, y_f32, make_glue<T>(gl, w.d), tok);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}

// act_ffn_masked_compact once its arguments are checked.
// dense: profiling site names only (a layer without anchor state in a chain).
int act_compact(const cgs_ffn& wc, const void* x, int S, const int32_t* idx, int K, const float* ya,
                const float* ha, void* y_out, float* y_f32, float* h_out, const cgs_glue* gl, void* ws,
                hipStream_t s, bool dense = false) {
  if (wc.dtype == CGS_BF16)
    return act_t<uint16_t, true>(wc, static_cast<const uint16_t*>(x), S, idx, K, ya, ha,
                                 static_cast<uint16_t*>(y_out), y_f32, h_out, gl, ws, s, dense);
  return act_t<float, true>(wc, static_cast<const float*>(x), S, idx, K, ya, ha, static_cast<float*>(y_out),
                            y_f32, h_out, gl, ws, s, dense);
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
                              float* y_f32_out, float* h_out, const cgs_glue* glue, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down || !valid_dtype(w->dtype) ||
      w->down_layout != CGS_DOWN_FD || !x || !y_out || (K > 0 && !idx) || !glue_ok(glue))
    return CGS_ERR_ARG;
  if (!act_shape_ok(w->d, w->ff)) return CGS_ERR_UNSUPPORTED;
  if (S < 0 || K < 0 || K > w->ff) return CGS_ERR_SHAPE;
  if (S == 0) return CGS_OK;
  if (!ws || ws_bytes < cgs_act_ffn_masked_workspace(S, K, w->d, w->ff)) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int st = validate_index(idx, K, w->ff, s)) return st;
  // An ascending, duplicate-free list of ff neurons is 0 .. ff-1: the full
  // weights are then the compact weights of the mask, and no kernel waits
  // for an index before it can address a weight row (the list still
  // addresses the h_anchor / h_out rows, off that chain).
  if (K == w->ff) {
    if (w->dtype == CGS_BF16)
      return act_t<uint16_t, true>(*w, static_cast<const uint16_t*>(x), S, idx, K, y_anchor, h_anchor,
                                   static_cast<uint16_t*>(y_out), y_f32_out, h_out, glue, ws, s, true);
    return act_t<float, true>(*w, static_cast<const float*>(x), S, idx, K, y_anchor, h_anchor,
                              static_cast<float*>(y_out), y_f32_out, h_out, glue, ws, s, true);
  }
  if (w->dtype == CGS_BF16)
    return act_t<uint16_t, false>(*w, static_cast<const uint16_t*>(x), S, idx, K, y_anchor, h_anchor,
                                  static_cast<uint16_t*>(y_out), y_f32_out, h_out, glue, ws, s, false);
  return act_t<float, false>(*w, static_cast<const float*>(x), S, idx, K, y_anchor, h_anchor,
                             static_cast<float*>(y_out), y_f32_out, h_out, glue, ws, s, false);
}

extern "C" int act_ffn_masked_compact(const cgs_ffn* wc, const void* x, int S, const int32_t* idx, int K,
                                      const float* y_anchor, const float* h_anchor, void* y_out,
                                      float* y_f32_out, float* h_out, const cgs_glue* glue, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (!wc || (K > 0 && (!wc->w_gate || !wc->w_up || !wc->w_down)) || !valid_dtype(wc->dtype) ||
      wc->down_layout != CGS_DOWN_FD || !x || !y_out || !glue_ok(glue) ||
      (K > 0 && !idx && (h_anchor || h_out)))
    return CGS_ERR_ARG;
  if (!act_shape_ok(wc->d, std::max(wc->ff, 1))) return CGS_ERR_UNSUPPORTED;
  if (S < 0 || K < 0 || K != wc->ff) return CGS_ERR_SHAPE;
  if (S == 0) return CGS_OK;
  if (!ws || ws_bytes < cgs_act_ffn_masked_workspace(S, K, wc->d, std::max(K, 1))) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int st = validate_index(idx, K, INT32_MAX, s)) return st;
  return act_compact(*wc, x, S, idx, K, y_anchor, h_anchor, y_out, y_f32_out, h_out, glue, ws, s);
}

namespace cgs {
namespace {
// The checks of act_ffn_masked_compact for one layer of a chain.
int masked_layer_status(const cgs_masked_layer& L, int d, int dtype) {
  const cgs_ffn& wc = L.w;
  const int K = wc.ff;
  if ((K > 0 && (!wc.w_gate || !wc.w_up || !wc.w_down)) || wc.dtype != dtype ||
      wc.down_layout != CGS_DOWN_FD || (K > 0 && !L.idx && (L.h_anchor || L.h_out)))
    return CGS_ERR_ARG;
  if (wc.d != d) return CGS_ERR_SHAPE;
  if (!act_shape_ok(wc.d, std::max(wc.ff, 1))) return CGS_ERR_UNSUPPORTED;
  if (K < 0) return CGS_ERR_SHAPE;
  return CGS_OK;
}
}  // namespace
}  // namespace cgs

extern "C" size_t cgs_act_masked_layers_workspace(int S, int d, int K_max) {
  if (S <= 0 || K_max < 0 || d <= 0) return 0;
  const size_t ffn = cgs_act_ffn_masked_workspace(S, std::max(K_max, 1), d, std::max(K_max, 1));
  if (ffn == 0) return 0;
  return ffn + align_up(static_cast<size_t>(S) * d * 4, 256);  // y of layers without y_out
}

extern "C" int act_masked_layers(const cgs_masked_layer* layers, int n, int S, float* r, void* x, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (n < 0 || S < 0) return CGS_ERR_SHAPE;
  if (n == 0 || S == 0) return CGS_OK;
  if (!layers || !r || !x) return CGS_ERR_ARG;
  const int d = layers[0].w.d, dt = layers[0].w.dtype;
  if (!valid_dtype(dt)) return CGS_ERR_ARG;
  int K_max = 0;
  for (int i = 0; i < n; ++i) {
    if (const int st = masked_layer_status(layers[i], d, dt)) return st;
    K_max = std::max(K_max, layers[i].w.ff);
  }
  const size_t need = cgs_act_masked_layers_workspace(S, d, K_max);
  if (need == 0) return CGS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < need) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_on())
    for (int i = 0; i < n; ++i)
      if (const int st = validate_index(layers[i].idx, layers[i].w.ff, INT32_MAX, s)) return st;
  const size_t ffn_ws = need - align_up(static_cast<size_t>(S) * d * 4, 256);
  void* y_scratch = static_cast<char*>(ws) + ffn_ws;
  const size_t row_bytes = static_cast<size_t>(S) * d * elem_bytes(dt);
  char* xs = static_cast<char*>(x);
  for (int i = 0; i < n; ++i) {
    const cgs_masked_layer& L = layers[i];
    cgs_glue g{};
    g.r = r;
    g.bias = L.bias;
    g.x_next = xs + (i + 1) * row_bytes;
    const int st = act_compact(L.w, xs + i * row_bytes, S, L.idx, L.w.ff, L.y_anchor, L.h_anchor,
                               L.y_out ? L.y_out : y_scratch, L.y_f32_out, L.h_out, &g, ws, s,
                               !L.y_anchor && !L.h_anchor);
    if (st != CGS_OK) return st;
  }
  return CGS_OK;
}

// Scratch of act_ffn_masked_compact_noalloc: the deltas and split partials
// that the caller's workspace holds otherwise.  Each GPU has its own copy;
// host code uses only the per-device address from hipGetSymbolAddress (the
// array's name on the host is a stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[CGS_NOALLOC_SCRATCH_BYTES];

namespace cgs {
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// The scratch array's device address on the current device, looked up once
// per device with that device current.
int scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return CGS_ERR_LAUNCH;
  if (s) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return CGS_ERR_ARG;
    if (sdev != dev) return CGS_ERR_ARG;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CGS_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CGS_OK;
}
}  // namespace
}  // namespace cgs

extern "C" int act_ffn_masked_compact_noalloc(const cgs_ffn* wc, const void* x, int S, const int32_t* idx,
                                              int K, const float* y_anchor, const float* h_anchor,
                                              void* y_out, float* y_f32_out, float* h_out,
                                              const cgs_glue* glue, void* stream) {
  if (!wc || (K > 0 && (!wc->w_gate || !wc->w_up || !wc->w_down)) || !valid_dtype(wc->dtype) ||
      wc->down_layout != CGS_DOWN_FD || !x || !y_out || !glue_ok(glue) ||
      (K > 0 && !idx && (h_anchor || h_out)))
    return CGS_ERR_ARG;
  if (!act_shape_ok(wc->d, std::max(wc->ff, 1))) return CGS_ERR_UNSUPPORTED;
  if (S < 0 || K < 0 || K != wc->ff) return CGS_ERR_SHAPE;
  if (S == 0) return CGS_OK;
  if (cgs_act_ffn_masked_workspace(S, K, wc->d, std::max(K, 1)) > CGS_NOALLOC_SCRATCH_BYTES)
    return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (const int st = scratch_address(s, &ws)) return st;
  // no checked-mode pass here: it synchronises and allocates
  return act_compact(*wc, x, S, idx, K, y_anchor, h_anchor, y_out, y_f32_out, h_out, glue, ws, s);
}

extern "C" int act_ffn_joint(const cgs_ffn* wc, const void* x, int S, const int32_t* tok, int k,
                             const int32_t* idx, int K, const float* y_anchor, const float* h_anchor,
                             void* y_out, float* y_f32_out, const cgs_glue* glue, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!wc || (K > 0 && (!wc->w_gate || !wc->w_up || !wc->w_down)) || !valid_dtype(wc->dtype) ||
      wc->down_layout != CGS_DOWN_FD || !x || !y_out || !y_anchor || !glue_ok(glue) ||
      (k > 0 && !tok) || (K > 0 && k > 0 && (!idx || !h_anchor)))
    return CGS_ERR_ARG;
  if (!act_shape_ok(wc->d, std::max(wc->ff, 1))) return CGS_ERR_UNSUPPORTED;
  if (S < 0 || k < 0 || k > S || K < 0 || K != wc->ff) return CGS_ERR_SHAPE;
  if (S == 0) return CGS_OK;
  if (!ws || ws_bytes < cgs_act_ffn_masked_workspace(std::max(k, 1), K, wc->d, std::max(K, 1)))
    return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int st = validate_index(tok, k, S, s)) return st;
  if (K > 0 && k > 0)
    if (const int st = validate_index(idx, K, INT32_MAX, s)) return st;
  // with k = 0 every row is unselected: no partials (tok is not read)
  if (wc->dtype == CGS_BF16)
    return act_t<uint16_t, true>(*wc, static_cast<const uint16_t*>(x), k, idx, K, y_anchor, h_anchor,
                                 static_cast<uint16_t*>(y_out), y_f32_out, nullptr, glue, ws, s, false, tok, S);
  return act_t<float, true>(*wc, static_cast<const float*>(x), k, idx, K, y_anchor, h_anchor,
                            static_cast<float*>(y_out), y_f32_out, nullptr, glue, ws, s, false, tok, S);
}

namespace {
template <typename T>
int gather_layers_t(const cgs_gather_layer* layers, int n, hipStream_t s) {
  GatherTable<T> tab{};
  tab.n = 0;
  tab.d = layers[0].w.d;
  int rows = 0;
  for (int i = 0; i < n; ++i) {
    const cgs_gather_layer& L = layers[i];
    if (L.K == 0) continue;
    const int l = tab.n++;
    tab.src[l][0] = static_cast<const T*>(L.w.w_gate);
    tab.src[l][1] = static_cast<const T*>(L.w.w_up);
    tab.src[l][2] = static_cast<const T*>(L.w.w_down);
    tab.dst[l][0] = static_cast<T*>(L.wg_out);
    tab.dst[l][1] = static_cast<T*>(L.wu_out);
    tab.dst[l][2] = static_cast<T*>(L.wd_out);
    tab.idx[l] = L.idx;
    tab.K[l] = L.K;
    tab.first[l] = rows;
    rows += 3 * L.K;
  }
  tab.first[tab.n] = rows;
  if (rows == 0) return CGS_OK;
  ProfScope ps("act.gather", s);
  const dim3 grid((rows + kThreads / 64 - 1) / (kThreads / 64));
  hipLaunchKernelGGL((gather_layers_kernel<T>), grid, dim3(kThreads), 0, s, tab);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}
}  // namespace

extern "C" int act_gather_rows_layers(const cgs_gather_layer* layers, int n, void* stream) {
  if (n < 1 || n > kGatherMaxLayers) return CGS_ERR_SHAPE;
  if (!layers) return CGS_ERR_ARG;
  const int d = layers[0].w.d, dt = layers[0].w.dtype;
  if (!valid_dtype(dt)) return CGS_ERR_ARG;
  long long rows = 0;
  for (int i = 0; i < n; ++i) {
    const cgs_gather_layer& L = layers[i];
    if (!L.w.w_gate || !L.w.w_up || !L.w.w_down || L.w.dtype != dt || L.w.down_layout != CGS_DOWN_FD)
      return CGS_ERR_ARG;
    if (L.w.d != d) return CGS_ERR_SHAPE;
    if (!act_shape_ok(L.w.d, L.w.ff)) return CGS_ERR_UNSUPPORTED;
    if (L.K < 0 || L.K > L.w.ff) return CGS_ERR_SHAPE;
    if (L.K > 0 && (!L.idx || !L.wg_out || !L.wu_out || !L.wd_out)) return CGS_ERR_ARG;
    rows += 3ll * L.K;
  }
  if (rows > INT32_MAX - 64) return CGS_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_on())
    for (int i = 0; i < n; ++i)
      if (const int st = validate_index(layers[i].idx, layers[i].K, layers[i].w.ff, s)) return st;
  return dt == CGS_BF16 ? gather_layers_t<uint16_t>(layers, n, s) : gather_layers_t<float>(layers, n, s);
}

extern "C" int act_gather_rows(const cgs_ffn* w, const int32_t* idx, int K, void* wg_out, void* wu_out,
                               void* wd_out, void* stream) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down || !valid_dtype(w->dtype) ||
      w->down_layout != CGS_DOWN_FD)
    return CGS_ERR_ARG;
  if (!act_shape_ok(w->d, w->ff)) return CGS_ERR_UNSUPPORTED;
  if (K < 0 || K > w->ff) return CGS_ERR_SHAPE;
  if (K == 0) return CGS_OK;
  if (!idx || !wg_out || !wu_out || !wd_out) return CGS_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int st = validate_index(idx, K, w->ff, s)) return st;
  ProfScope ps("act.gather", s);
  const dim3 grid((3 * K + kThreads / 64 - 1) / (kThreads / 64));
  if (w->dtype == CGS_BF16)
    hipLaunchKernelGGL((gather_rows_kernel<uint16_t>), grid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(w->w_gate), static_cast<const uint16_t*>(w->w_up),
                       static_cast<const uint16_t*>(w->w_down), idx, K, w->d, static_cast<uint16_t*>(wg_out),
                       static_cast<uint16_t*>(wu_out), static_cast<uint16_t*>(wd_out));
  else
    hipLaunchKernelGGL((gather_rows_kernel<float>), grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(w->w_gate), static_cast<const float*>(w->w_up),
                       static_cast<const float*>(w->w_down), idx, K, w->d, static_cast<float*>(wg_out),
                       static_cast<float*>(wu_out), static_cast<float*>(wd_out));
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}
