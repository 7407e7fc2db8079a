// Dense and gathered GeGLU FFN on bf16 MFMA (fp32 MFMA for fp32 data).
//
//   ctx_ffn_recompute  rMuscle §4.1, Eq. 3: recompute the FFN for the
//                      selected rows only and scatter them into a copy of the
//                      cached reference outputs.
//   ref_rebuild_dense  §4.2 (asynchronous online reconstruction): dense
//                      prefill of a compact entry into per-layer reference
//                      inputs and outputs.
//   cgs_residual_rmsnorm  residual add + RMSNorm glue between layers.
//
// Both projections run on the GEMM core of gemm.hpp (LDS-DMA pipelined bf16
// MFMA).  Gate/up fuses gelu_tanh(g) * u into its epilogue and stores h
// rounded to the activation type; the down projection splits K (ff) and
// writes fp32 partials, which the row-finish kernel sums in a fixed split
// order.  The finish scatters the selected rows into the output and copies
// the reference bits of the others (Context Cache), or adds the residual and
// normalises the next layer's input (rebuild).  Selected rows are gathered
// straight from x through the index list, never copied.
//
// Tile choice by the number of rows M (the selected tokens k, or P for the
// rebuild), all with 8 waves except the smallest:
//   M <= 64   64 x 128, 4 waves
//   M <= 128  128 x 128
//   M <= 256  128 x 256 gate/up tiles with 32 x 128 wave tiles (bf16 with
//             d % 256 == 0; the 231-row Context Cache layer: 2 x 128 tiles,
//             one round of 256 workgroups), 256 x 128 otherwise; the down
//             projection keeps 128 x 128 tiles (2 x 16 tiles x 8 K splits)
//   M > 256   192 x 256 (bf16 with d % 256 == 0: the 768-row rebuild is
//             4 x 128 gate/up tiles and 4 x 8 x 8 down tiles); gate/up at
//             2048 rows or more (a batched rebuild) 256 x 256; else 256 x 128.
// A launch with more tiles than CUs, full row tiles and no gathered rows
// runs persistently (launch_cfg): the 768-row gate/up projection as 256
// workgroups of 2 tiles, the 3072-row one (4 entries) of 6.
#include <algorithm>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "gemm.hpp"
#include "glue.hpp"
#include "profile.hpp"
#include "validate.hpp"

namespace cgs {
namespace {

constexpr int kRowThreads = 256;
constexpr int kFinishIdxLds = 4096;  // index lists up to this length are searched in LDS

// Tile configurations <BM, WM, WN, NT, SA, SB> (BN = 16 NT WN; A and B ring
// depths).  The weight (B) ring runs deeper: on the selective path the
// weights stream from HBM while the gathered rows (A) hit L2.  The 256 x 256
// tile of a batched rebuild is the exception: its x rows come back from the
// MALL (each XCD's L2 cannot hold a round's operands) while its weight tiles
// are shared by the XCD's workgroups, so its A ring is the deeper one
// (3 + 2 stages measured 3% faster than 2 + 3, bit-identical), and so is that
// of the 192 x 256 tile of a dense gate/up projection (768 and 1536 rows: 5%
// and 3% faster).  The down projection keeps 2 + 3 (1536 rows: 2.5% slower
// with 3 + 2).
using CfgS = GemmCfg<64, 2, 2, 4, 2, 4>;    //  64 x 128, 4 waves,  80 KB LDS
using CfgM = GemmCfg<128, 4, 2, 4, 2, 4>;   // 128 x 128, 8 waves,  96 KB
using CfgL = GemmCfg<256, 4, 2, 4, 2, 5>;   // 256 x 128, 8 waves, 144 KB
using CfgX = GemmCfg<192, 2, 4, 4, 2, 3>;   // 192 x 256, 8 waves, 144 KB
using CfgXG = GemmCfg<192, 2, 4, 4, 3, 2>;  // the same tile for a dense gate/up projection, 136 KB
using CfgG = GemmCfg<128, 4, 2, 8, 2, 4>;   // 128 x 256, 8 waves, 160 KB (32 x 128 wave tiles)
using CfgW = GemmCfg<256, 2, 4, 4, 3, 2>;   // 256 x 256, 8 waves, 160 KB (128 x 64 wave tiles)
enum TileId { kTileS = 0, kTileM = 1, kTileL = 2, kTileX = 3, kTileG = 4, kTileW = 5 };
// Rows from which the gate/up projection takes 256 x 256 tiles (a batched
// rebuild): a third more MFMA work per K tile's barrier and transfers than
// 192 x 256, and enough row tiles that the tiles divide evenly over the CUs.
constexpr int kWideRows = 2048;

constexpr int kLdsPerCu = 160 * 1024;

// Compute units of the current device, cached per device (0 if the query fails).
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(cache.size()) <= dev) cache.resize(dev + 1, -1);
  if (cache[dev] < 0) {
    int cus = 0;
    cache[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? cus : 0;
  }
  return cache[dev];
}

// A tile configuration whose LDS rings leave room for one workgroup per CU
// runs persistently when the launch has more tiles than CUs: one workgroup per
// CU (a multiple of 8, so that each keeps its tiles on its XCD) takes every
// gridDim-th tile, and its rings run on from one tile into the next.  The
// kernel needs the same K range length for every tile, at least as many K
// tiles as ring stages, and no ragged row tile; gathered rows keep one tile
// per workgroup.
template <typename Cfg, typename T, bool GLU, bool GATHER>
void launch_cfg(const GemmArgs<T>& g, const char* site, hipStream_t s) {
  ProfScope ps(site, s);
  const int nb = g.n_tiles * g.m_tiles * g.splits;
  if constexpr (!GATHER && 2 * Cfg::kLds > kLdsPerCu) {
    constexpr int bk = 128 / static_cast<int>(sizeof(T));
    const int cus = device_cus() / kXcds * kXcds;
    if (cus > 0 && nb > cus && g.M % Cfg::kBM == 0 && g.K % g.k_per_split == 0 &&
        g.k_per_split % bk == 0 && g.k_per_split / bk >= std::max(Cfg::kSA, Cfg::kSB)) {
      hipLaunchKernelGGL(
          (gemm_kernel_persist<T, Cfg::kBM, Cfg::kWM, Cfg::kWN, Cfg::kNT, Cfg::kSA, Cfg::kSB, GLU>),
          dim3(cus), dim3(Cfg::kThreads), 0, s, g);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_kernel<T, Cfg::kBM, Cfg::kWM, Cfg::kWN, Cfg::kNT, Cfg::kSA, Cfg::kSB, GLU, GATHER>),
                     dim3(nb), dim3(Cfg::kThreads), 0, s, g);
}

template <typename T, bool GLU, bool GATHER>
void launch_tile(int tile, const GemmArgs<T>& g, const char* site, hipStream_t s) {
  switch (tile) {
    case kTileS: launch_cfg<CfgS, T, GLU, GATHER>(g, site, s); break;
    case kTileM: launch_cfg<CfgM, T, GLU, GATHER>(g, site, s); break;
    case kTileL: launch_cfg<CfgL, T, GLU, GATHER>(g, site, s); break;
    case kTileG:
      if constexpr (sizeof(T) == 2) launch_cfg<CfgG, T, GLU, GATHER>(g, site, s);
      break;
    case kTileW:
      if constexpr (sizeof(T) == 2) launch_cfg<CfgW, T, GLU, GATHER>(g, site, s);
      break;
    default:
      if constexpr (sizeof(T) == 2) {
        if constexpr (GLU && !GATHER) launch_cfg<CfgXG, T, GLU, GATHER>(g, site, s);
        else launch_cfg<CfgX, T, GLU, GATHER>(g, site, s);
      }
      break;
  }
}

// One workgroup per output row p; each thread owns runs of 8 elements.
//   selected (p = idx[i] when scattering, every row otherwise): y_out[p] =
//     round(sum over splits of the partials of row i, in split order);
//   unselected: y_out[p] = y_ref[p], bit for bit;
//   then the optional glue on the row's output (r += y (+ bias), x_next =
//   RMSNorm(r)).
// The selected position of p is found by a binary search over the ascending
// index list (wave-uniform loads).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void row_finish_kernel(
    const float* __restrict__ part, int splits, size_t split_stride, int d, bool scatter,
    const int32_t* __restrict__ idx, int k, const T* __restrict__ y_ref, T* __restrict__ y_out,
    GlueArgs<T> glue) {
  __shared__ float red[kRowThreads / 64];
  __shared__ int32_t sidx[kFinishIdxLds];
  const int p = blockIdx.x;
  int i = p;
  bool sel = true;
  if (scatter) {
    // first position with idx[pos] >= p; the list is staged in LDS when it fits
    int lo = 0, hi = k;
    if (k <= kFinishIdxLds) {
      for (int q = threadIdx.x; q < k; q += kRowThreads) sidx[q] = idx[q];
      __syncthreads();
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sidx[mid] < p) lo = mid + 1; else hi = mid;
      }
      sel = (lo < k) && (sidx[lo] == p);
    } else {
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(idx[mid]) < p) lo = mid + 1; else hi = mid;
      }
      sel = (lo < k) && (idx[lo] == p);
    }
    i = lo;
  }
  const size_t ro = static_cast<size_t>(p) * d;
  const size_t io = static_cast<size_t>(i) * d;
  float ss = 0.f;
  float keep[kGlueKeep][8];
  int j = 0;
  for (int c = threadIdx.x * 8; c < d; c += kRowThreads * 8, ++j) {
    float v[8], rr[8], b[8];
    if (glue.r) glue_prefetch(glue, ro, c, rr, b);
    if (!sel) {
      Row8<T>::copy(y_ref + ro + c, y_out + ro + c);
      if (!glue.r) continue;
      Row8<T>::load(y_ref + ro + c, v);
    } else {
      Row8<float>::load(part + io + c, v);
      add_splits(part + split_stride + io + c, split_stride, splits - 1, v);
      Row8<T>::store(y_out + ro + c, v);
    }
    if (glue.r) {
      ss += glue_add(glue, ro, c, v, rr, b);
      if (j < kGlueKeep) {
#pragma unroll
        for (int e = 0; e < 8; ++e) keep[j][e] = rr[e];
      }
    }
  }
  if (glue.r && glue.x_next) glue_norm_t<T, kRowThreads>(glue, ro, d, ss, red, keep);
}

// The same finish for d = 8 kRowThreads (each thread owns one run of 8
// elements), with the row's latency chain shortened: the index list is
// loaded first, then every load that does not depend on whether p is
// selected (residual, bias, the cached output row, the next layer's cached
// input row) goes out before the search, and only the split partials of a
// selected row wait for it.  The presence of the optional arguments is a
// template parameter and every load is unconditional (an absent bias reads
// the residual row and is not added), so the waits for these loads stay in
// issue order.  SCORE implies GLUE.
template <typename T, bool SCATTER, bool GLUE, bool SCORE>
__global__ __launch_bounds__(kRowThreads) void row_finish1_kernel(
    const float* __restrict__ part, int splits, size_t split_stride, int d,
    const int32_t* __restrict__ idx, int k, const T* __restrict__ y_ref, T* __restrict__ y_out,
    GlueArgs<T> glue) {
  constexpr int IR = kFinishIdxLds / kRowThreads;            // index-list entries per thread
  constexpr int RW = 4 * static_cast<int>(sizeof(T)) / 8;    // 16-byte words of 8 elements
  __shared__ float red[kRowThreads / 64];
  __shared__ int32_t sidx[kFinishIdxLds];
  const int p = blockIdx.x, tid = threadIdx.x, c = tid * 8;
  const size_t ro = static_cast<size_t>(p) * d;
  const bool staged = SCATTER && k <= kFinishIdxLds;
  int32_t iv[IR];
  if constexpr (SCATTER) {
    // with k = 0 the (unused) loads read the partial buffer, which always exists
    const int32_t* isrc = k > 0 ? idx : reinterpret_cast<const int32_t*>(part);
    const int last = k > 0 ? min(k, kFinishIdxLds) - 1 : 0;
#pragma unroll
    for (int q = 0; q < IR; ++q) iv[q] = isrc[min(tid + q * kRowThreads, last)];
  }
  float rr[1][8], bb[8];
  u32x4_t yraw[RW], sraw[RW];
  if constexpr (GLUE) {
    Row8<float>::load(glue.r + ro + c, rr[0]);
    Row8<float>::load((glue.bias ? glue.bias : glue.r + ro) + c, bb);
  }
  if constexpr (SCATTER) {
#pragma unroll
    for (int w = 0; w < RW; ++w) yraw[w] = reinterpret_cast<const u32x4_t*>(y_ref + ro + c)[w];
  }
  if constexpr (SCORE) {
#pragma unroll
    for (int w = 0; w < RW; ++w) sraw[w] = reinterpret_cast<const u32x4_t*>(glue.score_ref + ro + c)[w];
  }
  int i = p;
  bool sel = true;
  if constexpr (SCATTER) {
    int lo = 0, hi = k;
    if (staged) {
#pragma unroll
      for (int q = 0; q < IR; ++q) {
        const int e = tid + q * kRowThreads;
        if (e < k) sidx[e] = iv[q];
      }
      __syncthreads();
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sidx[mid] < p) lo = mid + 1; else hi = mid;
      }
      sel = (lo < k) && (sidx[lo] == p);
    } else {
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(idx[mid]) < p) lo = mid + 1; else hi = mid;
      }
      sel = (lo < k) && (idx[lo] == p);
    }
    i = lo;
  }
  float v[8];
  if (!sel) {
    // the cached row, bit for bit
#pragma unroll
    for (int w = 0; w < RW; ++w) reinterpret_cast<u32x4_t*>(y_out + ro + c)[w] = yraw[w];
    if constexpr (!GLUE) return;
    raw_to_f32<T>(yraw, v);
  } else {
    const size_t io = static_cast<size_t>(i) * d;
    Row8<float>::load(part + io + c, v);
    add_splits(part + split_stride + io + c, split_stride, splits - 1, v);
    Row8<T>::store(y_out + ro + c, v);
  }
  if constexpr (GLUE) {
    const float ss = glue_add(glue, ro, c, v, rr[0], bb);
    if (glue.x_next) {
      float sr[1][8];
      if constexpr (SCORE) raw_to_f32<T>(sraw, sr[0]);
      glue_norm_t<T, kRowThreads>(glue, ro, d, ss, red, rr, SCORE ? sr : nullptr);
    }
  }
}

template <typename T>
void launch_finish1(dim3 grid, hipStream_t s, const float* part, int splits, size_t split_stride, int d,
                    bool scatter, const int32_t* idx, int k, const T* y_ref, T* y_out, const GlueArgs<T>& g) {
  if (!scatter)
    hipLaunchKernelGGL((row_finish1_kernel<T, false, true, false>), grid, dim3(kRowThreads), 0, s, part,
                       splits, split_stride, d, idx, k, y_ref, y_out, g);
  else if (!g.r)
    hipLaunchKernelGGL((row_finish1_kernel<T, true, false, false>), grid, dim3(kRowThreads), 0, s, part,
                       splits, split_stride, d, idx, k, y_ref, y_out, g);
  else if (!g.score_key)
    hipLaunchKernelGGL((row_finish1_kernel<T, true, true, false>), grid, dim3(kRowThreads), 0, s, part,
                       splits, split_stride, d, idx, k, y_ref, y_out, g);
  else
    hipLaunchKernelGGL((row_finish1_kernel<T, true, true, true>), grid, dim3(kRowThreads), 0, s, part,
                       splits, split_stride, d, idx, k, y_ref, y_out, g);
}

// r[m] = (r_src ? decode(r_src[m]) : r[m]) + (y ? decode(y[m]) : 0) + (bias ? bias : 0);
// x_out[m] = RMSNorm(r[m]).  One workgroup per row.
template <typename TS, typename TY, typename TO>
__global__ __launch_bounds__(kRowThreads) void residual_rmsnorm_kernel(
    const TS* __restrict__ r_src, float* __restrict__ r, const TY* __restrict__ y,
    const float* __restrict__ bias, int d, TO* __restrict__ x_out) {
  __shared__ float red[kRowThreads / 64];
  const size_t ro = static_cast<size_t>(blockIdx.x) * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 8; c < d; c += kRowThreads * 8) {
    float v[8], t[8];
    if (r_src) Row8<TS>::load(r_src + ro + c, v); else Row8<float>::load(r + ro + c, v);
    if (y) {
      Row8<TY>::load(y + ro + c, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += t[e];
    }
    if (bias) {
      Row8<float>::load(bias + c, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += t[e];
    }
    Row8<float>::store(r + ro + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  }
  if (!x_out) return;
  const float tot = block_sum<kRowThreads>(ss, red);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + 1e-6f);
  for (int c = threadIdx.x * 8; c < d; c += kRowThreads * 8) {
    float v[8];
    Row8<float>::load(r + ro + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= inv;
    Row8<TO>::store(x_out + ro + c, v);
  }
}

// ---------------------------------------------------------------------------
// Host planning
// ---------------------------------------------------------------------------
struct FfnPlan {
  int tile, bm, bn, m_tiles, glu_ntiles;       // gate/up projection
  int dtile, dbm, dbn, dm_tiles, down_ntiles;  // down projection
  int splits, k_per_split;
  size_t h_elems, part_elems;
};

bool ffn_shape_ok(int d, int ff, int dtype) {
  const int bk = 128 / elem_bytes(dtype);
  return d > 0 && ff > 0 && d % 128 == 0 && d % bk == 0 && ff % 64 == 0 && ff % bk == 0;
}

void pick_tile(int tile, int* bm, int* bn) {
  switch (tile) {
    case kTileS: *bm = CfgS::kBM; *bn = CfgS::kBN; break;
    case kTileM: *bm = CfgM::kBM; *bn = CfgM::kBN; break;
    case kTileL: *bm = CfgL::kBM; *bn = CfgL::kBN; break;
    case kTileG: *bm = CfgG::kBM; *bn = CfgG::kBN; break;
    case kTileW: *bm = CfgW::kBM; *bn = CfgW::kBN; break;
    default: *bm = CfgX::kBM; *bn = CfgX::kBN; break;
  }
}

FfnPlan plan_ffn(int M, int d, int ff, int dtype) {
  FfnPlan p{};
  const int bk = 128 / elem_bytes(dtype);
  const bool wide = dtype == CGS_BF16 && d % CfgX::kBN == 0 && ff % (CfgX::kBN / 2) == 0;
  if (M <= 64) p.tile = kTileS;
  else if (M <= 128) p.tile = kTileM;
  else if (M <= 256) p.tile = wide ? kTileG : kTileL;
  else if (wide && M >= kWideRows && M % CfgW::kBM == 0) p.tile = kTileW;
  else p.tile = wide ? kTileX : kTileL;
  // Down projection: 129..256 rows use two 128-row tiles, which keeps ~256
  // workgroups with half the K splits (half the fp32 partial traffic); the
  // 256 x 256 tile is for the gate/up projection only (as the down tile it
  // needs more K splits for the same rows: measured 1.4x slower at 3072 rows).
  p.dtile = (M > 128 && M <= 256) ? kTileM : (p.tile == kTileW ? kTileX : p.tile);
  pick_tile(p.tile, &p.bm, &p.bn);
  pick_tile(p.dtile, &p.dbm, &p.dbn);
  p.m_tiles = std::max(1, (M + p.bm - 1) / p.bm);
  p.glu_ntiles = ff / (p.bn / 2);
  p.dm_tiles = std::max(1, (M + p.dbm - 1) / p.dbm);
  p.down_ntiles = d / p.dbn;
  // split K of the down projection so that about 256 workgroups run
  const int base = p.down_ntiles * p.dm_tiles;
  const int max_splits = std::max(1, ff / (8 * bk));
  const int splits = std::min(max_splits, std::max(1, (256 + base - 1) / base));
  const int kt = ff / bk;                                 // K tiles in total
  const int tiles_per = (kt + splits - 1) / splits;
  p.k_per_split = tiles_per * bk;
  p.splits = (kt + tiles_per - 1) / tiles_per;
  p.h_elems = static_cast<size_t>(M) * ff;
  p.part_elems = static_cast<size_t>(p.splits) * M * d;
  return p;
}

// Gate/up + GeGLU then split-K down for M rows (gathered through a_rows).
template <typename T>
void launch_ffn_core(const cgs_ffn& w, const T* A, const int32_t* a_rows, int M, const FfnPlan& p,
                     T* H, float* part, const char* glu_site, const char* down_site, hipStream_t s) {
  GemmArgs<T> g{};
  g.A = A; g.lda = w.d; g.a_rows = a_rows; g.M = M;
  g.B0 = static_cast<const T*>(w.w_gate); g.B1 = static_cast<const T*>(w.w_up); g.ldb = w.d;
  g.K = w.d; g.k_per_split = w.d;
  g.n_tiles = p.glu_ntiles; g.m_tiles = p.m_tiles; g.splits = 1;
  g.H = H; g.ldh = w.ff;
  if (a_rows) launch_tile<T, true, true>(p.tile, g, glu_site, s);
  else launch_tile<T, true, false>(p.tile, g, glu_site, s);

  GemmArgs<T> q{};
  q.A = H; q.lda = w.ff; q.a_rows = nullptr; q.M = M;
  q.B0 = static_cast<const T*>(w.w_down); q.ldb = w.ff;
  q.K = w.ff; q.k_per_split = p.k_per_split;
  q.n_tiles = p.down_ntiles; q.m_tiles = p.dm_tiles; q.splits = p.splits;
  q.C = part; q.ldc = w.d; q.split_stride = static_cast<size_t>(M) * w.d;
  // The down projection's weight tiles (256 rows of ff) outweigh its h row
  // tiles, so an XCD's workgroups cover more row tiles of fewer weight tiles
  // (groups of 8: 1.5% faster at 3072 rows than 4).
  q.m_group = 8;
  launch_tile<T, false, false>(p.dtile, q, down_site, s);
}

bool ffn_ok(const cgs_ffn* w, int layout) {
  return w && w->w_gate && w->w_up && w->w_down && valid_dtype(w->dtype) &&
         w->down_layout == layout;
}

template <typename T>
int ctx_recompute_t(const cgs_ffn& w, const T* x, const T* y_ref, const int32_t* idx, int k, int P,
                    T* y_out, const cgs_glue* gl, void* ws, hipStream_t s) {
  const FfnPlan p = plan_ffn(std::max(k, 1), w.d, w.ff, w.dtype);
  Carve cv(ws);
  T* H = cv.take<T>(p.h_elems);
  float* part = cv.take<float>(p.part_elems);
  if (k > 0) {
    // k == P: an ascending, duplicate-free list of P positions in [0, P) is
    // 0 .. P-1, so the rows are read in place (no gather), which lets a
    // launch with more tiles than CUs run persistently.
    launch_ffn_core<T>(w, x, k == P ? nullptr : idx, k, p, H, part, "ctx.glu", "ctx.down", s);
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  {
    ProfScope ps("ctx.finish", s);
    if (w.d == 8 * kRowThreads)
      launch_finish1<T>(dim3(P), s, part, p.splits, static_cast<size_t>(k) * w.d, w.d, true, idx, k, y_ref,
                        y_out, make_glue<T>(gl, w.d));
    else
      hipLaunchKernelGGL((row_finish_kernel<T>), dim3(P), dim3(kRowThreads), 0, s, part, p.splits,
                         static_cast<size_t>(k) * w.d, w.d, true, idx, k, y_ref, y_out, make_glue<T>(gl, w.d));
  }
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}

template <typename T>
int rebuild_t(const cgs_ffn* layers, int L, const T* r0, int P, T* xo, T* yo, void* ws, hipStream_t s) {
  const cgs_ffn& w0 = layers[0];
  const FfnPlan p = plan_ffn(P, w0.d, w0.ff, w0.dtype);
  Carve cv(ws);
  float* r = cv.take<float>(static_cast<size_t>(P) * w0.d);
  T* H = cv.take<T>(p.h_elems);
  float* part = cv.take<float>(p.part_elems);
  const size_t lay = static_cast<size_t>(P) * w0.d;
  {
    ProfScope ps("rebuild.norm", s);
    hipLaunchKernelGGL((residual_rmsnorm_kernel<T, T, T>), dim3(P), dim3(kRowThreads), 0, s, r0, r,
                       static_cast<const T*>(nullptr), static_cast<const float*>(nullptr), w0.d, xo);
  }
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  for (int l = 0; l < L; ++l) {
    launch_ffn_core<T>(layers[l], xo + l * lay, nullptr, P, p, H, part, "rebuild.glu",
                       "rebuild.down", s);
    ProfScope ps("rebuild.finish", s);
    const GlueArgs<T> ga{r, nullptr, (l + 1 < L) ? xo + (l + 1) * lay : static_cast<T*>(nullptr),
                         nullptr, nullptr, 0, 0};
    if (w0.d == 8 * kRowThreads)
      launch_finish1<T>(dim3(P), s, part, p.splits, lay, w0.d, false, static_cast<const int32_t*>(nullptr), P,
                        static_cast<const T*>(nullptr), yo + l * lay, ga);
    else
      hipLaunchKernelGGL((row_finish_kernel<T>), dim3(P), dim3(kRowThreads), 0, s, part, p.splits, lay,
                         w0.d, false, static_cast<const int32_t*>(nullptr), P, static_cast<const T*>(nullptr),
                         yo + l * lay, ga);
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  return CGS_OK;
}

// Several entries rebuilt as one prefill over n P rows: the GEMMs run on
// contiguous work rows, and each layer's row finish writes its rows' outputs
// straight into every entry's own y_ref / x_ref.
constexpr int kBatchMax = 16;
template <typename T> struct RowDist {
  T* y[kBatchMax];
  T* x[kBatchMax];
};

// Row blockIdx.x of the work rows (entry row / P, position row % P) to
// x[e] + x_off: the first layer's input of every entry.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void distribute_rows_kernel(const T* __restrict__ xw, int P, int d,
                                                                      RowDist<T> dst, long long x_off) {
  const int row = blockIdx.x;
  const int e = row / P, p = row - e * P;
  const size_t src = static_cast<size_t>(row) * d, pos = static_cast<size_t>(p) * d;
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  for (int c = threadIdx.x * V; c < d; c += kRowThreads * V)
    *reinterpret_cast<u32x4_t*>(dst.x[e] + x_off + pos + c) = *reinterpret_cast<const u32x4_t*>(xw + src + c);
}

// Row finish of a batched rebuild, row p of the n P work rows (entry p / P,
// position p % P): y = the split sum of the partials, stored in the entry's
// y_ref of this layer (y_off); r += round(y); x_next = RMSNorm(r) into the
// work rows (the next layer's input) and the entry's x_ref of the next layer
// (x_off).  The same arithmetic as the single-entry finish.  RUNS: runs of 8
// a thread keeps between the residual update and the normalisation (1 when
// d = 8 kRowThreads, one run per thread; kGlueKeep otherwise).
template <typename T, int RUNS>
__global__ __launch_bounds__(kRowThreads) void rebuild_finish_kernel(const float* __restrict__ part, int splits,
                                                                     size_t split_stride, int d, int P,
                                                                     RowDist<T> dst, long long y_off,
                                                                     long long x_off, GlueArgs<T> glue) {
  __shared__ float red[kRowThreads / 64];
  const int p = blockIdx.x;
  const int e = p / P;
  const size_t ro = static_cast<size_t>(p) * d;
  const size_t qo = static_cast<size_t>(p - e * P) * d;
  T* const y_row = dst.y[e] + y_off + qo;
  if (glue.x_next) glue.x_copy = dst.x[e] + x_off + qo;
  float ss = 0.f;
  float keep[RUNS][8];
  int j = 0;
  for (int c = threadIdx.x * 8; c < d; c += kRowThreads * 8, ++j) {
    float v[8], rr[8], b[8];
    glue_prefetch(glue, ro, c, rr, b);
    Row8<float>::load(part + ro + c, v);
    add_splits(part + split_stride + ro + c, split_stride, splits - 1, v);
    Row8<T>::store(y_row + c, v);
    ss += glue_add(glue, ro, c, v, rr, b);
    if (j < RUNS) {
#pragma unroll
      for (int q = 0; q < 8; ++q) keep[j][q] = rr[q];
    }
  }
  if (glue.x_next) glue_norm_t<T, kRowThreads>(glue, ro, d, ss, red, keep);
}

template <typename T>
int rebuild_batch_t(const cgs_ffn* layers, int L, const T* r0, int n, int P, T* const* xo, T* const* yo,
                    void* ws, hipStream_t s) {
  const cgs_ffn& w0 = layers[0];
  const int M = n * P;
  const int d = w0.d;
  const FfnPlan p = plan_ffn(M, d, w0.ff, w0.dtype);
  Carve cv(ws);
  float* r = cv.take<float>(static_cast<size_t>(M) * d);
  T* xw = cv.take<T>(static_cast<size_t>(M) * d);
  T* H = cv.take<T>(p.h_elems);
  float* part = cv.take<float>(p.part_elems);
  const long long lay = static_cast<long long>(P) * d;
  RowDist<T> dst{};
  for (int e = 0; e < n; ++e) {
    dst.y[e] = yo[e];
    dst.x[e] = xo[e];
  }
  {
    ProfScope ps("rebuild.norm", s);
    hipLaunchKernelGGL((residual_rmsnorm_kernel<T, T, T>), dim3(M), dim3(kRowThreads), 0, s, r0, r,
                       static_cast<const T*>(nullptr), static_cast<const float*>(nullptr), d, xw);
    hipLaunchKernelGGL((distribute_rows_kernel<T>), dim3(M), dim3(kRowThreads), 0, s, xw, P, d, dst, 0ll);
  }
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  for (int l = 0; l < L; ++l) {
    launch_ffn_core<T>(layers[l], xw, nullptr, M, p, H, part, "rebuild.glu", "rebuild.down", s);
    ProfScope ps("rebuild.finish", s);
    const bool more = l + 1 < L;
    const GlueArgs<T> ga{r, nullptr, more ? xw : static_cast<T*>(nullptr), nullptr, nullptr, 0, 0, nullptr};
    const size_t split_stride = static_cast<size_t>(M) * d;
    const long long y_off = l * lay, x_off = more ? (l + 1) * lay : -1ll;
    if (d == 8 * kRowThreads)
      hipLaunchKernelGGL((rebuild_finish_kernel<T, 1>), dim3(M), dim3(kRowThreads), 0, s, part, p.splits,
                         split_stride, d, P, dst, y_off, x_off, ga);
    else
      hipLaunchKernelGGL((rebuild_finish_kernel<T, kGlueKeep>), dim3(M), dim3(kRowThreads), 0, s, part, p.splits,
                         split_stride, d, P, dst, y_off, x_off, ga);
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  return CGS_OK;
}

}  // namespace
}  // namespace cgs

using namespace cgs;

// Every LDS-DMA operand of the gate/up and down GEMMs spans < 2^32 bytes:
// the activations [P][d], the weights [ff][d] / [d][ff], the hidden rows [M][ff].
bool ffn_span_ok(long long P, long long M, int d, int ff, int dtype) {
  const int es = elem_bytes(dtype);
  return dma_span_ok(P, d, es) && dma_span_ok(ff, d, es) && dma_span_ok(M, ff, es);
}

extern "C" size_t cgs_ctx_ffn_recompute_workspace(int k, int P, int d, int ff, int dtype) {
  if (!valid_dtype(dtype) || !ffn_shape_ok(d, ff, dtype) || k < 0 || P < k || !ffn_span_ok(P, k, d, ff, dtype))
    return 0;
  const FfnPlan p = plan_ffn(std::max(k, 1), d, ff, dtype);
  Carve cv(nullptr);
  cv.take<char>(p.h_elems * elem_bytes(dtype));
  cv.take<float>(p.part_elems);
  return cv.bytes();
}

extern "C" int ctx_ffn_recompute(const cgs_ffn* w, const void* x, const void* y_ref,
                                 const int32_t* idx, int k, int P, void* y_out,
                                 const cgs_glue* glue, void* ws, size_t ws_bytes, void* stream) {
  if (!ffn_ok(w, CGS_DOWN_DF) || !x || !y_ref || !y_out || (k > 0 && !idx) || !glue_ok(glue))
    return CGS_ERR_ARG;
  if (!ffn_shape_ok(w->d, w->ff, w->dtype)) return CGS_ERR_UNSUPPORTED;
  if (P < 0 || k < 0 || k > P) return CGS_ERR_SHAPE;
  if (!ffn_span_ok(P, k, w->d, w->ff, w->dtype)) return CGS_ERR_UNSUPPORTED;
  if (P == 0) return CGS_OK;
  if (y_out == y_ref || y_out == x) return CGS_ERR_ARG;
  if (!ws || ws_bytes < cgs_ctx_ffn_recompute_workspace(k, P, w->d, w->ff, w->dtype))
    return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int st = validate_index(idx, k, P, s)) return st;
  if (w->dtype == CGS_BF16)
    return ctx_recompute_t<uint16_t>(*w, static_cast<const uint16_t*>(x),
                                     static_cast<const uint16_t*>(y_ref), idx, k, P,
                                     static_cast<uint16_t*>(y_out), glue, ws, s);
  return ctx_recompute_t<float>(*w, static_cast<const float*>(x), static_cast<const float*>(y_ref),
                                idx, k, P, static_cast<float*>(y_out), glue, ws, s);
}

extern "C" size_t cgs_ref_rebuild_dense_workspace(int L, int P, int d, int ff, int dtype) {
  (void)L;
  if (!valid_dtype(dtype) || !ffn_shape_ok(d, ff, dtype) || P <= 0 || !ffn_span_ok(P, P, d, ff, dtype)) return 0;
  const FfnPlan p = plan_ffn(P, d, ff, dtype);
  Carve cv(nullptr);
  cv.take<float>(static_cast<size_t>(P) * d);
  cv.take<char>(p.h_elems * elem_bytes(dtype));
  cv.take<float>(p.part_elems);
  return cv.bytes();
}

extern "C" int ref_rebuild_dense(const cgs_ffn* layers, int L, const void* r0, int P,
                                 void* x_ref_out, void* y_ref_out, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!layers || !r0 || !x_ref_out || !y_ref_out) return CGS_ERR_ARG;
  if (L <= 0 || P <= 0) return CGS_ERR_SHAPE;
  for (int l = 0; l < L; ++l) {
    if (!ffn_ok(&layers[l], CGS_DOWN_DF)) return CGS_ERR_ARG;
    if (layers[l].d != layers[0].d || layers[l].ff != layers[0].ff || layers[l].dtype != layers[0].dtype)
      return CGS_ERR_SHAPE;
  }
  const cgs_ffn& w0 = layers[0];
  if (!ffn_shape_ok(w0.d, w0.ff, w0.dtype) || !ffn_span_ok(P, P, w0.d, w0.ff, w0.dtype))
    return CGS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < cgs_ref_rebuild_dense_workspace(L, P, w0.d, w0.ff, w0.dtype))
    return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w0.dtype == CGS_BF16)
    return rebuild_t<uint16_t>(layers, L, static_cast<const uint16_t*>(r0), P,
                               static_cast<uint16_t*>(x_ref_out), static_cast<uint16_t*>(y_ref_out), ws, s);
  return rebuild_t<float>(layers, L, static_cast<const float*>(r0), P, static_cast<float*>(x_ref_out),
                          static_cast<float*>(y_ref_out), ws, s);
}

extern "C" size_t cgs_ref_rebuild_dense_batch_workspace(int L, int n, int P, int d, int ff, int dtype) {
  (void)L;
  if (n < 1 || n > kBatchMax || P <= 0 || !valid_dtype(dtype) || !ffn_shape_ok(d, ff, dtype)) return 0;
  const long long M = static_cast<long long>(n) * P;
  if (M > INT32_MAX || !ffn_span_ok(M, M, d, ff, dtype)) return 0;
  const FfnPlan p = plan_ffn(static_cast<int>(M), d, ff, dtype);
  Carve cv(nullptr);
  cv.take<float>(static_cast<size_t>(M) * d);
  cv.take<char>(static_cast<size_t>(M) * d * elem_bytes(dtype));
  cv.take<char>(p.h_elems * elem_bytes(dtype));
  cv.take<float>(p.part_elems);
  return cv.bytes();
}

extern "C" int ref_rebuild_dense_batch(const cgs_ffn* layers, int L, const void* r0, int n, int P,
                                       void* const* x_ref_out, void* const* y_ref_out, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (!layers || !r0 || !x_ref_out || !y_ref_out) return CGS_ERR_ARG;
  if (L <= 0 || P <= 0 || n < 1 || n > kBatchMax) return CGS_ERR_SHAPE;
  for (int e = 0; e < n; ++e)
    if (!x_ref_out[e] || !y_ref_out[e]) return CGS_ERR_ARG;
  for (int l = 0; l < L; ++l) {
    if (!ffn_ok(&layers[l], CGS_DOWN_DF)) return CGS_ERR_ARG;
    if (layers[l].d != layers[0].d || layers[l].ff != layers[0].ff || layers[l].dtype != layers[0].dtype)
      return CGS_ERR_SHAPE;
  }
  const cgs_ffn& w0 = layers[0];
  const size_t need = cgs_ref_rebuild_dense_batch_workspace(L, n, P, w0.d, w0.ff, w0.dtype);
  if (need == 0) return CGS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < need) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w0.dtype == CGS_BF16)
    return rebuild_batch_t<uint16_t>(layers, L, static_cast<const uint16_t*>(r0), n, P,
                                     reinterpret_cast<uint16_t* const*>(x_ref_out),
                                     reinterpret_cast<uint16_t* const*>(y_ref_out), ws, s);
  return rebuild_batch_t<float>(layers, L, static_cast<const float*>(r0), n, P,
                                reinterpret_cast<float* const*>(x_ref_out), reinterpret_cast<float* const*>(y_ref_out),
                                ws, s);
}

extern "C" int cgs_residual_rmsnorm(float* r, const float* r_in, const void* y, int y_dtype,
                                    const float* bias, int M, int d, void* x_out, int out_dtype,
                                    void* stream) {
  if (!r || (y && !valid_dtype(y_dtype)) || (x_out && !valid_dtype(out_dtype))) return CGS_ERR_ARG;
  if (M < 0 || d <= 0) return CGS_ERR_SHAPE;
  if (M == 0) return CGS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d % 8 != 0) return CGS_ERR_UNSUPPORTED;
  const dim3 grid(M), block(kRowThreads);
  ProfScope ps("glue.rmsnorm", s);
  if (y_dtype == CGS_BF16 || !y) {
    auto* yy = static_cast<const uint16_t*>(y);
    if (out_dtype == CGS_BF16)
      hipLaunchKernelGGL((residual_rmsnorm_kernel<float, uint16_t, uint16_t>), grid, block, 0, s, r_in, r, yy, bias, d, static_cast<uint16_t*>(x_out));
    else
      hipLaunchKernelGGL((residual_rmsnorm_kernel<float, uint16_t, float>), grid, block, 0, s, r_in, r, yy, bias, d, static_cast<float*>(x_out));
  } else {
    auto* yy = static_cast<const float*>(y);
    if (out_dtype == CGS_BF16)
      hipLaunchKernelGGL((residual_rmsnorm_kernel<float, float, uint16_t>), grid, block, 0, s, r_in, r, yy, bias, d, static_cast<uint16_t*>(x_out));
    else
      hipLaunchKernelGGL((residual_rmsnorm_kernel<float, float, float>), grid, block, 0, s, r_in, r, yy, bias, d, static_cast<float*>(x_out));
  }
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}
