// Dense and gathered GeGLU FFN on bf16 MFMA (fp32 MFMA for fp32 data).
//
//   ctx_ffn_recompute  rMuscle §4.1, Eq. 3: recompute the FFN for the
//                      selected rows only and scatter them into a copy of the
//                      cached reference outputs.
//   ref_rebuild_dense  §4.2: dense prefill of a compact entry into per-layer
//                      reference inputs/outputs.
//   cgs_residual_rmsnorm  residual add + RMSNorm glue between layers.
//
// One GEMM kernel serves both projections.  Both operands are K-contiguous
// (x rows / h rows against weight rows), so a wavefront's MFMA fragments are
// 16-byte vectors straight out of LDS:
//   * gate/up (GLU mode): a workgroup owns 64 neurons; its B tile stacks their
//     64 gate rows over their 64 up rows, so each wave holds the gate and up
//     accumulators of the same (row, neuron) in the same lane and applies
//     gelu_tanh(g) * u in registers before one rounded store of h;
//   * down: split-K over ff, fp32 partials, reduced in a fixed order by the
//     row-finish kernel, which also scatters into the output (selected rows)
//     or copies the reference bits (unselected rows), or adds the residual
//     and normalises the next layer's input (rebuild).
// A rows can be gathered through an index list (the selected tokens), so the
// selected rows are never copied into a compact buffer.  Tiles are K-steps of
// 128 bytes staged through LDS with a padded 144-byte row pitch (conflict-free
// 16-byte fragment reads), double-buffered through registers.  Workgroups are
// renumbered so that consecutive logical tiles, which share A and B slices,
// land on the same XCD (hardware deals workgroups round-robin over 8 XCDs).
#include <algorithm>

#include "common.hpp"
#include "mfma.hpp"
#include "profile.hpp"

namespace cgs {
namespace {

constexpr int kThreads = 256;
constexpr int kPitch = 144;  // LDS bytes per 128-byte tile row
constexpr int kBRows = 128;  // B rows per tile
constexpr int kXcds = 8;

template <typename T> struct GemmArgs {
  const T* A;              // [*][lda]; row r of the tile is a_rows[m0+r] or m0+r
  int lda;
  const int32_t* a_rows;   // gather list (NULL = identity)
  int M;                   // rows of the problem
  const T* B0;             // GLU: gate [ff][ldb]; else W [N][ldb]
  const T* B1;             // GLU: up [ff][ldb]
  int ldb;
  int K;
  int k_per_split;
  int n_tiles, m_tiles, splits;
  T* H;                    // GLU output [M][ldh]
  int ldh;
  float* C;                // partial output [splits][M][ldc]
  int ldc;
  size_t split_stride;
};

template <typename T, int BM, bool GLU, bool GATHER>
__global__ __launch_bounds__(kThreads) void ffn_gemm_kernel(GemmArgs<T> g) {
  constexpr int E = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int BK = 128 / sizeof(T);      // elements per K tile
  constexpr int KS = BK / 32;              // 32-wide MFMA K steps per tile (bf16: 2, f32: 1)
  constexpr int MT = BM / 32;              // 16-row MFMA tiles per wave (2x2 waves)
  constexpr int A_CH = BM * 8 / kThreads;  // 16-byte A chunks per thread per tile
  constexpr int B_CH = kBRows * 8 / kThreads;
  constexpr int STAGE = (BM + kBRows) * kPitch;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware renumbering of the workgroup
  const int nb = g.n_tiles * g.m_tiles * g.splits;
  int logical = blockIdx.x;
  if (nb % kXcds == 0) logical = (blockIdx.x % kXcds) * (nb / kXcds) + blockIdx.x / kXcds;
  const int mtile = logical % g.m_tiles;
  const int ntile = (logical / g.m_tiles) % g.n_tiles;
  const int split = logical / (g.m_tiles * g.n_tiles);
  const int m0 = mtile * BM;
  const int k_begin = split * g.k_per_split;
  const int k_end = min(g.K, k_begin + g.k_per_split);
  const int nk = (k_end - k_begin) / BK;

  // Source rows for this thread's A chunks (-1: past M, zero-filled)
  int a_src[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = (tid + kThreads * i) / 8;
    const int m = m0 + r;
    a_src[i] = (m < g.M) ? (GATHER ? g.a_rows[m] : m) : -1;
  }
  const T* b_src[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int r = (tid + kThreads * i) / 8;
    if (GLU) {
      const int n = ntile * 64 + (r & 63);
      b_src[i] = (r < 64 ? g.B0 : g.B1) + static_cast<size_t>(n) * g.ldb;
    } else {
      b_src[i] = g.B0 + static_cast<size_t>(ntile * kBRows + r) * g.ldb;
    }
  }
  const int chunk = tid & 7;

  f32x4_t acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int brow[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
    brow[nt] = GLU ? ((nt < 2) ? wn * 32 + nt * 16 : 64 + wn * 32 + (nt - 2) * 16) : wn * 64 + nt * 16;

  u32x4_t ra[A_CH], rb[B_CH];
  // global -> registers for K tile kt
#define CGS_LOAD_TILE(kt)                                                                      \
  {                                                                                            \
    const int k0_ = k_begin + (kt) * BK + chunk * E;                                           \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) ra[i] =                                   \
        a_src[i] >= 0 ? *reinterpret_cast<const u32x4_t*>(g.A + static_cast<size_t>(a_src[i]) * \
                                                             g.lda + k0_)                      \
                      : u32x4_t{0u, 0u, 0u, 0u};                                               \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) rb[i] =                                   \
        *reinterpret_cast<const u32x4_t*>(b_src[i] + k0_);                                     \
  }
  // registers -> LDS stage buf
#define CGS_STORE_TILE(buf)                                                                    \
  {                                                                                            \
    char* as_ = lds + (buf) * STAGE;                                                           \
    char* bs_ = as_ + BM * kPitch;                                                             \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) *reinterpret_cast<u32x4_t*>(              \
        as_ + ((tid + kThreads * i) / 8) * kPitch + chunk * 16) = ra[i];                       \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) *reinterpret_cast<u32x4_t*>(              \
        bs_ + ((tid + kThreads * i) / 8) * kPitch + chunk * 16) = rb[i];                       \
  }
  if (nk > 0) {
    CGS_LOAD_TILE(0);
    CGS_STORE_TILE(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) CGS_LOAD_TILE(kt + 1);
    const char* as = lds + (kt & 1) * STAGE;
    const char* bs = as + BM * kPitch;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = ks * 32 * static_cast<int>(sizeof(T)) + (lane >> 4) * Frag<T>::kBytes;
      Frag<T> af[MT], bfr[4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        af[mt].load(as + (wm * (BM / 2) + mt * 16 + (lane & 15)) * kPitch + off);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) bfr[nt].load(bs + (brow[nt] + (lane & 15)) * kPitch + off);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mma(af[mt], bfr[nt], acc[mt][nt]);
    }
    if (kt + 1 < nk) CGS_STORE_TILE((kt + 1) & 1);
    __syncthreads();
  }
#undef CGS_LOAD_TILE
#undef CGS_STORE_TILE

  // Epilogue
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * (BM / 2) + mt * 16 + 4 * (lane >> 4) + v;
      if (row >= g.M) continue;
      if (GLU) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int col = ntile * 64 + wn * 32 + nt * 16 + (lane & 15);
          const float h = gelu_tanh(acc[mt][nt][v]) * acc[mt][nt + 2][v];
          g.H[static_cast<size_t>(row) * g.ldh + col] = Elem<T>::from_f32(h);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int col = ntile * kBRows + wn * 64 + nt * 16 + (lane & 15);
          g.C[split * g.split_stride + static_cast<size_t>(row) * g.ldc + col] = acc[mt][nt][v];
        }
      }
    }
  }
}

// Block-wide float sum (256 threads).
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

// One workgroup per output row p.
//   selected (p in idx[0..k) when scatter, every row otherwise): y_out[p] = round(sum over splits of
//     the partials of row i, in split order); optionally r[p] += y_out[p] and
//     x_next[p] = RMSNorm(r[p]).
//   unselected: y_out[p] = y_ref[p], bit for bit.
template <typename T>
__global__ __launch_bounds__(kThreads) void row_finish_kernel(
    const float* __restrict__ part, int splits, size_t split_stride, int d, bool scatter,
    const int32_t* __restrict__ idx, int k, const T* __restrict__ y_ref, T* __restrict__ y_out,
    float* __restrict__ resid, T* __restrict__ x_next) {
  __shared__ float red[4];
  const int p = blockIdx.x;
  int i = p;
  bool sel = true;
  if (scatter) {
    int lo = 0, hi = k;  // first position with idx[pos] >= p
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx[mid] < p) lo = mid + 1; else hi = mid;
    }
    i = lo;
    sel = (lo < k) && (idx[lo] == p);
  }
  const size_t ro = static_cast<size_t>(p) * d;
  if (!sel) {
    for (int c = threadIdx.x; c < d; c += kThreads) y_out[ro + c] = y_ref[ro + c];
    return;
  }
  const size_t io = static_cast<size_t>(i) * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += kThreads) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += part[s * split_stride + io + c];
    const T yb = Elem<T>::from_f32(v);
    y_out[ro + c] = yb;
    if (resid) {
      const float r = resid[ro + c] + Elem<T>::to_f32(yb);
      resid[ro + c] = r;
      ss += r * r;
    }
  }
  if (resid && x_next) {
    const float tot = block_sum256(ss, red);
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + 1e-6f);
    for (int c = threadIdx.x; c < d; c += kThreads) x_next[ro + c] = Elem<T>::from_f32(resid[ro + c] * inv);
  }
}

// r[m] = (r_src ? decode(r_src[m]) : r[m]) + (y ? decode(y[m]) : 0) + (bias ? bias : 0);
// x_out[m] = RMSNorm(r[m]).  One workgroup per row.
template <typename TS, typename TY, typename TO>
__global__ __launch_bounds__(kThreads) void residual_rmsnorm_kernel(
    const TS* __restrict__ r_src, float* __restrict__ r, const TY* __restrict__ y,
    const float* __restrict__ bias, int d, TO* __restrict__ x_out) {
  __shared__ float red[4];
  const size_t ro = static_cast<size_t>(blockIdx.x) * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += kThreads) {
    float v = r_src ? Elem<TS>::to_f32(r_src[ro + c]) : r[ro + c];
    if (y) v += Elem<TY>::to_f32(y[ro + c]);
    if (bias) v += bias[c];
    r[ro + c] = v;
    ss += v * v;
  }
  if (!x_out) return;
  const float tot = block_sum256(ss, red);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + 1e-6f);
  for (int c = threadIdx.x; c < d; c += kThreads) x_out[ro + c] = Elem<TO>::from_f32(r[ro + c] * inv);
}

// ---------------------------------------------------------------------------
// Host planning
// ---------------------------------------------------------------------------
struct FfnPlan {
  int bm, m_tiles, glu_ntiles, down_ntiles, splits, k_per_split;
  size_t h_elems, part_elems;
};

bool ffn_shape_ok(int d, int ff, int dtype) {
  const int bk = 128 / elem_bytes(dtype);
  return d > 0 && ff > 0 && d % 128 == 0 && d % bk == 0 && ff % 64 == 0 && ff % bk == 0;
}

FfnPlan plan_ffn(int M, int d, int ff, int dtype) {
  FfnPlan p{};
  const int bk = 128 / elem_bytes(dtype);
  p.bm = M <= 64 ? 64 : (M <= 128 ? 128 : 256);
  p.m_tiles = std::max(1, (M + p.bm - 1) / p.bm);
  p.glu_ntiles = ff / 64;
  p.down_ntiles = d / kBRows;
  const int base = p.down_ntiles * p.m_tiles;
  const int max_splits = std::max(1, ff / (8 * bk));
  int splits = std::min(max_splits, std::max(1, (256 + base - 1) / base));
  const int kt = ff / bk;                                 // K tiles in total
  const int tiles_per = (kt + splits - 1) / splits;
  p.k_per_split = tiles_per * bk;
  p.splits = (kt + tiles_per - 1) / tiles_per;
  p.h_elems = static_cast<size_t>(M) * ff;
  p.part_elems = static_cast<size_t>(p.splits) * M * d;
  return p;
}

template <typename T, int BM, bool GLU, bool GATHER>
void launch_gemm_bm(const GemmArgs<T>& g, const char* site, hipStream_t s) {
  const int nb = g.n_tiles * g.m_tiles * g.splits;
  ProfScope ps(site, s);
  hipLaunchKernelGGL((ffn_gemm_kernel<T, BM, GLU, GATHER>), dim3(nb), dim3(kThreads), 0, s, g);
}

template <typename T, bool GLU, bool GATHER>
void launch_gemm(int bm, const GemmArgs<T>& g, const char* site, hipStream_t s) {
  if (bm == 64) launch_gemm_bm<T, 64, GLU, GATHER>(g, site, s);
  else if (bm == 128) launch_gemm_bm<T, 128, GLU, GATHER>(g, site, s);
  else launch_gemm_bm<T, 256, GLU, GATHER>(g, site, s);
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
  if (a_rows) launch_gemm<T, true, true>(p.bm, g, glu_site, s);
  else launch_gemm<T, true, false>(p.bm, g, glu_site, s);

  GemmArgs<T> q{};
  q.A = H; q.lda = w.ff; q.a_rows = nullptr; q.M = M;
  q.B0 = static_cast<const T*>(w.w_down); q.ldb = w.ff;
  q.K = w.ff; q.k_per_split = p.k_per_split;
  q.n_tiles = p.down_ntiles; q.m_tiles = p.m_tiles; q.splits = p.splits;
  q.C = part; q.ldc = w.d; q.split_stride = static_cast<size_t>(M) * w.d;
  launch_gemm<T, false, false>(p.bm, q, down_site, s);
}

bool ffn_ok(const cgs_ffn* w, int layout) {
  return w && w->w_gate && w->w_up && w->w_down && valid_dtype(w->dtype) &&
         w->down_layout == layout;
}

template <typename T>
int ctx_recompute_t(const cgs_ffn& w, const T* x, const T* y_ref, const int32_t* idx, int k, int P,
                    T* y_out, void* ws, hipStream_t s) {
  const FfnPlan p = plan_ffn(std::max(k, 1), w.d, w.ff, w.dtype);
  Carve cv(ws);
  T* H = cv.take<T>(p.h_elems);
  float* part = cv.take<float>(p.part_elems);
  if (k > 0) {
    launch_ffn_core<T>(w, x, idx, k, p, H, part, "ctx.glu", "ctx.down", s);
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  {
    ProfScope ps("ctx.finish", s);
    hipLaunchKernelGGL((row_finish_kernel<T>), dim3(P), dim3(kThreads), 0, s, part, p.splits,
                       static_cast<size_t>(k) * w.d, w.d, true, idx, k, y_ref, y_out, nullptr, nullptr);
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
    hipLaunchKernelGGL((residual_rmsnorm_kernel<T, T, T>), dim3(P), dim3(kThreads), 0, s, r0, r,
                       static_cast<const T*>(nullptr), static_cast<const float*>(nullptr), w0.d, xo);
  }
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  for (int l = 0; l < L; ++l) {
    launch_ffn_core<T>(layers[l], xo + l * lay, nullptr, P, p, H, part, "rebuild.glu",
                       "rebuild.down", s);
    ProfScope ps("rebuild.finish", s);
    hipLaunchKernelGGL((row_finish_kernel<T>), dim3(P), dim3(kThreads), 0, s, part, p.splits, lay,
                       w0.d, false, static_cast<const int32_t*>(nullptr), P, static_cast<const T*>(nullptr),
                       yo + l * lay, r, (l + 1 < L) ? xo + (l + 1) * lay : static_cast<T*>(nullptr));
    if (!launch_ok()) return CGS_ERR_LAUNCH;
  }
  return CGS_OK;
}

}  // namespace
}  // namespace cgs

using namespace cgs;

extern "C" size_t cgs_ctx_ffn_recompute_workspace(int k, int P, int d, int ff, int dtype) {
  (void)P;
  if (!valid_dtype(dtype) || !ffn_shape_ok(d, ff, dtype) || k < 0) return 0;
  const FfnPlan p = plan_ffn(std::max(k, 1), d, ff, dtype);
  Carve cv(nullptr);
  cv.take<char>(p.h_elems * elem_bytes(dtype));
  cv.take<float>(p.part_elems);
  return cv.bytes();
}

extern "C" int ctx_ffn_recompute(const cgs_ffn* w, const void* x, const void* y_ref,
                                 const int32_t* idx, int k, int P, void* y_out, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!ffn_ok(w, CGS_DOWN_DF) || !x || !y_ref || !y_out || (k > 0 && !idx)) return CGS_ERR_ARG;
  if (!ffn_shape_ok(w->d, w->ff, w->dtype)) return CGS_ERR_UNSUPPORTED;
  if (P < 0 || k < 0 || k > P) return CGS_ERR_SHAPE;
  if (P == 0) return CGS_OK;
  if (y_out == y_ref || y_out == x) return CGS_ERR_ARG;
  if (!ws || ws_bytes < cgs_ctx_ffn_recompute_workspace(k, P, w->d, w->ff, w->dtype))
    return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w->dtype == CGS_BF16)
    return ctx_recompute_t<uint16_t>(*w, static_cast<const uint16_t*>(x),
                                     static_cast<const uint16_t*>(y_ref), idx, k, P,
                                     static_cast<uint16_t*>(y_out), ws, s);
  return ctx_recompute_t<float>(*w, static_cast<const float*>(x), static_cast<const float*>(y_ref),
                                idx, k, P, static_cast<float*>(y_out), ws, s);
}

extern "C" size_t cgs_ref_rebuild_dense_workspace(int L, int P, int d, int ff, int dtype) {
  (void)L;
  if (!valid_dtype(dtype) || !ffn_shape_ok(d, ff, dtype) || P <= 0) return 0;
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
  if (!ffn_shape_ok(w0.d, w0.ff, w0.dtype)) return CGS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < cgs_ref_rebuild_dense_workspace(L, P, w0.d, w0.ff, w0.dtype))
    return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w0.dtype == CGS_BF16)
    return rebuild_t<uint16_t>(layers, L, static_cast<const uint16_t*>(r0), P,
                               static_cast<uint16_t*>(x_ref_out), static_cast<uint16_t*>(y_ref_out), ws, s);
  return rebuild_t<float>(layers, L, static_cast<const float*>(r0), P, static_cast<float*>(x_ref_out),
                          static_cast<float*>(y_ref_out), ws, s);
}

extern "C" int cgs_residual_rmsnorm(float* r, const float* r_in, const void* y, int y_dtype,
                                    const float* bias, int M, int d, void* x_out, int out_dtype,
                                    void* stream) {
  if (!r || (y && !valid_dtype(y_dtype)) || (x_out && !valid_dtype(out_dtype))) return CGS_ERR_ARG;
  if (M < 0 || d <= 0) return CGS_ERR_SHAPE;
  if (M == 0) return CGS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(M), block(kThreads);
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
