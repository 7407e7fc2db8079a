// MFMA GEMM core shared by the Context Cache recompute and the dense rebuild.
//
// C = A B^T with both operands K-contiguous (activation rows against weight
// rows), bf16 (or fp32) MFMA 16x16 with fp32 accumulation:
//   * GLU mode: the B tile stacks BN/2 gate rows over the same BN/2 up rows,
//     so a lane holds the gate and up accumulators of one (row, neuron) and
//     the epilogue stores h = gelu_tanh(g) * u rounded once;
//   * plain mode: fp32 partial sums of one K split, [split][M][ldc].
// A rows may be gathered through an index list (the selected tokens).
//
// Data movement (gfx950): K tiles of 128 bytes per row travel global -> LDS
// by LDS DMA (global_load_lds_dwordx4, 1 KB per wavefront instruction) into
// two rings (A tiles SA deep, B tiles SB deep; half of the waves load each
// operand), one workgroup barrier per K tile.  A tile row is 8 chunks of 16
// bytes; chunk c of row r sits at physical chunk c ^ (r & 7), so the 16-byte
// MFMA fragment reads of 8 consecutive rows fall in 8 distinct bank groups.
// The waves form a WM x WN grid; each owns (BM/WM) x 16 NT of the tile.
//
// gemm_kernel runs one tile per workgroup; gemm_kernel_persist runs the same
// tiles with fewer workgroups than tiles: each workgroup takes the tiles
// blockIdx.x, blockIdx.x + gridDim.x, ... and its rings run on across them,
// so the first K tiles of the next tile are in flight while the current one
// finishes and stores its epilogue.
#pragma once

#include "common.hpp"
#include "mfma.hpp"

namespace cgs {

constexpr int kXcds = 8;
constexpr int kMGroup = 4;  // default row tiles per group in the workgroup order

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
  int m_group;             // row tiles per group of the workgroup order (0 = kMGroup)
};

// LDS byte address (M0 / ds offset) of a __shared__ location.
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char_t*)p));
}

// One 1 KB global -> LDS transfer of a wavefront: lane i copies the 16 bytes
// at gbase + voff to LDS byte lds + 16 i.  Issued as inline assembly so that
// the only wait for it is the explicit vmcnt of wait_vm_barrier (the compiler
// would otherwise wait for every outstanding transfer before each LDS read).
// Nothing else in these kernels uses M0.
__device__ __forceinline__ void dma_1k(uint32_t lds, const void* gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// Wait until at most N of this wave's global loads are outstanding and its
// LDS reads are done, then barrier the workgroup: a K tile whose transfers
// every wave has waited for is visible to all, and a stage every wave has
// finished reading may be refilled.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait for the K tile whose transfers were followed by `ahead` more tiles of
// LPW transfers each (0 <= ahead <= MAXA), then barrier (wait_vm_barrier).
template <int LPW, int MAXA>
__device__ __forceinline__ void wait_tile(int ahead) {
  if constexpr (MAXA >= 4) { if (ahead >= 4) { wait_vm_barrier<4 * LPW>(); return; } }
  if constexpr (MAXA >= 3) { if (ahead == 3) { wait_vm_barrier<3 * LPW>(); return; } }
  if constexpr (MAXA >= 2) { if (ahead == 2) { wait_vm_barrier<2 * LPW>(); return; } }
  if constexpr (MAXA >= 1) { if (ahead == 1) { wait_vm_barrier<LPW>(); return; } }
  wait_vm_barrier<0>();
}

// Tile configuration: BM x BN workgroup tile (BN = 16 NT WN), WM x WN waves,
// SA-deep LDS ring for A tiles and SB-deep ring for B tiles.
template <int BM, int WM, int WN, int NT, int SA, int SB>
struct GemmCfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBN = 16 * NT * WN;                       // B rows per tile
  static constexpr int kLds = SA * BM * 128 + SB * kBN * 128;    // LDS bytes
  static constexpr int kBM = BM, kWM = WM, kWN = WN, kNT = NT, kSA = SA, kSB = SB;
};

// Output tile of logical workgroup v.  Workgroups are dealt round-robin over
// the 8 XCDs; renumber them so that consecutive logical tiles (same B tile,
// neighbouring A tiles) share an XCD and its L2.  With many row tiles (a
// batched rebuild) they go in groups of m_group: within an XCD the workgroups
// running together cover m_group row tiles of several weight tiles, instead of
// every row tile of a few weight tiles, so each XCD streams fewer distinct A
// rows per round.  The best group balances the A and B bytes an XCD fetches.
struct GemmTile {
  int m0, ntile, split;
};
template <typename T>
__device__ __forceinline__ GemmTile gemm_tile(const GemmArgs<T>& g, int bm, int v) {
  const int nb = g.n_tiles * g.m_tiles * g.splits;
  int logical = v;
  if (nb % kXcds == 0) logical = (v % kXcds) * (nb / kXcds) + v / kXcds;
  const int split = logical / (g.m_tiles * g.n_tiles);
  const int lt = logical - split * (g.m_tiles * g.n_tiles);
  const int mg = g.m_group > 0 ? g.m_group : kMGroup;
  const int gm = (g.m_tiles > mg && g.m_tiles % mg == 0) ? mg : g.m_tiles;
  const int mtile = (lt / (gm * g.n_tiles)) * gm + lt % gm;
  return GemmTile{mtile * bm, (lt / gm) % g.n_tiles, split};
}

// Epilogue of one tile: lane holds rows 4 (lane >> 4) + v of column lane & 15
// of each 16 x 16 accumulator tile.  bf16 h goes out in rows of 4 columns (8
// bytes per lane) after a quad transpose; fp32 h and the partial sums element
// by element.  Rows at or past M are dropped (CHECK; a launch of full row
// tiles has none).
template <typename T, int MT, int NT, int WTM, int BN, bool GLU, bool CHECK>
__device__ __forceinline__ void gemm_store(const GemmArgs<T>& g, const f32x4_t (&acc)[MT][NT], const GemmTile& t,
                                           int lane, int wm, int wn) {
  if constexpr (GLU && sizeof(T) == 2) {
    const QuadTranspose qt(lane);
    const int rq = 4 * (lane >> 4) + (lane & 3);
    const int cq = 4 * ((lane & 15) >> 2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = t.m0 + wm * WTM + mt * 16 + rq;
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt) {
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = gelu_tanh(acc[mt][nt][v]) * acc[mt][nt + NT / 2][v];
        const uint2 w = qt(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
        const int col = t.ntile * (BN / 2) + wn * 8 * NT + nt * 16 + cq;
        if (!CHECK || row < g.M) *reinterpret_cast<uint2*>(g.H + static_cast<size_t>(row) * g.ldh + col) = w;
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = t.m0 + wm * WTM + mt * 16 + 4 * (lane >> 4) + v;
        if (CHECK && row >= g.M) continue;
        if (GLU) {
#pragma unroll
          for (int nt = 0; nt < NT / 2; ++nt) {
            const int col = t.ntile * (BN / 2) + wn * 8 * NT + nt * 16 + (lane & 15);
            const float h = gelu_tanh(acc[mt][nt][v]) * acc[mt][nt + NT / 2][v];
            g.H[static_cast<size_t>(row) * g.ldh + col] = Elem<T>::from_f32(h);
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int col = t.ntile * BN + wn * 16 * NT + nt * 16 + (lane & 15);
            g.C[t.split * g.split_stride + static_cast<size_t>(row) * g.ldc + col] = acc[mt][nt][v];
          }
        }
      }
    }
  }
}

// Loader roles: waves 0 .. NW/2-1 move A tiles, waves NW/2 .. NW-1 move B
// tiles.  Each wave's vmcnt then counts transfers of one operand only, so the
// B (weight) ring can run SB-1 tiles ahead while the A ring runs SA-1 ahead:
// a wave waiting for tile t waits for exactly the transfers of its operand
// issued up to tile t.
template <typename T, int BM, int WM, int WN, int NT, int SA, int SB, bool GLU, bool GATHER>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs<T> g) {
  using Cfg = GemmCfg<BM, WM, WN, NT, SA, SB>;
  static_assert(!GLU || NT % 2 == 0, "GLU pairs gate and up tiles");
  static_assert(SA >= 2 && SB >= 2 && SA <= 6 && SB <= 6, "ring depth");
  constexpr int NW = Cfg::kWaves;
  static_assert(NW % 2 == 0, "two loader roles");
  constexpr int HW = NW / 2;                             // waves per loader role
  constexpr int BN = Cfg::kBN;
  constexpr int BK = 128 / static_cast<int>(sizeof(T));  // elements per K tile
  constexpr int KS = BK / 32;                            // 32-wide K steps per tile
  constexpr int FC = Frag<T>::kBytes / 16;               // 16-byte chunks per fragment
  constexpr int WTM = BM / WM;                           // wave tile rows
  constexpr int MT = WTM / 16;                           // MFMA row tiles per wave
  constexpr int A_DMA = BM / 8, B_DMA = BN / 8;          // 1 KB transfers per tile
  static_assert(A_DMA % HW == 0 && B_DMA % HW == 0, "transfers must split evenly");
  constexpr int LPW_A = A_DMA / HW, LPW_B = B_DMA / HW;  // transfers per loader wave per tile
  constexpr int LPW_M = LPW_A > LPW_B ? LPW_A : LPW_B;
  constexpr int A_RING = 0, B_RING = SA * BM * 128;      // LDS byte offsets of the rings
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool role_a = wave < HW;
  const int wr = role_a ? wave : wave - HW;  // index within the role

  const GemmTile tile = gemm_tile(g, BM, blockIdx.x);
  const int m0 = tile.m0, ntile = tile.ntile, split = tile.split;
  const int k_begin = split * g.k_per_split;
  const int k_end = min(g.K, k_begin + g.k_per_split);
  const int nk = (k_end - k_begin) / BK;

  // Transfer j of an A (B) tile covers tile rows 8j .. 8j+7; lane l fills
  // physical chunk l & 7 of row 8j + (l >> 3) with logical chunk
  // (l & 7) ^ (l >> 3).  Loader wave w of a role owns transfers w, w + HW, ...
  const int sub = lane >> 3;
  const uint32_t cbyte = static_cast<uint32_t>(((lane & 7) ^ sub) * 16);
  const uint32_t kbyte0 = static_cast<uint32_t>(k_begin) * sizeof(T);
  uint32_t off[LPW_M];
  const T* base[LPW_M];
#pragma unroll
  for (int i = 0; i < LPW_M; ++i) {
    const int j = wr + HW * i;
    off[i] = 0;
    base[i] = g.A;
    if (role_a) {
      if (i < LPW_A) {
        int m = min(m0 + 8 * j + sub, g.M - 1);  // rows past M repeat the last row; results dropped
        if (GATHER) m = g.a_rows[m];
        off[i] = static_cast<uint32_t>(m) * static_cast<uint32_t>(g.lda) * sizeof(T) + kbyte0 + cbyte;
      }
    } else if (i < LPW_B) {
      const int r8 = 8 * j;  // first B tile row of the transfer (wave-uniform)
      const int r = r8 + sub;
      int n;
      if (GLU) {
        n = ntile * (BN / 2) + (r % (BN / 2));
        base[i] = (r8 < BN / 2) ? g.B0 : g.B1;
      } else {
        n = ntile * BN + r;
        base[i] = g.B0;
      }
      off[i] = static_cast<uint32_t>(n) * static_cast<uint32_t>(g.ldb) * sizeof(T) + kbyte0 + cbyte;
    }
  }
  const uint32_t lds0 = lds_addr(lds);

  // Transfers of this wave's operand for K tile kt.
  auto issue = [&](int kt) {
    const uint32_t kb = static_cast<uint32_t>(kt) * 128u;
    if (role_a) {
      const uint32_t st = lds0 + A_RING + (kt % SA) * (BM * 128);
#pragma unroll
      for (int i = 0; i < LPW_A; ++i) dma_1k(st + (wr + HW * i) * 1024, base[i], off[i] + kb);
    } else {
      const uint32_t st = lds0 + B_RING + (kt % SB) * (BN * 128);
#pragma unroll
      for (int i = 0; i < LPW_B; ++i) dma_1k(st + (wr + HW * i) * 1024, base[i], off[i] + kb);
    }
  };
  // Wait until tile t has landed, given that tiles up to `last` were issued.
  auto wait_for = [&](int t, int last_a, int last_b) {
    if (role_a) wait_tile<LPW_A, SA - 1>(max(0, last_a - t));
    else wait_tile<LPW_B, SB - 1>(max(0, last_b - t));
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // B tile rows of this wave's NT 16-column MFMA tiles.  GLU: NT/2 gate tiles
  // and the NT/2 up tiles of the same 8 NT neurons.
  int brow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    brow[nt] = GLU ? ((nt < NT / 2) ? wn * 8 * NT + nt * 16 : BN / 2 + wn * 8 * NT + (nt - NT / 2) * 16)
                   : wn * 16 * NT + nt * 16;
  const int arow0 = wm * WTM + (lane & 15);
  const int swz = lane & 7;
  const int grp = lane >> 4;

  // Fragment reads of K step ks of tile kt: four B tiles, MT A tiles.
  auto load = [&](int kt, int ks, Frag<T> (&af)[MT], Frag<T> (&bf)[NT]) {
    const char* as = lds + A_RING + (kt % SA) * (BM * 128);
    const char* bs = lds + B_RING + (kt % SB) * (BN * 128);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const char* rowp = bs + (brow[nt] + (lane & 15)) * 128;
#pragma unroll
      for (int q = 0; q < FC; ++q)
        bf[nt].chunk(q) = *reinterpret_cast<const u32x4_t*>(rowp + (((ks * 4 + grp) * FC + q) ^ swz) * 16);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const char* rowp = as + (arow0 + mt * 16) * 128;
#pragma unroll
      for (int q = 0; q < FC; ++q)
        af[mt].chunk(q) = *reinterpret_cast<const u32x4_t*>(rowp + (((ks * 4 + grp) * FC + q) ^ swz) * 16);
    }
  };

  // Pipeline: before the loop, A tiles 0 .. SA-1 and B tiles 0 .. SB-1 are
  // in flight.  The fragments of the next K step are read before the MFMAs of
  // the current one; at the last K step of tile t the workgroup waits for
  // tile t+1 (all waves have then finished reading tile t, whose ring slots
  // take A tile t + SA and B tile t + SB).
  const int S_own = role_a ? SA : SB;
  if (nk > 0) {
    for (int p = 0; p < S_own - 1 && p < nk; ++p) issue(p);
    wait_for(0, min(SA - 2, nk - 1), min(SB - 2, nk - 1));
    if (S_own - 1 < nk) issue(S_own - 1);
  }
  auto mfmas = [&](const Frag<T> (&a)[MT], const Frag<T> (&b)[NT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mma(a[mt], b[nt], acc[mt][nt]);
  };
  // Every K step but the last loads the fragments of the next one before its
  // MFMAs; the loop covers all tiles but the last, so its loads are
  // unconditional and the fragment registers alternate without copies.
  Frag<T> ca[MT], cb[NT];
  if (nk > 0) {
    load(0, 0, ca, cb);
    for (int kt = 0; kt + 1 < nk; ++kt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<T> na[MT], nb_[NT];
        if (ks + 1 < KS) {
          load(kt, ks + 1, na, nb_);
        } else {
          wait_for(kt + 1, min(kt + SA - 1, nk - 1), min(kt + SB - 1, nk - 1));
          if (kt + S_own < nk) issue(kt + S_own);
          load(kt + 1, 0, na, nb_);
        }
        mfmas(ca, cb);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ca[mt] = na[mt];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) cb[nt] = nb_[nt];
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frag<T> na[MT], nb_[NT];
      if (ks + 1 < KS) load(nk - 1, ks + 1, na, nb_);
      mfmas(ca, cb);
      if (ks + 1 < KS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ca[mt] = na[mt];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) cb[nt] = nb_[nt];
      }
    }
  }

  gemm_store<T, MT, NT, WTM, BN, GLU, true>(g, acc, tile, lane, wm, wn);
}

// Persistent form of gemm_kernel for launches with more tiles than CUs: a
// grid of one workgroup per CU (a multiple of 8, so that each keeps its
// tiles on its XCD) takes every gridDim-th tile.  The host launches it only
// when every tile is full (M % BM == 0), A rows are not gathered, and every
// tile's K range has the same length of at least SA and SB K tiles.  Same
// pipeline and epilogue as gemm_kernel; the rings run on across the
// workgroup's tiles (the current tile's last K steps issue the next tile's
// first K tiles), and a tile's row and K offsets enter through the scalar
// base address of its transfers.
template <typename T, int BM, int WM, int WN, int NT, int SA, int SB, bool GLU>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel_persist(GemmArgs<T> g) {
  using Cfg = GemmCfg<BM, WM, WN, NT, SA, SB>;
  static_assert(!GLU || NT % 2 == 0, "GLU pairs gate and up tiles");
  static_assert(SA >= 2 && SB >= 2 && SA <= 6 && SB <= 6, "ring depth");
  constexpr int NW = Cfg::kWaves;
  static_assert(NW % 2 == 0, "two loader roles");
  constexpr int HW = NW / 2;
  constexpr int BN = Cfg::kBN;
  constexpr int BK = 128 / static_cast<int>(sizeof(T));
  constexpr int KS = BK / 32;
  constexpr int FC = Frag<T>::kBytes / 16;
  constexpr int WTM = BM / WM;
  constexpr int MT = WTM / 16;
  constexpr int A_DMA = BM / 8, B_DMA = BN / 8;
  static_assert(A_DMA % HW == 0 && B_DMA % HW == 0, "transfers must split evenly");
  constexpr int LPW_A = A_DMA / HW, LPW_B = B_DMA / HW;
  static_assert(!GLU || LPW_B % 2 == 0, "gate and up transfers split evenly");
  constexpr int A_RING = 0, B_RING = SA * BM * 128;
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool role_a = wave < HW;
  const int wr = role_a ? wave : wave - HW;
  const int nb = g.n_tiles * g.m_tiles * g.splits;
  auto tile_of = [&](int v) { return gemm_tile(g, BM, v); };
  // byte offset of a tile's operand rows and K range
  auto a_toff = [&](const GemmTile& t) {
    return static_cast<size_t>(t.m0) * g.lda * sizeof(T) + static_cast<size_t>(t.split) * g.k_per_split * sizeof(T);
  };
  auto b_toff = [&](const GemmTile& t) {
    return static_cast<size_t>(t.ntile) * (GLU ? BN / 2 : BN) * g.ldb * sizeof(T) +
           static_cast<size_t>(t.split) * g.k_per_split * sizeof(T);
  };
  GemmTile cur = tile_of(blockIdx.x);
  const int nk = (min(g.K, cur.split * g.k_per_split + g.k_per_split) - cur.split * g.k_per_split) / BK;

  // Transfer i of a loader wave covers tile rows 8 (wr + HW i) .. + 7 (as in
  // gemm_kernel): the lane's offset in transfer 0 plus i steps of 8 HW rows,
  // all within the tile.  In GLU mode a B loader's first LPW_B / 2 transfers
  // read gate rows and the rest the same rows of up.
  const int sub = lane >> 3;
  const uint32_t cbyte = static_cast<uint32_t>(((lane & 7) ^ sub) * 16);
  uint32_t off0 = 0;
  if (role_a) {
    // the row clamp of gemm_kernel, although every tile here is full (m - m0 =
    // 8 wr + sub): with the 256 x 256 tile near the 256-VGPR limit, this form
    // measured to keep its allocation free of scratch spills
    const int m = min(cur.m0 + 8 * wr + sub, g.M - 1);
    off0 = static_cast<uint32_t>(m - cur.m0) * static_cast<uint32_t>(g.lda) * sizeof(T) + cbyte;
  } else {
    const int r = 8 * wr + sub;
    off0 = static_cast<uint32_t>(GLU ? r % (BN / 2) : r) * static_cast<uint32_t>(g.ldb) * sizeof(T) + cbyte;
  }
  const uint32_t step = static_cast<uint32_t>(8 * HW) * static_cast<uint32_t>(role_a ? g.lda : g.ldb) * sizeof(T);
  const char* const ptr0 = reinterpret_cast<const char*>(role_a ? g.A : g.B0);
  const char* const ptr1 = reinterpret_cast<const char*>(role_a ? g.A : (GLU ? g.B1 : g.B0));
  const uint32_t lds0 = lds_addr(lds);

  // Transfers of this wave's operand for K tile kt of the tile at toff, into
  // stage q of its ring.  Everything but the lane's own offset off0 (the
  // tile, the K tile and the transfer's rows) goes into the scalar base
  // address, so a lane holds one offset register for all of its transfers.
  // Per-transfer sums in vector registers would cost one register each (253
  // instead of 243 on the 256 x 256 tile) and 2% of its time.
  auto issue = [&](size_t toff, int kt, int q) {
    const size_t kb = static_cast<size_t>(kt) * 128u;
    const char* const p0 = ptr0 + toff + kb;
    const char* const p1 = ptr1 + toff + kb;
    if (role_a) {
      const uint32_t st = lds0 + A_RING + q * (BM * 128);
#pragma unroll
      for (int i = 0; i < LPW_A; ++i) dma_1k(st + (wr + HW * i) * 1024, p0 + static_cast<size_t>(i) * step, off0);
    } else {
      constexpr int kHalf = GLU ? LPW_B / 2 : LPW_B;
      const uint32_t st = lds0 + B_RING + q * (BN * 128);
#pragma unroll
      for (int i = 0; i < LPW_B; ++i)
        dma_1k(st + (wr + HW * i) * 1024, (i < LPW_B / 2 ? p0 : p1) + static_cast<size_t>(i % kHalf) * step, off0);
    }
  };
  auto wait_for = [&](int t, int last_a, int last_b) {
    if (role_a) wait_tile<LPW_A, SA - 1>(max(0, last_a - t));
    else wait_tile<LPW_B, SB - 1>(max(0, last_b - t));
  };

  f32x4_t acc[MT][NT];
  int brow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    brow[nt] = GLU ? ((nt < NT / 2) ? wn * 8 * NT + nt * 16 : BN / 2 + wn * 8 * NT + (nt - NT / 2) * 16)
                   : wn * 16 * NT + nt * 16;
  const int arow0 = wm * WTM + (lane & 15);
  const int swz = lane & 7;
  const int grp = lane >> 4;

  // Ring stages of the K tile being computed: K tile kt + S of a tile (or
  // the next tile's K tile kt + S - nk) takes the stage of K tile kt.
  int qa = 0, qb = 0;
  auto advance = [&]() {
    qa = qa + 1 == SA ? 0 : qa + 1;
    qb = qb + 1 == SB ? 0 : qb + 1;
  };
  auto load = [&](int ks, Frag<T> (&af)[MT], Frag<T> (&bf)[NT]) {
    const char* as = lds + A_RING + qa * (BM * 128);
    const char* bs = lds + B_RING + qb * (BN * 128);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const char* rowp = bs + (brow[nt] + (lane & 15)) * 128;
#pragma unroll
      for (int q = 0; q < FC; ++q)
        bf[nt].chunk(q) = *reinterpret_cast<const u32x4_t*>(rowp + (((ks * 4 + grp) * FC + q) ^ swz) * 16);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const char* rowp = as + (arow0 + mt * 16) * 128;
#pragma unroll
      for (int q = 0; q < FC; ++q)
        af[mt].chunk(q) = *reinterpret_cast<const u32x4_t*>(rowp + (((ks * 4 + grp) * FC + q) ^ swz) * 16);
    }
  };
  auto mfmas = [&](const Frag<T> (&a)[MT], const Frag<T> (&b)[NT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mma(a[mt], b[nt], acc[mt][nt]);
  };

  const int S_own = role_a ? SA : SB;
  auto run_tile = [&](int vt) {
    const int vn = vt + static_cast<int>(gridDim.x);
    const bool has_next = vn < nb;
    const GemmTile nxt = has_next ? tile_of(vn) : cur;
    const size_t toff = role_a ? a_toff(cur) : b_toff(cur);
    const size_t toff_n = role_a ? a_toff(nxt) : b_toff(nxt);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // K tiles 0 .. S-2 are in flight: issued here for the first tile, by the
    // previous tile's last K steps otherwise.  Loads and stores share the
    // vector memory counter and may complete out of order with each other, so
    // a counted wait proves nothing while the previous tile's epilogue stores
    // are outstanding: after them the first wait is for every transfer and
    // store.
    if (nk > 0) {
      if (vt == static_cast<int>(blockIdx.x)) {
        for (int p = 0; p < S_own - 1 && p < nk; ++p) issue(toff, p, p);
        wait_for(0, min(SA - 2, nk - 1), min(SB - 2, nk - 1));
      } else {
        wait_vm_barrier<0>();
      }
      const int qo = role_a ? qa : qb;  // K tile S - 1 takes the stage before K tile 0's
      if (S_own - 1 < nk) issue(toff, S_own - 1, qo == 0 ? S_own - 1 : qo - 1);
    }
    Frag<T> ca[MT], cb[NT];
    if (nk > 0) {
      load(0, ca, cb);
      for (int kt = 0; kt + 1 < nk; ++kt) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frag<T> na[MT], nb_[NT];
          if (ks + 1 < KS) {
            load(ks + 1, na, nb_);
          } else {
            const int la = has_next ? kt + SA - 1 : min(kt + SA - 1, nk - 1);
            const int lb = has_next ? kt + SB - 1 : min(kt + SB - 1, nk - 1);
            wait_for(kt + 1, la, lb);
            const int q = role_a ? qa : qb;  // the stage of K tile kt, read by every wave by now
            if (kt + S_own < nk) issue(toff, kt + S_own, q);
            else if (has_next) issue(toff_n, kt + S_own - nk, q);
            advance();
            load(0, na, nb_);
          }
          mfmas(ca, cb);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) ca[mt] = na[mt];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) cb[nt] = nb_[nt];
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<T> na[MT], nb_[NT];
        if (ks + 1 < KS) load(ks + 1, na, nb_);
        mfmas(ca, cb);
        if (ks + 1 < KS) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) ca[mt] = na[mt];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) cb[nt] = nb_[nt];
        }
      }
    }
    gemm_store<T, MT, NT, WTM, BN, GLU, false>(g, acc, cur, lane, wm, wn);
    advance();
    cur = nxt;
  };
  for (int vt = blockIdx.x; vt < nb; vt += gridDim.x) run_tile(vt);
}

}  // namespace cgs
