// One masked denoising step of the action expert in a single persistent
// launch: every layer's Eq. 4 update (rMuscle §4.1, Eq. 4)
//   y_l = y_a,l + (h^M(x_l) - h_a,l^M) W_down[M],
// followed by the residual / RMSNorm glue r += round(y_l) (+ bias_l),
// x_{l+1} = RMSNorm(r), for all L layers.
//
// A masked layer of the 18-layer expert moves ~7.5 MB, about 1 us of HBM
// time, but has two all-to-all dependencies (every h needs all of x, every y
// needs all of h) and a row-wise one (RMSNorm).  As separate kernels each
// dependency costs a launch; here each costs one hand-off between
// workgroups.  Every workgroup stays resident for the whole step
// (one per CU) and runs two independent groups of four waves:
//
//   gate/up group   stage A of tile (token block, 16 mask positions): its
//                   weight rows, mask ids and anchor activations are loaded
//                   into registers while the previous layer is still
//                   running; it waits for its x rows, runs the MFMAs over
//                   its quarter of d per wave, sums the quarters in LDS and
//                   writes h (optional) and the rounded delta h - h_a.
//   down group      stage B of tile (K split, 32 output columns): its
//                   transposed W_down fragments are loaded ahead; it waits
//                   for its split of the deltas, runs the MFMAs and writes
//                   fp32 partials.  Workgroups that own a token row then
//                   run stage C: wait for the row's partials of every split,
//                   y = y_a + sum (split order), r += round(y) (+ bias),
//                   x_{l+1} = RMSNorm(r) (r stays in registers across layers).
//
// The two groups never wait for each other (no workgroup barrier after the
// start), so a group's outstanding weight loads never delay the other
// group's urgent ones.
//
// Hand-offs: producers write with device-coherent stores (cache policy sc1),
// wait until the stores are acknowledged and then set a ready flag per wave
// (x rows, gate/up tiles, down tiles); consumers poll only the flags they
// depend on (one per lane) and then read the data once with device-coherent
// loads.  No fence or grid barrier is involved (a device-scope fence writes
// back a whole XCD L2), and no consumer ever writes a location it polls or
// reads: a line a consumer wrote itself stays valid in its XCD's L2 and
// would hide later writes from other XCDs (the eight L2s are not kept
// coherent).  The flags are zeroed by a small kernel launched first.  The
// partial sums are double-buffered; a down tile overwrites layer l-2's
// partials only after its wait for layer l's deltas (or, for an empty K
// split, for layer l-1's inputs) has shown that their readers are done.
//
// Every wait is bounded: past a time limit (or once another wave has given
// up) a wave sets a device-wide abort flag, records CGS_ERR_TIMEOUT and
// leaves, so a violated precondition (too few co-resident workgroups, a
// concurrent launch on the same workspace) ends the launch instead of
// hanging it.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "mfma.hpp"
#include "profile.hpp"
#include "validate.hpp"

namespace cgs {
namespace {

constexpr int kStepThreads = 512;   // two groups of four waves
constexpr int kMaxStepLayers = 24;
constexpr int kStepTok = 64;        // token rows of the delta tiles (S <= 64)
constexpr int kStepSplits = 8;      // K splits of the down projection
constexpr int kStepCols = 32;       // output columns per down tile
constexpr int kStepMaxSteps = 16;   // 32-position steps per split (<= 512 positions)
constexpr int kCoh = 16;            // buffer cache policy: sc1 (device-coherent)
constexpr int kStepMaxTiles = 256;  // gate/up and down tiles per layer, at most

std::atomic<long long> g_wait_ticks{20000000};  // 0.2 s of the 100 MHz wall clock

struct StepLayer {
  const uint16_t* wg;     // [K][d]
  const uint16_t* wu;     // [K][d]
  const uint16_t* wdt;    // [d][ldk]
  const int32_t* idx;     // [K] neuron ids or NULL (identity)
  const float* ya;        // [S][d] or NULL
  const float* ha;        // [ff][S] or NULL
  const float* bias;      // [d] or NULL
  uint16_t* y_out;        // [S][d] or NULL
  float* y_f32;           // [S][d] or NULL
  float* h_out;           // [ff][S] or NULL
  uint16_t* dbuf;         // [64][kpad] deltas (workspace)
  int K, ldk, kpad, nblk, ntb, kc;
};

struct StepArgs {
  StepLayer lay[kMaxStepLayers];
  int L, S, G;
  float* r;               // [S][d]
  uint16_t* x;            // [L+1][S][d]
  float* pbuf;            // [2][kStepSplits][S][d]
  int32_t* xflag;         // [L+1][64][4]: input row published, per wave of its row finish
  int32_t* aflag;         // [L][2][256][4]: gate/up tile (token block, neuron block) done, per wave
  int32_t* bflag;         // [L][4][256]: down tile done, per wave (token rows 16 w ..)
  uint32_t* abort_flag;   // workspace word
  int32_t* status_out;    // or NULL
  long long wait_ticks;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Device-coherent loads.  The empty asm keeps a polling load inside its loop.
__device__ __forceinline__ u32x4_t ld_coh16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoh);
}

// Give up a wait once another wave aborted or the time limit passed.
__device__ __noinline__ bool keep_waiting(uint32_t* abort_flag, int32_t* status_out, long long limit,
                                          long long t0) {
  if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
  if (wall_clock64() - t0 > limit) {
    __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (status_out)
      __hip_atomic_store(status_out, static_cast<int32_t>(CGS_ERR_TIMEOUT), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  __builtin_amdgcn_s_sleep(1);
  return true;
}

// Barrier of the four waves of one group (LDS counter; the other group is
// not involved).  `target` advances by 4 per use.  Returns false (for the
// whole wave) if the launch was aborted meanwhile: a wave of the group that
// gave up a wait never arrives.
__device__ __forceinline__ bool group_sync(int* ctr, int& target, uint32_t* abort_flag) {
  target += 4;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    if (__hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    __builtin_amdgcn_s_sleep(0);
  }
  asm volatile("" ::: "memory");
  return true;
}

// True in every lane if any lane of the wave gave up (so the wave leaves as one).
__device__ __forceinline__ bool wave_any(bool v) { return __builtin_amdgcn_ballot_w64(v) != 0; }

__device__ __forceinline__ Frag<uint16_t> frag(u32x4_t v) {
  Frag<uint16_t> f;
  f.u = v;
  return f;
}

// Wait until flags[0 .. n) are all non-zero (n <= 256; lane i polls flags
// i, i + 64, i + 128, i + 192 with device-coherent loads).  The time limit
// and the abort flag are checked every 16 polls, so pollers do not all read
// one word.  Returns false, for the whole wave, if the launch gave up.
__device__ __forceinline__ bool wait_flags(const int32_t* flags, int n, const StepArgs& a) {
  const int lane = threadIdx.x & 63;
  const long long t0 = wall_clock64();
  for (int it = 1;; ++it) {
    bool ok = true;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = lane + 64 * q;
      asm volatile("" ::: "memory");
      if (i < n) ok = ok && __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    }
    if (!wave_any(!ok)) break;
    if ((it & 15) == 0 && wave_any(!keep_waiting(a.abort_flag, a.status_out, a.wait_ticks, t0))) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  return true;
}

// The four waves of a group wait for the same flags: wave 0 polls them and
// then writes the group's wait count to an LDS word the other waves watch
// (-1 if it gave up), so a flag line has one poller per group, not four.
// Every spin in this kernel ends: a wait on flags by its time limit, a wait
// on LDS words once the launch is aborted.
__device__ __forceinline__ bool group_wait_flags(const int32_t* flags, int n, const StepArgs& a, int* gw,
                                                 int& count) {
  ++count;
  const int wave = (threadIdx.x >> 6) & 3;
  if (wave == 0) {
    const bool ok = wait_flags(flags, n, a);
    if ((threadIdx.x & 63) == 0) __hip_atomic_store(gw, ok ? count : -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return ok;
  }
  // Wave 0 may have left the launch without releasing this wait: it leaves
  // a group barrier once the launch is aborted even if its siblings then
  // pass that barrier and reach this wait.  So also watch the abort flag.
  for (int it = 1;; ++it) {
    const int v = __hip_atomic_load(gw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (v < 0) return false;
    if (v >= count) break;
    if ((it & 15) == 0 && __hip_atomic_load(a.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  return true;
}

// A wave publishes its stores: wait until they are acknowledged (device-
// coherent stores are then visible device-wide), then set its flag.
__device__ __forceinline__ void publish(int32_t* flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Stage A: gate/up of tile (token block tb, positions nb*16 .. +15).
// Wave w covers d columns [w d/4, (w+1) d/4): KSA 32-wide K steps.
// ---------------------------------------------------------------------------
template <int D>
__device__ __attribute__((always_inline)) void step_gate_up(const StepArgs& a, int lw, float (*red)[4][2][kStepTok][16], int* ctr) {
  constexpr int KSA = D / 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, grp = lane >> 4;
  const int kq = wave * (D / 4);
  const int S = a.S;
  int target = 0, nwait = 0;
  int ntile = 0;  // A tiles processed: the LDS reduction buffer alternates per tile
  u32x4_t bg[KSA], bu[KSA];
  int hn[4];
  float ha[4];

  // Gate/up tile of this workgroup: neuron block nb goes to XCD nb % 8 (its
  // token blocks on one XCD, which shares their weight rows in L2), filling
  // each XCD's slots from the first; returns false if there is none.
  const int spx = a.G / 8, xcd = lw / spx, slot = lw % spx;
  auto tile_of = [&](const StepLayer& Ly, int& nb, int& tb) -> bool {
    tb = slot % Ly.ntb;
    nb = (slot / Ly.ntb) * 8 + xcd;
    return nb < Ly.nblk;
  };
  auto prefetch = [&](int l) {
    const StepLayer& Ly = a.lay[l];
    int nb, tb;
    if (!tile_of(Ly, nb, tb)) return;
    const int tt = 4 / Ly.ntb;
    const int i = nb * 16 + r;
    const bool v = i < Ly.K;
#pragma unroll
    for (int ks = 0; ks < KSA; ++ks) {
      const size_t off = static_cast<size_t>(v ? i : 0) * D + kq + ks * 32 + grp * 8;
      bg[ks] = v ? *reinterpret_cast<const u32x4_t*>(Ly.wg + off) : u32x4_t{0u, 0u, 0u, 0u};
      bu[ks] = v ? *reinterpret_cast<const u32x4_t*>(Ly.wu + off) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j;
      const int pos = nb * 16 + (e & 15), tok = tb * tt * 16 + (e >> 4);
      const bool ok = j < tt && pos < Ly.K && tok < S;
      hn[j] = ok ? (Ly.idx ? Ly.idx[pos] : pos) : 0;
      ha[j] = (ok && Ly.ha) ? Ly.ha[static_cast<size_t>(hn[j]) * S + tok] : 0.f;
    }
  };

  prefetch(0);
  for (int l = 0; l < a.L; ++l) {
    const StepLayer& Ly = a.lay[l];
    int nb, tb;
    if (tile_of(Ly, nb, tb)) {
      const int tt = 4 / Ly.ntb;
      const int t0 = tb * tt * 16;
      // the block's input rows (layer 0: the caller's input)
      const int nrows = min(S, t0 + 16 * tt) - t0;
      if (l > 0 && nrows > 0 &&
          !group_wait_flags(a.xflag + (static_cast<size_t>(l) * kStepTok + t0) * 4, nrows * 4, a, ctr + 2, nwait))
        return;
      const auto rx = rsrc(a.x + static_cast<size_t>(l) * S * D, static_cast<uint32_t>(S) * D * 2);
      f32x4_t ag[4], au[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) ag[mt] = au[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // x in two halves of this wave's K steps (registers)
      constexpr int KH = KSA / 2;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4_t xf[4][KH];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int tok = t0 + mt * 16 + r;
          const bool v = mt < tt && tok < S;
#pragma unroll
          for (int q = 0; q < KH; ++q)
            xf[mt][q] = v ? ld_coh16(rx, static_cast<uint32_t>((tok * D + kq + (h * KH + q) * 32 + grp * 8) * 2))
                          : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < KH; ++q) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            if (mt < tt) {
              ag[mt] = mma(frag(xf[mt][q]), frag(bg[h * KH + q]), ag[mt]);
              au[mt] = mma(frag(xf[mt][q]), frag(bu[h * KH + q]), au[mt]);
            }
          }
        }
      }
      // quarters of d summed in LDS in wave order; lane holds rows (tokens)
      // mt*16 + 4 grp + v of column (position) r
      float (*rb)[2][kStepTok][16] = red[ntile & 1];
      ++ntile;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < tt) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            rb[wave][0][mt * 16 + 4 * grp + v][r] = ag[mt][v];
            rb[wave][1][mt * 16 + 4 * grp + v][r] = au[mt][v];
          }
        }
      }
      if (!group_sync(ctr, target, a.abort_flag)) return;
      const auto rd = rsrc(Ly.dbuf, static_cast<uint32_t>(kStepTok) * Ly.kpad * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < tt) {
          const int e = tid + 256 * j;
          const int row = e >> 4, c = e & 15;
          const float g = ((rb[0][0][row][c] + rb[1][0][row][c]) + rb[2][0][row][c]) + rb[3][0][row][c];
          const float u = ((rb[0][1][row][c] + rb[1][1][row][c]) + rb[2][1][row][c]) + rb[3][1][row][c];
          const int pos = nb * 16 + c, tok = t0 + row;
          float delta = 0.f;
          if (pos < Ly.K && tok < S) {
            const float hv = gelu_tanh(g) * u;
            if (Ly.h_out) Ly.h_out[static_cast<size_t>(hn[j]) * S + tok] = hv;
            delta = hv - ha[j];
          }
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(delta), rd,
                                                static_cast<uint32_t>((tok * Ly.kpad + pos) * 2), 0, kCoh);
        }
      }
      publish(a.aflag + ((static_cast<size_t>(l) * 2 + tb) * kStepMaxTiles + nb) * 4 + wave);
    }
    if (l + 1 < a.L) prefetch(l + 1);
  }
}

// ---------------------------------------------------------------------------
// Stage B: down projection of tile (split ks, columns cb*32 .. +31); wave w
// covers tokens 16 w .. 16 w + 15.  Stage C: the row finish of token row lw.
// ---------------------------------------------------------------------------
template <int D, int MS>
__device__ __attribute__((always_inline)) void step_down_finish(const StepArgs& a, int lw, float (*red)[4], int* ctr) {
  constexpr int NCB = D / kStepCols;
  constexpr int NBT = kStepSplits * NCB;  // down tiles
  constexpr int CPT = D / 256;  // columns per thread in the row finish
  const int tid = threadIdx.x - 256, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, grp = lane >> 4;
  const int S = a.S;
  const bool have_b = lw < NBT;
  const int ks_ = lw / NCB, cb = lw % NCB;
  // token row finished by this workgroup (-1: none): rows spread over the
  // XCDs (row s on XCD s % 8), in the slots the gate/up tiles use last
  const int spx = a.G / 8, xcd = lw / spx, slot = lw % spx;
  const int row = (slot >= spx - (S + 7) / 8) ? (spx - 1 - slot) * 8 + xcd : -1;
  const bool owner = row >= 0 && row < S;
  const int c0 = tid * CPT;
  int target = 0, nwait = 0;

  float rr[CPT], ya[CPT], bi[CPT];
  if (owner) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) rr[c] = a.r[static_cast<size_t>(row) * D + c0 + c];
  }
  u32x4_t wf[MS][2];
  auto split_steps = [&](const StepLayer& Ly) {
    const int p0 = ks_ * Ly.kc;
    return p0 >= Ly.kpad ? 0 : min(Ly.kc, Ly.kpad - p0) / 32;
  };
  auto prefetch = [&](int l) {
    const StepLayer& Ly = a.lay[l];
    if (have_b) {
      const int nst = split_steps(Ly), p0 = ks_ * Ly.kc;
#pragma unroll
      for (int st = 0; st < MS; ++st) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int col = cb * kStepCols + nt * 16 + r;
          wf[st][nt] = st < nst ? *reinterpret_cast<const u32x4_t*>(
                                      Ly.wdt + static_cast<size_t>(col) * Ly.ldk + p0 + st * 32 + grp * 8)
                                : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    if (owner) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        ya[c] = Ly.ya ? Ly.ya[static_cast<size_t>(row) * D + c0 + c] : 0.f;
        bi[c] = Ly.bias ? Ly.bias[c0 + c] : 0.f;
      }
    }
  };

  const uint32_t pbytes = static_cast<uint32_t>(kStepSplits) * S * D * 4;
  prefetch(0);
  for (int l = 0; l < a.L; ++l) {
    const StepLayer& Ly = a.lay[l];
    const auto rp = rsrc(a.pbuf + static_cast<size_t>(l & 1) * kStepSplits * S * D, pbytes);
    if (have_b) {
      const int nst = split_steps(Ly), p0 = ks_ * Ly.kc;
      const int tok = wave * 16 + r;
      f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      if (nst > 0) {
        // deltas of this split for this wave's token rows: the gate/up tiles
        // of the split's neuron blocks and of the token block holding them
        const int nb0 = p0 / 16, nb1 = (p0 + nst * 32) / 16;
        // wave 0 polls for the whole group: every token block's tiles
        bool ok = true;
        for (int tb = 0; tb < Ly.ntb && ok; ++tb)
          ok = group_wait_flags(a.aflag + ((static_cast<size_t>(l) * 2 + tb) * kStepMaxTiles + nb0) * 4,
                                (nb1 - nb0) * 4, a, ctr + 2, nwait);
        if (!ok) return;
        const auto rd = rsrc(Ly.dbuf, static_cast<uint32_t>(kStepTok) * Ly.kpad * 2);
        constexpr int SH = MS / 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h * SH >= nst) break;
          u32x4_t df[SH];
#pragma unroll
          for (int q = 0; q < SH; ++q) {
            const int st = h * SH + q;
            df[q] = st < nst ? ld_coh16(rd, static_cast<uint32_t>((tok * Ly.kpad + p0 + st * 32 + grp * 8) * 2))
                             : u32x4_t{0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int q = 0; q < SH; ++q) {
            const int st = h * SH + q;
            if (st < nst) {
              acc[0] = mma(frag(df[q]), frag(wf[st][0]), acc[0]);
              acc[1] = mma(frag(df[q]), frag(wf[st][1]), acc[1]);
            }
          }
        }
      } else if (l >= 2) {
        // An empty split waits for nothing of this layer, but its zero
        // partials overwrite the buffer of layer l-2: first wait until those
        // rows' finishes of layer l-2 are done (implied by the published
        // inputs of layer l-1 for this wave's rows).
        if (!group_wait_flags(a.xflag + static_cast<size_t>(l - 1) * kStepTok * 4, S * 4, a, ctr + 2, nwait))
          return;
      }
      // fp32 partials [split][token][column]; rows past S are not stored
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int prow = wave * 16 + 4 * grp + v;
          const int col = cb * kStepCols + nt * 16 + r;
          if (prow < S)
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(acc[nt][v]), rp,
                static_cast<uint32_t>(((ks_ * S + prow) * D + col) * 4), 0, kCoh);
        }
      }
      publish(a.bflag + (static_cast<size_t>(l) * 4 + wave) * kStepMaxTiles + lw);
    }
    if (owner) {
      // partials of every split for this row: the wave row / 16 of every down tile
      if (!group_wait_flags(a.bflag + (static_cast<size_t>(l) * 4 + row / 16) * kStepMaxTiles, NBT, a, ctr + 2,
                            nwait))
        return;
      float pv[kStepSplits][CPT];
#pragma unroll
      for (int k = 0; k < kStepSplits; ++k) {
        const uint32_t off = static_cast<uint32_t>(((k * S + row) * D + c0) * 4);
        if constexpr (CPT == 4) {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kCoh);
#pragma unroll
          for (int c = 0; c < 4; ++c) pv[k][c] = __uint_as_float(v[c]);
        } else if constexpr (CPT == 2) {
          const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rp, off, 0, kCoh));
#pragma unroll
          for (int c = 0; c < 2; ++c) pv[k][c] = __uint_as_float(v[c]);
        } else {
          pv[k][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, kCoh));
        }
      }
      float ss = 0.f;
      float y[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        y[c] = ya[c];
#pragma unroll
        for (int k = 0; k < kStepSplits; ++k) y[c] += pv[k][c];
        const float yr = bf16_to_f32(f32_to_bf16(y[c]));
        rr[c] += yr;
        if (Ly.bias) rr[c] += bi[c];
        ss += rr[c] * rr[c];
      }
      const size_t ro = static_cast<size_t>(row) * D + c0;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        if (Ly.y_out) Ly.y_out[ro + c] = f32_to_bf16(y[c]);
        if (Ly.y_f32) Ly.y_f32[ro + c] = y[c];
      }
      ss = wave_sum(ss);
      float (*rb)[4] = red;
      if (lane == 0) rb[l & 1][wave] = ss;
      if (!group_sync(ctr, target, a.abort_flag)) return;
      const float tot = ((rb[l & 1][0] + rb[l & 1][1]) + rb[l & 1][2]) + rb[l & 1][3];
      const float inv = 1.0f / sqrtf(tot / static_cast<float>(D) + 1e-6f);
      const auto rx = rsrc(a.x + static_cast<size_t>(l + 1) * S * D, static_cast<uint32_t>(S) * D * 2);
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(rr[c] * inv), rx,
                                              static_cast<uint32_t>((row * D + c0 + c) * 2), 0, kCoh);
      publish(a.xflag + (static_cast<size_t>(l + 1) * kStepTok + row) * 4 + wave);
      if (l + 1 == a.L) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) a.r[ro + c] = rr[c];
      }
    }
    if (l + 1 < a.L) prefetch(l + 1);
  }
}

template <int D, int MS>
__global__ __launch_bounds__(kStepThreads) void act_step_kernel(StepArgs a) {
  __shared__ float red_a[2][4][2][kStepTok][16];
  __shared__ float red_b[2][4];
  __shared__ int ctr[6];  // per group: barrier counter, -, released wait count
  if (threadIdx.x < 6) ctr[threadIdx.x] = 0;
  __syncthreads();
  // logical tile of this workgroup: consecutive tiles on one XCD (workgroups
  // are dealt round-robin over the 8 XCDs), so the two token blocks of a
  // neuron block, and the column blocks of one K split, share an L2
  const int b = blockIdx.x;
  const int lw = (b % 8) * (a.G / 8) + b / 8;
  if (threadIdx.x < 256) step_gate_up<D>(a, lw, red_a, &ctr[0]);
  else step_down_finish<D, MS>(a, lw, red_b, &ctr[3]);
}

// Zero the ready flags and the abort flag of a launch (int32 words).
__global__ __launch_bounds__(256) void step_init_kernel(int32_t* flags, size_t n, uint32_t* abort_flag,
                                                        int32_t* status_out) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t j = i; j < n; j += stride) flags[j] = 0;
  if (i == 0) {
    *abort_flag = 0u;
    if (status_out) *status_out = 0;
  }
}

// Down weights of a mask, transposed: out[j][i] = wd[idx[i]][j] (i < K), 0
// for K <= i < ldk.  Tiles of 32 positions x 64 columns through LDS.
__global__ __launch_bounds__(256) void gather_down_t_kernel(const uint16_t* __restrict__ wd,
                                                            const int32_t* __restrict__ idx, int K, int d,
                                                            uint16_t* __restrict__ out, int ldk) {
  __shared__ uint16_t tile[32][64 + 8];
  const int i0 = blockIdx.x * 32, j0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  {
    const int row = t >> 3, ch = (t & 7) * 8;  // position row, 8 columns
    const int i = i0 + row;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (i < K) {
      const int n = idx ? idx[i] : i;
      v = *reinterpret_cast<const u32x4_t*>(wd + static_cast<size_t>(n) * d + j0 + ch);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[row][ch + 2 * e] = static_cast<uint16_t>(v[e] & 0xffffu);
      tile[row][ch + 2 * e + 1] = static_cast<uint16_t>(v[e] >> 16);
    }
  }
  __syncthreads();
  {
    const int j = t >> 2, pc = (t & 3) * 8;  // output row (column of wd), 8 positions
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = static_cast<uint32_t>(tile[pc + 2 * e][j]) | (static_cast<uint32_t>(tile[pc + 2 * e + 1][j]) << 16);
    if (i0 + pc < ldk) *reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(j0 + j) * ldk + i0 + pc) = v;
  }
}

// Rows idx[0..K) of two [ff][d] matrices into [K][d] buffers.
__global__ __launch_bounds__(256) void gather_two_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                         const int32_t* __restrict__ idx, int K, int d,
                                                         uint16_t* __restrict__ ao, uint16_t* __restrict__ bo) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= 2 * K) return;
  const int m = row / K, i = row - m * K;
  const int n = idx ? idx[i] : i;
  const uint16_t* src = (m == 0 ? a : b) + static_cast<size_t>(n) * d;
  uint16_t* dst = (m == 0 ? ao : bo) + static_cast<size_t>(i) * d;
  for (int e = (threadIdx.x & 63) * 8; e < d; e += 512)
    *reinterpret_cast<u32x4_t*>(dst + e) = *reinterpret_cast<const u32x4_t*>(src + e);
}

struct StepPlan {
  int kpad[kMaxStepLayers];
  size_t dbuf_off[kMaxStepLayers];  // elements
  size_t dbuf_elems, p_elems;
  size_t nx, na, nb;                // ready flags (int32) of each kind
  size_t bytes;
};

int round_up(int v, int m) { return (v + m - 1) / m * m; }

bool step_shape_ok(int L, int S, int d) {
  return L >= 1 && L <= kMaxStepLayers && S >= 1 && S <= kStepTok && (d == 256 || d == 512 || d == 1024);
}

StepPlan plan_step(int L, int S, int d, const int* K) {
  StepPlan p{};
  Carve cv(nullptr);
  size_t off = 0;
  for (int l = 0; l < L; ++l) {
    p.kpad[l] = round_up(std::max(K[l], 0), 32);
    p.dbuf_off[l] = off;
    off += static_cast<size_t>(kStepTok) * p.kpad[l];
  }
  p.dbuf_elems = off;
  p.p_elems = static_cast<size_t>(2) * kStepSplits * S * d;
  p.nx = static_cast<size_t>(L + 1) * kStepTok * 4;
  p.na = static_cast<size_t>(L) * 2 * kStepMaxTiles * 4;
  p.nb = static_cast<size_t>(L) * 4 * kStepMaxTiles;
  cv.take<uint16_t>(std::max<size_t>(p.dbuf_elems, 8));
  cv.take<float>(p.p_elems);
  cv.take<int32_t>(p.nx + p.na + p.nb);
  cv.take<uint32_t>(64);
  p.bytes = cv.bytes();
  return p;
}

// Resident workgroups available to the persistent kernel on the current
// device: one per CU (the kernel's LDS and 512 threads allow one), checked
// against the occupancy query once per device.
int step_grid(int d) {
  static std::mutex mu;
  static std::vector<int> cache;  // [device * 3 + d index]
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int di = d == 256 ? 0 : d == 512 ? 1 : 2;
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(cache.size()) <= dev * 3 + di) cache.resize(dev * 3 + 3, -1);
  int& g = cache[dev * 3 + di];
  if (g < 0) {
    int cus = 0, per = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) {
      if (d == 256) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, act_step_kernel<256, 16>, kStepThreads, 0);
      else if (d == 512) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, act_step_kernel<512, 16>, kStepThreads, 0);
      else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, act_step_kernel<1024, 16>, kStepThreads, 0);
    }
    g = (e == hipSuccess && per >= 1) ? std::min(cus, 256) : 0;
  }
  return g;
}

}  // namespace
}  // namespace cgs

using namespace cgs;

extern "C" long long cgs_set_step_wait_limit(long long ticks) {
  if (ticks < 0) return g_wait_ticks.load();
  return g_wait_ticks.exchange(ticks);
}

extern "C" size_t cgs_act_denoise_step_workspace(int L, int S, int d, int K_max) {
  if (!step_shape_ok(L, S, d) || K_max < 0) return 0;
  std::vector<int> K(L, K_max);
  return plan_step(L, S, d, K.data()).bytes;
}

extern "C" int act_gather_rows_t(const cgs_ffn* w, const int32_t* idx, int K, void* wg_out, void* wu_out,
                                 void* wdt_out, int ldk, void* stream) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down || w->dtype != CGS_BF16 || w->down_layout != CGS_DOWN_FD)
    return CGS_ERR_ARG;
  if (w->d <= 0 || w->d % 64 != 0 || w->ff <= 0) return CGS_ERR_UNSUPPORTED;
  if (K < 0 || K > w->ff || ldk < round_up(K, 32) || ldk % 8 != 0) return CGS_ERR_SHAPE;
  if ((K > 0 && (!wg_out || !wu_out)) || (ldk > 0 && !wdt_out)) return CGS_ERR_ARG;
  if (ldk == 0) return CGS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int st = validate_index(idx, K, w->ff, s)) return st;
  ProfScope ps("act.gather", s);
  const auto* wd = static_cast<const uint16_t*>(w->w_down);
  if (K > 0)
    hipLaunchKernelGGL(gather_two_kernel, dim3((2 * K + 3) / 4), dim3(256), 0, s,
                       static_cast<const uint16_t*>(w->w_gate), static_cast<const uint16_t*>(w->w_up), idx, K, w->d,
                       static_cast<uint16_t*>(wg_out), static_cast<uint16_t*>(wu_out));
  hipLaunchKernelGGL(gather_down_t_kernel, dim3((ldk + 31) / 32, w->d / 64), dim3(256), 0, s, wd, idx, K, w->d,
                     static_cast<uint16_t*>(wdt_out), ldk);
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}

extern "C" int act_denoise_step(const cgs_step_layer* layers, int L, int S, int d, int ff, float* r, void* x,
                                int32_t* status_out, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || !r || !x) return CGS_ERR_ARG;
  if (!step_shape_ok(L, S, d) || ff <= 0) return CGS_ERR_UNSUPPORTED;
  int K[kMaxStepLayers];
  for (int l = 0; l < L; ++l) {
    const cgs_step_layer& Ly = layers[l];
    K[l] = Ly.K;
    if (Ly.K < 0 || Ly.K > ff || Ly.K > kStepSplits * kStepMaxSteps * 32) return CGS_ERR_SHAPE;
    if (Ly.K > 0 && (!Ly.w_gate || !Ly.w_up || !Ly.w_down_t)) return CGS_ERR_ARG;
    if (Ly.ldk < round_up(Ly.K, 32) || Ly.ldk % 8 != 0) return CGS_ERR_SHAPE;
    if (!Ly.idx && Ly.K > 0 && (Ly.h_anchor || Ly.h_out) && Ly.K != ff) return CGS_ERR_ARG;
    if (!dma_span_ok(d, std::max(Ly.ldk, 1), 2) || !dma_span_ok(std::max(Ly.K, 1), d, 2)) return CGS_ERR_UNSUPPORTED;
  }
  const int G = step_grid(d);
  if (G % 8 != 0 || G < kStepSplits * (d / kStepCols) || G < 8 * ((S + 7) / 8)) return CGS_ERR_UNSUPPORTED;
  const StepPlan p = plan_step(L, S, d, K);
  if (!ws || ws_bytes < p.bytes) return CGS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int l = 0; l < L; ++l)
    if (layers[l].idx)
      if (const int st = validate_index(layers[l].idx, layers[l].K, ff, s)) return st;

  Carve cv(ws);
  uint16_t* dbuf = cv.take<uint16_t>(std::max<size_t>(p.dbuf_elems, 8));
  float* pbuf = cv.take<float>(p.p_elems);
  int32_t* flags = cv.take<int32_t>(p.nx + p.na + p.nb);
  uint32_t* abort_flag = cv.take<uint32_t>(64);
  StepArgs a{};
  a.L = L; a.S = S; a.G = G;
  a.r = r; a.x = static_cast<uint16_t*>(x); a.pbuf = pbuf; a.abort_flag = abort_flag;
  a.xflag = flags; a.aflag = flags + p.nx; a.bflag = flags + p.nx + p.na;
  a.status_out = status_out;
  a.wait_ticks = g_wait_ticks.load();
  for (int l = 0; l < L; ++l) {
    const cgs_step_layer& Ly = layers[l];
    StepLayer& q = a.lay[l];
    q.wg = static_cast<const uint16_t*>(Ly.w_gate);
    q.wu = static_cast<const uint16_t*>(Ly.w_up);
    q.wdt = static_cast<const uint16_t*>(Ly.w_down_t);
    q.idx = Ly.idx; q.ya = Ly.y_anchor; q.ha = Ly.h_anchor; q.bias = Ly.bias;
    q.y_out = static_cast<uint16_t*>(Ly.y_out); q.y_f32 = Ly.y_f32_out; q.h_out = Ly.h_out;
    q.dbuf = dbuf + p.dbuf_off[l];
    q.K = Ly.K; q.ldk = Ly.ldk; q.kpad = p.kpad[l];
    q.nblk = q.kpad / 16;
    if (q.nblk > G) return CGS_ERR_UNSUPPORTED;
    q.ntb = (q.nblk * 2 <= G) ? 2 : 1;
    q.kc = round_up((q.kpad + kStepSplits - 1) / kStepSplits, 32);
  }
  {
    ProfScope ps("act.step.init", s);
    hipLaunchKernelGGL(step_init_kernel, dim3(64), dim3(256), 0, s, flags, p.nx + p.na + p.nb, abort_flag,
                       status_out);
  }
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  // down fragments held per split: 8 steps of 32 positions cover masks of up
  // to 2048 neurons, 16 steps up to 4096 (the dense anchor of a 4096-wide FFN)
  int max_kc = 0;
  for (int l = 0; l < L; ++l) max_kc = std::max(max_kc, a.lay[l].kc);
  const bool wide = max_kc > 8 * 32;
  ProfScope ps("act.step", s);
#define CGS_STEP(D_, MS_) hipLaunchKernelGGL((act_step_kernel<D_, MS_>), dim3(G), dim3(kStepThreads), 0, s, a)
  if (d == 256) { if (wide) CGS_STEP(256, 16); else CGS_STEP(256, 8); }
  else if (d == 512) { if (wide) CGS_STEP(512, 16); else CGS_STEP(512, 8); }
  else { if (wide) CGS_STEP(1024, 16); else CGS_STEP(1024, 8); }
#undef CGS_STEP
  return launch_ok() ? CGS_OK : CGS_ERR_LAUNCH;
}
