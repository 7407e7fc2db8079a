// Row helpers shared by the finish kernels: 8-element row runs and the
// residual / RMSNorm glue between FFN layers (cgs_glue in cgs.h).
//
// Glue, per row, after the FFN output y of the row is final:
//   r += round(y) (+ bias),  x_next = RMSNorm(r) = r / sqrt(mean(r^2) + 1e-6),
// where round() is the rounding of y to the activation type (the residual
// stream adds the value the layer actually emits) and r stays fp32.
#pragma once

#include "common.hpp"
#include "score.hpp"

namespace cgs {

// Eight consecutive elements of a row as fp32 (16 bytes of bf16, 32 of fp32).
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    u32x4_t u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<u32x4_t*>(p) = u;
  }
  static __device__ __forceinline__ void round(float* v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(f32_to_bf16(v[i]));
  }
  static __device__ __forceinline__ void copy(const uint16_t* src, uint16_t* dst) {
    *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
  }
};
template <> struct Row8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0], b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  }
  static __device__ __forceinline__ void round(float*) {}
  static __device__ __forceinline__ void copy(const float* src, float* dst) {
    reinterpret_cast<f32x4_t*>(dst)[0] = reinterpret_cast<const f32x4_t*>(src)[0];
    reinterpret_cast<f32x4_t*>(dst)[1] = reinterpret_cast<const f32x4_t*>(src)[1];
  }
};

// Eight elements held as raw 16-byte words (one word of bf16, two of fp32)
// decoded to fp32.
template <typename T>
__device__ __forceinline__ void raw_to_f32(const u32x4_t* w, float* v) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[0][e] << 16);
      v[2 * e + 1] = __uint_as_float(w[0][e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(w[e / 4][e % 4]);
  }
}

// Sum over the threads of a workgroup of NT threads (NT/64 wave partials in
// `red`, summed in wave order).  Contains barriers: call from every thread.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// v += part[sp * stride .. +8] for sp = 0 .. splits-1, added in split order;
// the loads of up to 8 splits are in flight at once.
__device__ __forceinline__ void add_splits(const float* part, size_t stride, int splits, float* v) {
  constexpr int B = 8;
  for (int s0 = 0; s0 < splits; s0 += B) {
    float t[B][8];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (s0 + b < splits) Row8<float>::load(part + (s0 + b) * stride, t[b]);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (s0 + b < splits) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += t[b][e];
      }
    }
  }
}

template <typename T> struct GlueArgs {
  float* r;             // [rows][d] residual stream (NULL: no glue)
  const float* bias;    // [d] or NULL
  T* x_next;            // [rows][d] or NULL
  const T* score_ref;   // [rows][d] or NULL: score x_next against it (Eq. 2)
  double* score_key;    // [rows]
  int score_kind;       // cgs_score_kind
  long long score_floor;
  T* x_copy;            // this row's second x_next destination (row-relative) or NULL
};

inline bool glue_ok(const cgs_glue* g) {
  if (!g) return true;
  if (!g->r) return false;
  if (g->score_key && (!g->x_next || !g->score_ref)) return false;
  return g->score_kind == CGS_SCORE_REL_RMS || g->score_kind == CGS_SCORE_COSINE;
}

template <typename T>
inline GlueArgs<T> make_glue(const cgs_glue* g, int d) {
  GlueArgs<T> a{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
  if (g) {
    a.r = g->r; a.bias = g->bias; a.x_next = static_cast<T*>(g->x_next);
    if (g->score_key) {
      a.score_ref = static_cast<const T*>(g->score_ref);
      a.score_key = g->score_key;
      a.score_kind = g->score_kind;
      a.score_floor = score_floor(d);
    }
  }
  return a;
}

// Runs of 8 elements a thread keeps in registers between the residual update
// and the normalisation (rows of up to kGlueKeep x 8 x threads elements need
// no second read of r).
constexpr int kGlueKeep = 4;

// Loads of r[ro + c .. +8] and bias[c .. +8], issued early so that they are
// in flight with the loads of the row's output.
template <typename T>
__device__ __forceinline__ void glue_prefetch(const GlueArgs<T>& g, size_t ro, int c, float* rr, float* b) {
  Row8<float>::load(g.r + ro + c, rr);
  if (g.bias) Row8<float>::load(g.bias + c, b);
}

// rr += round(v) (+ b), stored back to r[ro + c .. +8]; returns the sum of
// squares of the updated values (left in rr).
template <typename T>
__device__ __forceinline__ float glue_add(const GlueArgs<T>& g, size_t ro, int c, float* v, float* rr,
                                          const float* b) {
  Row8<T>::round(v);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rr[e] += v[e];
    if (g.bias) rr[e] += b[e];
    ss += rr[e] * rr[e];
  }
  Row8<float>::store(g.r + ro + c, rr);
  return ss;
}

// Integer sum over a workgroup of NT threads (exact, so its order is free).
template <int NT>
__device__ __forceinline__ long long block_sum_i64(long long v, long long* red) {
  v = wave_sum_i64(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// x_next[row] = RMSNorm(r[row]) for the runs c = 8 threadIdx.x + 8 NT j that
// this thread updated with glue_add; `ss` is its partial sum of squares.  With
// a score reference, also the Eq. 2 key of the stored (rounded) x_next row
// against it, exactly as the standalone score kernel computes it.
// keep[j]: the updated r values of this thread's run j (j < kGlueKeep), as
// glue_add left them; later runs are read back from r.  sref (or NULL): the
// score reference runs j < kGlueKeep, already loaded by the caller.
template <typename T, int NT>
__device__ __forceinline__ void glue_norm_t(const GlueArgs<T>& g, size_t ro, int d, float ss, float* red,
                                            const float (*keep)[8], const float (*sref)[8] = nullptr) {
  const float tot = block_sum<NT>(ss, red);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + 1e-6f);
  ScoreSums sc;
  const bool cosine = g.score_kind == CGS_SCORE_COSINE;
  int j = 0;
  for (int c = threadIdx.x * 8; c < d; c += NT * 8, ++j) {
    float rr[8];
    if (j < kGlueKeep) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rr[e] = keep[j][e];
    } else {
      Row8<float>::load(g.r + ro + c, rr);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) rr[e] *= inv;
    Row8<T>::store(g.x_next + ro + c, rr);
    if (g.x_copy) Row8<T>::store(g.x_copy + c, rr);
    if (g.score_key) {
      float xr[8];
      Row8<T>::round(rr);
      if (sref && j < kGlueKeep) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[e] = sref[j][e];
      } else {
        Row8<T>::load(g.score_ref + ro + c, xr);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (cosine) sc.add<true>(static_cast<double>(rr[e]), static_cast<double>(xr[e]));
        else sc.add<false>(static_cast<double>(rr[e]), static_cast<double>(xr[e]));
      }
    }
  }
  if (g.score_key) {
    __shared__ long long lred[NT / 64];
    sc.sx = block_sum_i64<NT>(sc.sx, lred);
    if (cosine) {
      sc.sy = block_sum_i64<NT>(sc.sy, lred);
      sc.sxy = block_sum_i64<NT>(sc.sxy, lred);
    } else {
      sc.sd = block_sum_i64<NT>(sc.sd, lred);
    }
    if (threadIdx.x == 0)
      g.score_key[ro / d] = cosine ? score_key<true>(sc, g.score_floor) : score_key<false>(sc, g.score_floor);
  }
}

template <typename T>
__device__ __forceinline__ void glue_norm(const GlueArgs<T>& g, size_t ro, int d, float ss, float* red,
                                          const float (*keep)[8]) {
  glue_norm_t<T, 256>(g, ro, d, ss, red, keep);
}

}  // namespace cgs
