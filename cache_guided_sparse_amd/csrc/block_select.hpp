// Block-wide exact selection over 64-bit ordered keys, one workgroup of
// kSelThreads threads.  Larger keys rank first; equal keys rank by ascending
// index, so every key set has exactly one top-k set.
//
// The top k is found by an 8-pass radix descent over the key bytes (most
// significant first), which yields the k-th largest key value T and how many
// elements equal to T are still needed; a final pass in index order emits
// every element with key > T and the first `need` elements with key == T, in
// ascending index order.  All work is integer, so the result does not depend
// on thread scheduling.
#pragma once

#include "common.hpp"

namespace cgs {

constexpr int kSelThreads = 1024;

struct SelShared {
  uint32_t hist[256];
  unsigned long long hsum[256];
  long long scan[kSelThreads / kWave];
  uint64_t digit;
  long long above_cnt;
  long long above_sum;
  long long tie_z;
  int need;
};

// Threshold of the top k: returns T (the k-th largest key) and sets *need to
// the number of elements equal to T that belong to the top k (>= 1).
// Requires 1 <= k <= n.
template <class KeyFn>
__device__ uint64_t block_topk_threshold(KeyFn key_of, int n, int k, int* need, SelShared& sm) {
  uint64_t prefix = 0, pmask = 0;
  long long remaining = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += blockDim.x) sm.hist[b] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint64_t kv = key_of(i);
      if ((kv & pmask) == prefix) atomicAdd(&sm.hist[(kv >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      // lane owns bins 4*lane .. 4*lane+3; count of all bins above this lane's
      long long c = 0;
      for (int j = 0; j < 4; ++j) c += sm.hist[4 * lane + j];
      // suffix sum over higher lanes: scan in reversed lane order
      long long rev = c;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        long long u = __shfl_down(rev, o, kWave);
        if (lane + o < kWave) rev += u;
      }
      long long above = rev - c;  // elements in bins of higher lanes
      for (int j = 3; j >= 0; --j) {
        long long h = sm.hist[4 * lane + j];
        if (above < remaining && remaining <= above + h) {
          sm.digit = static_cast<uint64_t>(4 * lane + j);
          sm.above_cnt = above;
        }
        above += h;
      }
    }
    __syncthreads();
    prefix |= sm.digit << shift;
    pmask |= 0xffull << shift;
    remaining -= sm.above_cnt;
    __syncthreads();
  }
  *need = static_cast<int>(remaining);
  return prefix;
}

// Emit, in ascending index order, every i with key > T and the first `need`
// indices with key == T: emit(i, position).  Returns the number emitted.
template <class KeyFn, class EmitFn>
__device__ int block_emit_selected(KeyFn key_of, int n, uint64_t T, int need, EmitFn emit,
                                   SelShared& sm) {
  const int chunk = (n + blockDim.x - 1) / blockDim.x;
  const int lo = min(n, static_cast<int>(threadIdx.x) * chunk);
  const int hi = min(n, lo + chunk);
  long long eq = 0;
  for (int i = lo; i < hi; ++i) eq += (key_of(i) == T);
  long long tot;
  long long eq_before = block_exclusive_scan(eq, sm.scan, &tot);
  long long cnt = 0;
  {
    long long e = eq_before;
    for (int i = lo; i < hi; ++i) {
      uint64_t kv = key_of(i);
      bool s = kv > T;
      if (kv == T) { s = e < need; ++e; }
      cnt += s;
    }
  }
  long long pos = block_exclusive_scan(cnt, sm.scan, &tot);
  {
    long long e = eq_before;
    for (int i = lo; i < hi; ++i) {
      uint64_t kv = key_of(i);
      bool s = kv > T;
      if (kv == T) { s = e < need; ++e; }
      if (s) emit(i, static_cast<int>(pos++));
    }
  }
  return static_cast<int>(tot);
}

// Top k in ascending index order: emit(i, position) for each chosen i.
template <class KeyFn, class EmitFn>
__device__ int block_topk(KeyFn key_of, int n, int k, EmitFn emit, SelShared& sm) {
  if (k <= 0) return 0;
  if (k >= n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) emit(i, i);
    return n;
  }
  int need = 0;
  uint64_t T = block_topk_threshold(key_of, n, k, &need, sm);
  return block_emit_selected(key_of, n, T, need, emit, sm);
}

// Coverage cut: with elements ordered by (key desc, index asc) and weights
// z_of(i) >= 0, the shortest prefix whose weight sum S satisfies
// fl64(S) >= thr.  Emits that prefix in ascending index order and returns its
// length.  Requires thr <= fl64(sum of all weights) (sum < 2^63).
template <class KeyFn, class ZFn, class EmitFn>
__device__ int block_coverage_cut(KeyFn key_of, ZFn z_of, int n, double thr, EmitFn emit,
                                  SelShared& sm) {
  if (n <= 0 || !(thr > 0.0)) return 0;  // fl64(0) >= thr
  uint64_t prefix = 0, pmask = 0;
  long long before_sum = 0;  // weight of all elements ranked above the candidates
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += blockDim.x) { sm.hist[b] = 0; sm.hsum[b] = 0; }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint64_t kv = key_of(i);
      if ((kv & pmask) == prefix) {
        const int b = static_cast<int>((kv >> shift) & 255u);
        atomicAdd(&sm.hsum[b], static_cast<unsigned long long>(z_of(i)));
      }
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      long long c = 0;
      for (int j = 0; j < 4; ++j) c += static_cast<long long>(sm.hsum[4 * lane + j]);
      long long rev = c;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        long long u = __shfl_down(rev, o, kWave);
        if (lane + o < kWave) rev += u;
      }
      long long above = before_sum + (rev - c);
      // the first bucket (from the top) whose inclusive cumulative weight reaches thr
      for (int j = 3; j >= 0; --j) {
        long long h = static_cast<long long>(sm.hsum[4 * lane + j]);
        if (!(static_cast<double>(above) >= thr) && static_cast<double>(above + h) >= thr) {
          sm.digit = static_cast<uint64_t>(4 * lane + j);
          sm.above_sum = above;
        }
        above += h;
      }
    }
    __syncthreads();
    prefix |= sm.digit << shift;
    pmask |= 0xffull << shift;
    before_sum = sm.above_sum;
    __syncthreads();
  }
  // Elements with key == prefix share one weight zT (the weight is a function
  // of the key); take ties in index order until the cumulative weight
  // reaches thr.
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (key_of(i) == prefix) sm.tie_z = z_of(i);  // every writer stores the same value
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long zT = sm.tie_z;
    int j = 1;
    while (j < n && !(static_cast<double>(before_sum + j * zT) >= thr)) ++j;
    sm.need = j;
  }
  __syncthreads();
  const int need = sm.need;
  return block_emit_selected(key_of, n, prefix, need, emit, sm);
}

// ---------------------------------------------------------------------------
// Register-cached variant for n <= R * blockDim.x: every thread loads the keys
// (and, for the coverage cut, the weights) of its contiguous index chunk once;
// all radix passes and the emit pass then work on registers.  Same results as
// the functions above.
// ---------------------------------------------------------------------------
// hist[bin] += 1 (hist_count) or += val (hist_sum) for every lane with
// `valid`.  Radix passes over keys of similar magnitude put most lanes of a
// wave in one bin; when every valid lane of the wave agrees on the bin, one
// lane adds the wave's total (integer sums: the same result as one add per
// lane).  Wave-uniform control flow; ballots, readlane and DPP only.
__device__ __forceinline__ bool wave_same_bin(uint32_t bin, bool valid, uint64_t act, uint32_t* first) {
  const int fl = __builtin_ctzll(act);
  *first = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), fl));
  return __ballot(valid && bin != *first) == 0;
}

__device__ __forceinline__ void hist_count(uint32_t* hist, uint32_t bin, bool valid) {
  const uint64_t act = __ballot(valid);
  if (act == 0) return;
  uint32_t first;
  if (wave_same_bin(bin, valid, act, &first)) {
    if ((threadIdx.x & (kWave - 1)) == static_cast<unsigned>(__builtin_ctzll(act)))
      atomicAdd(&hist[first], static_cast<uint32_t>(__popcll(act)));
  } else if (valid) {
    atomicAdd(&hist[bin], 1u);
  }
}

__device__ __forceinline__ void hist_sum(unsigned long long* hist, uint32_t bin, bool valid,
                                         unsigned long long val) {
  const uint64_t act = __ballot(valid);
  if (act == 0) return;
  uint32_t first;
  if (wave_same_bin(bin, valid, act, &first)) {
    const unsigned long long tot = static_cast<unsigned long long>(wave_sum_i64(valid ? static_cast<long long>(val) : 0));
    if ((threadIdx.x & (kWave - 1)) == static_cast<unsigned>(__builtin_ctzll(act))) atomicAdd(&hist[first], tot);
  } else if (valid) {
    atomicAdd(&hist[bin], val);
  }
}

template <int R> struct SelChunk {
  int lo = 0, cnt = 0;
  uint64_t key[R];
  long long z[R];
};

// Chunk bounds of this thread and its keys key_of(lo + j).
template <int R, class KeyFn>
__device__ __forceinline__ void chunk_load(SelChunk<R>& c, int n, KeyFn key_of) {
  const int chunk = (n + static_cast<int>(blockDim.x) - 1) / static_cast<int>(blockDim.x);
  c.lo = min(n, static_cast<int>(threadIdx.x) * chunk);
  c.cnt = min(n, c.lo + chunk) - c.lo;
#pragma unroll
  for (int j = 0; j < R; ++j) c.key[j] = (j < c.cnt) ? key_of(c.lo + j) : 0ull;
}

constexpr int kResolveMax = 64;  // bucket size resolved by one wave instead of more passes

struct alignas(16) SelShared2 {
  uint32_t hist[2][256];
  unsigned long long hsum[2][256];
  uint32_t scan[kSelThreads / kWave];
  uint64_t digit[2];
  long long above[2];
  uint32_t inbin[2];   // candidates in the chosen bucket
  int need;
  long long tie_z;
  uint32_t nres;                     // resolve list length
  uint64_t rkey[kResolveMax];        // resolve list: keys and indices of the bucket
  int32_t ridx[kResolveMax];
  uint64_t rT;
  int rneed;
};

// One radix pass over the candidates (key & pmask) == prefix: the digit at
// `shift` whose bucket holds the rank-`remaining` element (counting from the
// top), and the count of candidates in higher buckets.  hist[b] must be zero
// on entry; hist[b ^ 1] is cleared here for the next pass.
template <int R>
__device__ __forceinline__ void chunk_pass(const SelChunk<R>& c, uint64_t prefix, uint64_t pmask,
                                           int shift, long long remaining, int b, SelShared2& sm) {
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const bool v = j < c.cnt && (c.key[j] & pmask) == prefix;
    hist_count(sm.hist[b], static_cast<uint32_t>((c.key[j] >> shift) & 255u), v);
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // lane owns bins 4 lane .. 4 lane + 3; count of candidates in the bins of
    // higher lanes = total - inclusive prefix (DPP scan, counts < 2^32)
    const int lane = threadIdx.x;
    const u32x4_t h4 = *reinterpret_cast<const u32x4_t*>(&sm.hist[b][4 * lane]);
    const uint32_t cs = h4[0] + h4[1] + h4[2] + h4[3];
    const uint32_t inc = wave_incl_scan_u32(cs);
    long long above = static_cast<long long>(wave_last_u32(inc) - inc);
    for (int j = 3; j >= 0; --j) {
      const long long h = h4[j];
      if (above < remaining && remaining <= above + h) {
        sm.digit[b] = static_cast<uint64_t>(4 * lane + j);
        sm.above[b] = above;
        sm.inbin[b] = static_cast<uint32_t>(h);
      }
      above += h;
    }
  } else {
    for (int q = static_cast<int>(threadIdx.x) - kWave; q < 256; q += static_cast<int>(blockDim.x) - kWave)
      sm.hist[b ^ 1][q] = 0;
  }
  __syncthreads();
}

// Emit, in ascending index order, every element with key > T and the first
// `need` elements with key == T: emit(i, position, j) with j the register slot.
template <int R, class EmitFn>
__device__ __forceinline__ int chunk_emit(const SelChunk<R>& c, uint64_t T, int need, EmitFn emit,
                                          SelShared2& sm) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < R; ++j)
    if (j < c.cnt) { gt += c.key[j] > T; eq += c.key[j] == T; }
  // one scan of (gt << 16 | eq) (both < 2^16 for n <= R blockDim <= 4096):
  // counts before this thread's chunk
  uint32_t tot;
  const uint32_t before = block_exclusive_scan_u32((gt << 16) | eq, sm.scan, &tot);
  const long long gt_before = static_cast<long long>(before >> 16);
  long long e = static_cast<long long>(before & 0xffffu);
  long long pos = gt_before + min(e, static_cast<long long>(need));
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j >= c.cnt) continue;
    bool s = c.key[j] > T;
    if (c.key[j] == T) { s = e < need; ++e; }
    if (s) emit(c.lo + j, static_cast<int>(pos++), j);
  }
  return static_cast<int>(tot >> 16) + need;
}

// Top k (1 <= k) of the cached keys in ascending index order.
template <int R, class EmitFn>
__device__ int chunk_topk(const SelChunk<R>& c, int n, int k, EmitFn emit, SelShared2& sm) {
  if (k <= 0) return 0;
  if (k >= n) {
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < c.cnt) emit(c.lo + j, c.lo + j, j);
    return n;
  }
  for (int q = threadIdx.x; q < 256; q += blockDim.x) sm.hist[0][q] = 0;
  if (threadIdx.x == 0) sm.nres = 0;
  __syncthreads();
  uint64_t prefix = 0, pmask = 0;
  long long remaining = k;
  int b = 0;
  for (int shift = 56; shift >= 0; shift -= 8, b ^= 1) {
    chunk_pass(c, prefix, pmask, shift, remaining, b, sm);
    prefix |= sm.digit[b] << shift;
    pmask |= 0xffull << shift;
    remaining -= sm.above[b];
    if (shift > 0 && sm.inbin[b] <= static_cast<uint32_t>(kResolveMax)) {
      // Few candidates left in the bucket: list them, and one wave ranks them
      // by (key desc, index asc); the rank-`remaining` one gives T, and `need`
      // counts the chosen elements equal to T.
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if (j < c.cnt && (c.key[j] & pmask) == prefix) {
          const uint32_t slot = atomicAdd(&sm.nres, 1u);
          sm.rkey[slot] = c.key[j];
          sm.ridx[slot] = c.lo + j;
        }
      }
      __syncthreads();
      if (threadIdx.x < kWave) {
        const int m = static_cast<int>(sm.nres);
        const int t = threadIdx.x;
        if (t < m) {
          const uint64_t kt = sm.rkey[t];
          const int it = sm.ridx[t];
          int rank = 0, gt = 0;
          for (int u = 0; u < m; ++u) {
            const uint64_t ku = sm.rkey[u];
            rank += (ku > kt) || (ku == kt && sm.ridx[u] < it);
            gt += ku > kt;
          }
          if (rank == remaining - 1) {
            sm.rT = kt;
            sm.rneed = static_cast<int>(remaining) - gt;
          }
        }
      }
      __syncthreads();
      return chunk_emit(c, sm.rT, sm.rneed, emit, sm);
    }
  }
  return chunk_emit(c, prefix, static_cast<int>(remaining), emit, sm);
}

// Coverage cut over the cached keys and weights c.z (see block_coverage_cut).
template <int R, class EmitFn>
__device__ int chunk_coverage_cut(const SelChunk<R>& c, int n, double thr, EmitFn emit, SelShared2& sm) {
  if (n <= 0 || !(thr > 0.0)) return 0;
  for (int q = threadIdx.x; q < 256; q += blockDim.x) sm.hsum[0][q] = 0;
  __syncthreads();
  uint64_t prefix = 0, pmask = 0;
  long long before_sum = 0;
  int b = 0;
  for (int shift = 56; shift >= 0; shift -= 8, b ^= 1) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const bool v = j < c.cnt && (c.key[j] & pmask) == prefix;
      hist_sum(sm.hsum[b], static_cast<uint32_t>((c.key[j] >> shift) & 255u), v,
               static_cast<unsigned long long>(v ? c.z[j] : 0));
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      uint64_t cs = 0;
      for (int j = 0; j < 4; ++j) cs += sm.hsum[b][4 * lane + j];
      const uint64_t inc = wave_incl_scan_u64(cs);
      long long above = before_sum + static_cast<long long>(wave_last_u64(inc) - inc);
      for (int j = 3; j >= 0; --j) {
        const long long h = static_cast<long long>(sm.hsum[b][4 * lane + j]);
        if (!(static_cast<double>(above) >= thr) && static_cast<double>(above + h) >= thr) {
          sm.digit[b] = static_cast<uint64_t>(4 * lane + j);
          sm.above[b] = above;
        }
        above += h;
      }
    } else {
      for (int q = static_cast<int>(threadIdx.x) - kWave; q < 256; q += static_cast<int>(blockDim.x) - kWave)
        sm.hsum[b ^ 1][q] = 0;
    }
    __syncthreads();
    prefix |= sm.digit[b] << shift;
    pmask |= 0xffull << shift;
    before_sum = sm.above[b];
  }
  // ties share one weight; take them in index order until thr is reached
#pragma unroll
  for (int j = 0; j < R; ++j)
    if (j < c.cnt && c.key[j] == prefix) sm.tie_z = c.z[j];
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long zT = sm.tie_z;
    int j = 1;
    while (j < n && !(static_cast<double>(before_sum + j * zT) >= thr)) ++j;
    sm.need = j;
  }
  __syncthreads();
  return chunk_emit(c, prefix, sm.need, emit, sm);
}

}  // namespace cgs
