// Workgroup-level scan and radix-cut helpers for the top-k kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sga_device.h"

namespace sga {

// Exclusive prefix sum of one uint32 per thread over a workgroup of NT threads
// (NT a multiple of 64). scratch: NT/64 + 1 words of LDS. All threads must call.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wid] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int i = 0; i < NT / 64; ++i) {
      uint32_t s = scratch[i];
      scratch[i] = acc;
      acc += s;
    }
    scratch[NT / 64] = acc;
  }
  __syncthreads();
  uint32_t r = scratch[wid] + x - v;
  *total = scratch[NT / 64];
  __syncthreads();
  return r;
}

// Radix cut over a histogram h[0..nbins) in LDS, digits ranked from the top:
// finds d with S(d+1) < r <= S(d), S(d) = sum of h[b] for b >= d, 1 <= r <= S(0).
// Writes res[0] = d and res[1] = S(d+1). Thread j owns a run of bins from the
// top; with fewer bins than threads the last threads own none.
template <int NT>
__device__ __forceinline__ void block_find_cut(const uint32_t* h, int nbins, uint32_t r,
                                               uint32_t* scratch, uint32_t* res) {
  const int per = (nbins + NT - 1) / NT;
  const int top = nbins - (int)threadIdx.x * per;
  const int cnt = top <= 0 ? 0 : (top < per ? top : per);
  uint32_t sum = 0;
  for (int i = 1; i <= cnt; ++i) sum += h[top - i];
  uint32_t total;
  uint32_t above = block_excl_scan<NT>(sum, scratch, &total);
  if (above < r && r <= above + sum) {
    uint32_t acc = above;
    for (int i = 1; i <= cnt; ++i) {
      uint32_t c = h[top - i];
      if (acc + c >= r) {
        res[0] = (uint32_t)(top - i);
        res[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Radix cut with two workgroup barriers: h[0..nbins) in LDS, ranked from the
// top, 1 <= r <= S(0). Finds d with S(d+1) < r <= S(d), S(d) = sum of h[b]
// for b >= d, and returns d and S(d+1) to every thread. Thread j owns a run
// of bins from the top; a wave scan gives each thread its running total and
// each wave adds the totals of the waves before it. scratch: NT/64 + 2
// words of LDS, free again once the function returns.
template <int NT>
__device__ __forceinline__ void block_cut(const uint32_t* h, int nbins, uint32_t r, uint32_t* scratch,
                                          uint32_t& d, uint32_t& above) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int per = (nbins + NT - 1) / NT;
  const int top = nbins - (int)threadIdx.x * per;
  const int cnt = top <= 0 ? 0 : (top < per ? top : per);
  uint32_t sum = 0;
  for (int i = 1; i <= cnt; ++i) sum += h[top - i];
  uint32_t x = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wid] = x;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (w < wid) before += scratch[w];
  const uint32_t incl = before + x, excl = incl - sum;
  if (excl < r && r <= incl) {
    uint32_t acc = excl;
    for (int i = 1; i <= cnt; ++i) {
      const uint32_t c = h[top - i];
      if (acc + c >= r) {
        scratch[kWaves] = (uint32_t)(top - i);
        scratch[kWaves + 1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  d = scratch[kWaves];
  above = scratch[kWaves + 1];
  __syncthreads();
}

// Exclusive prefix sums of two counters per thread over a workgroup, in one
// pass (the pair travels as one 64-bit value; neither total may reach 2^32).
// scratch: 2 * (NT/64) words of LDS, free again once the function returns.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t* scratch,
                                                 uint32_t& a_before, uint32_t& b_before) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  unsigned long long v = (unsigned long long)a | ((unsigned long long)b << 32), x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  unsigned long long* s64 = reinterpret_cast<unsigned long long*>(scratch);
  if (lane == 63) s64[wid] = x;
  __syncthreads();
  unsigned long long before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (w < wid) before += s64[w];
  const unsigned long long e = before + x - v;
  a_before = (uint32_t)e;
  b_before = (uint32_t)(e >> 32);
  __syncthreads();
}

// Device-scope relaxed load that bypasses the non-coherent vector L1.
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Adds a workgroup's LDS digit-1 histogram into the token's global histogram
// (relaxed device-scope atomics; visible to the next kernel on the stream).
// Two adjacent bins go in one 64-bit atomic: a bin counts at most one token's
// positions (< 2^32), so the low half never carries into the high half.
// No fence and no cross-workgroup hand-off: the cut is taken by the next kernel.
template <int NT>
__device__ __forceinline__ void hist1_flush(const uint32_t* lds_hist, uint32_t* ghist) {
  __syncthreads();
  unsigned long long* g64 = reinterpret_cast<unsigned long long*>(ghist);
  for (int b = threadIdx.x; b < kHist1 / 2; b += NT) {
    const uint32_t c0 = lds_hist[2 * b], c1 = lds_hist[2 * b + 1];
    if (c0 | c1) atomicAdd(g64 + b, (unsigned long long)c0 | ((unsigned long long)c1 << 32));
  }
}

// First radix cut of a token from its global digit-1 histogram: the digit of
// the k-th largest score and the count of scores with a larger digit.
// Every thread of the workgroup gets the result. lds_hist: kHist1 words;
// scratch: at least NT/64 + 2 words.
template <int NT>
__device__ __forceinline__ void hist1_cut(const uint32_t* ghist, uint32_t* lds_hist, uint32_t k,
                                          uint32_t* scratch, uint32_t& digit1, uint32_t& above1) {
  static_assert(kHist1 % NT == 0, "whole bins per thread");
  uint32_t h[kHist1 / NT];   // every load in flight before the first LDS store
#pragma unroll
  for (int u = 0; u < kHist1 / NT; ++u) h[u] = ghist[u * NT + threadIdx.x];
#pragma unroll
  for (int u = 0; u < kHist1 / NT; ++u) lds_hist[u * NT + threadIdx.x] = h[u];
  __syncthreads();
  block_cut<NT>(lds_hist, kHist1, k, scratch, digit1, above1);
}

}  // namespace sga
