// Workgroup-level scan and radix-cut helpers for the top-k kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sga_device.h"

namespace sga {

// DPP source of a row shift or row broadcast; lanes with no source (or in a
// row the mask leaves out) read 0, the identity of the sums below.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_shifted(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: shifts by
// 1, 2, 4 and 8 lanes inside each 16-lane row (DPP row_shr), then the last
// lane of rows 0 and 2 added into rows 1 and 3 (row_bcast:15), then the last
// lane of row 1 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_shifted<0x111, 0xf>(x);
  x += dpp_shifted<0x112, 0xf>(x);
  x += dpp_shifted<0x114, 0xf>(x);
  x += dpp_shifted<0x118, 0xf>(x);
  x += dpp_shifted<0x142, 0xa>(x);
  x += dpp_shifted<0x143, 0xc>(x);
  return x;
}

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
  const uint32_t x = wave_incl_scan(sum);
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
  const uint32_t xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) {
    scratch[wid] = xa;
    scratch[kWaves + wid] = xb;
  }
  __syncthreads();
  uint32_t ba = 0, bb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (w < wid) {
      ba += scratch[w];
      bb += scratch[kWaves + w];
    }
  a_before = ba + xa - a;
  b_before = bb + xb - b;
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

// Writes a workgroup's LDS digit-1 histogram (kHist1 bins) as a list into its
// slot of slot_words words, with plain stores: word 0 the number m of nonzero
// bins, then one entry (bin << 16 | count) per nonzero bin, or word 0 =
// kHistOverflow when m > slot_words - 1. Counts are below 2^16 (a chunk holds
// at most 4,096 positions). The entries are in ascending bin order rotated
// left by `rot` places (the reader sums them in any order; chunks of one
// token list mostly the same bins, and rotating each by its chunk index
// spreads the reader's same-offset LDS atomics over different bins). Thread j
// takes bins [P*j, P*j + P); a wave scan and one LDS exchange place its
// entries. scratch: NT/64 words of LDS. All threads must call; no barrier follows.
template <int NT>
__device__ __forceinline__ void hist1_list_store(const uint32_t* lds_hist, uint32_t* slot,
                                                 int slot_words, uint32_t rot, uint32_t* scratch) {
  constexpr int P = kHist1 / NT;
  constexpr int kWaves = NT / 64;
  static_assert(P % 4 == 0 && P * NT == kHist1, "whole 16-byte runs per thread");
  __syncthreads();
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b0 = (int)threadIdx.x * P;
  uint32_t h[P];
#pragma unroll
  for (int q = 0; q < P / 4; ++q) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(lds_hist + b0 + 4 * q);
    h[4 * q] = x.x;
    h[4 * q + 1] = x.y;
    h[4 * q + 2] = x.z;
    h[4 * q + 3] = x.w;
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) cnt += h[i] != 0u;
  const uint32_t x = wave_incl_scan(cnt);
  if (lane == 63) scratch[wid] = x;
  __syncthreads();
  uint32_t before = x - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t sw = scratch[w];
    if (w < wid) before += sw;
    total += sw;
  }
  if (total >= (uint32_t)slot_words) {
    if (threadIdx.x == 0) slot[0] = kHistOverflow;
    return;
  }
  if (total == 0) {
    if (threadIdx.x == 0) slot[0] = 0u;
    return;
  }
  // rank r goes to word 1 + (r + rot) mod total
  uint32_t o = before + rot % total;
  if (o >= total) o -= total;
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (h[i]) {
      slot[1 + o] = ((uint32_t)(b0 + i) << 16) | h[i];
      o = o + 1 == total ? 0u : o + 1;
    }
  if (threadIdx.x == 0) slot[0] = total;
}

// Zeroes one token's kHist2-word second-level histogram with 16-byte stores
// (a workgroup of NT threads, or one wave with NT = 64).
template <int NT>
__device__ __forceinline__ void hist2_zero(uint32_t* h2, int tid) {
  static_assert(kHist2 % (4 * NT) == 0, "whole 16-byte stores per thread");
#pragma unroll
  for (int q = 0; q < kHist2 / (4 * NT); ++q)
    reinterpret_cast<u32x4*>(h2)[q * NT + tid] = u32x4{0u, 0u, 0u, 0u};
}

// A radix cut straight from a histogram in global memory, with no LDS copy.
// Thread j holds bins [nbins - P(j+1), nbins - Pj) in registers (P = nbins/NT,
// a multiple of 4), so thread 0 holds the top bins. load() issues the loads;
// cut() waits for them and finds d with S(d+1) < r <= S(d), where S(d) is the
// sum of the bins >= d, for 1 <= r <= S(0). Every thread gets d, S(d+1) and
// the count of bin d. scratch: NT/64 + 3 words of LDS, free again on return.
template <int NT, int NBINS>
struct HistRun {
  static constexpr int P = NBINS / NT;
  static_assert(P % 4 == 0 && P * NT == NBINS, "whole 16-byte runs per thread");
  u32x4 v[P / 4];

  __device__ __forceinline__ void load(const uint32_t* ghist) {
    const u32x4* src = reinterpret_cast<const u32x4*>(ghist + NBINS - P * ((int)threadIdx.x + 1));
#pragma unroll
    for (int q = 0; q < P / 4; ++q) v[q] = src[q];
  }

  // The same runs, read from a histogram in LDS.
  __device__ __forceinline__ void load_lds(const uint32_t* lhist) {
    const u32x4* src = reinterpret_cast<const u32x4*>(lhist + NBINS - P * ((int)threadIdx.x + 1));
#pragma unroll
    for (int q = 0; q < P / 4; ++q) v[q] = src[q];
  }

  // After load() of a region of list slots (see hist1_list_store): adds every
  // listed entry into the LDS histogram lhist (zeroed, and the zeroing
  // published by a barrier) and marks overflowed slots in ovf (zeroed bit
  // mask, one bit per slot). Thread j holds region words [NBINS - P(j+1),
  // NBINS - Pj); a slot of sw words (16 <= P <= sw, sw <= 64 P) spans
  // sw / P consecutive lanes of one wave, its header word 0 held by the
  // highest of them. Slots at or past `slots` are not read.
  __device__ __forceinline__ void add_lists(int sw, int slots, uint32_t* lhist, uint32_t* ovf) const {
    const int lane = threadIdx.x & 63;
    const int w0 = NBINS - P * ((int)threadIdx.x + 1);   // first region word of this thread
    const int s = w0 / sw, o0 = w0 - s * sw;               // its slot and offset there
    const int tps = sw / P;                                 // threads per slot
    const uint32_t m = (uint32_t)__shfl((int)v[0].x, lane | (tps - 1));
    if (s >= slots) return;
    if (m == kHistOverflow) {
      if (o0 == 0) atomicOr(&ovf[s >> 5], 1u << (s & 31));
      return;
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint32_t o = (uint32_t)(o0 + i);
      const uint32_t e = v[i / 4][i % 4];
      if (o >= 1u && o <= m) atomicAdd(&lhist[e >> 16], e & 0xffffu);
    }
  }

  __device__ __forceinline__ void cut(uint32_t r, uint32_t* scratch, uint32_t& d, uint32_t& above,
                                      uint32_t& count) const {
    constexpr int kWaves = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < P / 4; ++q) sum += v[q].x + v[q].y + v[q].z + v[q].w;
    const uint32_t x = wave_incl_scan(sum);
    if (lane == 63) scratch[wid] = x;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (w < wid) before += scratch[w];
    const uint32_t incl = before + x, excl = incl - sum;
    if (excl < r && r <= incl) {
      // bins from the top of this run down: element e of v[q] is bin base + 4q + e
      const int base = NBINS - P * ((int)threadIdx.x + 1);
      uint32_t acc = excl;
      bool found = false;
#pragma unroll
      for (int i = P - 1; i >= 0; --i) {
        const uint32_t c = v[i / 4][i % 4];
        if (!found && acc + c >= r) {
          scratch[kWaves] = (uint32_t)(base + i);
          scratch[kWaves + 1] = acc;
          scratch[kWaves + 2] = c;
          found = true;
        }
        acc += c;
      }
    }
    __syncthreads();
    d = scratch[kWaves];
    above = scratch[kWaves + 1];
    count = scratch[kWaves + 2];
    __syncthreads();
  }
};

}  // namespace sga
