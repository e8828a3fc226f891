// Per-token top-k over indexer scores: keep the min(k, n) best positions,
// ties to the lower position, written in ascending order and -1 padded.
// Sources: A.X K2 fact sheet (archdb), token-selection fact: top-2048
// positions per query. rebasdaily article, section on long tasks that cannot
// re-read all old content: at most 2,048 positions per query.
//
// Exact radix select on order-preserving uint32 keys. For batches of many
// tokens (contexts up to 256K), topk_token_kernel does stages 2-3 below in
// one workgroup per token; otherwise they run as separate kernels over many
// workgroups per token. The stages:
//   1. digit-1 histogram: the top 12 key bits of every score, built in the
//      indexer epilogue (fused path) or by topk_hist_kernel.
//   2. topk_select_kernel (many workgroups per token): every workgroup first
//      finds digit1, the top-12-bit value of the k-th largest score, from the
//      histogram (the kernel boundary orders it after every histogram update,
//      so no cross-workgroup hand-off or device-scope fence is needed).
//      Positions whose digit is above digit1 go straight into a selection
//      bitmap; one ballot gives 64 positions. Positions whose digit equals
//      digit1 are appended, with their keys, to a candidate list.
//   3. topk_finalize_kernel (one workgroup per token): two more radix levels
//      (12 and 8 bits) over the candidates, staged in LDS when they fit, find
//      the exact k-th key. Ties at that key are kept lowest position first,
//      using a prefix count over a tie bitmap. An ordered compaction of the
//      bitmaps then writes the kept positions in ascending order.
// Every decision depends only on the score values, so the result is exact.
#include "sga_block.h"
#include "sga_kernels.h"

namespace sga {
namespace {

constexpr int kHistThreads = 256;
constexpr int kSelThreads = 256;
constexpr int kFinThreads = 1024;
constexpr int kCutThreads = 1024;

__global__ __launch_bounds__(256) void clear_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(TopkArgs a) {
  __shared__ uint32_t lds_hist[kHist1];
  const int t = blockIdx.y;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  for (int b = threadIdx.x; b < kHist1; b += kHistThreads) lds_hist[b] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * kIndexerChunk;
  const int c1 = min(n, c0 + kIndexerChunk);
  const float* srow = a.scores + (int64_t)t * a.ld;
  for (int p = c0 + threadIdx.x; p < c1; p += kHistThreads)
    atomicAdd(&lds_hist[score_key(srow[p]) >> (32 - kDigit1Bits)], 1u);
  hist1_flush<kHistThreads>(lds_hist, a.hist + (int64_t)t * kHist1);
}

// First radix cut of each token: digit1 and above1 from its histogram.
__global__ __launch_bounds__(kCutThreads) void topk_cut_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kHist1];
  __shared__ uint32_t scratch[32];
  const int t = blockIdx.x;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  if (n <= a.k) return;  // every visible position is kept
  uint32_t d1, above1;
  hist1_cut<kCutThreads>(a.hist + (int64_t)t * kHist1, hist, (uint32_t)a.k, scratch, d1, above1);
  if (threadIdx.x == 0) {
    a.ctrl[t].digit1 = d1;
    a.ctrl[t].above1 = above1;
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ uint32_t stage_pos[kSelectChunk];   // also holds the histogram for the cut
  __shared__ uint32_t stage_key[kSelectChunk];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t stage_count;
  __shared__ uint32_t stage_base;
  static_assert(kHist1 <= kSelectChunk, "the cut histogram lives in stage_pos");
  constexpr int kSteps = kSelectChunk / kSelThreads;   // 64-position steps per wave
  const int t = blockIdx.y;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  if (n <= a.k) return;  // every visible position is kept; finalize writes them
  const int c0 = blockIdx.x * kSelectChunk;
  if (c0 >= n) return;
  const int c1 = min(n, c0 + kSelectChunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* srow = a.scores + (int64_t)t * a.ld;
  // issue every score load of this workgroup at once
  float v[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) v[i] = srow[min(c0 + i * kSelThreads + wave * 64 + lane, c1 - 1)];
  // first radix cut, taken redundantly by every workgroup of the token from the
  // histogram the previous kernel completed (no cross-workgroup hand-off)
  uint32_t d1, above1;
  hist1_cut<kSelThreads>(a.hist + (int64_t)t * kHist1, stage_pos, (uint32_t)a.k, scratch, d1, above1);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.ctrl[t].digit1 = d1;
    a.ctrl[t].above1 = above1;
  }
  if (threadIdx.x == 0) stage_count = 0;
  __syncthreads();
  uint32_t* sel = a.sel + (int64_t)t * a.words;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int p0 = c0 + i * kSelThreads + wave * 64;
    if (p0 >= c1) break;
    const int p = p0 + lane;
    const bool valid = p < c1;
    const uint32_t key = score_key(v[i]);
    const uint32_t dig = key >> (32 - kDigit1Bits);
    const uint64_t above = __ballot(valid && dig > d1);
    const uint64_t cand = __ballot(valid && dig == d1);
    if (lane == 0) {
      sel[p0 >> 5] = (uint32_t)above;
      sel[(p0 >> 5) + 1] = (uint32_t)(above >> 32);
    }
    if (cand) {
      uint32_t off = 0;
      if (lane == 0) off = atomicAdd(&stage_count, (uint32_t)__popcll(cand));
      off = __shfl(off, 0);
      if (valid && dig == d1) {
        const uint32_t rank = (uint32_t)__popcll(cand & ((1ull << lane) - 1ull));
        stage_pos[off + rank] = (uint32_t)p;
        stage_key[off + rank] = key;
      }
    }
  }
  __syncthreads();
  const uint32_t cnt = stage_count;
  if (cnt == 0) return;
  if (threadIdx.x == 0) stage_base = atomicAdd(&a.ctrl[t].cand_count, cnt);
  __syncthreads();
  uint32_t* gpos = a.cand + (int64_t)t * a.cand_cap + stage_base;
  uint32_t* gkey = a.cand_key + (int64_t)t * a.cand_cap + stage_base;
  for (uint32_t i = threadIdx.x; i < cnt; i += kSelThreads) {
    gpos[i] = stage_pos[i];
    gkey[i] = stage_key[i];
  }
}

// Candidate i of the finalize kernel: from LDS when staged there, else global.
struct Cands {
  const uint32_t* pos;
  const uint32_t* key;
  __device__ __forceinline__ uint32_t p(uint32_t i) const { return pos[i]; }
  __device__ __forceinline__ uint32_t k(uint32_t i) const { return key[i]; }
};

// Dynamic LDS: level-2 histogram (4096) | level-3 histogram (256) | scratch
// (32) | tie bitmap (words) | selection bitmap (words) | staged candidate
// positions (lds_cand_cap) | their keys (lds_cand_cap).
__global__ __launch_bounds__(kFinThreads) void topk_finalize_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* hist2 = lds;
  uint32_t* hist3 = hist2 + kHist2;
  uint32_t* scratch = hist3 + kHist3;
  uint32_t* tie = scratch + 32;
  uint32_t* selL = tie + a.words;
  uint32_t* lpos = selL + a.words;
  uint32_t* lkey = lpos + a.lds_cand_cap;
  uint32_t* res = scratch + 24;
  const int t = blockIdx.x;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  int32_t* out = a.indices + (int64_t)t * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kFinThreads) out[i] = i < n ? i : -1;
    return;
  }
  const uint32_t m = a.ctrl[t].cand_count;
  const uint32_t d1 = a.ctrl[t].digit1;
  const uint32_t r1 = (uint32_t)a.k - a.ctrl[t].above1;  // still needed, 1 <= r1 <= m
  Cands c{a.cand + (int64_t)t * a.cand_cap, a.cand_key + (int64_t)t * a.cand_cap};
  const int words = (n + 31) >> 5;
  // stage: selection bitmap and candidates into LDS (four loads of each in
  // flight per thread); clear the histograms and the two candidate bitmaps
  {
    const uint32_t* sel = a.sel + (int64_t)t * a.words;
    for (int i0 = 0; i0 < words; i0 += 4 * kFinThreads) {
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = sel[min(i0 + u * kFinThreads + (int)threadIdx.x, words - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kFinThreads + threadIdx.x;
        if (i < words) {
          selL[i] = w[u];
          tie[i] = 0;
        }
      }
    }
    if (m <= (uint32_t)a.lds_cand_cap) {
      for (uint32_t i0 = 0; i0 < m; i0 += 4 * kFinThreads) {
        uint32_t pp[4], kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t i = min(i0 + u * kFinThreads + threadIdx.x, m - 1);
          pp[u] = c.pos[i];
          kk[u] = c.key[i];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t i = i0 + u * kFinThreads + threadIdx.x;
          if (i < m) {
            lpos[i] = pp[u];
            lkey[i] = kk[u];
          }
        }
      }
      c = Cands{lpos, lkey};
    }
    for (int b = threadIdx.x; b < kHist2 + kHist3; b += kFinThreads) hist2[b] = 0;
  }
  __syncthreads();

  // level 2: key bits 19..8 of the candidates
  for (uint32_t i = threadIdx.x; i < m; i += kFinThreads)
    atomicAdd(&hist2[(c.k(i) >> kDigit3Bits) & (kHist2 - 1)], 1u);
  __syncthreads();
  block_find_cut<kFinThreads>(hist2, kHist2, r1, scratch, res);
  const uint32_t d2 = res[0];
  const uint32_t r2 = r1 - res[1];
  // level 3: key bits 7..0 of the candidates that match digit 2
  for (uint32_t i = threadIdx.x; i < m; i += kFinThreads) {
    const uint32_t key = c.k(i);
    if (((key >> kDigit3Bits) & (kHist2 - 1)) == d2) atomicAdd(&hist3[key & (kHist3 - 1)], 1u);
  }
  __syncthreads();
  block_find_cut<kFinThreads>(hist3, kHist3, r2, scratch, res);
  const uint32_t d3 = res[0];
  const uint32_t ties_kept = r2 - res[1];  // positions with key == kth to keep
  const uint32_t kth = (d1 << (32 - kDigit1Bits)) | (d2 << kDigit3Bits) | d3;

  // candidates above the k-th key join the selection; ties at it are marked apart
  for (uint32_t i = threadIdx.x; i < m; i += kFinThreads) {
    const uint32_t key = c.k(i);
    if (key >= kth) {
      const uint32_t p = c.p(i);
      atomicOr(key > kth ? &selL[p >> 5] : &tie[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  // keep the ties_kept lowest-position ties: thread j owns a contiguous run of words
  const int per = (words + kFinThreads - 1) / kFinThreads;
  const int w0 = min(words, (int)threadIdx.x * per), w1 = min(words, w0 + per);
  {
    uint32_t cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(tie[i]);
    uint32_t total;
    uint32_t before = block_excl_scan<kFinThreads>(cnt, scratch, &total);
    for (int i = w0; i < w1; ++i) {
      uint32_t bits = tie[i];
      const uint32_t pc = __popc(bits);
      if (before >= ties_kept) {
        bits = 0;
      } else if (before + pc > ties_kept) {
        const uint32_t keep = ties_kept - before;  // keep the lowest `keep` set bits
        uint32_t nb = 0;
        for (uint32_t kept = 0; kept < keep; ++kept) {
          const uint32_t low = bits & (0u - bits);
          nb |= low;
          bits ^= low;
        }
        bits = nb;
      }
      before += pc;
      tie[i] = bits;   // only this thread reads these words below
    }
  }
  // ordered compaction of the selection and the kept ties
  uint32_t cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(selL[i] | tie[i]);
  uint32_t total;
  uint32_t off = block_excl_scan<kFinThreads>(cnt, scratch, &total);
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = selL[i] | tie[i];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (off < (uint32_t)a.k) out[off] = (i << 5) + b;
      ++off;
    }
  }
  for (int i = (int)total + threadIdx.x; i < a.k; i += kFinThreads) out[i] = -1;
}

// The whole selection of one token in one workgroup, for contexts whose two
// bitmaps fit in LDS: the first radix cut from the histogram, one streaming
// pass over the scores (bitmap + candidates), the two refining radix levels,
// the tie rule and the ordered compaction. Candidates beyond the LDS capacity
// spill to the workspace.
// Dynamic LDS: histogram (4096) | scratch (32) | selection bitmap (words) |
// tie/extra bitmap (words) | candidate positions (cap) | candidate keys (cap).
constexpr int kTokThreads = 1024;
constexpr int kTokWaves = kTokThreads / 64;
constexpr int kTokUnroll = 16;   // score loads in flight per lane
static_assert(kHist1 == kHist2, "one LDS histogram serves both levels");

__global__ __launch_bounds__(kTokThreads) void topk_token_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds[];
  const int C = a.lds_cand_cap;
  uint32_t* hist = lds;
  uint32_t* scratch = hist + kHist1;
  uint32_t* sel = scratch + 32;
  uint32_t* extra = sel + a.words;
  uint32_t* cpos = extra + a.words;
  uint32_t* ckey = cpos + C;
  uint32_t* res = scratch + 24;
  uint32_t* counter = scratch + 28;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  int32_t* out = a.indices + (int64_t)t * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kTokThreads) out[i] = i < n ? i : -1;
    return;
  }
  uint32_t* gpos = a.cand + (int64_t)t * a.cand_cap;
  uint32_t* gkey = a.cand_key + (int64_t)t * a.cand_cap;
  const float* srow = a.scores + (int64_t)t * a.ld;

  // 1. first radix cut
  {
    const uint32_t* gh = a.hist + (int64_t)t * kHist1;
    uint32_t h[kHist1 / kTokThreads];
#pragma unroll
    for (int u = 0; u < kHist1 / kTokThreads; ++u) h[u] = gh[u * kTokThreads + threadIdx.x];
#pragma unroll
    for (int u = 0; u < kHist1 / kTokThreads; ++u) hist[u * kTokThreads + threadIdx.x] = h[u];
  }
  if (threadIdx.x == 0) *counter = 0;
  __syncthreads();
  block_find_cut<kTokThreads>(hist, kHist1, (uint32_t)a.k, scratch, res);
  const uint32_t d1 = res[0];
  const uint32_t r1 = (uint32_t)a.k - res[1];   // still needed from the candidates
  __syncthreads();

  // 2. one pass over the scores: 64-position groups, kTokUnroll per lane in flight
  const int ngroups = (n + 63) >> 6;
  for (int gb = 0; gb < ngroups; gb += kTokWaves * kTokUnroll) {
    float v[kTokUnroll];
#pragma unroll
    for (int u = 0; u < kTokUnroll; ++u)
      v[u] = srow[min(((gb + u * kTokWaves + wave) << 6) + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < kTokUnroll; ++u) {
      const int gidx = gb + u * kTokWaves + wave;
      if (gidx >= ngroups) break;
      const int p = (gidx << 6) + lane;
      const bool valid = p < n;
      const uint32_t key = score_key(v[u]);
      const uint32_t dig = key >> (32 - kDigit1Bits);
      const uint64_t above = __ballot(valid && dig > d1);
      const uint64_t cand = __ballot(valid && dig == d1);
      if (lane == 0) {
        sel[2 * gidx] = (uint32_t)above;
        sel[2 * gidx + 1] = (uint32_t)(above >> 32);
      }
      if (cand) {
        uint32_t off = 0;
        if (lane == 0) off = atomicAdd(counter, (uint32_t)__popcll(cand));
        off = __shfl(off, 0);
        if (valid && dig == d1) {
          const uint32_t i = off + (uint32_t)__popcll(cand & ((1ull << lane) - 1ull));
          if (i < (uint32_t)C) {
            cpos[i] = (uint32_t)p;
            ckey[i] = key;
          } else {
            gpos[i - C] = (uint32_t)p;
            gkey[i - C] = key;
          }
        }
      }
    }
  }
  __syncthreads();
  const uint32_t m = *counter;
  auto KEY = [&](uint32_t i) -> uint32_t { return i < (uint32_t)C ? ckey[i] : gkey[i - C]; };
  auto POS = [&](uint32_t i) -> uint32_t { return i < (uint32_t)C ? cpos[i] : gpos[i - C]; };

  // 3. level 2: key bits 19..8 of the candidates
  for (int b = threadIdx.x; b < kHist2; b += kTokThreads) hist[b] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += kTokThreads)
    atomicAdd(&hist[(KEY(i) >> kDigit3Bits) & (kHist2 - 1)], 1u);
  __syncthreads();
  block_find_cut<kTokThreads>(hist, kHist2, r1, scratch, res);
  const uint32_t d2 = res[0];
  const uint32_t r2 = r1 - res[1];
  __syncthreads();
  // level 3: key bits 7..0 of the candidates that match digit 2
  for (int b = threadIdx.x; b < kHist3; b += kTokThreads) hist[b] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += kTokThreads) {
    const uint32_t key = KEY(i);
    if (((key >> kDigit3Bits) & (kHist2 - 1)) == d2) atomicAdd(&hist[key & (kHist3 - 1)], 1u);
  }
  __syncthreads();
  block_find_cut<kTokThreads>(hist, kHist3, r2, scratch, res);
  const uint32_t d3 = res[0];
  const uint32_t ties_kept = r2 - res[1];
  const uint32_t kth = (d1 << (32 - kDigit1Bits)) | (d2 << kDigit3Bits) | d3;
  __syncthreads();

  // 4. ties at the k-th key, lowest positions first; then the candidates above it
  const int words = (n + 31) >> 5;
  for (int i = threadIdx.x; i < words; i += kTokThreads) extra[i] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += kTokThreads) {
    if (KEY(i) == kth) {
      const uint32_t p = POS(i);
      atomicOr(&extra[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  const int per = (words + kTokThreads - 1) / kTokThreads;
  const int w0 = min(words, (int)threadIdx.x * per), w1 = min(words, w0 + per);
  {
    uint32_t cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(extra[i]);
    uint32_t total;
    uint32_t before = block_excl_scan<kTokThreads>(cnt, scratch, &total);
    for (int i = w0; i < w1; ++i) {
      uint32_t bits = extra[i];
      const uint32_t pc = __popc(bits);
      if (before >= ties_kept) {
        bits = 0;
      } else if (before + pc > ties_kept) {
        const uint32_t keep = ties_kept - before;
        uint32_t nb = 0;
        for (uint32_t kept = 0; kept < keep; ++kept) {
          const uint32_t low = bits & (0u - bits);
          nb |= low;
          bits ^= low;
        }
        bits = nb;
      }
      before += pc;
      extra[i] = bits;
    }
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += kTokThreads) {
    if (KEY(i) > kth) {
      const uint32_t p = POS(i);
      atomicOr(&extra[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  // 5. ordered compaction of sel | extra
  uint32_t cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(sel[i] | extra[i]);
  uint32_t total;
  uint32_t off = block_excl_scan<kTokThreads>(cnt, scratch, &total);
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = sel[i] | extra[i];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (off < (uint32_t)a.k) out[off] = (i << 5) + b;
      ++off;
    }
  }
  for (int i = (int)total + threadIdx.x; i < a.k; i += kTokThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_clear(uint32_t* p, int64_t words, hipStream_t s) {
  if (words <= 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  clear_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, words);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid((a.batch.max_len + kIndexerChunk - 1) / kIndexerChunk, a.num_tokens);
  topk_hist_kernel<<<grid, kHistThreads, 0, s>>>(a);
  return hipGetLastError();
}

int topk_token_lds_cap(int64_t words) {
  if (words > kMaxTokenWords) return 0;
  const int64_t fixed = (int64_t)(kHist1 + 32 + 2 * words) * (int64_t)sizeof(uint32_t);
  const int64_t cap = ((int64_t)kFinalizeLds - fixed) / (2 * (int64_t)sizeof(uint32_t));
  return cap > 0 ? (int)cap : 0;
}

hipError_t launch_topk_token(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_token_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFinalizeLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t lds = (size_t)(kHist1 + 32 + 2 * a.words + 2 * (int64_t)a.lds_cand_cap) * sizeof(uint32_t);
  topk_token_kernel<<<a.num_tokens, kTokThreads, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_cut(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  topk_cut_kernel<<<a.num_tokens, kCutThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid((a.batch.max_len + kSelectChunk - 1) / kSelectChunk, a.num_tokens);
  topk_select_kernel<<<grid, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

int topk_finalize_lds_cap(int64_t words) {
  const int64_t fixed = (int64_t)(kHist2 + kHist3 + 32 + 2 * words) * (int64_t)sizeof(uint32_t);
  const int64_t cap = ((int64_t)kFinalizeLds - fixed) / (2 * (int64_t)sizeof(uint32_t));
  return cap > 0 ? (int)cap : 0;
}

hipError_t launch_topk_finalize(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_finalize_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFinalizeLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t lds =
      (size_t)(kHist2 + kHist3 + 32 + 2 * a.words + 2 * (int64_t)a.lds_cand_cap) * sizeof(uint32_t);
  topk_finalize_kernel<<<a.num_tokens, kFinThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
