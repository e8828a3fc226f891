// Per-token top-k over indexer scores: keep the min(k, n) best positions,
// ties to the lower position, written in ascending order and -1 padded.
// Sources: A.X K2 fact sheet (archdb), token-selection fact: top-2048
// positions per query. rebasdaily article, section on long tasks that cannot
// re-read all old content: at most 2,048 positions per query.
//
// Exact radix select on order-preserving uint32 keys, in three stages:
//   1. digit-1 histogram: the top 11 key bits of every score, built from the
//      indexer epilogue (fused path) or by topk_hist_kernel.
//   2. topk_select_kernel (many workgroups per token): each workgroup first
//      reads the token's histogram and finds digit1, the top-11-bit value of
//      the k-th largest score. No cross-workgroup hand-off or device-scope
//      fence is needed. Positions whose digit is above digit1 go straight
//      into a selection bitmap; one ballot gives 64 positions. Positions whose
//      digit equals digit1 are appended to a candidate list.
//   3. topk_finalize_kernel (one workgroup per token): two more radix levels
//      (11 and 10 bits) over the candidates find the exact k-th key. Ties at
//      that key are kept lowest position first, using a prefix count over a
//      tie bitmap. An ordered compaction of the bitmaps then writes the kept
//      positions in ascending order.
// Every decision depends only on the score values, so the result is exact.
#include "sga_block.h"
#include "sga_kernels.h"

namespace sga {
namespace {

constexpr int kHistThreads = 256;
constexpr int kSelThreads = 256;
constexpr int kFinThreads = 1024;

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

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ uint32_t stage[kSelectChunk];   // also holds the histogram for the cut
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t stage_count;
  __shared__ uint32_t stage_base;
  const int t = blockIdx.y;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  if (n <= a.k) return;  // every visible position is kept; finalize writes them
  const int c0 = blockIdx.x * kSelectChunk;
  if (c0 >= n) return;
  const int c1 = min(n, c0 + kSelectChunk);
  // first radix cut, taken redundantly by every workgroup of the token
  uint32_t d1, above1;
  hist1_cut<kSelThreads>(a.hist + (int64_t)t * kHist1, stage, (uint32_t)a.k, scratch, d1, above1);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.ctrl[t].digit1 = d1;
    a.ctrl[t].above1 = above1;
  }
  if (threadIdx.x == 0) stage_count = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* srow = a.scores + (int64_t)t * a.ld;
  uint32_t* sel = a.sel + (int64_t)t * a.words;
  // each wave takes 64 consecutive positions per step
  for (int p0 = c0 + wave * 64; p0 < c1; p0 += kSelThreads) {
    const int p = p0 + lane;
    uint32_t dig = 0;
    bool valid = p < c1;
    if (valid) dig = score_key(srow[p]) >> (32 - kDigit1Bits);
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
        stage[off + rank] = (uint32_t)p;
      }
    }
  }
  __syncthreads();
  const uint32_t cnt = stage_count;
  if (cnt == 0) return;
  if (threadIdx.x == 0) stage_base = atomicAdd(&a.ctrl[t].cand_count, cnt);
  __syncthreads();
  uint32_t* cand = a.cand + (int64_t)t * a.cand_cap;
  for (uint32_t i = threadIdx.x; i < cnt; i += kSelThreads) cand[stage_base + i] = stage[i];
}

// Dynamic LDS: tie/extra bitmap (words) + digit histogram (2048) + scratch.
__global__ __launch_bounds__(kFinThreads) void topk_finalize_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* hist = lds;                      // kHist1 words
  uint32_t* scratch = lds + kHist1;          // 32 words
  uint32_t* extra = lds + kHist1 + 32;       // a.words words
  const int t = blockIdx.x;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  int32_t* out = a.indices + (int64_t)t * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kFinThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* srow = a.scores + (int64_t)t * a.ld;
  const uint32_t* cand = a.cand + (int64_t)t * a.cand_cap;
  const uint32_t m = a.ctrl[t].cand_count;
  const uint32_t d1 = a.ctrl[t].digit1;
  const uint32_t r1 = (uint32_t)a.k - a.ctrl[t].above1;  // still needed, 1 <= r1 <= m
  uint32_t* res = scratch + 24;

  // level 2: key bits 20..10 of the candidates
  for (int b = threadIdx.x; b < kHist1; b += kFinThreads) hist[b] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += kFinThreads) {
    uint32_t key = score_key(srow[cand[i]]);
    atomicAdd(&hist[(key >> 10) & 0x7FFu], 1u);
  }
  __syncthreads();
  block_find_cut<kFinThreads>(hist, 2048, r1, scratch, res);
  const uint32_t d2 = res[0];
  const uint32_t r2 = r1 - res[1];
  __syncthreads();

  // level 3: key bits 9..0 of the candidates that match digit 2
  for (int b = threadIdx.x; b < 1024; b += kFinThreads) hist[b] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += kFinThreads) {
    uint32_t key = score_key(srow[cand[i]]);
    if (((key >> 10) & 0x7FFu) == d2) atomicAdd(&hist[key & 0x3FFu], 1u);
  }
  __syncthreads();
  block_find_cut<kFinThreads>(hist, 1024, r2, scratch, res);
  const uint32_t d3 = res[0];
  const uint32_t ties_kept = r2 - res[1];  // positions with key == kth to keep
  const uint32_t kth = (d1 << 21) | (d2 << 10) | d3;
  __syncthreads();

  // ties: mark every position whose key equals the k-th key
  const int words = (n + 31) >> 5;
  for (int i = threadIdx.x; i < words; i += kFinThreads) extra[i] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < m; i += kFinThreads) {
    uint32_t p = cand[i];
    if (score_key(srow[p]) == kth) atomicOr(&extra[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  // keep the ties_kept lowest-position ties: thread j owns a contiguous run of words
  const int per = (words + kFinThreads - 1) / kFinThreads;
  const int w0 = min(words, (int)threadIdx.x * per), w1 = min(words, w0 + per);
  {
    uint32_t c = 0;
    for (int i = w0; i < w1; ++i) c += __popc(extra[i]);
    uint32_t total;
    uint32_t before = block_excl_scan<kFinThreads>(c, scratch, &total);
    for (int i = w0; i < w1; ++i) {
      uint32_t bits = extra[i];
      uint32_t pc = __popc(bits);
      if (before >= ties_kept) {
        bits = 0;
      } else if (before + pc > ties_kept) {
        uint32_t keep = ties_kept - before;  // keep the lowest `keep` set bits
        uint32_t kept = 0, nb = 0;
        while (kept < keep) {
          uint32_t low = bits & (0u - bits);
          nb |= low;
          bits ^= low;
          ++kept;
        }
        bits = nb;
      }
      before += pc;
      extra[i] = bits;
    }
  }
  __syncthreads();
  // candidates strictly above the k-th key
  for (uint32_t i = threadIdx.x; i < m; i += kFinThreads) {
    uint32_t p = cand[i];
    if (score_key(srow[p]) > kth) atomicOr(&extra[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  // ordered compaction of sel | extra
  const uint32_t* sel = a.sel + (int64_t)t * a.words;
  uint32_t c = 0;
  for (int i = w0; i < w1; ++i) c += __popc(sel[i] | extra[i]);
  uint32_t total;
  uint32_t off = block_excl_scan<kFinThreads>(c, scratch, &total);
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = sel[i] | extra[i];
    while (bits) {
      int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (off < (uint32_t)a.k) out[off] = (i << 5) + b;
      ++off;
    }
  }
  for (int i = (int)total + threadIdx.x; i < a.k; i += kFinThreads) out[i] = -1;
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

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid((a.batch.max_len + kSelectChunk - 1) / kSelectChunk, a.num_tokens);
  topk_select_kernel<<<grid, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

size_t topk_finalize_lds_bytes(int64_t words) {
  return (size_t)(kHist1 + 32 + words) * sizeof(uint32_t);
}

hipError_t launch_topk_finalize(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  size_t lds = topk_finalize_lds_bytes(a.words);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_finalize_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  topk_finalize_kernel<<<a.num_tokens, kFinThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
