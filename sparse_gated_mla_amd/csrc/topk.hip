// Per-token top-k over indexer scores: keep the min(k, n) best positions,
// ties to the lower position, written in ascending order and -1 padded.
// Sources: A.X K2 fact sheet (archdb), token-selection fact: top-2048
// positions per query. rebasdaily article, section on long tasks that cannot
// re-read all old content: at most 2,048 positions per query.
//
// Exact radix select on order-preserving uint32 keys. For batches of many
// tokens (contexts up to 256K), topk_token_kernel does stages 2-3 below in
// one workgroup per token; otherwise they run as two kernels. The stages:
//   1. digit-1 histogram: the top 12 key bits of every score, built in the
//      indexer epilogue (fused path) or by topk_hist_kernel.
//   2. topk_select_kernel (one workgroup per 4096 positions of a token):
//      every workgroup first finds digit1, the top-12-bit value of the k-th
//      largest score, from the histogram (the kernel boundary orders it after
//      every histogram update, so no cross-workgroup hand-off or device-scope
//      fence is needed). Positions whose digit is above digit1 go straight
//      into a selection bitmap; one ballot gives 64 positions. Positions whose
//      digit equals digit1 are written, with their keys, to the workgroup's
//      own slice of the candidate list, the workgroup records how many, and
//      their next 12 key bits are counted into the token's digit-2 histogram.
//   3. topk_finalize_kernel (one workgroup per token): the digit-2 cut from
//      that histogram, then the last 8 bits, over the candidates (staged in LDS
//      when they fit) that share both digits, find the exact k-th key: a wave
//      ranks them directly when they are few, else an 8-bit histogram does.
//      One ordered pass over the selection and tie bitmaps then writes the kept
//      positions in ascending order, ties at the k-th key lowest position first.
// Every decision depends only on the score values, so the result is exact.
#include "sga_block.h"
#include "sga_finalize.h"
#include "sga_kernels.h"

SGA_TL_RECORD(topk)

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
  __shared__ __attribute__((aligned(16))) uint32_t lds_hist[kHist1];
  __shared__ uint32_t scan_scratch[kHistThreads / 64];
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
  if (a.hist_slot_words) {
    if (blockIdx.x == 0) hist2_zero<kHistThreads>(a.hist2 + (int64_t)t * kHist2, threadIdx.x);
    hist1_list_store<kHistThreads>(lds_hist, a.hist + (int64_t)t * kHist1 + (int64_t)blockIdx.x * a.hist_slot_words,
                                   a.hist_slot_words, blockIdx.x, scan_scratch);
  } else {
    hist1_flush<kHistThreads>(lds_hist, a.hist + (int64_t)t * kHist1);
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs a) {
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t lds_count;
  __shared__ __attribute__((aligned(16))) uint32_t lds_h1[kHist1];   // list slots summed
  __shared__ uint32_t lds_ovf[kMaxHistSlots / 32];
  constexpr int kSteps = kSelectChunk / kSelThreads;   // 64-position steps per wave
  const int t = blockIdx.y;
  SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 0);
  SGA_TL_ID(blockIdx.y * gridDim.x + blockIdx.x);
  const int c0 = blockIdx.x * kSelectChunk;   // < max_len: the grid covers max_len
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* srow = a.scores + (int64_t)t * a.ld;
  // the histogram first, then every score load of this workgroup, before the
  // batch metadata (scalar loads): the cut is taken while the scores are still
  // in flight. Scores past the token's visible rows (below max_len, inside the
  // row) are read and then masked.
  HistRun<kSelThreads, kHist1> h1;
  h1.load(a.hist + (int64_t)t * kHist1);   // the dense histogram, or the region of list slots
  const rsrc_t srs = make_rsrc(srow + c0, (uint32_t)(min(a.batch.max_len, c0 + kSelectChunk) - c0) * 4u);
  float v[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
    v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, (i * kSelThreads + wave * 64 + lane) * 4, 0, 0));
  const int hsw = a.hist_slot_words;
  if (hsw) {
    // list slots: their entries are summed into an LDS histogram first
#pragma unroll
    for (int q = 0; q < kHist1 / (4 * kSelThreads); ++q)
      reinterpret_cast<u32x4*>(lds_h1)[q * kSelThreads + threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
    lds_ovf[threadIdx.x % (kMaxHistSlots / 32)] = 0u;   // no branch on the thread index here
  }
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  if (blockIdx.x == 0 && threadIdx.x == 0) a.ctrl[t].visible = (uint32_t)n;
  if (n <= a.k) return;  // every visible position is kept; finalize writes them
  if (c0 >= n) return;
  const int c1 = min(n, c0 + kSelectChunk);
  if (hsw) {
    __syncthreads();
    const int hc = a.hist_chunk;
    const int slots = (a.batch.max_len + hc - 1) / hc;
    SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 2);
    h1.add_lists(hsw, slots, lds_h1, lds_ovf);
    __syncthreads();
    SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 3);
    // a chunk whose bins did not fit its slot is counted from its scores
    // (positions [c * hc, min(n, (c + 1) * hc)), all written by the indexer)
    uint32_t ovf[kMaxHistSlots / 32];
#pragma unroll
    for (int wd = 0; wd < kMaxHistSlots / 32; ++wd) ovf[wd] = lds_ovf[wd];
    if (ovf[0] | ovf[1] | ovf[2] | ovf[3]) {
      for (int wd = 0; wd < kMaxHistSlots / 32; ++wd) {
        uint32_t bits = ovf[wd];
        while (bits) {
          const int c = 32 * wd + __ffs(bits) - 1;
          bits &= bits - 1u;
          const int p1 = min(n, (c + 1) * hc);
          for (int p = c * hc + (int)threadIdx.x; p < p1; p += kSelThreads)
            atomicAdd(&lds_h1[score_key(srow[p]) >> (32 - kDigit1Bits)], 1u);
        }
      }
      __syncthreads();
    }
    h1.load_lds(lds_h1);
  }
  if (threadIdx.x == 0) lds_count = 0;
  // first radix cut, taken redundantly by every workgroup of the token from the
  // histogram the previous kernel completed (no cross-workgroup hand-off)
  uint32_t d1, above1, n1;
  h1.cut((uint32_t)a.k, scratch, d1, above1, n1);
  SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 4);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.ctrl[t].digit1 = d1;
    a.ctrl[t].above1 = above1;
  }
  // classify: bitmap words for the digits above the cut, candidate masks kept
  uint32_t* sel = a.sel + (int64_t)t * a.words;
  uint64_t cmask[kSteps];
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int p0 = c0 + i * kSelThreads + wave * 64;
    const int p = p0 + lane;
    const bool valid = p < c1;
    const uint32_t dig = score_key(v[i]) >> (32 - kDigit1Bits);
    const uint64_t above = __ballot(valid && dig > d1);
    cmask[i] = __ballot(valid && dig == d1);
    total += (uint32_t)__popcll(cmask[i]);
    if (lane == 0 && p0 < c1) {
      sel[p0 >> 5] = (uint32_t)above;
      sel[(p0 >> 5) + 1] = (uint32_t)(above >> 32);
    }
  }
  // one LDS atomic per wave reserves its run of the workgroup's candidate slice
  uint32_t off = 0;
  if (lane == 0 && total) off = atomicAdd(&lds_count, total);
  off = __shfl(off, 0);
  uint32_t* gpos = a.cand + (int64_t)t * a.cand_cap + c0;
  uint32_t* gkey = a.cand_key + (int64_t)t * a.cand_cap + c0;
  const uint64_t lower = (1ull << lane) - 1ull;
  uint32_t* h2 = a.hist2 + (int64_t)t * kHist2;   // level 2 of the cut, counted here
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    if ((cmask[i] >> lane) & 1ull) {
      const uint32_t j = off + (uint32_t)__popcll(cmask[i] & lower);
      const uint32_t key = score_key(v[i]);
      gpos[j] = (uint32_t)(c0 + i * kSelThreads + wave * 64 + lane);
      gkey[j] = key;
      atomicAdd(h2 + ((key >> kDigit3Bits) & (kHist2 - 1)), 1u);
    }
    off += (uint32_t)__popcll(cmask[i]);
  }
  SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 5);
  __syncthreads();
  if (threadIdx.x == 0) a.wg_count[(int64_t)t * a.max_select_wgs + blockIdx.x] = lds_count;
  SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 1);
}

// The final stage (sga_finalize.h) for one window of ranks of one token:
// workgroup (g, t) writes ranks [g * W, min(k, (g + 1) * W)) of token t's
// selection (W = a.fin_window), staged in LDS for coalesced stores when the
// window holds at most 4,096 ranks. Several workgroups per token each run the
// stage's cut and counting and hand out only their own ranks, so the ordered
// pass over a long context is spread over them.
// Dynamic LDS: staged output (4096 words) | the stage's finalize_lds_words.
__global__ __launch_bounds__(kFinThreads) void topk_finalize_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* out_stage = lds;
  const int t = blockIdx.y;
  const uint32_t lo = (uint32_t)blockIdx.x * (uint32_t)a.fin_window;
  const uint32_t hi = min((uint32_t)a.k, lo + (uint32_t)a.fin_window);
  TokenFinalize<kFinThreads> fin;
  fin.prefetch(a, t);
  const int n = fin.visible();   // recorded by the select kernel
  int32_t* out = a.indices + (int64_t)t * a.k;
  if (n <= a.k) {
    for (int i = (int)lo + threadIdx.x; i < (int)hi; i += kFinThreads) out[i] = i < n ? i : -1;
    return;
  }
  int32_t* staged_out = reinterpret_cast<int32_t*>(out_stage);   // the window goes out coalesced
  const bool stage_out = hi - lo <= (uint32_t)kHist2;
  fin.run(a, n, out_stage + kHist2, lo, hi, [&](uint32_t o, uint32_t p) {
    if (stage_out) staged_out[o - lo] = (int32_t)p;
    else out[o] = (int32_t)p;
  });
  if (stage_out) {
    __syncthreads();
    for (int i = (int)lo + threadIdx.x; i < (int)hi; i += kFinThreads) out[i] = staged_out[i - lo];
  }
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
constexpr int kTokenHalfLdsMinCand = 2048;   // staged candidates that justify half the LDS
static_assert(kHist1 == kHist2, "one LDS histogram serves both levels");

__global__ __launch_bounds__(kTokThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void topk_token_kernel(TopkArgs a) {
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

  // 2. one pass over the scores: 64-position groups in batches of kTokUnroll
  // per lane; the next batch's loads are in flight while a batch is
  // classified
  const int ngroups = (n + 63) >> 6;
  constexpr int kBatch = kTokWaves * kTokUnroll;   // groups per batch
  // buffer loads: positions past n read zeros (and are masked below), and no
  // 64-bit address is formed per load
  const rsrc_t srs = make_rsrc(srow, (uint32_t)n * 4u);
  auto load_batch = [&](int gb, float (&v)[kTokUnroll]) {
#pragma unroll
    for (int u = 0; u < kTokUnroll; ++u)
      v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          srs, (((gb + u * kTokWaves + wave) << 6) + lane) * 4, 0, 0));
  };
  auto classify = [&](int gb, const float (&v)[kTokUnroll]) {
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
  };
  {
    float va[kTokUnroll], vb[kTokUnroll];
    load_batch(0, va);
    for (int gb = 0; gb < ngroups; gb += 2 * kBatch) {
      if (gb + kBatch < ngroups) load_batch(gb + kBatch, vb);
      classify(gb, va);
      if (gb + kBatch >= ngroups) break;
      if (gb + 2 * kBatch < ngroups) load_batch(gb + 2 * kBatch, va);
      classify(gb + kBatch, vb);
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

int topk_hist_slot_words(int max_len) {
  return hist_slot_words(((int64_t)max_len + kIndexerChunk - 1) / kIndexerChunk);
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
  // two workgroups per CU when half the LDS still stages a few thousand
  // candidates (at 128K about 4,000; more spill to the workspace), else one
  // workgroup with all of it
  const int64_t half = ((int64_t)kFinalizeLds / 2 - fixed) / (2 * (int64_t)sizeof(uint32_t));
  if (half >= kTokenHalfLdsMinCand) return (int)half;
  const int64_t cap = ((int64_t)kFinalizeLds - fixed) / (2 * (int64_t)sizeof(uint32_t));
  return cap > 0 ? (int)cap : 0;
}

hipError_t launch_topk_token(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)topk_token_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFinalizeLds);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)(kHist1 + 32 + 2 * a.words + 2 * (int64_t)a.lds_cand_cap) * sizeof(uint32_t);
  topk_token_kernel<<<a.num_tokens, kTokThreads, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid((a.batch.max_len + kSelectChunk - 1) / kSelectChunk, a.num_tokens);
  topk_select_kernel<<<grid, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_finalize(const TopkArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)topk_finalize_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFinalizeLds);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)(kHist2 + finalize_lds_words(a.words)) * sizeof(uint32_t);
  if (lds > kFinalizeLds) return hipErrorInvalidValue;
  if (a.fin_window < 1) return hipErrorInvalidValue;
  const unsigned windows = (unsigned)((a.k + a.fin_window - 1) / a.fin_window);
  topk_finalize_kernel<<<dim3(windows, a.num_tokens), kFinThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
