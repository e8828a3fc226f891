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
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t lds_count;
  constexpr int kSteps = kSelectChunk / kSelThreads;   // 64-position steps per wave
  const int t = blockIdx.y;
  const int c0 = blockIdx.x * kSelectChunk;   // < max_len: the grid covers max_len
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* srow = a.scores + (int64_t)t * a.ld;
  // the histogram first, then every score load of this workgroup, before the
  // batch metadata (scalar loads): the cut is taken while the scores are still
  // in flight. Scores past the token's visible rows (below max_len, inside the
  // row) are read and then masked.
  HistRun<kSelThreads, kHist1> h1;
  h1.load(a.hist + (int64_t)t * kHist1);
  const rsrc_t srs = make_rsrc(srow + c0, (uint32_t)(min(a.batch.max_len, c0 + kSelectChunk) - c0) * 4u);
  float v[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
    v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, (i * kSelThreads + wave * 64 + lane) * 4, 0, 0));
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  if (n <= a.k) return;  // every visible position is kept; finalize writes them
  if (c0 >= n) return;
  const int c1 = min(n, c0 + kSelectChunk);
  if (threadIdx.x == 0) lds_count = 0;
  // first radix cut, taken redundantly by every workgroup of the token from the
  // histogram the previous kernel completed (no cross-workgroup hand-off)
  uint32_t d1, above1, n1;
  h1.cut((uint32_t)a.k, scratch, d1, above1, n1);
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
  __syncthreads();
  if (threadIdx.x == 0) a.wg_count[(int64_t)t * a.max_select_wgs + blockIdx.x] = lds_count;
}

// Dynamic LDS: staged output (4096 words) | level-3 histogram or short key
// list (256) | scratch (64) | per-chunk selected and tie counts
// (2 * kMaxSelectWgs) | tie bitmap (words) | selection bitmap (words).
__global__ __launch_bounds__(kFinThreads) void topk_finalize_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds[];
  constexpr int kFinWaves = kFinThreads / 64;
  constexpr int kPreSlices = 4;   // slices per wave held in registers: 256K positions
  constexpr int kChunkWords = kSelectChunk / 32;   // bitmap words of one select chunk
  static_assert(kChunkWords == 128 && kMaxSelectWgs <= 128, "two words and two chunks per lane");
  uint32_t* out_stage = lds;
  uint32_t* hist3 = out_stage + kHist2;
  uint32_t* scratch = hist3 + kHist3;
  uint32_t* chunk_cnt = scratch + 64;
  uint32_t* tie = chunk_cnt + 2 * kMaxSelectWgs;
  uint32_t* selL = tie + a.words;
  uint32_t* n_few = scratch + 40;   // short-list length, then the k-th key and ties kept
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // One round of loads, issued before the batch metadata (scalar loads): the
  // cut, the digit-2 histogram, the first 4 * kFinThreads words of the
  // selection bitmap and, for wave w, the lengths of candidate slices
  // w + q * kFinWaves (q < kPreSlices) with their first 128 entries. All lie
  // inside this token's workspace rows; entries past the token's own are
  // loaded and not used.
  // (The cut is a per-lane vector load, lanes 0 and 1 reading its two words:
  // a uniform scalar load would be sunk past the metadata's branch.)
  static_assert(offsetof(TopkCtrl, above1) == offsetof(TopkCtrl, digit1) + sizeof(uint32_t),
                "the cut's two words are adjacent");
  const uint32_t ctrl_word = (&a.ctrl[t].digit1)[threadIdx.x & 1];
  HistRun<kFinThreads, kHist2> h2;
  h2.load(a.hist2 + (int64_t)t * kHist2);
  const uint32_t* sel = a.sel + (int64_t)t * a.words;
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) w[u] = sel[min(u * kFinThreads + (int)threadIdx.x, (int)a.words - 1)];
  const uint32_t* gpos = a.cand + (int64_t)t * a.cand_cap;
  const uint32_t* gkey = a.cand_key + (int64_t)t * a.cand_cap;
  const uint32_t* wgc = a.wg_count + (int64_t)t * a.max_select_wgs;
  // the wave index as a uniform value: branches on it stay scalar and leave t
  // uniform (a divergent branch here would turn the metadata loads into
  // vector loads)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t clen[kPreSlices], cpos[kPreSlices][2], ckey[kPreSlices][2];
#pragma unroll
  for (int q = 0; q < kPreSlices; ++q) {
    const int x = wv + q * kFinWaves;
    clen[q] = 0;
    if (x < a.max_select_wgs) {
      const int64_t o = (int64_t)x * kSelectChunk + lane;
      clen[q] = wgc[x];
      cpos[q][0] = gpos[o];
      ckey[q][0] = gkey[o];
      cpos[q][1] = gpos[o + 64];
      ckey[q][1] = gkey[o + 64];
    }
  }
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  int32_t* out = a.indices + (int64_t)t * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kFinThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int nsel = (n + kSelectChunk - 1) / kSelectChunk;
  const int words = (n + 31) >> 5;
  const uint32_t d1 = __builtin_amdgcn_readlane(ctrl_word, 0);
  const uint32_t r1 = (uint32_t)a.k - __builtin_amdgcn_readlane(ctrl_word, 1);  // still needed from the candidates
  for (int i0 = 0; i0 < words; i0 += 4 * kFinThreads) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = sel[min(i0 + u * kFinThreads + (int)threadIdx.x, words - 1)];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kFinThreads + threadIdx.x;
      if (i < words) {
        selL[i] = w[u];
        tie[i] = 0;
      }
    }
  }
  for (int b = threadIdx.x; b < kHist3; b += kFinThreads) hist3[b] = 0;
  if (threadIdx.x == 0) *n_few = 0;
  // level 2, from the histogram the select kernel counted (the cut's barriers
  // also publish the LDS stores above)
  uint32_t d2, above2, n3;   // n3: candidates with digit d2, usually a handful
  h2.cut(r1, scratch, d2, above2, n3);
  const uint32_t r2 = r1 - above2;

  // Calls f(position, key) for every candidate of this wave's slices x = wave,
  // wave + kFinWaves, ...: the first 128 entries of the first kPreSlices from
  // registers, the rest from global memory, four per lane per round.
  auto each_candidate = [&](auto&& f) {
    auto from_global = [&](int x, uint32_t j0, uint32_t len) {
      const uint32_t* sp = gpos + (int64_t)x * kSelectChunk;
      const uint32_t* sk = gkey + (int64_t)x * kSelectChunk;
      for (; j0 < len; j0 += 256) {
        uint32_t pp[4], kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t j = min(j0 + 64 * u + lane, len - 1);
          pp[u] = sp[j];
          kk[u] = sk[j];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j0 + 64 * u + lane < len) f(pp[u], kk[u]);
      }
    };
#pragma unroll
    for (int q = 0; q < kPreSlices; ++q) {
      const int x = wv + q * kFinWaves;
      if (x < nsel) {
        const uint32_t len = clen[q];
        if ((uint32_t)lane < len) f(cpos[q][0], ckey[q][0]);
        if ((uint32_t)lane + 64 < len) f(cpos[q][1], ckey[q][1]);
        from_global(x, 128, len);
      }
    }
    for (int x = wv + kPreSlices * kFinWaves; x < nsel; x += kFinWaves) from_global(x, 0, wgc[x]);
  };

  // level 3: the keys with digit d2 into a short list (at most 64) or their
  // low 8 bits into a histogram
  each_candidate([&](uint32_t, uint32_t key) {
    if (((key >> kDigit3Bits) & (kHist2 - 1)) != d2) return;
    if (n3 <= 64) hist3[atomicAdd(n_few, 1u)] = key;
    else atomicAdd(&hist3[key & (kHist3 - 1)], 1u);
  });
  __syncthreads();
  uint32_t kth, ties_kept;   // the k-th key and how many positions holding it to keep
  if (n3 <= 64) {
    if (wave == 0) {
      // lane l holds key l; it counts the keys above it and those not below it
      const uint32_t mine = lane < (int)n3 ? hist3[lane] : 0u;
      uint32_t gt = 0, ge = 0;
      for (int j = 0; j < (int)n3; ++j) {
        const uint32_t other = __builtin_amdgcn_readlane(mine, j);
        gt += other > mine;
        ge += other >= mine;
      }
      if (lane < (int)n3 && gt < r2 && r2 <= ge) {   // the lanes holding the k-th key agree
        n_few[1] = mine;
        n_few[2] = r2 - gt;
      }
    }
    __syncthreads();
    kth = n_few[1];
    ties_kept = n_few[2];
  } else {
    uint32_t d3, above3;
    block_cut<kFinThreads>(hist3, kHist3, r2, scratch, d3, above3);
    ties_kept = r2 - above3;
    kth = (d1 << (32 - kDigit1Bits)) | (d2 << kDigit3Bits) | d3;
  }

  // Candidates above the k-th key join the selection; ties at it are marked
  // apart. Slice x holds the candidates of bitmap chunk x (kChunkWords words,
  // positions [x * kSelectChunk, (x + 1) * kSelectChunk)), so wave x mod
  // kFinWaves marks only inside its own chunks.
  each_candidate([&](uint32_t p, uint32_t key) {
    if (key >= kth) atomicOr(key > kth ? &selL[p >> 5] : &tie[p >> 5], 1u << (p & 31));
  });
  int32_t* staged_out = reinterpret_cast<int32_t*>(out_stage);   // k <= kHist2: the output goes out coalesced
  const bool stage_out = a.k <= kHist2;
  // Keeps the selected positions of word i and its ties while fewer than
  // ties_kept lower ties were kept; o is the output slot of the word's first
  // kept position, ties_seen the ties before it.
  auto emit_word = [&](int i, uint32_t sbits, uint32_t tbits_all, uint32_t& o, uint32_t& ties_seen) {
    uint32_t tbits = tbits_all;
    if (ties_seen >= ties_kept) {
      tbits = 0;
    } else if (ties_seen + __popc(tbits) > ties_kept) {
      uint32_t keep = ties_kept - ties_seen, nb = 0;   // the lowest `keep` ties of this word
      for (; keep; --keep) {
        const uint32_t low = tbits & (0u - tbits);
        nb |= low;
        tbits ^= low;
      }
      tbits = nb;
    }
    ties_seen += __popc(tbits_all);
    uint32_t bits = sbits | tbits;
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (o < (uint32_t)a.k) {
        if (stage_out) staged_out[o] = (i << 5) + b;
        else out[o] = (i << 5) + b;
      }
      ++o;
    }
  };
  if (nsel >= kFinWaves) {
    // Long contexts: the wave that marked a chunk also counts and emits it,
    // with no barrier in between (a wave's LDS operations complete in order);
    // lane l holds words 2l and 2l + 1 of the chunk. One barrier publishes the
    // chunk counts.
    auto chunk_words = [&](int x, uint32_t (&sw)[2], uint32_t (&tw)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = x * kChunkWords + 2 * lane + u;
        sw[u] = i < words ? selL[i] : 0u;
        tw[u] = i < words ? tie[i] : 0u;
      }
    };
    for (int x = wv; x < nsel; x += kFinWaves) {
      uint32_t sw[2], tw[2];
      chunk_words(x, sw, tw);
      const uint32_t ss = wave_incl_scan(__popc(sw[0]) + __popc(sw[1]));
      const uint32_t ts = wave_incl_scan(__popc(tw[0]) + __popc(tw[1]));
      if (lane == 63) {
        chunk_cnt[x] = ss;
        chunk_cnt[kMaxSelectWgs + x] = ts;
      }
    }
    __syncthreads();
    // the chunks' exclusive prefix sums, lane l holding chunks 2l and 2l + 1
    const uint32_t cs0 = 2 * lane < nsel ? chunk_cnt[2 * lane] : 0u;
    const uint32_t cs1 = 2 * lane + 1 < nsel ? chunk_cnt[2 * lane + 1] : 0u;
    const uint32_t ct0 = 2 * lane < nsel ? chunk_cnt[kMaxSelectWgs + 2 * lane] : 0u;
    const uint32_t ct1 = 2 * lane + 1 < nsel ? chunk_cnt[kMaxSelectWgs + 2 * lane + 1] : 0u;
    const uint32_t cs_excl = wave_incl_scan(cs0 + cs1) - (cs0 + cs1);
    const uint32_t ct_excl = wave_incl_scan(ct0 + ct1) - (ct0 + ct1);
    for (int x = wv; x < nsel; x += kFinWaves) {
      const int L = x >> 1;
      uint32_t s_before = __builtin_amdgcn_readlane(cs_excl, L);
      uint32_t t_before = __builtin_amdgcn_readlane(ct_excl, L);
      if (x & 1) {
        s_before += __builtin_amdgcn_readlane(cs0, L);
        t_before += __builtin_amdgcn_readlane(ct0, L);
      }
      uint32_t sw[2], tw[2];
      chunk_words(x, sw, tw);
      const uint32_t s2 = __popc(sw[0]) + __popc(sw[1]), t2 = __popc(tw[0]) + __popc(tw[1]);
      s_before += wave_incl_scan(s2) - s2;
      t_before += wave_incl_scan(t2) - t2;
      uint32_t o = s_before + min(t_before, ties_kept);
      uint32_t ties_seen = t_before;
#pragma unroll
      for (int u = 0; u < 2; ++u) emit_word(x * kChunkWords + 2 * lane + u, sw[u], tw[u], o, ties_seen);
    }
  } else {
    // Short contexts (fewer chunks than waves): every thread takes a run of
    // words, and a block scan gives each run its output slot.
    __syncthreads();
    const int per = (words + kFinThreads - 1) / kFinThreads;
    const int w0 = min(words, (int)threadIdx.x * per), w1 = min(words, w0 + per);
    uint32_t ns = 0, nt = 0;
    for (int i = w0; i < w1; ++i) {
      ns += __popc(selL[i]);
      nt += __popc(tie[i]);
    }
    uint32_t s_before, t_before;
    block_excl_scan2<kFinThreads>(ns, nt, scratch, s_before, t_before);
    uint32_t o = s_before + min(t_before, ties_kept);
    uint32_t ties_seen = t_before;
    for (int i = w0; i < w1; ++i) emit_word(i, selL[i], tie[i], o, ties_seen);
  }
  if (stage_out) {
    __syncthreads();
    for (int i = threadIdx.x; i < a.k; i += kFinThreads) out[i] = staged_out[i];
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
  const size_t lds = (size_t)(kHist2 + kHist3 + 64 + 2 * kMaxSelectWgs + 2 * a.words) * sizeof(uint32_t);
  if (lds > kFinalizeLds) return hipErrorInvalidValue;
  topk_finalize_kernel<<<a.num_tokens, kFinThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
