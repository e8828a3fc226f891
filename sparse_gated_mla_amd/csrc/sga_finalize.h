// Final stage of the exact per-token top-k, shared by the stand-alone
// finalize kernel (one 1,024-thread workgroup per token) and the attention
// kernel that selects its own rows (one 512-thread workgroup per split of a
// token, each running the whole stage for its token).
// Sources: A.X K2 fact sheet (archdb), token-selection fact: top-2048
// positions per query. rebasdaily article, section on long tasks that cannot
// re-read all old content: at most 2,048 positions per query.
//
// Input (from the select kernel): the digit-1 cut d1 and the count above it,
// a selection bitmap of the positions whose top 12 key bits exceed d1, the
// digit-2 histogram of the candidates (top 12 bits equal to d1), and the
// candidates themselves, slice x holding those of bitmap chunk x (positions
// [x * 4096, (x + 1) * 4096)).
// The stage: the digit-2 cut from the histogram, then the last 8 bits, over
// the candidates that share both digits, give the exact k-th key; candidates
// above it join the selection, and ties at it are admitted lowest position
// first; one ordered pass over the bitmaps then hands every kept position,
// with its rank in ascending position order, to an emit callback. Every
// decision is an integer comparison of keys, so the result is exact.
#pragma once
#include "sga_block.h"
#include "sga_kernels.h"

namespace sga {

// LDS words the stage needs for a bitmap of `words` words: level-3 histogram
// or short key list (256) | scratch (64) | per-chunk selected and tie counts
// (2 * kMaxSelectWgs) | tie bitmap (words) | selection bitmap (words).
__host__ __device__ constexpr int64_t finalize_lds_words(int64_t words) {
  return kHist3 + 64 + 2 * kMaxSelectWgs + 2 * words;
}

template <int NT>
struct TokenFinalize {
  static constexpr int kWaves = NT / 64;
  static constexpr int kPreSlices = 4;                // candidate slices per wave held in registers
  static constexpr int kChunkWords = kSelectChunk / 32;   // bitmap words of one select chunk
  static_assert(kChunkWords == 128 && kMaxSelectWgs <= 128, "two words and two chunks per lane");
  static_assert(kWaves * 2 + 3 <= 40, "scratch words below the short-list slots");

  static constexpr int kPreWords = (8192 + NT - 1) / NT;   // bitmap words per thread in one round (256K)
  uint32_t ctrl_word;
  HistRun<NT, kHist2> h2;
  uint32_t w[kPreWords];
  uint32_t clen[kPreSlices], cpos[kPreSlices][2], ckey[kPreSlices][2];
  const uint32_t* sel;
  const uint32_t* gpos;
  const uint32_t* gkey;
  const uint32_t* wgc;
  int wv;

  // One round of loads that needs no batch metadata: the control block (the
  // cut and the token's visible count, recorded by the select kernel), the
  // digit-2 histogram, the first kPreWords * NT words of the selection bitmap
  // and, for wave w, the lengths of candidate slices w + q * kWaves
  // (q < kPreSlices) with their first 128 entries. All lie inside this
  // token's workspace rows; entries past the token's own are loaded and not
  // used. (The control block is a per-lane vector load, lane i reading word
  // i & 3: a uniform scalar load would be sunk past later branches.)
  __device__ __forceinline__ void prefetch(const TopkArgs& a, int t) {
    static_assert(sizeof(TopkCtrl) == 16 && offsetof(TopkCtrl, digit1) == 0 &&
                      offsetof(TopkCtrl, above1) == 4 && offsetof(TopkCtrl, visible) == 8,
                  "the control block's words");
    const int lane = threadIdx.x & 63;
    ctrl_word = reinterpret_cast<const uint32_t*>(a.ctrl + t)[threadIdx.x & 3];
    h2.load(a.hist2 + (int64_t)t * kHist2);
    sel = a.sel + (int64_t)t * a.words;
#pragma unroll
    for (int u = 0; u < kPreWords; ++u) w[u] = sel[min(u * NT + (int)threadIdx.x, (int)a.words - 1)];
    gpos = a.cand + (int64_t)t * a.cand_cap;
    gkey = a.cand_key + (int64_t)t * a.cand_cap;
    wgc = a.wg_count + (int64_t)t * a.max_select_wgs;
    // the wave index as a uniform value: branches on it stay scalar and leave
    // t uniform (a divergent branch here would turn the metadata loads into
    // vector loads)
    wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
#pragma unroll
    for (int q = 0; q < kPreSlices; ++q) {
      const int x = wv + q * kWaves;
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
  }

  // The token's visible positions, as the select kernel recorded them.
  __device__ __forceinline__ int visible() const { return (int)__builtin_amdgcn_readlane(ctrl_word, 2); }

  // For a token with n > k visible positions: calls emit(rank, position) for
  // every kept position (exactly k of them), ranks in ascending position
  // order; only ranks in [lo, hi) are handed over (the rest are skipped
  // cheaply where a whole word or chunk lies outside). lds: finalize_lds_words
  // words. All threads of the workgroup must call.
  template <class Emit>
  __device__ __forceinline__ void run(const TopkArgs& a, int n, uint32_t* lds, uint32_t lo, uint32_t hi,
                                      Emit&& emit) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t* hist3 = lds;
    uint32_t* scratch = hist3 + kHist3;
    uint32_t* chunk_cnt = scratch + 64;
    uint32_t* tie = chunk_cnt + 2 * kMaxSelectWgs;
    uint32_t* selL = tie + a.words;
    uint32_t* n_few = scratch + 40;   // short-list length, then the k-th key and ties kept
    const int nsel = (n + kSelectChunk - 1) / kSelectChunk;
    const int words = (n + 31) >> 5;
    const uint32_t d1 = __builtin_amdgcn_readlane(ctrl_word, 0);
    const uint32_t r1 = (uint32_t)a.k - __builtin_amdgcn_readlane(ctrl_word, 1);  // still needed from the candidates
    for (int i0 = 0; i0 < words; i0 += kPreWords * NT) {
      if (i0 > 0) {
#pragma unroll
        for (int u = 0; u < kPreWords; ++u) w[u] = sel[min(i0 + u * NT + (int)threadIdx.x, words - 1)];
      }
#pragma unroll
      for (int u = 0; u < kPreWords; ++u) {
        const int i = i0 + u * NT + threadIdx.x;
        if (i < words) {
          selL[i] = w[u];
          tie[i] = 0;
        }
      }
    }
    for (int b = threadIdx.x; b < kHist3; b += NT) hist3[b] = 0;
    if (threadIdx.x == 0) *n_few = 0;
    // level 2, from the histogram the select kernel counted (the cut's barriers
    // also publish the LDS stores above)
    uint32_t d2, above2, n3;   // n3: candidates with digit d2, usually a handful
    h2.cut(r1, scratch, d2, above2, n3);
    const uint32_t r2 = r1 - above2;

    // Calls f(position, key) for every candidate of this wave's slices x = wave,
    // wave + kWaves, ...: the first 128 entries of the first kPreSlices from
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
        const int x = wv + q * kWaves;
        if (x < nsel) {
          const uint32_t len = clen[q];
          if ((uint32_t)lane < len) f(cpos[q][0], ckey[q][0]);
          if ((uint32_t)lane + 64 < len) f(cpos[q][1], ckey[q][1]);
          from_global(x, 128, len);
        }
      }
      for (int x = wv + kPreSlices * kWaves; x < nsel; x += kWaves) from_global(x, 0, wgc[x]);
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
      block_cut<NT>(hist3, kHist3, r2, scratch, d3, above3);
      ties_kept = r2 - above3;
      kth = (d1 << (32 - kDigit1Bits)) | (d2 << kDigit3Bits) | d3;
    }

    // Candidates above the k-th key join the selection; ties at it are marked
    // apart. Slice x holds the candidates of bitmap chunk x (kChunkWords words,
    // positions [x * kSelectChunk, (x + 1) * kSelectChunk)), so wave x mod
    // kWaves marks only inside its own chunks.
    each_candidate([&](uint32_t p, uint32_t key) {
      if (key >= kth) atomicOr(key > kth ? &selL[p >> 5] : &tie[p >> 5], 1u << (p & 31));
    });
    // Keeps the selected positions of word i and its ties while fewer than
    // ties_kept lower ties were kept; o is the rank of the word's first kept
    // position, ties_seen the ties before it.
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
      const uint32_t cnt = __popc(bits);
      if (o < hi && o + cnt > lo) {
        while (bits) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          if (o >= lo && o < hi && o < (uint32_t)a.k) emit(o, (uint32_t)((i << 5) + b));
          ++o;
        }
      } else {
        o += cnt;
      }
    };
    if (nsel >= kWaves) {
      // Long contexts: the wave that marked a chunk also counts and emits it,
      // with no barrier in between (a wave's LDS operations complete in order);
      // lane l holds words 2l and 2l + 1 of the chunk. One barrier publishes
      // the chunk counts.
      auto chunk_words = [&](int x, uint32_t (&sw)[2], uint32_t (&tw)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = x * kChunkWords + 2 * lane + u;
          sw[u] = i < words ? selL[i] : 0u;
          tw[u] = i < words ? tie[i] : 0u;
        }
      };
      for (int x = wv; x < nsel; x += kWaves) {
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
      for (int x = wv; x < nsel; x += kWaves) {
        const int L = x >> 1;
        uint32_t s_before = __builtin_amdgcn_readlane(cs_excl, L);
        uint32_t t_before = __builtin_amdgcn_readlane(ct_excl, L);
        if (x & 1) {
          s_before += __builtin_amdgcn_readlane(cs0, L);
          t_before += __builtin_amdgcn_readlane(ct0, L);
        }
        // the chunk's ranks start at s_before + min(t_before, ties_kept) and
        // hold at most its selected count plus its admitted ties
        const uint32_t first_rank = s_before + min(t_before, ties_kept);
        const uint32_t cs_x = __builtin_amdgcn_readlane((x & 1) ? cs1 : cs0, L);
        const uint32_t ct_x = __builtin_amdgcn_readlane((x & 1) ? ct1 : ct0, L);
        if (first_rank >= hi || first_rank + cs_x + ct_x <= lo) continue;   // uniform: no rank of ours
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
      // words, and a block scan gives each run its rank.
      __syncthreads();
      const int per = (words + NT - 1) / NT;
      const int w0 = min(words, (int)threadIdx.x * per), w1 = min(words, w0 + per);
      uint32_t ns = 0, nt = 0;
      for (int i = w0; i < w1; ++i) {
        ns += __popc(selL[i]);
        nt += __popc(tie[i]);
      }
      uint32_t s_before, t_before;
      block_excl_scan2<NT>(ns, nt, scratch, s_before, t_before);
      uint32_t o = s_before + min(t_before, ties_kept);
      uint32_t ties_seen = t_before;
      for (int i = w0; i < w1; ++i) emit_word(i, selL[i], tie[i], o, ties_seen);
    }
  }
};

}  // namespace sga
