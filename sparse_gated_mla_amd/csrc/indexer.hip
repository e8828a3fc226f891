// Indexer kernel: I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]) over the
// visible positions s of token t (64 heads x 128; bf16 or fp8 keys).
// Source: A.X K2 fact sheet (archdb), token-selection fact: a DSA-style indexer
// of 64 ReLU-scored heads of width 128; cached indexer key width 128.
//
// Mapping onto gfx950:
// - Streaming. A workgroup streams indexer_chunk() positions of one token's key
//   cache (fewer for small batches, down to 128, so the grid fills the GPU);
//   its four waves take 32-position tiles in turn. Every load
//   instruction reads 1 KiB of contiguous keys (16 B per lane), so each wave
//   instruction covers whole cache lines. Each wave keeps two tiles of loads
//   in flight.
// - Re-layout. A wave writes its tile into a private 8 KiB LDS region. The
//   16-byte slots of each row are XOR-swizzled by row, so the 16 lanes of a
//   b128 write or read hit distinct banks. The wave then reads the tile back in
//   the operand layout of v_mfma_f32_32x32x16_bf16. No workgroup barrier is
//   needed: each wave owns its region, and its LDS operations complete in order.
// - Contraction.
//     A = query heads (M = 32 heads per block, two blocks), kept in registers;
//     B = keys (N = 32 positions, K = 16 dims per step, 8 steps).
//   The dims are visited in a permuted order, the same in A and B: lane group
//   g of step s covers dims 64g + 8s .. 64g + 8s + 7.
// - Epilogue, per lane: ReLU, times w, summed over the lane's 32 heads. One
//   cross-half shuffle then gives each position's score, which is kept in LDS
//   (and counted, see below) while the wave's next tiles are in flight. The
//   workgroup writes its chunk's scores in one contiguous run at the end.
// - fp8 and MX. Keys are widened to bf16 exactly on the LDS read. A per-row fp32
//   scale multiplies each head's dot product before the ReLU. An MX block-32
//   key (fact sheet, Training: MXFP8 with one scale per 32 consecutive
//   elements) has four E8M0 exponents per row; each is applied to its 32 dims
//   as they are widened by gfx950's scaled conversions (payload times a power
//   of two is exact in bf16), for E4M3FN or E2M1 (four-bit) payloads.
// - Fused top-k. The variant used by the whole forward pass also counts the
//   top 12 key bits of every score into a per-token histogram (the first radix
//   level of the top-k).
#include "sga_block.h"
#include "sga_kernels.h"

SGA_TL_RECORD(indexer)

namespace sga {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 32;
// key tiles in flight per wave: two (8 KiB for bf16 keys); three were 1.2 us
// slower on the ragged batch and 1 us on the 256K fp8 one, more slower still
constexpr int kStages = 2;

constexpr int kNonTemporal = 2;         // cache-policy bit: streaming (read-once) data

// A wave's key tile: 32 rows of one 128-row group of the chunk. The four
// waves share each group: load step s of wave w reads the 1 KiB block
// 4s + w of the group, so the four waves' loads of one step are adjacent and
// the workgroup streams through contiguous memory. Tile row r (the MFMA
// column) is group row (r / kRowsPerLoad) * 4 * kRowsPerLoad + w * kRowsPerLoad
// + r % kRowsPerLoad.
template <int kFmt>
struct KeyTile {
  static constexpr bool kFp8 = kFmt != kFmtBf16;   // a 32-bit scale word per row
  // A tile is kLoads loads of 1 KiB, kRowsPerLoad rows of kRowBytes each:
  //   bf16 (256 B rows): 8 loads of 4 rows; fp8 and MX8 (128 B): 4 loads of 8
  //   rows; MX4 (64 B): 2 loads of 16 rows. Load s, lane l -> tile row
  //   kRowsPerLoad*s + l/kChunksPerRow, 16-byte chunk l%kChunksPerRow. One-byte
  //   and four-bit tiles add the 32-bit scale word of tile row l%32 (the fp32
  //   row scale, or the four E8M0 block exponents).
  static constexpr int kRowBytes = row_bytes(kFmt, kIdxDim);
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kLoads = kTile * kRowBytes / 1024;
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
  static constexpr int kGroupRows = kWaves * kTile;
  u32x4 v[kLoads];
  uint32_t scale;

  // chunk position of tile row r of wave w in group grp
  static __device__ __forceinline__ int position(int grp, int w, int r) {
    return grp * kGroupRows + (r / kRowsPerLoad) * (kWaves * kRowsPerLoad) + w * kRowsPerLoad +
           r % kRowsPerLoad;
  }

  // Loads this wave's tile of group grp. Rows past the chunk read as zeros.
  __device__ __forceinline__ void load(rsrc_t keys, rsrc_t scales, int grp, int w, int lane) {
    const int off = grp * kGroupRows * kRowBytes + w * 1024 + lane * 16;
#pragma unroll
    for (int s = 0; s < kLoads; ++s)
      v[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(keys, off + s * kWaves * 1024, 0, kNonTemporal));
    if constexpr (kFp8)
      scale = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(scales, position(grp, w, lane & 31) * 4, 0, 0);
    // keep each tile's loads together and in program order, so the wait for
    // one tile never covers the loads of the tile issued after it
    __builtin_amdgcn_sched_barrier(0);
  }

  // swizzled 16-byte slot of chunk c in row r: the 16 rows that a b128 read
  // of one chunk meets in one pass land on 16 distinct 16-byte bank groups
  static __device__ __forceinline__ int slot(int r, int c) {
    return c ^ ((r / (16 / kChunksPerRow)) & (kChunksPerRow - 1));
  }

  __device__ __forceinline__ void store(uint8_t* lds, int lane) const {
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const int r = kRowsPerLoad * s + lane / kChunksPerRow;
      const int c = lane % kChunksPerRow;
      *reinterpret_cast<u32x4*>(lds + r * kRowBytes + 16 * slot(r, c)) = v[s];
    }
  }

  // B operands for the 8 k-steps: row n = lane%32, dims 64g + 8s .. +7 (g = lane/32).
  // sw: the row's scale word (MX: byte j is the exponent of dims 32j .. 32j+31).
  static __device__ __forceinline__ void operands(const uint8_t* lds, int lane, uint32_t sw,
                                                  u32x4 (&b)[8]) {
    const int n = lane & 31, g = lane >> 5;
    if constexpr (!kFp8) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        b[s] = *reinterpret_cast<const u32x4*>(lds + n * 256 + 16 * slot(n, 8 * g + s));
    } else if constexpr (kFmt == kFmtMx4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // chunk 2g + h holds dims 64g + 32h .. +31 (block 2g + h) = steps 4h .. 4h+3
        const u32x4 raw = *reinterpret_cast<const u32x4*>(lds + n * 64 + 16 * slot(n, 2 * g + h));
        const float bs = e8m0_to_f32((sw >> (8 * (2 * g + h))) & 0xFFu);
        b[4 * h] = e2m1x8_scaled_to_bf16x8(raw.x, bs);
        b[4 * h + 1] = e2m1x8_scaled_to_bf16x8(raw.y, bs);
        b[4 * h + 2] = e2m1x8_scaled_to_bf16x8(raw.z, bs);
        b[4 * h + 3] = e2m1x8_scaled_to_bf16x8(raw.w, bs);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // chunk 4g + s holds dims 64g + 16s .. +15 = steps 2s and 2s+1
        u32x4 raw = *reinterpret_cast<const u32x4*>(lds + n * 128 + 16 * slot(n, 4 * g + s));
        u32x2 a, bb, c, d;
        if constexpr (kFmt == kFmtMx) {
          // dims 64g + 16s .. +15 lie in block 2g + s/2
          const float bs = e8m0_to_f32((sw >> (8 * (2 * g + (s >> 1)))) & 0xFFu);
          a = e4m3x4_scaled_to_bf16x4(raw.x, bs);
          bb = e4m3x4_scaled_to_bf16x4(raw.y, bs);
          c = e4m3x4_scaled_to_bf16x4(raw.z, bs);
          d = e4m3x4_scaled_to_bf16x4(raw.w, bs);
        } else {
          a = e4m3x4_to_bf16x4(raw.x);
          bb = e4m3x4_to_bf16x4(raw.y);
          c = e4m3x4_to_bf16x4(raw.z);
          d = e4m3x4_to_bf16x4(raw.w);
        }
        b[2 * s] = u32x4{a.x, a.y, bb.x, bb.y};
        b[2 * s + 1] = u32x4{c.x, c.y, d.x, d.y};
      }
    }
  }
};

// The head weights of a lane's accumulator rows: weight vector k = 2q + mb
// holds w[32mb + 8q + 4g .. +3] (g = lane/32), read from the token's 64
// weights in LDS.
__device__ __forceinline__ f32x4 tile_weight(const float* lds_w, int lane, int k) {
  return *reinterpret_cast<const f32x4*>(lds_w + 32 * (k & 1) + 8 * (k >> 1) + 4 * (lane >> 5));
}

// max(x, 0) in one integer instruction: read as a signed integer, every
// negative float (-0 included) is negative and every positive one positive,
// so max(bits, 0) gives +0 for the former and x for the latter (a NaN with
// its sign bit clear passes through, where fmaxf would give 0). fmaxf on an
// MFMA result costs a second instruction, which quiets a signalling NaN
// first.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores one staged tile. Returns, in lanes 0..31, the score of tile row
// `lane` (lanes 32..63 hold the same values). wt(k): weight vector k of the
// lane (tile_weight, or a copy held in registers). sw: the scale word of row
// lane % 32.
template <int kFmt, class Weights>
__device__ __forceinline__ float score_tile(const uint8_t* lds, uint32_t sw, int lane,
                                            const u32x4 (&qa)[2][8], Weights wt) {
  u32x4 b[8];
  KeyTile<kFmt>::operands(lds, lane, sw, b);
  const float kscale = __uint_as_float(sw);
  // heads 0..31 first, then heads 32..63; the first block's ReLU and weighted
  // sum are scheduled between the second block's MFMAs, so the vector ALU
  // works while the matrix pipe runs
  f32x16 acc0 = {}, acc1 = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc0 = mfma32x32x16(qa[0][s], b[s], acc0);
#pragma unroll
  for (int s = 0; s < 8; ++s) acc1 = mfma32x32x16(qa[1][s], b[s], acc1);
  // accumulator rows 4q..4q+3 of block mb are heads 32mb + 8q + 4g + 0..3
  float sc0 = 0.0f, sc1 = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 w0 = wt(2 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float d0 = acc0[4 * q + j];
      if constexpr (kFmt == kFmtFp8) d0 *= kscale;
      sc0 = fmaf(w0[j], relu(d0), sc0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);     // block 0's MFMAs
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA of block 1
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then four VALU ops of block 0
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 w1 = wt(2 * q + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float d1 = acc1[4 * q + j];
      if constexpr (kFmt == kFmtFp8) d1 *= kscale;
      sc1 = fmaf(w1[j], relu(d1), sc1);
    }
  }
  return sum_xor32(sc0 + sc1);
}

// query heads as MFMA A operands: qa[mb][s] = q[32mb + l%32][64g + 8s .. +7]
__device__ __forceinline__ void load_query(const uint16_t* q, int lane, u32x4 (&qa)[2][8]) {
  const int nidx = lane & 31, g = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[mb][s] = *reinterpret_cast<const u32x4*>(q + (32 * mb + nidx) * kIdxDim + 64 * g + 8 * s);
}

template <int kFmt, bool kHist>
__global__ __launch_bounds__(kThreads, 2) void indexer_kernel(IndexerArgs a) {
  using Tile = KeyTile<kFmt>;
  constexpr bool kFp8 = Tile::kFp8;
  constexpr int kTileBytes = Tile::kRowBytes * kTile;
  __shared__ __attribute__((aligned(16))) uint8_t lds_tiles[kWaves * kTileBytes];
  __shared__ __attribute__((aligned(16))) float lds_w[kIdxHeads];
  __shared__ __attribute__((aligned(16))) uint32_t lds_hist[kHist ? kHist1 : 1];
  __shared__ uint32_t lds_scan[kWaves];
  __shared__ __attribute__((aligned(16))) float lds_sc[indexer_chunk(kFp8)];
  const int t = blockIdx.y;
  if constexpr (kHist) {
    SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 0);
    SGA_TL_ID(blockIdx.y * gridDim.x + blockIdx.x);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the head weights and the query need no batch metadata: their loads go
  // out first (the weights first, so that the wait for them leaves the query
  // in flight) and travel while the metadata's scalar rounds run
  // (every thread loads, clamped: a branch here would make t divergent and
  // turn the metadata's scalar loads into vector ones)
  const float wt = a.w[(int64_t)t * kIdxHeads + min((int)threadIdx.x, kIdxHeads - 1)];
  u32x4 qa[2][8];
  load_query(a.q_idx + (int64_t)t * kIdxHeads * kIdxDim, lane, qa);
  int64_t base;
  int n;
  a.batch.token(t, base, n);

  if constexpr (kHist) {
    for (int b = threadIdx.x; b < kHist1; b += kThreads) lds_hist[b] = 0;
  }
  if (threadIdx.x < kIdxHeads) lds_w[threadIdx.x] = wt;
  __syncthreads();

  const int chunk0 = blockIdx.x * a.chunk;
  const int len = min(n - chunk0, a.chunk);   // positions of this chunk (<= 0: none)
  if (len > 0) {
    uint8_t* lds = lds_tiles + wave * kTileBytes;

    const rsrc_t keys = make_rsrc(a.k_idx + (base + chunk0) * Tile::kRowBytes,
                                  (uint32_t)len * Tile::kRowBytes);
    const rsrc_t scales = make_rsrc(
        kFp8 ? (const void*)(static_cast<const uint32_t*>(a.k_scale) + base + chunk0) : (const void*)a.k_idx,
        kFp8 ? (uint32_t)len * 4u : 0u);
    const int ngroups = (len + Tile::kGroupRows - 1) / Tile::kGroupRows;
    if constexpr (kHist) SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 1);

    // this wave's tile of every group; kStages groups in flight. Loads are
    // never skipped (past the chunk they read zeros), so each wait is exact.
    constexpr int S = kStages;
    Tile st[S];
#pragma unroll
    for (int j = 0; j < S; ++j) st[j].load(keys, scales, j, wave, lane);
    for (int i = 0; i < ngroups; i += S) {
#pragma unroll
      for (int j = 0; j < S; ++j) {
        st[j].store(lds, lane);
        if constexpr (kHist) if (i == 0 && j == 0) SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 2);
        const uint32_t ks = st[j].scale;
        st[j].load(keys, scales, i + j + S, wave, lane);
        if (i + j < ngroups) {
          // each score is kept in LDS and counted while the wave's later
          // tiles are still in flight
          const float sc = score_tile<kFmt>(lds, ks, lane, qa,
                                            [&](int k) { return tile_weight(lds_w, lane, k); });
          const int p = Tile::position(i + j, wave, lane);
          if (lane < 32 && p < len) {
            lds_sc[p] = sc;
            if constexpr (kHist) atomicAdd(&lds_hist[score_key(sc) >> (32 - kDigit1Bits)], 1u);
          }
        }
      }
    }
  }
  // the chunk's scores go out in one contiguous run (16-byte stores where the
  // row is aligned): written in small pieces between the key loads, they cost
  // the stream about 4 us at 16 x 128K. The stores are streaming ones: the
  // select kernel reads the scores once, after the kernel boundary, and lines
  // left dirty in L2 would only be written back when the kernel ends (0.5 us
  // per step less at 16 x 128K)
  if constexpr (kHist) SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 3);
  __syncthreads();
  if (len > 0) {
    float* srow = a.scores + (int64_t)t * a.ld + chunk0;
    const int vec = ((reinterpret_cast<uintptr_t>(srow) & 15) == 0) ? (len & ~3) : 0;
    for (int i = 4 * (int)threadIdx.x; i < vec; i += 4 * kThreads)
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(lds_sc + i), reinterpret_cast<f32x4*>(srow + i));
    for (int i = vec + (int)threadIdx.x; i < len; i += kThreads) __builtin_nontemporal_store(lds_sc[i], srow + i);
  }
  if constexpr (kHist) {
    if (a.hist_slot_words) {
      // the chunk's bins as a list in its own slot; the first chunk's
      // workgroup zeroes the token's second-level histogram for the select
      // kernel (the kernel boundary orders both before it)
      if (blockIdx.x == 0) hist2_zero<kThreads>(a.hist2 + (int64_t)t * kHist2, threadIdx.x);
      hist1_list_store<kThreads>(lds_hist, a.hist + (int64_t)t * kHist1 + (int64_t)blockIdx.x * a.hist_slot_words,
                                 a.hist_slot_words, blockIdx.x, lds_scan);
    } else {
      hist1_flush<kThreads>(lds_hist, a.hist + (int64_t)t * kHist1);
    }
    SGA_TL_STAMP(blockIdx.y * gridDim.x + blockIdx.x, 4);
  }
}

// ---------------------------------------------------------------------------
// Many tokens over one sequence (chunked prefill). The kernel above would read
// the keys once per token; here eight tokens share every key tile. A
// workgroup of eight waves takes eight consecutive tokens, one per wave, each
// with its query in registers. The 512 threads load each 32-position key tile
// once (16 B apiece), through a ring of register stages into one of two LDS
// slots, in the same swizzled layout as above; after one barrier every wave
// scores the tile for its own token. The work is then bound by the MFMA
// pipe, not by memory. Each head block's ReLU and weighted sum run between
// MFMAs of the other block: block 0's during block 1's MFMAs of the same
// tile, block 1's during block 0's MFMAs of the next tile (its accumulators
// carry over the barrier), so no epilogue runs with the matrix pipe idle. Tokens of the eight that lie in different sequences
// are taken one sequence at a time. Each token's digit-1 histogram lives in
// LDS and, since one workgroup owns the token, goes out with plain stores.
constexpr int kPfTokens = 8;                  // tokens per workgroup, one per wave
constexpr int kPfThreads = kPfTokens * 64;
constexpr int kPfStages = 4;                  // key tiles in flight per thread

template <int kFmt, bool kHist>
__global__ __launch_bounds__(kPfThreads, 1) void indexer_prefill_kernel(IndexerArgs a) {
  using Tile = KeyTile<kFmt>;
  constexpr bool kFp8 = Tile::kFp8;
  constexpr int kTileBytes = Tile::kRowBytes * kTile;
  constexpr int kUnits = kTileBytes / 16;     // 16-byte units of a tile: 512 (bf16) or 256 (fp8)
  constexpr int kUnitsPerRow = Tile::kRowBytes / 16;
  static_assert(kUnits <= kPfThreads, "one unit per thread and tile");
  __shared__ __attribute__((aligned(16))) uint8_t lds_tiles[2][kTileBytes];
  __shared__ uint32_t lds_scale[2][kTile];
  __shared__ __attribute__((aligned(16))) float lds_w[kPfTokens][kIdxHeads];
  __shared__ uint32_t lds_hist[kHist ? kPfTokens : 1][kHist ? kHist1 : 1];
  __shared__ int32_t lds_seq[kPfTokens];
  __shared__ int32_t lds_n[kPfTokens];
  __shared__ int64_t lds_base[kPfTokens];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // waves w and w + 4 share a SIMD and leave each barrier together; the first
  // gets the higher issue priority, so it finishes its MFMAs first and runs its
  // epilogue while the second one's MFMAs are in the pipe
  if (wave < 4) __builtin_amdgcn_s_setprio(2);
  const int t = blockIdx.x * kPfTokens + wave;
  const bool live = t < a.num_tokens;
  int64_t base = 0;
  int n = 0;
  if (live) a.batch.token(t, base, n);
  if (lane == 0) {
    const int b = live ? a.batch.token_seq[t] : -1;
    lds_seq[wave] = (n > 0) ? b : -1;
    lds_n[wave] = n;
    lds_base[wave] = base;
  }
  if (lane < kIdxHeads / 4 && live)
    reinterpret_cast<f32x4*>(lds_w[wave])[lane] = reinterpret_cast<const f32x4*>(a.w + (int64_t)t * kIdxHeads)[lane];
  if constexpr (kHist)
    for (int b = lane; b < kHist1; b += 64) lds_hist[wave][b] = 0;
  __syncthreads();

  // the unit this thread loads in every tile, and where it goes in LDS
  const int u = threadIdx.x;
  const int ur = u / kUnitsPerRow, uc = u % kUnitsPerRow;
  const int lds_off = ur * Tile::kRowBytes + 16 * Tile::slot(ur, uc);
  const bool loader = u < kUnits;
  const bool scale_loader = kFp8 && threadIdx.x >= kUnits && threadIdx.x < kUnits + kTile;

  uint32_t done = 0;
  while (true) {
    // the next sequence among the eight tokens, its tokens and their longest
    // context. These come from LDS, so they are made uniform explicitly: the
    // key buffer's descriptor then stays in scalar registers (a descriptor
    // the compiler takes for divergent costs a readfirstlane loop around every
    // load).
    int lead = -1;
    for (int g = 0; g < kPfTokens; ++g)
      if (lead < 0 && !((done >> g) & 1u) && lds_seq[g] >= 0) lead = g;
    lead = __builtin_amdgcn_readfirstlane(lead);
    if (lead < 0) break;
    const int seq = __builtin_amdgcn_readfirstlane(lds_seq[lead]);
    uint32_t members = 0;
    int N = 0;
    for (int g = 0; g < kPfTokens; ++g)
      if (lds_seq[g] == seq) {
        members |= 1u << g;
        N = max(N, lds_n[g]);
      }
    members = __builtin_amdgcn_readfirstlane(members);
    N = __builtin_amdgcn_readfirstlane(N);
    done |= members;
    const bool mine = (members >> wave) & 1u;
    const int64_t base_l = lds_base[lead];
    const int64_t sbase = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base_l >> 32)) << 32) |
                                    (uint32_t)__builtin_amdgcn_readfirstlane((int)base_l));
    const rsrc_t keys = make_rsrc(a.k_idx + sbase * Tile::kRowBytes, (uint32_t)N * Tile::kRowBytes);
    const rsrc_t scales = make_rsrc(
        kFp8 ? (const void*)(static_cast<const uint32_t*>(a.k_scale) + sbase) : (const void*)a.k_idx,
        kFp8 ? (uint32_t)N * 4u : 0u);
    u32x4 qa[2][8];
    f32x4 wv[8];   // the token's head weights, held for the whole pass
    if (mine) {
      load_query(a.q_idx + (int64_t)t * kIdxHeads * kIdxDim, lane, qa);
#pragma unroll
      for (int k = 0; k < 8; ++k) wv[k] = tile_weight(lds_w[wave], lane, k);
    }
    float* srow = a.scores + (int64_t)t * a.ld;
    const int ntiles = (N + kTile - 1) / kTile;

    // register stages: tile i's unit is loaded kPfStages tiles ahead
    u32x4 stv[kPfStages];
    uint32_t sts[kPfStages];
    auto issue = [&](int j, int tile) {
      // units past the sequence (or idle threads) read zeros
      const int off = loader ? tile * kTileBytes + ur * Tile::kRowBytes + uc * 16 : (int)0x7ffffff0;
      stv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(keys, off, 0, kNonTemporal));
      if constexpr (kFp8)
        sts[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            scales, scale_loader ? (tile * kTile + (int)threadIdx.x - kUnits) * 4 : (int)0x7ffffff0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int j = 0; j < kPfStages; ++j) issue(j, j);
    static_assert(kPfStages % 2 == 0, "tile i uses LDS slot i & 1 == j & 1");
    // the second head block of tile i finishes during the first block's
    // MFMAs of tile i+1: its accumulators, the first block's sum, the row
    // scale and the tile's first position carry over (-1: nothing pending)
    f32x16 acc1p = {};
    float sc0p = 0.0f, ksp = 0.0f;
    int pp = -1;
    auto epi = [&](const f32x16& acc, int mb, float kscale) {
      float sc = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 w = wv[2 * q + mb];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float d = acc[4 * q + j];
          if constexpr (kFmt == kFmtFp8) d *= kscale;
          sc = fmaf(w[j], relu(d), sc);
        }
      }
      return sc;
    };
    auto emit = [&](float sc, int p0) {
      const int p = p0 + lane;
      if (lane < 32 && p < n) {
        srow[p] = sc;
        if constexpr (kHist) atomicAdd(&lds_hist[wave][score_key(sc) >> (32 - kDigit1Bits)], 1u);
      }
    };
    for (int i0 = 0; i0 < ntiles; i0 += kPfStages) {
#pragma unroll
      for (int j = 0; j < kPfStages; ++j) {
        const int i = i0 + j;
        const int slot = j & 1;   // == i & 1, known at compile time
        // slot i & 1 was last read two tiles ago, before the previous barrier
        if (loader) *reinterpret_cast<u32x4*>(&lds_tiles[slot][lds_off]) = stv[j];
        if constexpr (kFp8)
          if (scale_loader) lds_scale[slot][threadIdx.x - kUnits] = sts[j];
        issue(j, i + kPfStages);
        __syncthreads();
        if (mine && i < ntiles) {
          const uint32_t ks = kFp8 ? lds_scale[slot][lane & 31] : 0u;
          u32x4 b[8];
          Tile::operands(lds_tiles[slot], lane, ks, b);
          f32x16 acc0 = {};
#pragma unroll
          for (int s = 0; s < 8; ++s) acc0 = mfma32x32x16(qa[0][s], b[s], acc0);
          const float sc1p = epi(acc1p, 1, ksp);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
          const float scp = sum_xor32(sc0p + sc1p);
          if (pp >= 0) emit(scp, pp);
          f32x16 acc1 = {};
#pragma unroll
          for (int s = 0; s < 8; ++s) acc1 = mfma32x32x16(qa[1][s], b[s], acc1);
          const float sc0 = epi(acc0, 0, __uint_as_float(ks));
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
          acc1p = acc1;
          sc0p = sc0;
          ksp = __uint_as_float(ks);
          pp = i * kTile;   // tile row r is position 32i + r in this layout
        }
      }
    }
    if (mine && pp >= 0) emit(sum_xor32(sc0p + epi(acc1p, 1, ksp)), pp);
  }
  if constexpr (kHist) {
    __syncthreads();
    if (live) {
      uint32_t* gh = a.hist + (int64_t)t * kHist1;
      for (int b = lane; b < kHist1; b += 64) gh[b] = lds_hist[wave][b];
      // the second level, zeroed for the select kernel (the one-workgroup
      // top-k keeps its own in LDS)
      if (a.hist2) hist2_zero<64>(a.hist2 + (int64_t)t * kHist2, lane);
    }
  }
}

template <int kFmt>
hipError_t launch_prefill_fmt(const IndexerArgs& a, bool fused_hist, hipStream_t s) {
  const dim3 grid((a.num_tokens + kPfTokens - 1) / kPfTokens);
  if (fused_hist) indexer_prefill_kernel<kFmt, true><<<grid, kPfThreads, 0, s>>>(a);
  else indexer_prefill_kernel<kFmt, false><<<grid, kPfThreads, 0, s>>>(a);
  return hipGetLastError();
}

// Small batches take shorter chunks, halved until the grid has two workgroups
// per CU or a chunk is one 128-row group (4,096 positions x 4 tokens: 128
// workgroups instead of 8).
constexpr int kIndexerMinChunk = kWaves * kTile;
constexpr int64_t kIndexerWgTarget = 512;

int decode_chunk(int fmt, int max_len, int num_tokens) {
  int chunk = indexer_chunk(fmt != kFmtBf16);
  while (chunk > kIndexerMinChunk && (int64_t)((max_len + chunk - 1) / chunk) * num_tokens < kIndexerWgTarget)
    chunk >>= 1;
  return chunk;
}

template <int kFmt>
hipError_t launch_indexer_fmt(const IndexerArgs& args, bool fused_hist, hipStream_t s) {
  IndexerArgs a = args;
  a.chunk = decode_chunk(kFmt, a.batch.max_len, a.num_tokens);
  // list slots need one slot per chunk of the grid
  if (fused_hist && a.hist_slot_words &&
      (int64_t)a.hist_slot_words * ((a.batch.max_len + a.chunk - 1) / a.chunk) > kHist1)
    return hipErrorInvalidValue;
  const dim3 grid((a.batch.max_len + a.chunk - 1) / a.chunk, a.num_tokens);
  if (fused_hist) indexer_kernel<kFmt, true><<<grid, kThreads, 0, s>>>(a);
  else indexer_kernel<kFmt, false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_prefill(const IndexerArgs& a, int fmt, bool fused_hist, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (fmt == kFmtFp8) return launch_prefill_fmt<kFmtFp8>(a, fused_hist, s);
  if (fmt == kFmtMx) return launch_prefill_fmt<kFmtMx>(a, fused_hist, s);
  if (fmt == kFmtMx4) return launch_prefill_fmt<kFmtMx4>(a, fused_hist, s);
  return launch_prefill_fmt<kFmtBf16>(a, fused_hist, s);
}

int indexer_decode_chunk(int fmt, int max_len, int num_tokens) {
  return decode_chunk(fmt, max_len, num_tokens);
}

hipError_t launch_indexer(const IndexerArgs& a, int fmt, bool fused_hist, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (fmt == kFmtFp8) return launch_indexer_fmt<kFmtFp8>(a, fused_hist, s);
  if (fmt == kFmtMx) return launch_indexer_fmt<kFmtMx>(a, fused_hist, s);
  if (fmt == kFmtMx4) return launch_indexer_fmt<kFmtMx4>(a, fused_hist, s);
  return launch_indexer_fmt<kFmtBf16>(a, fused_hist, s);
}

}  // namespace sga
