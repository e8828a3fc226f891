// Sparse absorbed-MLA attention over the selected latent rows, with the
// per-head sigmoid output gate.
// Sources: A.X K2 fact sheet (archdb): 64 query heads; QK dim 192 = 128 NoPE +
// 64 RoPE; 512-wide compressed latent plus 64-wide shared RoPE key cached per
// token; no QK norm, no QKV bias; a head-specific sigmoid gate on the
// attention output before o_proj.
//
// Per token: z[h,j] = sm_scale * q_abs[h,:] . row_j[0:576],
// o[h,:] = softmax_j(z) . row_j[0:512], out = o * sigmoid(g[h]).
//
// Mapping onto gfx950. A workgroup of 8 waves takes one token and one slice
// (split) of its selected rows, 32 rows per tile. Wave w owns heads
// 16*(w%4) .. +15 and one half h = w/4 of the work:
//   logits: dims 288h .. 288h+287 (9 of the 18 k-steps of
//           v_mfma_f32_16x16x32_bf16, logits^T = rows x q^T); the two waves
//           of a pair swap their partial logits through LDS and add them
//           (fp32 addition commutes, so both hold identical logits);
//   output: latent columns 256h .. 256h+255 (o^T += rows^T x p^T), with the
//           rows^T operand read by ds_read_b64_tr_b16 from the row-major tile.
// Probabilities enter the value product as a bf16 hi/lo pair (p = hi + lo to
// about 16 bits). The online softmax runs in fp32, base 2.
//
// Row stream. The gather is a pipeline through registers: while a tile is
// attended, the rows of the next two tiles are in flight, and the indices of
// the tiles after those are loaded ahead of the rows that need them. Every
// load is an unconditional buffer load (a skipped row's offset lies past the
// end of the buffer and reads zeros), so the compiler's wait for one tile
// never covers the loads of a later one. Three LDS regions rotate, so one
// workgroup barrier per tile suffices: before it, each wave stores its part
// of tile i+1 and computes and posts its partial logits of tile i; after it,
// it reads its partner's partial logits and finishes tile i (softmax and
// value product). The region a wave stores into was last read two tiles
// earlier, before the previous barrier.
// fp8 rows are widened to bf16 exactly on their way into LDS; the row scale
// multiplies the row's logit and probability. MX block-32 rows (fact sheet,
// Training: MXFP8, one scale per 32 consecutive elements) have each 32-column
// block multiplied by its power-of-two scale as it is widened, which is exact
// in bf16, and are then attended like bf16 rows. The same holds for MX rows of
// four-bit E2M1 elements (two per byte).
//
// With several splits per token, each split writes its output normalised by
// its own exp-sum, in fp16 with a per-half scale, plus (max, exp-sum);
// combine_kernel merges the splits by log-sum-exp and applies the gate.
#include <string.h>

#include "sga_finalize.h"
#include "sga_kernels.h"

SGA_TL_RECORD(attn)

namespace sga {
namespace {

constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kRowStride = kDQK + 8;  // bf16 elements per LDS row (1168 B)
constexpr int kRegionBytes = kAttnTileRows * kRowStride * 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;  // base-2 headroom of the running max (probabilities <= 256)
constexpr int kNonTemporal = 2;   // cache-policy bit: rows are read once per token

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ float gate_factor(const float* gate, int64_t idx) {
  if (!gate) return 1.0f;
  return 1.0f / (1.0f + expf(-gate[idx]));
}

// One tile's rows in registers: thread x holds 16-byte units x, x + 512, ...
// of the tile (row u / kUnitsPerRow, unit u % kUnitsPerRow of that row).
template <int kFmt>
struct RowStage {
  static constexpr bool kFp8 = kFmt != kFmtBf16;                  // narrow payloads, widened in LDS
  static constexpr bool kMx = kFmt == kFmtMx || kFmt == kFmtMx4;  // E8M0 block exponents
  static constexpr int kRowBytes = row_bytes(kFmt, kDQK);         // cached bytes per row
  static constexpr int kUnitsPerRow = kRowBytes / 16;             // 72, 36 or 18
  static constexpr int kUnits = kAttnTileRows * kUnitsPerRow;     // 2304, 1152 or 576
  static constexpr int kPer = (kUnits + kAttnThreads - 1) / kAttnThreads;  // 5, 3 or 2
  u32x4 v[kPer];
  uint32_t s[kPer];     // the unit's fp32 row scale (fp8) or its block's E8M0 exponent (MX)
  int32_t idx[kPer];    // row indices for the next load_rows
  uint32_t ok;          // bit q: unit q of the loaded tile is a real row

  // Thread x holds units x + 512q; the last q may fall past the tile's units.
  // Every load below is issued by every thread, whatever its unit, and every
  // skipped load gets an offset past the end of its buffer (bit 31 set), so
  // no load sits under a branch and the compiler can count them exactly.
  static __device__ __forceinline__ int unit(int q) { return q * kAttnThreads + (int)threadIdx.x; }

  // indices of tile `tile` (relative to the split); past the split they read 0
  __device__ __forceinline__ void load_idx(rsrc_t idx_rs, int tile) {
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      idx[q] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
          idx_rs, (tile * kAttnTileRows + unit(q) / kUnitsPerRow) * 4, 0, 0);
  }

  // indices of tile `tile` from the split's indices in LDS (rows past the
  // split read some entry and are masked by the row count)
  __device__ __forceinline__ void load_idx_lds(const int32_t* lidx, int tile) {
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      idx[q] = lidx[min(tile * kAttnTileRows + unit(q) / kUnitsPerRow, kSelectMaxRows - 1)];
  }

  // rows of tile `tile`, from the indices loaded for it
  __device__ __forceinline__ void load_rows(rsrc_t rows, rsrc_t scales, int tile, int nrows, int n) {
    uint32_t m = 0;
    const int t0 = tile * kAttnTileRows;
    constexpr int kSkip = (int)0x80000000;   // an offset past the end of every buffer
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int u = unit(q);
      const int r = u / kUnitsPerRow;
      const int c = u - r * kUnitsPerRow;
      const int id = idx[q];
      // row t0 + r lies inside the split, and its index inside [0, n) (n >= 0;
      // a negative index compares unsigned as at least n)
      const bool real = (r < kAttnTileRows) & (t0 < nrows - r) & ((uint32_t)id < (uint32_t)n);
      m |= (uint32_t)real << q;
      v[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rows, real ? (int)((uint32_t)id * kRowBytes + 16u * c) : kSkip,
                                           0, kNonTemporal));
      if constexpr (kFmt == kFmtFp8)
        s[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(scales, real ? (int)((uint32_t)id * 4u) : kSkip, 0, 0);
      if constexpr (kMx)   // the unit's block: c/2 (16 E4M3FN bytes) or c (32 E2M1 nibbles)
        s[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
            scales,
            real ? (int)((uint32_t)id * (kDQK / 32) + (uint32_t)(kFmt == kFmtMx ? c >> 1 : c)) : kSkip, 0, 0);
    }
    ok = m;
    // keep each tile's loads together, in program order
    __builtin_amdgcn_sched_barrier(0);
  }

  // Stores the tile into an LDS region (bf16 rows of kRowStride elements) and
  // each row's flags: flags[r] is the bias added to the row's logit (0, or
  // -inf for a skipped row, whose zero data then gives a -inf logit), and for
  // fp8 flags[kAttnTileRows + r] is the row's scale (0 for a skipped row).
  __device__ __forceinline__ void store(uint8_t* region, float* flags) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int u = q * kAttnThreads + (int)threadIdx.x;
      if (u < kUnits) {
        const int r = u / kUnitsPerRow, c = u - r * kUnitsPerRow;
        uint8_t* row = region + r * (2 * kRowStride);
        if constexpr (!kFp8) {
          *reinterpret_cast<u32x4*>(row + 16 * c) = v[q];
        } else if constexpr (kFmt == kFmtMx4) {
          const float bs = e8m0_to_f32(s[q]);
          u32x4* dst = reinterpret_cast<u32x4*>(row + 64 * c);
          dst[0] = e2m1x8_scaled_to_bf16x8(v[q].x, bs);
          dst[1] = e2m1x8_scaled_to_bf16x8(v[q].y, bs);
          dst[2] = e2m1x8_scaled_to_bf16x8(v[q].z, bs);
          dst[3] = e2m1x8_scaled_to_bf16x8(v[q].w, bs);
        } else {
          u32x2 a0, a1, a2, a3;
          if constexpr (kFmt == kFmtMx) {
            const float bs = e8m0_to_f32(s[q]);
            a0 = e4m3x4_scaled_to_bf16x4(v[q].x, bs);
            a1 = e4m3x4_scaled_to_bf16x4(v[q].y, bs);
            a2 = e4m3x4_scaled_to_bf16x4(v[q].z, bs);
            a3 = e4m3x4_scaled_to_bf16x4(v[q].w, bs);
          } else {
            a0 = e4m3x4_to_bf16x4(v[q].x);
            a1 = e4m3x4_to_bf16x4(v[q].y);
            a2 = e4m3x4_to_bf16x4(v[q].z);
            a3 = e4m3x4_to_bf16x4(v[q].w);
          }
          u32x4* dst = reinterpret_cast<u32x4*>(row + 32 * c);
          dst[0] = u32x4{a0.x, a0.y, a1.x, a1.y};
          dst[1] = u32x4{a2.x, a2.y, a3.x, a3.y};
        }
        if (c == 0) {
          const bool real = (ok >> q) & 1u;
          flags[r] = real ? 0.0f : -INFINITY;
          if constexpr (kFmt == kFmtFp8) flags[kAttnTileRows + r] = real ? __uint_as_float(s[q]) : 0.0f;
        }
      }
    }
  }
};

// Online-softmax state of one wave: 16 heads (one per lane column) and its
// half of their latent-space output, o^T[256h + 16db + 4(lane/16) + r][head].
struct HalfState {
  float m_run, l_run;
  f32x4 o[16];
};

// First half of a tile for the wave's 16 heads: its partial logits^T over
// this half's 9 k-steps (one chain per row block), posted to its slot of
// xbuf for the partner wave and returned.
__device__ __forceinline__ void tile_partial_logits(const uint16_t* __restrict__ tile,
                                                    float* __restrict__ xbuf, const u32x4 (&qb)[9],
                                                    int lane, int wave, int half, f32x4 (&part)[2]) {
  const int n16 = lane & 15, g = lane >> 4;
  // one chain per row block; the two blocks' MFMAs alternate
  f32x4 acc[2] = {};
  const uint16_t* rowp0 = tile + n16 * kRowStride + 8 * g + 288 * half;
  const uint16_t* rowp1 = rowp0 + 16 * kRowStride;
#pragma unroll
  for (int s = 0; s < 9; ++s) {
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(rowp0 + 32 * s);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(rowp1 + 32 * s);
    acc[0] = mfma16x16x32(a0, qb[s], acc[0]);
    acc[1] = mfma16x16x32(a1, qb[s], acc[1]);
  }
  part[0] = acc[0];
  part[1] = acc[1];
  f32x4* mine = reinterpret_cast<f32x4*>(xbuf + (wave * 64 + lane) * 8);
  mine[0] = part[0];
  mine[1] = part[1];
}

// Second half of a tile, after the barrier: the full logits (own partial plus
// the partner's), the online softmax and the value product. flags: the rows'
// logit biases (0, or -inf for a skipped row) and, for fp8, their scales.
template <bool kFp8>
__device__ __forceinline__ void tile_finish(const uint16_t* __restrict__ tile,
                                            const float* __restrict__ flags,
                                            const float* __restrict__ xbuf, HalfState& st,
                                            const f32x4 (&part)[2], float zscale, int lane,
                                            int wave, int half) {
  const int g = lane >> 4;
  const f32x4* other = reinterpret_cast<const f32x4*>(xbuf + ((wave ^ 4) * 64 + lane) * 8);
  const f32x4 full[2] = {part[0] + other[0], part[1] + other[1]};
  float z[2][4], rsc[2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * b + 4 * g + r;
      float v = full[b][r];
      if constexpr (kFp8) {
        rsc[b][r] = flags[kAttnTileRows + row];
        v *= rsc[b][r];
      }
      z[b][r] = fmaf(v, zscale, flags[row]);
      tmax = fmaxf(tmax, z[b][r]);
    }
  tmax = max_xor32(max_xor16(tmax));
  // The running max moves only when the tile's max passes it by more than
  // kLazyMax (base 2): the probabilities then stay below 2^kLazyMax and the
  // accumulators are rescaled only on such a jump. Any reference point gives
  // the same softmax, as o and l share it; (m, l) record it for the merge.
  const float m_new = tmax > st.m_run + kLazyMax ? tmax : st.m_run;
  const float alpha = (st.m_run == -INFINITY || m_new == st.m_run)
                          ? 1.0f : __builtin_amdgcn_exp2f(st.m_run - m_new);
  // exp2(-inf - m) = 0 gives the skipped rows; a max that is still -inf (every
  // row so far skipped) is replaced by 0, so no -inf - -inf arises
  const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
  float p[2][4];
  float psum = 0.0f;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e = __builtin_amdgcn_exp2f(z[b][r] - m_ref);
      psum += e;
      if constexpr (kFp8) e *= rsc[b][r];
      p[b][r] = e;
    }
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int db = 0; db < 16; ++db) st.o[db] *= alpha;
  }
  // probabilities as bf16 hi/lo B operands: k-slot 8g+i <-> row 4g+i (i<4), 16+4g+i-4
  uint32_t lo[4];
  const u32x4 phi = {split_bf16x2(p[0][0], p[0][1], lo[0]), split_bf16x2(p[0][2], p[0][3], lo[1]),
                     split_bf16x2(p[1][0], p[1][1], lo[2]), split_bf16x2(p[1][2], p[1][3], lo[3])};
  const u32x4 plo = {lo[0], lo[1], lo[2], lo[3]};
  // transposed reads: lane s reads row 4(s/16) + (s%16)/4 [+16], columns 4(s%4) .. +3
  // of each 16-column block
  const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int tr_col = 4 * (lane & 3) + 256 * half;
  const uint16_t* tr0 = tile + tr_row * kRowStride + tr_col;
  const uint16_t* tr1 = tr0 + 16 * kRowStride;
#pragma unroll
  for (int db = 0; db < 16; ++db) {
    s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr0 + 16 * db));
    s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr1 + 16 * db));
    u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
    const u32x4 vt = {w0.x, w0.y, w1.x, w1.y};
    st.o[db] = mfma16x16x32(vt, phi, st.o[db]);
    st.o[db] = mfma16x16x32(vt, plo, st.o[db]);
  }
}

// Writes a wave's result: the gated, normalised output when the token has one
// split, else the split's partial plus (m, l).
__device__ __forceinline__ void finish_half(const AttnArgs& a, HalfState& st, int t, int split,
                                            int head, int lane, int half) {
  const int g = lane >> 4;
  const float l_tot = sum_xor32(sum_xor16(st.l_run));
  const int64_t th = (int64_t)t * kHeads + head;
  if (a.splits == 1) {
    const float gs = gate_factor(a.gate, th);
    const float inv = l_tot > 0.0f ? gs / l_tot : 0.0f;
    float* dst = a.out + th * kDLatent + 256 * half + 4 * g;
#pragma unroll
    for (int db = 0; db < 16; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = st.o[db] * inv;
    if (a.lse && g == 0 && half == 0)
      a.lse[th] = l_tot > 0.0f ? (st.m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    return;
  }
  // The split's output normalised by its exp-sum is a convex combination of
  // value rows; divided by its largest magnitude it lies in [-1, 1] and is
  // stored as fp16 (relative rounding 2^-11), with the scale kept in fp32.
  // Layout [token][split][column block db][head][16 columns]. Lane groups g
  // and g ^ 1 (lanes l and l ^ 16, same head) trade halves, so that for a pair
  // of column blocks the even group writes 8 columns of the first and the odd
  // group 8 of the second, each as one 16-byte store (0.5-0.8 us per step
  // less than 8-byte stores at 128K x 16 and 256K x 8).
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float amax = 0.0f;
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(st.o[db][r]));
  amax = max_xor32(max_xor16(amax));
  amax *= inv_l;
  const float scale = amax > 0.0f ? amax : 1.0f;
  const float k = inv_l / scale;
  const int64_t ts = (int64_t)t * a.splits + split;
  // the lane pair's 8 columns of the head in column block 0 of this half
  uint16_t* dst = a.part_o + ts * kHeads * kDLatent + 16 * half * (kHeads * 16) + head * 16 + 4 * (g & ~1);
  const bool odd = g & 1;
#pragma unroll
  for (int db = 0; db < 16; db += 2) {
    const f32x4 v0 = st.o[db] * k, v1 = st.o[db + 1] * k;
    const uint32_t p0x = pack_f16x2(v0[0], v0[1]), p0y = pack_f16x2(v0[2], v0[3]);
    const uint32_t p1x = pack_f16x2(v1[0], v1[1]), p1y = pack_f16x2(v1[2], v1[3]);
    // the even group sends its half of block db + 1, the odd one its half of db
    const uint32_t rx = (uint32_t)__shfl_xor((int)(odd ? p0x : p1x), 16);
    const uint32_t ry = (uint32_t)__shfl_xor((int)(odd ? p0y : p1y), 16);
    const u32x4 o = odd ? u32x4{rx, ry, p1x, p1y} : u32x4{p0x, p0y, rx, ry};
    // streaming store: the partials are read once, by the merge, and little
    // of them is left dirty in L2 when the kernel ends
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + (db + (odd ? 1 : 0)) * (kHeads * 16)));
  }
  if (g == 0) {
    float* ml = a.part_ml + 4 * (ts * kHeads + head);
    if (half == 0) {
      ml[0] = st.m_run;
      ml[1] = l_tot;
    }
    ml[2 + half] = scale;
  }
}

// The probabilities variant, after the barrier: each selected row's head-mean
// attention probability (1/64) sum_h exp(z_h - lse_h), with lse the
// attention's own log-sum-exp over all selected rows (an input). The waves of
// half 0 sum their 16 heads per row and post them; after a second barrier
// the first 32 threads add the four head groups and write the tile's rows.
template <bool kFp8>
__device__ __forceinline__ void tile_probs(const float* __restrict__ flags,
                                           const float* __restrict__ xbuf, float* __restrict__ psum,
                                           const f32x4 (&part)[2], float zscale, float lse2,
                                           float* __restrict__ prob_out, int nrows_left, int lane,
                                           int wave) {
  const int g = lane >> 4;
  if (wave < 4) {
    const f32x4* other = reinterpret_cast<const f32x4*>(xbuf + ((wave ^ 4) * 64 + lane) * 8);
    const f32x4 full[2] = {part[0] + other[0], part[1] + other[1]};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * b + 4 * g + r;
        float v = full[b][r] * zscale;
        if constexpr (kFp8) v *= flags[kAttnTileRows + row];
        float e = flags[row] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(v - lse2);
        // sum over the 16 heads of this lane group
        e += __shfl_xor(e, 1);
        e += __shfl_xor(e, 2);
        e += __shfl_xor(e, 4);
        e += __shfl_xor(e, 8);
        if ((lane & 15) == 0) psum[wave * kAttnTileRows + 16 * b + 4 * g + r] = e;
      }
  }
  __syncthreads();
  if (threadIdx.x < kAttnTileRows && (int)threadIdx.x < nrows_left) {
    const int r = threadIdx.x;
    const float sum = psum[r] + psum[kAttnTileRows + r] + psum[2 * kAttnTileRows + r] +
                      psum[3 * kAttnTileRows + r];
    prob_out[r] = sum * (1.0f / kHeads);
  }
}

// LDS of the attention kernel: three row regions, their flags, and the
// partial-logit exchange buffers, in one array (the selecting variant first
// runs the top-k's final stage in the same bytes).
constexpr int kFlagsOffset = 3 * kRegionBytes;
constexpr int kXbufOffset = kFlagsOffset + 3 * 2 * kAttnTileRows * 4;
constexpr int kAttnLdsBytes = kXbufOffset + 2 * kAttnWaves * 64 * 8 * 4;
static_assert(finalize_lds_words((kMaxLenRows + 63) / 64 * 2) * 4 <= kAttnLdsBytes,
              "the top-k's final stage fits in the attention's LDS at the longest context");

// kSelect: the kernel first finds its own rows of the token's top-k: every
// split of the token runs the top-k's final stage (sga_finalize.h) on the
// select kernel's output, keeps the ranks of its split in LDS (and writes them
// to indices_out when asked), then attends over them. The final stage's reads
// are a few tens of KB per token, served by L2.
template <int kFmt, bool kProbs, bool kSelect>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnArgs a, TopkArgs ta) {
  constexpr bool kRowScale = kFmt == kFmtFp8;
  __shared__ __attribute__((aligned(16))) uint8_t lds_main[kAttnLdsBytes];
  __shared__ float psum[kProbs ? 2 : 1][kProbs ? 4 * kAttnTileRows : 1];
  __shared__ int32_t lds_idx[kSelect ? kSelectMaxRows : 1];
  auto lds_tile = reinterpret_cast<uint8_t(*)[kRegionBytes]>(lds_main);
  auto lds_flags = reinterpret_cast<float(*)[2 * kAttnTileRows]>(lds_main + kFlagsOffset);
  auto xbuf = reinterpret_cast<float(*)[kAttnWaves * 64 * 8]>(lds_main + kXbufOffset);
  using Stage = RowStage<kFmt>;
  const int wg = xcd_grouped(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const int t = wg / a.splits, split = wg % a.splits;
  if constexpr (!kProbs) {
    SGA_TL_STAMP(wg, 0);
    SGA_TL_ID(wg);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the two waves of a pair share a SIMD and leave each barrier together; the
  // first gets the higher issue priority, so it reaches its value product while
  // the second one still runs its softmax
  if (wave < 4) __builtin_amdgcn_s_setprio(2);
  const int half = wave >> 2;
  const int head = 16 * (wave & 3) + (lane & 15);
  const int g = lane >> 4;
  const int j_begin = split * a.rows_per_split;
  const int nrows = max(0, min(a.k, j_begin + a.rows_per_split) - j_begin);
  const int ntiles = (nrows + kAttnTileRows - 1) / kAttnTileRows;
  const rsrc_t idx_rs = make_rsrc(a.indices + (int64_t)t * a.k + j_begin, (uint32_t)nrows * 4u);

  // the indices and the query do not depend on the batch metadata: their
  // loads go out first and travel while the metadata's two scalar rounds run
  // (the selecting variant issues the final stage's loads instead of the
  // indices)
  Stage s0, s1;
  TokenFinalize<kAttnThreads> fin;
  if constexpr (kSelect) {
    fin.prefetch(ta, t);
  } else {
    s0.load_idx(idx_rs, 0);
    s1.load_idx(idx_rs, 1);
  }
  u32x4 qb[9];
  {
    const uint16_t* q = a.q_abs + ((int64_t)t * kHeads + head) * kDQK + 288 * half + 8 * g;
#pragma unroll
    for (int s = 0; s < 9; ++s) qb[s] = *reinterpret_cast<const u32x4*>(q + 32 * s);
  }
  // the batch metadata (needed only for the row gathers): its two scalar
  // rounds run while the selecting variant's final stage works
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  if constexpr (kSelect) {
    // this split's ranks [j_begin, j_begin + nrows) of the token's selection;
    // the visible count comes with the cut, so the stage does not wait for the
    // batch metadata
    const int nv = fin.visible();
    if (nv <= a.k) {   // every visible position is kept: rank r is position r
      for (int j = threadIdx.x; j < nrows; j += kAttnThreads) lds_idx[j] = j_begin + j < nv ? j_begin + j : -1;
    } else {
      fin.run(ta, nv, reinterpret_cast<uint32_t*>(lds_main), (uint32_t)j_begin, (uint32_t)(j_begin + nrows),
              [&](uint32_t o, uint32_t p) { lds_idx[o - j_begin] = (int32_t)p; });
    }
    __syncthreads();   // the indices are in LDS, and the stage's LDS is free again
    if constexpr (!kProbs) SGA_TL_STAMP(wg, 1);
    if (a.indices_out)
      for (int j = threadIdx.x; j < nrows; j += kAttnThreads)
        a.indices_out[(int64_t)t * a.k + j_begin + j] = lds_idx[j];
    s0.load_idx_lds(lds_idx, 0);
    s1.load_idx_lds(lds_idx, 1);
  }
  const uint32_t rows_bytes = (uint32_t)max(n, 0) * Stage::kRowBytes;
  const rsrc_t rows = make_rsrc(a.kv + base * Stage::kRowBytes, rows_bytes);
  const rsrc_t scales =
      kFmt == kFmtFp8 ? make_rsrc(static_cast<const float*>(a.kv_scale) + base, (uint32_t)max(n, 0) * 4u)
      : Stage::kMx ? make_rsrc(static_cast<const uint8_t*>(a.kv_scale) + base * (kDQK / 32),
                               (uint32_t)max(n, 0) * (kDQK / 32))
                       : make_rsrc(a.kv, 0u);
  auto load_idx = [&](Stage& sg, int tile) {
    if constexpr (kSelect) sg.load_idx_lds(lds_idx, tile);
    else sg.load_idx(idx_rs, tile);
  };
  s0.load_rows(rows, scales, 0, nrows, n);
  load_idx(s0, 2);
  s1.load_rows(rows, scales, 1, nrows, n);
  load_idx(s1, 3);

  HalfState st;
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
#pragma unroll
  for (int db = 0; db < 16; ++db) st.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float zscale = a.sm_scale * kLog2e;
  float lse2 = 0.0f;   // the head's log-sum-exp in base 2 (probabilities variant)
  if constexpr (kProbs) lse2 = a.lse_in[(int64_t)t * kHeads + head] * kLog2e;

  // tile 0 into region 0; its stage is refilled with tile 2
  s0.store(lds_tile[0], lds_flags[0]);
  s0.load_rows(rows, scales, 2, nrows, n);
  load_idx(s0, 4);
  __syncthreads();
  if constexpr (!kProbs) SGA_TL_STAMP(wg, 2);

  // step i: store tile i+1 from its stage into region (i+1) % 3, refill the
  // stage with tile i+3 (indices loaded two tiles earlier) and the indices of
  // tile i+5, post the partial logits of tile i; barrier; finish tile i
  int cur = 0;   // region of tile i
  auto step = [&](Stage& sg, int i) {
    const int nxt = cur == 2 ? 0 : cur + 1;
    sg.store(lds_tile[nxt], lds_flags[nxt]);
    sg.load_rows(rows, scales, i + 3, nrows, n);
    load_idx(sg, i + 5);
    const uint16_t* tile = reinterpret_cast<const uint16_t*>(lds_tile[cur]);
    f32x4 part[2];
    if (i < ntiles) tile_partial_logits(tile, xbuf[i & 1], qb, lane, wave, half, part);
    __syncthreads();
    if constexpr (kProbs) {
      if (i < ntiles)
        tile_probs<kRowScale>(lds_flags[cur], xbuf[i & 1], psum[i & 1], part, zscale, lse2,
                              a.probs + (int64_t)t * a.k + j_begin + i * kAttnTileRows,
                              nrows - i * kAttnTileRows, lane, wave);
    } else {
      if (i < ntiles)
        tile_finish<kRowScale>(tile, lds_flags[cur], xbuf[i & 1], st, part, zscale, lane, wave, half);
    }
    cur = nxt;
  };
  for (int i = 0; i < ntiles; i += 2) {
    step(s1, i);
    step(s0, i + 1);
  }
  if constexpr (!kProbs) {
    SGA_TL_STAMP(wg, 3);
    finish_half(a, st, t, split, head, lane, half);
    SGA_TL_STAMP(wg, 4);
  }
}

// Merges the split partials by log-sum-exp, then gates. One workgroup of two
// waves per (column block db, token): thread j takes head j/2 and columns
// 16*db + 8*(j%2) .. +7. Up to 16 splits are merged per round, with every
// load of the round (one 16-byte (m, l, scales) record and one 16-byte slice
// of fp16 partial per split) issued before any is used. Against four threads
// of 8 bytes per head, this was 1.2-1.6 us faster per 128K decode step and
// on the ragged batch.
constexpr int kCombineRound = 16;

__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) {
  const int wg = xcd_grouped(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const int db = wg % (kDLatent / 16), t = wg / (kDLatent / 16);
  SGA_TL_STAMP(4096 + wg, 0);
  SGA_TL_ID(4096 + wg);
  const int h = threadIdx.x >> 1, q = threadIdx.x & 1;
  const int S = a.splits;
  const int64_t th = (int64_t)t * kHeads + h;
  const f32x4* ml = reinterpret_cast<const f32x4*>(a.part_ml) + (int64_t)t * S * kHeads + h;
  const uint16_t* po = a.part_o + (int64_t)t * S * kHeads * kDLatent + db * (kHeads * 16) + h * 16 + 8 * q;
  const int sc = 2 + (db >= 16);   // scale of this column half
  float M = -INFINITY, L = 0.0f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kCombineRound) {
    f32x4 r[kCombineRound];
    u32x4 v[kCombineRound];
#pragma unroll
    for (int u = 0; u < kCombineRound; ++u) {
      const int s = min(s0 + u, S - 1);
      r[u] = ml[(int64_t)s * kHeads];
      v[u] = *reinterpret_cast<const u32x4*>(po + (int64_t)s * kHeads * kDLatent);
    }
    float m_new = M;
#pragma unroll
    for (int u = 0; u < kCombineRound; ++u)
      if (s0 + u < S) m_new = fmaxf(m_new, r[u][0]);
    if (m_new == -INFINITY) continue;   // no rows so far
    const float alpha = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - m_new);
    L *= alpha;
    acc0 *= alpha;
    acc1 *= alpha;
#pragma unroll
    for (int u = 0; u < kCombineRound; ++u) {
      const float w = (s0 + u >= S || r[u][0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(r[u][0] - m_new);
      const float ls = r[u][1] * w;
      L += ls;
      const f32x2 a0 = unpack_f16x2(v[u].x), a1 = unpack_f16x2(v[u].y);
      const f32x2 a2 = unpack_f16x2(v[u].z), a3 = unpack_f16x2(v[u].w);
      const float f = ls * r[u][sc];
      acc0 += f32x4{a0.x, a0.y, a1.x, a1.y} * f;
      acc1 += f32x4{a2.x, a2.y, a3.x, a3.y} * f;
    }
    M = m_new;
  }
  const float gs = gate_factor(a.gate, th);
  const float inv = L > 0.0f ? gs / L : 0.0f;
  *reinterpret_cast<f32x4*>(a.out + th * kDLatent + 16 * db + 8 * q) = acc0 * inv;
  *reinterpret_cast<f32x4*>(a.out + th * kDLatent + 16 * db + 8 * q + 4) = acc1 * inv;
  if (a.lse && db == 0 && q == 0) a.lse[th] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
  SGA_TL_STAMP(4096 + wg, 1);
}

// The sparse indexer loss of one token: KL(p || q) over its selected rows,
// p the head-mean attention probabilities (from the probabilities variant),
// q the softmax of the indexer scores over the same rows. One workgroup per
// token: the scores' maximum, their log-sum-exp, then the KL sum.
__device__ __forceinline__ float block_reduce(float v, float* red, bool take_max) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = take_max ? fmaxf(v, w) : v + w;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = take_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__global__ __launch_bounds__(256) void indexer_loss_kernel(LossArgs a) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  const int32_t* idx = a.indices + (int64_t)t * a.k;
  const float* sc = a.scores + (int64_t)t * a.ld;
  const float* pr = a.probs + (int64_t)t * a.k;
  float m = -INFINITY;
  for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
    const int s = idx[j];
    if (s >= 0 && s < n) m = fmaxf(m, sc[s]);
  }
  m = block_reduce(m, red, true);
  if (m == -INFINITY) {   // nothing selected
    if (threadIdx.x == 0) a.loss[t] = 0.0f;
    return;
  }
  float z = 0.0f;
  for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
    const int s = idx[j];
    if (s >= 0 && s < n) z += expf(sc[s] - m);
  }
  const float lse = m + logf(block_reduce(z, red, false));
  float kl = 0.0f;
  for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
    const int s = idx[j];
    const float p = pr[j];
    if (s >= 0 && s < n && p > 0.0f) kl += p * (logf(p) - (sc[s] - lse));
  }
  kl = block_reduce(kl, red, false);
  if (threadIdx.x == 0) a.loss[t] = kl;
}

}  // namespace

template <bool kProbs, bool kSelect>
hipError_t launch_attn(const AttnArgs& a, const TopkArgs& ta, int fmt, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid(a.splits, a.num_tokens);
  if (fmt == kFmtFp8) attn_kernel<kFmtFp8, kProbs, kSelect><<<grid, kAttnThreads, 0, s>>>(a, ta);
  else if (fmt == kFmtMx) attn_kernel<kFmtMx, kProbs, kSelect><<<grid, kAttnThreads, 0, s>>>(a, ta);
  else if (fmt == kFmtMx4) attn_kernel<kFmtMx4, kProbs, kSelect><<<grid, kAttnThreads, 0, s>>>(a, ta);
  else attn_kernel<kFmtBf16, kProbs, kSelect><<<grid, kAttnThreads, 0, s>>>(a, ta);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int fmt, hipStream_t s) {
  TopkArgs unused;
  memset(&unused, 0, sizeof(unused));
  return launch_attn<false, false>(a, unused, fmt, s);
}

hipError_t launch_attention_select(const AttnArgs& a, const TopkArgs& ta, int fmt, hipStream_t s) {
  if (a.rows_per_split > kSelectMaxRows) return hipErrorInvalidValue;
  return launch_attn<false, true>(a, ta, fmt, s);
}

hipError_t launch_attention_probs(const AttnArgs& a, int fmt, hipStream_t s) {
  TopkArgs unused;
  memset(&unused, 0, sizeof(unused));
  return launch_attn<true, false>(a, unused, fmt, s);
}

hipError_t launch_indexer_loss(const LossArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  indexer_loss_kernel<<<a.num_tokens, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t s) {
  if (a.num_tokens == 0 || a.splits == 1) return hipSuccess;
  combine_kernel<<<dim3(kDLatent / 16, a.num_tokens), 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
