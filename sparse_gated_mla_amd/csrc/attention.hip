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
// Mapping onto gfx950: a workgroup takes one token and one slice of its
// selected rows. Rows are gathered 32 at a time into LDS and shared by all 64
// heads: each of the 4 waves owns 16 heads. With v_mfma_f32_16x16x32_bf16:
//   logits^T = rows(M=16 rows) x q^T(N=16 heads, K=576). q stays in registers.
//   o^T     += rows^T(M=16 latent dims, K=32 rows) x p^T(N=16 heads).
// The rows^T operand comes from ds_read_b64_tr_b16, which reads 4 rows of one
// column per lane. So the row-major tile needs no transpose pass.
// Probabilities enter the value product as a bf16 hi/lo pair (p = hi + lo to
// about 16 bits). The online softmax runs in fp32, base 2.
// fp8 rows are widened to bf16 exactly while staged. The row scale multiplies
// the logit and the probability of the row.
// Splits of one token write unnormalised partials. combine_kernel merges them
// by log-sum-exp and applies the gate.
#include "sga_kernels.h"

namespace sga {
namespace {

constexpr int kThreads = 256;
constexpr int kRowStride = kDQK + 8;  // bf16 elements per LDS row (1168 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNonTemporal = 2;   // cache-policy bit: rows are read once per token

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// s_waitcnt immediates that wait only for the vector-memory counter to fall to
// N (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8
// left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kVmcntWait[3] = {vmcnt_imm(10), vmcnt_imm(5), vmcnt_imm(0)};

__device__ __forceinline__ float gate_factor(const float* gate, int64_t idx) {
  if (!gate) return 1.0f;
  return 1.0f / (1.0f + expf(-gate[idx]));
}

template <bool kFp8>
struct TileLoader {
  // bf16: 32 rows x 72 chunks of 16 B = 2304 chunks -> 9 per thread.
  // fp8:  32 rows x 36 chunks of 16 B = 1152 chunks -> 4.5 per thread.
  static constexpr int kChunksPerRow = kFp8 ? 36 : 72;
  static constexpr int kChunks = kAttnTileRows * kChunksPerRow;
  static constexpr int kPerThread = (kChunks + kThreads - 1) / kThreads;
  u32x4 v[kPerThread];

  __device__ __forceinline__ void load(const AttnArgs& a, const int32_t* __restrict__ idx_row,
                                       int j_begin, int j_end, int64_t base, int n) {
#pragma unroll
    for (int it = 0; it < kPerThread; ++it) {
      const int c = threadIdx.x + it * kThreads;
      v[it] = u32x4{0u, 0u, 0u, 0u};
      if (c < kChunks) {
        const int r = c / kChunksPerRow, cc = c % kChunksPerRow;
        const int j = j_begin + r;
        int idx = j < j_end ? idx_row[j] : -1;
        if (idx >= 0 && idx < n) {
          const uint8_t* src = a.kv + (base + idx) * (kFp8 ? kDQK : 2 * kDQK) + cc * 16;
          v[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds_kv) const {
#pragma unroll
    for (int it = 0; it < kPerThread; ++it) {
      const int c = threadIdx.x + it * kThreads;
      if (c < kChunks) {
        const int r = c / kChunksPerRow, cc = c % kChunksPerRow;
        if constexpr (!kFp8) {
          *reinterpret_cast<u32x4*>(lds_kv + r * kRowStride + cc * 8) = v[it];
        } else {
          u32x2 a0 = e4m3x4_to_bf16x4(v[it].x), a1 = e4m3x4_to_bf16x4(v[it].y);
          u32x2 a2 = e4m3x4_to_bf16x4(v[it].z), a3 = e4m3x4_to_bf16x4(v[it].w);
          u32x4* dst = reinterpret_cast<u32x4*>(lds_kv + r * kRowStride + cc * 16);
          dst[0] = u32x4{a0.x, a0.y, a1.x, a1.y};
          dst[1] = u32x4{a2.x, a2.y, a3.x, a3.y};
        }
      }
    }
  }
};

// Online-softmax state of one wave: 16 heads (one per lane column) and their
// latent-space output o^T[d][head], d = 16*db + 4*(lane/16) + r.
struct HeadState {
  float m_run, l_run;
  f32x4 o[32];
};

__device__ __forceinline__ void init_state(HeadState& st) {
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
#pragma unroll
  for (int db = 0; db < 32; ++db) st.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Attends the wave's 16 heads over one staged 32-row tile (bf16 rows of
// kRowStride elements). rscale[r] is the row's scale (fp8), 1 (bf16), or
// negative for a skipped row.
template <bool kFp8>
__device__ __forceinline__ void attend_tile(const uint16_t* __restrict__ tile,
                                            const float* __restrict__ rscale, HeadState& st,
                                            const u32x4 (&qb)[18], float zscale, int lane) {
  const int n16 = lane & 15, g = lane >> 4;
  // logits^T for rows 16b + 4g + r
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint16_t* rowp = tile + (16 * b + n16) * kRowStride + 8 * g;
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      u32x4 av = *reinterpret_cast<const u32x4*>(rowp + 32 * s);
      acc[b] = mfma16x16x32(av, qb[s], acc[b]);
    }
  }
  float z[2][4], rsc[2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rs = rscale[16 * b + 4 * g + r];
      rsc[b][r] = rs;
      float v = acc[b][r] * zscale;
      if constexpr (kFp8) v *= rs;
      z[b][r] = rs < 0.0f ? -INFINITY : v;
      tmax = fmaxf(tmax, z[b][r]);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(st.m_run, tmax);
  const float alpha = (st.m_run == -INFINITY) ? (m_new == -INFINITY ? 1.0f : 0.0f)
                                              : __builtin_amdgcn_exp2f(st.m_run - m_new);
  float p[2][4];
  float psum = 0.0f;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e = (z[b][r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z[b][r] - m_new);
      psum += e;
      if constexpr (kFp8) e *= fmaxf(rsc[b][r], 0.0f);
      p[b][r] = e;
    }
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int db = 0; db < 32; ++db) st.o[db] *= alpha;
  }
  // probabilities as bf16 hi/lo B operands: k-slot 8g+i <-> row 4g+i (i<4), 16+4g+i-4
  uint32_t hi_b[8], lo_b[8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t h = f32_to_bf16_rne(p[b][r]);
      float rem = p[b][r] - __uint_as_float(h << 16);
      hi_b[4 * b + r] = h;
      lo_b[4 * b + r] = f32_to_bf16_rne(rem);
    }
  const u32x4 phi = {hi_b[0] | (hi_b[1] << 16), hi_b[2] | (hi_b[3] << 16),
                     hi_b[4] | (hi_b[5] << 16), hi_b[6] | (hi_b[7] << 16)};
  const u32x4 plo = {lo_b[0] | (lo_b[1] << 16), lo_b[2] | (lo_b[3] << 16),
                     lo_b[4] | (lo_b[5] << 16), lo_b[6] | (lo_b[7] << 16)};
  // transposed reads: lane s reads row 4(s/16) + (s%16)/4 [+16], columns 4(s%4) .. +3
  // of each 16-column block
  const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int tr_col = 4 * (lane & 3);
  const uint16_t* tr0 = tile + tr_row * kRowStride + tr_col;
  const uint16_t* tr1 = tr0 + 16 * kRowStride;
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr0 + 16 * db));
    s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr1 + 16 * db));
    u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
    const u32x4 vt = {w0.x, w0.y, w1.x, w1.y};
    st.o[db] = mfma16x16x32(vt, phi, st.o[db]);
    st.o[db] = mfma16x16x32(vt, plo, st.o[db]);
  }
}

// Writes a wave's result: the gated, normalised output when the token has one
// split, else the unnormalised partial plus (m, l).
__device__ __forceinline__ void finish(const AttnArgs& a, HeadState& st, int t, int split,
                                       int head, int lane) {
  const int g = lane >> 4;
  float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t th = (int64_t)t * kHeads + head;
  if (a.splits == 1) {
    const float gs = gate_factor(a.gate, th);
    const float inv = l_tot > 0.0f ? gs / l_tot : 0.0f;
    float* dst = a.out + th * kDLatent + 4 * g;
#pragma unroll
    for (int db = 0; db < 32; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = st.o[db] * inv;
    if (a.lse && g == 0) a.lse[th] = l_tot > 0.0f ? (st.m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    // The split's output normalised by its exp-sum is a convex combination of
    // value rows; divided by its largest magnitude it lies in [-1, 1] and is
    // stored as fp16 (relative rounding 2^-11), with the scale kept in fp32.
    // Layout [token][split][column block db][head][16 columns]: for one db the
    // wave stores one contiguous 512-byte block.
    const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float amax = 0.0f;
#pragma unroll
    for (int db = 0; db < 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(st.o[db][r]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    amax *= inv_l;
    const float scale = amax > 0.0f ? amax : 1.0f;
    const float k = inv_l / scale;
    const int64_t ts = (int64_t)t * a.splits + split;
    uint16_t* dst = a.part_o + ts * kHeads * kDLatent + head * 16 + 4 * g;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const f32x4 v = st.o[db] * k;
      u32x2 packed;
      packed.x = pack_f16x2(v[0], v[1]);
      packed.y = pack_f16x2(v[2], v[3]);
      *reinterpret_cast<u32x2*>(dst + db * (kHeads * 16)) = packed;
    }
    if (g == 0) {
      float* ml = a.part_ml + 4 * (ts * kHeads + head);
      ml[0] = st.m_run;
      ml[1] = l_tot;
      ml[2] = scale;
      ml[3] = scale;
    }
  }
}

__device__ __forceinline__ void load_query(const AttnArgs& a, int t, int head, int lane,
                                           u32x4 (&qb)[18]) {
  const int g = lane >> 4;
  const uint16_t* q = a.q_abs + ((int64_t)t * kHeads + head) * kDQK;
#pragma unroll
  for (int s = 0; s < 18; ++s) qb[s] = *reinterpret_cast<const u32x4*>(q + 32 * s + 8 * g);
}

// bf16 rows, staged straight from HBM into LDS: a workgroup issues every load
// of up to kSuperRows rows at once (buffer_load ... lds), waits once, then
// attends the staged tiles. LDS row r of tile i starts at 16-byte unit
// 73*r of the tile's region (72 units of data + 1 of padding).
constexpr int kSuperTiles = 4;
constexpr int kSuperRows = kSuperTiles * kAttnTileRows;      // 128
constexpr int kUnitsPerRow = kRowStride * 2 / 16;            // 73
constexpr int kTileLoads = (kAttnTileRows * kUnitsPerRow + 63) / 64;  // 37 wave loads
constexpr int kTileRegion = kTileLoads * 64 * 16;            // 37888 B

__global__ __launch_bounds__(kThreads) void attn_bf16_direct_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kSuperTiles * kTileRegion];
  __shared__ int32_t lds_idx[kSuperRows];
  __shared__ float lds_rscale[kSuperRows];
  const int t = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int head = 16 * wave + (lane & 15);
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  const int32_t* idx_row = a.indices + (int64_t)t * a.k;
  const int j_begin = split * a.rows_per_split;
  const int j_end = min(a.k, j_begin + a.rows_per_split);

  u32x4 qb[18];
  load_query(a, t, head, lane, qb);
  HeadState st;
  init_state(st);
  const float zscale = a.sm_scale * kLog2e;
  // rows of this token's sequence; out-of-range offsets read as zeros
  const uint32_t seq_bytes = (uint32_t)max(n, 0) * (2u * kDQK);
  const __amdgpu_buffer_rsrc_t rows = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.kv + base * 2 * kDQK), (short)0, (int)seq_bytes, 0x00020000);

  for (int j0 = j_begin; j0 < j_end; j0 += kSuperRows) {
    const int nrows = min(kSuperRows, j_end - j0);
    const int ntiles = (nrows + kAttnTileRows - 1) / kAttnTileRows;
    __syncthreads();  // the previous super-tile is fully consumed
    if (threadIdx.x < kSuperRows) {
      const int j = j0 + threadIdx.x;
      const int idx = j < j_end ? idx_row[j] : -1;
      const bool ok = idx >= 0 && idx < n;
      lds_idx[threadIdx.x] = ok ? idx : -1;
      lds_rscale[threadIdx.x] = ok ? 1.0f : -1.0f;
    }
    __syncthreads();
    for (int i = 0; i < ntiles; ++i) {
      // offsets of this wave's loads first (LDS index reads batched), then the loads
      constexpr int kPerWave = (kTileLoads + kThreads / 64 - 1) / (kThreads / 64);
      int offs[kPerWave];
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) {
        const int l = wave + q * (kThreads / 64);
        const int u = l * 64 + lane;
        const int r = u / kUnitsPerRow, c = u - r * kUnitsPerRow;
        int off = (int)seq_bytes;  // out of range: zeros
        if (l < kTileLoads && r < kAttnTileRows && c < kUnitsPerRow - 1) {
          const int idx = lds_idx[i * kAttnTileRows + r];
          if (idx >= 0) off = idx * (2 * kDQK) + c * 16;
        }
        offs[q] = off;
      }
#pragma unroll
      for (int q = 0; q < kPerWave; ++q) {
        const int l = wave + q * (kThreads / 64);
        if (l < kTileLoads)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rows, (__attribute__((address_space(3))) void*)(lds + i * kTileRegion + l * 1024), 16,
              offs[q], 0, 0, kNonTemporal);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = 0; i < ntiles; ++i)
      attend_tile<false>(reinterpret_cast<const uint16_t*>(lds + i * kTileRegion),
                         lds_rscale + i * kAttnTileRows, st, qb, zscale, lane);
  }
  finish(a, st, t, split, head, lane);
}

// ---------------------------------------------------------------------------
// bf16 rows, 8 waves in pairs. Wave w owns heads 16*(w%4) .. +15 and one half
// h = w/4 of the work:
//   logits: dims 288h .. 288h+287 (9 of the 18 k-steps); the two waves of a
//           pair swap their partial logits through LDS and add them (fp32
//           addition commutes, so both hold identical logits);
//   output: latent columns 256h .. 256h+255.
// So each wave holds 9 query k-steps (36 VGPRs) and 16 output blocks (64),
// two waves run per SIMD, and the LDS traffic and MFMA count per tile are the
// same as with four whole waves.
// Rows stream straight from HBM into LDS (buffer_load ... lds): a super-tile
// of three 32-row tiles is requested at once, and each tile is consumed as
// soon as its own loads have landed. Every wave issues exactly five 1 KiB
// loads per tile (units past the 32 rows read zeros into the region's tail),
// so the per-tile waits are fixed counts.
constexpr int kPairThreads = 512;
constexpr int kPairWaves = kPairThreads / 64;
constexpr int kPairTiles = 3;                                     // tiles per super-tile
constexpr int kPairRows = kPairTiles * kAttnTileRows;             // 96
constexpr int kPairLoads = 5;                                     // 1 KiB loads per wave per tile
constexpr int kPairRegion = kPairWaves * kPairLoads * 1024;       // 40960 B per tile
static_assert(kPairWaves * kPairLoads * 64 >= kAttnTileRows * kUnitsPerRow, "tile fits its loads");

struct HalfState {
  float m_run, l_run;
  f32x4 o[16];
};

__device__ __forceinline__ void attend_tile_half(const uint16_t* __restrict__ tile,
                                                 const float* __restrict__ rscale,
                                                 float* __restrict__ xbuf, HalfState& st,
                                                 const u32x4 (&qb)[9], float zscale, int lane,
                                                 int wave, int half) {
  const int n16 = lane & 15, g = lane >> 4;
  // partial logits^T over this half's 9 k-steps; two chains per row block
  f32x4 acc[2][2] = {};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint16_t* rowp = tile + (16 * b + n16) * kRowStride + 8 * g + 288 * half;
#pragma unroll
    for (int s = 0; s < 9; ++s) {
      u32x4 av = *reinterpret_cast<const u32x4*>(rowp + 32 * s);
      acc[b][s & 1] = mfma16x16x32(av, qb[s], acc[b][s & 1]);
    }
  }
  f32x4 part0 = acc[0][0] + acc[0][1], part1 = acc[1][0] + acc[1][1];
  f32x4* mine = reinterpret_cast<f32x4*>(xbuf + (wave * 64 + lane) * 8);
  mine[0] = part0;
  mine[1] = part1;
  __syncthreads();
  const f32x4* other = reinterpret_cast<const f32x4*>(xbuf + ((wave ^ 4) * 64 + lane) * 8);
  const f32x4 full[2] = {part0 + other[0], part1 + other[1]};

  float z[2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rs = rscale[16 * b + 4 * g + r];
      z[b][r] = rs < 0.0f ? -INFINITY : full[b][r] * zscale;
      tmax = fmaxf(tmax, z[b][r]);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(st.m_run, tmax);
  const float alpha = (st.m_run == -INFINITY) ? (m_new == -INFINITY ? 1.0f : 0.0f)
                                              : __builtin_amdgcn_exp2f(st.m_run - m_new);
  float p[2][4];
  float psum = 0.0f;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = (z[b][r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z[b][r] - m_new);
      psum += e;
      p[b][r] = e;
    }
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int db = 0; db < 16; ++db) st.o[db] *= alpha;
  }
  uint32_t hi_b[8], lo_b[8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t h = f32_to_bf16_rne(p[b][r]);
      hi_b[4 * b + r] = h;
      lo_b[4 * b + r] = f32_to_bf16_rne(p[b][r] - __uint_as_float(h << 16));
    }
  const u32x4 phi = {hi_b[0] | (hi_b[1] << 16), hi_b[2] | (hi_b[3] << 16),
                     hi_b[4] | (hi_b[5] << 16), hi_b[6] | (hi_b[7] << 16)};
  const u32x4 plo = {lo_b[0] | (lo_b[1] << 16), lo_b[2] | (lo_b[3] << 16),
                     lo_b[4] | (lo_b[5] << 16), lo_b[6] | (lo_b[7] << 16)};
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

__device__ __forceinline__ void finish_half(const AttnArgs& a, HalfState& st, int t, int split,
                                            int head, int lane, int half) {
  const int g = lane >> 4;
  float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
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
  // normalised, scaled fp16 partial (see finish); one scale per half
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float amax = 0.0f;
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(st.o[db][r]));
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  amax *= inv_l;
  const float scale = amax > 0.0f ? amax : 1.0f;
  const float k = inv_l / scale;
  const int64_t ts = (int64_t)t * a.splits + split;
  uint16_t* dst = a.part_o + ts * kHeads * kDLatent + 16 * half * (kHeads * 16) + head * 16 + 4 * g;
#pragma unroll
  for (int db = 0; db < 16; ++db) {
    const f32x4 v = st.o[db] * k;
    u32x2 packed;
    packed.x = pack_f16x2(v[0], v[1]);
    packed.y = pack_f16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(dst + db * (kHeads * 16)) = packed;
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

__global__ __launch_bounds__(kPairThreads) void attn_bf16_pair_kernel(AttnArgs a) {
  // one LDS object per tile, so the compiler's waits for a tile's direct loads
  // cover that tile only
  __shared__ __attribute__((aligned(16))) uint8_t lds_t0[kPairRegion];
  __shared__ __attribute__((aligned(16))) uint8_t lds_t1[kPairRegion];
  __shared__ __attribute__((aligned(16))) uint8_t lds_t2[kPairRegion];
  static_assert(kPairTiles == 3, "three tile objects");
  __shared__ __attribute__((aligned(16))) float xbuf[kPairWaves * 64 * 8];
  __shared__ int32_t lds_idx[kPairRows];
  __shared__ float lds_rscale[kPairRows];
  const int t = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = wave >> 2;
  const int head = 16 * (wave & 3) + (lane & 15);
  const int g = lane >> 4;
  int64_t base;
  int n;
  a.batch.token(t, base, n);
  const int32_t* idx_row = a.indices + (int64_t)t * a.k;
  const int j_begin = split * a.rows_per_split;
  const int j_end = min(a.k, j_begin + a.rows_per_split);

  u32x4 qb[9];
  {
    const uint16_t* q = a.q_abs + ((int64_t)t * kHeads + head) * kDQK + 288 * half + 8 * g;
#pragma unroll
    for (int s = 0; s < 9; ++s) qb[s] = *reinterpret_cast<const u32x4*>(q + 32 * s);
  }
  HalfState st;
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
#pragma unroll
  for (int db = 0; db < 16; ++db) st.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float zscale = a.sm_scale * kLog2e;
  const uint32_t seq_bytes = (uint32_t)max(n, 0) * (2u * kDQK);
  const __amdgpu_buffer_rsrc_t rows = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.kv + base * 2 * kDQK), (short)0, (int)seq_bytes, 0x00020000);

  for (int j0 = j_begin; j0 < j_end; j0 += kPairRows) {
    const int ntiles = min(kPairTiles, (j_end - j0 + kAttnTileRows - 1) / kAttnTileRows);
    __syncthreads();  // the previous super-tile is fully consumed
    if (threadIdx.x < kPairRows) {
      const int j = j0 + threadIdx.x;
      const int idx = j < j_end ? idx_row[j] : -1;
      const bool ok = idx >= 0 && idx < n;
      lds_idx[threadIdx.x] = ok ? idx : -1;
      lds_rscale[threadIdx.x] = ok ? 1.0f : -1.0f;
    }
    __syncthreads();
    // every wave issues kPairLoads loads for each of the kPairTiles tiles
#pragma unroll
    for (int i = 0; i < kPairTiles; ++i) {
      int offs[kPairLoads];
#pragma unroll
      for (int q = 0; q < kPairLoads; ++q) {
        const int u = (wave + q * kPairWaves) * 64 + lane;
        const int r = u / kUnitsPerRow, c = u - r * kUnitsPerRow;
        int off = (int)seq_bytes;  // out of range: zeros
        if (r < kAttnTileRows && c < kUnitsPerRow - 1) {
          const int idx = lds_idx[i * kAttnTileRows + r];
          if (idx >= 0) off = idx * (2 * kDQK) + c * 16;
        }
        offs[q] = off;
      }
      uint8_t* region = i == 0 ? lds_t0 : (i == 1 ? lds_t1 : lds_t2);
#pragma unroll
      for (int q = 0; q < kPairLoads; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rows,
            (__attribute__((address_space(3))) void*)(region + (wave + q * kPairWaves) * 1024),
            16, offs[q], 0, 0, kNonTemporal);
    }
    // consume each tile once its own loads have landed
#pragma unroll
    for (int i = 0; i < kPairTiles; ++i) {
      if (i >= ntiles) break;
      if (i == 0) __builtin_amdgcn_s_waitcnt(kVmcntWait[0]);
      else if (i == 1) __builtin_amdgcn_s_waitcnt(kVmcntWait[1]);
      else __builtin_amdgcn_s_waitcnt(kVmcntWait[2]);
      __syncthreads();
      const uint8_t* region = i == 0 ? lds_t0 : (i == 1 ? lds_t1 : lds_t2);
      attend_tile_half(reinterpret_cast<const uint16_t*>(region), lds_rscale + i * kAttnTileRows,
                       xbuf, st, qb, zscale, lane, wave, half);
    }
  }
  finish_half(a, st, t, split, head, lane, half);
}

// Rows staged through registers one tile ahead (fp8 rows are widened to bf16
// on the way into LDS).
template <bool kFp8>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_kv[kAttnTileRows * kRowStride];
  __shared__ float lds_rscale[kAttnTileRows];   // row scale, or -1 for a skipped row
  const int t = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int head = 16 * wave + (lane & 15);
  int64_t base;
  int n;
  a.batch.token(t, base, n);

  const int32_t* idx_row = a.indices + (int64_t)t * a.k;
  const int j_begin = split * a.rows_per_split;
  const int j_end = min(a.k, j_begin + a.rows_per_split);
  const int ntiles = j_end > j_begin ? (j_end - j_begin + kAttnTileRows - 1) / kAttnTileRows : 0;

  u32x4 qb[18];
  load_query(a, t, head, lane, qb);
  HeadState st;
  init_state(st);
  const float zscale = a.sm_scale * kLog2e;

  TileLoader<kFp8> ld;
  if (ntiles > 0) ld.load(a, idx_row, j_begin, j_end, base, n);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int jt = j_begin + tile * kAttnTileRows;
    __syncthreads();  // previous tile fully consumed
    ld.store(lds_kv);
    if (threadIdx.x < kAttnTileRows) {
      const int j = jt + threadIdx.x;
      const int idx = j < j_end ? idx_row[j] : -1;
      float rs = -1.0f;
      if (idx >= 0 && idx < n) rs = kFp8 ? a.kv_scale[base + idx] : 1.0f;
      lds_rscale[threadIdx.x] = rs;
    }
    __syncthreads();
    if (tile + 1 < ntiles) ld.load(a, idx_row, jt + kAttnTileRows, j_end, base, n);
    attend_tile<kFp8>(lds_kv, lds_rscale, st, qb, zscale, lane);
  }
  finish(a, st, t, split, head, lane);
}

// Merges the split partials by log-sum-exp, then gates. One workgroup per
// (column block db, token): thread j takes head j/4 and columns
// 16*db + 4*(j%4) .. +3; for each split it reads one contiguous 2 KiB block.
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  const int db = blockIdx.x, t = blockIdx.y;
  const int h = threadIdx.x >> 2, q = threadIdx.x & 3;
  const int S = a.splits;
  const int64_t th = (int64_t)t * kHeads + h;
  const float* ml = a.part_ml + 4 * ((int64_t)t * S * kHeads + h);   // stride 4*kHeads per split
  const int sc = 2 + (db >= 16);                                       // scale of this column half
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[4 * kHeads * s]);
  const uint16_t* po = a.part_o + (int64_t)t * S * kHeads * kDLatent + db * (kHeads * 16) + h * 16 + 4 * q;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 4) {
      u32x2 v[4];
      float wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = min(s0 + u, S - 1);
        v[u] = *reinterpret_cast<const u32x2*>(po + (int64_t)s * kHeads * kDLatent);
        const float ms = ml[4 * kHeads * s];
        const float w = (s0 + u >= S || ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
        const float ls = ml[4 * kHeads * s + 1] * w;
        L += ls;
        wv[u] = ls * ml[4 * kHeads * s + sc];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x2 lo = unpack_f16x2(v[u].x), hi = unpack_f16x2(v[u].y);
        acc += f32x4{lo.x, lo.y, hi.x, hi.y} * wv[u];
      }
    }
  }
  const float gs = gate_factor(a.gate, th);
  const float inv = L > 0.0f ? gs / L : 0.0f;
  *reinterpret_cast<f32x4*>(a.out + th * kDLatent + 16 * db + 4 * q) = acc * inv;
  if (a.lse && db == 0 && q == 0) a.lse[th] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, bool fp8, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid(a.splits, a.num_tokens);
  if (fp8) attn_kernel<true><<<grid, kThreads, 0, s>>>(a);
  else attn_bf16_pair_kernel<<<grid, kPairThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t s) {
  if (a.num_tokens == 0 || a.splits == 1) return hipSuccess;
  combine_kernel<<<dim3(kDLatent / 16, a.num_tokens), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
