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

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

template <bool kFp8>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_kv[kAttnTileRows * kRowStride];
  __shared__ float lds_rscale[kAttnTileRows];   // row scale, or -1 for a skipped row
  const int t = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int head = 16 * wave + n16;
  int64_t base;
  int n;
  a.batch.token(t, base, n);

  const int32_t* idx_row = a.indices + (int64_t)t * a.k;
  const int j_begin = split * a.rows_per_split;
  const int j_end = min(a.k, j_begin + a.rows_per_split);
  const int ntiles = j_end > j_begin ? (j_end - j_begin + kAttnTileRows - 1) / kAttnTileRows : 0;

  // absorbed query as the B operand: qb[s] = q[head][32s + 8g .. +7]
  u32x4 qb[18];
  const uint16_t* q = a.q_abs + ((int64_t)t * kHeads + head) * kDQK;
#pragma unroll
  for (int s = 0; s < 18; ++s) qb[s] = *reinterpret_cast<const u32x4*>(q + 32 * s + 8 * g);

  const float zscale = a.sm_scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  TileLoader<kFp8> ld;
  if (ntiles > 0) ld.load(a, idx_row, j_begin, j_end, base, n);

  // transposed-read addresses: lane s reads row (4(s/16) + (s%16)/4) [+16],
  // columns 4(s%4) .. +3 of each 16-column block
  const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int tr_col = 4 * (lane & 3);

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

    // logits^T for rows 16b + 4g + r
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint16_t* rowp = lds_kv + (16 * b + n16) * kRowStride + 8 * g;
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
        const float rs = lds_rscale[16 * b + 4 * g + r];
        rsc[b][r] = rs;
        float v = acc[b][r] * zscale;
        if constexpr (kFp8) v *= rs;
        z[b][r] = rs < 0.0f ? -INFINITY : v;
        tmax = fmaxf(tmax, z[b][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_run == -INFINITY) ? (m_new == -INFINITY ? 1.0f : 0.0f)
                                             : __builtin_amdgcn_exp2f(m_run - m_new);
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
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < 32; ++db) o[db] *= alpha;
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
    const uint16_t* tr0 = lds_kv + tr_row * kRowStride + tr_col;
    const uint16_t* tr1 = tr0 + 16 * kRowStride;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr0 + 16 * db));
      s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr1 + 16 * db));
      u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
      const u32x4 vt = {w0.x, w0.y, w1.x, w1.y};
      o[db] = mfma16x16x32(vt, phi, o[db]);
      o[db] = mfma16x16x32(vt, plo, o[db]);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t th = (int64_t)t * kHeads + head;
  if (a.splits == 1) {
    const float gs = gate_factor(a.gate, th);
    const float inv = l_tot > 0.0f ? gs / l_tot : 0.0f;
    float* dst = a.out + th * kDLatent + 4 * g;
#pragma unroll
    for (int db = 0; db < 32; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[db] * inv;
    if (a.lse && g == 0) a.lse[th] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t ps = ((int64_t)t * a.splits + split) * kHeads + head;
    float* dst = a.part_o + ps * kDLatent + 4 * g;
#pragma unroll
    for (int db = 0; db < 32; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[db];
    if (g == 0) {
      a.part_ml[2 * ps] = m_run;
      a.part_ml[2 * ps + 1] = l_tot;
    }
  }
}

// Merges the split partials of one (token, head) by log-sum-exp, then gates.
// One workgroup of 128 threads per (head, token); each thread owns 4 columns.
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, t = blockIdx.y;
  const int S = a.splits;
  const int64_t th = (int64_t)t * kHeads + h;
  const float* ml = a.part_ml + 2 * ((int64_t)t * S * kHeads + h);   // stride 2*kHeads per split
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * kHeads * s]);
  float L = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    const float* po = a.part_o + ((int64_t)t * S * kHeads + h) * kDLatent + 4 * threadIdx.x;
    for (int s = 0; s < S; ++s) {
      const float ms = ml[2 * kHeads * s];
      if (ms == -INFINITY) continue;
      const float wgt = __builtin_amdgcn_exp2f(ms - M);
      L += ml[2 * kHeads * s + 1] * wgt;
      acc += *reinterpret_cast<const f32x4*>(po + (int64_t)s * kHeads * kDLatent) * wgt;
    }
  }
  const float gs = gate_factor(a.gate, th);
  const float inv = L > 0.0f ? gs / L : 0.0f;
  *reinterpret_cast<f32x4*>(a.out + th * kDLatent + 4 * threadIdx.x) = acc * inv;
  if (a.lse && threadIdx.x == 0) a.lse[th] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, bool fp8, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid(a.splits, a.num_tokens);
  if (fp8) attn_kernel<true><<<grid, kThreads, 0, s>>>(a);
  else attn_kernel<false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t s) {
  if (a.num_tokens == 0 || a.splits == 1) return hipSuccess;
  combine_kernel<<<dim3(kHeads, a.num_tokens), 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
