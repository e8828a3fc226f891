// Cache append: the step just before the path in decode. Each token's new
// 576-wide latent row and 128-wide indexer key are written into row
// seq_start[b] + p of their caches, as bf16 (copied), as OCP E4M3FN with one
// fp32 scale per row, or as MX block-32 E4M3FN with one E8M0 exponent per 32
// consecutive elements (fact sheet, Training: MXFP8 E4M3, one scale per 32).
// Source: FP8 model card (nlp.com.ai, "A.X K2 FP8"): FP8 with dynamic, per-row
// activation scaling; fact sheet (archdb, "A.X K2"): per token the cache holds
// the 512 latent + 64 RoPE values and the 128-wide indexer key.
//
// fp8: scale = max|x| / 448 (binary32 division; 1 for a row of zeros), and each
// payload is x / scale rounded to the nearest E4M3FN value, ties to the even
// code, saturating at 448, the sign bit following x. The rounding is done from
// the format's definition: a value in binade [2^e, 2^(e+1)) (e >= -6) has code
// spacing 2^(e-3), below 2^-6 the spacing is 2^-9; scaling by the spacing is
// exact, rintf rounds to nearest even, and the result is re-encoded.
//
// MX: block exponent e - 127 = floor(log2 max|x|) - 8 (8 = exponent of 448),
// clamped to [-127, 127], e = 0 for a block of zeros (the Open Compute
// Project MX format's rule); each element is x * 2^(127 - e) (exact) encoded
// as above. With four-bit E2M1 elements the exponent is floor(log2 max|x|) - 2
// (6 = 1.5 * 2^2 is E2M1's largest value), the element spacing is 2^(e-1) in
// binade [2^e, 2^(e+1)) and 0.5 below 1, rounding is nearest-even, saturating
// at 6, and two elements share a byte, the lower-indexed one in the low nibble.
//
// Mapping: one workgroup of two waves per token; wave 0 writes the latent row
// (72 16-byte units, one or two per lane), wave 1 the indexer key (16 units).
#include "sga_kernels.h"

namespace sga {
namespace {

__device__ __forceinline__ uint32_t e4m3fn_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  int ea;
  frexpf(a, &ea);                       // a = f * 2^ea, f in [0.5, 1)
  const int eb = max(ea - 1, -6);       // binade exponent, subnormals share -6
  const float v = ldexpf(rintf(ldexpf(a, 3 - eb)), eb - 3);   // nearest code value
  if (v == 0.0f) return sign;
  int ev;
  frexpf(v, &ev);
  ev -= 1;                              // floor(log2 v)
  if (ev < -6) return sign | (uint32_t)ldexpf(v, 9);          // subnormal: v / 2^-9
  const uint32_t m = (uint32_t)ldexpf(v, 3 - ev) - 8u;        // v / 2^(ev-3) in [8, 16)
  return sign | ((uint32_t)(ev + 7) << 3) | m;
}

__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fminf(fabsf(x), 6.0f);
  int ea;
  frexpf(a, &ea);                       // a = f * 2^ea, f in [0.5, 1)
  const int eb = max(ea - 1, 0);        // binade exponent; below 1 the spacing stays 0.5
  const float v = ldexpf(rintf(ldexpf(a, 1 - eb)), eb - 1);   // nearest code value
  if (v == 0.0f) return sign;
  if (v < 1.0f) return sign | 1u;       // 0.5
  int ev;
  frexpf(v, &ev);
  ev -= 1;                              // floor(log2 v): 0, 1 or 2
  const uint32_t m = ldexpf(v, -ev) > 1.0f ? 1u : 0u;        // 1.5 * 2^ev
  return sign | ((uint32_t)(ev + 1) << 1) | m;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One row of `units` 16-byte units (8 bf16 each), lane l taking units l and l + 64.
// scale_out: the row's fp32 scale (kFmtFp8) or its E8M0 block exponents (kFmtMx).
template <int kUnits>
__device__ __forceinline__ void append_row(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                           void* __restrict__ scale_out, int fmt, int lane) {
  constexpr int kPer = (kUnits + 63) / 64;
  u32x4 v[kPer];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int u = lane + 64 * j;
    v[j] = u32x4{0u, 0u, 0u, 0u};
    if (u < kUnits) v[j] = *reinterpret_cast<const u32x4*>(src + 8 * u);
#pragma unroll
    for (int c = 0; c < 4; ++c) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[j][c])), fabsf(bf16_hi(v[j][c]))));
  }
  if (fmt == kFmtBf16) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int u = lane + 64 * j;
      if (u < kUnits) *reinterpret_cast<u32x4*>(dst + 16 * u) = v[j];
    }
    return;
  }
  if (fmt == kFmtMx || fmt == kFmtMx4) {
    const bool four = fmt == kFmtMx4;
    // a block of 32 elements is units 4b .. 4b+3: four neighbouring lanes
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int u = lane + 64 * j;
      float bmax = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) bmax = fmaxf(bmax, fmaxf(fabsf(bf16_lo(v[j][c])), fabsf(bf16_hi(v[j][c]))));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 1));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 2));
      int e = 0;
      if (bmax > 0.0f) {
        int ea;
        frexpf(bmax, &ea);                       // floor(log2 bmax) = ea - 1
        e = min(max(ea - 1 - (four ? 2 : 8), -127), 127) + 127;
      }
      if (u < kUnits) {
        if (four) {
          uint32_t out = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            out |= e2m1_encode(ldexpf(bf16_lo(v[j][c]), 127 - e)) << (8 * c);
            out |= e2m1_encode(ldexpf(bf16_hi(v[j][c]), 127 - e)) << (8 * c + 4);
          }
          *reinterpret_cast<uint32_t*>(dst + 4 * u) = out;
        } else {
          uint32_t b[8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            b[2 * c] = e4m3fn_encode(ldexpf(bf16_lo(v[j][c]), 127 - e));
            b[2 * c + 1] = e4m3fn_encode(ldexpf(bf16_hi(v[j][c]), 127 - e));
          }
          u32x2 out;
          out.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
          out.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
          *reinterpret_cast<u32x2*>(dst + 8 * u) = out;
        }
        if ((u & 3) == 0) static_cast<uint8_t*>(scale_out)[u >> 2] = (uint8_t)e;
      }
    }
    return;
  }
  amax = wave_max(amax);
  const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int u = lane + 64 * j;
    if (u < kUnits) {
      u32x2 out;
      uint32_t b[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        b[2 * c] = e4m3fn_encode(bf16_lo(v[j][c]) / scale);
        b[2 * c + 1] = e4m3fn_encode(bf16_hi(v[j][c]) / scale);
      }
      out.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      out.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
      *reinterpret_cast<u32x2*>(dst + 8 * u) = out;
    }
  }
  if (lane == 0) *static_cast<float*>(scale_out) = scale;
}

// Where row `row`'s scale goes: an fp32 per row, or width/32 E8M0 bytes per row.
__device__ __forceinline__ void* scale_row(void* base, int fmt, int64_t row, int width) {
  if (fmt == kFmtFp8) return static_cast<float*>(base) + row;
  if (fmt == kFmtMx || fmt == kFmtMx4) return static_cast<uint8_t*>(base) + row * (width / 32);
  return nullptr;
}

__global__ __launch_bounds__(128) void cache_append_kernel(CacheArgs a) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = a.batch.token_seq[t];
  if (b < 0 || b >= a.batch.num_seqs) return;
  const int p = a.batch.token_pos[t];
  if (p < 0 || p >= a.batch.seq_len[b]) return;
  const int64_t row = a.batch.seq_start[b] + p;
  if (row < 0 || row >= a.batch.cache_rows) return;
  if (wave == 0) {
    if (!a.latent || !a.kv) return;
    append_row<kDQK / 8>(a.latent + (int64_t)t * kDQK, a.kv + row * row_bytes(a.kv_fmt, kDQK),
                         scale_row(a.kv_scale, a.kv_fmt, row, kDQK), a.kv_fmt, lane);
  } else {
    if (!a.key || !a.k_idx) return;
    append_row<kIdxDim / 8>(a.key + (int64_t)t * kIdxDim,
                            a.k_idx + row * row_bytes(a.k_idx_fmt, kIdxDim),
                            scale_row(a.k_idx_scale, a.k_idx_fmt, row, kIdxDim), a.k_idx_fmt, lane);
  }
}

}  // namespace

hipError_t launch_cache_append(const CacheArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  cache_append_kernel<<<a.num_tokens, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
