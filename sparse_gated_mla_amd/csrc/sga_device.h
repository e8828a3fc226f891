// Device-side helpers shared by the SGA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sga {

// ---------------------------------------------------------------- vector types
// bf16 data travels as 16-bit integers. It is bit-cast to __bf16 vectors only
// at the MFMA call.
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeads = 64;
constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kDLatent = 512;
constexpr int kDQK = 576;

// ---------------------------------------------------------------- MFMA
// D(32x32) += A(32x16) * B(16x32). Lane l holds A[l%32][8*(l/32)+i] and
// B[8*(l/32)+i][l%32] (i = 0..7). Accumulator register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16). Lane l holds A[l%16][8*(l/16)+i] and
// B[8*(l/16)+i][l%16]. Accumulator register r holds D[4*(l/16)+r][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- buffer loads
// A gfx9 raw buffer resource over [p, p + bytes) (32-bit data format, no
// swizzle): loads past the end return zeros, and offsets are 32-bit.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

// ---------------------------------------------------------------- conversions
// Four OCP E4M3FN bytes -> four bf16, packed two per dword: the scaled
// conversion (v_cvt_scalef32_pk_bf16_fp8) with scale 1, two instructions for
// four values. Exact: every E4M3FN value, subnormals included, is a bf16 normal.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t packed) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, true));
  return r;
}

// The fp32 value of an E8M0 block exponent e: 2^(e - 127) (e = 0 is the
// subnormal 2^-127). e = 255 (NaN) is not a valid input.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

// Four OCP E4M3FN bytes times a power-of-two block scale -> four bf16, packed
// two per dword (v_cvt_scalef32_pk_bf16_fp8; exact whenever the products are
// bf16 normals or zero, i.e. for block scales >= 2^-117).
__device__ __forceinline__ u32x2 e4m3x4_scaled_to_bf16x4(uint32_t packed, float scale) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, scale, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, scale, true));
  return r;
}

// Eight OCP E2M1 nibbles (element 2i in the low nibble of byte i) times a
// power-of-two block scale -> eight bf16 (v_cvt_scalef32_pk_bf16_fp4; exact
// for block scales >= 2^-125).
__device__ __forceinline__ u32x4 e2m1x8_scaled_to_bf16x8(uint32_t packed, float scale) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 3))};
}

// Two fp32 -> two bf16 packed low then high, round to nearest even
// (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// The bf16 hi/lo pair of two fp32 values x0, x1: x = hi + lo to about 16
// significant bits. Returns the packed hi pair and stores the packed lo pair.
__device__ __forceinline__ uint32_t split_bf16x2(float x0, float x1, uint32_t& lo) {
  const uint32_t hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
  return hi;
}

// The max and the sum of x over the lane pairs (l, l ^ 16) and (l, l ^ 32):
// v_permlane16_swap / v_permlane32_swap hand each lane both values of its
// pair, in either order, without an LDS round trip.
__device__ __forceinline__ f32x2 pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor16(float x) { const f32x2 p = pair16(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float max_xor32(float x) { const f32x2 p = pair32(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum_xor16(float x) { const f32x2 p = pair16(x); return p.x + p.y; }
__device__ __forceinline__ float sum_xor32(float x) { const f32x2 p = pair32(x); return p.x + p.y; }

// Two fp32 -> two IEEE fp16 (round to nearest even), packed low then high.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 h;
  h.x = (_Float16)lo;
  h.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t u) {
  const f16x2 h = __builtin_bit_cast(f16x2, u);
  return f32x2{(float)h.x, (float)h.y};
}

// ---------------------------------------------------------------- radix keys
// Order-preserving map from fp32 scores to uint32 keys: a larger score gives a
// larger key. -0.0 maps to the key of +0.0, so they tie.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Radix digits of the select: 12 + 12 + 8 key bits.
constexpr int kDigit1Bits = 12;  // key bits 31..20
constexpr int kDigit2Bits = 12;  // key bits 19..8
constexpr int kDigit3Bits = 8;   // key bits 7..0
constexpr int kHist1 = 1 << kDigit1Bits;
constexpr int kHist2 = 1 << kDigit2Bits;
constexpr int kHist3 = 1 << kDigit3Bits;
constexpr uint32_t kHistOverflow = 0xffffffffu;   // list slot header: the bins did not fit

// ---------------------------------------------------------------- visibility
// Visible rows of a token, clamped so inconsistent metadata never leaves the
// caches or the output rows.
__device__ __forceinline__ int visible_rows(int pos, int seq_len, int max_len,
                                            int64_t seq_start, int64_t cache_rows) {
  int64_t n = (int64_t)pos + 1;
  if (n > seq_len) n = seq_len;
  if (n > max_len) n = max_len;
  int64_t room = cache_rows - seq_start;
  if (seq_start < 0) room = 0;
  if (n > room) n = room;
  return n > 0 ? (int)n : 0;
}

// A load through the constant address space: data no kernel of the launch
// writes, such as the batch metadata. Uniform addresses become scalar loads.
template <class T>
__device__ __forceinline__ T load_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

struct BatchView {
  const int32_t* token_seq;
  const int32_t* token_pos;
  const int64_t* seq_start;
  const int32_t* seq_len;
  int32_t num_seqs;
  int32_t max_len;
  int64_t cache_rows;

  // Resolves token t: first flat row of its sequence and its visible row count.
  // Two rounds of loads at most, with no branch between them: the token's
  // sequence and position, then the sequence's start and length (read for
  // sequence 0 when the token's id is invalid, and then not used). With a
  // workgroup-uniform t these are scalar loads, which leave the vector memory
  // counter to loads the caller issued before.
  __device__ __forceinline__ void token(int t, int64_t& base, int& n) const {
    if (num_seqs <= 0) { base = 0; n = 0; return; }
    const int b = load_const(token_seq, t);
    const int pos = load_const(token_pos, t);
    const bool ok = b >= 0 && b < num_seqs;
    const int bc = ok ? b : 0;
    const int64_t start = load_const(seq_start, bc);
    const int len = load_const(seq_len, bc);
    base = ok ? start : 0;
    n = ok ? visible_rows(pos, len, max_len, start, cache_rows) : 0;
  }
};

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// The dispatcher deals workgroups to the chip's 8 XCDs round-robin by linear
// id, and each XCD has its own L2. This maps linear id b (of `total`) to an
// index whose consecutive values run on one XCD: XCD x gets indices
// x*per + min(x, rem) + 0, 1, ..., so workgroups that share input (the splits
// of one token share its query) read it through one L2.
__device__ __forceinline__ int xcd_grouped(int b, int total) {
  constexpr int kXcds = 8;
  const int per = total / kXcds, rem = total % kXcds;
  const int x = b % kXcds, j = b / kXcds;
  return x * per + min(x, rem) + j;
}

// ---------------------------------------------------------------- timeline build
// Built with SGA_TIMELINE defined (`python -m sparse_gated_mla_amd.build
// --timeline`, into a library of its own), the step's kernels record, per
// workgroup, the 100 MHz real-time counter (s_memrealtime) at a few points and
// the workgroup's XCD and hardware ids, for the device-clock timeline that
// `bench.py --timeline` prints. Each source file that stamps holds its own
// record of 2^16 words, word 8s + k for point k of slot s (slots below 8,192;
// point 7 holds the ids: XCC_ID << 32 | HW_ID), and exports a reader and a
// clear (both synchronous copies, from or to a host buffer of 2^16 words). In the
// library that the path normally runs these expand to nothing.
#ifdef SGA_TIMELINE
#define SGA_TL_RECORD(tag)                                                                  \
  static __device__ uint64_t sga_tl_words[1 << 16];                                        \
  extern "C" __attribute__((visibility("default"))) int sga_tl_read_##tag(void* dst) {      \
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(sga_tl_words), sizeof(sga_tl_words), 0, \
                                    hipMemcpyDeviceToHost);                                \
  }                                                                                         \
  extern "C" __attribute__((visibility("default"))) int sga_tl_clear_##tag(const void* zeros) { \
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(sga_tl_words), zeros, sizeof(sga_tl_words), 0,   \
                                  hipMemcpyHostToDevice);                                     \
  }
#define SGA_TL_STAMP(slot, k)                                                 \
  do {                                                                        \
    const int sga_tl_slot = (slot);                                           \
    if (threadIdx.x == 0 && sga_tl_slot < 8192)                               \
      sga_tl_words[sga_tl_slot * 8 + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define SGA_TL_ID(slot)                                                                      \
  do {                                                                                       \
    const int sga_tl_slot = (slot);                                                          \
    if (threadIdx.x == 0 && sga_tl_slot < 8192)                                              \
      sga_tl_words[sga_tl_slot * 8 + 7] = ((uint64_t)__builtin_amdgcn_s_getreg(0x7814) << 32) | \
                                          (uint32_t)__builtin_amdgcn_s_getreg(0xF804);        \
  } while (0)
#else
#define SGA_TL_RECORD(tag)
#define SGA_TL_STAMP(slot, k) do {} while (0)
#define SGA_TL_ID(slot) do {} while (0)
#endif

}  // namespace sga
