// Output epilogue after the gate: the per-head value up-projection
// u[t,h,:] = W_UV[h] . o[t,h,:] (512 -> 128) and the output projection
// y[t,:] = W_O . u[t,:] (64 x 128 -> d_model).
// Sources: A.X K2 fact sheet (archdb): value dimension per head 128, hidden
// state 7,168, a head-specific gate on the attention output before o_proj.
//
// Both steps are C = A . B^T with A fp32 activations [M x K] and B bf16
// weights [N x K] (the row-major weight of a linear layer): the up-projection
// is 64 such products, one per head, through strides; the output projection is
// one. Mapping onto gfx950: a workgroup of 4 waves takes 16 rows of A and 64
// columns of C, 16 per wave, over one split of K. For each 256-wide chunk of K
// the workgroup stages A's 16 x 256 block in LDS as a bf16 hi/lo pair
// (a = hi + lo to about 16 bits), and each wave streams its 16 weight rows
// from memory straight into v_mfma_f32_16x16x32_bf16 B operands, two MFMAs per
// k-step (hi and lo). The k order inside a chunk is permuted the same way on
// both sides so that two consecutive k-steps of a lane read 32 contiguous
// bytes of its weight row: each pair of load instructions covers whole 128-byte
// lines. With several splits of K the partial sums go to a workspace and
// proj_reduce_kernel adds them in split order, so results do not depend on
// scheduling.
#include "sga_kernels.h"

namespace sga {
namespace {

constexpr int kProjThreads = 256;
constexpr int kProjStride = kProjChunk + 8;   // bf16 per LDS row (16-byte pad)

// k offset, inside a chunk, of the 8 elements lane group g holds at k-step s
__device__ __forceinline__ int proj_k(int s, int g) { return 64 * (s >> 1) + 16 * g + 8 * (s & 1); }

__global__ __launch_bounds__(kProjThreads) void proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[2][kProjRows][kProjStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[2][kProjRows][kProjStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int bz = blockIdx.z;
  const int batch = bz / a.splits, split = bz % a.splits;
  const int m0 = blockIdx.y * kProjRows;
  const int n = blockIdx.x * kProjCols + 16 * wave + n16;   // this lane's weight row
  const int chunks = a.K / kProjChunk / a.splits;
  const int k_begin = split * chunks * kProjChunk;
  const float* A = a.a + (int64_t)batch * a.a_batch;
  const uint16_t* B = a.b + (int64_t)batch * a.b_batch + (int64_t)n * a.ldb + k_begin;

  // A staging: thread x loads row x/16 of the block, k = 16*(x%16) .. +15
  const int am = threadIdx.x >> 4, ak = 16 * (threadIdx.x & 15);
  const bool arow = m0 + am < a.M;
  const float* Ap = A + (int64_t)(arow ? m0 + am : 0) * a.lda + k_begin + ak;
  f32x4 av[4];
  auto load_a = [&](int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      av[j] = arow ? *reinterpret_cast<const f32x4*>(Ap + c * kProjChunk + 4 * j) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto store_a = [&](int buf) {
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x0 = av[j >> 1][2 * (j & 1)], x1 = av[j >> 1][2 * (j & 1) + 1];
      const uint32_t h0 = f32_to_bf16_rne(x0), h1 = f32_to_bf16_rne(x1);
      hi[j] = h0 | (h1 << 16);
      lo[j] = f32_to_bf16_rne(x0 - __uint_as_float(h0 << 16)) |
              (f32_to_bf16_rne(x1 - __uint_as_float(h1 << 16)) << 16);
    }
    u32x4* ph = reinterpret_cast<u32x4*>(&lds_hi[buf][am][ak]);
    u32x4* pl = reinterpret_cast<u32x4*>(&lds_lo[buf][am][ak]);
    ph[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    ph[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
    pl[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    pl[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
  };
  // this lane's B operands of one chunk (8 k-steps)
  u32x4 bq[2][8];
  auto load_b = [&](u32x4 (&dst)[8], int c) {
    const uint16_t* p = B + c * kProjChunk;
#pragma unroll
    for (int s = 0; s < 8; ++s) dst[s] = *reinterpret_cast<const u32x4*>(p + proj_k(s, g));
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4 (&bs)[8], int buf) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k = proj_k(s, g);
      const u32x4 ahi = *reinterpret_cast<const u32x4*>(&lds_hi[buf][n16][k]);
      const u32x4 alo = *reinterpret_cast<const u32x4*>(&lds_lo[buf][n16][k]);
      acc = mfma16x16x32(ahi, bs[s], acc);
      acc = mfma16x16x32(alo, bs[s], acc);
    }
  };

  load_a(0);
  load_b(bq[0], 0);
  if (chunks > 1) load_b(bq[1], 1);
  store_a(0);
  if (chunks > 1) load_a(1);
  __syncthreads();
  // chunk c: its weights are in bq[c & 1], its A block in LDS buffer c & 1;
  // the A block of chunk c + 1 is in registers and goes to the other buffer
  for (int c = 0; c < chunks; c += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cc = c + h;
      if (cc < chunks) {
        compute(bq[h], h);
        if (cc + 2 < chunks) load_b(bq[h], cc + 2);
        if (cc + 1 < chunks) {
          store_a(h ^ 1);
          if (cc + 2 < chunks) load_a(cc + 2);
        }
        __syncthreads();
      }
    }
  }

  // acc[r] = C[m0 + 4g + r][column n of this lane's 16]
  const int col = blockIdx.x * kProjCols + 16 * wave + n16;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + 4 * g + r;
    if (m < a.M) {
      if (a.splits == 1)
        a.c[(int64_t)batch * a.c_batch + (int64_t)m * a.ldc + col] = acc[r];
      else
        a.part[(((int64_t)split * a.batch + batch) * a.M + m) * a.N + col] = acc[r];
    }
  }
}

// C[b][m][n] = sum over splits s, in order, of part[s][b][m][n].
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjArgs a) {
  const int64_t per = (int64_t)a.batch * a.M * a.N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < per;
       i += (int64_t)gridDim.x * blockDim.x) {
    float sum = 0.0f;
    for (int s = 0; s < a.splits; ++s) sum += a.part[(int64_t)s * per + i];
    const int64_t b = i / ((int64_t)a.M * a.N);
    const int64_t r = i - b * a.M * a.N;
    const int64_t m = r / a.N, nn = r - m * a.N;
    a.c[b * a.c_batch + m * a.ldc + nn] = sum;
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const dim3 grid(a.N / kProjCols, (a.M + kProjRows - 1) / kProjRows, a.batch * a.splits);
  proj_kernel<<<grid, kProjThreads, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t per = (int64_t)a.batch * a.M * a.N;
  const int64_t blocks = (per + 255) / 256;
  proj_reduce_kernel<<<(unsigned)(blocks < 2048 ? blocks : 2048), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
