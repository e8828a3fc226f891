// Output epilogue after the gate: the per-head value up-projection
// u[t,h,:] = W_UV[h] . o[t,h,:] (512 -> 128) and the output projection
// y[t,:] = W_O . u[t,:] (64 x 128 -> d_model).
// Sources: A.X K2 fact sheet (archdb): value dimension per head 128, hidden
// state 7,168, a head-specific gate on the attention output before o_proj.
//
// Both steps are C = A . B^T with A fp32 activations [M x K] and B bf16
// weights [N x K] (the row-major weight of a linear layer): the up-projection
// is 64 such products, one per head, through strides; the output projection is
// one. Mapping onto gfx950: a workgroup of 4 waves takes 16 * MB rows of A
// (MB = 1 for a few tokens, 4 from 32 tokens on) and 64 * NB columns of C
// (NB = 2 from 32 tokens on), 16 * NB per wave, over one split of K. For each chunk of K (256 wide, 128 when MB = 4)
// the workgroup stages A's block in LDS as a bf16 hi/lo pair (a = hi + lo to
// about 16 bits), and each wave streams its 16 weight rows from memory
// straight into v_mfma_f32_16x16x32_bf16 B operands; each B operand serves
// MB row blocks, two MFMAs each (hi and lo), so the weights are read once per
// 16 * MB rows. The k order inside a chunk is permuted the same way on both
// sides so that two consecutive k-steps of a lane read 32 contiguous bytes of
// its weight row: each pair of load instructions covers whole 128-byte lines.
// With several splits of K the partial sums go to a workspace and
// proj_reduce_kernel adds them in split order, so results do not depend on
// scheduling.
#include "sga_kernels.h"

namespace sga {
namespace {

constexpr int kProjThreads = 256;

// k offset, inside a chunk, of the 8 elements lane group g holds at k-step s
__device__ __forceinline__ int proj_k(int s, int g) { return 64 * (s >> 1) + 16 * g + 8 * (s & 1); }

template <int MB, int NB>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(ProjArgs a) {
  constexpr int kChunk = proj_chunk(MB);
  constexpr int kSteps = kChunk / 32;
  constexpr int kRows = kProjRows * MB;
  constexpr int kStride = kChunk + 8;                  // bf16 per LDS row (16-byte pad)
  constexpr int kPerThread = kRows * kChunk / kProjThreads;   // A floats each thread stages: 16 or 32
  constexpr int kThreadsPerRow = kChunk / kPerThread;
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[2][kRows][kStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[2][kRows][kStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int bz = blockIdx.z;
  const int batch = bz / a.splits, split = bz % a.splits;
  const int m0 = blockIdx.y * kRows;
  // this lane's weight row in column block 0; block j adds 64 * j
  const int n = blockIdx.x * (kProjCols * NB) + 16 * wave + n16;
  const int chunks = a.K / kChunk / a.splits;
  const int k_begin = split * chunks * kChunk;
  const float* A = a.a + (int64_t)batch * a.a_batch;
  const uint16_t* B = a.b + (int64_t)batch * a.b_batch + (int64_t)n * a.ldb + k_begin;
  const int64_t b_next = (int64_t)kProjCols * a.ldb;         // to column block j + 1

  // A staging: thread x loads row x / kThreadsPerRow of the block and
  // kPerThread consecutive k from kPerThread * (x % kThreadsPerRow)
  const int am = threadIdx.x / kThreadsPerRow, ak = kPerThread * (threadIdx.x % kThreadsPerRow);
  const bool arow = m0 + am < a.M;
  const float* Ap = A + (int64_t)(arow ? m0 + am : 0) * a.lda + k_begin + ak;
  f32x4 av[kPerThread / 4];
  auto load_a = [&](int c) {
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j)
      av[j] = arow ? *reinterpret_cast<const f32x4*>(Ap + c * kChunk + 4 * j) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kPerThread / 8; ++q) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hi[j] = split_bf16x2(av[2 * q + (j >> 1)][2 * (j & 1)], av[2 * q + (j >> 1)][2 * (j & 1) + 1], lo[j]);
      *reinterpret_cast<u32x4*>(&lds_hi[buf][am][ak + 8 * q]) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<u32x4*>(&lds_lo[buf][am][ak + 8 * q]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  };
  // this lane's B operands of one chunk, per column block
  u32x4 bq[2][NB][kSteps];
  auto load_b = [&](u32x4 (&dst)[NB][kSteps], int c) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint16_t* p = B + j * b_next + c * kChunk;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) dst[j][s] = *reinterpret_cast<const u32x4*>(p + proj_k(s, g));
    }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4 (&bs)[NB][kSteps], int buf) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int k = proj_k(s, g);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 ahi = *reinterpret_cast<const u32x4*>(&lds_hi[buf][16 * mb + n16][k]);
        const u32x4 alo = *reinterpret_cast<const u32x4*>(&lds_lo[buf][16 * mb + n16][k]);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc[mb][j] = mfma16x16x32(ahi, bs[j][s], acc[mb][j]);
          acc[mb][j] = mfma16x16x32(alo, bs[j][s], acc[mb][j]);
        }
      }
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

  // acc[mb][j][r] = C[m0 + 16 mb + 4g + r][n + 64 j]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mb + 4 * g + r;
        const int col = n + kProjCols * j;
        if (m < a.M) {
          if (a.splits == 1)
            a.c[(int64_t)batch * a.c_batch + (int64_t)m * a.ldc + col] = acc[mb][j][r];
          else
            a.part[(((int64_t)split * a.batch + batch) * a.M + m) * a.N + col] = acc[mb][j][r];
        }
      }
}

// The output projection for at most 16 rows (decode batches). Each wave
// streams 16 weight rows over the workgroup's K range, two 256-wide chunks of
// B operands in flight; the block of A over that range is split into its bf16
// hi/lo pair and staged in LDS once, after the first weight loads have gone
// out, so the weight stream runs with no barrier. Per column the K order, and
// the splits' order in proj_reduce_kernel, are those of proj_kernel<1, 1>.
constexpr int kVecThreads = 512;

__global__ __launch_bounds__(kVecThreads) void proj_vec_kernel(ProjArgs a) {
  constexpr int kChunk = 256;
  constexpr int kSteps = kChunk / 32;
  constexpr int kStride = kProjVecMaxK + 8;          // bf16 per LDS row (16-byte pad)
  constexpr int kUnits = kProjRows * kProjVecMaxK / 8;   // 8-float units of the largest block
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[kProjRows][kStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[kProjRows][kStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.y;
  const int kr = a.K / a.splits;   // this workgroup's K range: a multiple of kChunk, <= kProjVecMaxK
  const int chunks = kr / kChunk;
  const int k_begin = split * kr;
  const int n = blockIdx.x * kProjVecCols + 16 * wave + n16;
  const uint16_t* B = a.b + (int64_t)n * a.ldb + k_begin;

  u32x4 bq[2][kSteps];
  auto load_b = [&](u32x4 (&dst)[kSteps], int c) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) dst[s] = *reinterpret_cast<const u32x4*>(B + c * kChunk + proj_k(s, g));
  };
  load_b(bq[0], 0);
  if (chunks > 1) load_b(bq[1], 1);

  // A block: unit i holds row i / (kr / 8), floats 8 (i % (kr / 8)) .. +7;
  // rows past M are zeros
  const int per_row = kr / 8;
  const int units = kProjRows * per_row;
  f32x4 av[kUnits / kVecThreads][2];
#pragma unroll
  for (int q = 0; q < kUnits / kVecThreads; ++q) {
    const int i = q * kVecThreads + (int)threadIdx.x;
    const int m = i / per_row, c8 = i - m * per_row;
    const bool live = i < units && m < a.M;
    const float* p = a.a + (int64_t)(live ? m : 0) * a.lda + k_begin + 8 * c8;
    av[q][0] = live ? *reinterpret_cast<const f32x4*>(p) : f32x4{0.f, 0.f, 0.f, 0.f};
    av[q][1] = live ? *reinterpret_cast<const f32x4*>(p + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int q = 0; q < kUnits / kVecThreads; ++q) {
    const int i = q * kVecThreads + (int)threadIdx.x;
    if (i < units) {
      const int m = i / per_row, c8 = i - m * per_row;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hi[j] = split_bf16x2(av[q][j >> 1][2 * (j & 1)], av[q][j >> 1][2 * (j & 1) + 1], lo[j]);
      *reinterpret_cast<u32x4*>(&lds_hi[m][8 * c8]) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<u32x4*>(&lds_lo[m][8 * c8]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < chunks; c += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cc = c + h;
      if (cc < chunks) {
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const int k = cc * kChunk + proj_k(s, g);
          const u32x4 ahi = *reinterpret_cast<const u32x4*>(&lds_hi[n16][k]);
          const u32x4 alo = *reinterpret_cast<const u32x4*>(&lds_lo[n16][k]);
          acc = mfma16x16x32(ahi, bq[h][s], acc);
          acc = mfma16x16x32(alo, bq[h][s], acc);
        }
        if (cc + 2 < chunks) load_b(bq[h], cc + 2);
      }
    }
  }

  // acc[r] = C[4g + r][n]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g + r;
    if (m < a.M) {
      if (a.splits == 1)
        a.c[(int64_t)m * a.ldc + n] = acc[r];
      else
        a.part[((int64_t)split * a.M + m) * a.N + n] = acc[r];
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

void launch_proj_blocks(const ProjArgs& a, hipStream_t s) {
  const int mb = proj_row_blocks(a.M), nb = proj_col_blocks(a.M, a.N);
  const dim3 grid(a.N / (kProjCols * nb), (a.M + kProjRows * mb - 1) / (kProjRows * mb), a.batch * a.splits);
  if (mb == 4) {
    if (nb == 2) proj_kernel<4, 2><<<grid, kProjThreads, 0, s>>>(a);
    else proj_kernel<4, 1><<<grid, kProjThreads, 0, s>>>(a);
  } else {
    if (nb == 2) proj_kernel<1, 2><<<grid, kProjThreads, 0, s>>>(a);
    else proj_kernel<1, 1><<<grid, kProjThreads, 0, s>>>(a);
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const int kr = a.K / a.splits;
  if (proj_vec(a.M, a.N, a.batch) && kr * a.splits == a.K && kr % 256 == 0 && kr <= kProjVecMaxK) {
    proj_vec_kernel<<<dim3(a.N / kProjVecCols, a.splits), kVecThreads, 0, s>>>(a);
  } else {
    launch_proj_blocks(a, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t per = (int64_t)a.batch * a.M * a.N;
  const int64_t blocks = (per + 255) / 256;
  proj_reduce_kernel<<<(unsigned)(blocks < 2048 ? blocks : 2048), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sga
