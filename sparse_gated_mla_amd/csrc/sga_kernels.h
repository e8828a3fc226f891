// Internal launch interface between the C ABI (sga_api.hip) and the kernel
// translation units. Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sga_device.h"

namespace sga {

// Per-token top-k control block in the workspace, written by the first select
// workgroup of the token (16 bytes: the final stage reads it in one vector load).
struct TopkCtrl {
  uint32_t digit1;      // top 12 key bits of the k-th largest score
  uint32_t above1;      // scores whose top 12 key bits exceed digit1
  uint32_t visible;     // the token's visible positions n (written even when n <= k)
  uint32_t pad;
};

// Cache element formats (the values of sga_dtype).
constexpr int kFmtBf16 = 0;    // bf16 rows
constexpr int kFmtFp8 = 1;     // E4M3FN rows, one fp32 scale per row
constexpr int kFmtMx = 2;      // E4M3FN rows, one E8M0 exponent per 32 elements
constexpr int kFmtMx4 = 3;     // E2M1 rows (two per byte), one E8M0 exponent per 32 elements

// Cached bytes of a `width`-element row in format fmt (scales apart).
__host__ __device__ constexpr int row_bytes(int fmt, int width) {
  return fmt == kFmtBf16 ? 2 * width : fmt == kFmtMx4 ? width / 2 : width;
}

constexpr int kIndexerChunk = 2048;   // positions per indexer workgroup (bf16 keys)
// one-byte and four-bit keys: a workgroup takes twice the positions
// (measured: one round of workgroups streams fp8 keys best)
__host__ __device__ constexpr int indexer_chunk(bool fp8) { return fp8 ? 2 * kIndexerChunk : kIndexerChunk; }
constexpr int kSelectChunk = 4096;    // positions per select workgroup
constexpr int kMaxSelectWgs = 128;    // select workgroups of the longest context (512K)
constexpr int kAttnTileRows = 32;     // latent rows per attention tile
constexpr int kMaxLenRows = 1 << 19;  // longest visible context (SGA_MAX_LEN)

// First-level histogram lists. A decode indexer workgroup (token t, chunk c)
// writes the nonzero digit-1 bins of its chunk into slot c of the token's
// kHist1-word histogram region, with plain stores: word 0 holds the number m
// of entries, words 1..m one entry (bin << 16 | count) each, in ascending bin
// order; when more than slot_words - 1 bins are nonzero, word 0 holds
// kHistOverflow and the select kernel counts that chunk from its scores.
// Every workgroup writes its slot, so nothing needs zeroing beforehand (a
// dense histogram filled by atomics needs a cleared region and a kernel to
// clear it). Slots are powers of two from 32 to 256 words and fill at most
// the kHist1 words of the region; with more chunks per token than 128 the
// dense histogram is used.
constexpr int kHistSlotMin = 32;
constexpr int kHistSlotMax = 256;
constexpr int kMaxHistSlots = kHist1 / kHistSlotMin;   // 128 chunks per token
static_assert(kMaxHistSlots == 128, "the select kernel's overflow mask is four words");
__host__ __device__ constexpr int hist_slot_words(int64_t chunks) {
  int w = kHistSlotMax;
  while (w >= kHistSlotMin && (int64_t)w * chunks > kHist1) w >>= 1;
  return w >= kHistSlotMin ? w : 0;
}

struct IndexerArgs {
  BatchView batch;
  int num_tokens;
  const uint16_t* q_idx;   // [T,64,128] bf16
  const float* w;          // [T,64]
  const uint8_t* k_idx;    // [rows,128] bf16 (256 B) or E4M3FN (128 B) rows
  const void* k_scale;     // one 32-bit word per row: the fp32 scale (kFmtFp8) or
                           // the row's four E8M0 block exponents (kFmtMx)
  float* scores;           // [T,ld]
  int64_t ld;
  // top-k first level, filled by the fused variant
  uint32_t* hist;          // [T,4096] dense histogram, or the per-chunk lists
  uint32_t* hist2;         // [T,4096] second level: zeroed here for the select kernel
  int hist_slot_words;     // 0: dense histogram (atomics into a cleared region); else list slots
  TopkCtrl* ctrl;          // [T]
  int k;
  int chunk;               // positions per workgroup (set by the launch)
};

struct TopkArgs {
  BatchView batch;
  int num_tokens;
  const float* scores;
  int64_t ld;
  int k;
  int32_t* indices;        // [T,k]
  uint32_t* hist;          // [T,4096] digit-1 histogram (zeroed per call), or the per-chunk lists
  int hist_slot_words;     // 0: dense histogram; else words per list slot
  int hist_chunk;          // list slots: positions per slot's chunk
  uint32_t* hist2;         // [T,4096] digit-2 histogram of the candidates (zeroed per call)
  TopkCtrl* ctrl;          // [T]
  uint32_t* sel;           // [T,words]
  int64_t words;           // bitmap words per token
  uint32_t* cand;          // [T,cand_cap] candidate positions; select workgroup x of a
                           // token writes its candidates from slot x * kSelectChunk on
  uint32_t* cand_key;      // [T,cand_cap] their radix keys
  int64_t cand_cap;        // a multiple of kSelectChunk covering the longest context
  uint32_t* wg_count;      // [T,max_select_wgs] candidates each select workgroup wrote
  int max_select_wgs;
  int lds_cand_cap;        // candidates the one-kernel top-k can stage in LDS
  int fin_window;          // ranks per workgroup of the standalone final stage
};

struct AttnArgs {
  BatchView batch;
  int num_tokens;
  const uint16_t* q_abs;   // [T,64,576] bf16
  const uint8_t* kv;       // [rows,576] bf16 or E4M3FN
  const void* kv_scale;    // [rows] fp32 (kFmtFp8) or [rows,18] E8M0 bytes (kFmtMx)
  const int32_t* indices;  // [T,k]
  int k;
  float sm_scale;
  const float* gate;       // [T,64] or null
  float* out;              // [T,64,512]
  float* lse;              // [T,64] or null
  int32_t* indices_out;    // [T,k] or null: the selecting kernel writes the rows it attends
  int splits;              // row splits per token
  int rows_per_split;      // multiple of kAttnTileRows
  uint16_t* part_o;        // [T,splits,32 column blocks,64 heads,16] fp16, normalised
  float* part_ml;          // [T,splits,64,4]: max logit (base 2), exp-sum, output scale of
                           // columns 0..255 and of columns 256..511
  // probabilities variant (sparse indexer loss)
  const float* lse_in;     // [T,64] natural log-sum-exp of each head over the selected rows
  float* probs;            // [T,k] head-mean probability of each selected row
};

// Sparse indexer loss per token from the head-mean probabilities.
struct LossArgs {
  BatchView batch;
  int num_tokens;
  const int32_t* indices;  // [T,k]
  int k;
  const float* scores;     // [T,ld] indexer scores
  int64_t ld;
  const float* probs;      // [T,k]
  float* loss;             // [T]
};

// Cache append: token t writes row seq_start[b] + p of each given cache.
struct CacheArgs {
  BatchView batch;
  int num_tokens;
  const uint16_t* latent;  // [T,576] bf16, or null
  const uint16_t* key;     // [T,128] bf16, or null
  uint8_t* kv;             // [rows,576] bf16 or E4M3FN payload
  void* kv_scale;          // [rows] fp32 (kFmtFp8) or [rows,18] E8M0 bytes (kFmtMx)
  int kv_fmt;
  uint8_t* k_idx;          // [rows,128] bf16 or E4M3FN payload
  void* k_idx_scale;       // [rows] fp32 (kFmtFp8) or [rows,4] E8M0 bytes (kFmtMx)
  int k_idx_fmt;
};

// Output epilogue: C = A . B^T per batch entry, A fp32 [M x K] (row stride
// lda, batch stride a_batch), B bf16 [N x K] (ldb, b_batch), C fp32 [M x N]
// (ldc, c_batch). K a multiple of proj_chunk() * splits, N of kProjCols.
constexpr int kDV = 128;              // value dimension per head
constexpr int kProjRows = 16;         // rows of A per MFMA row block
constexpr int kProjCols = 64;         // columns of C per workgroup
// row blocks per workgroup: 4 (64 rows, weights read once per 64 rows) from
// 32 rows on, else 1; K per staged chunk: 256 with one row block, 128 with four
__host__ __device__ constexpr int proj_row_blocks(int M) { return M >= 32 ? 4 : 1; }
__host__ __device__ constexpr int proj_chunk(int mb) { return mb == 4 ? 128 : 256; }
// column blocks of 64 per workgroup: 2 from 32 rows on, when N allows it (each
// A element read from LDS then serves two weight rows; measured slower below)
__host__ __device__ constexpr int proj_col_blocks(int M, int N) {
  return (M >= 32 && N % (2 * kProjCols) == 0) ? 2 : 1;
}
// A few rows (at most one MFMA row block): the output projection's kernel for
// decode batches, 8 waves and 128 columns of C per workgroup, whose block of A
// over its K range (at most kProjVecMaxK) is staged in LDS once.
constexpr int kProjVecCols = 128;
constexpr int kProjVecMaxK = 2048;
__host__ __device__ constexpr bool proj_vec(int M, int N, int batch) {
  return M <= kProjRows && batch == 1 && N % kProjVecCols == 0;
}
struct ProjArgs {
  const float* a;
  int64_t lda, a_batch;
  const uint16_t* b;
  int64_t ldb, b_batch;
  float* c;
  int64_t ldc, c_batch;
  float* part;             // [splits][batch][M][N] partial sums when splits > 1
  int M, N, K, batch, splits;
};

hipError_t launch_clear(uint32_t* p, int64_t words, hipStream_t s);
hipError_t launch_proj(const ProjArgs& a, hipStream_t s);
hipError_t launch_cache_append(const CacheArgs& a, hipStream_t s);
hipError_t launch_indexer(const IndexerArgs& a, int fmt, bool fused_hist, hipStream_t s);
// Positions per workgroup of the decode indexer for this batch shape.
int indexer_decode_chunk(int fmt, int max_len, int num_tokens);
// Eight tokens per workgroup sharing each key tile: for batches with many
// tokens per sequence. With fused_hist it writes each token's digit-1
// histogram with plain stores (it owns the token).
hipError_t launch_indexer_prefill(const IndexerArgs& a, int fmt, bool fused_hist, hipStream_t s);
constexpr int kPrefillTokensPerSeq = 64;   // mean tokens per sequence from which it is used
hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t s);
// List slots for the stand-alone histogram kernel (kIndexerChunk positions per
// workgroup), 0 when the dense histogram is needed.
int topk_hist_slot_words(int max_len);
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s);
hipError_t launch_topk_finalize(const TopkArgs& a, hipStream_t s);
constexpr size_t kFinalizeLds = 160 * 1024;  // dynamic LDS of the finalize kernels
constexpr int64_t kMaxTokenWords = 8192;     // bitmap words for the one-kernel top-k (256K)
int topk_token_lds_cap(int64_t words);       // 0: use the multi-kernel top-k
hipError_t launch_topk_token(const TopkArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int fmt, hipStream_t s);
hipError_t launch_combine(const AttnArgs& a, hipStream_t s);
// The attention kernel that first takes its own rows of each token's top-k
// from the select kernel's output (the top-k's final stage runs inside it).
constexpr int kSelectMaxRows = 2048;   // split rows whose indices it holds in LDS
// Used up to 4,096 bitmap words (contexts of 128K): the final stage's work grows
// with the context, and beyond that the separate finalize kernel, with twice the
// threads per token, was measured faster (256K: 23.3 us for the two kernels
// against 25.0 us fused).
constexpr int64_t kSelectMaxWords = 4096;
hipError_t launch_attention_select(const AttnArgs& a, const TopkArgs& ta, int fmt, hipStream_t s);
hipError_t launch_attention_probs(const AttnArgs& a, int fmt, hipStream_t s);
hipError_t launch_indexer_loss(const LossArgs& a, hipStream_t s);

}  // namespace sga
