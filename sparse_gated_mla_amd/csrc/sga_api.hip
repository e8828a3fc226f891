// Host side of libsga: argument checks, workspace planning and kernel launches
// for the C ABI declared in include/sga.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "sga.h"
#include "sga_kernels.h"

namespace {

using sga::AttnArgs;
using sga::BatchView;
using sga::CacheArgs;
using sga::ProjArgs;
using sga::LossArgs;
using sga::IndexerArgs;
using sga::TopkArgs;
using sga::TopkCtrl;

constexpr size_t kAlign = 256;
constexpr int kTokenTopkMinTokens = 512;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Carves consecutive, 256-byte aligned regions out of a workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up(count * sizeof(T));
    return p;
  }
};

static_assert((SGA_MAX_LEN + sga::kSelectChunk - 1) / sga::kSelectChunk <= sga::kMaxSelectWgs,
              "the finalize kernel scans one slice count per select workgroup");

// Chunked prefill: tokens share their sequence's keys, so the indexer that
// reuses each key tile across eight tokens is the faster one.
bool many_tokens_per_seq(const sga_batch* b) {
  return (int64_t)b->num_tokens >= (int64_t)sga::kPrefillTokensPerSeq * b->num_seqs;
}

int64_t bitmap_words(int32_t max_len) { return ((int64_t)max_len + 63) / 64 * 2; }

// ---------------------------------------------------------------- top-k layout
struct TopkLayout {
  uint32_t* hist;   // digit-1 histograms, then the digit-2 ones
  TopkCtrl* ctrl;
  uint32_t* sel;
  uint32_t* cand;
  uint32_t* cand_key;
  uint32_t* wg_count;
  int64_t words, cand_cap;
  int max_select_wgs;
  size_t clear_words;  // the histograms, cleared per call
};

TopkLayout carve_topk(Carver& c, int32_t T, int32_t max_len) {
  TopkLayout L;
  L.words = bitmap_words(max_len);
  L.max_select_wgs = (max_len + sga::kSelectChunk - 1) / sga::kSelectChunk;
  L.cand_cap = (int64_t)L.max_select_wgs * sga::kSelectChunk;
  // both histogram levels, back to back, cleared by one fill kernel
  L.hist = c.take<uint32_t>((size_t)T * (sga::kHist1 + sga::kHist2));
  L.clear_words = (size_t)T * (sga::kHist1 + sga::kHist2);
  L.ctrl = c.take<TopkCtrl>((size_t)T);
  L.wg_count = c.take<uint32_t>((size_t)T * L.max_select_wgs);
  L.sel = c.take<uint32_t>((size_t)T * L.words);
  L.cand = c.take<uint32_t>((size_t)T * L.cand_cap);
  L.cand_key = c.take<uint32_t>((size_t)T * L.cand_cap);
  return L;
}

// ---------------------------------------------------------------- attention plan
struct AttnPlan {
  int splits, rows_per_split;
};

AttnPlan plan_attention(int32_t T, int32_t k) {
  const int tile = sga::kAttnTileRows;
  const int tiles = (k + tile - 1) / tile;
  int want = (T > 0) ? (256 + T - 1) / T : 1;   // aim for about 256 workgroups
  // at least 2 tiles per split: with fewer tokens than CUs the splits fill the
  // GPU (measured: 2-tile splits beat 4-tile ones at 4 and 8 tokens; single
  // tiles gain nothing and double the partials)
  int max_splits = tiles / 2 > 0 ? tiles / 2 : 1;
  if (max_splits > 64) max_splits = 64;          // the combine merges at most 64 partials
  int splits = want < max_splits ? want : max_splits;
  if (splits < 1) splits = 1;
  int tiles_per = (tiles + splits - 1) / splits;
  splits = (tiles + tiles_per - 1) / tiles_per;
  return AttnPlan{splits, tiles_per * tile};
}

struct AttnLayout {
  uint16_t* part_o;
  float* part_ml;
};

AttnLayout carve_attn(Carver& c, int32_t T, const AttnPlan& p) {
  AttnLayout L{nullptr, nullptr};
  if (p.splits > 1) {
    L.part_o = c.take<uint16_t>((size_t)T * p.splits * sga::kHeads * sga::kDLatent);
    L.part_ml = c.take<float>((size_t)T * p.splits * sga::kHeads * 4);
  }
  return L;
}

// ---------------------------------------------------------------- checks
sga_status check_batch(const sga_batch* b) {
  if (!b) return SGA_ERR_INVALID_ARG;
  if (b->num_tokens < 0 || b->num_seqs < 0 || b->reserved != 0) return SGA_ERR_INVALID_ARG;
  if (b->num_tokens == 0) return SGA_OK;
  if (b->num_seqs < 1 || b->max_len < 1 || b->cache_rows < 1) return SGA_ERR_INVALID_ARG;
  if (b->max_len > SGA_MAX_LEN || b->num_tokens > SGA_MAX_TOKENS) return SGA_ERR_UNSUPPORTED;
  if (!b->token_seq || !b->token_pos || !b->seq_start || !b->seq_len) return SGA_ERR_INVALID_ARG;
  return SGA_OK;
}

// A cache and its scales. mx_align: the alignment the kernels need of an MX
// exponent array (4 for the indexer keys, read one 32-bit word per row; 1 for
// the latent rows, read by byte).
sga_status check_store(const void* data, const void* scale, sga_dtype dt, uintptr_t mx_align) {
  if (!data || !aligned16(data)) return SGA_ERR_INVALID_ARG;
  const uintptr_t sa = reinterpret_cast<uintptr_t>(scale);
  if (dt == SGA_BF16) return scale ? SGA_ERR_INVALID_ARG : SGA_OK;
  if (dt == SGA_FP8_E4M3) return scale && sa % alignof(float) == 0 ? SGA_OK : SGA_ERR_INVALID_ARG;
  if (dt == SGA_MXFP8_E4M3 || dt == SGA_MXFP4_E2M1)
    return scale && sa % mx_align == 0 ? SGA_OK : SGA_ERR_INVALID_ARG;
  return SGA_ERR_UNSUPPORTED;
}

BatchView view_of(const sga_batch* b) {
  BatchView v;
  v.token_seq = b->token_seq;
  v.token_pos = b->token_pos;
  v.seq_start = b->seq_start;
  v.seq_len = b->seq_len;
  v.num_seqs = b->num_seqs;
  v.max_len = b->max_len;
  v.cache_rows = b->cache_rows;
  return v;
}

sga_status hip_status(hipError_t e) { return e == hipSuccess ? SGA_OK : SGA_ERR_HIP; }

#define SGA_TRY(expr)                      \
  do {                                     \
    sga_status _s = (expr);                \
    if (_s != SGA_OK) return _s;           \
  } while (0)
#define SGA_HIP(expr)                      \
  do {                                     \
    if ((expr) != hipSuccess) return SGA_ERR_HIP; \
  } while (0)

sga_status record(hipEvent_t e, hipStream_t s) {
  if (!e) return SGA_OK;
  return hip_status(hipEventRecord(e, s));
}

// First-level histogram form, fixed by whichever kernel fills it: list slots
// of hist_slot_words words, one per chunk of hist_chunk positions, or the
// dense histogram (hist_slot_words 0), which needs a cleared region.
struct HistForm {
  int slot_words, chunk;
};

TopkArgs topk_args(const sga_batch* batch, const float* scores, int64_t ld, int32_t k,
                   int32_t* indices, const TopkLayout& L, HistForm hf) {
  TopkArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = view_of(batch);
  a.num_tokens = batch->num_tokens;
  a.scores = scores;
  a.ld = ld;
  a.k = k;
  a.indices = indices;
  a.hist = L.hist;
  a.hist_slot_words = hf.slot_words;
  a.hist_chunk = hf.chunk;
  a.hist2 = L.hist + (size_t)batch->num_tokens * sga::kHist1;
  a.ctrl = L.ctrl;
  a.sel = L.sel;
  a.words = L.words;
  a.cand = L.cand;
  a.cand_key = L.cand_key;
  a.cand_cap = L.cand_cap;
  a.wg_count = L.wg_count;
  a.max_select_wgs = L.max_select_wgs;
  return a;
}

// One workgroup per token only when the batch alone fills the GPU.
bool use_token_topk(int32_t T, const TopkLayout& L) {
  return T >= kTokenTopkMinTokens && sga::topk_token_lds_cap(L.words) > 0;
}

// run_topk with hist_ready: the indexer has filled the first level in form
// hf and zeroed the second. Otherwise the histogram kernel fills it: as list
// slots when the context allows (and then zeroes the second level itself),
// else densely after a clear of both levels.
sga_status run_topk(const sga_batch* batch, const float* scores, int64_t ld, int32_t k,
                    int32_t* indices, const TopkLayout& L, bool hist_ready, HistForm hf,
                    hipStream_t stream) {
  // (the one-workgroup top-k reads only the dense form)
  const bool token_topk = use_token_topk(batch->num_tokens, L);
  if (!hist_ready)
    hf = HistForm{token_topk ? 0 : sga::topk_hist_slot_words(batch->max_len), sga::kIndexerChunk};
  TopkArgs a = topk_args(batch, scores, ld, k, indices, L, hf);
  if (!hist_ready) {
    if (!hf.slot_words) SGA_HIP(sga::launch_clear(L.hist, (int64_t)L.clear_words, stream));
    SGA_HIP(sga::launch_topk_hist(a, stream));
  }
  if (token_topk) {
    a.lds_cand_cap = sga::topk_token_lds_cap(L.words);
    SGA_HIP(sga::launch_topk_token(a, stream));
  } else {
    a.lds_cand_cap = 0;
    // the final stage's ordered pass spread over several workgroups per
    // token, about one per CU in all, each handing out a window of at least
    // 64 ranks
    int windows = 256 / (batch->num_tokens > 0 ? batch->num_tokens : 1);
    if (windows < 1) windows = 1;
    if (windows > (k + 63) / 64) windows = (k + 63) / 64;
    a.fin_window = (k + windows - 1) / windows;
    SGA_HIP(sga::launch_topk_select(a, stream));
    SGA_HIP(sga::launch_topk_finalize(a, stream));
  }
  return SGA_OK;
}

AttnArgs attn_args(const sga_batch* batch, const void* q_abs, const void* kv, const void* kv_scale,
                   const int32_t* indices, int32_t k, float sm_scale, const float* gate, float* out,
                   float* lse, const AttnPlan& plan, const AttnLayout& L) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = view_of(batch);
  a.num_tokens = batch->num_tokens;
  a.q_abs = static_cast<const uint16_t*>(q_abs);
  a.kv = static_cast<const uint8_t*>(kv);
  a.kv_scale = kv_scale;
  a.indices = indices;
  a.k = k;
  a.sm_scale = sm_scale;
  a.gate = gate;
  a.out = out;
  a.lse = lse;
  a.splits = plan.splits;
  a.rows_per_split = plan.rows_per_split;
  a.part_o = L.part_o;
  a.part_ml = L.part_ml;
  return a;
}

sga_status run_attention(const sga_batch* batch, const void* q_abs, const void* kv,
                         const void* kv_scale, sga_dtype kv_dtype, const int32_t* indices,
                         int32_t k, float sm_scale, const float* gate, float* out, float* lse,
                         const AttnPlan& plan, const AttnLayout& L, hipStream_t stream) {
  const AttnArgs a = attn_args(batch, q_abs, kv, kv_scale, indices, k, sm_scale, gate, out, lse, plan, L);
  SGA_HIP(sga::launch_attention(a, (int)kv_dtype, stream));
  SGA_HIP(sga::launch_combine(a, stream));
  return SGA_OK;
}

// ---------------------------------------------------------------- output epilogue
// Splits of K: the largest divisor of the chunk count that keeps the grid
// within about two workgroups per CU (measured best from 16 to 256 rows).
int proj_splits(int64_t tiles, int chunks) {
  int best = 1;
  for (int s = 1; s <= chunks; ++s)
    if (chunks % s == 0 && tiles * s <= 512) best = s;
  return best;
}

struct ProjPlan {
  int uv_splits, o_splits;
  size_t u_floats, part_floats;
};

ProjPlan plan_proj(int32_t T, int32_t d_model) {
  const int mb = sga::proj_row_blocks(T);
  const int64_t mt = (T + sga::kProjRows * mb - 1) / (sga::kProjRows * mb);
  const int chunk = sga::proj_chunk(mb);
  ProjPlan p;
  // the up-projection is 64 products with K = 512: never split (no second pass)
  p.uv_splits = 1;
  const int nb = sga::proj_col_blocks(T, d_model);
  p.o_splits = proj_splits(mt * (d_model / (sga::kProjCols * nb)), sga::kHeads * sga::kDV / chunk);
  if (sga::proj_vec(T, d_model, 1)) {
    // one workgroup per CU (its A block fills the LDS): the most splits of K
    // that keep the grid within 256 workgroups, each K range at most
    // kProjVecMaxK
    const int tiles = d_model / sga::kProjVecCols, kchunks = sga::kHeads * sga::kDV / 256;
    int best = 0;
    for (int s = 1; s <= kchunks; ++s) {
      if (kchunks % s || sga::kHeads * sga::kDV / s > sga::kProjVecMaxK) continue;
      if (best == 0 || tiles * s <= 256) best = s;
    }
    p.o_splits = best;
  }
  p.u_floats = (size_t)T * sga::kHeads * sga::kDV;
  const size_t uv_part = p.uv_splits > 1 ? (size_t)p.uv_splits * T * sga::kHeads * sga::kDV : 0;
  const size_t o_part = p.o_splits > 1 ? (size_t)p.o_splits * T * d_model : 0;
  p.part_floats = uv_part > o_part ? uv_part : o_part;
  return p;
}

size_t proj_ws(int32_t T, int32_t d_model) {
  const ProjPlan p = plan_proj(T, d_model);
  Carver c(nullptr);
  c.take<float>(p.u_floats);
  if (p.part_floats) c.take<float>(p.part_floats);
  return c.used;
}

size_t topk_ws(int32_t T, int32_t max_len) {
  Carver c(nullptr);
  carve_topk(c, T, max_len);
  return c.used;
}

size_t attn_ws(int32_t T, int32_t k) {
  Carver c(nullptr);
  carve_attn(c, T, plan_attention(T, k));
  return c.used;
}

}  // namespace

// ---------------------------------------------------------------- no-allocation scratch
// The workspace of sga_forward_noalloc: a file-scope device array that each
// GPU holds from module load until the process ends. In host code its name
// stands for a host-side symbol, not a device address, so the address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that pointer is passed to kernels.
static __device__ __align__(256) unsigned char scratch[SGA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device that runs work queued on `stream` (the current device for the
// null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  if (!stream) return hipGetDevice(dev);
  hipDevice_t d;
  const hipError_t e = hipStreamGetDevice(stream, &d);
  if (e == hipSuccess) *dev = (int)d;
  return e;
}

// The device address of `scratch` on device dev; found once per device.
sga_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return SGA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SGA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return SGA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return SGA_ERR_HIP;
    if (e != hipSuccess || !p) return SGA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SGA_OK;
}

}  // namespace

static_assert(SGA_BF16 == sga::kFmtBf16 && SGA_FP8_E4M3 == sga::kFmtFp8 &&
                  SGA_MXFP8_E4M3 == sga::kFmtMx && SGA_MXFP4_E2M1 == sga::kFmtMx4,
              "cache formats are passed to the kernels as their sga_dtype values");

extern "C" {

SGA_API const char* sga_status_string(sga_status s) {
  switch (s) {
    case SGA_OK: return "SGA_OK";
    case SGA_ERR_INVALID_ARG: return "SGA_ERR_INVALID_ARG: null pointer, bad size or non-finite scale";
    case SGA_ERR_UNSUPPORTED: return "SGA_ERR_UNSUPPORTED: dtype or size outside what the kernels handle";
    case SGA_ERR_WORKSPACE: return "SGA_ERR_WORKSPACE: workspace missing or too small";
    case SGA_ERR_HIP: return "SGA_ERR_HIP: a HIP launch or query failed";
  }
  return "unknown sga_status";
}

SGA_API int sga_version(void) { return 100; }

SGA_API sga_status sga_index_scores(const sga_batch* batch, const void* q_idx, const float* w,
                                    const void* k_idx, const void* k_idx_scale,
                                    sga_dtype k_idx_dtype, float* scores, int64_t ld,
                                    hipStream_t stream) {
  SGA_TRY(check_batch(batch));
  if (batch->num_tokens == 0) return SGA_OK;
  if (!q_idx || !w || !scores || !aligned16(q_idx) || !aligned16(w)) return SGA_ERR_INVALID_ARG;
  SGA_TRY(check_store(k_idx, k_idx_scale, k_idx_dtype, 4));
  if (ld < batch->max_len) return SGA_ERR_INVALID_ARG;
  IndexerArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = view_of(batch);
  a.num_tokens = batch->num_tokens;
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.w = w;
  a.k_idx = static_cast<const uint8_t*>(k_idx);
  a.k_scale = k_idx_scale;
  a.scores = scores;
  a.ld = ld;
  return hip_status(many_tokens_per_seq(batch)
                        ? sga::launch_indexer_prefill(a, (int)k_idx_dtype, false, stream)
                        : sga::launch_indexer(a, (int)k_idx_dtype, false, stream));
}

SGA_API size_t sga_topk_workspace_size(int32_t num_tokens, int32_t max_len, int32_t k) {
  (void)k;
  if (num_tokens <= 0 || max_len <= 0) return 0;
  return topk_ws(num_tokens, max_len);
}

SGA_API sga_status sga_topk(const sga_batch* batch, const float* scores, int64_t ld, int32_t k,
                            int32_t* indices, void* ws, size_t ws_bytes, hipStream_t stream) {
  SGA_TRY(check_batch(batch));
  if (k < 1) return SGA_ERR_INVALID_ARG;
  if (k > SGA_MAX_K) return SGA_ERR_UNSUPPORTED;
  if (batch->num_tokens == 0) return SGA_OK;
  if (!scores || !indices || ld < batch->max_len) return SGA_ERR_INVALID_ARG;
  size_t need = topk_ws(batch->num_tokens, batch->max_len);
  if (!ws || ws_bytes < need) return SGA_ERR_WORKSPACE;
  Carver c(ws);
  TopkLayout L = carve_topk(c, batch->num_tokens, batch->max_len);
  return run_topk(batch, scores, ld, k, indices, L, false, HistForm{0, 0}, stream);
}

SGA_API size_t sga_attn_workspace_size(int32_t num_tokens, int32_t k) {
  if (num_tokens <= 0 || k <= 0) return 0;
  return attn_ws(num_tokens, k);
}

SGA_API sga_status sga_sparse_mla_attn(const sga_batch* batch, const void* q_abs, const void* kv,
                                       const void* kv_scale, sga_dtype kv_dtype,
                                       const int32_t* indices, int32_t k, float sm_scale,
                                       const float* gate_logits, float* out, float* lse,
                                       void* ws, size_t ws_bytes, hipStream_t stream) {
  SGA_TRY(check_batch(batch));
  if (k < 1) return SGA_ERR_INVALID_ARG;
  if (k > SGA_MAX_K) return SGA_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale)) return SGA_ERR_INVALID_ARG;
  if (batch->num_tokens == 0) return SGA_OK;
  if (!q_abs || !indices || !out || !aligned16(q_abs) || !aligned16(out)) return SGA_ERR_INVALID_ARG;
  SGA_TRY(check_store(kv, kv_scale, kv_dtype, 1));
  AttnPlan plan = plan_attention(batch->num_tokens, k);
  size_t need = attn_ws(batch->num_tokens, k);
  if (need > 0 && (!ws || ws_bytes < need)) return SGA_ERR_WORKSPACE;
  Carver c(ws);
  AttnLayout L = carve_attn(c, batch->num_tokens, plan);
  return run_attention(batch, q_abs, kv, kv_scale, kv_dtype, indices, k, sm_scale, gate_logits,
                       out, lse, plan, L, stream);
}

SGA_API size_t sga_forward_workspace_size(int32_t num_tokens, int32_t max_len, int32_t k) {
  if (num_tokens <= 0 || max_len <= 0 || k <= 0) return 0;
  Carver c(nullptr);
  c.take<float>((size_t)num_tokens * max_len);     // scores
  c.take<int32_t>((size_t)num_tokens * k);         // indices
  carve_topk(c, num_tokens, max_len);
  carve_attn(c, num_tokens, plan_attention(num_tokens, k));
  return c.used;
}

SGA_API sga_status sga_forward(const sga_batch* batch, const void* q_idx, const float* w,
                               const void* k_idx, const void* k_idx_scale, sga_dtype k_idx_dtype,
                               const void* q_abs, const void* kv, const void* kv_scale,
                               sga_dtype kv_dtype, int32_t k, float sm_scale,
                               const float* gate_logits, float* out, float* lse,
                               int32_t* indices_out, void* ws, size_t ws_bytes,
                               const sga_trace* trace, hipStream_t stream) {
  SGA_TRY(check_batch(batch));
  if (k < 1) return SGA_ERR_INVALID_ARG;
  if (k > SGA_MAX_K) return SGA_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale)) return SGA_ERR_INVALID_ARG;
  if (batch->num_tokens == 0) return SGA_OK;
  if (!q_idx || !w || !aligned16(q_idx) || !aligned16(w)) return SGA_ERR_INVALID_ARG;
  if (!q_abs || !out || !aligned16(q_abs) || !aligned16(out)) return SGA_ERR_INVALID_ARG;
  SGA_TRY(check_store(k_idx, k_idx_scale, k_idx_dtype, 4));
  SGA_TRY(check_store(kv, kv_scale, kv_dtype, 1));
  const int32_t T = batch->num_tokens;
  size_t need = sga_forward_workspace_size(T, batch->max_len, k);
  if (!ws || ws_bytes < need) return SGA_ERR_WORKSPACE;

  Carver c(ws);
  float* scores = c.take<float>((size_t)T * batch->max_len);
  int32_t* idx_ws = c.take<int32_t>((size_t)T * k);
  TopkLayout TL = carve_topk(c, T, batch->max_len);
  AttnPlan plan = plan_attention(T, k);
  AttnLayout AL = carve_attn(c, T, plan);
  int32_t* indices = indices_out ? indices_out : idx_ws;

  const bool prefill_indexer = many_tokens_per_seq(batch);
  const bool token_topk = use_token_topk(T, TL);
  // The first level needs no cleared memory when each workgroup writes its own
  // part with plain stores: the prefill indexer stores each token's whole
  // histogram, and the decode indexer writes per-chunk lists (read by the
  // select kernel, not by the one-workgroup top-k). Both zero the second
  // level. Only the dense histogram of atomics needs the clear kernel.
  HistForm hf{0, 0};
  if (!prefill_indexer && !token_topk) {
    hf.chunk = sga::indexer_decode_chunk((int)k_idx_dtype, batch->max_len, T);
    hf.slot_words = sga::hist_slot_words(((int64_t)batch->max_len + hf.chunk - 1) / hf.chunk);
  }
  if (!prefill_indexer && !hf.slot_words)
    SGA_HIP(sga::launch_clear(TL.hist, (int64_t)TL.clear_words, stream));
  IndexerArgs ia;
  memset(&ia, 0, sizeof(ia));
  ia.batch = view_of(batch);
  ia.num_tokens = T;
  ia.q_idx = static_cast<const uint16_t*>(q_idx);
  ia.w = w;
  ia.k_idx = static_cast<const uint8_t*>(k_idx);
  ia.k_scale = k_idx_scale;
  ia.scores = scores;
  ia.ld = batch->max_len;
  ia.hist = TL.hist;
  ia.hist2 = TL.hist + (size_t)T * sga::kHist1;
  ia.hist_slot_words = hf.slot_words;
  ia.ctrl = TL.ctrl;
  ia.k = k;
  if (trace) SGA_TRY(record(trace->indexer_begin, stream));
  if (prefill_indexer)
    SGA_HIP(sga::launch_indexer_prefill(ia, (int)k_idx_dtype, true, stream));
  else
    SGA_HIP(sga::launch_indexer(ia, (int)k_idx_dtype, true, stream));
  if (trace) SGA_TRY(record(trace->indexer_end, stream));
  if (!token_topk && plan.rows_per_split <= sga::kSelectMaxRows &&
      TL.words <= sga::kSelectMaxWords) {
    // the top-k's final stage runs inside the attention kernel: each split
    // takes its own rows of the selection (and writes them to indices_out)
    const TopkArgs ta = topk_args(batch, scores, batch->max_len, k, nullptr, TL, hf);
    SGA_HIP(sga::launch_topk_select(ta, stream));
    if (trace) SGA_TRY(record(trace->topk_end, stream));
    AttnArgs aa = attn_args(batch, q_abs, kv, kv_scale, nullptr, k, sm_scale, gate_logits, out, lse,
                            plan, AL);
    aa.indices_out = indices_out;
    SGA_HIP(sga::launch_attention_select(aa, ta, (int)kv_dtype, stream));
    SGA_HIP(sga::launch_combine(aa, stream));
  } else {
    SGA_TRY(run_topk(batch, scores, batch->max_len, k, indices, TL, true, hf, stream));
    if (trace) SGA_TRY(record(trace->topk_end, stream));
    SGA_TRY(run_attention(batch, q_abs, kv, kv_scale, kv_dtype, indices, k, sm_scale, gate_logits,
                          out, lse, plan, AL, stream));
  }
  if (trace) SGA_TRY(record(trace->attn_end, stream));
  return SGA_OK;
}

SGA_API size_t sga_forward_noalloc_scratch_bytes(void) { return SGA_NOALLOC_SCRATCH_BYTES; }

SGA_API sga_status sga_forward_noalloc(const sga_batch* batch, const void* q_idx, const float* w,
                                       const void* k_idx, const void* k_idx_scale,
                                       sga_dtype k_idx_dtype, const void* q_abs, const void* kv,
                                       const void* kv_scale, sga_dtype kv_dtype, int32_t k,
                                       float sm_scale, const float* gate_logits, float* out,
                                       float* lse, int32_t* indices_out, const sga_trace* trace,
                                       hipStream_t stream) {
  // the size limit is checked before the device is touched
  SGA_TRY(check_batch(batch));
  if (k < 1) return SGA_ERR_INVALID_ARG;
  if (k > SGA_MAX_K) return SGA_ERR_UNSUPPORTED;
  if (batch->num_tokens == 0) return SGA_OK;
  const size_t need = sga_forward_workspace_size(batch->num_tokens, batch->max_len, k);
  if (need > SGA_NOALLOC_SCRATCH_BYTES) return SGA_ERR_WORKSPACE;
  int dev = -1;
  SGA_HIP(stream_device(stream, &dev));
  void* ws = nullptr;
  SGA_TRY(scratch_on(dev, &ws));
  return sga_forward(batch, q_idx, w, k_idx, k_idx_scale, k_idx_dtype, q_abs, kv, kv_scale, kv_dtype,
                     k, sm_scale, gate_logits, out, lse, indices_out, ws, SGA_NOALLOC_SCRATCH_BYTES,
                     trace, stream);
}

SGA_API sga_status sga_cache_append(const sga_batch* batch, const void* latent, const void* idx_key,
                                    void* kv, void* kv_scale, sga_dtype kv_dtype, void* k_idx,
                                    void* k_idx_scale, sga_dtype k_idx_dtype, hipStream_t stream) {
  SGA_TRY(check_batch(batch));
  if (!latent != !kv || !idx_key != !k_idx) return SGA_ERR_INVALID_ARG;
  const bool do_kv = latent != nullptr, do_key = idx_key != nullptr;
  if (do_kv) {
    if (!aligned16(latent)) return SGA_ERR_INVALID_ARG;
    SGA_TRY(check_store(kv, kv_scale, kv_dtype, 1));
  }
  if (do_key) {
    if (!aligned16(idx_key)) return SGA_ERR_INVALID_ARG;
    SGA_TRY(check_store(k_idx, k_idx_scale, k_idx_dtype, 1));
  }
  if (batch->num_tokens == 0 || (!do_kv && !do_key)) return SGA_OK;
  CacheArgs a;
  a.batch = view_of(batch);
  a.num_tokens = batch->num_tokens;
  a.latent = do_kv ? static_cast<const uint16_t*>(latent) : nullptr;
  a.key = do_key ? static_cast<const uint16_t*>(idx_key) : nullptr;
  a.kv = do_kv ? static_cast<uint8_t*>(kv) : nullptr;
  a.kv_scale = do_kv ? kv_scale : nullptr;
  a.kv_fmt = do_kv ? (int)kv_dtype : sga::kFmtBf16;
  a.k_idx = do_key ? static_cast<uint8_t*>(k_idx) : nullptr;
  a.k_idx_scale = do_key ? k_idx_scale : nullptr;
  a.k_idx_fmt = do_key ? (int)k_idx_dtype : sga::kFmtBf16;
  return hip_status(sga::launch_cache_append(a, stream));
}

SGA_API size_t sga_indexer_loss_workspace_size(int32_t num_tokens, int32_t k) {
  if (num_tokens <= 0 || k <= 0) return 0;
  Carver c(nullptr);
  c.take<float>((size_t)num_tokens * k);
  return c.used;
}

SGA_API sga_status sga_indexer_loss(const sga_batch* batch, const void* q_abs, const void* kv,
                                    const void* kv_scale, sga_dtype kv_dtype, const int32_t* indices,
                                    int32_t k, float sm_scale, const float* lse, const float* scores,
                                    int64_t ld, float* loss, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  SGA_TRY(check_batch(batch));
  if (k < 1) return SGA_ERR_INVALID_ARG;
  if (k > SGA_MAX_K) return SGA_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale)) return SGA_ERR_INVALID_ARG;
  if (batch->num_tokens == 0) return SGA_OK;
  if (!q_abs || !indices || !lse || !scores || !loss || !aligned16(q_abs)) return SGA_ERR_INVALID_ARG;
  if (ld < batch->max_len) return SGA_ERR_INVALID_ARG;
  SGA_TRY(check_store(kv, kv_scale, kv_dtype, 1));
  const size_t need = sga_indexer_loss_workspace_size(batch->num_tokens, k);
  if (!ws || ws_bytes < need) return SGA_ERR_WORKSPACE;
  Carver c(ws);
  float* probs = c.take<float>((size_t)batch->num_tokens * k);
  const AttnPlan plan = plan_attention(batch->num_tokens, k);
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = view_of(batch);
  a.num_tokens = batch->num_tokens;
  a.q_abs = static_cast<const uint16_t*>(q_abs);
  a.kv = static_cast<const uint8_t*>(kv);
  a.kv_scale = kv_scale;
  a.indices = indices;
  a.k = k;
  a.sm_scale = sm_scale;
  a.splits = plan.splits;
  a.rows_per_split = plan.rows_per_split;
  a.lse_in = lse;
  a.probs = probs;
  SGA_HIP(sga::launch_attention_probs(a, (int)kv_dtype, stream));
  LossArgs l;
  l.batch = a.batch;
  l.num_tokens = batch->num_tokens;
  l.indices = indices;
  l.k = k;
  l.scores = scores;
  l.ld = ld;
  l.probs = probs;
  l.loss = loss;
  SGA_HIP(sga::launch_indexer_loss(l, stream));
  return SGA_OK;
}

SGA_API size_t sga_output_proj_workspace_size(int32_t num_tokens, int32_t d_model) {
  if (num_tokens <= 0 || d_model <= 0 || d_model % sga::kProjCols != 0 || d_model > SGA_MAX_D_MODEL) return 0;
  return proj_ws(num_tokens, d_model);
}

SGA_API sga_status sga_output_proj(int32_t num_tokens, const float* o_latent, const void* w_uv,
                                   const void* w_o, int32_t d_model, float* y, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  if (num_tokens < 0 || d_model <= 0) return SGA_ERR_INVALID_ARG;
  if (num_tokens > SGA_MAX_TOKENS || d_model % sga::kProjCols != 0 || d_model > SGA_MAX_D_MODEL)
    return SGA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return SGA_OK;
  if (!o_latent || !w_uv || !w_o || !y) return SGA_ERR_INVALID_ARG;
  if (!aligned16(o_latent) || !aligned16(w_uv) || !aligned16(w_o) || !aligned16(y))
    return SGA_ERR_INVALID_ARG;
  const size_t need = proj_ws(num_tokens, d_model);
  if (!ws || ws_bytes < need) return SGA_ERR_WORKSPACE;
  const ProjPlan plan = plan_proj(num_tokens, d_model);
  Carver c(ws);
  float* u = c.take<float>(plan.u_floats);
  float* part = plan.part_floats ? c.take<float>(plan.part_floats) : nullptr;
  const int T = num_tokens, HV = sga::kHeads * sga::kDV;
  // u[t, h, v] = sum_k o[t, h, k] * w_uv[h, v, k]: one product per head
  ProjArgs uv;
  uv.a = o_latent;
  uv.lda = (int64_t)sga::kHeads * sga::kDLatent;
  uv.a_batch = sga::kDLatent;
  uv.b = static_cast<const uint16_t*>(w_uv);
  uv.ldb = sga::kDLatent;
  uv.b_batch = (int64_t)sga::kDV * sga::kDLatent;
  uv.c = u;
  uv.ldc = HV;
  uv.c_batch = sga::kDV;
  uv.part = part;
  uv.M = T;
  uv.N = sga::kDV;
  uv.K = sga::kDLatent;
  uv.batch = sga::kHeads;
  uv.splits = plan.uv_splits;
  SGA_HIP(sga::launch_proj(uv, stream));
  // y[t, n] = sum_j u[t, j] * w_o[n, j]
  ProjArgs op;
  op.a = u;
  op.lda = HV;
  op.a_batch = 0;
  op.b = static_cast<const uint16_t*>(w_o);
  op.ldb = HV;
  op.b_batch = 0;
  op.c = y;
  op.ldc = d_model;
  op.c_batch = 0;
  op.part = part;
  op.M = T;
  op.N = d_model;
  op.K = HV;
  op.batch = 1;
  op.splits = plan.o_splits;
  SGA_HIP(sga::launch_proj(op, stream));
  return SGA_OK;
}

}  // extern "C"
