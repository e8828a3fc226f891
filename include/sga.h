/*
 * sga.h: C ABI of libsga, a gfx950 (MI355X) implementation of Sparse Gated
 * Attention (SGA): indexer -> top-k -> sparse absorbed-MLA attention -> sigmoid
 * gate.
 *
 * Sources for what each call computes:
 * - A.X K2 fact sheet (archdb.vladsavinov.com, "A.X K2"), the facts on the
 *   token mixer, the attention shapes, the gate and the token-selection
 *   mechanism;
 * - the "A.X K2 Technical Report" abstract (arXiv:2608.30181), on SGA reading
 *   2,048 positions per query;
 * - the rebasdaily article on A.X K2, in its section on long tasks that cannot
 *   re-read all old content: at most 2,048 positions per query.
 *
 * Conventions that hold for every call:
 * - Pointers are device pointers unless marked (host). The caller owns every
 *   buffer. The library never allocates or frees device memory. Scratch comes
 *   from a caller-provided workspace `ws` of `ws_bytes` bytes, at least the
 *   matching *_workspace_size(); its contents on entry do not matter.
 * - Every call only enqueues work on `stream` and returns. The caller
 *   synchronises. Calls keep no state between them, so calls on different
 *   streams with different workspaces may run concurrently. Outputs must not
 *   alias inputs or the workspace.
 * - Errors: problems the host can see (null required pointers, bad sizes,
 *   unsupported dtypes, a small workspace, a non-finite sm_scale) make the call
 *   return a non-zero sga_status before anything is launched. Outputs are then
 *   left untouched. A failed launch returns SGA_ERR_HIP. Nothing aborts, and no
 *   C++ exception crosses the ABI.
 * - Fixed model dimensions: 64 query heads; indexer 64 heads x 128;
 *   cached latent row 576 = 512 latent + 64 RoPE key; values are the first
 *   512 columns.
 * - Element types: bf16 is IEEE bfloat16. SGA_FP8_E4M3 is OCP E4M3FN (max 448,
 *   no infinities) with one fp32 scale per cached row. A row's value is
 *   payload * scale. Scales must be finite and positive.
 * - SGA_MXFP8_E4M3 is the MX block-32 form (fact sheet, Training: MXFP8 E4M3
 *   with one scale per 32 consecutive elements): E4M3FN payloads plus one
 *   E8M0 byte e per 32 consecutive elements of a row, worth 2^(e - 127). The
 *   scale array is uint8 [rows, D/32], row-major: 4 bytes per indexer key row
 *   (read as one 32-bit word, so 4-byte aligned) and 18 per latent row.
 *   e = 255 (NaN) is not a valid exponent. The kernels widen payload * 2^(e-127)
 *   to bf16, which is exact while the products are bf16 normals or zero, so
 *   every exponent of a nonzero block must be at least 10 (scale >= 2^-117);
 *   below that the smallest values lose bits. It must also be at most 200
 *   (values below 2^82), so that fp32 sums over up to 65,536 rows stay finite.
 * - SGA_MXFP4_E2M1 is the same block-32 form with OCP E2M1 elements (values
 *   0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), two per byte, element
 *   2i in the low nibble of byte i: 64 payload bytes per indexer key row and
 *   288 per latent row, with the same exponent arrays. Exponents of nonzero
 *   blocks must lie in [2, 200] (scale >= 2^-125; values below 2^76).
 */
#ifndef SGA_H
#define SGA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGA_API __attribute__((visibility("default")))

#define SGA_HEADS 64        /* query heads */
#define SGA_IDX_HEADS 64    /* indexer heads */
#define SGA_IDX_DIM 128     /* indexer head width = cached indexer key width */
#define SGA_D_LATENT 512    /* compressed KV latent = value width */
#define SGA_D_ROPE 64       /* shared RoPE key width */
#define SGA_D_QK 576        /* cached latent row width, absorbed query width */
#define SGA_MAX_LEN (1 << 19) /* longest visible context a query may have (512K) */
#define SGA_MAX_K 65536     /* largest top-k */
#define SGA_MAX_TOKENS 65535 /* most query tokens in one call */
#define SGA_D_V 128         /* value dimension per head (output epilogue) */
#define SGA_MAX_D_MODEL 65536 /* widest hidden state sga_output_proj takes */

typedef enum sga_status {
  SGA_OK = 0,
  SGA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, non-finite scale */
  SGA_ERR_UNSUPPORTED = 2,  /* dtype or size outside what the kernels handle */
  SGA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  SGA_ERR_HIP = 4           /* a HIP launch or query failed */
} sga_status;

typedef enum sga_dtype {
  SGA_BF16 = 0,
  SGA_FP8_E4M3 = 1,         /* OCP E4M3FN payload + fp32 scale per row */
  SGA_MXFP8_E4M3 = 2,       /* OCP E4M3FN payload + E8M0 exponent per 32 elements */
  SGA_MXFP4_E2M1 = 3        /* OCP E2M1 payload, two per byte + E8M0 exponent per 32 elements */
} sga_dtype;

/*
 * A ragged batch of query tokens over per-sequence caches stored back to back
 * in flat row arrays. Token t belongs to sequence b = token_seq[t] and sits at
 * position p = token_pos[t] (0-based) of it.
 *
 * The token sees cached rows 0..p of its sequence, its own row included.
 * Those are flat rows seq_start[b] .. seq_start[b] + p.
 *
 * The host fields are read on the host. The pointer fields point to device
 * memory and are read only by kernels. The kernels clamp what they read:
 *   visible rows n_t = min(p + 1, seq_len[b], max_len, cache_rows - seq_start[b]).
 * Inconsistent metadata therefore never reads outside the caches or writes
 * outside the outputs. It only changes which rows count as visible. A token
 * with n_t <= 0 sees nothing: its indices are all -1, its output is 0 and its
 * lse is -inf.
 */
typedef struct sga_batch {
  int32_t num_tokens;        /* (host) 0 <= T <= SGA_MAX_TOKENS; T == 0 is a no-op */
  int32_t num_seqs;          /* (host) B >= 1 when T > 0 */
  int32_t max_len;           /* (host) >= p + 1 for every token; 1..SGA_MAX_LEN */
  int32_t reserved;          /* must be 0 */
  int64_t cache_rows;        /* (host) rows in the flat caches (k_idx and kv) */
  const int32_t* token_seq;  /* [T] */
  const int32_t* token_pos;  /* [T] */
  const int64_t* seq_start;  /* [B] first flat row of each sequence */
  const int32_t* seq_len;    /* [B] rows cached for each sequence */
} sga_batch;

/*
 * Optional timing hooks for sga_forward. Each non-NULL event is recorded on
 * the call's stream at the named point. Recording an event is the only effect.
 */
typedef struct sga_trace {
  hipEvent_t indexer_begin;  /* before the indexer kernel */
  hipEvent_t indexer_end;    /* after the indexer kernel */
  hipEvent_t topk_end;       /* after the last top-k kernel launched before the attention
                                (the top-k's final stage may run inside the attention kernel) */
  hipEvent_t attn_end;       /* after the attention (and combine) kernels */
} sga_trace;

/*
 * sga_index_scores: indexer scores.
 * Source: the fact sheet's token-selection fact (a DSA-style indexer of 64
 * ReLU-scored heads of width 128) and its cached-indexer-key-width fact (128).
 *
 * For each token t and each visible position s < n_t:
 *   scores[t*ld + s] = sum_h w[t*64+h] * max(0, sum_d q_idx[t,h,d] * key[row(s), d])
 * where key = k_idx (bf16), payload * k_idx_scale[row] (fp8), or payload
 * times its 32-element block's E8M0 scale (MX).
 *   q_idx       [T,64,128] bf16, row-major.
 *   w           [T,64] fp32 head weights, 16-byte aligned (read as 16-byte
 *               vectors).
 *   k_idx       [cache_rows,128] bf16, E4M3FN or packed E2M1 payload, row-major
 *               (256, 128 or 64 B per row).
 *   k_idx_scale [cache_rows] fp32 (fp8), [cache_rows,4] uint8 E8M0 (MX, both
 *               element types, 4-byte aligned); must be NULL for bf16.
 *   scores      [T, ld] fp32, ld >= max_len. Only entries s < n_t are written.
 * Accumulation is fp32 (bf16 products are exact in fp32). With integer-valued
 * inputs every partial sum is an integer, so the scores are exact whenever
 * |score| < 2^24. For fp8 keys each head's dot product is taken over the
 * payload and then multiplied by the row scale.
 */
SGA_API sga_status sga_index_scores(const sga_batch* batch, const void* q_idx, const float* w,
                                    const void* k_idx, const void* k_idx_scale,
                                    sga_dtype k_idx_dtype, float* scores, int64_t ld,
                                    hipStream_t stream);

/*
 * sga_topk: per-token top-k selection over indexer scores.
 * Source: the fact sheet's token-selection fact (top-2048 tokens per query);
 * the rebasdaily article (at most 2,048 positions per query at any length).
 *
 * For token t, positions 0..n_t-1 are ordered by scores[t*ld + s] descending.
 * Equal scores are ordered by lower position first, and -0.0 equals +0.0.
 * The first min(k, n_t) positions are kept and written to indices[t*k ..]
 * in ascending position order, then padded with -1.
 * The result is exact: it depends only on the score values, never on
 * rounding or scheduling. Scores must not be NaN; for NaN inputs the result is
 * unspecified but stays in bounds.
 *   scores  [T, ld] fp32, ld >= max_len. Entries below max_len may be read;
 *           only s < n_t affect the result. indices [T, k] int32.
 *   ws      >= sga_topk_workspace_size(T, max_len, k) bytes.
 */
SGA_API size_t sga_topk_workspace_size(int32_t num_tokens, int32_t max_len, int32_t k);
SGA_API sga_status sga_topk(const sga_batch* batch, const float* scores, int64_t ld, int32_t k,
                            int32_t* indices, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sga_sparse_mla_attn: absorbed MLA attention over the selected latent rows,
 * with the per-head sigmoid gate applied to the output.
 * Source: the fact sheet's attention facts (64 query heads; QK dim 192 =
 * 128 NoPE + 64 RoPE; 512-wide latent and 64-wide shared RoPE key cached per
 * token; no QK norm, no QKV bias) and its gate fact (a head-specific sigmoid
 * gate on the attention output before o_proj).
 *
 * For token t, let J = the entries j of indices[t*k .. t*k+k-1] with
 * 0 <= j < n_t. Other entries, -1 included, are skipped. For each head h:
 *   z_j   = sm_scale * sum_{c<576} q_abs[t,h,c] * row_j[c],  row_j = kv[seq_start[b] + j]
 *   o     = sum_j softmax(z)_j * row_j[0:512]
 *   out[t,h,:] = o * sigmoid(gate_logits[t*64+h])   (o itself when gate_logits == NULL)
 *   lse[t*64+h] = log(sum_j exp(z_j))                (natural log)
 * An fp8 row is payload * kv_scale[row]; an MX row is each payload times its
 * 32-column block's scale. With J empty, out = 0 and lse = -inf.
 *   q_abs [T,64,576] bf16. kv [cache_rows,576] bf16, E4M3FN or packed E2M1
 *   payload (1152, 576 or 288 B per row).
 *   kv_scale [cache_rows] fp32 (fp8), [cache_rows,18] uint8 E8M0 (MX), NULL
 *   for bf16. indices [T,k] int32.
 *   out [T,64,512] fp32. lse [T,64] fp32 or NULL.
 * Logits and softmax are fp32. Probabilities enter the value product as a
 * bf16 hi/lo pair (p = hi + lo, about 16 significant bits), and accumulation
 * is fp32. When a token's rows are split over several
 * workgroups, each split's normalised output is held in fp16, scaled per head
 * and 256-column half by its largest magnitude: a column then carries, beside
 * the relative rounding, an absolute error below 2^-25 of the largest value
 * in its half of the selected rows.
 */
SGA_API size_t sga_attn_workspace_size(int32_t num_tokens, int32_t k);
SGA_API sga_status sga_sparse_mla_attn(const sga_batch* batch, const void* q_abs, const void* kv,
                                       const void* kv_scale, sga_dtype kv_dtype,
                                       const int32_t* indices, int32_t k, float sm_scale,
                                       const float* gate_logits, float* out, float* lse,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sga_forward: the whole path, indexer -> top-k -> attention -> gate, for one
 * batch.
 * Source: the fact sheet's token-selection fact (a DSA-style indexer scores
 * the cached positions and the top 2,048 are attended), its attention facts
 * (absorbed MLA over the 576-wide latent rows, 64 heads) and its gate fact
 * (a head-specific sigmoid gate before o_proj); the technical report abstract
 * and the rebasdaily article (at most 2,048 positions read per query).
 * Its results equal sga_index_scores, then sga_topk, then
 * sga_sparse_mla_attn, called with the same arguments (w, q_idx, q_abs and
 * out 16-byte aligned, as there).
 * indices_out [T,k] receives the selected positions when non-NULL.
 * trace may be NULL.
 */
SGA_API size_t sga_forward_workspace_size(int32_t num_tokens, int32_t max_len, int32_t k);
SGA_API sga_status sga_forward(const sga_batch* batch,
                               const void* q_idx, const float* w, const void* k_idx,
                               const void* k_idx_scale, sga_dtype k_idx_dtype,
                               const void* q_abs, const void* kv, const void* kv_scale,
                               sga_dtype kv_dtype, int32_t k, float sm_scale,
                               const float* gate_logits, float* out, float* lse,
                               int32_t* indices_out, void* ws, size_t ws_bytes,
                               const sga_trace* trace, hipStream_t stream);

/*
 * sga_forward_noalloc: sga_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). It takes no workspace: its scratch is a device array of
 * SGA_NOALLOC_SCRATCH_BYTES bytes inside the library, which each GPU holds
 * from the library's first use on it until the process ends. The call itself
 * allocates and frees nothing.
 * Arguments and results are those of sga_forward (same kernels, same results).
 * A problem whose sga_forward_workspace_size(T, max_len, k) exceeds
 * SGA_NOALLOC_SCRATCH_BYTES returns SGA_ERR_WORKSPACE before anything is
 * launched. The first call on a device looks up the array's address on that
 * device (the device of `stream`).
 * Every call on one GPU shares that GPU's array and leaves its last contents
 * there: calls that overlap on one GPU (different streams, or host threads
 * racing on one stream) race on the scratch and must be serialised by the
 * caller.
 */
#define SGA_NOALLOC_SCRATCH_BYTES (64u << 20)   /* 64 MiB per GPU */
SGA_API size_t sga_forward_noalloc_scratch_bytes(void);
SGA_API sga_status sga_forward_noalloc(const sga_batch* batch,
                                       const void* q_idx, const float* w, const void* k_idx,
                                       const void* k_idx_scale, sga_dtype k_idx_dtype,
                                       const void* q_abs, const void* kv, const void* kv_scale,
                                       sga_dtype kv_dtype, int32_t k, float sm_scale,
                                       const float* gate_logits, float* out, float* lse,
                                       int32_t* indices_out, const sga_trace* trace,
                                       hipStream_t stream);

/*
 * sga_cache_append: writes each token's new cached rows (the step just before
 * the path in decode).
 * Source: the FP8 model card (nlp.com.ai, "A.X K2 FP8": FP8 with dynamic
 * per-row scaling), the fact sheet's per-token cache row (512 latent + 64
 * RoPE, 128-wide indexer key) and its Training section (MXFP8, one scale per
 * 32 consecutive elements).
 *
 * Token t of sequence b at position p writes flat row r = seq_start[b] + p:
 *   kv[r]    <- latent[t]  (576 values),  when latent and kv are non-NULL;
 *   k_idx[r] <- idx_key[t] (128 values),  when idx_key and k_idx are non-NULL.
 *   latent  [T,576] bf16, idx_key [T,128] bf16, row-major, 16-byte aligned.
 * Each pair is given whole or left out whole (both NULL): one NULL and one
 * non-NULL is SGA_ERR_INVALID_ARG. Caches are 16-byte aligned, fp32 scale
 * arrays 4-byte aligned; the caller owns every buffer and the call only writes
 * the rows (and scales) named above, asynchronously on `stream`.
 * A bf16 cache gets the bits copied. An SGA_FP8_E4M3 cache gets, per row,
 *   scale = max|x| / 448 (binary32 division; 1 for a row of zeros), stored in
 *   kv_scale[r] / k_idx_scale[r], and payload = x / scale (binary32) rounded to
 *   the nearest E4M3FN value, ties to the even code, saturating at 448; the
 *   sign bit follows x (so -0 gives 0x80).
 * An SGA_MXFP8_E4M3 cache gets, per run of 32 elements, the E8M0 exponent
 *   e = clamp(floor(log2 max|x|) - 8, -127, 127) + 127 (e = 0 for a block of
 *   zeros; 8 is the exponent of 448), stored in byte r*D/32 + block of the
 *   scale array, and payload = x * 2^(127 - e) encoded as above.
 * An SGA_MXFP4_E2M1 cache gets e = clamp(floor(log2 max|x|) - 2, -127, 127)
 *   + 127 (2 is the exponent of 6) and payload = x * 2^(127 - e) rounded to
 *   the nearest E2M1 value, ties to the even code, saturating at 6, packed two
 *   per byte, low nibble first.
 * The scale arrays must be NULL for a bf16 cache and non-NULL otherwise.
 * A token with b outside [0, num_seqs), p outside [0, seq_len[b]) or r outside
 * [0, cache_rows) writes nothing. Tokens writing the same row race; the
 * caller keeps rows distinct. max_len is checked as for the other calls but
 * not otherwise used. Inputs must be finite.
 */
SGA_API sga_status sga_cache_append(const sga_batch* batch, const void* latent, const void* idx_key,
                                    void* kv, void* kv_scale, sga_dtype kv_dtype, void* k_idx,
                                    void* k_idx_scale, sga_dtype k_idx_dtype, hipStream_t stream);

/*
 * sga_indexer_loss: the sparse indexer loss of each token.
 * Source: the technical report abstract (the indexer is warmed up against its
 * own sparse top-k selection rather than the dense attention distribution)
 * and the fact sheet's Training section (an indexer-only sparse warmup, then
 * joint training with the indexer loss down-weighted). The loss form is not
 * printed; this is the DSA-style reading restricted to the selected set.
 *
 * For token t let S = the entries j of indices[t*k ..] with 0 <= j < n_t.
 *   p[j] = (1/64) sum_h exp(z_h,j - lse[t*64+h]),  z_h,j = sm_scale * q_abs[t,h,:] . row_j
 *   q[j] = exp(scores[t*ld + j]) / sum_{i in S} exp(scores[t*ld + i])
 *   loss[t] = sum_{j in S, p[j] > 0} p[j] * (log p[j] - log q[j])     (KL(p || q))
 * lse must be the attention's own output for the same indices (then p sums to
 * one over S); scores are sga_index_scores' output ([T, ld], ld >= max_len).
 * A token with S empty gets loss 0. q_abs, kv, kv_scale, kv_dtype, indices,
 * k and sm_scale are as for sga_sparse_mla_attn. fp32 throughout.
 *   ws >= sga_indexer_loss_workspace_size(T, k) bytes.
 */
SGA_API size_t sga_indexer_loss_workspace_size(int32_t num_tokens, int32_t k);
SGA_API sga_status sga_indexer_loss(const sga_batch* batch, const void* q_abs, const void* kv,
                                    const void* kv_scale, sga_dtype kv_dtype, const int32_t* indices,
                                    int32_t k, float sm_scale, const float* lse, const float* scores,
                                    int64_t ld, float* loss, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/*
 * sga_output_proj: the output epilogue after the gate, for T tokens.
 * Source: the fact sheet's attention facts (value dimension per head 128;
 * hidden state 7,168; the head-specific gate acts on the attention output
 * before o_proj).
 *
 *   u[t, h, v] = sum_c w_uv[h, v, c] * o_latent[t, h, c]      (c < 512, v < 128)
 *   y[t, n]    = sum_j w_o[n, j] * u[t, j],  j = h * 128 + v  (n < d_model)
 *   o_latent [T,64,512] fp32: the gated output of sga_forward / sga_sparse_mla_attn.
 *   w_uv     [64,128,512] bf16: head h's value up-projection, row-major
 *            (output x input, the layout of a linear layer's weight).
 *   w_o      [d_model, 8192] bf16: the output projection, row-major (output x input).
 *   y        [T, d_model] fp32.
 *   ws       >= sga_output_proj_workspace_size(T, d_model) bytes.
 * d_model must be a positive multiple of 64, at most SGA_MAX_D_MODEL
 * (SGA_ERR_UNSUPPORTED otherwise). All four arrays are 16-byte aligned.
 * Activations enter the bf16 products as a hi/lo pair (about 16 bits) and
 * accumulation is fp32; the sum over K is split in a fixed way and added in a
 * fixed order, so results are deterministic.
 */
SGA_API size_t sga_output_proj_workspace_size(int32_t num_tokens, int32_t d_model);
SGA_API sga_status sga_output_proj(int32_t num_tokens, const float* o_latent, const void* w_uv,
                                   const void* w_o, int32_t d_model, float* y, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * sga_hbm_read_probe: a measurement helper, not a step of the method. Reads
 * the `bytes` bytes at device address `src` once, as the indexer reads its
 * keys (1 KiB of contiguous memory per wave instruction, streaming cache
 * policy, one contiguous chunk per workgroup, 1,024 workgroups), and folds
 * them into a value that is written to the device buffer `sink` only in a
 * case no input is expected to meet (sink must hold 262,144 uint32 words;
 * its contents are unspecified afterwards). Timing it gives the HBM read rate
 * this GPU reaches. bytes: a nonzero multiple of 4,096, with at most about
 * 4 GiB per workgroup chunk (SGA_ERR_UNSUPPORTED beyond). Asynchronous on
 * `stream`; the caller keeps src and sink alive until it completes.
 */
SGA_API sga_status sga_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink,
                                      hipStream_t stream);

/* Human-readable name of a status code (static string). */
SGA_API const char* sga_status_string(sga_status status);
/* Library version as major*10000 + minor*100 + patch. */
SGA_API int sga_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SGA_H */
