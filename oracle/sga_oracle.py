"""Plain, slow, float64 CPU oracle for the Sparse Gated Attention (SGA) hot path.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call or run this module. It shares no code with
the HIP library or its Python binding, and imports neither.

What it computes, and the passages it follows:

* Visibility. A query token at position p of its sequence sees the cached rows
  0..p, its own row included. The A.X K2 fact sheet (archdb.vladsavinov.com,
  "A.X K2") lists every layer as a global, full-context MLA layer. The news
  article (rebasdaily, section on long tasks that cannot re-read all old
  content) says each query reads at most 2,048 positions whatever the context
  length.
* Indexer (fact sheet, fact "token-selection mechanism inside global layers":
  a DSA-style indexer with 64 ReLU-scored heads of width 128; fact "width of the
  sparse-attention indexer key cached per token": 128). The score of cached
  position s for query t is I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]).
  The pages print no formula; this is the DSA-style form with per-query head
  weights.
* Top-k (same fact: top-2048 positions per query; news article: at most 2,048).
  Positions are ordered by score (descending), with equal scores ordered by
  lower position first. The first min(k, visible) positions are kept. They
  are returned in ascending position order, padded with -1.
* Absorbed MLA attention over the kept rows (fact sheet facts: 64 query heads;
  QK dim per head 192 = 128 NoPE + 64 RoPE; compressed KV latent 512; shared
  positional key 64; no QK normalisation; no QKV bias). Each cached row holds
  576 values: latent (512) then RoPE key (64). The absorbed query of head h
  also has 576 values. Logit z_j = sm_scale * q[h] . row_j over all 576
  columns. Values are the first 512 columns only (the latent). The output
  stays in latent space. The softmax is over the kept rows. lse is the natural
  log-sum-exp of z.
* Gate (fact sheet fact "gate applied to the attention output before the output
  projection": a head-specific sigmoid gate projected jointly with the query;
  the nlp.com.ai "A.X K2 FP8" summary says it is meant to suppress attention
  sinks). out[h,:] = o[h,:] * 1/(1+exp(-g[h])), one logit per (token, head).
  The gate multiplies each head's output by one scalar, and the later per-head
  value up-projection is linear. So gating the latent-space output is the same
  as gating after the up-projection.

Storage formats decoded here from their bit-level definitions:
- bf16: the upper 16 bits of an IEEE-754 binary32;
- OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; a zero
  exponent field is subnormal; S.1111.111 is NaN; there is no infinity.
An fp8 row's value is its decoded payload times its fp32 row scale.

Cache append (the step just before the path in decode; FP8 model card
(nlp.com.ai, "A.X K2 FP8"): FP8 with dynamic, per-row activation scaling).
The new token's 576-wide latent row and 128-wide indexer key go into row
seq_start[b] + p of their caches. For an fp8 cache the row scale is
max|x| / 448 and each payload is x / scale rounded to the nearest E4M3FN value,
ties to the even code, saturating at 448; both divisions are done in binary32,
the precision the stored scale has. A row of zeros gets scale 1. -0 and
negative values that round to zero keep the sign bit.

MX block-32 cache (fact sheet, Training: MXFP8 E4M3 with one scale per 32
consecutive elements). The pages give only the granularity; the block rule
taken here is the Open Compute Project MX format's: each run of 32 elements
shares one E8M0 scale 2^(e - 127) (e = 0..254; e = 255 is NaN), with
e - 127 = floor(log2(max|x|)) - 8, 8 being the exponent of E4M3FN's largest
normal (448 = 1.75 * 2^8), clamped to [-127, 127]; a block of zeros gets
e = 0. Each element is x / 2^(e - 127) rounded to the nearest E4M3FN value,
ties to the even code, saturating at 448 (a block whose maximum lies in
(448, 512) * 2^(e - 127) has its largest elements clamped). The value of a
stored element is its payload times its block's scale.

MX block-32 with 4-bit elements (the FP4 member of the same family; the pages
cite 4-bit serving): OCP E2M1 elements (1 sign bit, 2 exponent bits with bias
1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with the
lower-indexed element in the low nibble, and one E8M0 exponent per 32
elements with e - 127 = floor(log2(max|x|)) - 2 (2 = exponent of E2M1's
largest value, 6 = 1.5 * 2^2), clamped and zero-block handled as above;
elements nearest-even, saturating at 6.

Sparse indexer loss (technical report abstract: the indexer is warmed up
against its own sparse top-k selection rather than the dense attention
distribution; fact sheet, Training: an indexer-only sparse warmup, then joint
training with the indexer loss down-weighted). The loss form is not printed;
the reading taken is the DSA-style one restricted to the selected set S_t of
query t: the target p_t is the main attention's distribution over S_t,
averaged over the heads (each head's softmax of its logits over S_t), the
indexer's distribution q_t is the softmax of its scores over S_t, and the loss
is KL(p_t || q_t) = sum_s p_t[s] (log p_t[s] - log q_t[s]), one value per query.

Output epilogue (fact sheet facts: value dimension per head 128; hidden state
7,168; the gate sits on the attention output before o_proj). In the absorbed
form the attention output of head h stays in the 512-wide latent space; the
value up-projection of head h (128 x 512) takes it to the head's 128 value
columns, and the output projection (d_model x (64 * 128)) maps the 64 heads'
values, concatenated head-major, to the hidden state:
    u[t, h, :] = W_UV[h] @ o[t, h, :]     y[t, :] = W_O @ u[t].reshape(64 * 128)
Weights are given as bf16 in the row-major (output x input) layout of a
linear layer. o is the gated output, so the gate acts before o_proj.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = ["decode_bf16", "e4m3fn_table", "decode_e4m3fn", "Store", "index_scores",
           "select_topk", "sparse_mla", "sigmoid_gate", "forward", "D_LATENT",
           "encode_e4m3fn", "quantize_rows_e4m3fn", "cache_append", "e8m0_table", "MX_BLOCK",
           "quantize_blocks_mxfp8", "decode_mxfp8", "D_V", "output_projection",
           "e2m1_table", "encode_e2m1", "quantize_blocks_mxfp4", "decode_mxfp4",
           "sparse_indexer_loss", "indexer_loss"]

D_LATENT = 512
D_V = 128        # value dimension per head (fact sheet)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: a bf16 is the top half of a binary32."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """The 256 values of OCP E4M3FN, built from the format's field definition."""
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            table[code] = np.nan
        elif e == 0:
            table[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            table[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return table


_E4M3 = e4m3fn_table()


# the finite non-negative E4M3FN codes (0x00..0x7E) in increasing value
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALS = _E4M3[:0x7F]


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Each value to the nearest E4M3FN code, ties to the even code, |x| > 448
    saturating to 448; the sign bit follows the sign of x (-0 included)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), _POS_VALS[-1])
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(d_hi == 0, _POS_CODES[hi], code).astype(np.uint8)   # exact values
    return code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0)).astype(np.uint8)


def quantize_rows_e4m3fn(x: np.ndarray):
    """Rows [n, D] (binary32 values) -> (uint8 payloads [n, D], float32 scales [n]).
    scale = max|x| / 448 in binary32 (1 for a zero row); payload = E4M3FN(x / scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (x / scale[:, None]).astype(np.float32)
    return encode_e4m3fn(q), scale


MX_BLOCK = 32


def e8m0_table() -> np.ndarray:
    """The 256 values of E8M0 (an unsigned power-of-two exponent, bias 127; 255 is NaN)."""
    t = np.ldexp(1.0, np.arange(256) - 127)
    t[255] = np.nan
    return t


_E8M0 = e8m0_table()


def quantize_blocks_mxfp8(x: np.ndarray):
    """Rows [n, D] (D a multiple of 32) -> (uint8 E4M3FN payloads [n, D], uint8
    E8M0 block exponents [n, D/32]), one exponent per 32 consecutive elements."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    blocks = x.reshape(n, d // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    exps = np.zeros(amax.shape, dtype=np.uint8)
    nz = amax > 0
    _, e2 = np.frexp(amax[nz])                        # amax = f * 2^e2, f in [0.5, 1)
    exps[nz] = np.clip(e2 - 1 - 8, -127, 127) + 127   # floor(log2 amax) - 8, biased
    scale = _E8M0[exps]                               # 2^(e - 127)
    payload = encode_e4m3fn(blocks / scale[:, :, None]).reshape(n, d)
    return payload, exps


def e2m1_table() -> np.ndarray:
    """The 16 values of OCP E2M1, built from the format's field definition."""
    t = np.empty(16, dtype=np.float64)
    for c in range(16):
        e, m = (c >> 1) & 3, c & 1
        v = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        t[c] = -v if c & 8 else v
    return t


_E2M1 = e2m1_table()


def encode_e2m1(x: np.ndarray) -> np.ndarray:
    """Each value to the nearest E2M1 code (uint8 0..15), ties to the even code,
    |x| > 6 saturating to 6; the sign bit follows the sign of x."""
    x = np.asarray(x, dtype=np.float64)
    mags = _E2M1[:8]
    a = np.minimum(np.abs(x), mags[-1])
    d = np.abs(a[..., None] - mags)                    # distance to each magnitude code
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # ties: the even code (of two equidistant codes exactly one is even)
    even = cand & (np.arange(8) % 2 == 0)
    code = np.where(cand.sum(axis=-1) > 1, np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def quantize_blocks_mxfp4(x: np.ndarray):
    """Rows [n, D] (D a multiple of 32) -> (uint8 packed E2M1 payloads [n, D/2],
    element 2i in the low nibble of byte i; uint8 E8M0 exponents [n, D/32])."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    blocks = x.reshape(n, d // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    exps = np.zeros(amax.shape, dtype=np.uint8)
    nz = amax > 0
    _, e2 = np.frexp(amax[nz])
    exps[nz] = np.clip(e2 - 1 - 2, -127, 127) + 127   # floor(log2 amax) - 2, biased
    codes = encode_e2m1(blocks / _E8M0[exps][:, :, None]).reshape(n, d)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), exps


def decode_mxfp4(payload: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """uint8 packed payload rows [n, D/2] and E8M0 exponents [n, D/32] -> float64 [n, D]."""
    p = np.asarray(payload, dtype=np.uint8)
    n, half = p.shape
    codes = np.empty((n, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    vals = _E2M1[codes].reshape(n, 2 * half // MX_BLOCK, MX_BLOCK)
    return (vals * _E8M0[np.asarray(exps, dtype=np.uint8)][:, :, None]).reshape(n, 2 * half)


def decode_mxfp8(payload: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """uint8 payload rows [n, D] and E8M0 block exponents [n, D/32] -> float64 [n, D]."""
    p = np.asarray(payload, dtype=np.uint8)
    n, d = p.shape
    vals = _E4M3[p].reshape(n, d // MX_BLOCK, MX_BLOCK)
    return (vals * _E8M0[np.asarray(exps, dtype=np.uint8)][:, :, None]).reshape(n, d)


def cache_append(token_seq, token_pos, seq_start, seq_len, cache_rows: int, rows: np.ndarray,
                 fmt: str):
    """The rows the append writes: {cache row: (payload row, scale or None)}.
    rows: [T, D] bf16 bit patterns (uint16). fmt: "bf16" (copied bits),
    "e4m3fn" (quantised per row; the scale is a float32), "mxfp8" or "mxfp4"
    (quantised per 32-element block; the scale is the row's uint8 E8M0
    exponents, the mxfp4 payload two elements per byte). A token
    whose position lies outside its sequence's rows, or whose row lies outside
    the cache, writes nothing."""
    out = {}
    vals = decode_bf16(rows).astype(np.float32)
    for t in range(len(token_seq)):
        b, p = int(token_seq[t]), int(token_pos[t])
        if b < 0 or b >= len(seq_len) or p < 0 or p >= int(seq_len[b]):
            continue
        r = int(seq_start[b]) + p
        if r < 0 or r >= cache_rows:
            continue
        if fmt == "bf16":
            out[r] = (np.asarray(rows[t], dtype=np.uint16).copy(), None)
        elif fmt == "mxfp8":
            pay, ex = quantize_blocks_mxfp8(vals[t:t + 1])
            out[r] = (pay[0], ex[0])
        elif fmt == "mxfp4":
            pay, ex = quantize_blocks_mxfp4(vals[t:t + 1])
            out[r] = (pay[0], ex[0])
        else:
            pay, sc = quantize_rows_e4m3fn(vals[t:t + 1])
            out[r] = (pay[0], np.float32(sc[0]))
    return out


def decode_e4m3fn(payload: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """uint8 payload rows [n, D] and fp32 row scales [n] -> float64 [n, D]."""
    vals = _E4M3[np.asarray(payload, dtype=np.uint8)]
    return vals * np.asarray(scale, dtype=np.float64)[:, None]


@dataclass
class Store:
    """A flat cache: raw bits per row plus the format ('bf16', 'e4m3fn', 'mxfp8' or 'mxfp4')."""
    bits: np.ndarray                  # uint16 [rows, D] (bf16), uint8 [rows, D] (e4m3fn, mxfp8)
                                      # or uint8 [rows, D/2] (mxfp4, two elements per byte)
    fmt: str
    scale: Optional[np.ndarray] = None  # float32 [rows] (e4m3fn) or uint8 [rows, D/32] (mx)

    def rows(self, idx) -> np.ndarray:
        if self.fmt == "bf16":
            return decode_bf16(self.bits[idx])
        if self.fmt == "e4m3fn":
            return decode_e4m3fn(self.bits[idx], self.scale[idx])
        if self.fmt == "mxfp8":
            return decode_mxfp8(self.bits[idx], self.scale[idx])
        if self.fmt == "mxfp4":
            return decode_mxfp4(self.bits[idx], self.scale[idx])
        raise ValueError(self.fmt)


def index_scores(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """One query's indexer scores over `keys`.

    q_idx [H, D] indexer query heads, w [H] head weights, keys [n, D] -> [n].
    The per-head dot products are clipped at zero first, then weighted and summed.
    """
    dots = keys.astype(np.float64) @ q_idx.astype(np.float64).T      # [n, H]
    return np.maximum(dots, 0.0) @ w.astype(np.float64)              # [n]


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Keep the first min(k, n) positions in the order (score desc, position asc).

    Returns int32 [k]: the kept positions in ascending order, then -1 padding.
    -0.0 and +0.0 compare equal, so they tie and the tie goes to the lower position.
    """
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -np.asarray(scores, dtype=np.float64)))
    kept = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[:kept.shape[0]] = kept
    return out


def sparse_mla(q_abs: np.ndarray, rows: np.ndarray, sm_scale: float, d_v: int = D_LATENT):
    """Absorbed MLA attention of one query over the gathered cache rows.

    q_abs [H, 576], rows [m, 576] -> (o [H, d_v], lse [H]). With no rows the
    output is zero and lse is -inf.
    """
    H = q_abs.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    z = float(sm_scale) * (q_abs.astype(np.float64) @ rows.T)      # [H, m]
    zmax = z.max(axis=1)
    e = np.exp(z - zmax[:, None])
    denom = e.sum(axis=1)
    o = (e @ rows[:, :d_v]) / denom[:, None]
    lse = zmax + np.log(denom)
    return o, lse


def sigmoid_gate(o: np.ndarray, g: np.ndarray) -> np.ndarray:
    """out[h, :] = o[h, :] * sigmoid(g[h])."""
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))
    return o * sig[:, None]


def forward(token_seq, token_pos, seq_start, seq_len, q_idx, w, k_store: Store,
            q_abs, kv_store: Store, gate, k: int, sm_scale: float,
            tokens: Optional[Sequence[int]] = None, keep_scores: bool = False) -> dict:
    """Indexer -> top-k -> sparse MLA -> gate, one query token at a time.

    q_idx [T,H,128], w [T,H], q_abs [T,H,576], gate [T,H] or None (ungated).
    Returns indices int32 [n,k], out float64 [n,H,512], lse float64 [n,H] for
    the chosen tokens (all by default), and optionally the score rows.
    """
    T = len(token_pos)
    tokens = list(range(T)) if tokens is None else list(tokens)
    H = q_abs.shape[1]
    res = {"tokens": tokens,
           "indices": np.full((len(tokens), k), -1, dtype=np.int32),
           "out": np.zeros((len(tokens), H, D_LATENT)),
           "lse": np.full((len(tokens), H), -np.inf)}
    if keep_scores:
        res["scores"] = []
    for i, t in enumerate(tokens):
        b = int(token_seq[t])
        p = int(token_pos[t])
        assert p < int(seq_len[b]), "a token must sit inside its sequence"
        base = int(seq_start[b])
        n = p + 1                                         # rows 0..p are visible
        keys = k_store.rows(slice(base, base + n))
        scores = index_scores(np.asarray(q_idx[t], np.float64), np.asarray(w[t], np.float64), keys)
        idx = select_topk(scores, k)
        kept = idx[idx >= 0].astype(np.int64)
        o, lse = sparse_mla(np.asarray(q_abs[t], np.float64), kv_store.rows(base + kept), sm_scale)
        res["indices"][i] = idx
        res["out"][i] = o if gate is None else sigmoid_gate(o, gate[t])
        res["lse"][i] = lse
        if keep_scores:
            res["scores"].append(scores)
    return res


def output_projection(o: np.ndarray, w_uv: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """Gated latent outputs o [T, H, 512], value up-projections w_uv [H, 128, 512]
    and output projection w_o [d_model, H * 128] (float64 values of the bf16
    weights) -> hidden-state outputs [T, d_model]."""
    o = np.asarray(o, dtype=np.float64)
    T, H, _ = o.shape
    u = np.empty((T, H, D_V), dtype=np.float64)
    for h in range(H):
        u[:, h, :] = o[:, h, :] @ np.asarray(w_uv[h], dtype=np.float64).T
    return u.reshape(T, H * D_V) @ np.asarray(w_o, dtype=np.float64).T


def sparse_indexer_loss(q_abs: np.ndarray, rows: np.ndarray, sm_scale: float,
                        scores_sel: np.ndarray) -> float:
    """KL(p || q) over one query's selected rows: p is the head-mean of each
    head's attention softmax over the rows (logits sm_scale * q_abs[h] . row),
    q the softmax of the indexer scores of the same rows. q_abs [H, 576],
    rows [m, 576], scores_sel [m]. An empty selection gives 0."""
    if rows.shape[0] == 0:
        return 0.0
    z = sm_scale * (np.asarray(q_abs, dtype=np.float64) @ np.asarray(rows, dtype=np.float64).T)   # [H, m]
    ph = np.exp(z - z.max(axis=1, keepdims=True))
    ph /= ph.sum(axis=1, keepdims=True)
    p = ph.mean(axis=0)
    i = np.asarray(scores_sel, dtype=np.float64)
    log_q = i - (i.max() + np.log(np.exp(i - i.max()).sum()))
    pos = p > 0
    return float(np.sum(p[pos] * (np.log(p[pos]) - log_q[pos])))


def indexer_loss(token_seq, token_pos, seq_start, seq_len, q_idx, w, k_store: "Store", q_abs,
                 kv_store: "Store", k: int, sm_scale: float, tokens: Optional[Sequence[int]] = None):
    """The sparse indexer loss of each token: its scores, its top-k set, then
    sparse_indexer_loss over that set. Returns float64 [T] (or [len(tokens)])."""
    sel = range(len(token_seq)) if tokens is None else tokens
    out = []
    for t in sel:
        b, p = int(token_seq[t]), int(token_pos[t])
        n = min(p + 1, int(seq_len[b]))
        base = int(seq_start[b])
        scores = index_scores(q_idx[t], w[t], k_store.rows(np.arange(base, base + n)))
        idx = select_topk(scores, k)
        idx = idx[idx >= 0]
        out.append(sparse_indexer_loss(q_abs[t], kv_store.rows(base + idx), sm_scale, scores[idx]))
    return np.asarray(out, dtype=np.float64)
