"""Seeded synthetic workloads for the Sparse Gated Attention (SGA) hot path.

This module draws inputs only. It holds none of the method's arithmetic (no
scoring, selection, softmax or gating). Both the CPU oracle and the GPU path
read what it returns.

The shapes follow the A.X K2 fact sheet (archdb.vladsavinov.com, "A.X K2"):
- 64 query heads; 512-wide compressed KV latent plus a 64-wide shared RoPE key;
- an indexer with 64 heads of width 128 and a 128-wide cached indexer key;
- top-2048 selection.
The pages measure long context on RULER and LongBench. No item of those suites
is used here. Seeded random caches of the same context shapes (128K native,
256K extended) stand in for them.

Value recipe:
- indexer keys and queries: integers drawn uniformly from [-3, 3], stored as bf16
  (exact);
- indexer head weights: integers drawn uniformly from [0, 4], fp32;
- latent cache: N(0,1)/24 (24 = sqrt(576)), rounded to bf16 by round-to-nearest-even;
- absorbed queries: N(0,1) in bf16;
- gate logits: normal with sigma 2, fp32;
- softmax scale: 1/sqrt(192).
With these integer indexer inputs every score is an integer below 2**24, so
fp32 scores are exact and the selected index sets can be compared bit for bit.

fp8 caches use OCP E4M3FN with one fp32 scale per cached row:
- latent rows: scale = max|x| / 448, payload = round-to-nearest-even(x / scale);
- indexer keys: payload = the integer itself, scale = 2**u with u drawn
  uniformly from [-2, 2].
Power-of-two scales keep the scores exact.

MX block-32 caches (E4M3FN payloads, one E8M0 exponent per 32 elements) are
drawn in their stored form:
- latent rows: each block's exponent e is drawn uniformly from [118, 121]
  (scales 2^-9 .. 2^-6) and its payload is the N(0,1)/24 draw divided by
  2^(e - 127), cast to E4M3FN (nearest even, clamped to 448);
- indexer keys: payload = the integer itself, each block's exponent 127 + u
  with u drawn uniformly from [-2, 2].
The same with four-bit E2M1 elements (two per byte, low nibble first):
- latent rows: every element's code drawn uniformly from the 16 E2M1 codes,
  each block's exponent uniform in [119, 120];
- indexer keys: the E2M1 code of the integer (0, 1, 2, 3 are codes 0, 2, 4,
  5, negatives add the sign bit 8), exponents as above.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

N_HEADS = 64          # query heads (A.X K2 fact sheet: query heads in global layers)
IDX_HEADS = 64        # indexer heads
IDX_DIM = 128         # indexer head width = cached indexer key width
D_LATENT = 512        # compressed KV latent width
D_ROPE = 64           # shared positional key width
D_QK = D_LATENT + D_ROPE  # 576-wide cached row used by the absorbed query
TOP_K = 2048
SM_SCALE = 1.0 / math.sqrt(192.0)  # QK head dim 192 = 128 NoPE + 64 RoPE
E4M3_MAX = 448.0

CONFIG_NAMES = ("tiny_decode_4k", "batched_decode_ragged_16k_32k",
                "long_decode_128k", "chunked_prefill_128k", "extended_decode_256k_fp8",
                "extended_decode_256k_mxfp8", "extended_decode_256k_mxfp4")


@dataclass
class Workload:
    name: str
    seq_len: np.ndarray      # int32 [B]
    seq_start: np.ndarray    # int64 [B]
    token_seq: np.ndarray    # int32 [T]
    token_pos: np.ndarray    # int32 [T]
    q_idx: torch.Tensor      # bf16 [T, 64, 128]
    w: torch.Tensor          # fp32 [T, 64]
    k_idx: torch.Tensor      # bf16 or float8_e4m3fn [rows, 128], or uint8 [rows, 64] (E2M1 pairs)
    k_idx_scale: Optional[torch.Tensor]  # fp32 [rows] (fp8), uint8 [rows, 4] (MX), else None
    kv: torch.Tensor         # bf16 or float8_e4m3fn [rows, 576], or uint8 [rows, 288] (E2M1 pairs)
    kv_scale: Optional[torch.Tensor]     # fp32 [rows] (fp8), uint8 [rows, 18] (MX), else None
    q_abs: torch.Tensor      # bf16 [T, 64, 576]
    gate: torch.Tensor       # fp32 [T, 64]
    k: int = TOP_K
    sm_scale: float = SM_SCALE
    meta: dict = field(default_factory=dict)

    @property
    def num_tokens(self) -> int:
        return int(self.token_pos.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def cache_rows(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_len(self) -> int:
        if self.num_tokens == 0:
            return 1
        return int(self.token_pos.max()) + 1

    @property
    def cache_fmt(self) -> str:
        """The format name the oracle's Store uses: bf16, e4m3fn, mxfp8 or mxfp4."""
        return self.meta.get("fmt", "bf16")

    @property
    def fp8(self) -> bool:
        """Narrow payloads with scales (E4M3FN per row, or an MX format)."""
        return self.cache_fmt != "bf16"

    @property
    def mx(self) -> bool:
        return self.cache_fmt in ("mxfp8", "mxfp4")


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _to_e4m3(x: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)


def _quantize_rows_e4m3(x: np.ndarray):
    """Per-row scale = max|x|/448; payload = RNE(x/scale), saturating."""
    amax = np.abs(x).max(axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return _to_e4m3(x / scale[:, None]), torch.from_numpy(scale)


def build(name: str, lengths: Sequence[int], tokens: Sequence[tuple], seed: int, *,
          fp8: bool = False, kv_sigma: float = 1.0 / 24.0, q_abs_mult: float = 1.0,
          idx_range: int = 3, w_range: tuple = (0, 4), gate_sigma: float = 2.0,
          k: int = TOP_K, sm_scale: float = SM_SCALE, chunk_rows: int = 1 << 16,
          mx: bool = False, mx4: bool = False) -> Workload:
    """Draw one workload.

    lengths: cached rows per sequence. tokens: (sequence, position) per query token.
    Draw order: lengths are given; then indexer keys, indexer queries, head
    weights, latent cache (with each chunk's block exponents for MX), absorbed
    queries, gate logits, fp8 key-scale exponents. mx: MX block-32 caches
    with E4M3FN elements; mx4: with four-bit E2M1 elements.
    """
    fmt = "mxfp4" if mx4 else ("mxfp8" if mx else ("e4m3fn" if fp8 else "bf16"))
    fp8 = fmt != "bf16"
    mx = fmt in ("mxfp8", "mxfp4")
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = int(lengths.shape[0])
    rows = int(lengths.sum())
    seq_start = np.zeros(B, dtype=np.int64)
    if B > 1:
        seq_start[1:] = np.cumsum(lengths)[:-1]
    token_seq = np.asarray([t[0] for t in tokens], dtype=np.int32)
    token_pos = np.asarray([t[1] for t in tokens], dtype=np.int32)
    T = int(token_seq.shape[0])

    # indexer keys, drawn in row chunks (integers in [-idx_range, idx_range])
    k_parts = []
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        k_parts.append(rng.integers(-idx_range, idx_range + 1, size=(r1 - r0, IDX_DIM), dtype=np.int8))
    k_int = np.concatenate(k_parts) if k_parts else np.zeros((0, IDX_DIM), np.int8)
    q_idx = rng.integers(-idx_range, idx_range + 1, size=(T, IDX_HEADS, IDX_DIM)).astype(np.float32)
    w = rng.integers(w_range[0], w_range[1] + 1, size=(T, IDX_HEADS)).astype(np.float32)

    kv_parts, kv_scale_parts = [], []
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal(size=(r1 - r0, D_QK), dtype=np.float32)
        x *= np.float32(kv_sigma)
        if mx4:
            codes = rng.integers(0, 16, size=(r1 - r0, D_QK), dtype=np.uint8)
            e = rng.integers(119, 121, size=(r1 - r0, D_QK // 32))
            kv_parts.append(torch.from_numpy((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)))
            kv_scale_parts.append(torch.from_numpy(e.astype(np.uint8)))
        elif mx:
            e = rng.integers(118, 122, size=(r1 - r0, D_QK // 32))
            inv = np.ldexp(np.float32(1.0), 127 - e).astype(np.float32)
            kv_parts.append(_to_e4m3(x * np.repeat(inv, 32, axis=1)))
            kv_scale_parts.append(torch.from_numpy(e.astype(np.uint8)))
        elif fp8:
            p, s = _quantize_rows_e4m3(x)
            kv_parts.append(p)
            kv_scale_parts.append(s)
        else:
            kv_parts.append(_bf16(x))
    if kv_parts:
        kv = torch.cat(kv_parts)
    elif mx4:
        kv = torch.zeros((0, D_QK // 2), dtype=torch.uint8)
    else:
        kv = torch.zeros((0, D_QK), dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16)
    if mx:
        kv_scale = torch.cat(kv_scale_parts) if kv_scale_parts else torch.zeros((0, D_QK // 32), dtype=torch.uint8)
    else:
        kv_scale = (torch.cat(kv_scale_parts) if kv_scale_parts else torch.zeros(0)) if fp8 else None

    q_abs = rng.standard_normal(size=(T, N_HEADS, D_QK), dtype=np.float32) * np.float32(q_abs_mult)
    gate = (rng.standard_normal(size=(T, N_HEADS)) * gate_sigma).astype(np.float32)

    if mx4:
        u = rng.integers(-2, 3, size=(rows, IDX_DIM // 32))
        mag = np.array([0, 2, 4, 5], dtype=np.uint8)[np.abs(k_int)]     # E2M1 codes of 0..3
        codes = mag | np.where(k_int < 0, np.uint8(8), np.uint8(0)).astype(np.uint8)
        k_idx = torch.from_numpy((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
        k_idx_scale = torch.from_numpy((127 + u).astype(np.uint8))
    elif mx:
        u = rng.integers(-2, 3, size=(rows, IDX_DIM // 32))
        k_idx = _to_e4m3(k_int.astype(np.float32))
        k_idx_scale = torch.from_numpy((127 + u).astype(np.uint8))
    elif fp8:
        u = rng.integers(-2, 3, size=rows)
        k_idx = _to_e4m3(k_int.astype(np.float32))
        k_idx_scale = torch.from_numpy(np.ldexp(np.float32(1.0), u).astype(np.float32))
    else:
        k_idx = torch.from_numpy(k_int.astype(np.float32)).to(torch.bfloat16)
        k_idx_scale = None

    return Workload(name=name, seq_len=lengths.astype(np.int32), seq_start=seq_start,
                    token_seq=token_seq, token_pos=token_pos, q_idx=_bf16(q_idx),
                    w=torch.from_numpy(w), k_idx=k_idx, k_idx_scale=k_idx_scale, kv=kv,
                    kv_scale=kv_scale, q_abs=_bf16(q_abs), gate=torch.from_numpy(gate),
                    k=k, sm_scale=sm_scale, meta={"seed": seed, "fmt": fmt})


def append_rows(num_tokens: int, seed: int, *, kv_sigma: float = 1.0 / 24.0, key_sigma: float = 1.0,
                spread: int = 8):
    """New cache rows for a cache append: latent rows [T, 576] and indexer keys
    [T, 128], both bf16. Each row is N(0, sigma^2) times 2**u with u drawn
    uniformly from [-spread, spread], so the per-row fp8 scales span a wide
    range. Draw order: latent normals, latent exponents, key normals, key exponents."""
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal(size=(num_tokens, D_QK), dtype=np.float32) * np.float32(kv_sigma)
    lat *= np.ldexp(np.float32(1.0), rng.integers(-spread, spread + 1, size=(num_tokens, 1))).astype(np.float32)
    key = rng.standard_normal(size=(num_tokens, IDX_DIM), dtype=np.float32) * np.float32(key_sigma)
    key *= np.ldexp(np.float32(1.0), rng.integers(-spread, spread + 1, size=(num_tokens, 1))).astype(np.float32)
    return _bf16(lat), _bf16(key)


D_V = 128             # value dimension per head (fact sheet)
D_MODEL = 7168        # hidden state (fact sheet)


def proj_weights(seed: int, d_model: int = D_MODEL):
    """Synthetic output-epilogue weights in bf16: the value up-projections
    w_uv [64, 128, 512] ~ N(0, 1/512) and the output projection
    w_o [d_model, 64 * 128] ~ N(0, 1/8192), in that draw order."""
    rng = np.random.default_rng(seed)
    w_uv = rng.standard_normal((N_HEADS, D_V, D_LATENT), dtype=np.float32) / np.float32(math.sqrt(D_LATENT))
    w_o = rng.standard_normal((d_model, N_HEADS * D_V), dtype=np.float32) / np.float32(math.sqrt(N_HEADS * D_V))
    return _bf16(w_uv), _bf16(w_o)


def config(i: int, seed: Optional[int] = None) -> Workload:
    """The five workloads, then the 256K decode with MX block-32 caches of E4M3FN
    (6th) and of four-bit E2M1 elements (7th).
    The seed defaults to the workload's number."""
    s = i if seed is None else seed
    if i == 0:   # tiny decode: 1 sequence of 4096, tokens at 4092..4095
        return build(CONFIG_NAMES[0], [4096], [(0, p) for p in range(4092, 4096)], s)
    if i == 1:   # batched decode: 32 sequences, lengths uniform in [16384, 32768]
        rng = np.random.default_rng(1000 + s)
        lens = rng.integers(16384, 32768 + 1, size=32)
        return build(CONFIG_NAMES[1], lens, [(b, int(lens[b]) - 1) for b in range(32)], s)
    if i == 2:   # long-context decode: 16 x 131072
        return build(CONFIG_NAMES[2], [131072] * 16, [(b, 131071) for b in range(16)], s)
    if i == 3:   # chunked prefill: 8192 tokens at 122880..131071 of one 131072 cache
        return build(CONFIG_NAMES[3], [131072], [(0, p) for p in range(122880, 131072)], s)
    if i == 4:   # extended decode with fp8 caches: 8 x 262144
        return build(CONFIG_NAMES[4], [262144] * 8, [(b, 262143) for b in range(8)], s, fp8=True)
    if i == 5:   # the same shape with MX block-32 caches (the training recipe's format)
        return build(CONFIG_NAMES[5], [262144] * 8, [(b, 262143) for b in range(8)], s, mx=True)
    if i == 6:   # and with four-bit MX block-32 caches
        return build(CONFIG_NAMES[6], [262144] * 8, [(b, 262143) for b in range(8)], s, mx4=True)
    raise ValueError(f"no workload {i}")


def describe(wl: Workload) -> dict:
    return {"workload": wl.name, "batch": wl.num_seqs, "query_tokens": wl.num_tokens,
            "max_context": wl.max_len, "top_k": wl.k,
            "cache": {"bf16": "bf16", "e4m3fn": "fp8_e4m3", "mxfp8": "mxfp8_e4m3",
                      "mxfp4": "mxfp4_e2m1"}[wl.cache_fmt]}
