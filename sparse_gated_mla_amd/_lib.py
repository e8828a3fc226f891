"""ctypes binding of libsga (include/sga.h): argument marshalling only.

Each function takes torch device tensors, checks their dtype, device, shape
and contiguity, and passes raw pointers and the current HIP stream to the C
function of the same name. Every step of the computation runs in libsga's HIP
kernels. There is no fallback: if the library has not been built, load()
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsga.so")

SGA_OK, SGA_ERR_INVALID_ARG, SGA_ERR_UNSUPPORTED, SGA_ERR_WORKSPACE, SGA_ERR_HIP = range(5)
SGA_BF16, SGA_FP8_E4M3, SGA_MXFP8_E4M3, SGA_MXFP4_E2M1 = 0, 1, 2, 3
MX_BLOCK = 32
HEADS, IDX_HEADS, IDX_DIM, D_LATENT, D_QK, D_V = 64, 64, 128, 512, 576, 128

EXPORTS = ("sga_index_scores", "sga_topk_workspace_size", "sga_topk", "sga_attn_workspace_size",
           "sga_sparse_mla_attn", "sga_forward_workspace_size", "sga_forward",
           "sga_forward_noalloc_scratch_bytes", "sga_forward_noalloc",
           "sga_cache_append", "sga_output_proj_workspace_size", "sga_output_proj",
           "sga_indexer_loss_workspace_size", "sga_indexer_loss",
           "sga_hbm_read_probe", "sga_status_string", "sga_version")


class SgaBatch(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cache_rows", ctypes.c_int64), ("token_seq", ctypes.c_void_p),
                ("token_pos", ctypes.c_void_p), ("seq_start", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p)]


class SgaTrace(ctypes.Structure):
    _fields_ = [("indexer_begin", ctypes.c_void_p), ("indexer_end", ctypes.c_void_p),
                ("topk_end", ctypes.c_void_p), ("attn_end", ctypes.c_void_p)]


class SgaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status}: {status_string(status)}")
        self.status = status


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libsga.so (built in-tree by sparse_gated_mla_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m sparse_gated_mla_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    bp = ctypes.POINTER(SgaBatch)
    tp = ctypes.POINTER(SgaTrace)
    sig = {
        "sga_index_scores": ([bp, vp, vp, vp, vp, ctypes.c_int, vp, i64, vp], ctypes.c_int),
        "sga_topk_workspace_size": ([i32, i32, i32], sz),
        "sga_topk": ([bp, vp, i64, i32, vp, vp, sz, vp], ctypes.c_int),
        "sga_attn_workspace_size": ([i32, i32], sz),
        "sga_sparse_mla_attn": ([bp, vp, vp, vp, ctypes.c_int, vp, i32, f32, vp, vp, vp, vp, sz, vp],
                                ctypes.c_int),
        "sga_forward_workspace_size": ([i32, i32, i32], sz),
        "sga_forward": ([bp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i32, f32, vp, vp,
                         vp, vp, vp, sz, tp, vp], ctypes.c_int),
        "sga_forward_noalloc_scratch_bytes": ([], sz),
        "sga_forward_noalloc": ([bp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, i32, f32, vp,
                                 vp, vp, vp, tp, vp], ctypes.c_int),
        "sga_cache_append": ([bp, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp], ctypes.c_int),
        "sga_output_proj_workspace_size": ([i32, i32], sz),
        "sga_indexer_loss_workspace_size": ([i32, i32], sz),
        "sga_indexer_loss": ([bp, vp, vp, vp, ctypes.c_int, vp, i32, f32, vp, vp, i64, vp, vp, sz, vp],
                             ctypes.c_int),
        "sga_output_proj": ([i32, vp, vp, vp, i32, vp, vp, sz, vp], ctypes.c_int),
        "sga_hbm_read_probe": ([vp, sz, vp, vp], ctypes.c_int),
        "sga_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "sga_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sga_status_string(status).decode()


def version() -> int:
    return load().sga_version()


# ---------------------------------------------------------------- marshalling
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None:
        for i, (got, want) in enumerate(zip(t.shape, shape)):
            if want is not None and got != want:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if len(t.shape) != len(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


_E8M0 = tuple(d for d in (torch.uint8, getattr(torch, "float8_e8m0fnu", None)) if d is not None)
_FP4X2 = tuple(d for d in (torch.uint8, getattr(torch, "float4_e2m1fn_x2", None)) if d is not None)


def _cache_dtype(t: torch.Tensor, scale: Optional[torch.Tensor], name: str, rows: int, width: int) -> int:
    """Checks a cache of `rows` rows of `width` elements and its scales, and
    returns its sga_dtype from the tensors:
    - bfloat16 [rows, width], no scale;
    - float8_e4m3fn [rows, width] with fp32 scales [rows] (one per row);
    - float8_e4m3fn [rows, width] with E8M0 exponents [rows, width/32] (uint8 or
      float8_e8m0fnu): MX block-32;
    - uint8 or float4_e2m1fn_x2 [rows, width/2] (two E2M1 elements per byte,
      low nibble first) with E8M0 exponents [rows, width/32]: MX block-32, four-bit."""
    if t.dtype == torch.bfloat16:
        _check(t, name, (torch.bfloat16,), (rows, width))
        if scale is not None:
            raise ValueError(f"{name}: bf16 storage takes no scale")
        return SGA_BF16
    if scale is None:
        raise ValueError(f"{name}: {t.dtype} storage needs scales")
    if t.dtype == torch.float8_e4m3fn:
        _check(t, name, (torch.float8_e4m3fn,), (rows, width))
        if scale.dtype == torch.float32:
            _check(scale, name + "_scale", (torch.float32,), (rows,))
            return SGA_FP8_E4M3
        _check(scale, name + "_scale", _E8M0, (rows, width // MX_BLOCK))
        return SGA_MXFP8_E4M3
    if t.dtype in _FP4X2:
        _check(t, name, _FP4X2, (rows, width // 2))
        _check(scale, name + "_scale", _E8M0, (rows, width // MX_BLOCK))
        return SGA_MXFP4_E2M1
    raise TypeError(f"{name} must be bfloat16, float8_e4m3fn or packed four-bit (uint8), got {t.dtype}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _raise(fn: str, status: int):
    if status != SGA_OK:
        raise SgaError(fn, status)


class Batch:
    """A ragged batch of query tokens (sga_batch). Device metadata tensors plus
    host sizes: token_seq/token_pos int32 [T], seq_start int64 [B], seq_len int32 [B]."""

    def __init__(self, token_seq, token_pos, seq_start, seq_len, max_len: int, cache_rows: int):
        _check(token_seq, "token_seq", (torch.int32,))
        _check(token_pos, "token_pos", (torch.int32,), (token_seq.shape[0],))
        _check(seq_start, "seq_start", (torch.int64,))
        _check(seq_len, "seq_len", (torch.int32,), (seq_start.shape[0],))
        self.token_seq, self.token_pos, self.seq_start, self.seq_len = token_seq, token_pos, seq_start, seq_len
        self.num_tokens = int(token_seq.shape[0])
        self.num_seqs = int(seq_start.shape[0])
        self.max_len = int(max_len)
        self.cache_rows = int(cache_rows)
        self.device = token_seq.device

    def c(self) -> SgaBatch:
        return SgaBatch(self.num_tokens, self.num_seqs, self.max_len, 0, self.cache_rows,
                        self.token_seq.data_ptr(), self.token_pos.data_ptr(),
                        self.seq_start.data_ptr(), self.seq_len.data_ptr())


def workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer of at least nbytes (at least one byte)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points
def sga_index_scores(batch: Batch, q_idx, w, k_idx, k_idx_scale, scores) -> None:
    T = batch.num_tokens
    _check(q_idx, "q_idx", (torch.bfloat16,), (T, IDX_HEADS, IDX_DIM))
    _check(w, "w", (torch.float32,), (T, IDX_HEADS))
    dt = _cache_dtype(k_idx, k_idx_scale, "k_idx", batch.cache_rows, IDX_DIM)
    _check(scores, "scores", (torch.float32,), (T, None))
    b = batch.c()
    _raise("sga_index_scores", load().sga_index_scores(
        ctypes.byref(b), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_idx_scale), dt, _ptr(scores),
        scores.shape[1], _stream(q_idx)))


def sga_topk_workspace_size(num_tokens: int, max_len: int, k: int) -> int:
    return int(load().sga_topk_workspace_size(num_tokens, max_len, k))


def sga_topk(batch: Batch, scores, k: int, indices, ws: Optional[torch.Tensor] = None) -> None:
    T = batch.num_tokens
    _check(scores, "scores", (torch.float32,), (T, None))
    _check(indices, "indices", (torch.int32,), (T, k))
    if ws is None:
        ws = workspace(sga_topk_workspace_size(T, batch.max_len, k), scores.device)
    b = batch.c()
    _raise("sga_topk", load().sga_topk(ctypes.byref(b), _ptr(scores), scores.shape[1], k,
                                       _ptr(indices), _ptr(ws), ws.numel(), _stream(scores)))


def sga_attn_workspace_size(num_tokens: int, k: int) -> int:
    return int(load().sga_attn_workspace_size(num_tokens, k))


def sga_sparse_mla_attn(batch: Batch, q_abs, kv, kv_scale, indices, k: int, sm_scale: float,
                        gate, out, lse=None, ws: Optional[torch.Tensor] = None) -> None:
    T = batch.num_tokens
    _check(q_abs, "q_abs", (torch.bfloat16,), (T, HEADS, D_QK))
    dt = _cache_dtype(kv, kv_scale, "kv", batch.cache_rows, D_QK)
    _check(indices, "indices", (torch.int32,), (T, k))
    if gate is not None:
        _check(gate, "gate", (torch.float32,), (T, HEADS))
    _check(out, "out", (torch.float32,), (T, HEADS, D_LATENT))
    if lse is not None:
        _check(lse, "lse", (torch.float32,), (T, HEADS))
    if ws is None:
        ws = workspace(sga_attn_workspace_size(T, k), q_abs.device)
    b = batch.c()
    _raise("sga_sparse_mla_attn", load().sga_sparse_mla_attn(
        ctypes.byref(b), _ptr(q_abs), _ptr(kv), _ptr(kv_scale), dt, _ptr(indices), k,
        float(sm_scale), _ptr(gate), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(q_abs)))


def sga_forward_workspace_size(num_tokens: int, max_len: int, k: int) -> int:
    return int(load().sga_forward_workspace_size(num_tokens, max_len, k))


def sga_forward(batch: Batch, q_idx, w, k_idx, k_idx_scale, q_abs, kv, kv_scale, k: int,
                sm_scale: float, gate, out, lse=None, indices_out=None,
                ws: Optional[torch.Tensor] = None, trace: Optional[SgaTrace] = None) -> None:
    T = batch.num_tokens
    _check(q_idx, "q_idx", (torch.bfloat16,), (T, IDX_HEADS, IDX_DIM))
    _check(w, "w", (torch.float32,), (T, IDX_HEADS))
    kdt = _cache_dtype(k_idx, k_idx_scale, "k_idx", batch.cache_rows, IDX_DIM)
    _check(q_abs, "q_abs", (torch.bfloat16,), (T, HEADS, D_QK))
    vdt = _cache_dtype(kv, kv_scale, "kv", batch.cache_rows, D_QK)
    if gate is not None:
        _check(gate, "gate", (torch.float32,), (T, HEADS))
    _check(out, "out", (torch.float32,), (T, HEADS, D_LATENT))
    if lse is not None:
        _check(lse, "lse", (torch.float32,), (T, HEADS))
    if indices_out is not None:
        _check(indices_out, "indices_out", (torch.int32,), (T, k))
    if ws is None:
        ws = workspace(sga_forward_workspace_size(T, batch.max_len, k), q_abs.device)
    b = batch.c()
    _raise("sga_forward", load().sga_forward(
        ctypes.byref(b), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_idx_scale), kdt, _ptr(q_abs),
        _ptr(kv), _ptr(kv_scale), vdt, k, float(sm_scale), _ptr(gate), _ptr(out), _ptr(lse),
        _ptr(indices_out), _ptr(ws), ws.numel(), None if trace is None else ctypes.byref(trace),
        _stream(q_abs)))


def sga_forward_noalloc_scratch_bytes() -> int:
    return int(load().sga_forward_noalloc_scratch_bytes())


def sga_forward_noalloc(batch: Batch, q_idx, w, k_idx, k_idx_scale, q_abs, kv, kv_scale, k: int,
                        sm_scale: float, gate, out, lse=None, indices_out=None,
                        trace: Optional[SgaTrace] = None) -> None:
    """sga_forward with the library's own per-GPU scratch instead of a workspace:
    allocates nothing (for callers that cannot allocate)."""
    T = batch.num_tokens
    _check(q_idx, "q_idx", (torch.bfloat16,), (T, IDX_HEADS, IDX_DIM))
    _check(w, "w", (torch.float32,), (T, IDX_HEADS))
    kdt = _cache_dtype(k_idx, k_idx_scale, "k_idx", batch.cache_rows, IDX_DIM)
    _check(q_abs, "q_abs", (torch.bfloat16,), (T, HEADS, D_QK))
    vdt = _cache_dtype(kv, kv_scale, "kv", batch.cache_rows, D_QK)
    if gate is not None:
        _check(gate, "gate", (torch.float32,), (T, HEADS))
    _check(out, "out", (torch.float32,), (T, HEADS, D_LATENT))
    if lse is not None:
        _check(lse, "lse", (torch.float32,), (T, HEADS))
    if indices_out is not None:
        _check(indices_out, "indices_out", (torch.int32,), (T, k))
    b = batch.c()
    _raise("sga_forward_noalloc", load().sga_forward_noalloc(
        ctypes.byref(b), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_idx_scale), kdt, _ptr(q_abs),
        _ptr(kv), _ptr(kv_scale), vdt, k, float(sm_scale), _ptr(gate), _ptr(out), _ptr(lse),
        _ptr(indices_out), None if trace is None else ctypes.byref(trace), _stream(q_abs)))


def sga_cache_append(batch: Batch, latent=None, idx_key=None, kv=None, kv_scale=None,
                     k_idx=None, k_idx_scale=None) -> None:
    """Writes token t's latent row into kv[seq_start[b] + p] and its indexer key into
    k_idx[seq_start[b] + p]; an fp8 cache (float8_e4m3fn) gets one fp32 scale per row."""
    T = batch.num_tokens
    kdt = vdt = SGA_BF16
    if latent is not None:
        _check(latent, "latent", (torch.bfloat16,), (T, D_QK))
    if idx_key is not None:
        _check(idx_key, "idx_key", (torch.bfloat16,), (T, IDX_DIM))
    if kv is not None:
        vdt = _cache_dtype(kv, kv_scale, "kv", batch.cache_rows, D_QK)
    if k_idx is not None:
        kdt = _cache_dtype(k_idx, k_idx_scale, "k_idx", batch.cache_rows, IDX_DIM)
    ref = next((t for t in (latent, idx_key, kv, k_idx) if t is not None), batch.token_seq)
    b = batch.c()
    _raise("sga_cache_append", load().sga_cache_append(
        ctypes.byref(b), _ptr(latent), _ptr(idx_key), _ptr(kv), _ptr(kv_scale), vdt, _ptr(k_idx),
        _ptr(k_idx_scale), kdt, _stream(ref)))


def sga_output_proj_workspace_size(num_tokens: int, d_model: int) -> int:
    return int(load().sga_output_proj_workspace_size(num_tokens, d_model))


def sga_output_proj(o_latent, w_uv, w_o, y, ws: Optional[torch.Tensor] = None) -> None:
    """y[t] = w_o @ concat_h(w_uv[h] @ o_latent[t, h]): the value up-projection of
    each head and the output projection, after the gate."""
    _check(o_latent, "o_latent", (torch.float32,))
    T = int(o_latent.shape[0])
    _check(o_latent, "o_latent", (torch.float32,), (T, HEADS, D_LATENT))
    _check(w_uv, "w_uv", (torch.bfloat16,), (HEADS, D_V, D_LATENT))
    _check(w_o, "w_o", (torch.bfloat16,), (None, HEADS * D_V))
    d_model = int(w_o.shape[0])
    _check(y, "y", (torch.float32,), (T, d_model))
    if ws is None:
        ws = workspace(sga_output_proj_workspace_size(T, d_model), o_latent.device)
    _raise("sga_output_proj", load().sga_output_proj(
        T, _ptr(o_latent), _ptr(w_uv), _ptr(w_o), d_model, _ptr(y), _ptr(ws), ws.numel(),
        _stream(o_latent)))


def sga_indexer_loss_workspace_size(num_tokens: int, k: int) -> int:
    return int(load().sga_indexer_loss_workspace_size(num_tokens, k))


def sga_indexer_loss(batch: Batch, q_abs, kv, kv_scale, indices, k: int, sm_scale: float, lse,
                     scores, loss, ws: Optional[torch.Tensor] = None) -> None:
    """loss[t] = KL(p || q) over token t's selected rows: p the head-mean attention
    probabilities (with the attention's lse), q the softmax of the indexer scores."""
    T = batch.num_tokens
    _check(q_abs, "q_abs", (torch.bfloat16,), (T, HEADS, D_QK))
    dt = _cache_dtype(kv, kv_scale, "kv", batch.cache_rows, D_QK)
    _check(indices, "indices", (torch.int32,), (T, k))
    _check(lse, "lse", (torch.float32,), (T, HEADS))
    _check(scores, "scores", (torch.float32,), (T, None))
    _check(loss, "loss", (torch.float32,), (T,))
    if ws is None:
        ws = workspace(sga_indexer_loss_workspace_size(T, k), q_abs.device)
    b = batch.c()
    _raise("sga_indexer_loss", load().sga_indexer_loss(
        ctypes.byref(b), _ptr(q_abs), _ptr(kv), _ptr(kv_scale), dt, _ptr(indices), k, float(sm_scale),
        _ptr(lse), _ptr(scores), scores.shape[1], _ptr(loss), _ptr(ws), ws.numel(), _stream(q_abs)))


def sga_hbm_read_probe(src, sink) -> None:
    """Reads the device byte buffer src once in the indexer's access pattern
    (a measurement helper); sink: int32 device buffer of 262,144 words."""
    _check(src, "src", (torch.uint8,))
    _check(sink, "sink", (torch.int32,), (262144,))
    _raise("sga_hbm_read_probe",
           load().sga_hbm_read_probe(_ptr(src), src.numel(), _ptr(sink), _stream(src)))
