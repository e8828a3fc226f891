"""Sparse Gated Attention (SGA) on MI355X (gfx950).

The whole path runs in libsga.so: hand-written HIP kernels behind the C ABI in
include/sga.h. This package is its ctypes binding. The entry points are
sga_index_scores, sga_topk, sga_sparse_mla_attn, sga_forward,
sga_forward_noalloc, sga_cache_append, sga_output_proj and sga_indexer_loss, with the same names
and meaning as the C functions; sga_hbm_read_probe is a measurement helper.
"""
from ._lib import (Batch, SgaError, SgaTrace, load, status_string, version, workspace,
                   sga_index_scores, sga_topk, sga_topk_workspace_size, sga_sparse_mla_attn,
                   sga_attn_workspace_size, sga_forward, sga_forward_workspace_size,
                   sga_forward_noalloc, sga_forward_noalloc_scratch_bytes, sga_cache_append, sga_output_proj, sga_output_proj_workspace_size,
                   sga_indexer_loss, sga_indexer_loss_workspace_size, sga_hbm_read_probe, LIB_PATH,
                   EXPORTS)

__all__ = ["Batch", "SgaError", "SgaTrace", "load", "status_string", "version", "workspace",
           "sga_index_scores", "sga_topk", "sga_topk_workspace_size", "sga_sparse_mla_attn",
           "sga_attn_workspace_size", "sga_forward", "sga_forward_workspace_size",
           "sga_forward_noalloc", "sga_forward_noalloc_scratch_bytes", "sga_cache_append", "sga_output_proj", "sga_output_proj_workspace_size",
           "sga_indexer_loss", "sga_indexer_loss_workspace_size", "sga_hbm_read_probe",
           "batch_to_device", "LIB_PATH", "EXPORTS"]


def batch_to_device(token_seq, token_pos, seq_start, seq_len, cache_rows: int, device="cuda",
                    max_len=None) -> Batch:
    """Builds a Batch from host arrays (numpy or lists). max_len defaults to max(token_pos)+1."""
    import numpy as np
    import torch
    ts = torch.as_tensor(np.asarray(token_seq, dtype=np.int32), device=device)
    tp = torch.as_tensor(np.asarray(token_pos, dtype=np.int32), device=device)
    ss = torch.as_tensor(np.asarray(seq_start, dtype=np.int64), device=device)
    sl = torch.as_tensor(np.asarray(seq_len, dtype=np.int32), device=device)
    if max_len is None:
        max_len = int(np.max(token_pos)) + 1 if len(token_pos) else 1
    return Batch(ts, tp, ss, sl, max_len, cache_rows)
