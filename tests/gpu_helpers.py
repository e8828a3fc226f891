"""Shared helpers for the GPU parity tests: move a workload to the device, run the
oracle on the same inputs, compare results."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import sparse_gated_mla_amd as sga

# Tolerances on the attention output (bf16 caches / fp8 caches), as max |diff|
# and relative L2 over the whole output tensor.
BF16_MAX_ABS, BF16_REL_L2 = 1e-2, 2e-3
FP8_REL_L2 = 2e-2
LSE_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Dev:
    """A workload's tensors on the GPU plus its Batch."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.batch = sga.batch_to_device(wl.token_seq, wl.token_pos, wl.seq_start, wl.seq_len,
                                         wl.cache_rows, device=device, max_len=wl.max_len)
        d = lambda t: None if t is None else t.to(device)
        self.q_idx, self.w, self.k_idx, self.k_idx_scale = d(wl.q_idx), d(wl.w), d(wl.k_idx), d(wl.k_idx_scale)
        self.kv, self.kv_scale, self.q_abs, self.gate = d(wl.kv), d(wl.kv_scale), d(wl.q_abs), d(wl.gate)
        self.device = device

    def forward(self, gate=True, k=None):
        T, kk = self.wl.num_tokens, (k or self.wl.k)
        out = torch.empty((T, 64, 512), dtype=torch.float32, device=self.device)
        lse = torch.empty((T, 64), dtype=torch.float32, device=self.device)
        idx = torch.empty((T, kk), dtype=torch.int32, device=self.device)
        sga.sga_forward(self.batch, self.q_idx, self.w, self.k_idx, self.k_idx_scale, self.q_abs,
                        self.kv, self.kv_scale, kk, self.wl.sm_scale, self.gate if gate else None,
                        out, lse, idx)
        torch.cuda.synchronize()
        return idx, out, lse

    def scores(self, ld=None):
        T = self.wl.num_tokens
        ld = ld or self.wl.max_len
        s = torch.full((T, ld), float("nan"), dtype=torch.float32, device=self.device)
        sga.sga_index_scores(self.batch, self.q_idx, self.w, self.k_idx, self.k_idx_scale, s)
        torch.cuda.synchronize()
        return s

    def topk(self, scores, k=None):
        kk = k or self.wl.k
        idx = torch.full((self.wl.num_tokens, kk), -7, dtype=torch.int32, device=self.device)
        sga.sga_topk(self.batch, scores, kk, idx)
        torch.cuda.synchronize()
        return idx

    def attention(self, indices, gate=True, k=None):
        T, kk = self.wl.num_tokens, (k or self.wl.k)
        out = torch.empty((T, 64, 512), dtype=torch.float32, device=self.device)
        lse = torch.empty((T, 64), dtype=torch.float32, device=self.device)
        sga.sga_sparse_mla_attn(self.batch, self.q_abs, self.kv, self.kv_scale, indices, kk,
                                self.wl.sm_scale, self.gate if gate else None, out, lse)
        torch.cuda.synchronize()
        return out, lse


def stores(wl):
    """The oracle's views of the caches: raw bits plus format."""
    if wl.fp8:
        ks = oracle.Store(wl.k_idx.view(torch.uint8).numpy(), wl.cache_fmt, wl.k_idx_scale.numpy())
        vs = oracle.Store(wl.kv.view(torch.uint8).numpy(), wl.cache_fmt, wl.kv_scale.numpy())
    else:
        ks = oracle.Store(wl.k_idx.view(torch.int16).numpy().view(np.uint16), "bf16")
        vs = oracle.Store(wl.kv.view(torch.int16).numpy().view(np.uint16), "bf16")
    return ks, vs


def run_oracle(wl, tokens=None, gate=True, keep_scores=False, k=None):
    ks, vs = stores(wl)
    return oracle.forward(wl.token_seq, wl.token_pos, wl.seq_start, wl.seq_len,
                          wl.q_idx.double().numpy(), wl.w.double().numpy(), ks,
                          wl.q_abs.double().numpy(), vs,
                          wl.gate.double().numpy() if gate else None, k or wl.k, wl.sm_scale,
                          tokens=tokens, keep_scores=keep_scores)


def out_errors(got: np.ndarray, ref: np.ndarray):
    diff = got.astype(np.float64) - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / denom if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_out_close(got: np.ndarray, ref: np.ndarray, fp8: bool, what=""):
    max_abs, rel = out_errors(got, ref)
    say(f"  {what} out: max|diff| {max_abs:.3e}  rel-L2 {rel:.3e}")
    if fp8:
        assert rel <= FP8_REL_L2, (what, rel)
    else:
        assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, rel)


def assert_lse_close(got: np.ndarray, ref: np.ndarray, what=""):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), what
    assert np.all(got[~fin] == ref[~fin]), what
    if fin.any():
        d = float(np.abs(got[fin] - ref[fin]).max())
        say(f"  {what} lse: max|diff| {d:.3e}")
        assert d <= LSE_ABS, (what, d)
