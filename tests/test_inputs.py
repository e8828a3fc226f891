"""The seeded workload generator: shapes, value sets and reproducibility."""
import numpy as np
import torch

import sga_inputs as si


def test_tiny_decode_shapes_and_values():
    wl = si.config(0)
    assert wl.num_tokens == 4 and wl.num_seqs == 1 and wl.cache_rows == 4096
    assert wl.token_pos.tolist() == [4092, 4093, 4094, 4095]
    assert tuple(wl.q_idx.shape) == (4, 64, 128) and wl.q_idx.dtype == torch.bfloat16
    assert tuple(wl.kv.shape) == (4096, 576) and wl.kv.dtype == torch.bfloat16
    assert tuple(wl.q_abs.shape) == (4, 64, 576) and tuple(wl.gate.shape) == (4, 64)
    k = wl.k_idx.float()
    assert set(torch.unique(k).tolist()) <= set(range(-3, 4))
    assert set(torch.unique(wl.w).tolist()) <= set(range(0, 5))
    assert 0.035 < wl.kv.float().std().item() < 0.048          # N(0,1)/24
    assert 1.5 < wl.gate.std().item() < 2.5                      # sigma 2
    assert wl.max_len == 4096 and wl.k == 2048


def test_reproducible():
    a, b = si.config(0), si.config(0)
    assert torch.equal(a.kv, b.kv) and torch.equal(a.q_abs, b.q_abs) and torch.equal(a.k_idx, b.k_idx)
    c = si.config(0, seed=99)
    assert not torch.equal(a.kv, c.kv)


def test_fp8_recipe_small():
    wl = si.build("fp8_small", [300, 200], [(0, 299), (1, 150)], seed=4, fp8=True)
    assert wl.kv.dtype == torch.float8_e4m3fn and wl.kv_scale.shape == (500,)
    vals = wl.kv.float()
    amax = vals.abs().max(dim=1).values
    assert torch.all(amax == 448.0)                              # scale = max|x|/448
    s = wl.k_idx_scale
    assert set(torch.log2(s).round().tolist()) <= {-2, -1, 0, 1, 2}
    assert set(torch.unique(wl.k_idx.float()).tolist()) <= set(range(-3, 4))
    assert wl.seq_start.tolist() == [0, 300]
