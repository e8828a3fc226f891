"""GPU parity for sga_output_proj (the value up-projection of each head and the
output projection, after the gate) against the oracle's output projection."""
import numpy as np
import pytest
import torch

import oracle
import sga_inputs as si
import sparse_gated_mla_amd as sga
from gpu_helpers import Dev, say

pytestmark = pytest.mark.gpu

# Activations enter the bf16 products as a hi/lo pair (relative error about
# 2^-17 per element) and the sums are fp32 over at most 8,192 terms, so the
# result is within about 1e-5 of the float64 product; the bar leaves margin.
PROJ_REL_L2 = 1e-4


def _oracle(o, w_uv, w_o):
    return oracle.output_projection(o.double().numpy(), w_uv.double().numpy(), w_o.double().numpy())


def _check(got, ref, what):
    diff = got.astype(np.float64) - ref
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    worst = float(np.abs(diff).max() / np.abs(ref).max())
    say(f"  {what}: rel-L2 {rel:.3e}  max|diff|/max|y| {worst:.3e}")
    assert rel <= PROJ_REL_L2 and worst <= PROJ_REL_L2, (what, rel, worst)


def _run(o, w_uv, w_o):
    T, d_model = o.shape[0], w_o.shape[0]
    y = torch.full((T, d_model), float("nan"), dtype=torch.float32, device="cuda")
    sga.sga_output_proj(o.cuda(), w_uv.cuda(), w_o.cuda(), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("T,d_model", [(1, 256), (5, 7168), (16, 7168), (17, 448), (40, 7168)])
def test_output_proj_matches_oracle(T, d_model):
    say(f"[output_proj] T={T} d_model={d_model}")
    rng = np.random.default_rng(T * 1000 + d_model)
    o = torch.from_numpy(rng.standard_normal((T, 64, 512), dtype=np.float32) * np.float32(3e-3))
    w_uv, w_o = si.proj_weights(seed=T, d_model=d_model)
    _check(_run(o, w_uv, w_o), _oracle(o, w_uv, w_o), f"T={T} d_model={d_model}")


def test_output_proj_after_forward():
    # the gated output of the whole path, projected
    wl = si.config(0)
    dev = Dev(wl)
    _, out, _ = dev.forward()
    w_uv, w_o = si.proj_weights(seed=5)
    say("[output_proj] after sga_forward, tiny decode")
    o = out.cpu()
    _check(_run(o, w_uv, w_o), _oracle(o, w_uv, w_o), "after forward")


def test_output_proj_prefill_sampled():
    # the 8,192-token prefill size, checked on sampled tokens
    T = 8192
    rng = np.random.default_rng(31)
    o = torch.from_numpy(rng.standard_normal((T, 64, 512), dtype=np.float32) * np.float32(3e-3))
    w_uv, w_o = si.proj_weights(seed=31)
    say(f"[output_proj] T={T} d_model=7168, sampled rows")
    y = _run(o, w_uv, w_o)
    sample = sorted({0, 1, 15, 16, 4095, 8190, 8191, *range(0, T, 1021)})
    _check(y[sample], _oracle(o[sample], w_uv, w_o), "prefill sample")
    assert np.all(np.isfinite(y))


def test_output_proj_deterministic():
    rng = np.random.default_rng(32)
    o = torch.from_numpy(rng.standard_normal((16, 64, 512), dtype=np.float32))
    w_uv, w_o = si.proj_weights(seed=32)
    a, b = _run(o, w_uv, w_o), _run(o, w_uv, w_o)
    assert np.array_equal(a, b)
