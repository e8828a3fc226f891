"""sga_forward_noalloc (no workspace argument: the library's own per-GPU scratch
array) against sga_forward on the same inputs, two calls in a row, the second
on a smaller batch, so the second call meets the first call's leftovers in the
scratch."""
import numpy as np
import pytest
import torch

import sga_inputs as si
import sparse_gated_mla_amd as sga
from gpu_helpers import BF16_MAX_ABS, BF16_REL_L2, Dev, out_errors, say

pytestmark = pytest.mark.gpu


def _run(dev, noalloc):
    wl = dev.wl
    T = wl.num_tokens
    out = torch.full((T, 64, 512), float("nan"), dtype=torch.float32, device=dev.device)
    lse = torch.full((T, 64), float("nan"), dtype=torch.float32, device=dev.device)
    idx = torch.full((T, wl.k), -7, dtype=torch.int32, device=dev.device)
    fn = sga.sga_forward_noalloc if noalloc else sga.sga_forward
    fn(dev.batch, dev.q_idx, dev.w, dev.k_idx, dev.k_idx_scale, dev.q_abs, dev.kv, dev.kv_scale,
       wl.k, wl.sm_scale, dev.gate, out, lse, idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def _compare(a, b, what):
    assert np.array_equal(a[0], b[0]), f"{what}: indices differ"
    max_abs, rel = out_errors(a[1], b[1].astype(np.float64))
    say(f"  {what}: out max|diff| {max_abs:.3e} rel-L2 {rel:.3e}")
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, rel)
    assert np.array_equal(np.isfinite(a[2]), np.isfinite(b[2])), what
    fin = np.isfinite(b[2])
    assert np.abs(a[2][fin] - b[2][fin]).max() <= 1e-3, what


def test_noalloc_matches_forward_on_two_calls():
    big = si.build("noalloc_big", [20000, 9000, 3000],
                   [(0, 19999), (1, 8999), (2, 2999), (0, 12000), (1, 100)], seed=41)
    small = si.build("noalloc_small", [5000], [(0, 4999), (0, 4000)], seed=42)
    for wl in (big, small):
        say(f"[noalloc] {wl.name}: T={wl.num_tokens} max_len={wl.max_len} k={wl.k}")
        dev = Dev(wl)
        got = _run(dev, noalloc=True)
        ref = _run(dev, noalloc=False)
        _compare(got, ref, wl.name)


def test_noalloc_rejects_oversize():
    # 64 tokens with a 512K max_len need 128 MB of scores alone: rejected on the
    # host before anything is launched (the metadata is never read)
    wl = si.build("noalloc_limit", [4096], [(0, 4095)] * 64, seed=43)
    dev = Dev(wl)
    batch = dev.batch
    batch.max_len = 1 << 19
    assert sga.sga_forward_workspace_size(64, 1 << 19, wl.k) > sga.sga_forward_noalloc_scratch_bytes()
    out = torch.empty((64, 64, 512), dtype=torch.float32, device=dev.device)
    with pytest.raises(sga.SgaError) as e:
        sga.sga_forward_noalloc(batch, dev.q_idx, dev.w, dev.k_idx, dev.k_idx_scale, dev.q_abs, dev.kv,
                                dev.kv_scale, wl.k, wl.sm_scale, dev.gate, out)
    assert e.value.status == 3
