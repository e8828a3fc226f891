"""sga_forward_noalloc and sga_forward (with a workspace allocated beforehand)
captured in a HIP graph: replayed several times, with eager work and
synchronisations between the replays, every replay equals the eager call bit
for bit."""
import pytest
import torch

import sga_inputs as si
import sparse_gated_mla_amd as sga
from gpu_helpers import Dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("noalloc", [True, False])
def test_forward_replayed_from_a_graph(noalloc):
    wl = si.build("graph", [20000, 9000], [(0, 19999), (1, 8999), (0, 5000)], seed=44)
    dev = Dev(wl)
    T = wl.num_tokens
    out = torch.zeros((T, 64, 512), dtype=torch.float32, device="cuda")
    lse = torch.zeros((T, 64), dtype=torch.float32, device="cuda")
    idx = torch.zeros((T, wl.k), dtype=torch.int32, device="cuda")
    ws = None if noalloc else sga.workspace(sga.sga_forward_workspace_size(T, wl.max_len, wl.k), "cuda")

    def call():
        args = (dev.batch, dev.q_idx, dev.w, dev.k_idx, dev.k_idx_scale, dev.q_abs, dev.kv, dev.kv_scale,
                wl.k, wl.sm_scale, dev.gate, out, lse, idx)
        if noalloc:
            sga.sga_forward_noalloc(*args)
        else:
            sga.sga_forward(*args, ws=ws)

    say(f"[graph] noalloc={noalloc}: eager reference")
    call()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("[graph] capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        say(f"[graph] replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"replay {r}: indices"
        assert torch.equal(out, ref[1]), f"replay {r}: out"
        assert torch.equal(lse, ref[2]), f"replay {r}: lse"
        # the program's own work between replays
        x = torch.randn(1 << 20, device="cuda")
        float(x.sum())
