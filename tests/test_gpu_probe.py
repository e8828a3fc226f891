"""The HBM read probe (a measurement helper): it reads the whole buffer and
leaves the sink untouched for data that does not fold to its trigger value."""
import pytest
import torch

import sparse_gated_mla_amd as sga
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [4096, 3 * 4096 * 1024 + 4096, 64 << 20])
def test_hbm_read_probe_runs_and_leaves_the_sink(nbytes):
    say(f"[hbm_read_probe] {nbytes} bytes")
    buf = torch.full((nbytes,), 1, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(262144, dtype=torch.int32, device="cuda")
    sga.sga_hbm_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_hbm_read_probe_rejects_a_partial_page():
    buf = torch.zeros(4096 + 16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(262144, dtype=torch.int32, device="cuda")
    with pytest.raises(sga.SgaError):
        sga.sga_hbm_read_probe(buf, sink)
