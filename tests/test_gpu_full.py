"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (sga_forward). Decode workloads are checked in full against
the oracle. The 8192-token chunked prefill is checked on a stated sample of
tokens that the oracle computes one by one."""
import numpy as np
import pytest

import sga_inputs as si
from gpu_helpers import Dev, assert_lse_close, assert_out_close, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2, 4, 5, 6])
def test_decode_workload_full(cfg):
    wl = si.config(cfg)
    say(f"[full] {wl.name}: T={wl.num_tokens} B={wl.num_seqs} max_len={wl.max_len} fp8={wl.fp8}")
    dev = Dev(wl)
    idx, out, lse = dev.forward()
    del dev
    ref = run_oracle(wl)
    got_idx = idx.cpu().numpy()
    bad = [t for t in range(wl.num_tokens) if not np.array_equal(got_idx[t], ref["indices"][t])]
    assert not bad, f"indices differ for tokens {bad}"
    assert_out_close(out.cpu().numpy(), ref["out"], wl.fp8 and not wl.mx, wl.name)
    assert_lse_close(lse.cpu().numpy(), ref["lse"], wl.name)


def test_chunked_prefill_sampled():
    wl = si.config(3)
    say(f"[full] {wl.name}: T={wl.num_tokens} max_len={wl.max_len}")
    dev = Dev(wl)
    idx, out, lse = dev.forward()
    del dev
    # sample: first, last and evenly spaced tokens of the 8192-token chunk, and
    # eight consecutive tokens at eight places, so every one of the eight
    # token slots of the prefill indexer's workgroup is checked
    sample = sorted({0, 1, 4095, 8190, 8191, *range(0, 8192, 1024),
                     *(1024 * i + j for i in range(8) for j in range(8))})
    ref = run_oracle(wl, tokens=sample)
    got_idx = idx.cpu().numpy()[sample]
    assert np.array_equal(got_idx, ref["indices"])
    assert_out_close(out.cpu().numpy()[sample], ref["out"], False, "prefill sample")
    assert_lse_close(lse.cpu().numpy()[sample], ref["lse"], "prefill sample")
