"""Seeded random batches against the oracle: ragged sequence lengths, several
tokens per sequence at random positions, random k and cache formats, so that
the launch-time choices (indexer chunk length, the selecting attention or the
windowed final stage, split counts) meet odd sizes. Indices bit-exact, outputs
at the bf16 bar (MX and bf16 caches) or the fp8 bar."""
import numpy as np
import pytest

import sga_inputs as si
from gpu_helpers import Dev, assert_lse_close, assert_out_close, run_oracle, say

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 6))
    top = int(rng.choice([3000, 20000, 70000, 150000]))
    lengths = [int(x) for x in rng.integers(1, top + 1, size=B)]
    tokens = []
    for b, n in enumerate(lengths):
        for _ in range(int(rng.integers(1, 4))):
            tokens.append((b, int(rng.integers(0, n))))
        tokens.append((b, n - 1))
    k = int(rng.choice([1, 64, 777, 2048, 3000, 5000]))
    fmt = str(rng.choice(["bf16", "fp8", "mx", "mx4"]))
    return lengths, tokens, k, fmt


@pytest.mark.parametrize("seed", range(12))
def test_random_batch(seed):
    lengths, tokens, k, fmt = _draw(seed)
    wl = si.build(f"random{seed}", lengths, tokens, seed=6000 + seed, k=k,
                  fp8=fmt == "fp8", mx=fmt == "mx", mx4=fmt == "mx4")
    say(f"[random {seed}] B={len(lengths)} T={wl.num_tokens} max_len={wl.max_len} k={k} fmt={fmt}")
    idx, out, lse = Dev(wl).forward()
    ref = run_oracle(wl)
    got = idx.cpu().numpy()
    bad = [t for t in range(wl.num_tokens) if not np.array_equal(got[t], ref["indices"][t])]
    assert not bad, f"indices differ for tokens {bad}"
    assert_out_close(out.cpu().numpy(), ref["out"], wl.fp8 and not wl.mx, wl.name)
    assert_lse_close(lse.cpu().numpy(), ref["lse"], wl.name)
