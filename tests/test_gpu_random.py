"""Seeded random batches against the oracle: ragged sequence lengths, several
tokens per sequence at random positions (or 64-99, for the indexer that
shares key tiles across tokens), random k and cache formats, so that
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


def _draw_many_tokens(seed):
    # 64-99 tokens at distinct random positions of each of one or two
    # sequences: the indexer that shares key tiles across eight tokens runs
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 3))
    lengths = [int(x) for x in rng.integers(200, 20001, size=B)]
    tokens = []
    for b, n in enumerate(lengths):
        for p in rng.choice(n, size=int(rng.integers(64, 100)), replace=False):
            tokens.append((b, int(p)))
    k = int(rng.choice([1, 64, 777, 2048, 3000]))
    fmt = str(rng.choice(["bf16", "fp8", "mx", "mx4"]))
    return lengths, tokens, k, fmt


def _check(name, lengths, tokens, k, fmt, seed):
    wl = si.build(name, lengths, tokens, seed=seed, k=k,
                  fp8=fmt == "fp8", mx=fmt == "mx", mx4=fmt == "mx4")
    say(f"[{name}] B={len(lengths)} T={wl.num_tokens} max_len={wl.max_len} k={k} fmt={fmt}")
    idx, out, lse = Dev(wl).forward()
    ref = run_oracle(wl)
    got = idx.cpu().numpy()
    bad = [t for t in range(wl.num_tokens) if not np.array_equal(got[t], ref["indices"][t])]
    assert not bad, f"indices differ for tokens {bad}"
    assert_out_close(out.cpu().numpy(), ref["out"], wl.fp8 and not wl.mx, wl.name)
    assert_lse_close(lse.cpu().numpy(), ref["lse"], wl.name)


@pytest.mark.parametrize("seed", range(12))
def test_random_batch(seed):
    _check(f"random{seed}", *_draw(seed), seed=6000 + seed)


@pytest.mark.parametrize("seed", [4, 9, 14, 19])
def test_random_batch_many_tokens_per_sequence(seed):
    _check(f"random_many{seed}", *_draw_many_tokens(seed), seed=7000 + seed)
