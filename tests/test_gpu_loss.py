"""GPU parity for sga_indexer_loss (the sparse indexer loss: KL from the
head-mean attention distribution over each token's selected rows to the softmax
of its indexer scores over them) against the oracle's indexer loss."""
import numpy as np
import pytest
import torch

import oracle
import sga_inputs as si
import sparse_gated_mla_amd as sga
from gpu_helpers import Dev, say, stores

pytestmark = pytest.mark.gpu

# fp32 throughout: logits and exponentials to about 1e-6 relative, sums over at
# most a few thousand selected rows
LOSS_REL, LOSS_ABS = 1e-4, 1e-6


def _gpu_loss(wl, dev):
    idx, _, lse = dev.forward()
    scores = dev.scores()
    loss = torch.full((wl.num_tokens,), float("nan"), dtype=torch.float32, device="cuda")
    sga.sga_indexer_loss(dev.batch, dev.q_abs, dev.kv, dev.kv_scale, idx, wl.k, wl.sm_scale, lse,
                         scores, loss)
    torch.cuda.synchronize()
    return loss.cpu().numpy()


def _oracle_loss(wl, tokens=None):
    ks, vs = stores(wl)
    return oracle.indexer_loss(wl.token_seq, wl.token_pos, wl.seq_start, wl.seq_len,
                               wl.q_idx.double().numpy(), wl.w.double().numpy(), ks,
                               wl.q_abs.double().numpy(), vs, wl.k, wl.sm_scale, tokens=tokens)


def _check(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    say(f"  {what}: loss {np.round(ref[:4], 5)} max|diff| {err.max():.3e}")
    assert np.all(err <= LOSS_ABS + LOSS_REL * np.abs(ref)), (what, got, ref)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mx", "mx4"])
def test_indexer_loss_matches_oracle(fmt):
    kw = {"bf16": {}, "fp8": {"fp8": True}, "mx": {"mx": True}, "mx4": {"mx4": True}}[fmt]
    wl = si.build(f"loss_{fmt}", [3000, 2100, 900], [(0, 2999), (1, 2099), (0, 1500), (2, 899)],
                  seed=40, **kw)
    say(f"[indexer_loss] {fmt}")
    dev = Dev(wl)
    _check(_gpu_loss(wl, dev), _oracle_loss(wl), fmt)


def test_indexer_loss_sharp_and_edge_tokens():
    # a sharp softmax (q x 8); a token that keeps every visible row; a token
    # with no visible rows (its sequence has length 0) gets loss 0
    wl = si.build("loss_edge", [5000, 40, 0], [(0, 4999), (1, 39), (0, 100), (2, 0)], seed=41,
                  q_abs_mult=8.0)
    say("[indexer_loss] sharp softmax, k above the visible rows, an empty token")
    dev = Dev(wl)
    got = _gpu_loss(wl, dev)
    assert got[3] == 0.0
    _check(got[:3], _oracle_loss(wl, tokens=[0, 1, 2]), "edge")


def test_indexer_loss_full_size_decode():
    wl = si.config(2)
    say(f"[indexer_loss] {wl.name}")
    dev = Dev(wl)
    got = _gpu_loss(wl, dev)
    del dev
    _check(got, _oracle_loss(wl), wl.name)
