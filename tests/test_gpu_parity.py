"""GPU parity: each C-ABI entry point against the CPU oracle on seeded inputs,
at sizes the oracle finishes in seconds, plus edge cases."""
import numpy as np
import pytest
import torch

import oracle
import sga_inputs as si
from gpu_helpers import (Dev, assert_lse_close, assert_out_close, run_oracle, say, stores)

pytestmark = pytest.mark.gpu


def _check_forward(wl, gate=True, what=""):
    say(f"[forward] {what or wl.name}: T={wl.num_tokens} max_len={wl.max_len} k={wl.k} fp8={wl.fp8}")
    dev = Dev(wl)
    idx, out, lse = dev.forward(gate=gate)
    ref = run_oracle(wl, gate=gate)
    assert np.array_equal(idx.cpu().numpy(), ref["indices"]), "indices differ"
    # MX rows decode exactly to bf16 values: they are held to the bf16 bar
    assert_out_close(out.cpu().numpy(), ref["out"], wl.fp8 and not wl.mx, what)
    assert_lse_close(lse.cpu().numpy(), ref["lse"], what)
    return dev, (idx, out, lse), ref


def test_index_scores_tiny_exact():
    wl = si.config(0)
    say("[index_scores] tiny decode")
    dev = Dev(wl)
    s = dev.scores().cpu().numpy()
    ref = run_oracle(wl, keep_scores=True)
    for i, r in enumerate(ref["scores"]):
        n = r.shape[0]
        assert np.array_equal(s[i, :n].astype(np.float64), r), f"token {i}"
        assert np.all(np.isnan(s[i, n:])), "wrote beyond the visible rows"


def test_topk_tiny_exact():
    wl = si.config(0)
    say("[topk] tiny decode, oracle scores")
    dev = Dev(wl)
    ref = run_oracle(wl, keep_scores=True)
    sc = torch.full((wl.num_tokens, wl.max_len), float("nan"))
    for i, r in enumerate(ref["scores"]):
        sc[i, :r.shape[0]] = torch.from_numpy(r.astype(np.float32))
    idx = dev.topk(sc.cuda())
    assert np.array_equal(idx.cpu().numpy(), ref["indices"])


def test_topk_ties_across_chunks():
    # contexts of 61,439 to 131,072 positions on synthetic scores: from 16
    # chunks of 4,096 positions on, the wave that marks a chunk's candidates
    # also counts and emits it, and ties at the k-th score are kept by lowest
    # position across chunk boundaries. Past each token's visible rows the
    # scores are NaN and must not count.
    wl = si.build("topk_ties", [70001, 131072],
                  [(0, 70000), (1, 131071), (1, 100000), (1, 65535), (1, 61439)], seed=23)
    say("[topk] ties across chunks, 61K-128K positions")
    dev = Dev(wl)
    rng = np.random.default_rng(23)
    sc = np.full((wl.num_tokens, wl.max_len), np.nan, dtype=np.float32)
    # token 0: low scores before 7,001; then zeros of both signs, and 500 high
    # scores after it, so the kept ties run from 7,001 across the chunk edge at 8,192
    n0 = 70001
    s0 = np.where(rng.random(n0) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    s0[:7001] = -1.0 - 2.0 * rng.random(7001)
    s0[rng.choice(np.arange(7001, n0), 500, replace=False)] = 1.0 + rng.random(500)
    sc[0, :n0] = s0
    # token 1: every score equal
    sc[1, :131072] = 0.5
    # tokens 2-4: scores on a grid of 1/4, so the k-th score is shared by
    # positions in every chunk (4: 15 chunks, below the threshold)
    for t, n in ((2, 100001), (3, 65536), (4, 61440)):
        sc[t, :n] = np.round(rng.standard_normal(n) * 4.0) / 4.0
    idx = dev.topk(torch.from_numpy(sc).cuda()).cpu().numpy()
    for t in range(wl.num_tokens):
        n = int(np.sum(~np.isnan(sc[t])))
        ref = oracle.select_topk(sc[t, :n].astype(np.float64), wl.k)
        assert np.array_equal(idx[t], ref), f"token {t} (n={n})"
    ties0 = idx[0][s0[idx[0]] == 0.0]   # kept zeros, either sign
    assert ties0.min() < 8192 < ties0.max(), "the kept ties should cross a chunk edge"
    assert idx[1].tolist() == list(range(2048))


def test_topk_one_kernel_ties_and_spill():
    # 512 tokens: one workgroup per token selects. Rows of equal scores, and
    # scores on a 1/4 grid, put thousands of candidates at the cut, more than
    # the workgroup stages in LDS, so the rest spill to the workspace.
    rng = np.random.default_rng(29)
    n_seq = 20000
    pos = np.sort(rng.integers(0, n_seq, 512))
    pos[-1] = n_seq - 1
    wl = si.build("topk_one_kernel", [n_seq], [(0, int(p)) for p in pos], seed=29)
    say("[topk] one workgroup per token, 512 tokens, ties spilling from LDS")
    dev = Dev(wl)
    sc = np.full((wl.num_tokens, wl.max_len), np.nan, dtype=np.float32)
    for t, p in enumerate(pos):
        n = int(p) + 1
        if t % 2 == 0:
            sc[t, :n] = 1.25
        else:
            sc[t, :n] = np.round(rng.standard_normal(n) * 4.0) / 4.0
    idx = dev.topk(torch.from_numpy(sc).cuda()).cpu().numpy()
    for t, p in enumerate(pos):
        n = int(p) + 1
        ref = oracle.select_topk(sc[t, :n].astype(np.float64), wl.k)
        assert np.array_equal(idx[t], ref), f"token {t} (n={n})"


def test_attention_tiny_given_indices():
    wl = si.config(0)
    say("[attention] tiny decode, oracle indices")
    dev = Dev(wl)
    for gate in (True, False):
        ref = run_oracle(wl, gate=gate)
        out, lse = dev.attention(torch.from_numpy(ref["indices"]).cuda(), gate=gate)
        assert_out_close(out.cpu().numpy(), ref["out"], False, f"gate={gate}")
        assert_lse_close(lse.cpu().numpy(), ref["lse"])


def test_forward_tiny():
    _check_forward(si.config(0))


@pytest.mark.parametrize("S", [1, 2, 31, 33, 2047, 2048, 2049, 5000])
def test_context_lengths_around_k(S):
    # one sequence; tokens at its last position and at a few earlier ones
    pos = sorted({S - 1, max(0, S // 2), 0})
    wl = si.build(f"len{S}", [S], [(0, p) for p in pos], seed=S)
    _check_forward(wl)


@pytest.mark.parametrize("k", [1, 7, 100, 1000])
def test_small_k(k):
    wl = si.build(f"k{k}", [3000], [(0, 2999), (0, 1500)], seed=k, k=k)
    _check_forward(wl)


def test_all_equal_scores():
    wl = si.build("equal", [6000], [(0, 5999), (0, 4000)], seed=3)
    wl.q_idx.zero_()                               # every score is 0: ties everywhere
    _, (idx, _, _), _ = _check_forward(wl)
    assert idx.cpu().numpy()[0].tolist() == list(range(2048))


def test_negative_weights_and_wide_values():
    wl = si.build("negw", [5000], [(0, 4999), (0, 2500), (0, 2100)], seed=4, w_range=(-4, 4))
    _check_forward(wl)


def test_gate_infinities():
    wl = si.build("gate_inf", [3000], [(0, 2999), (0, 2000)], seed=5)
    dev = Dev(wl)
    _, ungated, _ = dev.forward(gate=False)
    dev.gate = torch.full_like(dev.gate, float("inf"))
    _, g_pos, _ = dev.forward()
    assert torch.equal(g_pos, ungated), "gate logit +inf must give the ungated output exactly"
    dev.gate = torch.full_like(dev.gate, float("-inf"))
    _, g_neg, _ = dev.forward()
    assert torch.all(g_neg == 0)


def test_sharp_softmax():
    wl = si.build("sharp", [4500], [(0, 4499), (0, 3000)], seed=6, q_abs_mult=8.0)
    _check_forward(wl)


def test_ragged_batch_many_tokens_per_sequence():
    lens = [100, 2500, 4097, 1, 2049]
    rng = np.random.default_rng(7)
    toks = []
    for b, L in enumerate(lens):
        for p in rng.choice(L, size=min(L, 3), replace=False):
            toks.append((b, int(p)))
    rng.shuffle(toks)
    wl = si.build("ragged", lens, toks, seed=7)
    _check_forward(wl)


def test_histogram_lists_overflow_to_scores():
    # Keys scaled by powers of two (row r by 2^(r mod 10) in alternate blocks of
    # 2,048 rows, else by 2^(r mod 3)): a 256-position indexer chunk then holds
    # 70-85 distinct first-level bins in the wide blocks, more than its list
    # slot takes (63 entries at 64 chunks per token), and 25-30 in the others.
    # The select kernel counts the overflowed chunks from their scores and the
    # rest from their lists. Scores stay integers below 2^24, so exact.
    lengths = [16384, 12000, 16384, 9000, 16384, 15000, 16384, 700]
    wl = si.build("hist_overflow", lengths, [(b, L - 1) for b, L in enumerate(lengths)], seed=41)
    r = torch.arange(wl.k_idx.shape[0])
    mult = torch.pow(2.0, torch.where((r // 2048) % 2 == 0, r % 10, r % 3)).unsqueeze(1)
    wl.k_idx = (wl.k_idx.float() * mult).to(torch.bfloat16)
    say(f"[forward] {wl.name}: T={wl.num_tokens} max_len={wl.max_len}")
    ref = run_oracle(wl, keep_scores=True)
    spread = 0
    for sc in ref["scores"]:
        assert np.all(sc == np.round(sc)) and np.abs(sc).max() < 2.0 ** 24
        keys = sc.astype(np.float32).view(np.uint32)
        digit = np.where(keys >> 31, ~keys, keys | np.uint32(0x80000000)) >> 20
        spread += sum(len(np.unique(digit[c:c + 256])) > 63 for c in range(0, sc.shape[0], 256))
    assert spread > 0, "no chunk holds more bins than its slot"
    idx, out, lse = Dev(wl).forward()
    assert np.array_equal(idx.cpu().numpy(), ref["indices"]), "indices differ"
    assert_out_close(out.cpu().numpy(), ref["out"], False, wl.name)
    assert_lse_close(lse.cpu().numpy(), ref["lse"], wl.name)


def test_many_short_sequences_one_token_each():
    # 520 sequences with one decode token each: with 512 or more tokens the
    # one-workgroup top-k selects, so the decode indexer adds into a dense
    # first-level histogram, which the clear kernel zeroes first
    rng = np.random.default_rng(43)
    lens = rng.integers(300, 700, 520).tolist()
    wl = si.build("many_short_seqs", lens, [(b, L - 1) for b, L in enumerate(lens)], seed=43, k=128)
    _check_forward(wl)


def test_fp8_caches_small():
    wl = si.build("fp8_small", [3000, 2100], [(0, 2999), (1, 2099), (0, 1000)], seed=8, fp8=True)
    _check_forward(wl)


def test_attention_skips_invalid_indices():
    wl = si.build("badidx", [3000], [(0, 2999), (0, 1200)], seed=9)
    dev = Dev(wl)
    ref = run_oracle(wl)
    idx = ref["indices"].copy()
    # poison some entries: -1, beyond the visible rows, far out of range
    idx[0, 5] = -1
    idx[0, 9] = 3000
    idx[1, 3] = 1300
    idx[1, 4] = 1 << 30
    keep = [[j for j in row if 0 <= j <= p] for row, p in zip(idx, wl.token_pos)]
    ks, vs = stores(wl)
    want = []
    for i, kept in enumerate(keep):
        o, l = oracle.sparse_mla(wl.q_abs[i].double().numpy(), vs.rows(np.array(kept, np.int64)), wl.sm_scale)
        want.append(oracle.sigmoid_gate(o, wl.gate[i].double().numpy()))
    out, _ = dev.attention(torch.from_numpy(idx).cuda())
    assert_out_close(out.cpu().numpy(), np.stack(want), False, "poisoned indices")


def test_attention_running_max_jumps():
    # Rows planted in the later tiles of every split whose logits rise far
    # above the rest (by about 15, 30 and 45, natural log, plus a per-split
    # offset): each split's running max jumps after its first tile, so its
    # accumulators are rescaled mid-split, and the merge of the splits meets
    # very different maxima. The lift sits in the 64 RoPE columns, which enter
    # the logits only, so the outputs keep their usual size.
    n = 6000
    wl = si.build("maxjump", [n], [(0, n - 1)], seed=42)
    rng = np.random.default_rng(43)
    sel = np.sort(rng.choice(n, size=wl.k, replace=False)).astype(np.int32)
    q = wl.q_abs[0].double().numpy()
    qsum = q[:, 512:].sum(axis=0)
    unit = qsum / np.linalg.norm(qsum)                  # a RoPE direction every head's query favours
    per_head = q[:, 512:] @ unit                        # logit per unit of length, before sm_scale
    rows_per_split, tile = 128, 32                      # one token: 16 splits of 4 tiles
    kv = wl.kv.clone()
    for s in range(wl.k // rows_per_split):
        for i, lift in ((1, 15.0), (2, 30.0), (3, 45.0)):
            pos = int(sel[s * rows_per_split + i * tile + 7])
            length = (lift + 2.0 * s) / (wl.sm_scale * float(per_head.mean()))
            kv[pos, 512:] = torch.from_numpy(length * unit).to(torch.bfloat16)
    wl.kv = kv
    dev = Dev(wl)
    say("[attention] running max jumps inside splits")
    out, lse = dev.attention(torch.from_numpy(sel[None, :]).cuda())
    _, vs = stores(wl)
    o, l = oracle.sparse_mla(q, vs.rows(sel.astype(np.int64)), wl.sm_scale)
    want = oracle.sigmoid_gate(o, wl.gate[0].double().numpy())
    assert_out_close(out.cpu().numpy()[0], want, False, "max jumps")
    assert_lse_close(lse.cpu().numpy()[0], l, "max jumps")


def test_token_without_visible_rows():
    wl = si.build("novis", [50], [(0, 10), (0, 49)], seed=10)
    dev = Dev(wl)
    dev.batch.token_pos[0] = -1                  # sees nothing
    idx, out, lse = dev.forward()
    assert torch.all(idx[0] == -1)
    assert torch.all(out[0] == 0)
    assert torch.all(torch.isneginf(lse[0]))
    ref = run_oracle(wl, tokens=[1])
    assert np.array_equal(idx[1].cpu().numpy(), ref["indices"][0])


def test_empty_batch_is_a_noop():
    wl = si.build("empty", [10], [], seed=11)
    dev = Dev(wl)
    out = torch.empty((0, 64, 512), dtype=torch.float32, device="cuda")
    import sparse_gated_mla_amd as sga
    sga.sga_forward(dev.batch, dev.q_idx, dev.w, dev.k_idx, None, dev.q_abs, dev.kv, None, 2048,
                    wl.sm_scale, dev.gate, out)
    torch.cuda.synchronize()


def test_unfused_steps_equal_forward():
    wl = si.build("steps", [7000, 3000], [(0, 6999), (1, 2999), (0, 5000)], seed=12)
    dev = Dev(wl)
    idx_f, out_f, lse_f = dev.forward()
    s = dev.scores()
    idx_s = dev.topk(s)
    out_s, lse_s = dev.attention(idx_s)
    assert torch.equal(idx_f, idx_s)
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)


def test_repeat_calls_are_deterministic():
    wl = si.build("repeat", [9000, 4000], [(0, 8999), (1, 3999)], seed=13)
    dev = Dev(wl)
    a = dev.forward()
    b = dev.forward()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_all_equal_scores_spill_past_lds():
    # 50000 tied candidates, two tokens (the cut / select / finalize kernels)
    wl = si.build("equal_spill", [50000], [(0, 49999), (0, 30000)], seed=14)
    wl.q_idx.zero_()
    _, (idx, _, _), _ = _check_forward(wl)
    assert idx.cpu().numpy()[1].tolist() == list(range(2048))


def test_context_beyond_256k_multikernel_topk():
    # above 256K positions the top-k runs as cut / select / finalize kernels
    wl = si.build("len300k", [300000, 5000], [(0, 299999), (1, 4999), (0, 262144)], seed=15)
    _check_forward(wl)


def test_longest_supported_context():
    # 512K positions: the largest visible context the library accepts
    wl = si.build("len512k", [1 << 19], [(0, (1 << 19) - 1), (0, 70000)], seed=16)
    _check_forward(wl)


def test_prefill_many_tokens_one_sequence():
    # at least 64 tokens per sequence: the indexer that shares key tiles across
    # eight tokens runs (its groups of eight hold one sequence here)
    rng = np.random.default_rng(17)
    pos = sorted(rng.choice(5000, size=72, replace=False).tolist())
    wl = si.build("prefill_one_seq", [5000], [(0, p) for p in pos], seed=17)
    _check_forward(wl)


def test_prefill_mixed_sequences_in_a_group():
    # tokens of two sequences interleaved: every group of eight spans both
    rng = np.random.default_rng(18)
    toks = []
    for i in range(136):
        b = i % 2
        toks.append((b, int(rng.integers(0, [3000, 4500][b]))))
    wl = si.build("prefill_mixed", [3000, 4500], toks, seed=18)
    _check_forward(wl)


def test_prefill_fp8():
    rng = np.random.default_rng(19)
    pos = sorted(rng.choice(4200, size=70, replace=False).tolist())
    wl = si.build("prefill_fp8", [4200], [(0, p) for p in pos], seed=19, fp8=True)
    _check_forward(wl)


def test_prefill_index_scores_exact():
    # the unfused scores of the prefill indexer, bit for bit, beyond the chunk of 8
    rng = np.random.default_rng(20)
    pos = sorted(rng.choice(3000, size=67, replace=False).tolist())
    wl = si.build("prefill_scores", [3000], [(0, p) for p in pos], seed=20)
    say("[index_scores] prefill path")
    dev = Dev(wl)
    s = dev.scores().cpu().numpy()
    ref = run_oracle(wl, keep_scores=True)
    for i, r in enumerate(ref["scores"]):
        n = r.shape[0]
        assert np.array_equal(s[i, :n].astype(np.float64), r), f"token {i}"
        assert np.all(np.isnan(s[i, n:])), "wrote beyond the visible rows"


def test_mx_caches_small():
    wl = si.build("mx_small", [3000, 2100], [(0, 2999), (1, 2099), (0, 1000)], seed=21, mx=True)
    _check_forward(wl)


def test_mx_index_scores_exact():
    # integer keys times power-of-two block scales: every score is exact
    wl = si.build("mx_scores", [2500, 700], [(0, 2499), (1, 699), (0, 31)], seed=22, mx=True)
    say("[index_scores] MX keys")
    dev = Dev(wl)
    s = dev.scores().cpu().numpy()
    ref = run_oracle(wl, keep_scores=True)
    for i, r in enumerate(ref["scores"]):
        n = r.shape[0]
        assert np.array_equal(s[i, :n].astype(np.float64), r), f"token {i}"


def test_mx_attention_given_indices():
    wl = si.build("mx_attn", [3000], [(0, 2999), (0, 2047)], seed=23, mx=True)
    say("[attention] MX rows, oracle indices")
    dev = Dev(wl)
    ref = run_oracle(wl)
    out, lse = dev.attention(torch.from_numpy(ref["indices"]).cuda())
    assert_out_close(out.cpu().numpy(), ref["out"], False, "mx attention")
    assert_lse_close(lse.cpu().numpy(), ref["lse"], "mx attention")


def test_prefill_mx():
    rng = np.random.default_rng(24)
    pos = sorted(rng.choice(4200, size=70, replace=False).tolist())
    wl = si.build("prefill_mx", [4200], [(0, p) for p in pos], seed=24, mx=True)
    _check_forward(wl)


def test_mx4_caches_small():
    wl = si.build("mx4_small", [3000, 2100], [(0, 2999), (1, 2099), (0, 1000)], seed=25, mx4=True)
    _check_forward(wl)


def test_mx4_index_scores_exact():
    wl = si.build("mx4_scores", [2500, 700], [(0, 2499), (1, 699), (0, 31)], seed=26, mx4=True)
    say("[index_scores] four-bit MX keys")
    dev = Dev(wl)
    s = dev.scores().cpu().numpy()
    ref = run_oracle(wl, keep_scores=True)
    for i, r in enumerate(ref["scores"]):
        n = r.shape[0]
        assert np.array_equal(s[i, :n].astype(np.float64), r), f"token {i}"


def test_mx4_attention_given_indices():
    wl = si.build("mx4_attn", [3000], [(0, 2999), (0, 2047)], seed=27, mx4=True)
    say("[attention] four-bit MX rows, oracle indices")
    dev = Dev(wl)
    ref = run_oracle(wl)
    out, lse = dev.attention(torch.from_numpy(ref["indices"]).cuda())
    assert_out_close(out.cpu().numpy(), ref["out"], False, "mx4 attention")
    assert_lse_close(lse.cpu().numpy(), ref["lse"], "mx4 attention")


def test_prefill_mx4():
    rng = np.random.default_rng(28)
    pos = sorted(rng.choice(4200, size=70, replace=False).tolist())
    wl = si.build("prefill_mx4", [4200], [(0, p) for p in pos], seed=28, mx4=True)
    _check_forward(wl)


# ------------------------------------------------------------------ k above 4096
def test_k_6000_two_tokens():
    # two tokens: the select kernels and the top-k stage inside the attention
    # (47 splits, so the merge takes three rounds); the standalone top-k on the
    # oracle's scores stores its output unstaged (k > 4096)
    wl = si.build("k6000_t2", [20000], [(0, 19999), (0, 15000)], seed=35, k=6000)
    _, (idx, _, _), ref = _check_forward(wl)
    say("[topk] k=6000, oracle scores, select + finalize")
    ref_s = run_oracle(wl, keep_scores=True)
    sc = torch.full((wl.num_tokens, wl.max_len), float("nan"))
    for i, r in enumerate(ref_s["scores"]):
        sc[i, :r.shape[0]] = torch.from_numpy(r.astype(np.float32))
    got = Dev(wl).topk(sc.cuda()).cpu().numpy()
    assert np.array_equal(got, ref["indices"])


def test_k_6000_many_tokens():
    # 512 tokens: one workgroup per token selects, one split per token
    rng = np.random.default_rng(36)
    pos = np.sort(rng.integers(0, 20000, 512))
    pos[-1] = 19999
    pos[:8] = np.arange(8)          # a few tokens with fewer positions than k
    wl = si.build("k6000_t512", [20000], [(0, int(p)) for p in pos], seed=36, k=6000)
    _check_forward(wl)


def test_k_65536_at_100k():
    # the largest k: 64 splits of 1,024 rows, merged in four rounds
    wl = si.build("k65536", [100000], [(0, 99999), (0, 70000)], seed=37, k=65536)
    _check_forward(wl)
    say("[topk] k=65536, oracle scores, select + finalize")
    ref_s = run_oracle(wl, keep_scores=True)
    sc = torch.full((wl.num_tokens, wl.max_len), float("nan"))
    for i, r in enumerate(ref_s["scores"]):
        sc[i, :r.shape[0]] = torch.from_numpy(r.astype(np.float32))
    got = Dev(wl).topk(sc.cuda()).cpu().numpy()
    assert np.array_equal(got, ref_s["indices"])


# ------------------------------------------- MX block exponents over their range
MX_EXP_MIN = {"mx": 10, "mx4": 2}
MX_EXP_MAX = 200


def _mx_build(fmt, name, lengths, tokens, seed, **kw):
    return si.build(name, lengths, tokens, seed, mx=fmt == "mx", mx4=fmt == "mx4", **kw)


@pytest.mark.parametrize("fmt", ["mx", "mx4"])
def test_mx_attention_exponent_range_single_rows(fmt):
    # every block exponent of the latent rows drawn over the whole accepted
    # range; each of 256 tokens (one split each) attends to a single row, so its
    # output is that row's decoded values, exactly, and its lse is 0
    T, k = 256, 64
    wl = _mx_build(fmt, f"{fmt}_exp_rows", [4096], [(0, 4095)] * T, 38, k=k)
    rng = np.random.default_rng(38)
    e = rng.integers(MX_EXP_MIN[fmt], MX_EXP_MAX + 1, size=tuple(wl.kv_scale.shape))
    wl.kv_scale = torch.from_numpy(e.astype(np.uint8))
    wl.q_abs.zero_()
    rows = rng.choice(4096, size=T, replace=False)
    ind = np.full((T, k), -1, dtype=np.int32)
    ind[np.arange(T), rng.integers(0, k, size=T)] = rows
    say(f"[attention] {fmt} rows, block exponents {MX_EXP_MIN[fmt]}..{MX_EXP_MAX}, one row per token")
    out, lse = Dev(wl).attention(torch.from_numpy(ind).cuda(), gate=False)
    _, vs = stores(wl)
    got, got_lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy()
    for t in range(T):
        o, l = oracle.sparse_mla(wl.q_abs[t].double().numpy(), vs.rows(rows[t:t + 1]), wl.sm_scale)
        assert np.array_equal(got[t], o), f"token {t}"
        assert np.array_equal(got_lse[t], l), f"token {t}"


@pytest.mark.parametrize("fmt", ["mx", "mx4"])
def test_mx_attention_exponent_range_oracle_indices(fmt):
    # the first 256 latent columns (values only: their query columns are zero)
    # take block exponents over the whole accepted range; the rest keep the
    # usual ones. Two tokens, 16 splits each: every column is held to its
    # error bound, 2^-8 of sum_j p_j |v_j| plus 2^-24 of the largest |v| in its
    # half of the selected rows (the fp16 partials)
    wl = _mx_build(fmt, f"{fmt}_exp_attn", [6000], [(0, 5999), (0, 3000)], 39)
    rng = np.random.default_rng(39)
    e = wl.kv_scale.numpy().copy()
    e[:, :8] = rng.integers(MX_EXP_MIN[fmt], MX_EXP_MAX + 1, size=(e.shape[0], 8))
    wl.kv_scale = torch.from_numpy(e)
    wl.q_abs[:, :, :256] = 0
    ref = run_oracle(wl, gate=False)
    say(f"[attention] {fmt} rows, value-block exponents {MX_EXP_MIN[fmt]}..{MX_EXP_MAX}, oracle indices")
    out, lse = Dev(wl).attention(torch.from_numpy(ref["indices"]).cuda(), gate=False)
    assert_lse_close(lse.cpu().numpy(), ref["lse"], f"{fmt} exponent range")
    got = out.cpu().numpy().astype(np.float64)
    _, vs = stores(wl)
    for t in range(wl.num_tokens):
        kept = ref["indices"][t][ref["indices"][t] >= 0].astype(np.int64)
        v = vs.rows(int(wl.seq_start[wl.token_seq[t]]) + kept)
        z = wl.sm_scale * (wl.q_abs[t].double().numpy() @ v.T)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        a = p @ np.abs(v[:, :512])
        half_max = np.repeat([np.abs(v[:, :256]).max(), np.abs(v[:, 256:512]).max()], 256)
        bound = 2.0 ** -8 * a + 2.0 ** -24 * half_max[None, :] + 2.0 ** -140
        err = np.abs(got[t] - ref["out"][t])
        assert np.all(err <= bound), (fmt, t, float((err / bound).max()))


@pytest.mark.parametrize("fmt", ["mx", "mx4"])
def test_mx_index_scores_exponent_range(fmt):
    # each key row keeps one nonzero 32-element block, whose exponent is drawn
    # over the whole accepted range: every score is still an exact sum of
    # same-scale integers, so scores and indices match bit for bit
    wl = _mx_build(fmt, f"{fmt}_key_exps", [3000, 900], [(0, 2999), (1, 899), (0, 100)], 40)
    rng = np.random.default_rng(40)
    rows = wl.k_idx.shape[0]
    keep = rng.integers(0, 4, size=rows)
    raw = wl.k_idx.view(torch.uint8).numpy().copy()
    per_block = raw.shape[1] // 4
    for b in range(4):
        raw[keep != b, b * per_block:(b + 1) * per_block] = 0      # +0 in both element codes
    e = rng.integers(MX_EXP_MIN[fmt], MX_EXP_MAX + 1, size=(rows, 4))
    wl.k_idx = torch.from_numpy(raw).view(wl.k_idx.dtype)
    wl.k_idx_scale = torch.from_numpy(e.astype(np.uint8))
    say(f"[index_scores] {fmt} keys, block exponents {MX_EXP_MIN[fmt]}..{MX_EXP_MAX}")
    s = Dev(wl).scores().cpu().numpy()
    ref = run_oracle(wl, keep_scores=True)
    for i, r in enumerate(ref["scores"]):
        n = r.shape[0]
        assert np.array_equal(s[i, :n].astype(np.float64), r), f"token {i}"
    _check_forward(wl, what=f"{fmt} keys over the exponent range")
