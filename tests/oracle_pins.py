"""Checks that pin the CPU oracle to facts outside itself.

Each check takes the oracle module and raises AssertionError when it disagrees
with one of these:
- a hand-worked example (tests/golden);
- a closed form;
- a library routine (torch's scaled_dot_product_attention, logsumexp, dtype casts);
- a brute-force definition on tiny inputs.
test_oracle_pins.py runs the checks on the real oracle. test_oracle_mutations.py
runs them on oracles with planted mistakes and expects at least one check to fail.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats
def check_bf16_decode(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.decode_bf16(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "bf16 decode disagrees with torch's bfloat16"


def check_e4m3fn_table(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3fn_table()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "E4M3FN table disagrees with torch.float8_e4m3fn"
    # named values of the OCP format: max normal, min subnormal, one, NaN
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    scaled = orc.decode_e4m3fn(np.array([[0x38, 0x7E]], np.uint8), np.array([0.25], np.float32))
    assert scaled.tolist() == [[0.25, 112.0]]


def check_e4m3fn_encode(orc):
    # against torch's float8_e4m3fn cast (round to nearest, ties to even): random
    # values over many magnitudes, every midpoint between neighbours, every
    # representable value, both signs
    rng = np.random.default_rng(0)
    x = rng.normal(size=20000) * rng.choice([1e-3, 0.1, 1.0, 100.0], size=20000)
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    vals = orc.e4m3fn_table()[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, vals.astype(np.float32), -vals.astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.encode_e4m3fn(x.astype(np.float64))
    assert np.array_equal(got, ref), "E4M3FN encode disagrees with torch.float8_e4m3fn"
    # the reading's saturation at 448, and the sign of zero
    assert orc.encode_e4m3fn(np.array([500.0, -1e6, -0.0, 0.0])).tolist() == [0x7E, 0xFE, 0x80, 0x00]


def check_quantize_rows(orc):
    rng = np.random.default_rng(1)
    x = (rng.normal(size=(64, 576)) / 24).astype(np.float32)
    x[5] *= 1e-6              # small rows still use the full range
    x[3] = 0.0
    pay, sc = orc.quantize_rows_e4m3fn(x)
    dec = orc.decode_e4m3fn(pay, sc)
    table = orc.e4m3fn_table()
    for i in range(len(x)):
        if i == 3:
            assert sc[i] == 1.0 and not pay[i].any(), "a zero row"
            continue
        # the row's largest magnitude lands on the largest code, 448
        assert np.abs(table[pay[i]]).max() == 448.0
        # round to nearest: the error is at most half the code spacing (1/8 of
        # the binade, 2^-9 below the normals) times the scale
        a = np.abs(x[i].astype(np.float64)) / float(sc[i])
        spacing = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3), 2.0 ** -9)
        err = np.abs(dec[i] - x[i].astype(np.float64))
        assert np.all(err <= 0.5 * spacing * float(sc[i]) * (1 + 1e-6)), i


def check_cache_append(orc):
    # sequence 0 at rows 0..4, sequence 1 at rows 10..12
    token_seq = np.array([0, 1, 1, 2, 0], np.int32)
    token_pos = np.array([4, 2, 3, 0, -1], np.int32)
    seq_start = np.array([0, 10], np.int64)
    seq_len = np.array([5, 3], np.int32)
    rows = np.arange(5 * 8, dtype=np.uint16).reshape(5, 8) + 0x3F80
    got = orc.cache_append(token_seq, token_pos, seq_start, seq_len, 13, rows, "bf16")
    assert sorted(got) == [4, 12], sorted(got)
    assert np.array_equal(got[4][0], rows[0]) and np.array_equal(got[12][0], rows[1])
    q = orc.cache_append(token_seq, token_pos, seq_start, seq_len, 13, rows, "e4m3fn")
    assert sorted(q) == [4, 12]
    assert np.allclose(orc.decode_e4m3fn(q[4][0][None], np.array([q[4][1]]))[0],
                       orc.decode_bf16(rows[0]), rtol=1 / 16, atol=0)
    f4 = orc.cache_append(token_seq, token_pos, seq_start, seq_len, 13,
                          np.tile(rows, (1, 4)), "mxfp4")
    assert sorted(f4) == [4, 12] and f4[4][0].shape == (16,) and f4[4][1].shape == (1,)
    m = orc.cache_append(token_seq, token_pos, seq_start, seq_len, 13,
                         np.tile(rows, (1, 4)), "mxfp8")
    assert sorted(m) == [4, 12] and m[4][1].shape == (1,)
    assert np.allclose(orc.decode_mxfp8(m[12][0][None], m[12][1][None])[0],
                       orc.decode_bf16(np.tile(rows[1], 4)), rtol=1 / 16, atol=0)


def check_e8m0_table(orc):
    # against torch's float8_e8m0fnu -> float32 for every code (255 is NaN)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    got = orc.e8m0_table()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255].astype(np.float64)), "E8M0 table disagrees with torch"


def check_mxfp8_worked_example(orc):
    g = _golden("mxfp8_worked_example.json")
    x = np.zeros((1, 96))
    for blk, off in (("block0", 0), ("block1", 32)):
        for i, v in g[blk]["values"].items():
            x[0, off + int(i)] = v
    pay, ex = orc.quantize_blocks_mxfp8(x)
    assert ex.tolist() == [[g["block0"]["exp"], g["block1"]["exp"], g["zero_block"]["exp"]]], ex
    for blk, off in (("block0", 0), ("block1", 32)):
        for i, c in g[blk]["codes"].items():
            assert int(pay[0, off + int(i)]) == c, (blk, i, int(pay[0, off + int(i)]), c)
    assert not pay[0, 64:].any()


def check_mxfp8_brute_force(orc):
    # every element is the nearest of all finite E4M3FN values times its block's
    # scale (ties to the even code, beyond 448 the largest), and the block's
    # exponent is floor(log2 max|x|) - 8, found by search over powers of two
    rng = np.random.default_rng(3)
    x = rng.normal(size=(6, 128)) * np.ldexp(1.0, rng.integers(-20, 20, size=(6, 1)))
    x[2, 32:64] = 0.0
    x[4, :32] = 0.0                                  # max 1: scale 2^-8, ties among subnormals
    x[4, 0] = 1.0
    x[4, 1:4] = np.array([1.5, 0.5, 2.5]) * 2.0 ** -17
    pay, ex = orc.quantize_blocks_mxfp8(x)
    table = orc.e4m3fn_table()
    codes = np.array([c for c in range(256) if not np.isnan(table[c])])
    for r in range(x.shape[0]):
        for b in range(4):
            blk = x[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                assert ex[r, b] == 0 and not pay[r, 32 * b:32 * b + 32].any()
                continue
            e = 0
            while 2.0 ** (e + 1) <= amax:
                e += 1
            while 2.0 ** e > amax:
                e -= 1
            assert int(ex[r, b]) == e - 8 + 127, (r, b)
            sc = 2.0 ** (e - 8)
            for j, v in enumerate(blk):
                a = min(abs(v) / sc, 448.0)
                d = np.abs(np.abs(table[codes]) - a)
                best = codes[(d == d.min()) & (codes < 0x80)]
                want = best[best % 2 == 0][0] if len(best) > 1 else best[0]
                if v < 0 or (v == 0 and np.signbit(v)):
                    want |= 0x80
                assert int(pay[r, 32 * b + j]) == int(want), (r, b, j, v)


def check_mxfp8_scale_invariance(orc):
    # scaling a block by 2^k keeps its payload and moves its exponent by k
    rng = np.random.default_rng(4)
    x = rng.normal(size=(3, 64))
    p0, e0 = orc.quantize_blocks_mxfp8(x)
    for k in (-9, 1, 17):
        p1, e1 = orc.quantize_blocks_mxfp8(np.ldexp(x, k))
        assert np.array_equal(p0, p1) and np.array_equal(e1.astype(int), e0.astype(int) + k)
    dec = orc.decode_mxfp8(p0, e0)
    assert np.allclose(dec, x, rtol=1 / 16, atol=0)


def check_e2m1_table(orc):
    # the format's value list (OCP E2M1): 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = orc.e2m1_table()
    assert t[:8].tolist() == mags and t[8:].tolist() == [-m for m in mags]
    assert np.signbit(t[8])


def check_mxfp4_worked_example(orc):
    g = _golden("mxfp4_worked_example.json")
    x = np.zeros((1, 32))
    for i, v in g["values"].items():
        x[0, int(i)] = v
    pay, ex = orc.quantize_blocks_mxfp4(x)
    assert ex.tolist() == [[g["exp"]]], ex
    for i, b in g["bytes"].items():
        assert int(pay[0, int(i)]) == b, (i, int(pay[0, int(i)]), b)
    assert not pay[0, 4:].any()


def check_mxfp4_brute_force(orc):
    # every element is the nearest of the 16 E2M1 values times its block's scale
    # (ties to the even code, beyond 6 the largest); exponent found by search
    rng = np.random.default_rng(5)
    x = rng.normal(size=(5, 96)) * np.ldexp(1.0, rng.integers(-15, 15, size=(5, 1)))
    x[1, 32:64] = 0.0
    x[2, :32] = 0.0
    x[2, 0] = 4.0                                     # scale 1: ties among the codes
    x[2, 1:9] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75]
    pay, ex = orc.quantize_blocks_mxfp4(x)
    codes = np.empty(x.shape, dtype=np.uint8)
    codes[:, 0::2], codes[:, 1::2] = pay & 0xF, pay >> 4
    table = orc.e2m1_table()
    for r in range(x.shape[0]):
        for b in range(3):
            blk = x[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                assert ex[r, b] == 0 and not codes[r, 32 * b:32 * b + 32].any()
                continue
            e = 0
            while 2.0 ** (e + 1) <= amax:
                e += 1
            while 2.0 ** e > amax:
                e -= 1
            assert int(ex[r, b]) == e - 2 + 127, (r, b)
            sc = 2.0 ** (e - 2)
            for j, v in enumerate(blk):
                a = min(abs(v) / sc, 6.0)
                d = np.abs(table[:8] - a)
                best = np.flatnonzero(d == d.min())
                want = best[best % 2 == 0][0] if len(best) > 1 else best[0]
                if v < 0 or (v == 0 and np.signbit(v)):
                    want |= 8
                assert int(codes[r, 32 * b + j]) == int(want), (r, b, j, v)


def check_mxfp4_scale_invariance(orc):
    rng = np.random.default_rng(6)
    x = rng.normal(size=(3, 64))
    p0, e0 = orc.quantize_blocks_mxfp4(x)
    for k in (-11, 2, 30):
        p1, e1 = orc.quantize_blocks_mxfp4(np.ldexp(x, k))
        assert np.array_equal(p0, p1) and np.array_equal(e1.astype(int), e0.astype(int) + k)
    dec = orc.decode_mxfp4(p0, e0)
    amax = np.abs(x).reshape(3, 2, 32).max(axis=2).repeat(32, axis=1)
    assert np.all(np.abs(dec - x) <= amax / 4 + 1e-12)   # half of E2M1's widest step, scaled


def check_forward_mxfp4_store(orc):
    """The path over MX block-32 stores with E2M1 elements equals the path over
    the same values stored exactly in bf16."""
    rng = np.random.default_rng(14)
    n = 24
    codes = rng.integers(0, 16, (n, 576)).astype(np.uint8)
    exps = rng.integers(118, 126, (n, 18)).astype(np.uint8)
    vals = orc.e2m1_table()[codes] * np.ldexp(1.0, exps.astype(int) - 127).repeat(32, axis=1)
    vals_bits = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(vals_bits.double().numpy(), vals)
    kint = rng.integers(-3, 4, (n, 128))
    kcodes = orc.encode_e2m1(kint.astype(float))
    kexps = rng.integers(125, 130, (n, 4)).astype(np.uint8)
    kvals = torch.from_numpy((kint * np.ldexp(1.0, kexps.astype(int) - 127).repeat(32, axis=1)).astype(np.float32))
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    q_idx = rng.integers(-3, 4, (1, 64, 128)).astype(float)
    w = rng.integers(0, 5, (1, 64)).astype(float)
    q_abs = rng.standard_normal((1, 64, 576))
    tau = 1 / math.sqrt(192)
    args = (np.zeros(1, np.int32), np.array([n - 1], np.int32), np.zeros(1, np.int64), np.array([n], np.int32))
    a = orc.forward(*args, q_idx, w, orc.Store(pack(kcodes), "mxfp4", kexps), q_abs,
                    orc.Store(pack(codes), "mxfp4", exps), None, 5, tau)
    b = orc.forward(*args, q_idx, w, orc.Store(kvals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), "bf16"),
                    q_abs, orc.Store(vals_bits.view(torch.int16).numpy().view(np.uint16), "bf16"), None, 5, tau)
    assert np.array_equal(a["indices"], b["indices"])
    assert np.allclose(a["out"], b["out"], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- indexer
def check_indexer_worked_example(orc):
    g = _golden("indexer_worked_example.json")
    s = orc.index_scores(np.array(g["q_idx"], float), np.array(g["w"], float), np.array(g["keys"], float))
    assert s.tolist() == [float(x) for x in g["scores"]], s


def check_indexer_exact_integer(orc):
    """For integer inputs the fp64 result must be the exact integer result
    (|sums| < 2**53). Also checks that positive scaling of a key scales its score."""
    rng = np.random.default_rng(5)
    q = rng.integers(-3, 4, size=(64, 128))
    w = rng.integers(-4, 5, size=64)
    keys = rng.integers(-3, 4, size=(300, 128))
    got = orc.index_scores(q.astype(float), w.astype(float), keys.astype(float))
    # exact integer arithmetic, one head at a time
    exact = np.zeros(300, dtype=np.int64)
    for h in range(64):
        d = keys.astype(np.int64) @ q[h].astype(np.int64)
        exact += w[h] * np.where(d > 0, d, 0)
    assert np.array_equal(got, exact.astype(float))
    got2 = orc.index_scores(q.astype(float), w.astype(float), 4.0 * keys.astype(float))
    assert np.array_equal(got2, 4.0 * got)


# ---------------------------------------------------------------- top-k
def _rank_select(scores, k):
    """Definition by rank: position i is kept iff fewer than k positions precede
    it (higher score, or equal score at a lower position)."""
    n = len(scores)
    kept = []
    for i in range(n):
        ahead = sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if ahead < k:
            kept.append(i)
    return kept + [-1] * (k - len(kept))


def check_topk_worked_example(orc):
    g = _golden("indexer_worked_example.json")
    for k, exp in g["topk"].items():
        got = orc.select_topk(np.array(g["scores"], float), int(k))
        assert got.tolist() == exp, (k, got)


def check_topk_rank_definition(orc):
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(1, 120))
        k = int(rng.integers(1, 140))
        scores = rng.integers(-4, 5, size=n).astype(float)   # many ties on purpose
        if trial % 5 == 0:
            scores = rng.standard_normal(n)
        got = orc.select_topk(scores, k)
        assert got.tolist() == _rank_select(list(scores), k), (n, k)


def check_topk_enumeration(orc):
    """For n <= 8 enumerate every subset of size min(k, n) and keep those in which
    every member precedes every non-member; exactly one must exist, and it is the
    oracle's answer."""
    rng = np.random.default_rng(11)
    for _ in range(60):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 10))
        scores = rng.integers(0, 3, size=n).astype(float)
        m = min(k, n)

        def before(i, j):
            return scores[i] > scores[j] or (scores[i] == scores[j] and i < j)

        winners = [set(c) for c in itertools.combinations(range(n), m)
                   if all(before(i, j) for i in c for j in range(n) if j not in c)]
        assert len(winners) == 1
        got = orc.select_topk(scores, k)
        assert sorted(winners[0]) + [-1] * (k - m) == got.tolist()


def check_topk_special_cases(orc):
    assert orc.select_topk(np.full(50, 7.0), 10).tolist() == list(range(10))
    assert orc.select_topk(np.arange(5, 0, -1, dtype=float), 8).tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    # -0.0 and +0.0 tie: the lower position wins
    assert orc.select_topk(np.array([-1.0, 0.0, -0.0, 0.0]), 2).tolist() == [1, 2]
    assert orc.select_topk(np.array([-1.0, -0.0, 0.0]), 1).tolist() == [1]
    assert orc.select_topk(np.array([3.0]), 1).tolist() == [0]


# ---------------------------------------------------------------- attention
def check_attention_closed_form(orc):
    g = _golden("attention_two_rows.json")
    rows = np.zeros((2, 576))
    rows[0, 530] = g["a"]
    rows[0, :3] = g["v0"]
    rows[1, :3] = g["v1"]
    q = np.zeros((1, 576))
    q[0, 530] = math.log(3.0) / (g["sm_scale"] * g["a"])
    o, lse = orc.sparse_mla(q, rows, g["sm_scale"])
    assert o.shape == (1, 512)
    assert np.allclose(o[0, :3], g["expected_o_first3"], rtol=0, atol=1e-14)
    assert np.all(o[0, 3:] == 0.0)
    assert abs(lse[0] - g["expected_lse"]) < 1e-14
    gated = orc.sigmoid_gate(o, np.array([g["gate_logit"]]))
    assert np.allclose(gated[0, :3], g["expected_gated_first3"], rtol=0, atol=1e-14)


def check_attention_vs_sdpa(orc):
    """Selecting every row reproduces dense attention over those rows
    (torch scaled_dot_product_attention, fp64, one shared K/V for all heads)."""
    rng = np.random.default_rng(3)
    m = 37
    rows = rng.standard_normal((m, 576)) / 24
    q = rng.standard_normal((64, 576)) * 4        # sharp softmax
    tau = 1 / math.sqrt(192)
    o, lse = orc.sparse_mla(q, rows, tau)
    Q = torch.from_numpy(q)[None, :, None, :]                       # [1,H,1,576]
    K = torch.from_numpy(rows)[None, None].expand(1, 64, m, 576)
    V = torch.from_numpy(rows[:, :512])[None, None].expand(1, 64, m, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=tau)[0, :, 0].numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-14)
    z = torch.from_numpy(tau * (q @ rows.T))
    assert np.allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=1e-13, atol=1e-13)


def check_attention_special_cases(orc):
    rng = np.random.default_rng(4)
    rows = rng.standard_normal((9, 576))
    q = rng.standard_normal((64, 576))
    o1, lse1 = orc.sparse_mla(q, rows[3:4], 0.07)
    assert np.array_equal(o1, np.broadcast_to(rows[3, :512], (64, 512)))   # one row: weight 1
    assert np.allclose(lse1, 0.07 * (q @ rows[3]), rtol=1e-14, atol=1e-14)
    o0, _ = orc.sparse_mla(np.zeros((64, 576)), rows, 0.07)                 # zero query: mean
    assert np.allclose(o0, np.broadcast_to(rows[:, :512].mean(axis=0), (64, 512)), rtol=1e-13, atol=1e-15)
    perm = rng.permutation(9)                                               # order of rows is irrelevant
    a, la = orc.sparse_mla(q, rows, 0.07)
    b, lb = orc.sparse_mla(q, rows[perm], 0.07)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15) and np.allclose(la, lb, rtol=1e-13)
    oe, le = orc.sparse_mla(q, rows[:0], 0.07)                              # no rows
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def check_gate(orc):
    rng = np.random.default_rng(6)
    o = rng.standard_normal((64, 512))
    g = np.full(64, np.inf)
    assert np.array_equal(orc.sigmoid_gate(o, g), o)                        # +inf: ungated
    out = orc.sigmoid_gate(o, -g)
    assert np.all(out == 0)                                                 # -inf: closed
    assert np.array_equal(orc.sigmoid_gate(o, np.zeros(64)), 0.5 * o)       # 0: half
    h = orc.sigmoid_gate(o, np.full(64, math.log(3.0)))                     # sigmoid(ln 3) = 3/4
    assert np.allclose(h, 0.75 * o, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- whole path
def _dense_causal_gated(q_abs, kv, pos, tau, gate):
    """Dense causal attention through torch SDPA with an explicit mask s <= p,
    then the sigmoid gate (torch.sigmoid)."""
    n = kv.shape[0]
    T = q_abs.shape[0]
    mask = torch.from_numpy(np.arange(n)[None, :] <= np.asarray(pos)[:, None])    # [T, n]
    Q = torch.from_numpy(q_abs).permute(1, 0, 2)[None]                             # [1,H,T,576]
    K = torch.from_numpy(kv)[None, None].expand(1, q_abs.shape[1], n, 576)
    V = torch.from_numpy(kv[:, :512])[None, None].expand(1, q_abs.shape[1], n, 512)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask[None, None], scale=tau)
    o = o[0].permute(1, 0, 2)                                                      # [T,H,512]
    return (o * torch.sigmoid(torch.from_numpy(gate))[..., None]).numpy()


def check_forward_dense_limit(orc):
    """With k at least the context, the whole path is dense causal attention
    (own row included) followed by the gate."""
    rng = np.random.default_rng(8)
    n = 40
    kv_bits = torch.from_numpy(rng.standard_normal((n, 576)).astype(np.float32) / 24).to(torch.bfloat16)
    kv = kv_bits.to(torch.float64).numpy()
    k_bits = torch.from_numpy(rng.integers(-3, 4, (n, 128)).astype(np.float32)).to(torch.bfloat16)
    pos = np.array([0, 1, 17, 39], dtype=np.int32)
    T = len(pos)
    q_idx = rng.integers(-3, 4, (T, 64, 128)).astype(float)
    w = rng.integers(0, 5, (T, 64)).astype(float)
    q_abs = rng.standard_normal((T, 64, 576))
    gate = rng.standard_normal((T, 64)) * 2
    tau = 1 / math.sqrt(192)
    ks = orc.Store(k_bits.view(torch.int16).numpy().view(np.uint16), "bf16")
    vs = orc.Store(kv_bits.view(torch.int16).numpy().view(np.uint16), "bf16")
    res = orc.forward(np.zeros(T, np.int32), pos, np.zeros(1, np.int64), np.array([n], np.int32),
                      q_idx, w, ks, q_abs, vs, gate, 64, tau)
    ref = _dense_causal_gated(q_abs, kv, pos, tau, gate)
    assert np.allclose(res["out"], ref, rtol=1e-11, atol=1e-14)
    for i, p in enumerate(pos):
        assert res["indices"][i].tolist() == list(range(p + 1)) + [-1] * (64 - p - 1)


def check_forward_selects_by_indexer(orc):
    """When k is smaller than the context, the kept rows are the top-k rows of the
    indexer score under the tie rule (rank definition), and the attention equals
    dense attention restricted to exactly those rows."""
    rng = np.random.default_rng(9)
    n = 30
    kv_bits = torch.from_numpy(rng.standard_normal((n, 576)).astype(np.float32) / 24).to(torch.bfloat16)
    kv = kv_bits.to(torch.float64).numpy()
    k_int = rng.integers(-1, 2, (n, 128))
    k_bits = torch.from_numpy(k_int.astype(np.float32)).to(torch.bfloat16)
    pos = np.array([29, 12], dtype=np.int32)
    q_idx = rng.integers(-1, 2, (2, 64, 128)).astype(float)
    w = rng.integers(0, 3, (2, 64)).astype(float)
    q_abs = rng.standard_normal((2, 64, 576))
    tau = 1 / math.sqrt(192)
    ks = orc.Store(k_bits.view(torch.int16).numpy().view(np.uint16), "bf16")
    vs = orc.Store(kv_bits.view(torch.int16).numpy().view(np.uint16), "bf16")
    k = 7
    res = orc.forward(np.zeros(2, np.int32), pos, np.zeros(1, np.int64), np.array([n], np.int32),
                      q_idx, w, ks, q_abs, vs, None, k, tau)
    for i, p in enumerate(pos):
        # exact integer scores over rows 0..p
        sc = []
        for s in range(p + 1):
            tot = 0
            for h in range(64):
                d = int(np.dot(k_int[s], q_idx[i, h].astype(int)))
                tot += int(w[i, h]) * max(d, 0)
            sc.append(tot)
        want = _rank_select(sc, k)
        assert res["indices"][i].tolist() == want
        kept = [s for s in want if s >= 0]
        Q = torch.from_numpy(q_abs[i])[None, :, None, :]
        K = torch.from_numpy(kv[kept])[None, None].expand(1, 64, len(kept), 576)
        V = torch.from_numpy(kv[kept, :512])[None, None].expand(1, 64, len(kept), 512)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=tau)[0, :, 0].numpy()
        assert np.allclose(res["out"][i], ref, rtol=1e-11, atol=1e-14)


def check_forward_fp8_store(orc):
    """An fp8 cache row is its decoded payload times its scale: the path over an
    fp8 store equals the path over the same values stored exactly in bf16
    (E4M3 values times powers of two are exact in bf16)."""
    rng = np.random.default_rng(10)
    n = 24
    codes = rng.integers(0, 256, (n, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                         # no NaN codes
    scale = np.ldexp(1.0, rng.integers(-3, 3, n)).astype(np.float32)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(scale)[:, None]
    vals_bits = vals.to(torch.bfloat16)
    assert torch.equal(vals_bits.to(torch.float32), vals)
    kcodes = torch.from_numpy(rng.integers(-3, 4, (n, 128)).astype(np.float32)).to(torch.float8_e4m3fn)
    kscale = np.ldexp(1.0, rng.integers(-2, 3, n)).astype(np.float32)
    kvals = (kcodes.to(torch.float32) * torch.from_numpy(kscale)[:, None]).to(torch.bfloat16)
    q_idx = rng.integers(-3, 4, (1, 64, 128)).astype(float)
    w = rng.integers(0, 5, (1, 64)).astype(float)
    q_abs = rng.standard_normal((1, 64, 576))
    tau = 1 / math.sqrt(192)
    args = (np.zeros(1, np.int32), np.array([n - 1], np.int32), np.zeros(1, np.int64), np.array([n], np.int32))
    a = orc.forward(*args, q_idx, w, orc.Store(kcodes.view(torch.uint8).numpy(), "e4m3fn", kscale), q_abs,
                    orc.Store(codes, "e4m3fn", scale), None, 5, tau)
    b = orc.forward(*args, q_idx, w, orc.Store(kvals.view(torch.int16).numpy().view(np.uint16), "bf16"), q_abs,
                    orc.Store(vals_bits.view(torch.int16).numpy().view(np.uint16), "bf16"), None, 5, tau)
    assert np.array_equal(a["indices"], b["indices"])
    assert np.allclose(a["out"], b["out"], rtol=1e-13, atol=1e-15)


def check_forward_mxfp8_store(orc):
    """An MX block-32 cache holds payload times block scale: the path over an MX
    store equals the path over the same values stored exactly in bf16."""
    rng = np.random.default_rng(11)
    n = 24
    codes = rng.integers(0, 256, (n, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    exps = rng.integers(120, 130, (n, 18)).astype(np.uint8)
    vals = (torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
            * torch.from_numpy(np.ldexp(1.0, exps.astype(int) - 127).astype(np.float32)).repeat_interleave(32, 1))
    vals_bits = vals.to(torch.bfloat16)
    assert torch.equal(vals_bits.to(torch.float32), vals)
    kcodes = rng.integers(-3, 4, (n, 128)).astype(np.float32)
    kexps = rng.integers(125, 130, (n, 4)).astype(np.uint8)
    kpay = torch.from_numpy(kcodes).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kvals = torch.from_numpy(kcodes * np.ldexp(1.0, kexps.astype(int) - 127).repeat(32, 1)).to(torch.bfloat16)
    q_idx = rng.integers(-3, 4, (1, 64, 128)).astype(float)
    w = rng.integers(0, 5, (1, 64)).astype(float)
    q_abs = rng.standard_normal((1, 64, 576))
    tau = 1 / math.sqrt(192)
    args = (np.zeros(1, np.int32), np.array([n - 1], np.int32), np.zeros(1, np.int64), np.array([n], np.int32))
    a = orc.forward(*args, q_idx, w, orc.Store(kpay, "mxfp8", kexps), q_abs,
                    orc.Store(codes, "mxfp8", exps), None, 5, tau)
    b = orc.forward(*args, q_idx, w, orc.Store(kvals.view(torch.int16).numpy().view(np.uint16), "bf16"), q_abs,
                    orc.Store(vals_bits.view(torch.int16).numpy().view(np.uint16), "bf16"), None, 5, tau)
    assert np.array_equal(a["indices"], b["indices"])
    assert np.allclose(a["out"], b["out"], rtol=1e-13, atol=1e-15)


def check_output_projection_unabsorbed(orc):
    """The absorbed path followed by the output epilogue equals MLA computed
    without absorbing W_UV: each head's values are the selected latent rows
    times its up-projection, attended with the same probabilities, then the
    heads are concatenated and projected. Also: gating before o_proj equals
    scaling each head's values before the projection."""
    rng = np.random.default_rng(12)
    H, n, dm = 64, 40, 96
    rows = rng.standard_normal((n, 576))
    q = rng.standard_normal((H, 576))
    g = rng.standard_normal(H) * 2
    tau = 1 / math.sqrt(192)
    w_uv = rng.standard_normal((H, 128, 512)) / 24
    w_o = rng.standard_normal((dm, H * 128)) / 90
    o, _ = orc.sparse_mla(q, rows, tau)
    y = orc.output_projection(orc.sigmoid_gate(o, g)[None], w_uv, w_o)[0]
    # unabsorbed: values per head, softmax written out, gate on the value vectors
    z = tau * (q @ rows.T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    vals = np.stack([p[h] @ (rows[:, :512] @ w_uv[h].T) for h in range(H)])     # [H, 128]
    vals *= (1 / (1 + np.exp(-g)))[:, None]
    ref = w_o @ vals.reshape(-1)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def check_output_projection_selection(orc):
    """Selection weights: W_UV[h] picks latent columns 128h' .. of head h, W_O
    picks one value column per output: the projection returns those entries."""
    rng = np.random.default_rng(13)
    T, H = 3, 64
    o = rng.standard_normal((T, H, 512))
    w_uv = np.zeros((H, 128, 512))
    for h in range(H):
        w_uv[h, np.arange(128), (np.arange(128) + 3 * h) % 512] = 1.0
    pick = rng.integers(0, H * 128, size=50)
    w_o = np.zeros((50, H * 128))
    w_o[np.arange(50), pick] = 2.0
    y = orc.output_projection(o, w_uv, w_o)
    hh, vv = pick // 128, pick % 128
    ref = 2.0 * o[:, hh, (vv + 3 * hh) % 512]
    assert np.array_equal(y, ref)


def check_indexer_loss_worked_example(orc):
    g = _golden("indexer_loss_worked_example.json")
    rows = np.zeros((2, 576))
    rows[:, 0] = g["rows_col0"]
    q = np.zeros((2, 576))
    q[:, 0] = g["q_col0"]
    got = orc.sparse_indexer_loss(q, rows, 1.0, np.array(g["scores"]))
    assert abs(got - g["loss"]) < 1e-14, got


def check_indexer_loss_properties(orc):
    """KL against torch's kl_div on the same distributions; zero when the
    indexer's softmax equals the target; invariant to a shift of the scores and
    to the order of the selected rows; non-negative."""
    rng = np.random.default_rng(15)
    H, m = 64, 300
    q = rng.standard_normal((H, 576))
    rows = rng.standard_normal((m, 576)) / 24
    sc = rng.standard_normal(m) * 3
    tau = 1 / math.sqrt(192)
    got = orc.sparse_indexer_loss(q, rows, tau, sc)
    zt = torch.from_numpy(tau * q @ rows.T)
    p = torch.softmax(zt, dim=1).mean(dim=0)
    ref = torch.nn.functional.kl_div(torch.log_softmax(torch.from_numpy(sc), 0), p, reduction="sum").item()
    assert abs(got - ref) < 1e-12 * max(1.0, abs(ref)) and got >= 0
    assert abs(orc.sparse_indexer_loss(q, rows, tau, np.log(p.numpy()) + 7.0)) < 1e-12
    assert abs(orc.sparse_indexer_loss(q, rows, tau, sc + 100.0) - got) < 1e-12
    perm = rng.permutation(m)
    assert abs(orc.sparse_indexer_loss(q, rows[perm], tau, sc[perm]) - got) < 1e-12


# ---------------------------------------------------------------- ragged batches
def _flat_batch(rng, lens, gap=3):
    """Sequences of the given lengths stored back to back in flat caches, with
    `gap` junk rows before each (large values, so a row read from the wrong
    place changes every result). Returns the flat bf16 latent rows (float64
    values and raw bits), integer indexer keys (int64 and raw bits) and
    seq_start."""
    starts, rows = [], 0
    for n in lens:
        rows += gap
        starts.append(rows)
        rows += n
    kv = rng.standard_normal((rows, 576)) / 24
    k_int = rng.integers(-2, 3, (rows, 128))
    for s0, n in zip(starts, lens):          # junk in the gaps
        kv[s0 - gap:s0] = 5.0 + rng.standard_normal((gap, 576))
        k_int[s0 - gap:s0] = 3
    kv_bits = torch.from_numpy(kv.astype(np.float32)).to(torch.bfloat16)
    k_bits = torch.from_numpy(k_int.astype(np.float32)).to(torch.bfloat16)
    return (kv_bits.to(torch.float64).numpy(), kv_bits.view(torch.int16).numpy().view(np.uint16),
            k_int, k_bits.view(torch.int16).numpy().view(np.uint16), np.array(starts, np.int64))


def _int_scores(k_int, q_int, w_int):
    """Exact integer indexer scores of integer keys [n, 128] for one token."""
    d = k_int.astype(np.int64) @ q_int.astype(np.int64).T            # [n, 64]
    return (np.where(d > 0, d, 0) * w_int.astype(np.int64)[None, :]).sum(axis=1)


def check_forward_multi_sequence(orc):
    """Three sequences at nonzero offsets of the flat caches: each token sees only
    rows seq_start[b] .. seq_start[b] + p. A token with k at least its visible
    count gets dense causal attention over its own sequence (torch SDPA); a
    token with fewer gets the rank-defined top-k of its exact integer scores
    and SDPA over exactly those rows."""
    rng = np.random.default_rng(16)
    lens = [9, 14, 6]
    kv, kv_bits, k_int, k_bits, starts = _flat_batch(rng, lens)
    token_seq = np.array([0, 1, 1, 2, 0], np.int32)
    token_pos = np.array([8, 13, 4, 5, 2], np.int32)
    T, k = len(token_seq), 5
    q_int = rng.integers(-2, 3, (T, 64, 128))
    w_int = rng.integers(0, 4, (T, 64))
    q_abs = rng.standard_normal((T, 64, 576))
    gate = rng.standard_normal((T, 64)) * 2
    tau = 1 / math.sqrt(192)
    ks = orc.Store(k_bits, "bf16")
    vs = orc.Store(kv_bits, "bf16")
    res = orc.forward(token_seq, token_pos, starts, np.array(lens, np.int32), q_int.astype(float),
                      w_int.astype(float), ks, q_abs, vs, gate, k, tau)
    for t in range(T):
        b, p = int(token_seq[t]), int(token_pos[t])
        rows = np.arange(starts[b], starts[b] + p + 1)
        want = _rank_select(list(_int_scores(k_int[rows], q_int[t], w_int[t])), k)
        assert res["indices"][t].tolist() == want, (t, res["indices"][t], want)
        kept = rows[[s for s in want if s >= 0]]
        if p + 1 <= k:
            assert len(kept) == p + 1
        Q = torch.from_numpy(q_abs[t])[None, :, None, :]
        K = torch.from_numpy(kv[kept])[None, None].expand(1, 64, len(kept), 576)
        V = torch.from_numpy(kv[kept, :512])[None, None].expand(1, 64, len(kept), 512)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=tau)[0, :, 0]
        ref = (o * torch.sigmoid(torch.from_numpy(gate[t]))[:, None]).numpy()
        assert np.allclose(res["out"][t], ref, rtol=1e-11, atol=1e-14), t
        z = torch.from_numpy(tau * (q_abs[t] @ kv[kept].T))
        assert np.allclose(res["lse"][t], torch.logsumexp(z, dim=1).numpy(), rtol=1e-13, atol=1e-13)


def check_indexer_loss_multi_sequence(orc):
    """The per-token wrapper of the loss over a ragged batch at nonzero offsets:
    one token keeping fewer rows than it sees, one keeping all of them (its
    index row is padded with -1, which must not count), one in an empty
    sequence (loss 0). Composed independently: exact integer scores, the rank
    definition of the top-k, each head's torch softmax over the kept rows,
    their mean, then torch's kl_div against the log-softmax of the scores."""
    rng = np.random.default_rng(17)
    lens = [12, 5, 0]
    kv, kv_bits, k_int, k_bits, starts = _flat_batch(rng, lens)
    token_seq = np.array([0, 1, 2, 0], np.int32)
    token_pos = np.array([11, 4, 0, 3], np.int32)
    T, k = len(token_seq), 6
    q_int = rng.integers(-2, 3, (T, 64, 128))
    w_int = rng.integers(0, 4, (T, 64))
    q_abs = rng.standard_normal((T, 64, 576)) * 3
    tau = 1 / math.sqrt(192)
    got = orc.indexer_loss(token_seq, token_pos, starts, np.array(lens, np.int32), q_int.astype(float),
                           w_int.astype(float), orc.Store(k_bits, "bf16"), q_abs,
                           orc.Store(kv_bits, "bf16"), k, tau)
    assert got.shape == (T,)
    for t in range(T):
        b, p = int(token_seq[t]), int(token_pos[t])
        n = min(p + 1, lens[b])
        if n == 0:
            assert got[t] == 0.0, (t, got[t])
            continue
        rows = np.arange(starts[b], starts[b] + n)
        sc = _int_scores(k_int[rows], q_int[t], w_int[t])
        sel = [s for s in _rank_select(list(sc), k) if s >= 0]
        z = torch.from_numpy(tau * (q_abs[t] @ kv[rows[sel]].T))                # [64, m]
        target = torch.softmax(z, dim=1).mean(dim=0)
        logq = torch.log_softmax(torch.from_numpy(sc[sel].astype(np.float64)), dim=0)
        ref = torch.nn.functional.kl_div(logq, target, reduction="sum").item()
        assert abs(got[t] - ref) < 1e-12 * max(1.0, abs(ref)), (t, got[t], ref)


ALL_CHECKS = [check_bf16_decode, check_e4m3fn_table, check_indexer_worked_example,
              check_indexer_exact_integer, check_topk_worked_example, check_topk_rank_definition,
              check_topk_enumeration, check_topk_special_cases, check_attention_closed_form,
              check_attention_vs_sdpa, check_attention_special_cases, check_gate,
              check_forward_dense_limit, check_forward_selects_by_indexer, check_forward_fp8_store,
              check_e4m3fn_encode, check_quantize_rows, check_cache_append, check_e8m0_table,
              check_mxfp8_worked_example, check_mxfp8_brute_force, check_mxfp8_scale_invariance,
              check_forward_mxfp8_store, check_output_projection_unabsorbed,
              check_output_projection_selection, check_e2m1_table, check_mxfp4_worked_example,
              check_mxfp4_brute_force, check_mxfp4_scale_invariance, check_forward_mxfp4_store,
              check_indexer_loss_worked_example, check_indexer_loss_properties,
              check_forward_multi_sequence, check_indexer_loss_multi_sequence]
