"""GPU parity for sga_cache_append: the bytes it writes into bf16, fp8 (one
scale per row) and MX block-32 caches, and their scales, against the oracle's
cache append, bit for bit; rows it must not touch keep their contents."""
import numpy as np
import pytest
import torch

import oracle
import sga_inputs as si
import sparse_gated_mla_amd as sga
from gpu_helpers import say

pytestmark = pytest.mark.gpu

SENT_BF16 = -0x5A5B          # int16 fill of untouched bf16 rows (0xA5A5)
SENT_FP8 = 0xA5              # byte fill of untouched fp8 rows
SENT_SCALE = -3.0            # fill of untouched fp32 row scales
SENT_MX = 0xA5               # fill of untouched E8M0 exponents


def _meta(lengths, tokens, starts=None):
    lengths = np.asarray(lengths, dtype=np.int32)
    if starts is None:
        starts = np.zeros(len(lengths), dtype=np.int64)
        starts[1:] = np.cumsum(lengths.astype(np.int64))[:-1]
    seq = np.asarray([t[0] for t in tokens], dtype=np.int32)
    pos = np.asarray([t[1] for t in tokens], dtype=np.int32)
    return seq, pos, np.asarray(starts, dtype=np.int64), lengths


def _cache(rows, width, fmt):
    if fmt == "bf16":
        return torch.full((rows, width), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16), None
    if fmt == "mx4":
        return (torch.full((rows, width // 2), SENT_FP8, dtype=torch.uint8, device="cuda"),
                torch.full((rows, width // 32), SENT_MX, dtype=torch.uint8, device="cuda"))
    data = torch.full((rows, width), SENT_FP8, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    if fmt == "mx":
        return data, torch.full((rows, width // 32), SENT_MX, dtype=torch.uint8, device="cuda")
    return data, torch.full((rows,), SENT_SCALE, dtype=torch.float32, device="cuda")


def _bits(t, rows=None):
    if rows is not None:
        t = t[torch.as_tensor(rows, dtype=torch.int64, device=t.device)]
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.uint8).cpu().numpy()


def _check_cache(data, scale, fmt, expect, rows_to_check=None):
    """expect: {row: (payload, scale|None)} from the oracle. Every row in
    rows_to_check (all rows by default) either holds the oracle's bytes or the fill."""
    rows = list(range(data.shape[0])) if rows_to_check is None else list(rows_to_check)
    bits = _bits(data, None if rows_to_check is None else rows)
    sc = None if scale is None else scale.cpu().numpy()
    if fmt in ("mx", "mx4"):
        for i, r in enumerate(rows):
            if r in expect:
                pay, ex = expect[r]
                assert np.array_equal(bits[i], pay), f"row {r}: payload differs"
                assert np.array_equal(sc[r], ex), f"row {r}: exponents {sc[r]} != {ex}"
            else:
                assert np.all(bits[i] == SENT_FP8) and np.all(sc[r] == SENT_MX), f"row {r} was written"
        return
    fill = np.uint16(0xA5A5) if fmt == "bf16" else np.uint8(SENT_FP8)
    for i, r in enumerate(rows):
        if r in expect:
            pay, s = expect[r]
            assert np.array_equal(bits[i], pay), f"row {r}: payload differs"
            if fmt != "bf16":
                assert np.float32(sc[r]).view(np.uint32) == np.float32(s).view(np.uint32), \
                    f"row {r}: scale {sc[r]!r} != {s!r}"
        else:
            assert np.all(bits[i] == fill), f"row {r} was written"
            if sc is not None:
                assert sc[r] == SENT_SCALE, f"row {r}: scale was written"


def _append(meta, cache_rows, latent, key, kv_fmt, key_fmt, max_len=None):
    seq, pos, starts, lens = meta
    batch = sga.batch_to_device(seq, pos, starts, lens, cache_rows,
                                max_len=max_len or max(1, int(lens.max())))
    kv, kv_s = _cache(cache_rows, 576, kv_fmt) if kv_fmt else (None, None)
    kidx, kidx_s = _cache(cache_rows, 128, key_fmt) if key_fmt else (None, None)
    sga.sga_cache_append(batch, latent.cuda() if kv_fmt else None, key.cuda() if key_fmt else None,
                         kv, kv_s, kidx, kidx_s)
    torch.cuda.synchronize()
    return (kv, kv_s), (kidx, kidx_s)


def _oracle(meta, cache_rows, rows, fmt):
    seq, pos, starts, lens = meta
    bits = rows.view(torch.int16).numpy().view(np.uint16)
    name = {"bf16": "bf16", "fp8": "e4m3fn", "mx": "mxfp8", "mx4": "mxfp4"}[fmt]
    return oracle.cache_append(seq, pos, starts, lens, cache_rows, bits, name)


def _run_and_check(meta, cache_rows, latent, key, kv_fmt, key_fmt, rows_to_check=None, what=""):
    say(f"[cache_append] {what}: T={len(meta[0])} rows={cache_rows} kv={kv_fmt} key={key_fmt}")
    (kv, kv_s), (kidx, kidx_s) = _append(meta, cache_rows, latent, key, kv_fmt, key_fmt)
    if kv_fmt:
        _check_cache(kv, kv_s, kv_fmt, _oracle(meta, cache_rows, latent, kv_fmt), rows_to_check)
    if key_fmt:
        _check_cache(kidx, kidx_s, key_fmt, _oracle(meta, cache_rows, key, key_fmt), rows_to_check)


@pytest.mark.parametrize("kv_fmt,key_fmt", [("bf16", "bf16"), ("fp8", "fp8"), ("bf16", "fp8"),
                                            ("fp8", "bf16"), ("fp8", None), (None, "fp8"),
                                            ("mx", "mx"), ("mx", "fp8"), ("bf16", "mx"),
                                            ("mx4", "mx4"), ("mx4", "bf16"), ("fp8", "mx4")])
def test_ragged_batch(kv_fmt, key_fmt):
    lens = [37, 300, 5, 1000]
    toks = [(0, 0), (0, 36), (1, 299), (1, 150), (1, 0), (2, 4), (3, 999), (3, 998), (3, 500), (0, 17)]
    meta = _meta(lens, toks)
    lat, key = si.append_rows(len(toks), seed=11)
    _run_and_check(meta, sum(lens) + 7, lat, key, kv_fmt, key_fmt, what="ragged")


def test_out_of_range_tokens_write_nothing():
    lens = [10, 20, 30]
    starts = [0, 10, 45]                          # the last sequence overruns a 60-row cache
    toks = [(0, 9), (-1, 3), (3, 0), (1, -1), (1, 20), (1, 19), (2, 14), (2, 15), (2, 29), (0, 0)]
    meta = _meta(lens, toks, starts)
    lat, key = si.append_rows(len(toks), seed=12)
    for fmt in ("bf16", "fp8", "mx", "mx4"):
        expect = _oracle(meta, 60, lat, fmt)
        assert sorted(expect) == [0, 9, 29, 59], sorted(expect)      # the oracle's skip rules
        _run_and_check(meta, 60, lat, key, fmt, fmt, what=f"skips {fmt}")


def _edge_rows():
    """Hand-picked bf16 rows: zero rows, -0, exact E4M3FN ties at scale 1,
    subnormal codes and ties, underflow, huge and tiny magnitudes, bf16 subnormals."""
    rows = []
    z = np.zeros(576, np.float32)
    rows.append(z.copy())                                             # scale 1, all codes 0
    rows.append(-z)                                                   # all -0: code 0x80
    r = z.copy(); r[0] = 448.0                                        # amax 448: scale exactly 1
    ties = [1.0625, 1.1875, 2.125, 2.375, 0.5 * (2.0 ** -9), 1.5 * (2.0 ** -9), 2.5 * (2.0 ** -9),
            7.5 * (2.0 ** -9), 15.5 * (2.0 ** -9), 2.0 ** -20, 240.0 + 8.0, 416.0 + 16.0, 3.0, 0.09375]
    r[1:1 + len(ties)] = ties
    r[20:20 + len(ties)] = -np.asarray(ties, np.float32)
    rows.append(r)
    r = z.copy(); r[5] = -448.0; r[6:40] = np.arange(34, dtype=np.float32) * 0.125   # negative amax
    rows.append(r)
    r = np.full(576, 3.0e38, np.float32); r[1::3] = 1e-30; r[2::3] = -2.5e37      # near bf16 max
    rows.append(r)
    r = np.full(576, 1.0e-39, np.float32); r[::5] = -3.0e-39                      # bf16 subnormals
    rows.append(r)
    r = np.full(576, 0.7, np.float32)                                            # all equal
    rows.append(r)
    r = z.copy(); r[300] = 1e-5                                                  # single nonzero
    rows.append(r)
    x = np.stack(rows)
    return torch.from_numpy(x).to(torch.bfloat16)


def test_edge_values():
    lat = _edge_rows()
    key = lat[:, :128].contiguous()
    T = lat.shape[0]
    meta = _meta([T], [(0, p) for p in range(T)])
    for fmt in ("bf16", "fp8", "mx", "mx4"):
        _run_and_check(meta, T, lat, key, fmt, fmt, what=f"edge {fmt}")


def test_prefill_chunk():
    # one sequence of 8192 rows; the second half is appended at once
    meta = _meta([8192], [(0, p) for p in range(4096, 8192)])
    lat, key = si.append_rows(4096, seed=13)
    _run_and_check(meta, 8192, lat, key, "fp8", "fp8", what="prefill fp8")
    _run_and_check(meta, 8192, lat, key, "bf16", "bf16", what="prefill bf16")
    _run_and_check(meta, 8192, lat, key, "mx", "mx", what="prefill mx")
    _run_and_check(meta, 8192, lat, key, "mx4", "mx4", what="prefill mx4")


@pytest.mark.parametrize("cfg", [2, 4, 5, 6])
def test_full_size_decode(cfg):
    # the long-context decode shapes: 16 x 131072 bf16, 8 x 262144 fp8 or MX; one new row per sequence
    B, S, fmt = {2: (16, 131072, "bf16"), 4: (8, 262144, "fp8"), 5: (8, 262144, "mx"), 6: (8, 262144, "mx4")}[cfg]
    meta = _meta([S] * B, [(b, S - 1) for b in range(B)])
    lat, key = si.append_rows(B, seed=20 + cfg)
    rows = B * S
    check = sorted({r for b in range(B) for r in (b * S, b * S + S - 2, b * S + S - 1)})
    _run_and_check(meta, rows, lat, key, fmt, fmt, rows_to_check=check, what=f"full size {fmt}")


def test_appended_fp8_rows_decode_close_to_inputs():
    # payload x scale is within half an E4M3FN step of x: the step at scaled
    # value q is 2^(floor(log2 q) - 3) for normals, 2^-9 below 2^-6
    lat, key = si.append_rows(64, seed=14)
    meta = _meta([64], [(0, p) for p in range(64)])
    (kv, kv_s), _ = _append(meta, 64, lat, key, "fp8", None)
    s = kv_s.cpu().numpy().astype(np.float64)[:, None]
    got = kv.float().cpu().numpy().astype(np.float64) * s
    x = lat.float().numpy().astype(np.float64)
    q = np.abs(x) / s
    half = 0.5 * np.maximum(q * 2.0 ** -3, 2.0 ** -9) * s
    assert np.all(np.abs(got - x) <= half * (1 + 1e-5))


def test_mx_edge_blocks():
    # blocks whose maximum sits just below, at and above 448 * 2^k, blocks of
    # bf16 subnormals, a block with one huge value, alternating signs, -0
    rng = np.random.default_rng(15)
    x = rng.normal(size=(6, 576)).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 0] = 448.0 * 2.0 ** -5                      # scale 2^-5 exactly, payload 448
    x[0, 32:64] = 15.5                               # saturates: 496 * 2^-5 clamps to 448
    x[0, 64:96] = -0.0
    x[1, :32] = 1.0e-39                              # bf16 subnormals: exponent clamps at 0
    x[1, 32:64] = 3.0e38                             # near the top of bf16
    x[1, 64] = -3.0e38
    x[2, ::2] *= -1.0
    x[3, 100] = 1e20                                 # one block dominated by one value
    lat = torch.from_numpy(x).to(torch.bfloat16)
    key = lat[:, :128].contiguous()
    T = lat.shape[0]
    meta = _meta([T], [(0, p) for p in range(T)])
    _run_and_check(meta, T, lat, key, "mx", "mx", what="mx edge blocks")
    _run_and_check(meta, T, lat, key, "mx4", "mx4", what="mx4 edge blocks")
