"""Plant plausible mistakes in copies of the oracle (CPU only) and check that the
pins catch every one of them."""
import types

import numpy as np
import pytest

import oracle
import oracle_pins
from oracle import sga_oracle as base


def _clone(**overrides):
    m = types.ModuleType("mutant")
    for name in dir(base):
        setattr(m, name, getattr(base, name))
    for k, v in overrides.items():
        setattr(m, k, v)
    # forward must call the mutated pieces
    def forward(*a, **kw):
        saved = {k: getattr(base, k) for k in overrides}
        try:
            for k, v in overrides.items():
                setattr(base, k, v)
            return base.forward(*a, **kw)
        finally:
            for k, v in saved.items():
                setattr(base, k, v)
    m.forward = forward
    return m


def _relu_after_weight(q, w, keys):
    return np.maximum((keys @ q.T) @ w, 0.0)


def _weight_then_relu(q, w, keys):
    return np.maximum((keys @ q.T) * w[None, :], 0.0).sum(axis=1)


def _ties_high_index(scores, k):
    n = scores.shape[0]
    order = np.lexsort((-np.arange(n), -scores))
    kept = np.sort(order[:min(k, n)])
    out = np.full(k, -1, np.int32)
    out[:kept.shape[0]] = kept
    return out


def _unsorted_output(scores, k):
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))[:min(k, n)]
    out = np.full(k, -1, np.int32)
    out[:order.shape[0]] = order
    return out


def _values_from_tail(q, rows, s, d_v=512):
    z = s * (q @ rows.T)
    e = np.exp(z - z.max(1, keepdims=True))
    return (e @ rows[:, 64:]) / e.sum(1, keepdims=True), z.max(1) + np.log(np.exp(z - z.max(1, keepdims=True)).sum(1))


def _logits_latent_only(q, rows, s, d_v=512):
    z = s * (q[:, :512] @ rows[:, :512].T)
    zm = z.max(1)
    e = np.exp(z - zm[:, None])
    return (e @ rows[:, :512]) / e.sum(1)[:, None], zm + np.log(e.sum(1))


_ORIG_MLA = base.sparse_mla


def _lse_log2(q, rows, s, d_v=512):
    o, lse = _ORIG_MLA(q, rows, s, d_v)
    return o, lse / np.log(2.0)


def _gate_sign(o, g):
    return o * (1.0 / (1.0 + np.exp(np.asarray(g, float))))[:, None]


def _bad_e4m3_table():
    t = base.e4m3fn_table().copy()
    t[1:8] = t[1:8] * 2          # subnormals with the wrong exponent
    return t


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    vals = base.e4m3fn_table()[:0x7F]
    a = np.minimum(np.abs(x), 448.0)
    code = np.array([int(np.argmin(np.abs(vals - v) - 1e-12 * vals)) for v in a], np.uint8)
    return code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0)).astype(np.uint8)


def _quantize_scale_240(x):
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(240.0), np.float32(1.0)).astype(np.float32)
    return base.encode_e4m3fn((x / scale[:, None]).astype(np.float32)), scale


def _append_row_plus_one(token_seq, token_pos, seq_start, seq_len, cache_rows, rows, fmt):
    got = _ORIG_APPEND(token_seq, token_pos, seq_start, seq_len, cache_rows, rows, fmt)
    return {r + 1: v for r, v in got.items()}


_ORIG_APPEND = base.cache_append


def _mx_quantize(x, shift=8, block=32, ceil=False):
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    blocks = x.reshape(n, d // block, block)
    amax = np.max(np.abs(blocks), axis=2)
    exps = np.zeros(amax.shape, dtype=np.uint8)
    nz = amax > 0
    lg = np.ceil(np.log2(amax[nz])) if ceil else np.floor(np.log2(amax[nz]))
    exps[nz] = np.clip(lg - shift, -127, 127) + 127
    scale = np.ldexp(1.0, exps.astype(int) - 127)
    pay = base.encode_e4m3fn(blocks / scale[:, :, None]).reshape(n, d)
    if block != 32:          # report one exponent per 32 as the format stores
        exps = exps[:, ::32 // block]
    return pay, exps


def _mx_decode_bias_128(payload, exps):
    p = np.asarray(payload, dtype=np.uint8)
    n, d = p.shape
    vals = base.e4m3fn_table()[p].reshape(n, d // 32, 32)
    return (vals * np.ldexp(1.0, np.asarray(exps, int) - 128)[:, :, None]).reshape(n, d)


def _proj_transposed_uv(o, w_uv, w_o):
    # the up-projection taken as (input x output): columns instead of rows
    o = np.asarray(o, dtype=np.float64)
    T, H, _ = o.shape
    u = np.stack([o[:, h, :128] @ np.asarray(w_uv[h])[:, :128] for h in range(H)], axis=1)
    return u.reshape(T, -1) @ np.asarray(w_o).T


def _proj_value_major(o, w_uv, w_o):
    # heads concatenated value-major (v * 64 + h) instead of head-major
    o = np.asarray(o, dtype=np.float64)
    T, H, _ = o.shape
    u = np.stack([o[:, h, :] @ np.asarray(w_uv[h]).T for h in range(H)], axis=2)   # [T, 128, H]
    return u.reshape(T, -1) @ np.asarray(w_o).T


def _mx4_nibbles_swapped(x):
    pay, ex = _ORIG_MX4(x)
    return ((pay >> 4) | ((pay & 0xF) << 4)).astype(np.uint8), ex


def _mx4_exponent_like_fp8(x):
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    blocks = x.reshape(n, d // 32, 32)
    amax = np.max(np.abs(blocks), axis=2)
    exps = np.zeros(amax.shape, dtype=np.uint8)
    nz = amax > 0
    exps[nz] = np.clip(np.floor(np.log2(amax[nz])) - 8, -127, 127) + 127
    codes = base.encode_e2m1(blocks / np.ldexp(1.0, exps.astype(int) - 127)[:, :, None]).reshape(n, d)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), exps


_ORIG_MX4 = base.quantize_blocks_mxfp4


def _loss_reversed_kl(q_abs, rows, sm_scale, scores_sel):
    # KL(q || p) instead of KL(p || q)
    z = sm_scale * (np.asarray(q_abs, float) @ np.asarray(rows, float).T)
    ph = np.exp(z - z.max(axis=1, keepdims=True))
    p = (ph / ph.sum(axis=1, keepdims=True)).mean(axis=0)
    i = np.asarray(scores_sel, float)
    qd = np.exp(i - i.max())
    qd /= qd.sum()
    return float(np.sum(qd * (np.log(qd) - np.log(p))))


def _loss_pooled_logits(q_abs, rows, sm_scale, scores_sel):
    # one softmax of the head-mean logits instead of the mean of per-head softmaxes
    z = (sm_scale * (np.asarray(q_abs, float) @ np.asarray(rows, float).T)).mean(axis=0)
    p = np.exp(z - z.max())
    p /= p.sum()
    i = np.asarray(scores_sel, float)
    log_q = i - (i.max() + np.log(np.exp(i - i.max()).sum()))
    return float(np.sum(p * (np.log(p) - log_q)))


def _forward_base_dropped(token_seq, token_pos, seq_start, seq_len, q_idx, w, k_store, q_abs,
                          kv_store, gate, k, sm_scale, tokens=None, keep_scores=False):
    # every sequence addressed as if it started at flat row 0
    return _ORIG_FORWARD(token_seq, token_pos, np.zeros_like(np.asarray(seq_start)), seq_len, q_idx,
                         w, k_store, q_abs, kv_store, gate, k, sm_scale, tokens=tokens,
                         keep_scores=keep_scores)


_ORIG_FORWARD = base.forward


def _loss_keeps_padding(token_seq, token_pos, seq_start, seq_len, q_idx, w, k_store, q_abs,
                        kv_store, k, sm_scale, tokens=None):
    # the -1 padding of a short selection is not dropped (it reads the row
    # before the sequence and the last score)
    sel = range(len(token_seq)) if tokens is None else tokens
    out = []
    for t in sel:
        b, p = int(token_seq[t]), int(token_pos[t])
        n = min(p + 1, int(seq_len[b]))
        b0 = int(seq_start[b])
        scores = base.index_scores(q_idx[t], w[t], k_store.rows(np.arange(b0, b0 + n)))
        idx = base.select_topk(scores, k)
        if n == 0:
            out.append(0.0)
            continue
        out.append(base.sparse_indexer_loss(q_abs[t], kv_store.rows(b0 + idx), sm_scale, scores[idx]))
    return np.asarray(out, dtype=np.float64)


def _loss_visible_off_by_one(token_seq, token_pos, seq_start, seq_len, q_idx, w, k_store, q_abs,
                             kv_store, k, sm_scale, tokens=None):
    # the token's own row left out of the visible rows
    return _ORIG_LOSS(token_seq, np.maximum(np.asarray(token_pos) - 1, 0), seq_start, seq_len, q_idx,
                      w, k_store, q_abs, kv_store, k, sm_scale, tokens=tokens)


_ORIG_LOSS = base.indexer_loss

MUTANTS = {
    "relu_after_weighting": dict(index_scores=_relu_after_weight),
    "weight_inside_relu": dict(index_scores=_weight_then_relu),
    "ties_to_high_index": dict(select_topk=_ties_high_index),
    "indices_not_ascending": dict(select_topk=_unsorted_output),
    "values_from_wrong_columns": dict(sparse_mla=_values_from_tail),
    "rope_dropped_from_logits": dict(sparse_mla=_logits_latent_only),
    "lse_in_base_2": dict(sparse_mla=_lse_log2),
    "gate_sign_flipped": dict(sigmoid_gate=_gate_sign),
    "e4m3_subnormals": dict(e4m3fn_table=_bad_e4m3_table),
    "e4m3_encode_ties_away": dict(encode_e4m3fn=_encode_ties_away),
    "quantize_scale_240": dict(quantize_rows_e4m3fn=_quantize_scale_240),
    "append_row_off_by_one": dict(cache_append=_append_row_plus_one),
    "mx_exponent_off_by_one": dict(quantize_blocks_mxfp8=lambda x: _mx_quantize(x, shift=7)),
    "mx_exponent_from_ceil": dict(quantize_blocks_mxfp8=lambda x: _mx_quantize(x, ceil=True)),
    "mx_blocks_of_16": dict(quantize_blocks_mxfp8=lambda x: _mx_quantize(x, block=16)),
    "mx_decode_bias_128": dict(decode_mxfp8=_mx_decode_bias_128),
    "proj_uv_transposed": dict(output_projection=_proj_transposed_uv),
    "proj_heads_value_major": dict(output_projection=_proj_value_major),
    "mx4_nibbles_swapped": dict(quantize_blocks_mxfp4=_mx4_nibbles_swapped),
    "mx4_exponent_offset_8": dict(quantize_blocks_mxfp4=_mx4_exponent_like_fp8),
    "loss_reversed_kl": dict(sparse_indexer_loss=_loss_reversed_kl),
    "loss_pooled_logits": dict(sparse_indexer_loss=_loss_pooled_logits),
    "forward_seq_start_dropped": dict(forward=_forward_base_dropped),
    "loss_padding_kept": dict(indexer_loss=_loss_keeps_padding),
    "loss_visible_off_by_one": dict(indexer_loss=_loss_visible_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mutant = _clone(**MUTANTS[name])
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_real_oracle_passes_all_pins():
    for check in oracle_pins.ALL_CHECKS:
        check(oracle)


@pytest.mark.parametrize("name,pin", [("forward_seq_start_dropped", "check_forward_multi_sequence"),
                                      ("loss_padding_kept", "check_indexer_loss_multi_sequence"),
                                      ("loss_visible_off_by_one", "check_indexer_loss_multi_sequence")])
def test_multi_sequence_pins_catch(name, pin):
    mutant = _clone(**MUTANTS[name])
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            caught.append(check.__name__)
    assert pin in caught, (name, caught)
