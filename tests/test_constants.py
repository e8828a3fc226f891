"""Constants the A.X K2 pages fix, and the workload constants derived from them."""
import math

import sga_inputs as si


def test_attention_shape_constants():
    # fact sheet: 64 query heads; QK dim 192 (128 NoPE + 64 RoPE); V dim 128;
    # latent 512; shared RoPE key 64; query projection width 64 x 192
    assert si.N_HEADS == 64
    assert si.D_LATENT == 512 and si.D_ROPE == 64 and si.D_QK == 576
    assert 128 + 64 == 192 and 64 * 192 == 12288
    assert math.isclose(si.SM_SCALE, 0.0721687836, rel_tol=1e-9)


def test_indexer_constants():
    # fact sheet: 64 indexer heads of width 128, 128-wide cached key, top-2048
    assert si.IDX_HEADS == 64 and si.IDX_DIM == 128 and si.TOP_K == 2048


def test_cache_payload_constants():
    # fact sheet KV figures: 704 elements per token per layer, 61 layers, bf16
    per_layer = si.D_LATENT + si.D_ROPE + si.IDX_DIM
    assert per_layer == 704
    assert 61 * per_layer * 2 == 85888
    assert 85888 * 131072 == 11257511936


def test_sparsity_fractions():
    # news article: about 1.6 % of a 128K context and about 0.8 % of 256K
    assert round(100 * 2048 / 131072, 1) == 1.6
    assert round(100 * 2048 / 262144, 1) == 0.8
