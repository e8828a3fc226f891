"""The C ABI without a GPU: the library loads, exports every function that
include/sga.h declares, and rejects bad arguments on the host before any launch."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sga.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_gated_mla_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_gated_mla_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"SGA_API\s+[\w\s\*]+?\b(sga_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sga_index_scores", "sga_topk", "sga_sparse_mla_attn", "sga_forward", "sga_cache_append",
              "sga_output_proj", "sga_indexer_loss"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from sparse_gated_mla_amd import _lib
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    from sparse_gated_mla_amd import _lib
    assert lib.sga_version() >= 100
    for s in range(5):
        assert _lib.status_string(s).startswith(["SGA_OK", "SGA_ERR_INVALID_ARG", "SGA_ERR_UNSUPPORTED",
                                                  "SGA_ERR_WORKSPACE", "SGA_ERR_HIP"][s])
    assert _lib.status_string(99) == "unknown sga_status"


def _batch(T=2, B=1, max_len=100, rows=100, ptr=0x1000):
    from sparse_gated_mla_amd._lib import SgaBatch
    p = ptr if ptr else None
    return SgaBatch(T, B, max_len, 0, rows, p, p, p, p)


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails its host checks
FAKE_ODD = ctypes.c_void_p(0x10004)  # not 16-byte aligned


def test_index_scores_rejects_bad_arguments(lib):
    b = _batch()
    call = lambda bb, q=FAKE, w=FAKE, k=FAKE, ks=None, dt=0, s=FAKE, ld=100: lib.sga_index_scores(
        ctypes.byref(bb), q, w, k, ks, dt, s, ld, None)
    assert call(b, q=None) == 1
    assert call(b, w=None) == 1
    assert call(b, k=None) == 1
    assert call(b, s=None) == 1
    assert call(b, q=FAKE_ODD) == 1
    assert call(b, w=FAKE_ODD) == 1            # head weights are read as 16-byte vectors
    assert call(b, ld=99) == 1                 # ld < max_len
    assert call(b, ks=FAKE, dt=0) == 1         # bf16 keys take no scale
    assert call(b, ks=None, dt=1) == 1         # fp8 keys need scales
    assert call(b, dt=7) == 2                  # unknown dtype
    assert call(b, ks=None, dt=2) == 1         # MX keys need exponents
    assert call(b, ks=ctypes.c_void_p(0x10002), dt=2) == 1   # read as 32-bit words: 4-byte aligned
    assert call(_batch(T=-1)) == 1
    assert call(_batch(B=0)) == 1
    assert call(_batch(max_len=(1 << 19) + 1)) == 2
    assert call(_batch(ptr=0)) == 1            # null metadata
    bad = _batch()
    bad.reserved = 3
    assert call(bad) == 1
    assert call(_batch(T=0, ptr=0), q=None, w=None, k=None, s=None) == 0   # empty batch: no-op


def test_topk_rejects_bad_arguments(lib):
    b = _batch()
    call = lambda bb, s=FAKE, ld=100, k=8, idx=FAKE, ws=FAKE, nb=1 << 30: lib.sga_topk(
        ctypes.byref(bb), s, ld, k, idx, ws, nb, None)
    assert call(b, k=0) == 1
    assert call(b, k=(1 << 16) + 1) == 2
    assert call(b, s=None) == 1
    assert call(b, idx=None) == 1
    assert call(b, ld=50) == 1
    assert call(b, ws=None) == 3
    assert call(b, nb=lib.sga_topk_workspace_size(2, 100, 8) - 1) == 3


def test_attention_rejects_bad_arguments(lib):
    b = _batch()
    call = lambda bb, q=FAKE, kv=FAKE, sc=None, dt=0, idx=FAKE, k=8, tau=0.07, out=FAKE: \
        lib.sga_sparse_mla_attn(ctypes.byref(bb), q, kv, sc, dt, idx, k, tau, None, out, None,
                                FAKE, 1 << 30, None)
    assert call(b, tau=math.inf) == 1
    assert call(b, tau=math.nan) == 1
    assert call(b, k=0) == 1
    assert call(b, q=None) == 1
    assert call(b, idx=None) == 1
    assert call(b, out=None) == 1
    assert call(b, out=FAKE_ODD) == 1
    assert call(b, kv=FAKE_ODD) == 1
    assert call(b, dt=1) == 1                  # fp8 without scales
    assert call(b, dt=2) == 1                  # MX without exponents
    assert call(b, dt=3) == 1
    assert call(b, dt=4) == 2


def test_forward_rejects_bad_arguments(lib):
    b = _batch()
    need = lib.sga_forward_workspace_size(2, 100, 8)
    assert need > 0

    def call(ws=FAKE, nb=need, tau=0.07, k=8, kscale=None, kdt=0, w=FAKE, q=FAKE):
        return lib.sga_forward(ctypes.byref(b), q, w, FAKE, kscale, kdt, FAKE, FAKE, None, 0,
                               k, tau, None, FAKE, None, None, ws, nb, None, None)
    assert call(w=FAKE_ODD) == 1
    assert call(q=FAKE_ODD) == 1
    assert call(ws=None) == 3
    assert call(nb=need - 1) == 3
    assert call(tau=math.inf) == 1
    assert call(k=0) == 1
    assert call(kdt=1) == 1


def test_forward_noalloc_rejects_oversize_before_touching_the_device(lib):
    # the scratch limit is checked on the host first: these calls return without
    # any HIP call, so they run without a GPU
    limit = lib.sga_forward_noalloc_scratch_bytes()
    assert limit == 64 << 20

    def call(bb, k=2048):
        return lib.sga_forward_noalloc(ctypes.byref(bb), FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None,
                                       0, k, 0.07, None, FAKE, None, None, None, None)
    big = _batch(T=64, max_len=1 << 19, rows=1 << 19)
    assert lib.sga_forward_workspace_size(64, 1 << 19, 2048) > limit
    assert call(big) == 3                      # needs more scratch than the library holds
    assert call(_batch(), k=0) == 1
    assert call(_batch(), k=(1 << 16) + 1) == 2
    assert call(_batch(T=-1)) == 1
    assert call(_batch(T=0, ptr=0)) == 0       # empty batch: nothing to do


def test_cache_append_rejects_bad_arguments(lib):
    b = _batch()

    def call(bb=b, lat=FAKE, kv=FAKE, kvs=None, kvdt=0, key=FAKE, kidx=FAKE, ks=None, kdt=0):
        return lib.sga_cache_append(ctypes.byref(bb), lat, key, kv, kvs, kvdt, kidx, ks, kdt, None)
    assert call(lat=None) == 1                 # half a pair
    assert call(kv=None) == 1
    assert call(key=None) == 1
    assert call(kidx=None) == 1
    assert call(lat=FAKE_ODD) == 1
    assert call(key=FAKE_ODD) == 1
    assert call(kv=FAKE_ODD) == 1
    assert call(kidx=FAKE_ODD) == 1
    assert call(kvdt=1) == 1                   # fp8 cache without scales
    assert call(kdt=1) == 1
    assert call(kvs=FAKE) == 1                 # bf16 cache with scales
    assert call(kvdt=1, kvs=ctypes.c_void_p(0x10002)) == 1   # misaligned scales
    assert call(kvdt=5) == 2
    assert call(kvdt=2) == 1                   # MX cache without exponents
    assert call(kdt=2) == 1
    assert call(_batch(T=-1)) == 1
    assert call(_batch(ptr=0)) == 1
    assert call(_batch(max_len=(1 << 19) + 1)) == 2
    assert call(_batch(T=0, ptr=0), lat=None, kv=None, key=None, kidx=None) == 0
    assert call(_batch(T=0, ptr=0)) == 0       # empty batch: nothing launched
    assert call(lat=None, kv=None, key=None, kidx=None) == 0   # nothing to write


def test_output_proj_rejects_bad_arguments(lib):
    need = lib.sga_output_proj_workspace_size(2, 256)
    assert need > 0

    def call(T=2, o=FAKE, uv=FAKE, wo=FAKE, dm=256, y=FAKE, ws=FAKE, nb=need):
        return lib.sga_output_proj(T, o, uv, wo, dm, y, ws, nb, None)
    assert call(T=-1) == 1
    assert call(dm=0) == 1
    assert call(dm=100) == 2                   # not a multiple of 64
    assert call(dm=(1 << 16) + 64) == 2
    assert call(T=65536) == 2
    assert call(o=None) == 1
    assert call(uv=None) == 1
    assert call(wo=None) == 1
    assert call(y=None) == 1
    assert call(o=FAKE_ODD) == 1
    assert call(wo=FAKE_ODD) == 1
    assert call(ws=None) == 3
    assert call(nb=need - 1) == 3
    assert call(T=0, o=None, uv=None, wo=None, y=None, ws=None, nb=0) == 0
    assert lib.sga_output_proj_workspace_size(16, 7168) >= 16 * 8192 * 4
    assert lib.sga_output_proj_workspace_size(0, 7168) == 0


def test_indexer_loss_rejects_bad_arguments(lib):
    b = _batch()
    need = lib.sga_indexer_loss_workspace_size(2, 8)
    assert need >= 2 * 8 * 4

    def call(bb=b, q=FAKE, kv=FAKE, sc=None, dt=0, idx=FAKE, k=8, tau=0.07, lse=FAKE, s=FAKE,
             ld=100, loss=FAKE, ws=FAKE, nb=need):
        return lib.sga_indexer_loss(ctypes.byref(bb), q, kv, sc, dt, idx, k, tau, lse, s, ld, loss,
                                    ws, nb, None)
    assert call(k=0) == 1
    assert call(k=(1 << 16) + 1) == 2
    assert call(tau=math.nan) == 1
    assert call(q=None) == 1
    assert call(q=FAKE_ODD) == 1
    assert call(idx=None) == 1
    assert call(lse=None) == 1
    assert call(s=None) == 1
    assert call(loss=None) == 1
    assert call(ld=50) == 1
    assert call(dt=1) == 1                     # fp8 without scales
    assert call(dt=9) == 2
    assert call(ws=None) == 3
    assert call(nb=need - 1) == 3
    assert call(bb=_batch(T=0, ptr=0), q=None, idx=None, lse=None, s=None, loss=None) == 0


def test_workspace_sizes_grow_with_the_problem(lib):
    a = lib.sga_forward_workspace_size(16, 131072, 2048)
    b = lib.sga_forward_workspace_size(16, 262144, 2048)
    assert 0 < a < b
    assert lib.sga_forward_workspace_size(0, 100, 8) == 0
    assert lib.sga_topk_workspace_size(4, 4096, 2048) > 4 * 4096 * 4


def test_hbm_read_probe_rejects_bad_arguments(lib):
    dummy = ctypes.c_void_p(0x1000)
    # null pointers, an empty read and a size that is not a multiple of 4 KiB
    assert lib.sga_hbm_read_probe(None, 4096, dummy, None) == 1
    assert lib.sga_hbm_read_probe(dummy, 4096, None, None) == 1
    assert lib.sga_hbm_read_probe(dummy, 0, dummy, None) == 1
    assert lib.sga_hbm_read_probe(dummy, 4097, dummy, None) == 1
