"""CPU checks of the C ABI: the library loads without a GPU, exports every
symbol include/gist_attn.h declares, and validates arguments on the host
before any HIP call (so every error path below runs with no device)."""

import ctypes
import json
import os
import re

import pytest

from gist_compressed_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gist_attn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "byte_counts.json")

BF16, F32, FP8 = _lib.GIST_BF16, _lib.GIST_F32, _lib.GIST_FP8_E4M3
FAKE = ctypes.c_void_p(1 << 20)  # an aligned address that is never dereferenced


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_every_declared_symbol_is_exported_and_bound(L):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(L, n)


def test_pool_bytes_matches_printed_per_item_size(L):
    g = json.load(open(GOLDEN))
    for e in g["per_item_gist"]:
        assert L.gist_pool_bytes(e["L"], 1, e["k"], e["H"], e["h"], BF16) == e["bytes"]
    for e in g["pool_totals_100k_items_k8"]:
        n = L.gist_pool_bytes(e["L"], e["items"], e["k"], e["H"], e["h"], BF16)
        assert abs(n / 2**30 - e["gib"]) <= e["rel_tol"] * e["gib"]
    assert L.gist_pool_bytes(1, 2, 8, 1, 64, F32) == 2 * 2 * 8 * 64 * 4
    assert L.gist_pool_bytes(0, 2, 8, 1, 64, BF16) == 0
    assert L.gist_pool_bytes(1, 2, 8, 1, 64, 7) == 0


def _create(L, *args):
    h = ctypes.c_void_p()
    st = L.gist_pool_create(ctypes.byref(h), *args)
    return st, h


def test_pool_create_validation(L):
    nbytes = L.gist_pool_bytes(2, 10, 8, 2, 64, BF16)
    st, h = _create(L, 2, 10, 8, 2, 64, BF16, FAKE, nbytes)
    assert st == _lib.GIST_OK and h.value
    assert L.gist_pool_destroy(h) == _lib.GIST_OK
    cases = [
        ((2, 10, 8, 2, 64, BF16, None, nbytes), _lib.GIST_ERR_INVALID_ARG, "NULL"),
        ((2, 10, 8, 2, 64, BF16, FAKE, nbytes - 2), _lib.GIST_ERR_INVALID_ARG, "storage_bytes"),
        ((2, 10, 8, 2, 64, BF16, ctypes.c_void_p((1 << 20) + 8), nbytes),
         _lib.GIST_ERR_INVALID_ARG, "aligned"),
        ((2, 10, 8, 2, 96, BF16, FAKE, L.gist_pool_bytes(2, 10, 8, 2, 96, BF16)),
         _lib.GIST_ERR_UNSUPPORTED, "head_dim"),
        ((2, 10, 65, 2, 64, BF16, FAKE, L.gist_pool_bytes(2, 10, 65, 2, 64, BF16)),
         _lib.GIST_ERR_UNSUPPORTED, "k must"),
        ((0, 10, 8, 2, 64, BF16, FAKE, 0), _lib.GIST_ERR_INVALID_ARG, "positive"),
        ((2, 10, 8, 2, 64, 5, FAKE, nbytes), _lib.GIST_ERR_INVALID_ARG, "dtype"),
    ]
    for args, code, msg in cases:
        st, h = _create(L, *args)
        assert st == code, (args, st)
        assert h.value is None
        assert msg in L.gist_last_error().decode()
    assert L.gist_pool_create(None, 2, 10, 8, 2, 64, BF16, FAKE, nbytes) == _lib.GIST_ERR_INVALID_ARG
    assert L.gist_pool_destroy(None) == _lib.GIST_OK


def _pool(L, Lyr=2, N=10, k=8, H=2, d=64, dt=BF16):
    st, h = _create(L, Lyr, N, k, H, d, dt, FAKE, L.gist_pool_bytes(Lyr, N, k, H, d, dt))
    assert st == 0
    return h


def _fwd(L, pool, layer=0, P=4, ell=16, Hq=14, pos0=9, base=1e4, scale=0.125, qpool=None,
         qids=None, ptr=FAKE, ids=FAKE):
    return L.gist_attn_forward(pool, layer, ids, P, ell, Hq, ptr, ptr, ptr, pos0, base, scale,
                               qpool, qids, ptr, None)


def test_forward_validation(L):
    pool = _pool(L)
    try:
        assert _fwd(L, None) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, layer=2) == _lib.GIST_ERR_OUT_OF_RANGE
        assert _fwd(L, pool, layer=-1) == _lib.GIST_ERR_OUT_OF_RANGE
        assert _fwd(L, pool, P=-1) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, ell=0) == _lib.GIST_ERR_UNSUPPORTED
        assert _fwd(L, pool, ell=1025) == _lib.GIST_ERR_UNSUPPORTED
        assert _fwd(L, pool, Hq=13) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, Hq=1) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, Hq=66) == _lib.GIST_ERR_UNSUPPORTED
        assert _fwd(L, pool, scale=0.0) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, scale=float("nan")) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, base=-1.0) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, ptr=None) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, ids=None) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, ptr=ctypes.c_void_p((1 << 20) + 4)) == _lib.GIST_ERR_INVALID_ARG
        # an empty batch is accepted without touching the device
        assert _fwd(L, pool, P=0, ptr=None, ids=None) == _lib.GIST_OK
        # query-gist pool must match the item pool
        other = _pool(L, d=128)
        try:
            assert _fwd(L, pool, qpool=other, qids=FAKE) == _lib.GIST_ERR_INVALID_ARG
        finally:
            L.gist_pool_destroy(other)
        same = _pool(L, k=4)
        try:
            assert _fwd(L, pool, qpool=same, qids=None) == _lib.GIST_ERR_INVALID_ARG
        finally:
            L.gist_pool_destroy(same)
    finally:
        L.gist_pool_destroy(pool)


def _grp(L, pool, groups, ell=16, Hq=14, qpool=None, base=1e4, scale=0.125, n=None):
    arr = (_lib.GistGroup * max(len(groups), 1))(*[_lib.GistGroup(*g) for g in groups])
    return L.gist_attn_forward_grouped(pool, qpool, arr if groups or n else None,
                                       len(groups) if n is None else n, ell, Hq, 9, base, scale,
                                       None)


def _g(layer=0, P=4, ptr=FAKE, ids=FAKE, qids=None):
    return (layer, P, ids, qids, ptr, ptr, ptr, ptr)


def test_grouped_validation(L):
    pool = _pool(L)
    f32 = _pool(L, dt=F32)
    try:
        assert _grp(L, None, [_g()]) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [], n=-1) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g()] * 33) == _lib.GIST_ERR_UNSUPPORTED
        assert "32" in L.gist_last_error().decode()
        assert L.gist_attn_forward_grouped(pool, None, None, 2, 16, 14, 9, 1e4, 0.125,
                                           None) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g(), _g(layer=2)]) == _lib.GIST_ERR_OUT_OF_RANGE
        assert _grp(L, pool, [_g(layer=-1)]) == _lib.GIST_ERR_OUT_OF_RANGE
        assert _grp(L, pool, [_g(P=-1)]) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g(), _g(ptr=None)]) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g(ids=None)]) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g(ptr=ctypes.c_void_p((1 << 20) + 4))]) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g()], Hq=13) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g()], Hq=66) == _lib.GIST_ERR_UNSUPPORTED
        assert _grp(L, pool, [_g()], scale=0.0) == _lib.GIST_ERR_INVALID_ARG
        assert _grp(L, pool, [_g()], base=float("inf")) == _lib.GIST_ERR_INVALID_ARG
        # groups run the EOS kernel (ell = 1) or the l >= 2 kernel
        assert _grp(L, pool, [_g()], ell=1, Hq=34) == _lib.GIST_ERR_UNSUPPORTED  # Hq/H = 17
        assert _grp(L, pool, [_g(P=0, ptr=None, ids=None)], ell=1) == _lib.GIST_OK
        assert _grp(L, pool, [_g()], ell=65) == _lib.GIST_ERR_UNSUPPORTED
        assert _grp(L, pool, [_g()], ell=121) == _lib.GIST_ERR_UNSUPPORTED  # 8 + 121 keys
        assert _grp(L, f32, [_g()]) == _lib.GIST_ERR_UNSUPPORTED
        # a query-gist pool needs q_ids in every group that has pairs
        q4 = _pool(L, k=4)
        try:
            assert _grp(L, pool, [_g(qids=FAKE), _g()], qpool=q4) == _lib.GIST_ERR_INVALID_ARG
            assert _grp(L, pool, [_g(P=0, ptr=None, ids=None)], qpool=q4) == _lib.GIST_OK
        finally:
            L.gist_pool_destroy(q4)
        # no pairs at all: a no-op that touches nothing
        assert _grp(L, pool, []) == _lib.GIST_OK
        assert _grp(L, pool, [_g(P=0, ptr=None, ids=None)] * 32) == _lib.GIST_OK
    finally:
        L.gist_pool_destroy(pool)
        L.gist_pool_destroy(f32)


def test_pool_write_validation(L):
    pool = _pool(L)
    try:
        w = L.gist_pool_write
        assert w(None, 0, FAKE, 1, FAKE, FAKE, 1, 1e4, None) == _lib.GIST_ERR_INVALID_ARG
        assert w(pool, 5, FAKE, 1, FAKE, FAKE, 1, 1e4, None) == _lib.GIST_ERR_OUT_OF_RANGE
        assert w(pool, 0, FAKE, -1, FAKE, FAKE, 1, 1e4, None) == _lib.GIST_ERR_INVALID_ARG
        assert w(pool, 0, None, 1, FAKE, FAKE, 1, 1e4, None) == _lib.GIST_ERR_INVALID_ARG
        assert w(pool, 0, FAKE, 1, FAKE, FAKE, 1, 0.0, None) == _lib.GIST_ERR_INVALID_ARG
        assert w(pool, 0, None, 0, None, None, 1, 1e4, None) == _lib.GIST_OK
    finally:
        L.gist_pool_destroy(pool)


def _dec(L, R=2, Hq=4, H=2, d=64, bs=16, max_blk=4, nblk=8, dt=BF16, ws_bytes=None, ptr=FAKE,
         scale=0.125):
    if ws_bytes is None:
        ws_bytes = L.paged_decode_workspace_bytes(R, Hq, max_blk, bs, d)
    return L.paged_decode_attn(ptr, ptr, nblk, bs, ptr, max_blk, ptr, R, ptr, ptr, ptr, ptr, Hq,
                               H, d, dt, 1e4, scale, ptr, ptr, ws_bytes, None)


def test_paged_decode_validation(L):
    assert L.paged_decode_workspace_bytes(32, 32, 16, 256, 128) == 32 * 32 * 16 * 132 * 4
    assert L.paged_decode_workspace_bytes(1, 1, 1, 16, 64) == 68 * 4
    assert L.paged_decode_workspace_bytes(0, 4, 4, 16, 64) == 0
    assert _dec(L, R=-1) == _lib.GIST_ERR_INVALID_ARG
    assert _dec(L, Hq=5) == _lib.GIST_ERR_INVALID_ARG
    assert _dec(L, Hq=32, H=2) == _lib.GIST_ERR_UNSUPPORTED
    assert _dec(L, d=96) == _lib.GIST_ERR_UNSUPPORTED
    assert _dec(L, bs=24) == _lib.GIST_ERR_UNSUPPORTED
    assert _dec(L, nblk=0) == _lib.GIST_ERR_INVALID_ARG
    assert _dec(L, max_blk=0) == _lib.GIST_ERR_INVALID_ARG
    assert _dec(L, dt=3) == _lib.GIST_ERR_INVALID_ARG
    assert _dec(L, dt=FP8) == _lib.GIST_ERR_INVALID_ARG  # fp8 caches have their own entry point
    assert _dec(L, scale=-1.0) == _lib.GIST_ERR_INVALID_ARG
    assert _dec(L, ptr=None) == _lib.GIST_ERR_INVALID_ARG
    assert _dec(L, ws_bytes=16) == _lib.GIST_ERR_INVALID_ARG
    assert "workspace too small" in L.gist_last_error().decode()
    assert _dec(L, R=0, ptr=None) == _lib.GIST_OK


def _decn(L, R=2, Hq=4, H=2, d=64, bs=16, max_blk=4, nblk=8, dt=BF16, ptr=FAKE, scale=0.125):
    return L.paged_decode_attn_noalloc(ptr, ptr, nblk, bs, ptr, max_blk, ptr, R, ptr, ptr, ptr,
                                       ptr, Hq, H, d, dt, 1e4, scale, ptr, None)


def test_paged_decode_noalloc_validation(L):
    # every rejection happens on the host, before the scratch address is looked up
    assert _decn(L, R=-1) == _lib.GIST_ERR_INVALID_ARG
    assert _decn(L, Hq=5) == _lib.GIST_ERR_INVALID_ARG
    assert _decn(L, d=96) == _lib.GIST_ERR_UNSUPPORTED
    assert _decn(L, bs=24) == _lib.GIST_ERR_UNSUPPORTED
    assert _decn(L, dt=FP8) == _lib.GIST_ERR_INVALID_ARG
    assert _decn(L, ptr=None) == _lib.GIST_ERR_INVALID_ARG
    assert "paged_decode_attn_noalloc" in L.gist_last_error().decode()
    assert _decn(L, R=0, ptr=None) == _lib.GIST_OK
    # 16 MiB of split-K partials at most: 32 x 32 x 16 splits fits, 64 x 32 x 64 does not
    assert L.paged_decode_workspace_bytes(32, 32, 16, 256, 128) <= 16 << 20
    assert L.paged_decode_workspace_bytes(64, 32, 64, 256, 128) > 16 << 20
    assert _decn(L, R=64, Hq=32, H=32, d=128, bs=256, max_blk=64) == _lib.GIST_ERR_UNSUPPORTED
    msg = L.gist_last_error().decode()
    assert "scratch" in msg and str(16 << 20) in msg


def _dec8(L, R=2, Hq=4, H=2, d=64, bs=16, max_blk=4, nblk=8, ws_bytes=None, ptr=FAKE, sptr=FAKE,
          scale=0.125):
    if ws_bytes is None:
        ws_bytes = L.paged_decode_workspace_bytes(R, Hq, max_blk, bs, d)
    return L.paged_decode_attn_fp8(ptr, ptr, sptr, sptr, nblk, bs, ptr, max_blk, ptr, R, ptr, ptr,
                                   ptr, ptr, Hq, H, d, 1e4, scale, ptr, ptr, ws_bytes, None)


def test_paged_decode_fp8_validation(L):
    assert _dec8(L, R=-1) == _lib.GIST_ERR_INVALID_ARG
    assert _dec8(L, Hq=5) == _lib.GIST_ERR_INVALID_ARG
    assert _dec8(L, d=96) == _lib.GIST_ERR_UNSUPPORTED
    assert _dec8(L, bs=24) == _lib.GIST_ERR_UNSUPPORTED
    assert _dec8(L, sptr=None) == _lib.GIST_ERR_INVALID_ARG
    assert "paged_decode_attn_fp8" in L.gist_last_error().decode()
    assert _dec8(L, sptr=ctypes.c_void_p((1 << 20) + 2)) == _lib.GIST_ERR_INVALID_ARG
    assert "4-byte aligned" in L.gist_last_error().decode()
    assert _dec8(L, ws_bytes=16) == _lib.GIST_ERR_INVALID_ARG
    assert _dec8(L, R=0, ptr=None, sptr=None) == _lib.GIST_OK


def test_fp8_pool_bytes_and_create(L):
    # codes (one byte per element) plus one fp32 scale per (layer, item, K/V, head)
    assert L.gist_pool_bytes(28, 1, 8, 8, 128, FP8) == 28 * (2 * 8 * 8 * 128 + 2 * 8 * 4)
    assert L.gist_pool_bytes(2, 10, 8, 2, 64, FP8) == 2 * 10 * (2 * 8 * 2 * 64 + 16)
    nbytes = L.gist_pool_bytes(2, 10, 8, 2, 64, FP8)
    st, h = _create(L, 2, 10, 8, 2, 64, FP8, FAKE, nbytes)
    assert st == _lib.GIST_OK and h.value
    L.gist_pool_destroy(h)
    st, h = _create(L, 2, 10, 8, 2, 64, FP8, FAKE, nbytes + 1)
    assert st == _lib.GIST_ERR_INVALID_ARG and "storage_bytes" in L.gist_last_error().decode()


def test_fp8_pool_forward_limits(L):
    pool = _pool(L, dt=FP8)
    qp8 = _pool(L, k=8, dt=FP8)
    qbf = _pool(L, k=8, dt=BF16)
    big = _pool(L, k=30, dt=FP8)  # k + k' = 38 > 32
    p64 = _pool(L, k=64, dt=FP8)
    try:
        # fp8 pools run on the MFMA kernel (2 <= ell <= 64, k + k' + ell <= 128)
        # and the EOS kernel (ell = 1, Hq/H <= 16, k + k' <= 32) only
        assert _fwd(L, pool, ell=65) == _lib.GIST_ERR_UNSUPPORTED
        assert "fp8" in L.gist_last_error().decode()
        assert _fwd(L, p64, ell=2, qpool=p64, qids=FAKE) == _lib.GIST_ERR_UNSUPPORTED
        assert _fwd(L, pool, ell=1, Hq=34) == _lib.GIST_ERR_UNSUPPORTED
        assert _fwd(L, pool, ell=1, qpool=big, qids=FAKE) == _lib.GIST_ERR_UNSUPPORTED
        # in range: validated, nothing launched for P = 0
        assert _fwd(L, pool, ell=16, P=0, ptr=None, ids=None) == _lib.GIST_OK
        assert _fwd(L, p64, ell=64, P=0, ptr=None, ids=None) == _lib.GIST_OK
        # the query-gist pool must be fp8 too
        assert _fwd(L, pool, ell=1, qpool=qbf, qids=FAKE) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, ell=16, qpool=qbf, qids=FAKE) == _lib.GIST_ERR_INVALID_ARG
        assert _fwd(L, pool, ell=1, P=0, qpool=qp8, qids=FAKE, ptr=None, ids=None) == _lib.GIST_OK
    finally:
        for h in (pool, qp8, qbf, big, p64):
            L.gist_pool_destroy(h)


def _pf(L, B=2, T=100, max_len=64, Hq=4, H=2, d=64, ptr=FAKE, ws=None, pool=None, layer=0,
        ids=FAKE, scale=0.125, base=1e4):
    if ws is None:
        ws = L.gist_prefill_workspace_bytes(T, H, d)
    return L.gist_prefill_attn(ptr, ptr, ptr, ptr, B, T, max_len, Hq, H, d, base, scale, ptr, ptr,
                               ws, pool, layer, ids, None)


def test_prefill_validation(L):
    # the rotated K as a bf16 pair: two bf16 values per element
    assert L.gist_prefill_workspace_bytes(1000, 2, 64) == 2 * 1000 * 2 * 64 * 2
    assert L.gist_prefill_workspace_bytes(-1, 2, 64) == 0
    assert _pf(L, B=-1) == _lib.GIST_ERR_INVALID_ARG
    assert _pf(L, max_len=0) == _lib.GIST_ERR_INVALID_ARG
    assert _pf(L, Hq=5) == _lib.GIST_ERR_INVALID_ARG
    assert _pf(L, d=96) == _lib.GIST_ERR_UNSUPPORTED
    assert _pf(L, scale=0.0) == _lib.GIST_ERR_INVALID_ARG
    assert _pf(L, base=float("inf")) == _lib.GIST_ERR_INVALID_ARG
    assert _pf(L, ptr=None) == _lib.GIST_ERR_INVALID_ARG
    assert _pf(L, ptr=ctypes.c_void_p((1 << 20) + 8)) == _lib.GIST_ERR_INVALID_ARG
    assert _pf(L, ws=100) == _lib.GIST_ERR_INVALID_ARG
    assert "workspace too small" in L.gist_last_error().decode()
    assert _pf(L, B=0, ptr=None) == _lib.GIST_OK
    assert _pf(L, B=70000) == _lib.GIST_ERR_UNSUPPORTED
    bf = _pool(L, H=2, d=64)
    f32 = _pool(L, H=2, d=64, dt=F32)
    other = _pool(L, H=1, d=64)
    try:
        assert _pf(L, pool=f32) == _lib.GIST_ERR_UNSUPPORTED
        assert _pf(L, pool=other) == _lib.GIST_ERR_INVALID_ARG
        assert _pf(L, pool=bf, layer=2) == _lib.GIST_ERR_OUT_OF_RANGE
        assert _pf(L, pool=bf, ids=None) == _lib.GIST_ERR_INVALID_ARG
        assert _pf(L, pool=bf, B=0, ptr=None, ids=None) == _lib.GIST_OK
    finally:
        for hd in (bf, f32, other):
            L.gist_pool_destroy(hd)


def _pg(L, nblk=8, bs=16, k=8, kq=8, q_row0=8, P=4, ell=1, Hq=16, H=2, d=64, ptr=FAKE, qb=FAKE,
        scale=0.125):
    return L.gist_attn_forward_paged(ptr, ptr, nblk, bs, ptr, k, qb, kq, q_row0, P, ell, Hq, H, d,
                                     ptr, ptr, ptr, k + kq + 1, 1e4, scale, ptr, None)


def test_paged_gist_validation(L):
    assert _pg(L, P=-1) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, nblk=0) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, bs=0) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, d=96) == _lib.GIST_ERR_UNSUPPORTED
    assert _pg(L, Hq=3) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, Hq=34) == _lib.GIST_ERR_UNSUPPORTED
    assert _pg(L, k=0) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, k=17) == _lib.GIST_ERR_INVALID_ARG        # item gist past the block
    assert _pg(L, q_row0=9) == _lib.GIST_ERR_INVALID_ARG    # query gist past the block
    assert _pg(L, bs=64, k=20, kq=20, q_row0=20) == _lib.GIST_ERR_UNSUPPORTED  # k + k' > 32
    assert _pg(L, qb=None) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, ptr=None) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, ptr=ctypes.c_void_p((1 << 20) + 4)) == _lib.GIST_ERR_INVALID_ARG
    assert _pg(L, P=0, ptr=None) == _lib.GIST_OK
    assert _pg(L, kq=0, qb=None, P=0, ptr=None) == _lib.GIST_OK
    # ell >= 2 (the l >= 2 kernel over paged gists)
    assert _pg(L, ell=0) == _lib.GIST_ERR_UNSUPPORTED
    assert _pg(L, ell=65) == _lib.GIST_ERR_UNSUPPORTED
    assert _pg(L, ell=2, Hq=66, H=2) == _lib.GIST_ERR_UNSUPPORTED           # Hq/H > 32
    assert _pg(L, ell=64, bs=64, k=64, kq=1, q_row0=63) == _lib.GIST_ERR_UNSUPPORTED  # 129 keys
    assert _pg(L, ell=64, bs=64, k=20, kq=20, q_row0=20, ptr=None) == _lib.GIST_ERR_INVALID_ARG
    assert "keys" not in L.gist_last_error().decode()  # k + k' > 32 is fine for ell >= 2
    assert _pg(L, ell=16, Hq=34, H=2, P=0, ptr=None) == _lib.GIST_OK         # Hq/H = 17


def _pg8(L, nblk=8, bs=16, k=8, kq=8, q_row0=8, P=4, ell=1, Hq=16, H=2, d=64, ptr=FAKE, qb=FAKE,
         ks=FAKE, vs=FAKE):
    return L.gist_attn_forward_paged_fp8(ptr, ptr, ks, vs, nblk, bs, ptr, k, qb, kq, q_row0, P, ell,
                                         Hq, H, d, ptr, ptr, ptr, k + kq + 1, 1e4, 0.125, ptr, None)


def test_paged_gist_fp8_validation(L):
    # the checks of the bf16 entry point, plus the two scale arrays
    assert _pg8(L, P=-1) == _lib.GIST_ERR_INVALID_ARG
    assert _pg8(L, d=96) == _lib.GIST_ERR_UNSUPPORTED
    assert _pg8(L, Hq=34) == _lib.GIST_ERR_UNSUPPORTED
    assert _pg8(L, k=17) == _lib.GIST_ERR_INVALID_ARG
    assert _pg8(L, bs=64, k=20, kq=20, q_row0=20) == _lib.GIST_ERR_UNSUPPORTED
    assert _pg8(L, ks=None) == _lib.GIST_ERR_INVALID_ARG
    assert _pg8(L, vs=None) == _lib.GIST_ERR_INVALID_ARG
    assert _pg8(L, vs=ctypes.c_void_p((1 << 20) + 2)) == _lib.GIST_ERR_INVALID_ARG
    assert "4-byte" in L.gist_last_error().decode()
    assert _pg8(L, P=0, ptr=None, ks=None, vs=None) == _lib.GIST_OK


def test_last_error_is_per_thread(L):
    # gist_last_error reports the last failing call of the calling thread:
    # two threads that fail in different ways each read their own message
    import threading

    pool = _pool(L)
    seen = {}
    ready = threading.Barrier(2)

    def worker(name, kwargs):
        st = _fwd(L, pool, **kwargs)
        ready.wait()  # both calls have failed before either message is read
        seen[name] = (st, L.gist_last_error().decode())

    try:
        ts = [threading.Thread(target=worker, args=("layer", {"layer": 5})),
              threading.Thread(target=worker, args=("scale", {"scale": 0.0}))]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    finally:
        L.gist_pool_destroy(pool)
    assert seen["layer"][0] == _lib.GIST_ERR_OUT_OF_RANGE
    assert seen["scale"][0] == _lib.GIST_ERR_INVALID_ARG
    assert seen["layer"][1] != seen["scale"][1]
    assert "layer" in seen["layer"][1] and "scale" in seen["scale"][1]
