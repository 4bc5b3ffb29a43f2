"""Argument checks of the Python binding.

The library reads every tensor at the extents that the call's sizes imply,
so the binding must reject a tensor whose dtype or shape disagrees with them
before anything reaches the library.  The checks run on all of a call's
tensors first; only tensors that pass them are then required to be on the
GPU.  Here every tensor lives on the CPU, so a consistent call stops at that
last check and the library's entry points are never called.
"""

import types

import pytest
import torch

import gist_compressed_kv_amd as G

BF = torch.bfloat16
I32 = torch.int32
F32 = torch.float32
U8 = torch.uint8
ON_GPU = "must live on the GPU"


def z(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


# the forward wrappers read only these attributes of the pool before the checks
POOL = types.SimpleNamespace(k=8, H=2, d=64, act_dtype=BF, handle=None)
P, ELL, HQ, H, D = 3, 16, 14, 2, 64


def test_pool_write_source_shape():
    with pytest.raises(ValueError, match="k_src must have shape"):
        G.gist_pool_write(POOL, 0, z(4, dtype=I32), z(4, 7, H, D), z(4, 8, H, D))
    with pytest.raises(ValueError, match=ON_GPU):
        G.gist_pool_write(POOL, 0, z(4, dtype=I32), z(4, 8, H, D), z(4, 8, H, D))


def test_forward_q_head_dim_must_be_the_pools():
    kv = z(P, ELL, H, D)
    with pytest.raises(ValueError, match="q must have shape"):
        G.gist_attn_forward(POOL, 0, z(P, dtype=I32), z(P, ELL, HQ, 32), kv, kv)
    with pytest.raises(ValueError, match="k_new must have shape"):
        G.gist_attn_forward(POOL, 0, z(P, dtype=I32), z(P, ELL, HQ, D), z(P, ELL + 1, H, D), kv)
    with pytest.raises(TypeError, match="q must be"):
        G.gist_attn_forward(POOL, 0, z(P, dtype=I32), z(P, ELL, HQ, D, dtype=F32), kv, kv)
    with pytest.raises(ValueError, match=ON_GPU):
        G.gist_attn_forward(POOL, 0, z(P, dtype=I32), z(P, ELL, HQ, D), kv, kv)


def test_forward_last_q_head_dim_must_be_the_pools():
    kv = z(P, ELL, H, D)
    with pytest.raises(ValueError, match="q_last must have shape"):
        G.gist_attn_forward_last(POOL, 0, z(P, dtype=I32), z(P, HQ, 128), kv, kv)
    with pytest.raises(ValueError, match=ON_GPU):
        G.gist_attn_forward_last(POOL, 0, z(P, dtype=I32), z(P, HQ, D), kv, kv)


def test_paged_gist_q_head_dim_must_be_the_caches():
    kc = z(10, H, 16, D)
    kv = z(P, H, D)
    with pytest.raises(ValueError, match="q must have shape"):
        G.gist_attn_forward_paged(kc, kc, z(P, dtype=I32), 8, z(P, HQ, 32), kv, kv)
    with pytest.raises(ValueError, match=ON_GPU):
        G.gist_attn_forward_paged(kc, kc, z(P, dtype=I32), 8, z(P, HQ, D), kv, kv)


def test_paged_gist_fp8_q_head_dim_must_be_the_caches():
    kc = z(10, H, 16, D, dtype=U8)
    sc = z(10, H, dtype=F32)
    kv = z(P, H, D)
    with pytest.raises(ValueError, match="q must have shape"):
        G.gist_attn_forward_paged_fp8(kc, kc, sc, sc, z(P, dtype=I32), 8, z(P, HQ, 32), kv, kv)
    with pytest.raises(ValueError, match="k_scale must have shape"):
        G.gist_attn_forward_paged_fp8(kc, kc, z(10, H + 1, dtype=F32), sc, z(P, dtype=I32), 8,
                                      z(P, HQ, D), kv, kv)
    with pytest.raises(ValueError, match=ON_GPU):
        G.gist_attn_forward_paged_fp8(kc, kc, sc, sc, z(P, dtype=I32), 8, z(P, HQ, D), kv, kv)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_paged_decode_q_and_block_table_shapes(fp8):
    R, hq, h, bs, d, mb = 3, 8, 2, 16, 64, 4
    kc = z(12, h, bs, d, dtype=U8 if fp8 else BF)
    kv, pos, lens = z(R, h, d), z(R, dtype=I32), z(R, dtype=I32)

    def call(table, q):
        if fp8:
            sc = z(12, h, dtype=F32)
            return G.paged_decode_attn_fp8(kc, kc, sc, sc, table, lens, q, kv, kv, pos)
        return G.paged_decode_attn(kc, kc, table, lens, q, kv, kv, pos)

    with pytest.raises(ValueError, match="q must have shape"):
        call(z(R, mb, dtype=I32), z(R, hq, 32))
    with pytest.raises(ValueError, match=r"block_table must be \[R, max_blocks\]"):
        call(z(R * mb, dtype=I32), z(R, hq, d))
    with pytest.raises(ValueError, match="block_table must have shape"):
        call(z(R + 1, mb, dtype=I32), z(R, hq, d))
    with pytest.raises(ValueError, match=ON_GPU):
        call(z(R, mb, dtype=I32), z(R, hq, d))


def _grp(P_=P, ell=ELL, hq=HQ, d=D, kv_h=H, q_ids=False):
    g = {"layer": 0, "item_ids": z(P_, dtype=I32), "q": z(P_, ell, hq, d),
         "k_new": z(P_, ell, kv_h, D), "v_new": z(P_, ell, kv_h, D)}
    if q_ids:
        g["q_ids"] = z(P_, dtype=I32)
    return g


def test_grouped_shapes_are_checked_group_by_group():
    # every group shares ell and Hq with the first, and its head size is the pool's
    with pytest.raises(ValueError, match="one ell and Hq"):
        G.GroupedForward(POOL, [_grp(), _grp(ell=ELL + 1)])
    with pytest.raises(ValueError, match="one ell and Hq"):
        G.GroupedForward(POOL, [_grp(), _grp(hq=HQ + 2)])
    with pytest.raises(ValueError, match="one ell and Hq"):
        G.GroupedForward(POOL, [_grp(d=32)])
    with pytest.raises(ValueError, match="k_new must have shape"):
        G.GroupedForward(POOL, [_grp(), _grp(kv_h=H + 1)])
    with pytest.raises(ValueError, match=r"q must have shape \[P, ell, Hq, d\]"):
        G.GroupedForward(POOL, [{"layer": 0, "item_ids": z(P, dtype=I32), "q": z(P, HQ, D),
                                 "k_new": z(P, H, D), "v_new": z(P, H, D)}])
    # a consistent table stops at the device check, before the library
    with pytest.raises(ValueError, match=ON_GPU):
        G.GroupedForward(POOL, [_grp(), _grp(P_=5)])
    # no groups: nothing to launch
    assert G.gist_attn_forward_grouped(POOL, []) == []


def test_grouped_query_gist_ids_are_required():
    qpool = types.SimpleNamespace(k=8, H=2, d=64, act_dtype=BF, handle=None)
    with pytest.raises(KeyError):
        G.GroupedForward(POOL, [_grp()], qpool=qpool)
    with pytest.raises(ValueError, match=ON_GPU):
        G.GroupedForward(POOL, [_grp(q_ids=True)], qpool=qpool)
