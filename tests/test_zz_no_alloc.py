"""The allocation-free decode entry point (paged_decode_attn_noalloc): its
output equals paged_decode_attn's with a caller workspace, bit for bit, and
the oracle's within the bf16 bar, on two calls in a row, the second smaller
(the library's scratch keeps the first call's contents)."""

import numpy as np
import pytest
import torch

from gpu_cases import ROPE_BASE, TOL, DecodeCase, f64, say

pytestmark = pytest.mark.gpu


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    import gist_compressed_kv_amd as G
    cases = [
        # n_blocks, h, bs, d, hq, lens (the first: 12 requests x 32 heads x 32
        # splits of 132 floats = 6.5 MB of the 16 MiB scratch)
        DecodeCase(384, 4, 256, 128, 32, [8192, 4096, 17, 0, 2048, 8191, 1, 256, 300, 7000,
                                          512, 4000], torch.bfloat16, 901),
        DecodeCase(12, 2, 64, 64, 4, [100, 1, 250], torch.bfloat16, 902),
    ]
    for i, case in enumerate(cases):
        say(f"noalloc call {i}: R={case.q.shape[0]} Hq={case.q.shape[1]} d={case.q.shape[2]}")
        ref = case.run()
        got = G.paged_decode_attn_noalloc(case.kc, case.vc, case.table, case.lens, case.q, case.kn,
                                          case.vn, case.positions, ROPE_BASE, case.scale)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "noalloc output differs from the workspace entry point"
        err = float(np.abs(f64(got) - case.oracle()).max())
        say(f"noalloc call {i}: equal to paged_decode_attn; max-abs err vs oracle {err:.3g}")
        assert err <= TOL[torch.bfloat16]


def test_noalloc_decode_rejects_calls_past_the_scratch():
    import gist_compressed_kv_amd as G
    from gist_compressed_kv_amd import _lib
    # 64 requests x 32 heads x 64 splits x 132 floats = 69 MB > 16 MiB: refused
    # on the host, before anything is launched
    R, H, bs, d, max_blocks = 64, 32, 256, 128, 64
    q = torch.zeros((R, H, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((R, H, d), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((R, max_blocks), dtype=torch.int32, device="cuda")
    lens = torch.ones(R, dtype=torch.int32, device="cuda")
    kc = torch.zeros((4, H, bs, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.GistError) as e:
        G.paged_decode_attn_noalloc(kc, kc, table, lens, q, kv, kv, lens + 1)
    assert "GIST_ERR_UNSUPPORTED" in str(e.value) and "scratch" in str(e.value)
