"""GPU parity: the HIP library (called through its C ABI) against the fp64 oracle.

Bars: max-abs error <= 2e-2 for bf16 inputs (fp32 accumulation) and <= 1e-5
for fp32, on every element checked.  Small cases are checked in full; the
full-size workloads (100k-item pools, 24/28/32 layers) are checked on
seeded samples of pairs/requests, every head and token of each.
"""

import math

import numpy as np
import pytest
import torch

import gist_compressed_kv_amd as G
from gpu_cases import TOL, DecodeCase, GistCase, f64, say
from gist_compressed_kv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _cleanup():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_gist(case, layers=None, sample=None, label=""):
    layers = case.act_layers if layers is None else layers
    worst = 0.0
    for li in layers:
        out = case.run(li)
        torch.cuda.synchronize()
        s = np.arange(case.pairs) if sample is None else sample
        err = case.max_err(li, out, s)
        worst = max(worst, err)
        assert err <= TOL[case.dtype], f"{label} layer {li}: max-abs err {err}"
    say(f"{label}: max-abs err {worst:.3g}")
    return worst


# ---------------------------------------------------------------------------
# The tiny fp32 workload, in full
# ---------------------------------------------------------------------------


def test_tiny_fp32_workload():
    wl = synth.TINY
    case = GistCase(1, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype, wl.seed,
                    ids=torch.tensor([0, 1, 0, 1]))
    check_gist(case, label="tiny fp32")


# ---------------------------------------------------------------------------
# MFMA path (bf16, 2 <= ell <= 64, k + k' + ell <= 128)
# ---------------------------------------------------------------------------

MFMA_SHAPES = [
    # ell, k, kq, hq, h, d, pairs
    (2, 8, 0, 14, 2, 64, 3),
    (16, 8, 0, 4, 1, 64, 4),
    (37, 8, 0, 14, 2, 64, 5),
    (64, 8, 0, 14, 2, 64, 6),
    (64, 8, 0, 64, 8, 128, 3),
    (33, 1, 0, 8, 8, 64, 3),
    (64, 64, 0, 8, 2, 64, 2),
    (20, 8, 8, 16, 2, 128, 3),
    (63, 5, 0, 7, 1, 64, 2),
    (64, 24, 0, 32, 1, 128, 2),
    (48, 8, 0, 16, 2, 64, 5),
    # k + k' + ell exactly 128 with a query gist
    (64, 32, 32, 8, 2, 64, 2),
]


@pytest.mark.parametrize("shape", MFMA_SHAPES, ids=lambda s: "ell%d_k%d_kq%d_hq%d_h%d_d%d" % s[:6])
def test_mfma_path_shapes(shape):
    ell, k, kq, hq, h, d, P = shape
    qids = torch.arange(P) % 2 if kq else None
    case = GistCase(2, 7, k, ell, hq, h, d, P, torch.bfloat16, 100 + ell, kq=kq, n_qrows=2,
                    q_ids=qids)
    check_gist(case, label=f"mfma {shape}")


# ---------------------------------------------------------------------------
# VALU path (ell = 1, long ell, fp32)
# ---------------------------------------------------------------------------

# ell = 1 in bf16 with G <= 16 and k + k' <= 32 runs the MFMA EOS kernel;
# the rest of this list runs the VALU kernel
VALU_SHAPES = [
    # ell, k, kq, hq, h, d, pairs, dtype
    (1, 12, 8, 16, 2, 128, 3, torch.bfloat16),
    (1, 20, 0, 8, 1, 64, 3, torch.bfloat16),
    (1, 8, 0, 34, 2, 64, 3, torch.bfloat16),
    (1, 40, 0, 4, 2, 64, 2, torch.bfloat16),
    (1, 8, 0, 14, 2, 64, 5, torch.bfloat16),
    (1, 8, 8, 64, 8, 128, 4, torch.bfloat16),
    (1, 8, 8, 8, 4, 64, 4, torch.bfloat16),
    (1, 3, 0, 3, 1, 128, 3, torch.bfloat16),
    # the EOS kernel at both of its limits: k + k' = 32 and G = 16
    (1, 16, 16, 16, 1, 64, 3, torch.bfloat16),
    # G = 16 at d = 128: two Q units per lane and a 16-row output block
    (1, 8, 8, 32, 2, 128, 3, torch.bfloat16),
    (100, 8, 0, 14, 2, 64, 2, torch.bfloat16),
    (70, 64, 0, 4, 2, 128, 2, torch.bfloat16),
    (1, 8, 0, 14, 2, 64, 3, torch.float32),
    (7, 8, 8, 16, 2, 128, 3, torch.float32),
    (64, 8, 0, 14, 2, 64, 2, torch.float32),
    (5, 2, 0, 32, 1, 64, 2, torch.float32),
    # one past the MFMA kernel's ell limit, and the largest ell accepted
    (65, 8, 0, 14, 2, 64, 2, torch.bfloat16),
    (1024, 8, 0, 4, 1, 64, 1, torch.bfloat16),
    (1024, 64, 0, 2, 1, 128, 1, torch.float32),
]


@pytest.mark.parametrize("shape", VALU_SHAPES,
                         ids=lambda s: "ell%d_k%d_kq%d_hq%d_h%d_d%d_%s" % (*s[:6], str(s[7])[6:]))
def test_valu_path_shapes(shape):
    ell, k, kq, hq, h, d, P, dtype = shape
    qids = (torch.arange(P) * 3) % 2 if kq else None
    case = GistCase(2, 6, k, ell, hq, h, d, P, dtype, 200 + ell, kq=kq, n_qrows=2, q_ids=qids)
    check_gist(case, label=f"valu {shape}")


# ---------------------------------------------------------------------------
# Full-size workloads (sampled pairs)
# ---------------------------------------------------------------------------


def _ids(wl, device="cuda"):
    return synth.item_ids_per_query(wl.queries, wl.pairs // wl.queries, wl.n_items, wl.seed, device)


def test_single_layer_workload_all_pairs():
    wl = synth.SINGLE_LAYER
    case = GistCase(1, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype, wl.seed,
                    ids=_ids(wl))
    check_gist(case, label="single layer, 500 pairs (all checked)")


@pytest.mark.parametrize("wl", [synth.L24_B500, synth.L24_B2000], ids=["b500", "b2000"])
def test_24_layer_workload_sampled(wl):
    case = GistCase(wl.layers, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype,
                    wl.seed, ids=_ids(wl))
    rng = np.random.default_rng(wl.seed)
    sample = np.unique(np.concatenate([[0, wl.pairs - 1], rng.integers(0, wl.pairs, 6)]))
    check_gist(case, sample=sample, label=f"24 layers, {wl.pairs} pairs (sampled)")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("hq", [14, 16], ids=["G7", "G8"])
def test_several_workgroup_generations_sampled(hq, fp8):
    # 700 pairs x 2 KV heads = 1400 workgroups: more than the GPU holds at
    # once, which selects the deeper Q prefetch of the unrolled instances
    # (bf16 and fp8 pools each have their own)
    case = GistCase(1, 3000, 8, 64, hq, 2, 64, 700, torch.bfloat16, 321 + hq, fp8=fp8)
    sample = np.array([0, 1, 349, 511, 512, 698, 699])
    check_gist(case, sample=sample, label=f"700 pairs, Hq={hq}, {'fp8' if fp8 else 'bf16'} pool (sampled)")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("hq", [14, 16], ids=["G7", "G8"])
def test_single_and_multi_generation_instances_agree_bitwise(hq, fp8):
    # The same pairs through the single-generation instance (300 pairs x 2
    # KV heads = 600 workgroups, all resident: one head of Q before the
    # staging, three after it, wave priorities by remaining work) and, as the
    # first 300 of 700 pairs, through the several-generation one (two heads
    # of Q, the hardware's issue order).  Only the schedule differs, so the
    # rows must be identical bit for bit.
    big = GistCase(1, 3000, 8, 64, hq, 2, 64, 700, torch.bfloat16, 611 + hq, fp8=fp8)
    n = 300
    ids = big.ids[:n].contiguous()
    q, kn, vn = (t[0][:n].contiguous() for t in (big.q, big.kn, big.vn))
    small = G.gist_attn_forward(big.pool, 0, ids, q, kn, vn, big.pos0, 10000.0, big.scale)
    full = big.run(0)
    torch.cuda.synchronize()
    assert torch.equal(small.view(torch.int16), full[:n].view(torch.int16))
    assert torch.isfinite(full.float()).all()


def _wide_sample(wl, seed):
    # 32 seeded pairs plus the first and last two
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, wl.pairs - 2, wl.pairs - 1],
                                     rng.choice(wl.pairs, 32, replace=False)]))


def test_wide_ell64_workload_sampled():
    wl = synth.WIDE_ELL64
    # the whole 28-layer pool (92 GB: layer 27's records lie past 2^31
    # elements), activations for the first and the last layer
    case = GistCase(wl.layers, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype,
                    wl.seed, ids=_ids(wl), act_layers=[0, wl.layers - 1])
    check_gist(case, sample=_wide_sample(wl, 31), label="wide ell=64, 2000 pairs, layers 0 and 27 (sampled)")


def test_wide_ell64_fp8_workload_sampled():
    wl = synth.WIDE_ELL64_FP8
    case = GistCase(wl.layers, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype,
                    wl.seed, ids=_ids(wl), fp8=True, act_layers=[0, wl.layers - 1])
    check_gist(case, sample=_wide_sample(wl, 32),
               label="wide ell=64 over fp8 pools, 2000 pairs, layers 0 and 27 (sampled)")


def test_wide_eos_query_gist_workload():
    wl = synth.WIDE_EOS
    qids = torch.arange(wl.pairs) // (wl.pairs // wl.queries)
    case = GistCase(wl.layers, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype,
                    wl.seed, kq=wl.kq, n_qrows=wl.queries, ids=_ids(wl), q_ids=qids,
                    act_layers=[0, wl.layers - 1])
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([[0, wl.pairs - 1], rng.integers(0, wl.pairs, 62)]))
    check_gist(case, sample=sample, label="wide EOS over item+query gist, 2000 pairs")


# ---------------------------------------------------------------------------
# Paged decode
# ---------------------------------------------------------------------------


def test_paged_decode_workload():
    wl = synth.PAGED
    n_blocks = wl.requests * wl.blocks_per_request
    worst = 0.0
    for layer in (0, wl.layers - 1):
        case = DecodeCase(n_blocks, wl.h, wl.block_size, wl.d, wl.hq, [wl.context] * wl.requests,
                          wl.dtype, synth.tensor_seed(wl.seed, 0, layer),
                          table=synth.block_table(wl.requests, wl.blocks_per_request, n_blocks,
                                                  wl.seed, "cuda"))
        out = case.run()
        torch.cuda.synchronize()
        err = float(np.abs(f64(out) - case.oracle()).max())
        worst = max(worst, err)
        assert err <= TOL[wl.dtype], f"layer {layer}: {err}"
        del case, out
    say(f"paged decode 32x4096: max-abs err {worst:.3g}")


DECODE_SHAPES = [
    # hq, h, d, bs, lens, dtype
    (32, 32, 128, 256, [4096, 0, 1, 255, 256, 257, 4000], torch.bfloat16),
    (8, 2, 64, 16, [0, 15, 16, 17, 100, 333], torch.bfloat16),
    (28, 4, 128, 64, [1, 64, 129, 900], torch.bfloat16),
    (4, 4, 64, 32, [0, 31, 32, 77, 500], torch.float32),
    (16, 2, 128, 256, [1, 300, 1000], torch.float32),
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "hq%d_h%d_d%d_bs%d" % s[:4] + "_" + str(s[5])[6:])
def test_paged_decode_shapes(shape):
    hq, h, d, bs, lens, dtype = shape
    max_blocks = -(-max(lens) // bs) + 1  # one spare table column
    n_blocks = len(lens) * max_blocks + 5
    case = DecodeCase(n_blocks, h, bs, d, hq, lens, dtype, 300 + d, max_blocks=max_blocks)
    out = case.run()
    torch.cuda.synchronize()
    err = float(np.abs(f64(out) - case.oracle()).max())
    say(f"decode {shape[:4]} {str(dtype)}: max-abs err {err:.3g}")
    assert err <= TOL[dtype]


# ---------------------------------------------------------------------------
# Error behaviour and determinism
# ---------------------------------------------------------------------------


def test_out_of_range_ids_give_nan_rows_only():
    case = GistCase(1, 5, 8, 16, 14, 2, 64, 4, torch.bfloat16, 401,
                    ids=torch.tensor([0, -1, 5, 3]))
    out = case.run(0)
    torch.cuda.synchronize()
    o = f64(out)
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all()
    assert np.isfinite(o[0]).all() and np.isfinite(o[3]).all()
    assert case.max_err(0, out, [0, 3]) <= 2e-2
    # the VALU path (ell = 1) does the same
    case1 = GistCase(1, 5, 8, 1, 14, 2, 64, 3, torch.bfloat16, 402, ids=torch.tensor([7, 1, 2]))
    o1 = f64(case1.run(0))
    assert np.isnan(o1[0]).all() and np.isfinite(o1[1:]).all()


def test_bad_block_table_entry_gives_nan_for_that_request():
    case = DecodeCase(40, 2, 16, 64, 4, [30, 30, 30], torch.bfloat16, 403)
    case.table[1, 1] = 1000
    o = f64(case.run())
    assert np.isnan(o[1]).all()
    ok = [0, 2]
    assert np.abs(o[ok] - case.oracle(ok)).max() <= 2e-2


def test_bitwise_deterministic_reruns():
    case = GistCase(1, 50, 8, 64, 14, 2, 64, 64, torch.bfloat16, 404)
    a = case.run(0).clone()
    b = case.run(0).clone()
    assert torch.equal(a, b)
    dc = DecodeCase(64, 4, 256, 128, 8, [1000, 2000, 17], torch.bfloat16, 405)
    assert torch.equal(dc.run().clone(), dc.run().clone())


def test_hip_graph_capture_replays_match_eager():
    # A 24-layer pass of l = 64 calls (the single-generation instance), an
    # l = 1 call with a query gist (the EOS kernel) and a paged decode step
    # (split and combine kernels), captured once into a HIP graph.  The library allocates nothing and issues no memsets, so the
    # calls capture as plain kernel launches.  Each replay, with eager work on
    # the outputs in between, must give the eager rows bit for bit.
    case = GistCase(24, 500, 8, 64, 14, 2, 64, 40, torch.bfloat16, 771)
    eos = GistCase(1, 60, 8, 1, 64, 8, 128, 48, torch.bfloat16, 772, kq=8, n_qrows=3,
                   q_ids=torch.arange(48) % 3)
    dc = DecodeCase(64, 4, 256, 128, 8, [1000, 2000, 17], torch.bfloat16, 773)
    eager = [case.run(li).clone() for li in range(24)] + [eos.run(0).clone(), dc.run().clone()]
    torch.cuda.synchronize()
    outs = [torch.empty_like(o) for o in eager]
    ws = torch.empty(G.paged_decode_workspace_bytes(3, 8, dc.table.shape[1], 256, 128),
                     dtype=torch.uint8, device="cuda")

    def calls():
        for li in range(24):
            case.run(li, out=outs[li])
        eos.run(0, out=outs[24])
        dc.run(out=outs[25], workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the first calls on the capture stream run eagerly
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}"


def test_calls_on_concurrent_streams_match_sequential():
    # The library keeps no device state between calls (the paged decode
    # scratch of the allocation-free entry point aside), so calls in flight on
    # several streams at once give the rows they give one after the other.
    case = GistCase(4, 500, 8, 64, 14, 2, 64, 300, torch.bfloat16, 781)
    eos = GistCase(1, 60, 8, 1, 64, 8, 128, 200, torch.bfloat16, 782, kq=8, n_qrows=4,
                   q_ids=torch.arange(200) % 4)
    seq = [case.run(li).clone() for li in range(4)] + [eos.run(0).clone()]
    torch.cuda.synchronize()
    outs = [torch.full_like(o, float("nan")) for o in seq]
    streams = [torch.cuda.Stream() for _ in range(5)]
    torch.cuda.synchronize()
    for i, st in enumerate(streams):
        if i < 4:
            G.gist_attn_forward(case.pool, i, case.ids, case.q[i], case.kn[i], case.vn[i],
                                case.pos0, 10000.0, case.scale, out=outs[i], stream=st)
        else:
            G.gist_attn_forward(eos.pool, 0, eos.ids, eos.q[0], eos.kn[0], eos.vn[0], eos.pos0,
                                10000.0, eos.scale, qpool=eos.qpool, q_ids=eos.q_ids,
                                out=outs[4], stream=st)
    torch.cuda.synchronize()
    for o, e in zip(outs, seq):
        assert torch.equal(o.view(torch.int16), e.view(torch.int16))


def test_empty_batch_is_a_noop():
    import gist_compressed_kv_amd as G
    case = GistCase(1, 3, 8, 16, 4, 1, 64, 1, torch.bfloat16, 406)
    e = torch.empty((0, 16, 4, 64), dtype=torch.bfloat16, device="cuda")
    ek = torch.empty((0, 16, 1, 64), dtype=torch.bfloat16, device="cuda")
    out = G.gist_attn_forward(case.pool, 0, torch.empty(0, dtype=torch.int32, device="cuda"), e,
                              ek, ek)
    assert out.shape == (0, 16, 4, 64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("src_pos0", [1, 38])
def test_pool_write_matches_oracle(dtype, src_pos0):
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    L, N, k, h, d, n = 2, 9, 8, 2, 128, 4
    pool_t = torch.zeros((L, N, 2, h, k, d), dtype=dtype, device="cuda")
    pool = G.GistPool(pool_t)
    ids = torch.tensor([3, 0, 8, 5], dtype=torch.int32, device="cuda")
    ks = synth.randn((n, k, h, d), 500, dtype, "cuda")
    vs = synth.randn((n, k, h, d), 501, dtype, "cuda")
    G.gist_pool_write(pool, 1, ids, ks, vs, src_pos0=src_pos0, rope_base=10000.0)
    torch.cuda.synchronize()
    ref = O.pool_write(np.zeros((L, N, 2, h, k, d)), 1, ids.cpu().numpy(), f64(ks), f64(vs),
                       src_pos0, 10000.0)
    got = f64(pool_t)
    # bf16 storage rounds the re-rotated K once (half an ulp, <= 2^-9 relative)
    tol = 1e-6 if dtype == torch.float32 else 2.0 ** -8 * np.abs(ref).max()
    assert np.abs(got - ref).max() <= tol
    if src_pos0 == 1:
        assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# Positions at the int32 limit: the kernels form pos0 + t (and the pool
# writer 1 - src_pos0) in double, so positions past 2^31 - 1 are rotated by
# their true angle, as the oracle does with int64 positions.
# ---------------------------------------------------------------------------

INT32_MAX = 2 ** 31 - 1


@pytest.mark.parametrize("ell,last", [(16, False), (16, True), (100, False), (100, True), (1, False)],
                         ids=["mfma", "mfma_last", "valu", "valu_last", "eos"])
def test_positions_past_int32_limit(ell, last):
    case = GistCase(1, 5, 8, ell, 14, 2, 64, 3, torch.bfloat16, 900 + ell)
    case.pos0 = INT32_MAX - ell // 2  # the last positions lie past 2^31 - 1
    if not last:
        check_gist(case, label=f"pos0 {case.pos0}, ell {ell}")
        return
    out = case.run_last(0)
    torch.cuda.synchronize()
    ref = case.oracle(0, np.arange(case.pairs))[:, -1]
    err = float(np.abs(f64(out) - ref).max())
    say(f"pos0 {case.pos0}, ell {ell}, last token: max-abs err {err:.3g}")
    assert err <= TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_pool_write_at_int32_min_position(dtype):
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    L, N, k, h, d, n = 1, 4, 8, 2, 64, 3
    src_pos0 = -2 ** 31  # re-rotation by 1 - src_pos0 = 2^31 + 1
    pool_t = torch.zeros((L, N, 2, h, k, d), dtype=dtype, device="cuda")
    pool = G.GistPool(pool_t)
    ids = torch.tensor([2, 0, 3], dtype=torch.int32, device="cuda")
    ks = synth.randn((n, k, h, d), 510, dtype, "cuda")
    vs = synth.randn((n, k, h, d), 511, dtype, "cuda")
    G.gist_pool_write(pool, 0, ids, ks, vs, src_pos0=src_pos0, rope_base=10000.0)
    torch.cuda.synchronize()
    ref = O.pool_write(np.zeros((L, N, 2, h, k, d)), 0, ids.cpu().numpy(), f64(ks), f64(vs),
                       src_pos0, 10000.0)
    got = f64(pool_t)
    if dtype == torch.float32:
        # the angle (2^31 + 1) * theta carries up to 2^-52 of itself in fp64
        # on either side: 2^-51 * 2^31 rad per unit of |x|, on top of the 1e-6
        # of the fp32 rotation at small angles
        tol = 1e-6 + 2.0 ** -51 * (2.0 ** 31 + 1) * np.abs(f64(ks)).max()
    else:
        tol = 2.0 ** -8 * np.abs(ref).max()
    assert np.abs(got - ref).max() <= tol


# ---------------------------------------------------------------------------
# Robustness: peaky softmax (Q scaled by 8) and outlier K channels (x10).
# The oracle reads the same scaled device tensors back and is exact (fp64
# RoPE and attention); every path is held to 2e-2 against it.  With logits
# this large, rounding the rotated Q and new K to bf16 alone would move the
# outputs by more than that: the MFMA paths carry them as bf16 pairs hi + lo,
# paged decode keeps them in fp32.
# ---------------------------------------------------------------------------

OUTLIER_CH = [3, 17, 40]


def _boost(case, layer, peaky, outliers):
    if peaky:
        case.q[layer].mul_(8)  # a power of two: exact in bf16
    if outliers:
        case.kn[layer][..., OUTLIER_CH] *= 10
        case.pool_t[layer][:, 0, :, :, OUTLIER_CH] *= 10  # K half of every record


@pytest.mark.parametrize("peaky,outliers", [(True, False), (False, True), (True, True)],
                         ids=["peaky", "outlier_k", "both"])
def test_robust_mfma(peaky, outliers):
    case = GistCase(1, 40, 8, 64, 14, 2, 64, 24, torch.bfloat16, 501)
    _boost(case, 0, peaky, outliers)
    check_gist(case, label=f"mfma robust peaky={peaky} outliers={outliers}")


@pytest.mark.parametrize("peaky,outliers", [(True, False), (False, True), (True, True)],
                         ids=["peaky", "outlier_k", "both"])
def test_robust_eos(peaky, outliers):
    qids = torch.arange(8) % 2
    case = GistCase(1, 30, 8, 1, 64, 8, 128, 8, torch.bfloat16, 502, kq=8, n_qrows=2, q_ids=qids)
    _boost(case, 0, peaky, outliers)
    if outliers:
        case.qpool_t[0][:, 0, :, :, OUTLIER_CH] *= 10
    check_gist(case, label=f"eos robust peaky={peaky} outliers={outliers}")


def test_robust_paged_decode():
    case = DecodeCase(48, 4, 256, 128, 8, [1500, 777, 3000], torch.bfloat16, 503)
    case.q.mul_(8)
    case.kc[..., OUTLIER_CH] *= 10
    case.kn[..., OUTLIER_CH] *= 10
    out = case.run()
    torch.cuda.synchronize()
    err = float(np.abs(f64(out) - case.oracle()).max())
    say(f"paged robust: max-abs err {err:.3g}")
    assert err <= TOL[torch.bfloat16]


# ---------------------------------------------------------------------------
# Paged decode over an fp8 (E4M3) cache with per-(block, head) scales.  The
# oracle decodes the same codes exactly, so the bar is the bf16 one.
# ---------------------------------------------------------------------------

FP8_SHAPES = [
    # n_blocks, h, bs, d, hq, lens
    (70, 4, 256, 128, 4, [4096 - 7, 1, 255, 257]),
    (70, 2, 64, 64, 8, [640, 1000, 0, 16]),
    (80, 8, 16, 128, 32, [120, 384, 33]),
    (30, 1, 128, 64, 2, [1500, 77]),
]


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "h%d_bs%d_d%d_hq%d" % s[1:5])
def test_paged_decode_fp8_shapes(shape):
    n_blocks, h, bs, d, hq, lens = shape
    max_blocks = max(1, -(-max(lens) // bs))
    case = DecodeCase(n_blocks, h, bs, d, hq, lens, torch.bfloat16, 600 + d + hq, fp8=True,
                      max_blocks=max_blocks)
    out = case.run()
    torch.cuda.synchronize()
    err = float(np.abs(f64(out) - case.oracle()).max())
    say(f"paged fp8 {shape[:5]}: max-abs err {err:.3g}")
    assert err <= TOL[torch.bfloat16]


def test_paged_decode_fp8_workload():
    wl = synth.PAGED_FP8
    n_blocks = wl.requests * wl.blocks_per_request
    case = DecodeCase(n_blocks, wl.h, wl.block_size, wl.d, wl.hq, [wl.context] * wl.requests,
                      wl.dtype, wl.seed, fp8=True)
    out = case.run()
    torch.cuda.synchronize()
    err = float(np.abs(f64(out) - case.oracle()).max())
    say(f"paged fp8 workload (one layer, all 32 requests): max-abs err {err:.3g}")
    assert err <= TOL[torch.bfloat16]


def test_paged_decode_fp8_bad_block_is_nan():
    case = DecodeCase(20, 2, 64, 64, 4, [200, 200], torch.bfloat16, 604, fp8=True)
    case.table[1, 1] = 999  # out of range for request 1 only
    out = case.run().float()
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all() and torch.isfinite(out[0]).all()
    err = float(np.abs(f64(out[0:1]) - case.oracle([0])).max())
    assert err <= TOL[torch.bfloat16]



# ---------------------------------------------------------------------------
# fp8 (E4M3) gist pools: the EOS kernel decodes each gist row, scales it by
# its (item or query, K or V, head) scale and rounds it to bf16 on load.  The
# oracle decodes the same codes exactly (fp64), so the comparison is the bf16
# one; quantization error is not part of it.
# ---------------------------------------------------------------------------

EOS_FP8_SHAPES = [
    # k, kq, hq, h, d, pairs
    (8, 8, 64, 8, 128, 40),
    (8, 0, 14, 2, 64, 30),
    (12, 12, 16, 2, 128, 9),
    (20, 0, 8, 1, 64, 7),
    (3, 0, 3, 1, 128, 5),
    (16, 16, 32, 2, 64, 11),
    (1, 0, 1, 1, 64, 3),
    (8, 8, 32, 2, 128, 5),
]


@pytest.mark.parametrize("shape", EOS_FP8_SHAPES,
                         ids=lambda s: "k%d_kq%d_hq%d_h%d_d%d_p%d" % s)
def test_eos_fp8_pool_shapes(shape):
    k, kq, hq, h, d, P = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(2, 7, k, 1, hq, h, d, P, torch.bfloat16, 600 + k + kq + hq, kq=kq, n_qrows=3,
                    q_ids=qids, fp8=True)
    check_gist(case, label=f"eos fp8 {shape}")


def test_wide_eos_fp8_workload_sampled():
    wl = synth.WIDE_EOS_FP8
    qids = torch.arange(wl.pairs) // (wl.pairs // wl.queries)
    case = GistCase(wl.layers, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype,
                    wl.seed, kq=wl.kq, n_qrows=wl.queries, ids=_ids(wl), q_ids=qids, fp8=True,
                    act_layers=[0, wl.layers - 1])
    rng = np.random.default_rng(8)
    sample = np.unique(np.concatenate([[0, wl.pairs - 1], rng.integers(0, wl.pairs, 62)]))
    check_gist(case, sample=sample, label="wide EOS, fp8 item+query gist, 2000 pairs")


# The ell >= 2 (MFMA) kernel over fp8 pools: codes decoded exactly into the
# bf16 rows it stages, K scales on the gist logits, V scales on the gist
# weights of the P·V product.
MFMA_FP8_SHAPES = [
    # k, kq, ell, hq, h, d, pairs
    (8, 0, 64, 14, 2, 64, 40),    # the b500 shape
    (8, 0, 64, 64, 8, 128, 6),    # the wide ell = 64 shape
    (8, 8, 16, 64, 8, 128, 9),    # item + query gist, d = 128
    (17, 0, 40, 12, 3, 64, 7),    # gist keys over two key tiles
    (20, 12, 64, 16, 2, 64, 5),   # 96 keys: the 128-key instance, d = 64
    (16, 16, 60, 8, 1, 128, 4),   # 92 keys: the 128-key instance, d = 128
    (3, 0, 2, 8, 1, 64, 5),       # ell = 2
]


@pytest.mark.parametrize("shape", MFMA_FP8_SHAPES,
                         ids=lambda s: "k%d_kq%d_ell%d_hq%d_h%d_d%d_p%d" % s)
def test_mfma_fp8_pool_shapes(shape):
    k, kq, ell, hq, h, d, P = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(2, 7, k, ell, hq, h, d, P, torch.bfloat16, 640 + k + kq + ell, kq=kq, n_qrows=3,
                    q_ids=qids, fp8=True)
    check_gist(case, label=f"mfma fp8 {shape}")


def test_robust_mfma_fp8_pool():
    # fp8 gist pool: the staged gist K (decoded code times scale) is carried
    # as a bf16 pair like the new keys, so peaky Q and outlier new-K channels
    # stay within the bar against the oracle over the decoded pool
    case = GistCase(1, 40, 8, 64, 14, 2, 64, 24, torch.bfloat16, 504, fp8=True)
    case.q[0].mul_(8)
    case.kn[0][..., OUTLIER_CH] *= 10
    check_gist(case, label="mfma fp8 pool robust (peaky, outlier new K)")


@pytest.mark.parametrize("shape", [MFMA_FP8_SHAPES[0], MFMA_FP8_SHAPES[2]],
                         ids=lambda s: "k%d_kq%d_ell%d_hq%d_h%d_d%d_p%d" % s)
def test_mfma_fp8_last_token_equals_last_row(shape):
    k, kq, ell, hq, h, d, P = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(1, 7, k, ell, hq, h, d, P, torch.bfloat16, 660 + ell, kq=kq, n_qrows=3,
                    q_ids=qids, fp8=True)
    full = case.run(0).clone()
    last = case.run_last(0)
    torch.cuda.synchronize()
    assert torch.equal(last, full[:, -1])
    ref = case.oracle(0, np.arange(P))[:, -1]
    assert float(np.abs(f64(last) - ref).max()) <= 2e-2


@pytest.mark.parametrize("scales", ["k", "v", "kv"])
@pytest.mark.parametrize("shape", [MFMA_FP8_SHAPES[0], MFMA_FP8_SHAPES[2], MFMA_FP8_SHAPES[4],
                                   (8, 8, 1, 64, 8, 128, 9), (8, 0, 1, 14, 2, 64, 11)],
                         ids=lambda s: "k%d_kq%d_ell%d_hq%d_h%d_d%d_p%d" % s)
def test_fp8_pool_with_power_of_two_scales_equals_bf16_pool(shape, scales):
    # with every scale a power of two, scaling the logits and weights commutes
    # with every rounding, so an fp8 pool must give the bf16 pool of its
    # decoded values bit for bit (the ell = 1 shapes run the EOS kernel)
    import gist_compressed_kv_amd as G
    from gpu_cases import ROPE_BASE
    k, kq, ell, hq, h, d, P = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(1, 7, k, ell, hq, h, d, P, torch.bfloat16, 680 + ell + hq, kq=kq, n_qrows=3,
                    q_ids=qids, fp8=True)
    ks = 2.0 ** -7 if "k" in scales else 1.0
    vs = 2.0 ** -6 if "v" in scales else 1.0
    bf = []
    for pl in [case.pool] + ([case.qpool] if case.qpool is not None else []):
        pl.scales[:, :, 0].fill_(ks)
        pl.scales[:, :, 1].fill_(vs)
        vals = pl.codes.view(torch.float8_e4m3fn).float()
        vals[:, :, 0] *= ks
        vals[:, :, 1] *= vs
        bf.append(G.GistPool(vals.to(torch.bfloat16).contiguous()))
    o8 = case.run(0).clone()
    ob = G.gist_attn_forward(bf[0], 0, case.ids, case.q[0], case.kn[0], case.vn[0], case.pos0,
                             ROPE_BASE, case.scale, qpool=bf[1] if kq else None, q_ids=case.q_ids)
    torch.cuda.synchronize()
    assert torch.equal(o8, ob)


@pytest.mark.parametrize("shape", [(8, 8, 1, 64, 8, 128, 9), (8, 8, 1, 16, 2, 64, 5),
                                   (8, 8, 64, 64, 8, 128, 3), (8, 0, 64, 14, 2, 64, 5)],
                         ids=lambda s: "k%d_kq%d_ell%d_hq%d_h%d_d%d_p%d" % s)
def test_fp8_pool_every_finite_code_equals_bf16_pool(shape):
    # every finite E4M3 code (both signs, the subnormals 0x01-0x07, +-448) in
    # every gist record, K and V, at unit scales: the fp8 pool must give the
    # bf16 pool of its decoded values (torch's decode) bit for bit, so each
    # code decodes exactly, on the EOS kernel (ell = 1) and the ell >= 2 one
    import gist_compressed_kv_amd as G
    from gpu_cases import ROPE_BASE
    k, kq, ell, hq, h, d, P = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(1, 7, k, ell, hq, h, d, P, torch.bfloat16, 690 + ell + hq, kq=kq, n_qrows=3,
                    q_ids=qids, fp8=True)
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    bf = []
    for j, pl in enumerate([case.pool] + ([case.qpool] if case.qpool is not None else [])):
        n = pl.codes.numel()
        # 7 is prime to 254: each run of 254 consecutive elements, hence each
        # K half and each V half of every record, holds every finite code
        idx = (torch.arange(n) * 7 + 13 * j) % 254
        pl.codes.copy_(finite[idx].view(pl.codes.shape).to(pl.codes.device))
        pl.scales.fill_(1.0)
        bf.append(G.GistPool(pl.codes.view(torch.float8_e4m3fn).float().to(torch.bfloat16).contiguous()))
    assert h * min(k, kq or k) * d >= 254
    o8 = case.run(0).clone()
    ob = G.gist_attn_forward(bf[0], 0, case.ids, case.q[0], case.kn[0], case.vn[0], case.pos0,
                             ROPE_BASE, case.scale, qpool=bf[1] if kq else None, q_ids=case.q_ids)
    torch.cuda.synchronize()
    assert torch.isfinite(o8.float()).all()
    assert torch.equal(o8, ob)


def test_mfma_fp8_out_of_range_ids_give_nan_rows_only():
    case = GistCase(1, 6, 8, 64, 14, 2, 64, 5, torch.bfloat16, 670, ids=torch.tensor([0, 6, 2, -1, 5]),
                    fp8=True)
    o = f64(case.run(0))
    torch.cuda.synchronize()
    assert np.isnan(o[[1, 3]]).all() and np.isfinite(o[[0, 2, 4]]).all()
    assert case.max_err(0, case.run(0), [0, 2, 4]) <= 2e-2


def test_eos_fp8_out_of_range_ids_give_nan_rows_only():
    case = GistCase(1, 6, 8, 1, 64, 8, 128, 5, torch.bfloat16, 610, kq=8, n_qrows=2,
                    ids=torch.tensor([0, 6, 2, 5, -3]), q_ids=torch.tensor([0, 1, 2, 1, 0]),
                    fp8=True)
    o = f64(case.run(0))
    torch.cuda.synchronize()
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all() and np.isnan(o[4]).all()
    assert np.isfinite(o[[0, 3]]).all()
    assert case.max_err(0, case.run(0), [0, 3]) <= 2e-2


@pytest.mark.parametrize("src_pos0", [1, 38])
def test_pool_write_fp8_matches_oracle(src_pos0):
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    L, N, k, h, d, n = 2, 9, 8, 2, 128, 4
    st = G.gist_pool_fp8_storage(L, N, k, h, d)
    st.zero_()
    pool = G.GistPool(st, shape=(L, N, k, h, d))
    ids = torch.tensor([3, 0, 8, 5], dtype=torch.int32, device="cuda")
    ks = synth.randn((n, k, h, d), 520, torch.bfloat16, "cuda")
    vs = synth.randn((n, k, h, d), 521, torch.bfloat16, "cuda")
    ks[1, :, 1] = 0          # an all-zero block: scale 1, codes 0
    vs[2, :, 0] *= 1e-4      # small values: subnormal codes
    vs[3, :, 1] *= 300.0     # large values
    G.gist_pool_write(pool, 1, ids, ks, vs, src_pos0=src_pos0, rope_base=10000.0)
    torch.cuda.synchronize()
    rc, rs = O.pool_write_fp8(np.zeros((L, N, 2, h, k, d), np.uint8), np.zeros((L, N, 2, h), np.float32),
                              1, ids.cpu().numpy(), f64(ks), f64(vs), src_pos0, 10000.0)
    gc, gs = pool.codes.cpu().numpy(), pool.scales.cpu().numpy()
    # V blocks and untouched items: bit-exact (the codes are decided in fp32 on both sides)
    assert np.array_equal(gc[:, :, 1], rc[:, :, 1]) and np.array_equal(gs[:, :, 1], rs[:, :, 1])
    assert np.array_equal(gc[0], rc[0]) and not gc[1, [1, 2, 4, 6, 7]].any()
    if src_pos0 == 1:  # no re-rotation: K is bit-exact too
        assert np.array_equal(gc, rc) and np.array_equal(gs, rs)
    else:
        # K is re-rotated in fp32 on the GPU and in fp64 by the oracle: the
        # scales agree to a few ulps, and a code may differ only by one step,
        # where the value sits on the midpoint between the two codes
        kg, kr = gs[1, :, 0], rs[1, :, 0]
        assert np.allclose(kg, kr, rtol=1e-6, atol=0)
        a, b = gc[1, :, 0].astype(np.int64), rc[1, :, 0].astype(np.int64)
        diff = a != b
        say(f"fp8 pool write, src_pos0={src_pos0}: {int(diff.sum())} of {a.size} K codes differ")
        assert diff.sum() <= a.size // 1000
        assert ((a[diff] & 0x80) == (b[diff] & 0x80)).all()
        assert (np.abs((a[diff] & 0x7F) - (b[diff] & 0x7F)) == 1).all()
    # the written pool read by the EOS kernel, against the oracle on its decoded contents
    q = synth.randn((n, 1, 4, d), 522, torch.bfloat16, "cuda")
    kn = synth.randn((n, 1, h, d), 523, torch.bfloat16, "cuda")
    vn = synth.randn((n, 1, h, d), 524, torch.bfloat16, "cuda")
    out = G.gist_attn_forward(pool, 1, ids, q, kn, vn, k + 1, 10000.0, d ** -0.5)
    torch.cuda.synchronize()
    deq = O.dequantize_gist(gc, gs)
    ref = O.gist_attn_forward(deq, 1, ids.cpu().numpy(), f64(q), f64(kn), f64(vn), k + 1, 10000.0,
                              d ** -0.5)
    # outputs are convex combinations of V rows: the error is measured in units
    # of the largest |V| the query head can see (the x300 block makes outputs
    # of a few hundred, whose bf16 rounding alone is about 1)
    vmax = np.maximum(np.abs(deq[1, ids.cpu().numpy(), 1]).max(axis=(2, 3)),
                      np.abs(f64(vn)).max(axis=(1, 3)))                # [n][h]
    vmax = np.repeat(np.maximum(vmax, 1.0), 4 // h, axis=1)[:, None, :, None]  # per query head
    assert (np.abs(f64(out) - ref) / vmax).max() <= 2e-2


# ---------------------------------------------------------------------------
# Offline gist extraction: causal prefill over packed [item ; gist] sequences
# ---------------------------------------------------------------------------

from gpu_cases import ROPE_BASE, PrefillCase  # noqa: E402

PREFILL_SHAPES = [
    # lengths, hq, h, d
    ([1, 2, 16, 31, 32, 33], 4, 2, 64),
    ([127, 128, 129], 14, 2, 64),
    ([300, 5, 257], 8, 1, 128),
    ([200, 64], 16, 2, 128),
    ([97], 7, 7, 64),
]


@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=lambda s: "L%s_hq%d_h%d_d%d" % (
    "-".join(map(str, s[0])), s[1], s[2], s[3]))
def test_prefill_shapes(shape):
    lens, hq, h, d = shape
    case = PrefillCase(lens, hq, h, d, 700 + sum(lens))
    out = case.run()
    torch.cuda.synchronize()
    err = case.max_err(out)
    say(f"prefill {shape}: max-abs err {err:.3g}")
    assert err <= 2e-2


def test_prefill_item_length_workload_sampled():
    wl = synth.PREFILL
    lens = synth.prefill_lengths(wl, "cpu").tolist()
    case = PrefillCase(lens, wl.hq, wl.h, wl.d, wl.seed)
    out = case.run()
    torch.cuda.synchronize()
    seqs = [0, len(lens) // 2, len(lens) - 1]
    err = case.max_err(out, seqs)
    say(f"prefill workload ({len(lens)} items, {case.T} tokens), sequences {seqs}: max-abs err {err:.3g}")
    assert err <= 2e-2


def test_prefill_peaky_softmax_moves_the_running_maximum():
    # Q x 8: logits of tens, so the running maximum moves many times
    case = PrefillCase([400, 77], 8, 2, 64, 711)
    case.q.mul_(8.0)
    out = case.run()
    torch.cuda.synchronize()
    err = case.max_err(out)
    say(f"prefill peaky: max-abs err {err:.3g}")
    assert err <= 2e-2


def test_prefill_outlier_k_channels():
    # three K channels x10 and Q x8: the rotated K must keep its precision too
    case = PrefillCase([300, 41], 8, 2, 64, 713)
    case.q.mul_(8.0)
    case.k[..., OUTLIER_CH] *= 10
    out = case.run()
    torch.cuda.synchronize()
    err = case.max_err(out)
    say(f"prefill peaky + outlier K: max-abs err {err:.3g}")
    assert err <= 2e-2


def test_prefill_writes_the_gist_rows_to_the_pool():
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    lens, kk, h, d = [40, 9, 3, 25], 8, 2, 64
    case = PrefillCase(lens, 4, h, d, 712)
    L, N = 2, 6
    pool_t = torch.zeros((L, N, 2, h, kk, d), dtype=torch.bfloat16, device="cuda")
    pool = G.GistPool(pool_t)
    ids = torch.tensor([4, 0, 2, 9], dtype=torch.int32, device="cuda")  # 9: out of range
    out = case.run(pool=pool, layer=1, item_ids=ids)
    torch.cuda.synchronize()
    assert case.max_err(out) <= 2e-2
    st = case.seq_start.cpu().numpy()
    gk, gv = O.gist_rows_from_prefill(f64(case.k), f64(case.v), st, kk, ROPE_BASE)
    got = f64(pool_t)
    for b, item in [(0, 4), (1, 0)]:
        ref_k = gk[b].transpose(1, 0, 2)
        # K rotated in fp32 and rounded to bf16 once: half an ulp, <= 2^-9 relative
        assert np.abs(got[1, item, 0] - ref_k).max() <= 2.0 ** -8 * np.abs(ref_k).max()
        assert np.array_equal(got[1, item, 1], gv[b].transpose(1, 0, 2))
    # sequence 2 is shorter than k and sequence 3 has an out-of-range id:
    # nothing else was written, and layer 0 is untouched
    assert not got[1, [1, 2, 3, 5]].any() and not got[0].any()


def test_prefill_skips_a_sequence_with_bad_bounds():
    case = PrefillCase([20, 30, 10], 4, 1, 64, 713)
    st = case.seq_start.clone()
    st[2] = st[1] - 1  # sequence 1 ends before it starts; sequence 2 starts early
    out = torch.full_like(case.q, 7.0)
    G_ = __import__("gist_compressed_kv_amd")
    G_.gist_prefill_attn(case.q, case.k, case.v, st, 30, 1e4, case.scale, out=out)
    torch.cuda.synchronize()
    o = f64(out)
    assert (o[20:60] == 7.0).all()  # sequences 1 and 2 (longer than max_len now) skipped
    idx, ref = case.oracle([0])
    assert np.abs(o[idx] - ref).max() <= 2e-2


# ---------------------------------------------------------------------------
# Last token only (the final layer of a scoring pass)
# ---------------------------------------------------------------------------

LAST_SHAPES = [
    # layers, items, k, ell, kq, hq, h, d, pairs, dtype
    (1, 50, 8, 64, 0, 14, 2, 64, 40, torch.bfloat16),    # ell=64 MFMA kernel (b500 shape)
    (1, 9, 8, 17, 8, 16, 2, 128, 9, torch.bfloat16),     # MFMA, query gist, d=128
    (1, 9, 3, 2, 0, 8, 1, 64, 5, torch.bfloat16),        # MFMA, ell=2
    (1, 9, 8, 33, 0, 16, 4, 64, 1200, torch.bfloat16),   # MFMA, several workgroup generations
    (1, 9, 8, 1, 8, 64, 8, 128, 7, torch.bfloat16),      # ell=1: the EOS kernel
    (1, 9, 8, 100, 0, 14, 2, 64, 3, torch.bfloat16),     # VALU kernel (ell > 64)
    (1, 9, 8, 7, 8, 16, 2, 128, 3, torch.float32),       # VALU kernel, fp32
]


@pytest.mark.parametrize("shape", LAST_SHAPES, ids=lambda s: "ell%d_k%d_kq%d_hq%d_h%d_d%d_p%d_%s" % (
    s[3], s[2], s[4], s[5], s[6], s[7], s[8], str(s[9])[6:]))
def test_last_token_only_equals_last_row(shape):
    layers, items, k, ell, kq, hq, h, d, P, dtype = shape
    qids = (torch.arange(P) * 7) % 3 if kq else None
    case = GistCase(layers, items, k, ell, hq, h, d, P, dtype, 800 + ell + hq, kq=kq, n_qrows=3,
                    q_ids=qids)
    full = case.run(0).clone()
    last = case.run_last(0)
    torch.cuda.synchronize()
    # the same kernels compute the last row either way
    assert torch.equal(last, full[:, -1])
    sample = np.arange(P) if P <= 64 else np.unique(np.r_[0, P - 1, np.arange(0, P, 97)])
    ref = case.oracle(0, sample)[:, -1]
    err = float(np.abs(f64(last[torch.as_tensor(sample, device="cuda")]) - ref).max())
    say(f"last token {shape}: max-abs err {err:.3g}")
    assert err <= TOL[dtype]


def test_last_token_only_bad_ids_give_nan_rows():
    case = GistCase(1, 6, 8, 64, 14, 2, 64, 4, torch.bfloat16, 820, ids=torch.tensor([0, 6, 3, -1]))
    o = f64(case.run_last(0))
    torch.cuda.synchronize()
    assert np.isnan(o[[1, 3]]).all() and np.isfinite(o[[0, 2]]).all()


# ---------------------------------------------------------------------------
# Gists read from a paged cache (the decode cache layout)
# ---------------------------------------------------------------------------


def _paged_from_case(case, bs, same_block):
    """The case's layer-0 gists in a paged cache: item gist of pair p in rows
    0..k-1 of block 2p (or p), query gist in rows k.. of the same block or
    rows 0.. of block 2p+1."""
    P, h, d, k, kq = case.pairs, case.h, case.d, case.k, case.kq
    nb = P if same_block else 2 * P
    kc = torch.zeros((nb, h, bs, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ib = torch.arange(P, device="cuda") * (1 if same_block else 2)
    qb = ib if same_block else ib + 1
    q_row0 = k if same_block else 0
    rec = case.pool_t[0][case.ids.long()]  # [P][2][H][k][d]
    kc[ib, :, :k], vc[ib, :, :k] = rec[:, 0], rec[:, 1]
    if kq:
        qrec = case.qpool_t[0][case.q_ids.long()]
        kc[qb, :, q_row0:q_row0 + kq], vc[qb, :, q_row0:q_row0 + kq] = qrec[:, 0], qrec[:, 1]
    return kc, vc, ib.to(torch.int32), qb.to(torch.int32), q_row0


PAGED_GIST_SHAPES = [
    # k, kq, hq, h, d, pairs, block size, same block
    (8, 8, 64, 8, 128, 40, 16, True),     # 8 + 8 gist rows fill one 16-token block
    (8, 8, 64, 8, 128, 40, 16, False),    # item and query gist in separate blocks
    (8, 0, 14, 2, 64, 30, 16, False),
    (12, 12, 16, 2, 128, 9, 32, True),
    (5, 3, 8, 1, 64, 7, 16, False),
]


@pytest.mark.parametrize("shape", PAGED_GIST_SHAPES, ids=lambda s: "k%d_kq%d_hq%d_h%d_d%d_p%d_bs%d_%s" % (
    s[0], s[1], s[2], s[3], s[4], s[5], s[6], "one" if s[7] else "two"))
def test_paged_gist_eos_equals_pooled(shape):
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    k, kq, hq, h, d, P, bs, same = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(1, 11, k, 1, hq, h, d, P, torch.bfloat16, 900 + k + kq + hq, kq=kq, n_qrows=3,
                    q_ids=qids)
    pooled = case.run(0)
    kc, vc, ib, qb, q_row0 = _paged_from_case(case, bs, same)
    paged = G.gist_attn_forward_paged(kc, vc, ib, k, case.q[0][:, 0].contiguous(), case.kn[0][:, 0],
                                      case.vn[0][:, 0], query_blocks=qb if kq else None, kq=kq,
                                      q_row0=q_row0, pos0=case.pos0, scale=case.scale)
    torch.cuda.synchronize()
    # the same kernel reads the same rows through another address
    assert torch.equal(paged, pooled[:, 0])
    pool, qpool = O.paged_gist_pools(f64(kc), f64(vc), ib.cpu().numpy(), k,
                                     qb.cpu().numpy() if kq else None, kq, q_row0)
    ref = O.gist_attn_forward(pool, 0, np.arange(P), f64(case.q[0]), f64(case.kn[0]), f64(case.vn[0]),
                              case.pos0, ROPE_BASE, case.scale, qpool=qpool,
                              q_ids=np.arange(P) if kq else None)[:, 0]
    err = float(np.abs(f64(paged) - ref).max())
    say(f"paged gist {shape}: max-abs err {err:.3g}")
    assert err <= 2e-2


def _paged_fp8_from_case(case, bs):
    """The case's layer-0 fp8 gists in a paged fp8 cache: item gist of pair p
    in rows 0..k-1 of block 2p, query gist in rows 0.. of block 2p+1, each
    block with its gist's (K, V) scales per head."""
    P, h, d, k, kq = case.pairs, case.h, case.d, case.k, case.kq
    kc = torch.zeros((2 * P, h, bs, d), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.ones((2 * P, h), dtype=torch.float32, device="cuda")
    vs = torch.ones_like(ks)
    ib = torch.arange(P, device="cuda") * 2
    qb = ib + 1
    ids = case.ids.long()
    kc[ib, :, :k], vc[ib, :, :k] = case.pool.codes[0, ids, 0], case.pool.codes[0, ids, 1]
    ks[ib], vs[ib] = case.pool.scales[0, ids, 0], case.pool.scales[0, ids, 1]
    if kq:
        qids = case.q_ids.long()
        kc[qb, :, :kq], vc[qb, :, :kq] = case.qpool.codes[0, qids, 0], case.qpool.codes[0, qids, 1]
        ks[qb], vs[qb] = case.qpool.scales[0, qids, 0], case.qpool.scales[0, qids, 1]
    return kc, vc, ks, vs, ib.to(torch.int32), qb.to(torch.int32)


@pytest.mark.parametrize("shape", [s for s in PAGED_GIST_SHAPES if not s[7]],
                         ids=lambda s: "k%d_kq%d_hq%d_h%d_d%d_p%d_bs%d" % s[:7])
def test_paged_gist_fp8_equals_pooled_fp8(shape):
    import gist_compressed_kv_amd as G
    k, kq, hq, h, d, P, bs, _ = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(1, 11, k, 1, hq, h, d, P, torch.bfloat16, 940 + k + kq + hq, kq=kq, n_qrows=3,
                    q_ids=qids, fp8=True)
    pooled = case.run(0)
    kc, vc, ks, vs, ib, qb = _paged_fp8_from_case(case, bs)
    paged = G.gist_attn_forward_paged_fp8(kc, vc, ks, vs, ib, k, case.q[0][:, 0].contiguous(),
                                          case.kn[0][:, 0], case.vn[0][:, 0],
                                          query_blocks=qb if kq else None, kq=kq, pos0=case.pos0,
                                          scale=case.scale)
    torch.cuda.synchronize()
    # the same kernel reads the same codes and scales through other addresses
    assert torch.equal(paged, pooled[:, 0])


def test_paged_gist_fp8_one_block_matches_oracle():
    # item and query gist in one 16-row block share that block's scales
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    P, k, kq, hq, h, d, bs = 9, 8, 8, 32, 4, 128, 16
    kc, ks = synth.randn_fp8_blocks((P + 3, h, bs, d), 951, "cuda")
    vc, vs = synth.randn_fp8_blocks((P + 3, h, bs, d), 952, "cuda")
    ib = torch.tensor([(5 * p + 2) % (P + 3) for p in range(P)], dtype=torch.int32, device="cuda")
    q = synth.randn((P, hq, d), 953, torch.bfloat16, "cuda")
    kn = synth.randn((P, h, d), 954, torch.bfloat16, "cuda")
    vn = synth.randn((P, h, d), 955, torch.bfloat16, "cuda")
    pos0, scale = k + kq + 1, 1.0 / math.sqrt(d)
    out = G.gist_attn_forward_paged_fp8(kc, vc, ks, vs, ib, k, q, kn, vn, query_blocks=ib, kq=kq,
                                        q_row0=k, pos0=pos0, scale=scale)
    torch.cuda.synchronize()
    kf = O.dequantize_blocks(kc.cpu().numpy(), ks.cpu().numpy())
    vf = O.dequantize_blocks(vc.cpu().numpy(), vs.cpu().numpy())
    pool, qpool = O.paged_gist_pools(kf, vf, ib.cpu().numpy(), k, ib.cpu().numpy(), kq, k)
    ref = O.gist_attn_forward(pool, 0, np.arange(P), f64(q)[:, None], f64(kn)[:, None],
                              f64(vn)[:, None], pos0, ROPE_BASE, scale, qpool=qpool,
                              q_ids=np.arange(P))[:, 0]
    err = float(np.abs(f64(out) - ref).max())
    say(f"paged fp8 gist, one block: max-abs err {err:.3g}")
    assert err <= 2e-2


def test_paged_gist_fp8_bad_block_gives_nan_rows():
    import gist_compressed_kv_amd as G
    case = GistCase(1, 11, 8, 1, 16, 2, 64, 4, torch.bfloat16, 960, kq=8, n_qrows=3,
                    q_ids=torch.tensor([0, 1, 2, 0]), fp8=True)
    kc, vc, ks, vs, ib, qb = _paged_fp8_from_case(case, 16)
    ib[1] = 99
    qb[2] = -1
    o = f64(G.gist_attn_forward_paged_fp8(kc, vc, ks, vs, ib, 8, case.q[0][:, 0].contiguous(),
                                          case.kn[0][:, 0], case.vn[0][:, 0], query_blocks=qb, kq=8))
    torch.cuda.synchronize()
    assert np.isnan(o[[1, 2]]).all() and np.isfinite(o[[0, 3]]).all()


def test_paged_gist_bad_block_gives_nan_rows():
    import gist_compressed_kv_amd as G
    case = GistCase(1, 11, 8, 1, 16, 2, 64, 4, torch.bfloat16, 930, kq=8, n_qrows=3,
                    q_ids=torch.tensor([0, 1, 2, 0]))
    kc, vc, ib, qb, q_row0 = _paged_from_case(case, 16, True)
    ib[1] = 99
    qb[2] = -1
    o = f64(G.gist_attn_forward_paged(kc, vc, ib, 8, case.q[0][:, 0].contiguous(), case.kn[0][:, 0],
                                      case.vn[0][:, 0], query_blocks=qb, kq=8, q_row0=8))
    torch.cuda.synchronize()
    assert np.isnan(o[[1, 2]]).all() and np.isfinite(o[[0, 3]]).all()


# ell >= 2: the ell-token kernel reading its gists from the paged cache
PAGED_GIST_ELL_SHAPES = [
    # k, kq, ell, hq, h, d, pairs, block size, same block
    (8, 0, 64, 14, 2, 64, 40, 16, False),    # the 500-pair workload's shape
    (8, 8, 64, 14, 2, 64, 24, 16, True),
    (8, 8, 64, 64, 8, 128, 6, 16, False),    # the wide workload's shape
    (8, 0, 64, 64, 8, 128, 6, 16, True),
    (12, 12, 16, 16, 2, 128, 9, 32, True),
    (20, 12, 37, 8, 1, 64, 5, 32, False),    # ragged key and query tiles
]


def _ell_ids(s):
    return "k%d_kq%d_l%d_hq%d_h%d_d%d_p%d_bs%d_%s" % (*s[:8], "one" if s[8] else "two")


@pytest.mark.parametrize("shape", PAGED_GIST_ELL_SHAPES, ids=_ell_ids)
def test_paged_gist_ell_equals_pooled(shape):
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    k, kq, ell, hq, h, d, P, bs, same = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(1, 11, k, ell, hq, h, d, P, torch.bfloat16, 1000 + k + kq + ell + hq, kq=kq,
                    n_qrows=3, q_ids=qids)
    pooled = case.run(0)
    kc, vc, ib, qb, q_row0 = _paged_from_case(case, bs, same)
    paged = G.gist_attn_forward_paged(kc, vc, ib, k, case.q[0], case.kn[0], case.vn[0],
                                      query_blocks=qb if kq else None, kq=kq, q_row0=q_row0,
                                      pos0=case.pos0, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(paged, pooled)
    pool, qpool = O.paged_gist_pools(f64(kc), f64(vc), ib.cpu().numpy(), k,
                                     qb.cpu().numpy() if kq else None, kq, q_row0)
    ref = O.gist_attn_forward(pool, 0, np.arange(P), f64(case.q[0]), f64(case.kn[0]), f64(case.vn[0]),
                              case.pos0, ROPE_BASE, case.scale, qpool=qpool,
                              q_ids=np.arange(P) if kq else None)
    err = float(np.abs(f64(paged) - ref).max())
    say(f"paged gist ell {shape}: max-abs err {err:.3g}")
    assert err <= 2e-2


@pytest.mark.parametrize("shape", [s for s in PAGED_GIST_ELL_SHAPES if not s[8]], ids=_ell_ids)
def test_paged_gist_ell_fp8_equals_pooled_fp8(shape):
    import gist_compressed_kv_amd as G
    from oracle import gist_oracle as O
    k, kq, ell, hq, h, d, P, bs, _ = shape
    qids = (torch.arange(P) * 5) % 3 if kq else None
    case = GistCase(1, 11, k, ell, hq, h, d, P, torch.bfloat16, 1040 + k + kq + ell + hq, kq=kq,
                    n_qrows=3, q_ids=qids, fp8=True)
    pooled = case.run(0)
    kc, vc, ks, vs, ib, qb = _paged_fp8_from_case(case, bs)
    paged = G.gist_attn_forward_paged_fp8(kc, vc, ks, vs, ib, k, case.q[0], case.kn[0], case.vn[0],
                                          query_blocks=qb if kq else None, kq=kq, pos0=case.pos0,
                                          scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(paged, pooled)
    kf = O.dequantize_blocks(kc.cpu().numpy(), ks.cpu().numpy())
    vf = O.dequantize_blocks(vc.cpu().numpy(), vs.cpu().numpy())
    pool, qpool = O.paged_gist_pools(kf, vf, ib.cpu().numpy(), k, qb.cpu().numpy() if kq else None,
                                     kq, 0)
    ref = O.gist_attn_forward(pool, 0, np.arange(P), f64(case.q[0]), f64(case.kn[0]), f64(case.vn[0]),
                              case.pos0, ROPE_BASE, case.scale, qpool=qpool,
                              q_ids=np.arange(P) if kq else None)
    err = float(np.abs(f64(paged) - ref).max())
    say(f"paged fp8 gist ell {shape}: max-abs err {err:.3g}")
    assert err <= 2e-2


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_paged_gist_ell_bad_block_gives_nan_rows(fp8):
    import gist_compressed_kv_amd as G
    case = GistCase(1, 11, 8, 64, 14, 2, 64, 4, torch.bfloat16, 1090, kq=8, n_qrows=3,
                    q_ids=torch.tensor([0, 1, 2, 0]), fp8=fp8)
    if fp8:
        kc, vc, ks, vs, ib, qb = _paged_fp8_from_case(case, 16)
    else:
        kc, vc, ib, qb, q_row0 = _paged_from_case(case, 16, False)
    ib[1] = 99
    qb[2] = -1
    args = (ib, 8, case.q[0], case.kn[0], case.vn[0])
    o = (G.gist_attn_forward_paged_fp8(kc, vc, ks, vs, *args, query_blocks=qb, kq=8) if fp8 else
         G.gist_attn_forward_paged(kc, vc, *args, query_blocks=qb, kq=8))
    o = f64(o)
    torch.cuda.synchronize()
    assert np.isnan(o[[1, 2]]).all() and np.isfinite(o[[0, 3]]).all()


# ---------------------------------------------------------------------------
# Grouped launch: several calls of one shape in one launch
# ---------------------------------------------------------------------------


def _grouped_vs_calls(case, groups, qpool=None):
    """groups: (layer, P) over the case's activations of that layer (the first
    P pairs).  Runs them as one grouped launch and as one call each; returns
    the grouped outputs after checking them equal to the calls' bit for bit."""
    import gist_compressed_kv_amd as G
    specs = []
    for layer, P in groups:
        spec = {"layer": layer, "item_ids": case.ids[:P], "q": case.q[layer][:P],
                "k_new": case.kn[layer][:P], "v_new": case.vn[layer][:P]}
        if case.qpool is not None:
            spec["q_ids"] = case.q_ids[:P]
        specs.append(spec)
    outs = G.gist_attn_forward_grouped(case.pool, specs, pos0=case.pos0, rope_base=ROPE_BASE,
                                       scale=case.scale, qpool=case.qpool)
    torch.cuda.synchronize()
    for (layer, P), sp, o in zip(groups, specs, outs):
        ref = G.gist_attn_forward(case.pool, layer, sp["item_ids"], sp["q"], sp["k_new"],
                                  sp["v_new"], case.pos0, ROPE_BASE, case.scale, qpool=case.qpool,
                                  q_ids=sp.get("q_ids"))
        torch.cuda.synchronize()
        assert torch.equal(o, ref), (layer, P)
    return outs


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_grouped_24_layer_pool_equals_calls(fp8):
    # the 24-layer, 100k-item pool of the 500-pair workload (layer 23's
    # records lie past 2^31 elements); groups of several sizes, a layer twice
    wl = synth.L24_B500
    case = GistCase(wl.layers, wl.n_items, wl.k, wl.ell, wl.hq, wl.h, wl.d, wl.pairs, wl.dtype,
                    wl.seed + 40, ids=_ids(wl), fp8=fp8, act_layers=[0, 5, 23])
    groups = [(23, 500), (0, 37), (5, 1), (23, 200), (0, 500)]
    outs = _grouped_vs_calls(case, groups)
    sample = np.array([0, 1, 36, 250, 499])
    err = case.max_err(23, outs[0], sample)
    say(f"grouped, layer 23 of 24 ({'fp8' if fp8 else 'bf16'}): max-abs err {err:.3g}")
    assert err <= TOL[torch.bfloat16]


def test_grouped_query_gist_and_many_groups():
    # k' = 8 query gists; 32 groups (the most one launch takes), 3 pairs each
    qids = torch.arange(60) % 4
    case = GistCase(6, 50, 8, 24, 16, 2, 128, 60, torch.bfloat16, 1200, kq=8, n_qrows=4,
                    q_ids=qids)
    groups = [(i % 6, 3 + (i % 5) * 10) for i in range(32)]
    outs = _grouped_vs_calls(case, groups)
    err = max(case.max_err(layer, o, np.arange(P)) for (layer, P), o in zip(groups[:6], outs[:6]))
    say(f"grouped, 32 groups with query gists: max-abs err {err:.3g}")
    assert err <= TOL[torch.bfloat16]


def test_grouped_bad_id_only_touches_its_group():
    import gist_compressed_kv_amd as G
    case = GistCase(2, 11, 8, 64, 14, 2, 64, 6, torch.bfloat16, 1210)
    bad = case.ids.clone()
    bad[2] = 11
    specs = [{"layer": 0, "item_ids": case.ids, "q": case.q[0], "k_new": case.kn[0], "v_new": case.vn[0]},
             {"layer": 1, "item_ids": bad, "q": case.q[1], "k_new": case.kn[1], "v_new": case.vn[1]}]
    o0, o1 = G.gist_attn_forward_grouped(case.pool, specs, pos0=case.pos0, rope_base=ROPE_BASE,
                                         scale=case.scale)
    torch.cuda.synchronize()
    o0, o1 = f64(o0), f64(o1)
    assert np.isfinite(o0).all()
    assert np.isnan(o1[2]).all() and np.isfinite(np.delete(o1, 2, axis=0)).all()


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_grouped_eos_equals_calls(fp8):
    # the EOS step (ell = 1, item gist + query gist + itself) at the wide
    # shape, grouped over layers of a 4-layer pool, groups of several sizes
    qids = torch.arange(300) // 50
    case = GistCase(4, 1000, 8, 1, 64, 8, 128, 300, torch.bfloat16, 1300, kq=8, n_qrows=6,
                    q_ids=qids, fp8=fp8)
    groups = [(3, 300), (0, 17), (2, 1), (3, 64), (1, 300)]
    outs = _grouped_vs_calls(case, groups)
    err = max(case.max_err(layer, o, np.array([0, P // 2, P - 1]))
              for (layer, P), o in zip(groups, outs))
    say(f"grouped EOS ({'fp8' if fp8 else 'bf16'}): max-abs err {err:.3g}")
    assert err <= TOL[torch.bfloat16]


def test_grouped_eos_bad_id_only_touches_its_group():
    import gist_compressed_kv_amd as G
    case = GistCase(2, 11, 8, 1, 16, 2, 64, 5, torch.bfloat16, 1310)
    bad = case.ids.clone()
    bad[3] = -1
    specs = [{"layer": 1, "item_ids": bad, "q": case.q[1], "k_new": case.kn[1], "v_new": case.vn[1]},
             {"layer": 0, "item_ids": case.ids, "q": case.q[0], "k_new": case.kn[0], "v_new": case.vn[0]}]
    o1, o0 = G.gist_attn_forward_grouped(case.pool, specs, pos0=case.pos0, rope_base=ROPE_BASE,
                                         scale=case.scale)
    torch.cuda.synchronize()
    o0, o1 = f64(o0), f64(o1)
    assert np.isfinite(o0).all()
    assert np.isnan(o1[3]).all() and np.isfinite(np.delete(o1, 3, axis=0)).all()
