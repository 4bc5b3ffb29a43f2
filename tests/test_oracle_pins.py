"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden/byte_counts.json), closed forms, invariants, and an
independent library routine (torch's scaled_dot_product_attention on the CPU
in float64).  Page references are by title and section:

* [GIST] liam.page "把 item 压成 KV：gist 能不能用在相关性任务上"
* [KVC]  mcfzz.com "为什么自回归推理缓存 KV，而不缓存历史 Q？"
* [SFX]  icman.com.cn/news/64898 (suffix cache article)
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import gist_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "byte_counts.json")
GIB = 1 << 30


def rng(seed):
    return np.random.default_rng(seed)


def sdpa(q, k, v, **kw):
    """torch SDPA on float64 CPU tensors; q [Hq,T,d], k/v [H,S,d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)[None]
    return F.scaled_dot_product_attention(t(q), t(k), t(v), **kw)[0].numpy()


# ---------------------------------------------------------------------------
# Byte counts printed on the pages
# ---------------------------------------------------------------------------


def test_bytes_per_position_and_item_match_printed_values():
    g = json.load(open(GOLDEN))
    for e in g["per_position"]:
        assert O.kv_bytes_per_position(e["L"], e["H"], e["h"], e["b"]) == e["bytes"]
    for e in g["per_item_gist"]:
        assert O.gist_bytes_per_item(e["L"], e["k"], e["H"], e["h"], e["b"]) == e["bytes"]


def test_pool_totals_match_printed_rounded_values():
    g = json.load(open(GOLDEN))
    for e in g["pool_totals_100k_items_k8"]:
        total = e["items"] * O.gist_bytes_per_item(e["L"], e["k"], e["H"], e["h"], e["b"])
        assert abs(total / GIB - e["gib"]) <= e["rel_tol"] * e["gib"], e
    e = g["pool_total_10M_items_first_shape"]
    total = e["items"] * O.gist_bytes_per_item(e["L"], e["k"], e["H"], e["h"], e["b"])
    assert abs(total / GIB - e["gib"]) <= e["rel_tol"] * e["gib"]


def test_raw_prefix_cost_and_ratio():
    e = json.load(open(GOLDEN))["raw_prefix"]
    per_item = e["tokens"] * O.kv_bytes_per_position(e["L"], e["H"], e["h"], e["b"])
    assert abs(per_item / (1 << 20) - e["per_item_mib"]) <= e["per_item_rel_tol"] * e["per_item_mib"]
    assert abs(per_item * e["items"] / 1e12 - e["total_tb"]) <= e["total_rel_tol"] * e["total_tb"]
    ratio = per_item / O.gist_bytes_per_item(e["L"], 8, e["H"], e["h"], e["b"])
    assert abs(ratio - e["ratio_vs_gist_k8"]) <= e["ratio_rel_tol"] * e["ratio_vs_gist_k8"]


def test_kv_cache_formula_matches_mha_request_example():
    e = json.load(open(GOLDEN))["mha_request_cache"]
    # MHA: one KV head per query head, so H·h equals the hidden size.
    n = O.kv_cache_bytes(e["B"], e["L"], e["T"], 32, e["hidden"] // 32, e["b"])
    assert n == e["bytes"]
    assert n * e["requests"] == e["total_gb_printed"] * GIB
    # the cache formula is the per-position formula times tokens and batch
    assert n == e["T"] * O.kv_bytes_per_position(e["L"], 32, 128, e["b"])


# ---------------------------------------------------------------------------
# RoPE: closed forms and invariants
# ---------------------------------------------------------------------------


def test_rope_identity_at_zero_and_norm_preserved():
    x = rng(0).standard_normal((5, 64))
    assert np.array_equal(O.rope(x, np.zeros(5), 10000.0), x)
    y = O.rope(x, np.arange(5) * 37 + 3, 10000.0)
    # every channel pair (i, i+d/2) keeps its length
    assert np.allclose(x[:, :32] ** 2 + x[:, 32:] ** 2, y[:, :32] ** 2 + y[:, 32:] ** 2,
                       rtol=0, atol=1e-12)


def test_rope_closed_form_values():
    # d = 2: one pair with theta_0 = 1, so position p turns (x, y) by p radians.
    y = O.rope(np.array([[1.0, 0.0]]), [math.pi / 2], 10000.0)
    assert np.allclose(y, [[0.0, 1.0]], atol=1e-15)
    y = O.rope(np.array([[0.0, 1.0]]), [math.pi / 2], 10000.0)
    assert np.allclose(y, [[-1.0, 0.0]], atol=1e-15)
    # d = 4, base 10000: the second pair turns at 10000**(-1/2) = 0.01 rad/pos
    x = np.array([[0.0, 1.0, 0.0, 0.0]])  # channel 1 pairs with channel 3
    p = 50 * math.pi  # 0.01 * p = pi/2
    y = O.rope(x, [p], 10000.0)
    assert np.allclose(y, [[0.0, 0.0, 0.0, 1.0]], atol=1e-12)


def test_rope_equals_complex_multiplication():
    # Pair (i, i+d/2) read as the complex number x_i + 1j*x_{i+d/2} is
    # multiplied by exp(1j * pos * theta_i), with theta_0 = 1 and a constant
    # ratio base**(-2/d) between consecutive frequencies.
    d, base = 16, 500.0
    x = rng(1).standard_normal((3, d))
    pos = np.array([2.0, 11.0, 123.0])
    y = O.rope(x, pos, base)
    ratio = base ** (-2.0 / d)
    theta = ratio ** np.arange(d // 2)
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * theta[None, :])
    assert np.allclose(y[:, : d // 2], z.real, atol=1e-12)
    assert np.allclose(y[:, d // 2:], z.imag, atol=1e-12)


def test_rope_composes_and_depends_only_on_differences():
    r = rng(2)
    x = r.standard_normal((4, 64))
    a = np.array([3.0, 17.0, 100.0, 9.0])
    b = np.array([5.0, 1.0, 2000.0, 0.5])
    assert np.allclose(O.rope(O.rope(x, a, 1e4), b, 1e4), O.rope(x, a + b, 1e4), atol=1e-10)
    q, k = r.standard_normal((2, 64)), r.standard_normal((2, 64))
    for c in (1.0, 7.0, 1000.0):
        d0 = O.rope(q, [12, 12], 1e4) @ O.rope(k, [4, 9], 1e4).T
        d1 = O.rope(q, [12 + c, 12 + c], 1e4) @ O.rope(k, [4 + c, 9 + c], 1e4).T
        assert np.allclose(d0, d1, atol=1e-9)


# ---------------------------------------------------------------------------
# Attention: closed forms and an independent library routine
# ---------------------------------------------------------------------------


def test_single_visible_key_returns_its_value():
    r = rng(3)
    q, k, v = r.standard_normal((1, 8)), r.standard_normal((5, 8)), r.standard_normal((5, 3))
    mask = np.array([[False, False, True, False, False]])
    assert np.array_equal(O.attention(q, k, v, mask, 0.3), v[2:3])


def test_zero_query_gives_mean_of_visible_values_per_row():
    # With q = 0 every visible logit is 0, so o_t is the plain mean of the
    # values that token t may see: all n_gist gist rows and new rows 0..t.
    r = rng(4)
    n_gist, ell, d = 5, 9, 8
    gk, gv = r.standard_normal((n_gist, d)), r.standard_normal((n_gist, d))
    kn, vn = r.standard_normal((ell, d)), r.standard_normal((ell, d))
    out = O.gist_pair_attention(gk, gv, np.zeros((ell, d)), kn, vn, n_gist + 1, 1e4, 0.125)
    for t in range(ell):
        expect = np.vstack([gv, vn[: t + 1]]).mean(axis=0)
        assert np.allclose(out[t], expect, atol=1e-14)


def test_constant_values_pass_through():
    r = rng(5)
    gk, kn, q = r.standard_normal((3, 16)), r.standard_normal((4, 16)), r.standard_normal((4, 16))
    c = r.standard_normal(16)
    out = O.gist_pair_attention(gk, np.tile(c, (3, 1)), q, kn, np.tile(c, (4, 1)), 4, 1e4, 0.25)
    assert np.allclose(out, np.tile(c, (4, 1)), atol=1e-14)


def test_gist_pair_attention_is_last_rows_of_causal_attention():
    # The online sequence [gist ; new] under a plain causal mask gives new
    # token t exactly the gist plus new tokens 0..t.  torch SDPA (float64,
    # is_causal, default scale 1/sqrt(d)) is an independent routine for it.
    r = rng(6)
    n_gist, ell, d = 8, 16, 64
    gk, gv = r.standard_normal((n_gist, d)), r.standard_normal((n_gist, d))
    q, kn, vn = (r.standard_normal((ell, d)) for _ in range(3))
    pos0 = n_gist + 1
    out = O.gist_pair_attention(gk, gv, q, kn, vn, pos0, 1e4, 1 / math.sqrt(d))
    pos = pos0 + np.arange(ell)
    qs = np.vstack([np.zeros((n_gist, d)), O.rope(q, pos, 1e4)])
    ks = np.vstack([gk, O.rope(kn, pos, 1e4)])
    vs = np.vstack([gv, vn])
    ref = sdpa(qs[None], ks[None], vs[None], is_causal=True)[0][n_gist:]
    assert np.allclose(out, ref, atol=1e-12)


def test_no_gist_reduces_to_textbook_causal_attention():
    r = rng(7)
    ell, d = 12, 32
    q, kn, vn = (r.standard_normal((ell, d)) for _ in range(3))
    out = O.gist_pair_attention(np.zeros((0, d)), np.zeros((0, d)), q, kn, vn, 1, 1e4, 1 / math.sqrt(d))
    pos = 1 + np.arange(ell)
    ref = sdpa(O.rope(q, pos, 1e4)[None], O.rope(kn, pos, 1e4)[None], vn[None], is_causal=True)[0]
    assert np.allclose(out, ref, atol=1e-12)


def _random_batch(r, n_items, layers, n_pairs, ell, hq, h, k, d):
    pool = r.standard_normal((layers, n_items, 2, h, k, d))
    ids = r.integers(0, n_items, n_pairs)
    q = r.standard_normal((n_pairs, ell, hq, d))
    kn = r.standard_normal((n_pairs, ell, h, d))
    vn = r.standard_normal((n_pairs, ell, h, d))
    return pool, ids, q, kn, vn


def test_gqa_grouping_matches_library_gqa():
    # SDPA's enable_gqa repeats each KV head over a contiguous block of
    # Hq/H query heads, the grouping the oracle reads as h // (Hq/H).
    r = rng(8)
    n_items, k, ell, hq, h, d = 3, 8, 10, 14, 2, 64
    pool, ids, q, kn, vn = _random_batch(r, n_items, 2, 4, ell, hq, h, k, d)
    out = O.gist_attn_forward(pool, 1, ids, q, kn, vn, k + 1, 1e4, 1 / math.sqrt(d))
    pos = k + 1 + np.arange(ell)
    for p in range(4):
        g = pool[1, ids[p]]
        qs = np.concatenate([np.zeros((hq, k, d)),
                             O.rope(q[p].transpose(1, 0, 2), pos, 1e4)], axis=1)
        ks = np.concatenate([g[0], O.rope(kn[p].transpose(1, 0, 2), pos, 1e4)], axis=1)
        vs = np.concatenate([g[1], vn[p].transpose(1, 0, 2)], axis=1)
        ref = sdpa(qs, ks, vs, is_causal=True, enable_gqa=True)[:, k:, :]
        assert np.allclose(out[p], ref.transpose(1, 0, 2), atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    r = rng(9)
    k, ell, hq, h, d = 8, 6, 8, 2, 16
    pool, ids, q, kn, vn = _random_batch(r, 2, 1, 3, ell, hq, h, k, d)
    out = O.gist_attn_forward(pool, 0, ids, q, kn, vn, k + 1, 1e4, 0.25)
    rep = hq // h
    out_mha = O.gist_attn_forward(np.repeat(pool, rep, axis=3), 0, ids, q,
                                  np.repeat(kn, rep, axis=2), np.repeat(vn, rep, axis=2),
                                  k + 1, 1e4, 0.25)
    assert np.array_equal(out, out_mha)


# ---------------------------------------------------------------------------
# Positions: uniform shift invariance ([GIST] 在线的一次 attention)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("c", [1, 7, 1000, 100000])
def test_uniform_position_shift_leaves_outputs_unchanged(c):
    r = rng(10)
    k, ell, hq, h, d = 8, 16, 4, 1, 64
    gk_raw = r.standard_normal((2, h, k, d))
    pool = np.empty((1, 2, 2, h, k, d))
    pool[0, :, 1] = r.standard_normal((2, h, k, d))
    q, kn, vn = (r.standard_normal((3, ell, n, d)) for n in (hq, h, h))
    ids = [0, 1, 0]
    pool[0, :, 0] = O.rope(gk_raw, 1 + np.arange(k), 1e4)
    base_out = O.gist_attn_forward(pool, 0, ids, q, kn, vn, k + 1, 1e4, 0.125)
    shifted = pool.copy()
    shifted[0, :, 0] = O.rope(gk_raw, 1 + c + np.arange(k), 1e4)
    out = O.gist_attn_forward(shifted, 0, ids, q, kn, vn, k + 1 + c, 1e4, 0.125)
    # fp64 angles of size ~c carry ~c·1e-16 absolute error
    assert np.allclose(out, base_out, rtol=0, atol=max(1e-12, c * 1e-14))
    # while a query numbered from 1 instead of k+1 changes the result
    wrong = O.gist_attn_forward(pool, 0, ids, q, kn, vn, 1, 1e4, 0.125)
    assert np.abs(wrong - base_out).max() > 1e-3


# ---------------------------------------------------------------------------
# The gist mask in the training layout ([GIST] 论文做了什么 / 在线的一次 attention)
# ---------------------------------------------------------------------------


def training_mask(j, k, ell):
    """Causal mask over [item j ; gist k ; query ell] with the block where
    post-gist tokens would read pre-gist tokens removed."""
    n = j + k + ell
    a = np.arange(n)[:, None]
    b = np.arange(n)[None, :]
    return (b <= a) & ~((a >= j + k) & (b < j))


def test_training_layout_matches_compact_online_sequence():
    r = rng(11)
    j, k, ell, d = 20, 8, 12, 64
    n = j + k + ell
    q, kk, v = (r.standard_normal((n, d)) for _ in range(3))
    pos = 1 + np.arange(n)
    m = training_mask(j, k, ell)
    full = O.attention(O.rope(q, pos, 1e4), O.rope(kk, pos, 1e4), v, m, 1 / 8)
    query_rows = full[j + k:]

    # (a) the mask blocks every query -> item path: item K/V are irrelevant
    kk2, v2 = kk.copy(), v.copy()
    kk2[:j] = r.standard_normal((j, d)) * 5
    v2[:j] = r.standard_normal((j, d)) * 5
    full2 = O.attention(O.rope(q, pos, 1e4), O.rope(kk2, pos, 1e4), v2, m, 1 / 8)
    assert np.array_equal(full2[j + k:], query_rows)

    # (b) identical to the compact [gist ; query] sequence, gist stored at
    # 1..k and the query numbered from k+1 (a uniform shift by -j)
    gk = O.rope(kk[j:j + k], 1 + np.arange(k), 1e4)
    compact = O.gist_pair_attention(gk, v[j:j + k], q[j + k:], kk[j + k:], v[j + k:],
                                    k + 1, 1e4, 1 / 8)
    assert np.allclose(compact, query_rows, atol=1e-12)

    # the same rows from SDPA with an explicit boolean mask
    qr, kr = O.rope(q, pos, 1e4), O.rope(kk, pos, 1e4)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a)[None] for a in (qr, kr, v)),
                                         attn_mask=torch.from_numpy(m)[None],
                                         scale=1 / 8)[0].numpy()
    assert np.allclose(ref[j + k:], query_rows, atol=1e-12)

    # (c) negative control: the item left in the sequence as zeros and not
    # masked (the zero-fill trap) gives a different answer
    kz, vz = kk.copy(), v.copy()
    kz[:j] = 0.0
    vz[:j] = 0.0
    causal = np.tril(np.ones((n, n), bool))
    trap = O.attention(O.rope(q, pos, 1e4), O.rope(kz, pos, 1e4), vz, causal, 1 / 8)
    assert np.abs(trap[j + k:] - query_rows).max() > 1e-2


def test_pool_write_rerotates_to_canonical_positions():
    r = rng(12)
    j, k, h, d = 37, 8, 2, 64
    k_raw = r.standard_normal((1, k, h, d))
    v = r.standard_normal((1, k, h, d))
    # K as produced in the training layout: rotated at j+1 .. j+k
    k_train = O.rope(k_raw.transpose(0, 2, 1, 3), j + 1 + np.arange(k), 1e4).transpose(0, 2, 1, 3)
    pool = np.zeros((1, 3, 2, h, k, d))
    pool = O.pool_write(pool, 0, [2], k_train, v, j + 1, 1e4)
    expect = O.rope(k_raw[0].transpose(1, 0, 2), 1 + np.arange(k), 1e4)
    assert np.allclose(pool[0, 2, 0], expect, atol=1e-12)
    assert np.array_equal(pool[0, 2, 1], v[0].transpose(1, 0, 2))
    assert not pool[0, :2].any()


# ---------------------------------------------------------------------------
# Toy two-layer model: offline gist extraction, then the online pass
# ---------------------------------------------------------------------------


def test_two_layer_toy_model_offline_then_online():
    r = rng(13)
    j, k, ell, dm, hq, h, d = 11, 4, 7, 32, 4, 2, 8
    n = j + k + ell
    layers = []
    for _ in range(2):
        layers.append(dict(wq=r.standard_normal((dm, hq * d)) / math.sqrt(dm),
                           wk=r.standard_normal((dm, h * d)) / math.sqrt(dm),
                           wv=r.standard_normal((dm, h * d)) / math.sqrt(dm),
                           wo=r.standard_normal((hq * d, dm)) / math.sqrt(hq * d),
                           w1=r.standard_normal((dm, 2 * dm)) / math.sqrt(dm),
                           w2=r.standard_normal((2 * dm, dm)) / math.sqrt(2 * dm)))
    x0 = r.standard_normal((n, dm))
    scale = 1 / math.sqrt(d)

    def mlp(L, x):
        return np.tanh(x @ L["w1"]) @ L["w2"]

    # training layout: every token in the sequence, gist mask, SDPA
    x = x0.copy()
    pos = 1 + np.arange(n)
    mask = torch.from_numpy(training_mask(j, k, ell))
    stored = []
    for L in layers:
        qh = (x @ L["wq"]).reshape(n, hq, d).transpose(1, 0, 2)
        kh = (x @ L["wk"]).reshape(n, h, d).transpose(1, 0, 2)
        vh = (x @ L["wv"]).reshape(n, h, d).transpose(1, 0, 2)
        # what the offline pass keeps: the gist positions' K (rotated back to
        # 1..k) and V in this layer
        stored.append((O.rope(kh[:, j:j + k], 1 + np.arange(k), 1e4), vh[:, j:j + k]))
        a = F.scaled_dot_product_attention(
            torch.from_numpy(O.rope(qh, pos, 1e4))[None],
            torch.from_numpy(O.rope(kh, pos, 1e4))[None],
            torch.from_numpy(vh)[None], attn_mask=mask[None], scale=scale,
            enable_gqa=True)[0].numpy()
        x = x + a.transpose(1, 0, 2).reshape(n, hq * d) @ L["wo"]
        x = x + mlp(L, x)
    train_rows = x[j + k:]

    # online: only the query tokens, the gist injected as KV, pos0 = k+1
    pool = np.zeros((2, 1, 2, h, k, d))
    for li, (gk, gv) in enumerate(stored):
        pool[li, 0, 0], pool[li, 0, 1] = gk, gv
    x = x0[j + k:].copy()
    for li, L in enumerate(layers):
        qn = (x @ L["wq"]).reshape(1, ell, hq, d)
        kn = (x @ L["wk"]).reshape(1, ell, h, d)
        vn = (x @ L["wv"]).reshape(1, ell, h, d)
        a = O.gist_attn_forward(pool, li, [0], qn, kn, vn, k + 1, 1e4, scale)[0]
        x = x + a.reshape(ell, hq * d) @ L["wo"]
        x = x + mlp(L, x)
    assert np.allclose(x, train_rows, atol=1e-10)


# ---------------------------------------------------------------------------
# Query also compressed: EOS over [item gist ; query gist ; itself]
# ---------------------------------------------------------------------------


def test_query_gist_path_is_last_row_of_causal_attention():
    r = rng(14)
    k, kq, hq, h, d = 8, 8, 8, 2, 32
    pool = r.standard_normal((1, 5, 2, h, k, d))
    qpool = r.standard_normal((1, 3, 2, h, kq, d))
    ids, qids = [4, 1], [2, 0]
    q, kn, vn = (r.standard_normal((2, 1, n, d)) for n in (hq, h, h))
    pos0 = k + kq + 1
    out = O.gist_attn_forward(pool, 0, ids, q, kn, vn, pos0, 1e4, 1 / math.sqrt(d),
                              qpool=qpool, q_ids=qids)
    for p in range(2):
        ks = np.concatenate([pool[0, ids[p], 0], qpool[0, qids[p], 0],
                             O.rope(kn[p].transpose(1, 0, 2), [pos0], 1e4)], axis=1)
        vs = np.concatenate([pool[0, ids[p], 1], qpool[0, qids[p], 1],
                             vn[p].transpose(1, 0, 2)], axis=1)
        qs = O.rope(q[p].transpose(1, 0, 2), [pos0], 1e4)
        ref = sdpa(qs, ks, vs, enable_gqa=True)  # one query row sees all 17 keys
        assert np.allclose(out[p, 0], ref[:, 0], atol=1e-12)


# ---------------------------------------------------------------------------
# Paged decode ([KVC] Reusable-state; [SFX] section 6 problem 4)
# ---------------------------------------------------------------------------


def _paged_from_contiguous(r, kc, vc, bs, extra_blocks=3):
    """Scatter contiguous caches [R][H][T][d] into a shuffled block pool."""
    n_req, h, t, d = kc.shape
    nb = -(-t // bs)
    total = n_req * nb + extra_blocks
    perm = r.permutation(total)
    kpool = r.standard_normal((total, h, bs, d))  # unused rows hold noise
    vpool = r.standard_normal((total, h, bs, d))
    table = np.zeros((n_req, nb), np.int64)
    for q_ in range(n_req):
        for b in range(nb):
            phys = perm[q_ * nb + b]
            table[q_, b] = phys
            rows = slice(b * bs, min(t, (b + 1) * bs))
            kpool[phys, :, : rows.stop - rows.start] = kc[q_, :, rows]
            vpool[phys, :, : rows.stop - rows.start] = vc[q_, :, rows]
    return kpool, vpool, table


def test_cached_decode_equals_full_recompute():
    # The last row of causal attention over T+1 tokens equals one decode step
    # over the T cached (already rotated) keys plus the new token itself.
    r = rng(15)
    n_req, hq, h, t, d, bs = 2, 4, 2, 45, 32, 16
    q_raw = r.standard_normal((n_req, hq, t + 1, d))
    k_raw = r.standard_normal((n_req, h, t + 1, d))
    v = r.standard_normal((n_req, h, t + 1, d))
    pos = 1 + np.arange(t + 1)
    k_rot = O.rope(k_raw, pos, 1e4)
    kp, vp, table = _paged_from_contiguous(r, k_rot[:, :, :t], v[:, :, :t], bs)
    out = O.paged_decode(kp, vp, table, [t, t], q_raw[:, :, t], k_raw[:, :, t], v[:, :, t],
                         [t + 1, t + 1], 1e4, 1 / math.sqrt(d))
    for q_ in range(n_req):
        ref = sdpa(O.rope(q_raw[q_], pos, 1e4), k_rot[q_], v[q_], is_causal=True,
                   enable_gqa=True)
        assert np.allclose(out[q_], ref[:, t], atol=1e-12)


def test_block_table_permutation_and_ragged_contexts():
    r = rng(16)
    n_req, hq, h, d, bs = 3, 2, 2, 16, 8
    lens = [0, 19, 24]
    t = max(lens)
    kc = r.standard_normal((n_req, h, t, d))
    vc = r.standard_normal((n_req, h, t, d))
    q, kn, vn = (r.standard_normal((n_req, n, d)) for n in (hq, h, h))
    pos = [1, 20, 25]
    kp, vp, table = _paged_from_contiguous(r, kc, vc, bs)
    out = O.paged_decode(kp, vp, table, lens, q, kn, vn, pos, 1e4, 0.25)
    # contiguous layout: request q's blocks in order, identity table
    nb = table.shape[1]
    kp2 = np.zeros((n_req * nb, h, bs, d))
    vp2 = np.zeros_like(kp2)
    for q_ in range(n_req):
        for b in range(nb):
            kp2[q_ * nb + b] = kp[table[q_, b]]
            vp2[q_ * nb + b] = vp[table[q_, b]]
    ident = np.arange(n_req * nb).reshape(n_req, nb)
    out2 = O.paged_decode(kp2, vp2, ident, lens, q, kn, vn, pos, 1e4, 0.25)
    assert np.array_equal(out, out2)
    # an empty cache leaves only the token itself: output = its own value
    assert np.allclose(out[0], np.repeat(vn[0], hq // h, axis=0), atol=1e-15)


def test_multi_token_block_equals_successive_decode_steps():
    # ell new tokens at once equal ell one-token steps, each appending its own
    # rotated K and its V to the cache ([KVC] Reusable-state).
    r = rng(17)
    k, ell, hq, h, d, bs = 8, 10, 4, 2, 16, 4
    pool = r.standard_normal((1, 1, 2, h, k, d))
    q, kn, vn = (r.standard_normal((1, ell, n, d)) for n in (hq, h, h))
    block = O.gist_attn_forward(pool, 0, [0], q, kn, vn, k + 1, 1e4, 0.25)[0]
    ktot = k + ell
    kc = np.zeros((1, h, ktot, d))
    vc = np.zeros((1, h, ktot, d))
    kc[0, :, :k], vc[0, :, :k] = pool[0, 0, 0], pool[0, 0, 1]
    for t in range(ell):
        kp, vp, table = _paged_from_contiguous(r, kc[:, :, :k + t], vc[:, :, :k + t], bs)
        step = O.paged_decode(kp, vp, table, [k + t], q[:, t], kn[:, t], vn[:, t],
                              [k + 1 + t], 1e4, 0.25)
        assert np.allclose(step[0], block[t], atol=1e-12)
        kc[0, :, k + t] = O.rope(kn[0, t], [k + 1 + t] * h, 1e4)
        vc[0, :, k + t] = vn[0, t]


# ---------------------------------------------------------------------------
# fp8 (OCP E4M3) cache decode
# ---------------------------------------------------------------------------


def test_decode_e4m3_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.decode_e4m3(codes), ref)


def test_decode_e4m3_landmarks():
    v = O.decode_e4m3(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0x7F, 0x80, 0xB8, 0xFE],
                               np.uint8))
    assert v[0] == 0.0 and v[1] == 2.0 ** -9 and v[2] == 7 * 2.0 ** -9
    assert v[3] == 2.0 ** -6 and v[4] == 1.0 and v[5] == 448.0
    assert np.isnan(v[6]) and v[7] == 0.0 and np.signbit(v[7])
    assert v[8] == -1.0 and v[9] == -448.0


def test_dequantize_blocks_applies_one_scale_per_block_and_head():
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 0x7E, (3, 2, 4, 5)).astype(np.uint8)
    scales = np.array([[1.0, 2.0], [0.5, 4.0], [3.0, 0.25]])
    d = O.dequantize_blocks(codes, scales)
    for b in range(3):
        for h in range(2):
            np.testing.assert_array_equal(d[b, h], O.decode_e4m3(codes[b, h]) * scales[b, h])


# ---------------------------------------------------------------------------
# fp8 (E4M3) encoding and the fp8 gist pool writer
# ---------------------------------------------------------------------------


def _torch_e4m3(y):
    """torch's own fp32 -> float8_e4m3fn conversion (round to nearest even)."""
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_e4m3_matches_torch_on_values_ties_and_neighbours():
    t = O.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (t[:-1] + t[1:]) / 2  # exact in fp32: one more mantissa bit than E4M3
    m32 = mids.astype(np.float32)
    ys = np.concatenate([
        t, -t, mids, -mids,
        np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0)),
        rng(30).choice([-1.0, 1.0], 50000) * np.exp2(rng(31).uniform(-13, 8.8, 50000)),
    ]).astype(np.float32)
    ys = ys[np.abs(ys) <= 448]
    np.testing.assert_array_equal(O.encode_e4m3(ys.astype(np.float64)), _torch_e4m3(ys))


def test_encode_e4m3_is_a_nearest_value_by_brute_force():
    t = O.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    y = rng(32).uniform(-448, 448, 4000) * np.exp2(rng(33).integers(-14, 1, 4000))
    got = O.decode_e4m3(O.encode_e4m3(y))
    best = np.min(np.abs(np.abs(y)[:, None] - t[None, :]), axis=1)
    assert np.array_equal(np.abs(np.abs(got) - np.abs(y)), best)
    assert np.array_equal(np.signbit(got), np.signbit(y))


def test_encode_e4m3_landmarks_and_clamp():
    e = O.encode_e4m3
    assert e([0.0])[0] == 0x00 and e([-0.0])[0] == 0x80 and e([-1e-9])[0] == 0x80
    assert e([2.0 ** -9])[0] == 0x01 and e([2.0 ** -10])[0] == 0x00  # tie -> even (0)
    assert e([3 * 2.0 ** -10])[0] == 0x02                             # tie 1.5 -> 2
    assert e([1.0])[0] == 0x38 and e([1.0625])[0] == 0x38 and e([1.1875])[0] == 0x3A
    assert e([448.0])[0] == 0x7E and e([-448.0])[0] == 0xFE
    # beyond the largest finite value: clamped (torch's conversion gives NaN there)
    assert e([464.0])[0] == 0x7E and e([1e9])[0] == 0x7E and e([-500.0])[0] == 0xFE


def test_quantize_block_scale_and_error_bound():
    x = rng(34).standard_normal((8, 128)) * 3.0
    codes, scale = O.quantize_e4m3_block(x)
    x32 = x.astype(np.float32)
    amax = float(np.max(np.abs(x32)))
    assert scale.dtype == np.float32 and scale == np.float32(np.float32(amax) / np.float32(448))
    deq = O.decode_e4m3(codes) * float(scale)
    # the largest element lands on +-448 * scale
    i = np.argmax(np.abs(x32))
    assert abs(O.decode_e4m3(codes.reshape(-1)[i:i + 1])[0]) == 448.0
    # normal range: half a step of 2^-3 relative; subnormal range: 2^-10 * scale absolute
    err = np.abs(deq - x32)
    bound = np.maximum(2.0 ** -4 * np.abs(x32), 2.0 ** -10 * float(scale)) * (1 + 1e-6)
    assert (err <= bound).all()
    zc, zs = O.quantize_e4m3_block(np.zeros((4, 64)))
    assert zs == np.float32(1) and not zc.any()


def test_pool_write_fp8_quantizes_each_block_after_rerotation():
    r = rng(35)
    n, k, h, d = 3, 8, 2, 64
    ks = r.standard_normal((n, k, h, d))
    vs = r.standard_normal((n, k, h, d)) * 0.01
    codes = np.zeros((2, 5, 2, h, k, d), np.uint8)
    scales = np.zeros((2, 5, 2, h), np.float32)
    c2, s2 = O.pool_write_fp8(codes, scales, 1, [4, 0, 2], ks, vs, 11, 1e4)
    rot = O.pool_write(np.zeros((2, 5, 2, h, k, d)), 1, [4, 0, 2], ks, vs, 11, 1e4)
    for i, item in enumerate([4, 0, 2]):
        for g in range(h):
            for kv in range(2):
                x = rot[1, item, kv, g]
                amax = np.max(np.abs(x.astype(np.float32)))
                assert s2[1, item, kv, g] == np.float32(amax / np.float32(448))
                deq = O.dequantize_gist(c2[1, item], s2[1, item])[kv, g]
                assert np.abs(deq - x).max() <= 2.0 ** -4 * amax * (1 + 1e-6)
    untouched = [1, 3]
    assert not c2[1, untouched].any() and not s2[1, untouched].any() and not c2[0].any()


def test_dequantize_gist_scales_each_k_v_head_block():
    r = rng(36)
    codes = r.integers(0, 0x7E, (2, 2, 3, 4, 8)).astype(np.uint8)   # [items][2][H][k][d]
    scales = r.uniform(0.1, 4.0, (2, 2, 3)).astype(np.float32)
    d = O.dequantize_gist(codes, scales)
    for i in range(2):
        for kv in range(2):
            for g in range(3):
                np.testing.assert_array_equal(
                    d[i, kv, g], O.decode_e4m3(codes[i, kv, g]) * float(scales[i, kv, g]))


# ---------------------------------------------------------------------------
# Offline gist extraction: causal prefill over [item ; gist] and the gist rows
# ---------------------------------------------------------------------------


def _packed(r, lens, hq, h, d):
    T = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return (r.standard_normal((T, hq, d)), r.standard_normal((T, h, d)),
            r.standard_normal((T, h, d)), starts)


def test_prefill_matches_sdpa_causal_per_sequence():
    r = rng(40)
    hq, h, d = 6, 2, 16
    lens = [9, 1, 17, 4]
    q, k, v, st = _packed(r, lens, hq, h, d)
    out = O.prefill_attention(q, k, v, st, 1e4, 0.3)
    for b, n in enumerate(lens):
        s = slice(st[b], st[b + 1])
        pos = 1 + np.arange(n)
        qr = O.rope(q[s].transpose(1, 0, 2), pos, 1e4)
        kr = O.rope(k[s].transpose(1, 0, 2), pos, 1e4)
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(qr)[None], torch.from_numpy(kr)[None],
            torch.from_numpy(v[s].transpose(1, 0, 2).copy())[None], is_causal=True, scale=0.3,
            enable_gqa=True)[0].numpy().transpose(1, 0, 2)
        assert np.allclose(out[s], ref, atol=1e-12)


def test_prefill_sequences_are_independent_and_causal():
    r = rng(41)
    hq, h, d = 4, 1, 8
    lens = [7, 12]
    q, k, v, st = _packed(r, lens, hq, h, d)
    out = O.prefill_attention(q, k, v, st, 1e4, 0.5)
    # each sequence alone, numbered from 1
    for b in range(2):
        s = slice(st[b], st[b + 1])
        alone = O.prefill_attention(q[s], k[s], v[s], [0, lens[b]], 1e4, 0.5)
        assert np.array_equal(out[s], alone)
    # changing tokens after t leaves rows <= t of the same sequence unchanged
    t = 4
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[t + 1:7] += 3.0
    v2[t + 1:7] -= 2.0
    q2[t + 1:7] *= -1.0
    out2 = O.prefill_attention(q2, k2, v2, st, 1e4, 0.5)
    assert np.array_equal(out2[:t + 1], out[:t + 1]) and not np.allclose(out2[t + 1:7], out[t + 1:7])
    assert np.array_equal(out2[7:], out[7:])


def test_gist_rows_equal_the_pool_write_of_the_prefill_keys():
    r = rng(42)
    h, d, n_gist = 2, 16, 4
    lens = [11, 6]
    _, k, v, st = _packed(r, lens, 2, h, d)
    gk, gv = O.gist_rows_from_prefill(k, v, st, n_gist, 1e4)
    for b, n in enumerate(lens):
        j = n - n_gist
        rows = slice(st[b] + j, st[b + 1])
        # the keys as the prefill rotates them: at j+1 .. j+n_gist
        k_at = O.rope(k[rows].transpose(1, 0, 2), j + 1 + np.arange(n_gist), 1e4).transpose(1, 0, 2)
        pool = O.pool_write(np.zeros((1, 1, 2, h, n_gist, d)), 0, [0], k_at[None], v[rows][None],
                            j + 1, 1e4)
        assert np.allclose(gk[b].transpose(1, 0, 2), pool[0, 0, 0], atol=1e-12)
        assert np.array_equal(gv[b].transpose(1, 0, 2), pool[0, 0, 1])


def test_toy_model_offline_extraction_by_prefill_then_online():
    """Two random-weight layers: the offline pass runs the prefill over [item ;
    gist] only and keeps its gist rows; the online pass over the query tokens
    then reproduces the query rows of the training layout [item ; gist ;
    query] under the gist mask (computed with torch's SDPA)."""
    r = rng(43)
    j, k, ell, dm, hq, h, d = 13, 4, 6, 32, 4, 2, 8
    n = j + k + ell
    layers = [dict(wq=r.standard_normal((dm, hq * d)) / math.sqrt(dm),
                   wk=r.standard_normal((dm, h * d)) / math.sqrt(dm),
                   wv=r.standard_normal((dm, h * d)) / math.sqrt(dm),
                   wo=r.standard_normal((hq * d, dm)) / math.sqrt(hq * d)) for _ in range(2)]
    x0 = r.standard_normal((n, dm))
    scale = 1 / math.sqrt(d)
    mlp = lambda x: np.tanh(x)  # noqa: E731

    x = x0.copy()
    pos = 1 + np.arange(n)
    mask = torch.from_numpy(training_mask(j, k, ell))
    for L in layers:
        qh = (x @ L["wq"]).reshape(n, hq, d).transpose(1, 0, 2)
        kh = (x @ L["wk"]).reshape(n, h, d).transpose(1, 0, 2)
        vh = (x @ L["wv"]).reshape(n, h, d).transpose(1, 0, 2)
        a = F.scaled_dot_product_attention(
            torch.from_numpy(O.rope(qh, pos, 1e4))[None], torch.from_numpy(O.rope(kh, pos, 1e4))[None],
            torch.from_numpy(vh)[None], attn_mask=mask[None], scale=scale, enable_gqa=True)[0].numpy()
        x = x + a.transpose(1, 0, 2).reshape(n, hq * d) @ L["wo"]
        x = x + mlp(x)
    train_rows = x[j + k:]

    # offline: prefill over [item ; gist] only, gist rows kept per layer
    pool = np.zeros((2, 1, 2, h, k, d))
    xo = x0[:j + k].copy()
    st = [0, j + k]
    for li, L in enumerate(layers):
        qn = (xo @ L["wq"]).reshape(j + k, hq, d)
        kn = (xo @ L["wk"]).reshape(j + k, h, d)
        vn = (xo @ L["wv"]).reshape(j + k, h, d)
        gk, gv = O.gist_rows_from_prefill(kn, vn, st, k, 1e4)
        pool[li, 0, 0], pool[li, 0, 1] = gk[0].transpose(1, 0, 2), gv[0].transpose(1, 0, 2)
        a = O.prefill_attention(qn, kn, vn, st, 1e4, scale)
        xo = xo + a.reshape(j + k, hq * d) @ L["wo"]
        xo = xo + mlp(xo)
    assert np.allclose(xo, x[:j + k], atol=1e-10)  # item and gist rows: the prefill is exact

    # online: only the query tokens, the gist injected as KV, pos0 = k+1
    x = x0[j + k:].copy()
    for li, L in enumerate(layers):
        qn = (x @ L["wq"]).reshape(1, ell, hq, d)
        kn = (x @ L["wk"]).reshape(1, ell, h, d)
        vn = (x @ L["wv"]).reshape(1, ell, h, d)
        a = O.gist_attn_forward(pool, li, [0], qn, kn, vn, k + 1, 1e4, scale)[0]
        x = x + a.reshape(ell, hq * d) @ L["wo"]
        x = x + mlp(x)
    assert np.allclose(x, train_rows, atol=1e-10)


def test_paged_gist_pools_round_trip_and_attention():
    r = rng(50)
    P, H, d, k, kq, bs, nb = 5, 2, 16, 4, 3, 8, 12
    pool = r.standard_normal((1, P, 2, H, k, d))
    qpool = r.standard_normal((1, P, 2, H, kq, d))
    kc = np.zeros((nb, H, bs, d))
    vc = np.zeros_like(kc)
    ib = np.array([3, 0, 7, 11, 5])
    qb = np.array([1, 2, 4, 6, 8])
    q_row0 = 2
    for p in range(P):
        for g in range(H):
            kc[ib[p], g, :k], vc[ib[p], g, :k] = pool[0, p, 0, g], pool[0, p, 1, g]
            kc[qb[p], g, q_row0:q_row0 + kq] = qpool[0, p, 0, g]
            vc[qb[p], g, q_row0:q_row0 + kq] = qpool[0, p, 1, g]
    gp, gq = O.paged_gist_pools(kc, vc, ib, k, qb, kq, q_row0)
    assert np.array_equal(gp, pool) and np.array_equal(gq, qpool)
    # both gists in one block (item rows 0..k-1, query rows k..k+kq-1)
    kc1 = np.zeros((P, H, bs, d))
    vc1 = np.zeros_like(kc1)
    kc1[:, :, :k], vc1[:, :, :k] = pool[0, :, 0], pool[0, :, 1]
    kc1[:, :, k:k + kq], vc1[:, :, k:k + kq] = qpool[0, :, 0], qpool[0, :, 1]
    gp1, gq1 = O.paged_gist_pools(kc1, vc1, np.arange(P), k, np.arange(P), kq, k)
    assert np.array_equal(gp1, pool) and np.array_equal(gq1, qpool)
    gp0, gq0 = O.paged_gist_pools(kc, vc, ib, k, None, 0, 0)
    assert gq0 is None and np.array_equal(gp0, pool)


# ---------------------------------------------------------------------------
# Direct pins of the mask and gather helpers (also covered through the
# attention pins above)
# ---------------------------------------------------------------------------


def test_causal_mask_is_torch_tril():
    for n in (1, 2, 7, 64):
        want = torch.tril(torch.ones(n, n, dtype=torch.bool)).numpy()
        assert np.array_equal(O.causal_mask(n), want)


def test_gist_online_mask_is_the_training_mask_seen_from_the_query():
    # [GIST] 论文做了什么: the sequence [item ; gist ; query] is causal, and
    # every token after the gist has the item block dug out.  The query rows
    # over the [gist ; query] columns are the online pass's mask.
    for n_item, n_gist, ell in ((5, 3, 4), (1, 8, 1), (9, 1, 6), (2, 4, 16)):
        n = n_item + n_gist + ell
        m = torch.tril(torch.ones(n, n, dtype=torch.bool)).numpy()
        m[n_item + n_gist:, :n_item] = False
        assert np.array_equal(O.gist_online_mask(n_gist, ell), m[n_item + n_gist:, n_item:])


def test_gather_logical_inverts_a_block_table_scatter():
    # a logical sequence written block by block into the physical blocks a
    # permuted table names (the other rows hold unrelated values) comes back
    # in order
    rng = np.random.default_rng(5)
    n_blocks, h, bs, d, g = 9, 2, 4, 3, 1
    for n_tokens in (0, 1, 4, 5, 13):
        x = rng.standard_normal((n_tokens, d))
        nb = -(-n_tokens // bs)
        table = rng.permutation(n_blocks)[:max(nb, 1)]
        cache = rng.standard_normal((n_blocks, h, bs, d))
        for i in range(nb):
            chunk = x[i * bs:(i + 1) * bs]
            cache[table[i], g, :len(chunk)] = chunk
        got = O.gather_logical(cache, table, n_tokens, g)
        assert got.shape == (n_tokens, d)
        assert np.array_equal(got, x)
