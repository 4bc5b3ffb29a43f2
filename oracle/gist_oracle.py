"""Plain fp64 CPU oracle for gist-compressed KV attention and paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or constant with the HIP library under ``gist_compressed_kv_amd/``.

Sources (web pages; cited by title and section):

* [GIST] liam.page, "把 item 压成 KV：gist 能不能用在相关性任务上"
  (compressing an item into KV for relevance scoring), sections
  "论文做了什么" (the gist mask), "在线的一次 attention" (the online pass,
  the query position numbering), "收益有多大：存储" (bytes per position),
  "能不能再进一步" (query also compressed; only EOS stays online).
* [KVC] mcfzz.com, "为什么自回归推理缓存 KV，而不缓存历史 Q？", sections
  "Reusable-state" (the decode equation with the 1/sqrt(d_k) softmax scale),
  "Memory" (M_KV = 2·B·L·T·h_kv·d_h·b).
* [SFX] icman.com.cn/news/64898 (suffix cache article), section 5 step 1
  (256-token KV blocks) and section 6 problem 4 (logical-to-physical block
  table consulted by attention).

Everything is fp64 numpy.  The method is exact attention once the gist K/V
are given, so each function below is the plain definition written out: RoPE,
an explicit key/value sequence, an explicit boolean mask and a softmax.
There is no blocking, no online softmax and no fusion here.

Readings of points the pages leave open (each is a free choice that the GPU
library makes identically):

* RoPE pairs channel i with channel i + d/2 ("rotate half") and uses the
  frequency base**(-2i/d); positions are 1-based.
* The stored gist K is already rotated, at the canonical positions 1..k
  (item gist) and k+1..k+k' (query gist); only Q and the new K are rotated
  online, at positions pos0 + t.
* Query head h reads KV head h // (Hq/H) (contiguous GQA groups).
* A query token sees every gist key and the new keys up to and including
  itself; a decode token sees the whole cache and itself.
* fp8 storage (the pages name KV quantization as a lever but fix no scheme):
  OCP FP8 E4M3 codes with one fp32 scale per block (a paged-cache (block,
  head); a gist pool's (item, K or V, head)), scale = amax / 448, codes the
  nearest E4M3 value of x / scale, ties to even, decided in fp32.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Byte counts ([GIST] "收益有多大：存储"; [KVC] "Memory"; [SFX] section 2)
# ---------------------------------------------------------------------------


def kv_bytes_per_position(n_layers: int, n_kv_heads: int, head_dim: int,
                          elem_bytes: int) -> int:
    """K and V of every layer for one sequence position: 2·L·H·h·b bytes."""
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes


def gist_bytes_per_item(n_layers: int, n_gist: int, n_kv_heads: int,
                        head_dim: int, elem_bytes: int) -> int:
    """One item's stored gist object G: k positions' K and V in every layer
    ([GIST] "在线的一次 attention": 2·L·k·H·h elements per item)."""
    return n_gist * kv_bytes_per_position(n_layers, n_kv_heads, head_dim,
                                          elem_bytes)


def kv_cache_bytes(batch: int, n_layers: int, seq_len: int, n_kv_heads: int,
                   head_dim: int, elem_bytes: int) -> int:
    """Whole KV cache of a batch: 2·B·L·T·h_kv·d_h·b ([KVC] "Memory")."""
    return 2 * batch * n_layers * seq_len * n_kv_heads * head_dim * elem_bytes


# ---------------------------------------------------------------------------
# RoPE ([GIST] "在线的一次 attention": only position differences matter)
# ---------------------------------------------------------------------------


def rope_frequencies(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base**(-2i/d) for i in [0, d/2)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Rotate the rows of ``x`` (shape [..., T, d]) to ``positions`` ([T]).

    Channel pair (i, i + d/2) is turned by the angle positions[t]·theta_i:
    x'[i] = x[i]·cos − x[i+d/2]·sin,  x'[i+d/2] = x[i+d/2]·cos + x[i]·sin.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    half = d // 2
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    assert pos.shape[0] == x.shape[-2]
    angle = pos[:, None] * rope_frequencies(d, base)[None, :]
    c, s = np.cos(angle), np.sin(angle)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------------------
# Masked softmax attention ([KVC] "Reusable-state": o = softmax(q Kᵀ/√d_k) V)
# ---------------------------------------------------------------------------


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
              scale: float) -> np.ndarray:
    """q [T, d], k [S, d], v [S, dv], mask bool [T, S] (True = visible).

    Every row must see at least one key.  Returns [T, dv].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    mask = np.asarray(mask, bool)
    assert mask.shape == (q.shape[0], k.shape[0])
    assert mask.any(axis=1).all(), "a query row sees no key"
    logits = scale * (q @ k.T)
    logits = np.where(mask, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ v


def gist_online_mask(n_gist: int, ell: int) -> np.ndarray:
    """Mask of the online sequence [gist (n_gist) ; new tokens (ell)].

    Query token t sees every gist key and new keys 0..t (itself included).
    """
    t = np.arange(ell)[:, None]
    j = np.arange(n_gist + ell)[None, :]
    return (j < n_gist) | ((j - n_gist) <= t)


def gist_pair_attention(gist_k: np.ndarray, gist_v: np.ndarray,
                        q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                        pos0: int, base: float, scale: float) -> np.ndarray:
    """One (item, query) pair, one query head ([GIST] "在线的一次 attention").

    gist_k, gist_v: [n_gist, d], K already rotated at its canonical
    positions.  q, k_new, v_new: [ell, d], not yet rotated; they sit at
    positions pos0 .. pos0+ell-1.  Keys are cat(gist, new); values likewise.
    """
    ell = q.shape[0]
    n_gist = gist_k.shape[0]
    pos = pos0 + np.arange(ell)
    keys = np.concatenate([gist_k, rope(k_new, pos, base)], axis=0)
    vals = np.concatenate([gist_v, v_new], axis=0)
    return attention(rope(q, pos, base), keys, vals,
                     gist_online_mask(n_gist, ell), scale)


def gist_attn_forward(pool: np.ndarray, layer: int, item_ids, q: np.ndarray,
                      k_new: np.ndarray, v_new: np.ndarray, pos0: int,
                      base: float, scale: float, qpool: np.ndarray | None = None,
                      q_ids=None) -> np.ndarray:
    """Gist attention of a batch of pairs in one layer.

    pool:  [L][N][2][H][k][d]  (index 0 of the third axis = K, 1 = V)
    q:     [P][ell][Hq][d];  k_new, v_new: [P][ell][H][d]
    qpool: optional query-gist pool [L][Nq][2][H][k'][d], row q_ids[p]; its
           rows follow the item gist in key order ([GIST] "能不能再进一步").
    Returns [P][ell][Hq][d].
    """
    pool = np.asarray(pool, np.float64)
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    n_pairs, ell, hq, d = q.shape
    h_kv = k_new.shape[2]
    assert hq % h_kv == 0
    group = hq // h_kv
    out = np.zeros((n_pairs, ell, hq, d), np.float64)
    for p in range(n_pairs):
        item = int(item_ids[p])
        for h in range(hq):
            g = h // group
            gk = pool[layer, item, 0, g]
            gv = pool[layer, item, 1, g]
            if qpool is not None:
                qrow = int(q_ids[p])
                gk = np.concatenate([gk, np.asarray(qpool[layer, qrow, 0, g], np.float64)], axis=0)
                gv = np.concatenate([gv, np.asarray(qpool[layer, qrow, 1, g], np.float64)], axis=0)
            out[p, :, h, :] = gist_pair_attention(
                gk, gv, q[p, :, h, :], k_new[p, :, g, :], v_new[p, :, g, :],
                pos0, base, scale)
    return out


def pool_write(pool: np.ndarray, layer: int, ids, k_src: np.ndarray,
               v_src: np.ndarray, src_pos0: int, base: float) -> np.ndarray:
    """Store gist K/V rows into a pool (returns the updated copy).

    k_src, v_src: [n][k][H][d].  k_src row i is rotated at position
    src_pos0 + i; it is stored rotated at the canonical position 1 + i, so
    the query-to-gist distance matches the one seen in training ([GIST]
    "在线的一次 attention").  Re-rotating by (1 - src_pos0) is exact in real
    arithmetic because rotations compose additively.
    """
    out = np.array(pool, dtype=np.float64, copy=True)
    k_src = np.asarray(k_src, np.float64)
    v_src = np.asarray(v_src, np.float64)
    n, k, h_kv, d = k_src.shape
    shift = np.full(k, 1 - src_pos0, dtype=np.float64)
    for i in range(n):
        for g in range(h_kv):
            out[layer, int(ids[i]), 0, g] = rope(k_src[i, :, g, :], shift, base)
            out[layer, int(ids[i]), 1, g] = v_src[i, :, g, :]
    return out


def paged_gist_pools(k_cache, v_cache, item_blocks, k: int, query_blocks, kq: int, q_row0: int):
    """Gists held in a paged cache [n_blocks][H][bs][d] as one-layer pools:
    pair p's item gist is rows 0..k-1 of block item_blocks[p] and its query
    gist rows q_row0..q_row0+kq-1 of block query_blocks[p].  Returns (pool,
    qpool), each [1][P][2][H][rows][d] (qpool None when kq = 0), to be read
    with item id p and query id p."""
    kc = np.asarray(k_cache, np.float64)
    vc = np.asarray(v_cache, np.float64)
    ib = np.asarray(item_blocks, np.int64)
    pool = np.stack([kc[ib, :, :k], vc[ib, :, :k]], axis=1)[None]
    qpool = None
    if kq:
        qb = np.asarray(query_blocks, np.int64)
        rows = slice(q_row0, q_row0 + kq)
        qpool = np.stack([kc[qb, :, rows], vc[qb, :, rows]], axis=1)[None]
    return pool, qpool


# ---------------------------------------------------------------------------
# Offline gist extraction, one layer ([GIST] "论文做了什么": the item is run
# with its k gist tokens appended and the gist positions' K/V are kept;
# "在线的一次 attention": they are stored for the query to meet at distance k)
# ---------------------------------------------------------------------------


def causal_mask(n: int) -> np.ndarray:
    """Token t sees tokens 0..t."""
    return np.arange(n)[None, :] <= np.arange(n)[:, None]


def prefill_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_start, base: float,
                      scale: float) -> np.ndarray:
    """Causal self-attention of B packed sequences [item tokens ; gist tokens].

    q [T][Hq][d]; k, v [T][H][d], not rotated.  Sequence b is tokens
    seq_start[b] .. seq_start[b+1]-1, at positions 1..len.  Query head h reads
    KV head h // (Hq/H).  Over [item ; gist] alone the gist mask of training
    is the causal mask: it only removes item keys from tokens after the gist,
    and none are present.
    Returns out [T][Hq][d].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hq, h_kv = q.shape[1], k.shape[1]
    group = hq // h_kv
    out = np.zeros_like(q)
    starts = np.asarray(seq_start, np.int64)
    for b in range(len(starts) - 1):
        s0, s1 = int(starts[b]), int(starts[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        pos = 1 + np.arange(n)
        mask = causal_mask(n)
        for hh in range(hq):
            g = hh // group
            qr = rope(q[s0:s1, hh], pos, base)
            kr = rope(k[s0:s1, g], pos, base)
            out[s0:s1, hh] = attention(qr, kr, v[s0:s1, g], mask, scale)
    return out


def gist_rows_from_prefill(k: np.ndarray, v: np.ndarray, seq_start, n_gist: int,
                           base: float):
    """The last n_gist tokens of each packed sequence are its gist: their K,
    rotated at the canonical positions 1..n_gist (the K the prefill rotates at
    j+1..j+n_gist, turned back by j), and their V.  Returns (gk, gv), each
    [B][n_gist][H][d], in the row order gist_pool_write takes."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    starts = np.asarray(seq_start, np.int64)
    B = len(starts) - 1
    gk = np.zeros((B, n_gist) + k.shape[1:])
    gv = np.zeros_like(gk)
    for b in range(B):
        e = int(starts[b + 1])
        rows = slice(e - n_gist, e)
        gk[b] = rope(k[rows].transpose(1, 0, 2), 1 + np.arange(n_gist), base).transpose(1, 0, 2)
        gv[b] = v[rows]
    return gk, gv


# ---------------------------------------------------------------------------
# Paged decode ([KVC] "Reusable-state"; [SFX] section 6 problem 4)
# ---------------------------------------------------------------------------


def decode_e4m3(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (uint8): 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent 0 holds the subnormals m * 2**-9;
    exponent 15 with mantissa 7 is NaN (there is no infinity), so the largest
    finite value is 1.75 * 2**8 = 448."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (c & 7 == 7), np.nan, val)
    return sign * val


def dequantize_blocks(codes, scales) -> np.ndarray:
    """Paged cache of E4M3 codes [n_blocks][H][block][d] with one scale per
    (block, head) [n_blocks][H]: element = decode(code) * scale."""
    return decode_e4m3(codes) * np.asarray(scales, np.float64)[:, :, None, None]


def encode_e4m3(y) -> np.ndarray:
    """E4M3 code of the finite value nearest to y.  A tie goes to the code with
    the even mantissa (round to nearest even), |y| is clamped to 448 first and
    the sign bit is kept (a negative y that rounds to zero gives 0x80, -0).

    Written as a nearest-neighbour search over the 127 non-negative finite
    values (codes 0x00..0x7E, increasing in value), so every step can be
    checked against the format's definition in decode_e4m3."""
    y = np.asarray(y, np.float64)
    table = decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(y), 448.0)
    hi = np.minimum(np.searchsorted(table, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - table[lo], table[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_e4m3_block(x):
    """One block of values quantized the way the fp8 pool writer does it, in
    fp32 (the precision in which the codes are decided): amax = max |x|,
    scale = amax / 448 (1 for an all-zero block), codes = nearest E4M3 value
    of the fp32 quotient x / scale.  Returns (codes uint8, scale float32)."""
    x32 = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    scale = np.float32(amax / np.float32(448)) if amax > 0 else np.float32(1)
    return encode_e4m3((x32 / scale).astype(np.float64)), scale


def pool_write_fp8(codes: np.ndarray, scales: np.ndarray, layer: int, ids, k_src: np.ndarray,
                   v_src: np.ndarray, src_pos0: int, base: float):
    """pool_write into an fp8 pool: codes [L][N][2][H][k][d], scales
    [L][N][2][H] (returns updated copies).  K is re-rotated as in pool_write
    (here in fp64, then taken to fp32) and every (item, K or V, head) block of
    k*d values is quantized by quantize_e4m3_block."""
    codes = np.array(codes, dtype=np.uint8, copy=True)
    scales = np.array(scales, dtype=np.float32, copy=True)
    k_src = np.asarray(k_src, np.float64)
    v_src = np.asarray(v_src, np.float64)
    n, k, h_kv, d = k_src.shape
    shift = np.full(k, 1 - src_pos0, dtype=np.float64)
    for i in range(n):
        for g in range(h_kv):
            for kv, x in ((0, rope(k_src[i, :, g, :], shift, base)), (1, v_src[i, :, g, :])):
                c, sc = quantize_e4m3_block(x)
                codes[layer, int(ids[i]), kv, g] = c
                scales[layer, int(ids[i]), kv, g] = sc
    return codes, scales


def dequantize_gist(codes, scales) -> np.ndarray:
    """fp8 gist records [...][2][H][k][d] with scales [...][2][H]: element =
    decode(code) * scale of its (item, K or V, head)."""
    return decode_e4m3(codes) * np.asarray(scales, np.float64)[..., None, None]


def gather_logical(cache: np.ndarray, block_row, n_tokens: int, g: int) -> np.ndarray:
    """Rows 0..n_tokens-1 of one request, KV head g, in logical order.

    cache: [n_blocks][H][bs][d]; logical token j lives in physical block
    block_row[j // bs] at row j % bs.
    """
    bs = cache.shape[2]
    j = np.arange(n_tokens)
    blocks = np.asarray(block_row, dtype=np.int64)[j // bs]
    return np.asarray(cache[blocks, g, j % bs], np.float64).reshape(n_tokens, cache.shape[3])


def paged_decode(k_cache: np.ndarray, v_cache: np.ndarray, block_table,
                 context_lens, q: np.ndarray, k_new: np.ndarray,
                 v_new: np.ndarray, positions, base: float,
                 scale: float) -> np.ndarray:
    """One decode step for R requests.

    k_cache, v_cache: [n_blocks][H][bs][d], cached K already rotated.
    block_table: [R][max_blocks]; context_lens: [R] cached tokens.
    q: [R][Hq][d]; k_new, v_new: [R][H][d]; positions: [R] position of the
    new token.  Keys are [cache in logical order ; the new token's own key],
    so the new token attends to itself (K_{<=t} = [K_{<t}; k_t]).
    Returns [R][Hq][d].
    """
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    n_req, hq, d = q.shape
    h_kv = k_new.shape[1]
    group = hq // h_kv
    out = np.zeros((n_req, hq, d), np.float64)
    for r in range(n_req):
        t_ctx = int(context_lens[r])
        pos = [int(positions[r])]
        for h in range(hq):
            g = h // group
            keys = np.concatenate([gather_logical(k_cache, block_table[r], t_ctx, g),
                                   rope(k_new[r, g][None, :], pos, base)], axis=0)
            vals = np.concatenate([gather_logical(v_cache, block_table[r], t_ctx, g),
                                   v_new[r, g][None, :]], axis=0)
            qr = rope(q[r, h][None, :], pos, base)
            mask = np.ones((1, t_ctx + 1), bool)
            out[r, h] = attention(qr, keys, vals, mask, scale)[0]
    return out
