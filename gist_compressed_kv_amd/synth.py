"""Seeded synthetic inputs and workload shapes.

Only random-number generation and bookkeeping live here; none of the
attention arithmetic does.  The oracle and the HIP path both consume what
these functions produce (the oracle always receives the exact device
values, copied back).

Workloads mirror the shapes the gist article works with (liam.page
"把 item 压成 KV：gist 能不能用在相关性任务上": 24 layers / 2 KV heads /
head_dim 64 and 28 layers / 8 KV heads / head_dim 128 in 收益有多大：存储,
k = 8 gist positions, ell = 64 query tokens (63 + EOS), 50 candidates per
query in 装不下的时候自然要分片, query gist k' = 8 in 能不能再进一步) and,
for paged decode, 256-token blocks (icman.com.cn news 64898, section 5).
Every tensor is N(0, 1) in fp32, rounded once to the target dtype.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, seed: int, dtype: torch.dtype, device, chunk_elems: int = 1 << 27) -> torch.Tensor:
    """N(0,1) drawn in fp32 from a seeded generator, rounded to ``dtype``.

    Large tensors are filled in chunks along the first axis so that the fp32
    staging buffer stays bounded.
    """
    out = torch.empty(shape, dtype=dtype, device=device)
    g = generator(seed, device)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        stop = min(n, start + chunk_elems)
        flat[start:stop].copy_(torch.randn(stop - start, generator=g, device=device,
                                           dtype=torch.float32))
    return out


def randn_fp8_blocks(shape, seed: int, device):
    """A synthetic fp8 paged cache [n_blocks][H][block][d]: N(0,1) values (as
    ``randn``) stored as OCP E4M3 codes with one fp32 scale per (block, head),
    scale = amax / 448, quantized by torch's own E4M3 conversion.  Returns
    (codes uint8, scales fp32 [n_blocks][H])."""
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    scales = torch.empty(shape[:2], dtype=torch.float32, device=device)
    g = generator(seed, device)
    per_block = shape[1] * shape[2] * shape[3]
    step = max(1, (1 << 27) // per_block)
    for b0 in range(0, shape[0], step):
        b1 = min(shape[0], b0 + step)
        x = torch.randn((b1 - b0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        amax = x.abs().amax(dim=(2, 3))
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        codes[b0:b1] = (x / sc[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        scales[b0:b1] = sc
    return codes, scales


def randn_fp8_gist_pool(L: int, N: int, k: int, H: int, d: int, seed: int, device) -> torch.Tensor:
    """Flat storage of a synthetic fp8 gist pool: the codes [L][N][2][H][k][d]
    of N(0,1) values (as ``randn``) followed by their fp32 scales [L][N][2][H],
    one per (layer, item, K or V, head) block, scale = amax / 448, quantized
    by torch's own E4M3 conversion."""
    ncode = L * N * 2 * H * k * d
    storage = torch.empty(ncode + L * N * 2 * H * 4, dtype=torch.uint8, device=device)
    codes = storage[:ncode].view(L, N, 2, H, k, d)
    scales = storage[ncode:].view(torch.float32).view(L, N, 2, H)
    g = generator(seed, device)
    step = max(1, (1 << 27) // (2 * H * k * d))
    for li in range(L):
        for i0 in range(0, N, step):
            i1 = min(N, i0 + step)
            x = torch.randn((i1 - i0, 2, H, k, d), generator=g, device=device, dtype=torch.float32)
            amax = x.abs().amax(dim=(3, 4))
            sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
            codes[li, i0:i1] = (x / sc[..., None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
            scales[li, i0:i1] = sc
    return storage


def item_ids_per_query(n_queries: int, n_candidates: int, n_items: int, seed: int,
                       device) -> torch.Tensor:
    """Candidate ids, query-major: each query draws n_candidates distinct items
    uniformly (a prefix of a random permutation)."""
    g = generator(seed, "cpu")
    rows = [torch.randperm(n_items, generator=g)[:n_candidates] for _ in range(n_queries)]
    return torch.cat(rows).to(torch.int32).to(device)


def block_table(n_requests: int, blocks_per_request: int, n_blocks: int, seed: int,
                device) -> torch.Tensor:
    """Each request's logical blocks map to distinct physical blocks drawn from
    a seeded random permutation of the block pool."""
    g = generator(seed, "cpu")
    perm = torch.randperm(n_blocks, generator=g)[: n_requests * blocks_per_request]
    return perm.view(n_requests, blocks_per_request).to(torch.int32).to(device)


def tensor_seed(seed: int, tensor_id: int, layer: int = 0) -> int:
    return seed * 1000 + tensor_id + 100003 * layer


@dataclass(frozen=True)
class GistWorkload:
    name: str
    layers: int
    n_items: int
    k: int
    ell: int
    hq: int
    h: int
    d: int
    pairs: int
    queries: int
    dtype: torch.dtype
    seed: int
    kq: int = 0  # query-gist positions (0 = no query gist)
    fp8: bool = False  # gist pools in fp8 E4M3 (activations stay in dtype)

    @property
    def pos0(self) -> int:
        return self.k + self.kq + 1


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    layers: int
    requests: int
    context: int
    block_size: int
    hq: int
    h: int
    d: int
    dtype: torch.dtype
    seed: int

    @property
    def blocks_per_request(self) -> int:
        return -(-self.context // self.block_size)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    layers: int
    items: int
    min_item: int  # item tokens, drawn uniformly in [min_item, max_item]
    max_item: int
    k: int         # gist tokens appended to every item
    hq: int
    h: int
    d: int
    seed: int


def prefill_lengths(wl: PrefillWorkload, device) -> torch.Tensor:
    """Sequence lengths (item tokens + k gist tokens) of a prefill workload."""
    g = generator(wl.seed, "cpu")
    items = torch.randint(wl.min_item, wl.max_item + 1, (wl.items,), generator=g)
    return (items + wl.k).to(torch.int32).to(device)


TINY = GistWorkload("tiny: 1 layer, 4 pairs over 2 items, k=8, ell=16, Hq=4, H=1, d=64, fp32",
                    1, 2, 8, 16, 4, 1, 64, 4, 2, torch.float32, 1)
SINGLE_LAYER = GistWorkload("1 layer, Hq=14, H=2, d=64, k=8, ell=64, 500 pairs, 100k-item pool, bf16",
                            1, 100_000, 8, 64, 14, 2, 64, 500, 10, torch.bfloat16, 2)
L24_B500 = GistWorkload("24 layers, Hq=14, H=2, d=64, k=8, ell=64, 500 pairs, 100k-item pools, bf16",
                        24, 100_000, 8, 64, 14, 2, 64, 500, 10, torch.bfloat16, 3)
L24_B2000 = GistWorkload("24 layers, Hq=14, H=2, d=64, k=8, ell=64, 2000 pairs, 100k-item pools, bf16",
                         24, 100_000, 8, 64, 14, 2, 64, 2000, 40, torch.bfloat16, 3)
WIDE_ELL64 = GistWorkload("28 layers, Hq=64, H=8, d=128, k=8, ell=64, 2000 pairs, 100k-item pool, bf16",
                          28, 100_000, 8, 64, 64, 8, 128, 2000, 40, torch.bfloat16, 4)
WIDE_EOS = GistWorkload("28 layers, Hq=64, H=8, d=128, item gist k=8 + query gist k'=8 + EOS (ell=1), "
                        "2000 pairs, bf16", 28, 100_000, 8, 1, 64, 8, 128, 2000, 40,
                        torch.bfloat16, 4, kq=8)
PAGED = DecodeWorkload("paged decode: 32 requests x 4096 cached tokens in 256-token blocks, "
                       "Hq=H=32, d=128, 32 layers, bf16", 32, 32, 4096, 256, 32, 32, 128,
                       torch.bfloat16, 5)

WIDE_EOS_FP8 = GistWorkload("28 layers, Hq=64, H=8, d=128, item gist k=8 + query gist k'=8 + EOS "
                            "(ell=1), 2000 pairs, fp8 E4M3 gist pools with per-(item, K/V, head) "
                            "scales, bf16 activations", 28, 100_000, 8, 1, 64, 8, 128, 2000, 40,
                            torch.bfloat16, 7, kq=8, fp8=True)

WIDE_ELL64_FP8 = GistWorkload("28 layers, Hq=64, H=8, d=128, k=8, ell=64, 2000 pairs, 100k-item "
                              "pool as fp8 E4M3 with per-(item, K/V, head) scales, bf16 activations",
                              28, 100_000, 8, 64, 64, 8, 128, 2000, 40, torch.bfloat16, 9, fp8=True)

PAGED_FP8 = DecodeWorkload("paged decode, fp8 E4M3 cache with per-(block, head) scales: 32 requests "
                           "x 4096 cached tokens in 256-token blocks, Hq=H=32, d=128, 32 layers, "
                           "bf16 activations", 32, 32, 4096, 256, 32, 32, 128, torch.bfloat16, 6)

PREFILL = PrefillWorkload("offline gist extraction: 256 items of 900-1100 tokens + 8 gist tokens, "
                          "causal prefill, Hq=14, H=2, d=64, 24 layers, bf16", 24, 256, 900, 1100, 8,
                          14, 2, 64, 8)
