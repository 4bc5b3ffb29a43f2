"""Gist-compressed KV attention and paged decode for AMD MI355X (gfx950).

Thin torch-facing binding over libgist_attn.so: every function here only
checks and marshals arguments (device pointers, sizes, the current HIP
stream) and calls the C entry point of the same name.  All computation runs
in the library's HIP kernels; torch provides device memory and streams.
"""

from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import GIST_BF16, GIST_F32, GIST_FP8_E4M3, GistError  # noqa: F401

__all__ = [
    "GistPool", "GistError", "gist_pool_bytes", "gist_pool_fp8_storage", "gist_pool_create",
    "gist_pool_write",
    "gist_attn_forward", "gist_attn_forward_last", "gist_attn_forward_paged",
    "gist_attn_forward_paged_fp8",
    "gist_prefill_workspace_bytes",
    "gist_prefill_attn",
    "paged_decode_workspace_bytes", "paged_decode_attn", "paged_decode_attn_fp8",
    "paged_decode_attn_noalloc",
]

_DTYPES = {torch.bfloat16: GIST_BF16, torch.float32: GIST_F32}


def _code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}; use torch.bfloat16 or torch.float32")
    return _DTYPES[dtype]


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    # dtype and shape first: the library reads every tensor at the extents
    # its sizes imply, so a mismatch must never reach it
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    return t.data_ptr()


def _ptrs(*specs):
    """Device pointers of a call's tensors, each spec (tensor, name, dtype,
    shape) or None (passed on as None).  Types, dtypes, shapes and contiguity
    of all of them are checked before any is required to be on the GPU."""
    for sp in specs:
        if sp is not None:
            t, name, dtype, shape = (tuple(sp) + (None, None))[:4]
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if dtype is not None and t.dtype != dtype:
                raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
            if shape is not None and tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return tuple(None if sp is None else _dev(*sp) for sp in specs)


def gist_pool_bytes(L: int, N: int, k: int, H: int, d: int, dtype) -> int:
    """dtype: torch.bfloat16, torch.float32, or "fp8" (E4M3 codes + fp32 scales)."""
    code = GIST_FP8_E4M3 if dtype == "fp8" else _code(dtype)
    return _lib.lib().gist_pool_bytes(L, N, k, H, d, code)


def gist_pool_fp8_storage(L: int, N: int, k: int, H: int, d: int, device="cuda") -> torch.Tensor:
    """Uninitialised uint8 device storage for an fp8 pool of this shape."""
    n = gist_pool_bytes(L, N, k, H, d, "fp8")
    if n == 0:
        raise ValueError("invalid fp8 pool shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


class GistPool:
    """A gist pool over caller-owned device storage.

    bf16 / fp32: a tensor [L][N][2][H][k][d].  fp8: a flat uint8 tensor of
    gist_pool_bytes(L, N, k, H, d, "fp8") bytes plus ``shape=(L, N, k, H, d)``;
    ``codes`` [L][N][2][H][k][d] (uint8) and ``scales`` [L][N][2][H] (fp32)
    are views of it.  Calls on an fp8 pool take bf16 activations."""

    def __init__(self, storage: torch.Tensor, shape=None):
        self.fp8 = storage.dtype == torch.uint8
        if self.fp8:
            if shape is None or len(shape) != 5:
                raise ValueError("an fp8 pool needs shape=(L, N, k, H, d)")
            L, N, k, H, d = (int(x) for x in shape)
            if storage.dim() != 1:
                raise ValueError("fp8 pool storage must be a flat uint8 tensor")
            ncode = L * N * 2 * H * k * d
            if storage.numel() == ncode + L * N * 2 * H * 4:
                self.codes = storage[:ncode].view(L, N, 2, H, k, d)
                self.scales = storage[ncode:].view(torch.float32).view(L, N, 2, H)
            code, self.act_dtype = GIST_FP8_E4M3, torch.bfloat16
        else:
            if storage.dim() != 6 or storage.shape[2] != 2:
                raise ValueError("storage must have shape [L, N, 2, H, k, d]")
            L, N, _, H, k, d = storage.shape
            code, self.act_dtype = _code(storage.dtype), storage.dtype
        self.storage = storage
        self.L, self.N, self.H, self.k, self.d = L, N, H, k, d
        self.dtype = storage.dtype
        handle = _lib.ctypes.c_void_p()
        _lib.check(_lib.lib().gist_pool_create(
            _lib.ctypes.byref(handle), L, N, k, H, d, code,
            _dev(storage, "storage"), storage.numel() * storage.element_size()),
            "gist_pool_create")
        self._handle = handle

    @property
    def handle(self):
        return self._handle

    def close(self):
        if getattr(self, "_handle", None) is not None and self._handle.value:
            _lib.lib().gist_pool_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gist_pool_create(storage: torch.Tensor, shape=None) -> GistPool:
    return GistPool(storage, shape)


def gist_pool_write(pool: GistPool, layer: int, ids: torch.Tensor, k_src: torch.Tensor,
                    v_src: torch.Tensor, src_pos0: int = 1, rope_base: float = 10000.0,
                    stream=None) -> None:
    n = ids.numel()
    shape = (n, pool.k, pool.H, pool.d)
    args = _ptrs((ids, "ids", torch.int32), (k_src, "k_src", pool.act_dtype, shape),
                 (v_src, "v_src", pool.act_dtype, shape))
    _lib.check(_lib.lib().gist_pool_write(pool.handle, layer, args[0], n, args[1], args[2],
                                          src_pos0, rope_base, _stream_ptr(stream)),
               "gist_pool_write")


def gist_attn_forward(pool: GistPool, layer: int, item_ids: torch.Tensor, q: torch.Tensor,
                      k_new: torch.Tensor, v_new: torch.Tensor, pos0: int | None = None,
                      rope_base: float = 10000.0, scale: float | None = None,
                      qpool: GistPool | None = None, q_ids: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [P, ell, Hq, d]; k_new, v_new [P, ell, H, d]; returns out [P, ell, Hq, d]."""
    if q.dim() != 4:
        raise ValueError("q must have shape [P, ell, Hq, d]")
    P, ell, Hq, d = q.shape
    if pos0 is None:
        pos0 = pool.k + (qpool.k if qpool is not None else 0) + 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    kv_shape = (P, ell, pool.H, pool.d)
    dt = pool.act_dtype
    ptrs = _ptrs((item_ids, "item_ids", torch.int32, (P,)), (q, "q", dt, (P, ell, Hq, pool.d)),
                 (k_new, "k_new", dt, kv_shape), (v_new, "v_new", dt, kv_shape),
                 (out, "out", dt, q.shape))
    qh, qi = None, None
    if qpool is not None:
        qh = qpool.handle
        qi = _dev(q_ids, "q_ids", torch.int32, (P,))
    _lib.check(_lib.lib().gist_attn_forward(pool.handle, layer, ptrs[0], P, ell, Hq, ptrs[1],
                                            ptrs[2], ptrs[3], pos0, rope_base, scale, qh, qi,
                                            ptrs[4], _stream_ptr(stream)), "gist_attn_forward")
    return out


class GroupedForward:
    """A prepared gist_attn_forward_grouped call: the group table is checked
    and marshalled once, and each call launches it (for loops that run the
    same groups repeatedly).  groups: a sequence of dicts with keys layer,
    item_ids, q [P, ell, Hq, d], k_new and v_new [P, ell, H, d], optional out,
    and q_ids when qpool is given (every group has the same ell and Hq)."""

    def __init__(self, pool: GistPool, groups, pos0: int | None = None,
                 rope_base: float = 10000.0, scale: float | None = None,
                 qpool: GistPool | None = None):
        groups = list(groups)
        self.pool, self.qpool, self.outs = pool, qpool, []
        self.ell = self.Hq = 0
        self.table = (_lib.GistGroup * max(len(groups), 1))()
        self.n = len(groups)
        if not groups:
            self.pos0, self.rope_base, self.scale = 0, rope_base, 1.0
            return
        q0 = groups[0]["q"]
        if q0.dim() != 4:
            raise ValueError("q must have shape [P, ell, Hq, d]")
        _, self.ell, self.Hq, d = q0.shape
        self.pos0 = pool.k + (qpool.k if qpool is not None else 0) + 1 if pos0 is None else pos0
        self.rope_base = rope_base
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        dt = pool.act_dtype
        # every group's tensors are checked before any is required to be on
        # the GPU (one _ptrs call over the whole table)
        specs, per = [], 6
        for gr in groups:
            q = gr["q"]
            if q.dim() != 4 or tuple(q.shape[1:]) != (self.ell, self.Hq, pool.d):
                raise ValueError("every group's q must have shape [P, ell, Hq, d] with one ell and Hq")
            P = q.shape[0]
            out = gr.get("out")
            if out is None:
                out = torch.empty_like(q)
            kv_shape = (P, self.ell, pool.H, pool.d)
            specs += [(gr["item_ids"], "item_ids", torch.int32, (P,)), (q, "q", dt, q.shape),
                      (gr["k_new"], "k_new", dt, kv_shape), (gr["v_new"], "v_new", dt, kv_shape),
                      (out, "out", dt, q.shape),
                      (gr["q_ids"], "q_ids", torch.int32, (P,)) if qpool is not None else None]
            self.outs.append(out)
        ptrs = _ptrs(*specs)
        for i, gr in enumerate(groups):
            item, q, kn, vn, out, qi = ptrs[per * i:per * (i + 1)]
            self.table[i] = _lib.GistGroup(int(gr["layer"]), groups[i]["q"].shape[0], item, qi, q,
                                           kn, vn, out)
        # the tensors stay referenced as long as the table points at them
        self._keep = groups

    def __call__(self, stream=None) -> list:
        _lib.check(_lib.lib().gist_attn_forward_grouped(
            self.pool.handle, self.qpool.handle if self.qpool is not None else None, self.table,
            self.n, self.ell, self.Hq, self.pos0, self.rope_base, self.scale, _stream_ptr(stream)),
            "gist_attn_forward_grouped")
        return self.outs


def gist_attn_forward_grouped(pool: GistPool, groups, pos0: int | None = None,
                              rope_base: float = 10000.0, scale: float | None = None,
                              qpool: GistPool | None = None, stream=None) -> list:
    """Several gist_attn_forward calls of one shape in one launch (groups as
    for GroupedForward); returns the outputs in group order."""
    groups = list(groups)
    if not groups:
        return []
    return GroupedForward(pool, groups, pos0, rope_base, scale, qpool)(stream)


def gist_attn_forward_last(pool: GistPool, layer: int, item_ids: torch.Tensor, q_last: torch.Tensor,
                           k_new: torch.Tensor, v_new: torch.Tensor, pos0: int | None = None,
                           rope_base: float = 10000.0, scale: float | None = None,
                           qpool: GistPool | None = None, q_ids: torch.Tensor | None = None,
                           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The last token only: q_last [P, Hq, d] (token ell-1); k_new, v_new
    [P, ell, H, d]; returns out [P, Hq, d], row ell-1 of gist_attn_forward."""
    if q_last.dim() != 3 or k_new.dim() != 4:
        raise ValueError("q_last must be [P, Hq, d] and k_new, v_new [P, ell, H, d]")
    P, Hq, d = q_last.shape
    ell = k_new.shape[1]
    if pos0 is None:
        pos0 = pool.k + (qpool.k if qpool is not None else 0) + 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q_last)
    kv_shape = (P, ell, pool.H, pool.d)
    dt = pool.act_dtype
    ptrs = _ptrs((item_ids, "item_ids", torch.int32, (P,)), (q_last, "q_last", dt, (P, Hq, pool.d)),
                 (k_new, "k_new", dt, kv_shape), (v_new, "v_new", dt, kv_shape),
                 (out, "out", dt, q_last.shape))
    qh, qi = None, None
    if qpool is not None:
        qh = qpool.handle
        qi = _dev(q_ids, "q_ids", torch.int32, (P,))
    _lib.check(_lib.lib().gist_attn_forward_last(
        pool.handle, layer, ptrs[0], P, ell, Hq, ptrs[1], ptrs[2], ptrs[3], pos0, rope_base, scale,
        qh, qi, ptrs[4], _stream_ptr(stream)), "gist_attn_forward_last")
    return out


def _paged_shapes(k_cache, q, k_new):
    """(n_blocks, H, block_size, d, P, ell, Hq, q shape, k_new shape) of a
    paged-gist call: q is [P, Hq, d] (ell = 1) or [P, ell, Hq, d]."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [n_blocks, H, block_size, d]")
    n_blocks, H, bs, d = k_cache.shape
    if q.dim() == 3:
        (P, Hq, _), ell = q.shape, 1
        q_shape, kv_shape = (P, Hq, d), (P, H, d)
    elif q.dim() == 4:
        P, ell, Hq, _ = q.shape
        q_shape, kv_shape = (P, ell, Hq, d), (P, ell, H, d)
    else:
        raise ValueError("q must be [P, Hq, d] or [P, ell, Hq, d]")
    return n_blocks, H, bs, d, P, ell, Hq, q_shape, kv_shape


def gist_attn_forward_paged(k_cache: torch.Tensor, v_cache: torch.Tensor, item_blocks: torch.Tensor,
                            k: int, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            query_blocks: torch.Tensor | None = None, kq: int = 0, q_row0: int = 0,
                            pos0: int | None = None, rope_base: float = 10000.0,
                            scale: float | None = None, out: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Gist attention over gists held in a paged cache: k_cache, v_cache bf16
    [n_blocks, H, block_size, d]; item gist = rows 0..k-1 of item_blocks[p],
    query gist = rows q_row0..q_row0+kq-1 of query_blocks[p]; q [P, Hq, d]
    (the EOS step, ell = 1) or [P, ell, Hq, d], k_new and v_new [P, H, d] or
    [P, ell, H, d]; returns out shaped like q."""
    n_blocks, H, bs, d, P, ell, Hq, q_shape, kv_shape = _paged_shapes(k_cache, q, k_new)
    if pos0 is None:
        pos0 = k + kq + 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    bf = torch.bfloat16
    ptrs = _ptrs((k_cache, "k_cache", bf), (v_cache, "v_cache", bf, k_cache.shape),
                 (item_blocks, "item_blocks", torch.int32, (P,)),
                 (query_blocks, "query_blocks", torch.int32, (P,)) if kq else None,
                 (q, "q", bf, q_shape), (k_new, "k_new", bf, kv_shape), (v_new, "v_new", bf, kv_shape),
                 (out, "out", bf, q.shape))
    _lib.check(_lib.lib().gist_attn_forward_paged(
        ptrs[0], ptrs[1], n_blocks, bs, ptrs[2], k, ptrs[3], kq, q_row0, P, ell, Hq, H, d, ptrs[4],
        ptrs[5], ptrs[6], pos0, rope_base, scale, ptrs[7], _stream_ptr(stream)),
        "gist_attn_forward_paged")
    return out


def gist_attn_forward_paged_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor,
                                k_scale: torch.Tensor, v_scale: torch.Tensor,
                                item_blocks: torch.Tensor, k: int, q: torch.Tensor,
                                k_new: torch.Tensor, v_new: torch.Tensor,
                                query_blocks: torch.Tensor | None = None, kq: int = 0,
                                q_row0: int = 0, pos0: int | None = None,
                                rope_base: float = 10000.0, scale: float | None = None,
                                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """gist_attn_forward_paged over an fp8 cache: k_cache, v_cache uint8 E4M3
    codes [n_blocks, H, block_size, d]; k_scale, v_scale fp32 [n_blocks, H];
    q, k_new, v_new bf16 as in gist_attn_forward_paged; returns out shaped
    like q."""
    n_blocks, H, bs, d, P, ell, Hq, q_shape, kv_shape = _paged_shapes(k_cache, q, k_new)
    if pos0 is None:
        pos0 = k + kq + 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    bf = torch.bfloat16
    ptrs = _ptrs((k_cache, "k_cache", torch.uint8), (v_cache, "v_cache", torch.uint8, k_cache.shape),
                 (k_scale, "k_scale", torch.float32, (n_blocks, H)),
                 (v_scale, "v_scale", torch.float32, (n_blocks, H)),
                 (item_blocks, "item_blocks", torch.int32, (P,)),
                 (query_blocks, "query_blocks", torch.int32, (P,)) if kq else None,
                 (q, "q", bf, q_shape), (k_new, "k_new", bf, kv_shape), (v_new, "v_new", bf, kv_shape),
                 (out, "out", bf, q.shape))
    _lib.check(_lib.lib().gist_attn_forward_paged_fp8(
        ptrs[0], ptrs[1], ptrs[2], ptrs[3], n_blocks, bs, ptrs[4], k, ptrs[5], kq, q_row0, P, ell, Hq,
        H, d, ptrs[6], ptrs[7], ptrs[8], pos0, rope_base, scale, ptrs[9], _stream_ptr(stream)),
        "gist_attn_forward_paged_fp8")
    return out


def gist_prefill_workspace_bytes(n_tokens: int, H: int, d: int) -> int:
    return _lib.lib().gist_prefill_workspace_bytes(n_tokens, H, d)


def gist_prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_start: torch.Tensor,
                      max_len: int | None = None, rope_base: float = 10000.0,
                      scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, pool: GistPool | None = None,
                      layer: int = 0, item_ids: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Causal attention over packed bf16 sequences [item ; gist] (one layer of
    the offline gist extraction): q [T, Hq, d], k, v [T, H, d], seq_start int32
    [B+1].  With a pool, each sequence's last pool.k tokens are stored as the
    gist of item item_ids[b].  Returns out [T, Hq, d]."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [T, Hq, d] and k, v [T, H, d]")
    T, Hq, d = q.shape
    H = k.shape[1]
    B = seq_start.numel() - 1
    if max_len is None:
        lens = (seq_start[1:] - seq_start[:-1]) if B > 0 else seq_start[:0]
        max_len = max(1, int(lens.max().item())) if B > 0 else 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(max(gist_prefill_workspace_bytes(T, H, d), 16), dtype=torch.uint8,
                                device=q.device)
    bf = torch.bfloat16
    ptrs = _ptrs((q, "q", bf), (k, "k", bf, (T, H, d)), (v, "v", bf, (T, H, d)),
                 (seq_start, "seq_start", torch.int32), (out, "out", bf, q.shape),
                 (workspace, "workspace"))
    ph, ids = None, None
    if pool is not None:
        ph = pool.handle
        ids = _dev(item_ids, "item_ids", torch.int32, (B,))
    _lib.check(_lib.lib().gist_prefill_attn(
        ptrs[0], ptrs[1], ptrs[2], ptrs[3], B, T, max_len, Hq, H, d, rope_base, scale, ptrs[4],
        ptrs[5], workspace.numel() * workspace.element_size(), ph, layer, ids,
        _stream_ptr(stream)), "gist_prefill_attn")
    return out


def paged_decode_workspace_bytes(R: int, Hq: int, max_blocks: int, block_size: int,
                                 d: int) -> int:
    return _lib.lib().paged_decode_workspace_bytes(R, Hq, max_blocks, block_size, d)


def paged_decode_attn(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                      context_lens: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                      v_new: torch.Tensor, positions: torch.Tensor, rope_base: float = 10000.0,
                      scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """k_cache, v_cache [n_blocks, H, block_size, d]; block_table [R, max_blocks];
    q [R, Hq, d]; k_new, v_new [R, H, d]; returns out [R, Hq, d]."""
    n_blocks, H, bs, d = k_cache.shape
    R, Hq, _ = q.shape
    if block_table.dim() != 2:
        raise ValueError("block_table must be [R, max_blocks]")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    need = paged_decode_workspace_bytes(R, Hq, max(max_blocks, 1), bs, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dt = k_cache.dtype
    ptrs = _ptrs((k_cache, "k_cache", dt), (v_cache, "v_cache", dt, k_cache.shape),
                 (block_table, "block_table", torch.int32, (R, max_blocks)),
                 (context_lens, "context_lens", torch.int32, (R,)),
                 (q, "q", dt, (R, Hq, d)), (k_new, "k_new", dt, (R, H, d)), (v_new, "v_new", dt, (R, H, d)),
                 (positions, "positions", torch.int32, (R,)), (out, "out", dt, q.shape),
                 (workspace, "workspace"))
    _lib.check(_lib.lib().paged_decode_attn(
        ptrs[0], ptrs[1], n_blocks, bs, ptrs[2], max_blocks, ptrs[3], R, ptrs[4], ptrs[5], ptrs[6],
        ptrs[7], Hq, H, d, _code(dt), rope_base, scale, ptrs[8], ptrs[9],
        workspace.numel() * workspace.element_size(), _stream_ptr(stream)), "paged_decode_attn")
    return out


def paged_decode_attn_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                          v_scale: torch.Tensor, block_table: torch.Tensor,
                          context_lens: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                          v_new: torch.Tensor, positions: torch.Tensor,
                          rope_base: float = 10000.0, scale: float | None = None,
                          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """k_cache, v_cache uint8 E4M3 codes [n_blocks, H, block_size, d]; k_scale, v_scale
    fp32 [n_blocks, H]; q [R, Hq, d], k_new, v_new [R, H, d] bf16; returns out [R, Hq, d]."""
    n_blocks, H, bs, d = k_cache.shape
    R, Hq, _ = q.shape
    if block_table.dim() != 2:
        raise ValueError("block_table must be [R, max_blocks]")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    need = paged_decode_workspace_bytes(R, Hq, max(max_blocks, 1), bs, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    bf = torch.bfloat16
    ptrs = _ptrs((k_cache, "k_cache", torch.uint8), (v_cache, "v_cache", torch.uint8, k_cache.shape),
                 (k_scale, "k_scale", torch.float32, (n_blocks, H)),
                 (v_scale, "v_scale", torch.float32, (n_blocks, H)),
                 (block_table, "block_table", torch.int32, (R, max_blocks)),
                 (context_lens, "context_lens", torch.int32, (R,)),
                 (q, "q", bf, (R, Hq, d)), (k_new, "k_new", bf, (R, H, d)), (v_new, "v_new", bf, (R, H, d)),
                 (positions, "positions", torch.int32, (R,)), (out, "out", bf, q.shape),
                 (workspace, "workspace"))
    _lib.check(_lib.lib().paged_decode_attn_fp8(
        ptrs[0], ptrs[1], ptrs[2], ptrs[3], n_blocks, bs, ptrs[4], max_blocks, ptrs[5], R, ptrs[6],
        ptrs[7], ptrs[8], ptrs[9], Hq, H, d, rope_base, scale, ptrs[10], ptrs[11],
        workspace.numel() * workspace.element_size(), _stream_ptr(stream)), "paged_decode_attn_fp8")
    return out


def paged_decode_attn_noalloc(k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_table: torch.Tensor, context_lens: torch.Tensor,
                              q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                              positions: torch.Tensor, rope_base: float = 10000.0,
                              scale: float | None = None, out: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """paged_decode_attn with the library's own split-K scratch (no workspace;
    the C call allocates nothing).  Calls that overlap on one GPU race."""
    n_blocks, H, bs, d = k_cache.shape
    R, Hq, _ = q.shape
    if block_table.dim() != 2:
        raise ValueError("block_table must be [R, max_blocks]")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    dt = k_cache.dtype
    ptrs = _ptrs((k_cache, "k_cache", dt), (v_cache, "v_cache", dt, k_cache.shape),
                 (block_table, "block_table", torch.int32, (R, max_blocks)),
                 (context_lens, "context_lens", torch.int32, (R,)),
                 (q, "q", dt, (R, Hq, d)), (k_new, "k_new", dt, (R, H, d)), (v_new, "v_new", dt, (R, H, d)),
                 (positions, "positions", torch.int32, (R,)), (out, "out", dt, q.shape))
    _lib.check(_lib.lib().paged_decode_attn_noalloc(
        ptrs[0], ptrs[1], n_blocks, bs, ptrs[2], max_blocks, ptrs[3], R, ptrs[4], ptrs[5], ptrs[6],
        ptrs[7], Hq, H, d, _code(dt), rope_base, scale, ptrs[8], _stream_ptr(stream)),
        "paged_decode_attn_noalloc")
    return out
