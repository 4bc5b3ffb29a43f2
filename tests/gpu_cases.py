"""Helpers shared by the GPU parity tests: build seeded inputs on the device,
run the library through its C ABI (via the ctypes binding), copy the exact
device values back and compare with the fp64 oracle."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import gist_compressed_kv_amd as G
from gist_compressed_kv_amd import synth
from oracle import gist_oracle as O

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}
ROPE_BASE = 10000.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


class GistCase:
    """One layer-set of gist attention inputs on the GPU."""

    def __init__(self, layers, n_items, k, ell, hq, h, d, pairs, dtype, seed, kq=0,
                 n_qrows=0, ids=None, q_ids=None, device="cuda", fp8=False, act_layers=None):
        """act_layers: the layers that get activations (default: all); the
        pools always hold every layer."""
        self.layers, self.n_items, self.k, self.ell = layers, n_items, k, ell
        self.hq, self.h, self.d, self.pairs, self.dtype, self.kq = hq, h, d, pairs, dtype, kq
        self.fp8 = fp8
        if fp8:  # E4M3 gist pools; activations in bf16
            self.dtype = dtype = torch.bfloat16
            self.pool_t = synth.randn_fp8_gist_pool(layers, n_items, k, h, d,
                                                    synth.tensor_seed(seed, 1), device)
            self.pool = G.GistPool(self.pool_t, shape=(layers, n_items, k, h, d))
        else:
            self.pool_t = synth.randn((layers, n_items, 2, h, k, d), synth.tensor_seed(seed, 1),
                                      dtype, device)
            self.pool = G.GistPool(self.pool_t)
        if ids is None:
            ids = torch.randint(0, n_items, (pairs,), generator=synth.generator(seed, "cpu"),
                                dtype=torch.int32)
        self.ids = ids.to(device=device, dtype=torch.int32)
        self.qpool_t = self.qpool = self.q_ids = None
        if kq and fp8:
            self.qpool_t = synth.randn_fp8_gist_pool(layers, n_qrows, kq, h, d,
                                                     synth.tensor_seed(seed, 2), device)
            self.qpool = G.GistPool(self.qpool_t, shape=(layers, n_qrows, kq, h, d))
            self.q_ids = q_ids.to(device=device, dtype=torch.int32)
        elif kq:
            self.qpool_t = synth.randn((layers, n_qrows, 2, h, kq, d), synth.tensor_seed(seed, 2),
                                       dtype, device)
            self.qpool = G.GistPool(self.qpool_t)
            self.q_ids = q_ids.to(device=device, dtype=torch.int32)
        self.act_layers = list(range(layers)) if act_layers is None else list(act_layers)
        self.q, self.kn, self.vn = {}, {}, {}
        for li in self.act_layers:
            self.q[li] = synth.randn((pairs, ell, hq, d), synth.tensor_seed(seed, 3, li), dtype, device)
            self.kn[li] = synth.randn((pairs, ell, h, d), synth.tensor_seed(seed, 4, li), dtype, device)
            self.vn[li] = synth.randn((pairs, ell, h, d), synth.tensor_seed(seed, 5, li), dtype, device)
        self.pos0 = k + kq + 1
        self.scale = 1.0 / math.sqrt(d)

    def run(self, layer, out=None):
        return G.gist_attn_forward(self.pool, layer, self.ids, self.q[layer], self.kn[layer],
                                   self.vn[layer], self.pos0, ROPE_BASE, self.scale,
                                   qpool=self.qpool, q_ids=self.q_ids, out=out)

    def run_last(self, layer, out=None):
        """gist_attn_forward_last with the last token's Q of this case."""
        return G.gist_attn_forward_last(self.pool, layer, self.ids, self.q[layer][:, -1].contiguous(),
                                        self.kn[layer], self.vn[layer], self.pos0, ROPE_BASE,
                                        self.scale, qpool=self.qpool, q_ids=self.q_ids, out=out)

    def oracle(self, layer, sample):
        """Oracle rows for the sampled pairs; only the referenced pool rows are
        copied back."""
        sample = np.asarray(sample)
        idx = torch.as_tensor(sample, device=self.ids.device)
        ids = self.ids[idx].long()
        pool = self._rows(self.pool, layer, ids)  # [1][S][2][H][k][d]
        qpool = qids = None
        if self.qpool is not None:
            qr = self.q_ids[idx].long()
            qpool = self._rows(self.qpool, layer, qr)
            qids = np.arange(len(sample))
        return O.gist_attn_forward(pool, 0, np.arange(len(sample)), f64(self.q[layer][idx]),
                                   f64(self.kn[layer][idx]), f64(self.vn[layer][idx]),
                                   self.pos0, ROPE_BASE, self.scale, qpool=qpool, q_ids=qids)

    @staticmethod
    def _rows(pool, layer, rows):
        """Pool records of the given rows of one layer, as fp64 values
        [1][S][2][H][k][d] (fp8 pools: decoded and scaled by the oracle)."""
        if pool.fp8:
            return O.dequantize_gist(pool.codes[layer][rows].cpu().numpy(),
                                     pool.scales[layer][rows].cpu().numpy())[None]
        return f64(pool.storage[layer][rows])[None]

    def max_err(self, layer, out, sample):
        ref = self.oracle(layer, sample)
        got = f64(out[torch.as_tensor(np.asarray(sample), device=out.device)])
        assert np.isfinite(got).all(), "non-finite output"
        return float(np.abs(got - ref).max())


class DecodeCase:
    def __init__(self, n_blocks, h, bs, d, hq, lens, dtype, seed, table=None, max_blocks=None,
                 device="cuda", fp8=False):
        self.fp8 = fp8
        if fp8:  # E4M3 codes with per-(block, head) scales; activations in bf16
            dtype = torch.bfloat16
            self.kc, self.ksc = synth.randn_fp8_blocks((n_blocks, h, bs, d),
                                                       synth.tensor_seed(seed, 11), device)
            self.vc, self.vsc = synth.randn_fp8_blocks((n_blocks, h, bs, d),
                                                       synth.tensor_seed(seed, 12), device)
        else:
            self.kc = synth.randn((n_blocks, h, bs, d), synth.tensor_seed(seed, 11), dtype, device)
            self.vc = synth.randn((n_blocks, h, bs, d), synth.tensor_seed(seed, 12), dtype, device)
        R = len(lens)
        if max_blocks is None:
            max_blocks = max(1, -(-max(lens) // bs))
        if table is None:
            table = synth.block_table(R, max_blocks, n_blocks, seed, device)
        self.table = table.to(device=device, dtype=torch.int32)
        self.lens = torch.as_tensor(lens, dtype=torch.int32, device=device)
        self.positions = self.lens + 1
        self.q = synth.randn((R, hq, d), synth.tensor_seed(seed, 13), dtype, device)
        self.kn = synth.randn((R, h, d), synth.tensor_seed(seed, 14), dtype, device)
        self.vn = synth.randn((R, h, d), synth.tensor_seed(seed, 15), dtype, device)
        self.scale = 1.0 / math.sqrt(d)
        self.dtype = dtype

    def run(self, out=None, workspace=None):
        if self.fp8:
            return G.paged_decode_attn_fp8(self.kc, self.vc, self.ksc, self.vsc, self.table,
                                           self.lens, self.q, self.kn, self.vn, self.positions,
                                           ROPE_BASE, self.scale, out=out, workspace=workspace)
        return G.paged_decode_attn(self.kc, self.vc, self.table, self.lens, self.q, self.kn,
                                   self.vn, self.positions, ROPE_BASE, self.scale, out=out,
                                   workspace=workspace)

    def oracle(self, reqs=None):
        R = self.q.shape[0]
        reqs = np.arange(R) if reqs is None else np.asarray(reqs)
        table = self.table.cpu().numpy()[reqs]
        lens = self.lens.cpu().numpy()[reqs]
        # copy back only the referenced blocks
        used = sorted({int(b) for r in range(len(reqs))
                       for b in table[r][: -(-int(lens[r]) // self.kc.shape[2])]} | {0})
        remap = {b: i for i, b in enumerate(used)}
        used_t = torch.as_tensor(used, device=self.kc.device)
        if self.fp8:
            kc = O.dequantize_blocks(self.kc[used_t].cpu().numpy(), self.ksc[used_t].cpu().numpy())
            vc = O.dequantize_blocks(self.vc[used_t].cpu().numpy(), self.vsc[used_t].cpu().numpy())
        else:
            kc = f64(self.kc[used_t])
            vc = f64(self.vc[used_t])
        t2 = np.vectorize(lambda b: remap.get(int(b), 0))(table)
        idx = torch.as_tensor(reqs, device=self.q.device)
        return O.paged_decode(kc, vc, t2, lens, f64(self.q[idx]), f64(self.kn[idx]),
                              f64(self.vn[idx]), self.positions.cpu().numpy()[reqs], ROPE_BASE,
                              self.scale)


class PrefillCase:
    """Packed bf16 sequences [item ; gist] for the offline gist extraction."""

    def __init__(self, lens, hq, h, d, seed, device="cuda"):
        self.lens = list(lens)
        self.hq, self.h, self.d = hq, h, d
        T = sum(self.lens)
        self.T = T
        st = np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32)
        self.seq_start = torch.as_tensor(st, device=device)
        self.q = synth.randn((T, hq, d), synth.tensor_seed(seed, 21), torch.bfloat16, device)
        self.k = synth.randn((T, h, d), synth.tensor_seed(seed, 22), torch.bfloat16, device)
        self.v = synth.randn((T, h, d), synth.tensor_seed(seed, 23), torch.bfloat16, device)
        self.scale = 1.0 / math.sqrt(d)

    def run(self, out=None, pool=None, layer=0, item_ids=None):
        return G.gist_prefill_attn(self.q, self.k, self.v, self.seq_start, max(self.lens), ROPE_BASE,
                                   self.scale, out=out, pool=pool, layer=layer, item_ids=item_ids)

    def oracle(self, seqs=None):
        """Oracle rows of the listed sequences, as (rows index, values)."""
        seqs = range(len(self.lens)) if seqs is None else seqs
        st = self.seq_start.cpu().numpy()
        idx, vals = [], []
        for b in seqs:
            s = slice(int(st[b]), int(st[b + 1]))
            ref = O.prefill_attention(f64(self.q[s]), f64(self.k[s]), f64(self.v[s]),
                                      [0, self.lens[b]], ROPE_BASE, self.scale)
            idx.append(np.arange(s.start, s.stop))
            vals.append(ref)
        return np.concatenate(idx), np.concatenate(vals)

    def max_err(self, out, seqs=None):
        idx, ref = self.oracle(seqs)
        got = f64(out[torch.as_tensor(idx, device=out.device)])
        assert np.isfinite(got).all(), "non-finite output"
        return float(np.abs(got - ref).max())
