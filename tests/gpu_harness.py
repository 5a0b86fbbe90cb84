"""Shared helpers for the GPU tests: build device inputs from a seeded
workload, run the library through its Python binding, and build the
oracle's view of the same inputs.  The oracle side never sees a value the
GPU computed."""
from __future__ import annotations

import numpy as np
import torch

from mla_synth import Workload
from oracle import fp8, mla_oracle

SENTINEL_BYTE = 0xA5


def tdtype(wl: Workload):
    return torch.bfloat16 if wl.shape.dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, dtype, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev).to(dtype)


def i32(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(dev)


class GpuCase:
    """Device-side state of one workload: folded layer, filled cache, queries."""

    def __init__(self, wl: Workload, dev="cuda", fill_sentinel=True, seq_group=8):
        import mla_compressed_latent_amd as mla
        self.mla = mla
        self.wl = wl
        s = wl.shape
        dt = tdtype(wl)
        self.dt = dt
        self.cfg = mla.config_from_shape(s)
        self.w_dkv = wl.w_dkv()
        self.w_uk = wl.w_uk()
        self.w_uv = wl.w_uv()
        self.layer = mla.mla_fold_weights(self.cfg, to_dev(self.w_dkv, dt), to_dev(self.w_uk, dt),
                                          to_dev(self.w_uv, dt))
        table, num_pages = wl.page_table()
        self.table_np = table
        self.page_table = i32(table)
        self.num_pages = num_pages
        if s.cache_format == "fp8":   # pages of 640-byte rows, then the rows' fp32 scales
            self.cache = torch.empty((num_pages, s.page_size * s.cache_token_bytes), dtype=torch.uint8,
                                     device=dev)
        else:
            self.cache = torch.empty((num_pages, s.page_size, s.row_width), dtype=dt, device=dev)
        if fill_sentinel:
            self.cache.view(torch.uint8).fill_(SENTINEL_BYTE)
        self.prefix = wl.prefix_lens()
        self.q_lens = wl.q_lens()
        self.seq_lens_np = wl.seq_lens()
        self.seq_lens = i32(self.seq_lens_np)
        self.cu_q = i32(wl.cu_q())
        self.max_q_len = int(self.q_lens.max())
        self.max_seq_len = int(self.seq_lens_np.max())
        self._fill_prefix(seq_group)
        # new tokens: append, then they are the queries
        self.x_new = wl.new_hidden()
        self.q = wl.queries()
        self.q_dev = to_dev(self.q, dt)
        self.x_new_dev = to_dev(self.x_new, dt)
        self.prefix_dev = i32(self.prefix)

    def _fill_prefix(self, seq_group):
        import concurrent.futures as cf
        wl, mla = self.wl, self.mla
        B = wl.batch
        pool = cf.ThreadPoolExecutor(max_workers=8)   # the generator's draws release the GIL
        if wl.prefix_source == "hidden":
            for b0 in range(0, B, seq_group):
                bs = list(range(b0, min(B, b0 + seq_group)))
                xs = list(pool.map(wl.prefix_hidden, bs))
                lens = np.array([x.shape[0] for x in xs], dtype=np.int64)
                cu = np.zeros(B + 1, dtype=np.int64)
                for j, b in enumerate(bs):
                    cu[b + 1] = lens[j]
                cu = np.cumsum(cu)
                x = to_dev(np.concatenate(xs, axis=0), self.dt)
                mla.mla_append_latent(self.layer, x, i32(cu), i32(np.zeros(B)), self.page_table, self.cache)
                del x
        else:
            if wl.shape.cache_format == "fp8":
                raise ValueError("fp8 caches are filled through the append path (hidden prefixes)")
            ps = wl.shape.page_size
            futs = {b: pool.submit(wl.prefix_latent, b) for b in range(min(B, 16))}
            for b in range(B):
                rows = futs.pop(b).result()
                if b + 16 < B:
                    futs[b + 16] = pool.submit(wl.prefix_latent, b + 16)
                rd = to_dev(rows, self.dt)
                P = rows.shape[0]
                for p0 in range(0, P, ps):
                    page = int(self.table_np[b, p0 // ps])
                    n = min(ps, P - p0)
                    self.cache[page, :n] = rd[p0:p0 + n]
        pool.shutdown()
        torch.cuda.synchronize()

    def append_new(self, stream=None):
        self.mla.mla_append_latent(self.layer, self.x_new_dev, self.cu_q, self.prefix_dev, self.page_table,
                                   self.cache, stream=stream)

    def decode(self, kv_chunk=0, out=None, stream=None):
        s = self.wl.shape
        if out is None:
            out = torch.empty((self.q.shape[0], s.H, s.d_v), dtype=self.dt, device=self.q_dev.device)
        self.mla.mla_decode(self.layer, self.q_dev, self.cu_q, self.seq_lens, self.page_table, self.cache, out,
                            self.max_q_len, self.max_seq_len, kv_chunk=kv_chunk, stream=stream)
        return out

    def extend(self, path, out=None, workspace=None, stream=None):
        s = self.wl.shape
        if out is None:
            out = torch.empty((self.q.shape[0], s.H, s.d_v), dtype=self.dt, device=self.q_dev.device)
        self.mla.mla_extend(self.layer, self.q_dev, self.cu_q, self.seq_lens, self.page_table, self.cache, out,
                            self.max_q_len, self.max_seq_len, path=path, workspace=workspace, stream=stream)
        return out

    def logical_rows(self, b):
        """Sequence b's cached rows as stored on the GPU (for placement checks)."""
        ps = self.wl.shape.page_size
        L = int(self.seq_lens_np[b])
        pages = self.table_np[b, : (L + ps - 1) // ps]
        rows = self.cache[torch.from_numpy(pages.astype(np.int64)).to(self.cache.device)].reshape(-1, self.cache.shape[-1])
        return rows[:L]


def oracle_cache(wl: Workload, b: int, w_dkv=None, quantize=True) -> np.ndarray:
    """The oracle's float64 rows of sequence b after the new tokens are
    appended (for an fp8 cache: with the latent quantized and dequantized by
    the oracle's own row quantizer, unless quantize is False)."""
    s = wl.shape
    w_dkv = wl.w_dkv() if w_dkv is None else w_dkv
    P = int(wl.prefix_lens()[b])
    if wl.prefix_source == "hidden":
        pre = mla_oracle.latent_rows(wl.prefix_hidden(b), w_dkv, np.arange(P), s.d_c, s.rope_base)
    else:
        pre = wl.prefix_latent(b).astype(np.float64)
    new = mla_oracle.latent_rows(wl.new_hidden(b), w_dkv, P + np.arange(int(wl.q_lens()[b])), s.d_c, s.rope_base)
    rows = np.concatenate([pre, new], axis=0)
    if s.cache_format == "fp8" and quantize:
        rows = fp8.fp8_rows(rows, s.d_c)
    return rows


def oracle_outputs(wl: Workload, b: int, heads=None, w_dkv=None, w_uk=None, w_uv=None) -> np.ndarray:
    """Oracle output [q_len_b][len(heads)][d_v] for sequence b."""
    s = wl.shape
    cache = oracle_cache(wl, b, w_dkv)
    w_uk = wl.w_uk() if w_uk is None else w_uk
    w_uv = wl.w_uv() if w_uv is None else w_uv
    scale = mla_oracle.default_scale(s.d_nope, s.d_rope)
    return mla_oracle.attend_sequence(wl.queries(b), cache, w_uk, w_uv, s.H, s.d_nope, s.d_v, s.rope_base,
                                      scale, heads)


def oracle_query(wl: Workload, b: int, i: int, heads, cache: np.ndarray, q_b: np.ndarray, w_uk, w_uv) -> np.ndarray:
    """Oracle output [len(heads)][d_v] of query i of sequence b alone: the
    query sits at position L - q_len + i, so it is the last query of the
    oracle's call over rows 0 .. that position."""
    s = wl.shape
    L, lq = cache.shape[0], q_b.shape[0]
    pos = L - lq + i
    scale = mla_oracle.default_scale(s.d_nope, s.d_rope)
    return mla_oracle.attend_sequence(q_b[i:i + 1], cache[:pos + 1], w_uk, w_uv, s.H, s.d_nope, s.d_v,
                                      s.rope_base, scale, heads)[0]


def errors(gpu: np.ndarray, ref: np.ndarray):
    """(max|d| / max|ref|, rms(d) / rms(ref), max|d| / rms(ref)) for d = gpu - ref."""
    ref = np.asarray(ref, np.float64)
    d = np.asarray(gpu, np.float64) - ref
    rms = np.sqrt(np.mean(ref ** 2))
    return (float(np.abs(d).max() / np.abs(ref).max()), float(np.sqrt(np.mean(d ** 2)) / rms),
            float(np.abs(d).max() / rms))
