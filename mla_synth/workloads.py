"""Seeded synthetic workloads for one MLA decode layer.

Every tensor is drawn from ``numpy.random.default_rng`` (PCG64), keyed by
``SeedSequence(entropy=seed, spawn_key=(stream, [sequence]))`` so that any
one sequence's data can be regenerated without drawing the others.  Values
are standard normal, weights scaled by ``1/sqrt(fan_in)``; everything is
rounded to the storage dtype (round-to-nearest-even for bf16) before either
side sees it, so the GPU library and the oracle receive identical numbers.

Shapes follow the five workloads the decode step is measured on: a tiny fp32
case, the DeepSeek-V2 shape (128 heads, d_c 512, d_rope 64) at batch 32 x
4096, the Llama-2-7B shape with an MLA latent (32 heads) at batch 64 x 8192,
the DeepSeek-V2 shape at batch 8 x 131072, and a ragged paged batch of 256
sequences.  The field names of ``Shape`` reuse the Hugging Face config
names quoted on the glossary page "Multi-Head Latent Attention (MLA)".
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

# Stream identifiers: one independent random stream per input tensor kind.
STREAM_W_DKV = 0
STREAM_W_UK = 1
STREAM_W_UV = 2
STREAM_PREFIX = 3
STREAM_X_NEW = 4
STREAM_CTX = 5
STREAM_QLEN = 6
STREAM_PAGES = 7
STREAM_Q = 8
STREAM_W_O = 9
STREAM_W_Q = 10


# ---------------------------------------------------------------- bf16 I/O --
def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs must be finite float32.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ shapes --
@dataclass(frozen=True)
class Shape:
    d_model: int
    num_attention_heads: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    v_head_dim: int
    kv_lora_rank: int
    dtype: str = "bf16"          # "bf16" or "f32": storage dtype of every tensor
    rope_base: float = 10000.0
    page_size: int = 64
    cache_format: str = "dtype"  # "dtype": rows in dtype; "fp8": 8-bit float latent pages

    # short aliases
    @property
    def H(self) -> int:
        return self.num_attention_heads

    @property
    def d_nope(self) -> int:
        return self.qk_nope_head_dim

    @property
    def d_rope(self) -> int:
        return self.qk_rope_head_dim

    @property
    def d_v(self) -> int:
        return self.v_head_dim

    @property
    def d_c(self) -> int:
        return self.kv_lora_rank

    @property
    def row_width(self) -> int:
        """Elements in one cached row: the latent followed by the rope key."""
        return self.kv_lora_rank + self.qk_rope_head_dim

    @property
    def cache_token_bytes(self) -> int:
        """Bytes one cached token takes in a page (row, plus its scale for fp8)."""
        if self.cache_format == "fp8":
            return 512 + 2 * self.qk_rope_head_dim + 4
        return self.row_width * self.elem_bytes

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


TINY = Shape(64, 4, 16, 8, 16, 32, dtype="f32")
DSV2 = Shape(5120, 128, 128, 64, 128, 512)
LLAMA2_7B_MLA = Shape(4096, 32, 128, 64, 128, 512)


@dataclass(frozen=True)
class Workload:
    """One decode step's inputs: B sequences, each with a cached prefix and
    q_len new tokens that are appended to the cache and then used as queries.
    """

    name: str
    shape: Shape
    batch: int
    seed: int
    prefix_source: str                # "hidden": prefix latents come from hidden states
                                      # "latent": prefix rows are drawn directly
    paging: str = "identity"          # "identity" or "random"
    fixed_prefix: Optional[int] = None
    max_prefix: int = 0               # ragged: prefix ~ U{1..max_prefix}
    fixed_q_len: Optional[int] = 1
    max_q_len: int = 1                # ragged: q_len ~ U{1..max_q_len}
    spare_page_frac: float = 0.0
    description: str = ""
    kind: str = "decode"              # "decode": the step is append + mla_decode;
                                      # "extend": append + mla_extend (long chunks);
                                      # "project": append + mla_decode_project
                                      # "hidden": append + mla_decode_hidden
    layers: int = 0                   # > 0: a stack of this many layers sharing one
                                      # page-pool table (one timed pass = all layers)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    # ------------------------------------------------------------ streams
    def rng(self, stream: int, *key: int) -> np.random.Generator:
        ss = np.random.SeedSequence(entropy=self.seed, spawn_key=(stream,) + tuple(key))
        return np.random.default_rng(ss)

    def _store(self, a: np.ndarray) -> np.ndarray:
        return round_to_bf16(a) if self.shape.dtype == "bf16" else np.ascontiguousarray(a, np.float32)

    def _normal(self, rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
        a = rng.standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        return self._store(a)

    # ------------------------------------------------------------ lengths
    def prefix_lens(self) -> np.ndarray:
        if self.fixed_prefix is not None:
            return np.full(self.batch, self.fixed_prefix, dtype=np.int32)
        r = self.rng(STREAM_CTX)
        return r.integers(1, self.max_prefix + 1, size=self.batch, dtype=np.int64).astype(np.int32)

    def q_lens(self) -> np.ndarray:
        if self.fixed_q_len is not None:
            return np.full(self.batch, self.fixed_q_len, dtype=np.int32)
        r = self.rng(STREAM_QLEN)
        return r.integers(1, self.max_q_len + 1, size=self.batch, dtype=np.int64).astype(np.int32)

    def seq_lens(self) -> np.ndarray:
        return (self.prefix_lens().astype(np.int64) + self.q_lens()).astype(np.int32)

    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens())]).astype(np.int32)

    def total_q(self) -> int:
        return int(self.q_lens().sum())

    # ------------------------------------------------------------ weights
    def w_dkv(self) -> np.ndarray:
        s = self.shape
        return self._normal(self.rng(STREAM_W_DKV), (s.d_model, s.row_width), 1.0 / np.sqrt(s.d_model))

    def w_uk(self) -> np.ndarray:
        s = self.shape
        return self._normal(self.rng(STREAM_W_UK), (s.d_c, s.H * s.d_nope), 1.0 / np.sqrt(s.d_c))

    def w_uv(self) -> np.ndarray:
        s = self.shape
        return self._normal(self.rng(STREAM_W_UV), (s.d_c, s.H * s.d_v), 1.0 / np.sqrt(s.d_c))

    def w_o(self) -> np.ndarray:
        """Output projection [H * d_v][d_model]: concatenated heads -> hidden size."""
        s = self.shape
        return self._normal(self.rng(STREAM_W_O), (s.H * s.d_v, s.d_model), 1.0 / np.sqrt(s.H * s.d_v))

    def w_q(self) -> np.ndarray:
        """Query projection [d_model][H * (d_nope + d_rope)]: head h owns the
        columns h*(d_nope + d_rope) .., its content part first."""
        s = self.shape
        return self._normal(self.rng(STREAM_W_Q), (s.d_model, s.H * (s.d_nope + s.d_rope)),
                            1.0 / np.sqrt(s.d_model))

    # ------------------------------------------------------------ activations
    def prefix_hidden(self, b: int) -> np.ndarray:
        """Hidden states of sequence b's cached prefix, [P_b][d_model]."""
        assert self.prefix_source == "hidden"
        p = int(self.prefix_lens()[b])
        return self._normal(self.rng(STREAM_PREFIX, b), (p, self.shape.d_model))

    def prefix_latent(self, b: int) -> np.ndarray:
        """Directly drawn cached rows of sequence b's prefix, [P_b][d_c + d_rope].

        These rows are the cache contents as given (the rope block is taken
        as already rotated)."""
        assert self.prefix_source == "latent"
        p = int(self.prefix_lens()[b])
        return self._normal(self.rng(STREAM_PREFIX, b), (p, self.shape.row_width))

    def new_hidden(self, b: Optional[int] = None) -> np.ndarray:
        """Hidden states of the new tokens, [q_len_b][d_model] for one
        sequence, or all sequences concatenated in batch order."""
        ql = self.q_lens()
        if b is not None:
            return self._normal(self.rng(STREAM_X_NEW, b), (int(ql[b]), self.shape.d_model))
        return np.concatenate([self.new_hidden(i) for i in range(self.batch)], axis=0)

    def queries(self, b: Optional[int] = None) -> np.ndarray:
        """Pre-rotation queries [q_len][H][d_nope + d_rope] (the model's W_q
        projection is outside the layer; its output is drawn directly)."""
        s = self.shape
        ql = self.q_lens()
        if b is not None:
            return self._normal(self.rng(STREAM_Q, b), (int(ql[b]), s.H, s.d_nope + s.d_rope))
        return np.concatenate([self.queries(i) for i in range(self.batch)], axis=0)

    # ------------------------------------------------------------ paging
    def pages_per_seq(self) -> np.ndarray:
        ps = self.shape.page_size
        return ((self.seq_lens().astype(np.int64) + ps - 1) // ps).astype(np.int32)

    def page_table(self):
        """Returns (table [B][max_pages] int32 padded with -1, num_pages)."""
        npg = self.pages_per_seq()
        max_pages = int(npg.max())
        table = np.full((self.batch, max_pages), -1, dtype=np.int32)
        if self.paging == "identity":
            for b in range(self.batch):
                table[b, : npg[b]] = b * max_pages + np.arange(npg[b], dtype=np.int32)
            return table, self.batch * max_pages
        needed = int(npg.sum())
        total = needed + int(np.ceil(self.spare_page_frac * needed))
        perm = self.rng(STREAM_PAGES).permutation(total).astype(np.int32)
        off = 0
        for b in range(self.batch):
            table[b, : npg[b]] = perm[off: off + npg[b]]
            off += int(npg[b])
        return table, total


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", TINY, batch=1, seed=1, prefix_source="hidden", fixed_prefix=127,
        description="fp32; d_model 64, 4 heads, d_nope 16, d_rope 8, d_v 16, d_c 32; "
                    "batch 1, context 128, 1 query token; contiguous cache"),
    "dsv2_b32_ctx4096": Workload(
        "dsv2_b32_ctx4096", DSV2, batch=32, seed=2, prefix_source="hidden", fixed_prefix=4095,
        description="bf16; DeepSeek-V2 shape, batch 32, every context 4096, q_len 1"),
    "llama2_7b_mla_b64_ctx8192": Workload(
        "llama2_7b_mla_b64_ctx8192", LLAMA2_7B_MLA, batch=64, seed=3, prefix_source="hidden",
        fixed_prefix=8191,
        description="bf16; Llama-2-7B shape with a 512-wide latent, batch 64, every context 8192"),
    "dsv2_b8_ctx131072": Workload(
        "dsv2_b8_ctx131072", DSV2, batch=8, seed=4, prefix_source="latent", fixed_prefix=131071,
        description="bf16; DeepSeek-V2 shape, batch 8, every context 131072 (1.2 GB of latent)"),
    "dsv2_ragged_paged_256": Workload(
        "dsv2_ragged_paged_256", DSV2, batch=256, seed=5, prefix_source="latent", paging="random",
        fixed_prefix=None, max_prefix=32768, fixed_q_len=None, max_q_len=2, spare_page_frac=0.05,
        description="bf16; DeepSeek-V2 shape, 256 sequences, prefix ~ U[1, 32768], q_len ~ U{1,2}, "
                    "64-token pages under a random page table, new tokens appended first"),
    "dsv2_b32_ctx4096_fp8": Workload(
        "dsv2_b32_ctx4096_fp8", replace(DSV2, cache_format="fp8"), batch=32, seed=2, prefix_source="hidden",
        fixed_prefix=4095,
        description="bf16 layer over an FP8 latent cache (E4M3 codes, per-row power-of-two scale); "
                    "DeepSeek-V2 shape, batch 32, every context 4096, q_len 1"),
    "llama2_7b_mla_b64_ctx8192_fp8": Workload(
        "llama2_7b_mla_b64_ctx8192_fp8", replace(LLAMA2_7B_MLA, cache_format="fp8"), batch=64, seed=3,
        prefix_source="hidden", fixed_prefix=8191,
        description="bf16 layer over an FP8 latent cache; Llama-2-7B shape with a 512-wide latent, "
                    "batch 64, every context 8192"),
    "dsv2_b32_ctx4096_project": Workload(
        "dsv2_b32_ctx4096_project", DSV2, batch=32, seed=2, prefix_source="hidden", fixed_prefix=4095,
        kind="project",
        description="bf16; DeepSeek-V2 shape, batch 32, every context 4096, q_len 1, decode and the "
                    "output projection W_o (the value up-projection folded into it or not)"),
    "dsv2_b32_ctx4096_hidden": Workload(
        "dsv2_b32_ctx4096_hidden", DSV2, batch=32, seed=2, prefix_source="hidden", fixed_prefix=4095,
        kind="hidden",
        description="bf16; DeepSeek-V2 shape, batch 32, every context 4096, q_len 1, decode with the "
                    "queries projected from the layer input (W_uk folded into W_q or not)"),
    "dsv2_60layers_b32_ctx4096": Workload(
        "dsv2_60layers_b32_ctx4096", DSV2, batch=32, seed=2, prefix_source="hidden", fixed_prefix=4095,
        layers=60,
        description="bf16; DeepSeek-V2 shape, all 60 layers (one page-pool table), batch 32, "
                    "every context 4096, q_len 1"),
    "dsv2_extend_b4_p3072_c1024": Workload(
        "dsv2_extend_b4_p3072_c1024", DSV2, batch=4, seed=6, prefix_source="hidden", fixed_prefix=3072,
        fixed_q_len=1024, max_q_len=1024, kind="extend",
        description="bf16; DeepSeek-V2 shape, chunked extend: 4 sequences, cached prefix 3072, "
                    "a 1024-token chunk appended and attended causally (context 4096)"),
    "dsv2_prefill_b2_4096": Workload(
        "dsv2_prefill_b2_4096", DSV2, batch=2, seed=7, prefix_source="hidden", fixed_prefix=0,
        fixed_q_len=4096, max_q_len=4096, kind="extend",
        description="bf16; DeepSeek-V2 shape, prefill: 2 sequences of 4096 new tokens, empty cache"),
}


def workload(key: str, **overrides) -> Workload:
    wl = WORKLOADS[key]
    return wl.with_(**overrides) if overrides else wl
