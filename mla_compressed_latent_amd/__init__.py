"""Python binding of the MLA decode library (libmla.so, HIP for gfx950).

A thin ctypes layer over the C ABI in ``include/mla.h``: each function has
the C call's name, checks that the tensors it is handed are device-resident,
contiguous and of the layer's dtype, and passes raw pointers.  All arithmetic
runs in the library's kernels; PyTorch only supplies device memory and the
current stream.  Importing this package fails loudly when libmla.so is
missing -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MlaError", "MlaConfig", "Layer", "LIB_PATH", "lib",
    "mla_folded_bytes", "mla_fold_weights", "mla_layer_free", "mla_layer_set_attention_rows",
    "mla_cache_bytes_per_token",
    "mla_append_workspace_bytes", "mla_append_latent", "mla_decode_kv_chunk",
    "mla_decode_workspace_bytes", "mla_decode", "mla_decode_phases", "mla_decode_no_alloc",
    "MLA_NO_ALLOC_SCRATCH_BYTES", "mla_status_string", "mla_last_error",
    "config_from_shape", "EXPORTED_SYMBOLS", "MLA_PHASE_ABSORB", "MLA_PHASE_ATTEND", "MLA_PHASE_OUTPUT",
    "MLA_PHASE_ALL", "mla_extend_choose_path", "mla_extend_workspace_bytes", "mla_extend",
    "MLA_EXTEND_AUTO", "MLA_EXTEND_ABSORBED", "MLA_EXTEND_EXPANDED",
    "MlaCachePlan", "mla_plan_cache", "mla_plan_max_sequences", "PagePool", "MLA_CACHE_DTYPE", "MLA_CACHE_FP8",
    "mla_output_choose_form", "mla_output_folded_bytes", "mla_fold_output", "mla_decode_project_workspace_bytes",
    "mla_decode_project", "MLA_OUTPUT_AUTO", "MLA_OUTPUT_UNFOLDED", "MLA_OUTPUT_FOLDED",
    "mla_decode_step_workspace_bytes", "mla_decode_step",
    "mla_query_choose_form", "mla_query_folded_bytes", "mla_fold_query", "mla_decode_hidden_workspace_bytes",
    "mla_decode_hidden", "MLA_QUERY_AUTO", "MLA_QUERY_UNFOLDED", "MLA_QUERY_FOLDED",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MLA_LIBRARY=debug selects the checking build (device-resident lengths and
# page ids verified before each call's kernels; see include/mla.h).
LIBRARIES = {"release": os.path.join(_PKG_DIR, "libmla.so"), "debug": os.path.join(_PKG_DIR, "libmla_debug.so")}
LIB_VARIANT = os.environ.get("MLA_LIBRARY", "release")
if LIB_VARIANT not in LIBRARIES:
    raise ImportError(f"MLA_LIBRARY={LIB_VARIANT!r}: expected one of {sorted(LIBRARIES)}")
LIB_PATH = LIBRARIES[LIB_VARIANT]

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP, MLA_ERR_INSUFFICIENT_WORKSPACE = range(5)
MLA_DTYPE_F32, MLA_DTYPE_BF16 = 0, 1
MLA_PHASE_ABSORB, MLA_PHASE_ATTEND, MLA_PHASE_OUTPUT, MLA_PHASE_ALL = 1, 2, 4, 7
MLA_EXTEND_AUTO, MLA_EXTEND_ABSORBED, MLA_EXTEND_EXPANDED = 0, 1, 2
MLA_CACHE_DTYPE, MLA_CACHE_FP8 = 0, 1
MLA_OUTPUT_AUTO, MLA_OUTPUT_UNFOLDED, MLA_OUTPUT_FOLDED = 0, 1, 2
MLA_QUERY_AUTO, MLA_QUERY_UNFOLDED, MLA_QUERY_FOLDED = 0, 1, 2
MLA_NO_ALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED_SYMBOLS = (
    "mla_folded_bytes", "mla_fold_weights", "mla_layer_free", "mla_layer_set_attention_rows",
    "mla_cache_bytes_per_token",
    "mla_append_workspace_bytes", "mla_append_latent", "mla_decode_kv_chunk",
    "mla_decode_workspace_bytes", "mla_decode", "mla_decode_phases", "mla_decode_no_alloc",
    "mla_extend_choose_path",
    "mla_extend_workspace_bytes", "mla_extend", "mla_plan_cache", "mla_plan_max_sequences",
    "mla_pool_create", "mla_pool_destroy", "mla_pool_reserve", "mla_pool_release", "mla_pool_free_pages",
    "mla_pool_length", "mla_pool_page_table", "mla_output_choose_form", "mla_output_folded_bytes",
    "mla_fold_output", "mla_decode_project_workspace_bytes", "mla_decode_project",
    "mla_decode_step_workspace_bytes", "mla_decode_step", "mla_query_choose_form", "mla_query_folded_bytes",
    "mla_fold_query", "mla_decode_hidden_workspace_bytes", "mla_decode_hidden", "mla_status_string",
    "mla_last_error",
)


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {detail}")


class MlaConfig(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32),
        ("num_attention_heads", ctypes.c_int32),
        ("qk_nope_head_dim", ctypes.c_int32),
        ("qk_rope_head_dim", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("cache_format", ctypes.c_int32),
    ]

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == MLA_DTYPE_BF16 else torch.float32

    @property
    def cache_torch_dtype(self):
        """Element type of cache tensors: the layer dtype, or bytes for FP8 pages."""
        return torch.uint8 if self.cache_format == MLA_CACHE_FP8 else self.torch_dtype


class MlaCachePlan(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("page_bytes", ctypes.c_size_t),
        ("layer_bytes", ctypes.c_size_t),
        ("total_bytes", ctypes.c_size_t),
        ("bytes_per_token", ctypes.c_size_t),
    ]


def _load(path=None):
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python mla_compressed_latent_amd/build.py` "
            "(the decode path has no CPU fallback)")
    L = ctypes.CDLL(path)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    cfgp = ctypes.POINTER(MlaConfig)
    sig = {
        "mla_folded_bytes": (S, [cfgp]),
        "mla_fold_weights": (I32, [cfgp, P, P, P, P, S, P, ctypes.POINTER(P)]),
        "mla_layer_free": (None, [P]),
        "mla_layer_set_attention_rows": (I32, [P, I32]),
        "mla_cache_bytes_per_token": (S, [cfgp]),
        "mla_append_workspace_bytes": (S, [P, I32]),
        "mla_append_latent": (I32, [P, P, P, P, P, I32, I32, I32, P, I64, P, S, P]),
        "mla_decode_kv_chunk": (I32, [P, I32, I32, I32, I32]),
        "mla_decode_workspace_bytes": (S, [P, I32, I32, I32, I32, I32]),
        "mla_decode": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, P, I64, P, P, S, P]),
        "mla_decode_phases": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, P, I64, P, P, S, P,
                                    ctypes.c_uint32]),
        "mla_decode_no_alloc": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, P, I64, P, P]),
        "mla_decode_step_workspace_bytes": (S, [P, I32, I32, I32, I32, I32, I32]),
        "mla_decode_step": (I32, [P, P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, P, I64, P, P, S,
                                  P]),
        "mla_extend_choose_path": (I32, [cfgp, I32, I32, I32, I32]),
        "mla_extend_workspace_bytes": (S, [P, I32, I32, I32, I32, I32]),
        "mla_extend": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, P, I64, P, P, S, P]),
        "mla_plan_cache": (I32, [cfgp, I32, S, ctypes.POINTER(MlaCachePlan)]),
        "mla_plan_max_sequences": (I64, [cfgp, I32, S, I64]),
        "mla_pool_create": (I32, [I64, I32, I32, I32, ctypes.POINTER(P)]),
        "mla_pool_destroy": (None, [P]),
        "mla_pool_reserve": (I32, [P, I32, I64]),
        "mla_pool_release": (I32, [P, I32]),
        "mla_pool_free_pages": (I64, [P]),
        "mla_pool_length": (I64, [P, I32]),
        "mla_pool_page_table": (I32, [P, P, I32, P]),
        "mla_output_choose_form": (I32, [cfgp, I32]),
        "mla_output_folded_bytes": (S, [cfgp, I32]),
        "mla_fold_output": (I32, [P, P, P, I32, P, S, P]),
        "mla_decode_project_workspace_bytes": (S, [P, I32, I32, I32, I32]),
        "mla_decode_project": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, P, I64, P, P, S, P]),
        "mla_query_choose_form": (I32, [cfgp, I32]),
        "mla_query_folded_bytes": (S, [cfgp, I32]),
        "mla_fold_query": (I32, [P, P, P, I32, P, S, P]),
        "mla_decode_hidden_workspace_bytes": (S, [P, I32, I32, I32, I32]),
        "mla_decode_hidden": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, P, I64, P, P, S, P]),
        "mla_status_string": (ctypes.c_char_p, [I32]),
        "mla_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def use_library(variant: str):
    """Bind every function of this module to another build of the library
    ("release" or "debug") from now on.  Handles (layers, pools) made under
    one build must be released before switching and are not used across."""
    global lib, LIB_VARIANT, LIB_PATH
    lib = _load(LIBRARIES[variant])
    LIB_VARIANT, LIB_PATH = variant, LIBRARIES[variant]


def _status_name(s: int) -> str:
    return lib.mla_status_string(s).decode()


def mla_status_string(s: int) -> str:
    return _status_name(s)


def mla_last_error() -> str:
    return lib.mla_last_error().decode()


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where, mla_last_error())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str, dtype=None) -> ctypes.c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def config_from_shape(shape, softmax_scale: float = 0.0) -> MlaConfig:
    """MlaConfig from an object with the Hugging Face field names (and an
    optional ``cache_format``: "dtype" or "fp8")."""
    return MlaConfig(
        d_model=shape.d_model,
        num_attention_heads=shape.num_attention_heads,
        qk_nope_head_dim=shape.qk_nope_head_dim,
        qk_rope_head_dim=shape.qk_rope_head_dim,
        v_head_dim=shape.v_head_dim,
        kv_lora_rank=shape.kv_lora_rank,
        page_size=shape.page_size,
        rope_base=float(shape.rope_base),
        softmax_scale=float(softmax_scale),
        dtype=MLA_DTYPE_BF16 if shape.dtype == "bf16" else MLA_DTYPE_F32,
        cache_format=MLA_CACHE_FP8 if getattr(shape, "cache_format", "dtype") == "fp8" else MLA_CACHE_DTYPE,
    )


class Layer:
    """Host handle of a folded layer; keeps the folded device buffer alive."""

    def __init__(self, handle: ctypes.c_void_p, cfg: MlaConfig, folded: torch.Tensor):
        self.handle = handle
        self.cfg = cfg
        self.folded = folded
        self._free = lib.mla_layer_free   # the build that made the handle releases it

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            self._free(h)
            self.handle = None


def mla_folded_bytes(cfg: MlaConfig) -> int:
    return int(lib.mla_folded_bytes(ctypes.byref(cfg)))


def mla_cache_bytes_per_token(cfg: MlaConfig) -> int:
    return int(lib.mla_cache_bytes_per_token(ctypes.byref(cfg)))


def mla_fold_weights(cfg: MlaConfig, w_dkv, w_uk, w_uv, folded=None, stream=None) -> Layer:
    dt = cfg.torch_dtype
    n = mla_folded_bytes(cfg)
    if n == 0:
        # let the library report why
        _check(lib.mla_fold_weights(ctypes.byref(cfg), None, None, None, None, 0, None,
                                    ctypes.byref(ctypes.c_void_p())), "mla_fold_weights")
    if folded is None:
        folded = torch.empty(n, dtype=torch.uint8, device=w_dkv.device)
    handle = ctypes.c_void_p()
    _check(lib.mla_fold_weights(ctypes.byref(cfg), _dev(w_dkv, "w_dkv", dt), _dev(w_uk, "w_uk", dt),
                                _dev(w_uv, "w_uv", dt), _dev(folded, "folded"), folded.numel() * folded.element_size(),
                                _stream(stream), ctypes.byref(handle)), "mla_fold_weights")
    return Layer(handle, cfg, folded)


def mla_layer_free(layer: Layer):
    if layer.handle:
        layer._free(layer.handle)
        layer.handle = None


def mla_layer_set_attention_rows(layer: Layer, rows: int):
    """Split-KV rows per workgroup for later decode calls: 0 by shape, 64 or 128."""
    _check(lib.mla_layer_set_attention_rows(layer.handle, int(rows)), "mla_layer_set_attention_rows")


def mla_append_workspace_bytes(layer: Layer, total_new: int) -> int:
    return int(lib.mla_append_workspace_bytes(layer.handle, int(total_new)))


def mla_append_latent(layer: Layer, x, cu_new, prefix_lens, page_table, cache, workspace=None,
                      stream=None):
    """Append the rows of x ([total_new][d_model]) at positions prefix_lens[b] + j."""
    dt = layer.cfg.torch_dtype
    total_new = int(x.shape[0])
    batch = int(prefix_lens.shape[0])
    if workspace is None:
        workspace = torch.empty(max(1, mla_append_workspace_bytes(layer, total_new)), dtype=torch.uint8,
                                device=x.device)
    _check(lib.mla_append_latent(
        layer.handle, _dev(x, "x", dt), _dev(cu_new, "cu_new", torch.int32),
        _dev(prefix_lens, "prefix_lens", torch.int32), _dev(page_table, "page_table", torch.int32),
        int(page_table.shape[1]), batch, total_new, _dev(cache, "cache", layer.cfg.cache_torch_dtype), int(cache.shape[0]),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)),
        "mla_append_latent")


def mla_decode_kv_chunk(layer: Layer, batch: int, max_q_len: int, max_seq_len: int, kv_chunk: int = 0) -> int:
    return int(lib.mla_decode_kv_chunk(layer.handle, batch, max_q_len, max_seq_len, kv_chunk))


def mla_decode_workspace_bytes(layer: Layer, batch: int, total_q: int, max_q_len: int, max_seq_len: int,
                               kv_chunk: int = 0) -> int:
    return int(lib.mla_decode_workspace_bytes(layer.handle, batch, total_q, max_q_len, max_seq_len, kv_chunk))


def mla_decode(layer: Layer, q, cu_q, seq_lens, page_table, cache, out, max_q_len: int, max_seq_len: int,
               kv_chunk: int = 0, workspace=None, stream=None):
    """out[t][h] = attention of query t, head h over its sequence's cached rows."""
    return mla_decode_phases(layer, q, cu_q, seq_lens, page_table, cache, out, max_q_len, max_seq_len,
                             kv_chunk, workspace, stream, MLA_PHASE_ALL)


def mla_decode_phases(layer: Layer, q, cu_q, seq_lens, page_table, cache, out, max_q_len: int,
                      max_seq_len: int, kv_chunk: int = 0, workspace=None, stream=None,
                      phases: int = MLA_PHASE_ALL):
    """Run the selected phases of mla_decode (see include/mla.h)."""
    dt = layer.cfg.torch_dtype
    total_q = int(q.shape[0])
    batch = int(seq_lens.shape[0])
    if workspace is None:
        if phases != MLA_PHASE_ALL:
            raise ValueError("a partial phase mask needs the caller's workspace")
        n = mla_decode_workspace_bytes(layer, batch, total_q, max_q_len, max_seq_len, kv_chunk)
        workspace = torch.empty(max(1, n), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_phases(
        layer.handle, _dev(q, "q", dt), _dev(cu_q, "cu_q", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(page_table, "page_table", torch.int32), int(page_table.shape[1]), batch, total_q, int(max_q_len),
        int(max_seq_len), int(kv_chunk), _dev(cache, "cache", layer.cfg.cache_torch_dtype), int(cache.shape[0]), _dev(out, "out", dt),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream),
        int(phases)), "mla_decode")


def mla_decode_no_alloc(layer: Layer, q, cu_q, seq_lens, page_table, cache, out, max_q_len: int,
                        max_seq_len: int, kv_chunk: int = 0, stream=None):
    """mla_decode in the library's static device scratch: allocates nothing (see include/mla.h)."""
    dt = layer.cfg.torch_dtype
    _check(lib.mla_decode_no_alloc(
        layer.handle, _dev(q, "q", dt), _dev(cu_q, "cu_q", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(page_table, "page_table", torch.int32), int(page_table.shape[1]), int(seq_lens.shape[0]),
        int(q.shape[0]), int(max_q_len), int(max_seq_len), int(kv_chunk),
        _dev(cache, "cache", layer.cfg.cache_torch_dtype), int(cache.shape[0]), _dev(out, "out", dt),
        _stream(stream)), "mla_decode_no_alloc")


def mla_decode_step_workspace_bytes(layer: Layer, batch: int, total_new: int, total_q: int, max_q_len: int,
                                    max_seq_len: int, kv_chunk: int = 0) -> int:
    return int(lib.mla_decode_step_workspace_bytes(layer.handle, batch, total_new, total_q, max_q_len,
                                                   max_seq_len, kv_chunk))


def mla_decode_step(layer: Layer, x, cu_new, prefix_lens, q, cu_q, seq_lens, page_table, cache, out,
                    max_q_len: int, max_seq_len: int, kv_chunk: int = 0, workspace=None, stream=None):
    """mla_append_latent of x's rows, then mla_decode of q, in fewer launches (see include/mla.h)."""
    dt = layer.cfg.torch_dtype
    total_new, total_q = int(x.shape[0]), int(q.shape[0])
    batch = int(seq_lens.shape[0])
    if workspace is None:
        n = mla_decode_step_workspace_bytes(layer, batch, total_new, total_q, max_q_len, max_seq_len, kv_chunk)
        workspace = torch.empty(max(1, n), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_step(
        layer.handle, _dev(x, "x", dt), _dev(cu_new, "cu_new", torch.int32),
        _dev(prefix_lens, "prefix_lens", torch.int32), total_new, _dev(q, "q", dt),
        _dev(cu_q, "cu_q", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(page_table, "page_table", torch.int32), int(page_table.shape[1]), batch, total_q, int(max_q_len),
        int(max_seq_len), int(kv_chunk), _dev(cache, "cache", layer.cfg.cache_torch_dtype), int(cache.shape[0]),
        _dev(out, "out", dt), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), "mla_decode_step")


def mla_extend_choose_path(cfg: MlaConfig, batch: int, total_q: int, max_q_len: int, max_seq_len: int) -> int:
    """The form MLA_EXTEND_AUTO takes for these bounds (host only; -1 if invalid)."""
    return int(lib.mla_extend_choose_path(ctypes.byref(cfg), int(batch), int(total_q), int(max_q_len),
                                          int(max_seq_len)))


def mla_extend_workspace_bytes(layer: Layer, batch: int, total_q: int, max_q_len: int, max_seq_len: int,
                               path: int = MLA_EXTEND_AUTO) -> int:
    return int(lib.mla_extend_workspace_bytes(layer.handle, int(batch), int(total_q), int(max_q_len),
                                              int(max_seq_len), int(path)))


def mla_extend(layer: Layer, q, cu_q, seq_lens, page_table, cache, out, max_q_len: int, max_seq_len: int,
               path: int = MLA_EXTEND_AUTO, workspace=None, stream=None):
    """Prefill / chunked extend: the result of mla_decode, by the absorbed or
    the expanded form (see include/mla.h)."""
    dt = layer.cfg.torch_dtype
    total_q = int(q.shape[0])
    batch = int(seq_lens.shape[0])
    if workspace is None:
        n = mla_extend_workspace_bytes(layer, batch, total_q, max_q_len, max_seq_len, path)
        workspace = torch.empty(max(1, n), dtype=torch.uint8, device=q.device)
    _check(lib.mla_extend(
        layer.handle, _dev(q, "q", dt), _dev(cu_q, "cu_q", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(page_table, "page_table", torch.int32), int(page_table.shape[1]), batch, total_q, int(max_q_len),
        int(max_seq_len), int(path), _dev(cache, "cache", layer.cfg.cache_torch_dtype), int(cache.shape[0]), _dev(out, "out", dt),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)),
        "mla_extend")


def mla_plan_cache(cfg: MlaConfig, num_layers: int, budget_bytes: int) -> MlaCachePlan:
    plan = MlaCachePlan()
    _check(lib.mla_plan_cache(ctypes.byref(cfg), int(num_layers), int(budget_bytes), ctypes.byref(plan)),
           "mla_plan_cache")
    return plan


def mla_plan_max_sequences(cfg: MlaConfig, num_layers: int, budget_bytes: int, context: int) -> int:
    return int(lib.mla_plan_max_sequences(ctypes.byref(cfg), int(num_layers), int(budget_bytes), int(context)))


class PagePool:
    """Host page allocator shared by every layer's cache (mla_pool_*)."""

    def __init__(self, num_pages: int, page_size: int, max_seqs: int, max_pages_per_seq: int):
        h = ctypes.c_void_p()
        _check(lib.mla_pool_create(int(num_pages), int(page_size), int(max_seqs), int(max_pages_per_seq),
                                   ctypes.byref(h)), "mla_pool_create")
        self.handle = h
        self.max_pages_per_seq = int(max_pages_per_seq)
        self._destroy = lib.mla_pool_destroy   # still bound at interpreter exit

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            self._destroy(h)
            self.handle = None

    def reserve(self, seq: int, length: int):
        _check(lib.mla_pool_reserve(self.handle, int(seq), int(length)), "mla_pool_reserve")

    def release(self, seq: int):
        _check(lib.mla_pool_release(self.handle, int(seq)), "mla_pool_release")

    def free_pages(self) -> int:
        return int(lib.mla_pool_free_pages(self.handle))

    def length(self, seq: int) -> int:
        return int(lib.mla_pool_length(self.handle, int(seq)))

    def page_table(self, seqs):
        """int32 host array [len(seqs)][max_pages_per_seq]."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        out = np.empty((ids.shape[0], self.max_pages_per_seq), dtype=np.int32)
        _check(lib.mla_pool_page_table(self.handle, ids.ctypes.data_as(ctypes.c_void_p), int(ids.shape[0]),
                                       out.ctypes.data_as(ctypes.c_void_p)), "mla_pool_page_table")
        return out


def mla_output_choose_form(cfg: MlaConfig, total_q: int) -> int:
    return int(lib.mla_output_choose_form(ctypes.byref(cfg), int(total_q)))


def mla_output_folded_bytes(cfg: MlaConfig, form: int) -> int:
    return int(lib.mla_output_folded_bytes(ctypes.byref(cfg), int(form)))


def mla_fold_output(layer: Layer, w_uv, w_o, form: int = MLA_OUTPUT_AUTO, folded=None, stream=None):
    """Attach the output projection (W_o, or W_uv W_o folded) to the layer."""
    dt = layer.cfg.torch_dtype
    if form == MLA_OUTPUT_AUTO:
        form = mla_output_choose_form(layer.cfg, 1)
    n = mla_output_folded_bytes(layer.cfg, form)
    if folded is None:
        folded = torch.empty(max(1, n), dtype=torch.uint8, device=w_o.device)
    _check(lib.mla_fold_output(layer.handle, None if w_uv is None else _dev(w_uv, "w_uv", dt), _dev(w_o, "w_o", dt),
                               int(form), _dev(folded, "folded"), folded.numel(), _stream(stream)),
           "mla_fold_output")
    layer.out_folded = folded     # the layer reads it from now on
    layer.out_form = form
    return form


def mla_query_choose_form(cfg: MlaConfig, total_q: int) -> int:
    return int(lib.mla_query_choose_form(ctypes.byref(cfg), int(total_q)))


def mla_query_folded_bytes(cfg: MlaConfig, form: int) -> int:
    return int(lib.mla_query_folded_bytes(ctypes.byref(cfg), int(form)))


def mla_fold_query(layer: Layer, w_q, w_uk, form: int = MLA_QUERY_AUTO, folded=None, stream=None):
    """Attach the query projection (W_q, or W_q_h W_uk_h^T folded) to the layer."""
    dt = layer.cfg.torch_dtype
    if form == MLA_QUERY_AUTO:
        form = mla_query_choose_form(layer.cfg, 1)
    n = mla_query_folded_bytes(layer.cfg, form)
    if folded is None:
        folded = torch.empty(max(1, n), dtype=torch.uint8, device=w_q.device)
    _check(lib.mla_fold_query(layer.handle, _dev(w_q, "w_q", dt), None if w_uk is None else _dev(w_uk, "w_uk", dt),
                              int(form), _dev(folded, "folded"), folded.numel(), _stream(stream)),
           "mla_fold_query")
    layer.q_folded = folded       # the layer reads it from now on
    layer.q_form = form
    return form


def mla_decode_hidden_workspace_bytes(layer: Layer, batch: int, total_q: int, max_q_len: int,
                                      max_seq_len: int) -> int:
    return int(lib.mla_decode_hidden_workspace_bytes(layer.handle, batch, total_q, max_q_len, max_seq_len))


def mla_decode_hidden(layer: Layer, x, cu_q, seq_lens, page_table, cache, out, max_q_len: int, max_seq_len: int,
                      workspace=None, stream=None):
    """Decode with the queries projected from the layer input x [total_q][d_model]."""
    dt = layer.cfg.torch_dtype
    total_q = int(x.shape[0])
    batch = int(seq_lens.shape[0])
    if workspace is None:
        n = mla_decode_hidden_workspace_bytes(layer, batch, total_q, max_q_len, max_seq_len)
        workspace = torch.empty(max(1, n), dtype=torch.uint8, device=x.device)
    _check(lib.mla_decode_hidden(
        layer.handle, _dev(x, "x", dt), _dev(cu_q, "cu_q", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(page_table, "page_table", torch.int32), int(page_table.shape[1]), batch, total_q, int(max_q_len),
        int(max_seq_len), _dev(cache, "cache", layer.cfg.cache_torch_dtype), int(cache.shape[0]),
        _dev(out, "out", dt), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)),
        "mla_decode_hidden")


def mla_decode_project_workspace_bytes(layer: Layer, batch: int, total_q: int, max_q_len: int,
                                       max_seq_len: int) -> int:
    return int(lib.mla_decode_project_workspace_bytes(layer.handle, batch, total_q, max_q_len, max_seq_len))


def mla_decode_project(layer: Layer, q, cu_q, seq_lens, page_table, cache, y, max_q_len: int, max_seq_len: int,
                       workspace=None, stream=None):
    """Decode plus output projection: y [total_q][d_model]."""
    dt = layer.cfg.torch_dtype
    total_q = int(q.shape[0])
    batch = int(seq_lens.shape[0])
    if workspace is None:
        n = mla_decode_project_workspace_bytes(layer, batch, total_q, max_q_len, max_seq_len)
        workspace = torch.empty(max(1, n), dtype=torch.uint8, device=q.device)
    _check(lib.mla_decode_project(
        layer.handle, _dev(q, "q", dt), _dev(cu_q, "cu_q", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        _dev(page_table, "page_table", torch.int32), int(page_table.shape[1]), batch, total_q, int(max_q_len),
        int(max_seq_len), _dev(cache, "cache", layer.cfg.cache_torch_dtype), int(cache.shape[0]), _dev(y, "y", dt),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)),
        "mla_decode_project")
