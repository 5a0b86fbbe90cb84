"""The C ABI library: it loads, exports every function include/mla.h
declares, and rejects bad arguments on the host before touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def mla():
    import mla_compressed_latent_amd as m
    return m


@pytest.mark.parametrize("variant", ["release", "debug"])
def test_header_and_exports_agree(mla, variant):
    """Both builds (release and the checking build) export exactly the header's calls."""
    declared = _declared()
    assert set(declared) == set(mla.EXPORTED_SYMBOLS)
    path = mla.LIBRARIES[variant]
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (mla_[a-z_]+)$", out, flags=re.M))
    assert set(declared) <= exported, set(declared) - exported
    assert exported <= set(declared), f"undeclared exports {exported - set(declared)}"
    lib = ctypes.CDLL(path)
    for name in declared:
        assert hasattr(lib, name)


def _cfg(mla, **kw):
    base = dict(d_model=5120, num_attention_heads=128, qk_nope_head_dim=128, qk_rope_head_dim=64,
                v_head_dim=128, kv_lora_rank=512, page_size=64, rope_base=10000.0, softmax_scale=0.0,
                dtype=1)
    base.update(kw)
    return mla.MlaConfig(**base)


def test_cache_bytes_per_token(mla):
    # one latent plus one rope key per token, independent of the head count
    assert mla.mla_cache_bytes_per_token(_cfg(mla)) == 576 * 2
    assert mla.mla_cache_bytes_per_token(_cfg(mla, num_attention_heads=32, d_model=4096)) == 1152
    tiny = _cfg(mla, d_model=64, num_attention_heads=4, qk_nope_head_dim=16, qk_rope_head_dim=8,
                v_head_dim=16, kv_lora_rank=32, dtype=0)
    assert mla.mla_cache_bytes_per_token(tiny) == 40 * 4


def test_folded_bytes_covers_packed_weights(mla):
    # W_dkv, W_uk, W_uv and (bf16) the transposed W_uk of the expanded path
    n = mla.mla_folded_bytes(_cfg(mla))
    w = (5120 * 576 + 512 * 128 * 128 * 3) * 2
    assert w <= n < w + 4 * 256
    tiny = _cfg(mla, d_model=64, num_attention_heads=4, qk_nope_head_dim=16, qk_rope_head_dim=8,
                v_head_dim=16, kv_lora_rank=32, dtype=0)
    w = (64 * 40 + 32 * 4 * 16 * 2) * 4
    assert w <= mla.mla_folded_bytes(tiny) < w + 3 * 256


@pytest.mark.parametrize("kw,status", [
    (dict(qk_rope_head_dim=63, dtype=0), 1),
    (dict(page_size=48), 1),
    (dict(num_attention_heads=0), 1),
    (dict(dtype=7), 1),
    (dict(kv_lora_rank=256), 2),          # bf16 path is built for d_c = 512
    (dict(qk_rope_head_dim=32), 2),
    (dict(d_model=5000), 2),
])
def test_config_rejections(mla, kw, status):
    cfg = _cfg(mla, **kw)
    assert mla.mla_folded_bytes(cfg) == 0
    h = ctypes.c_void_p()
    st = mla.lib.mla_fold_weights(ctypes.byref(cfg), ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1),
                                  ctypes.c_void_p(256), 1 << 40, None, ctypes.byref(h))
    assert st == status, mla.mla_last_error()
    assert mla.mla_last_error()


def test_null_and_size_errors(mla):
    cfg = _cfg(mla)
    h = ctypes.c_void_p()
    assert mla.lib.mla_fold_weights(ctypes.byref(cfg), None, None, None, None, 0, None, ctypes.byref(h)) == 1
    assert "null" in mla.mla_last_error()
    # misaligned folded buffer
    assert mla.lib.mla_fold_weights(ctypes.byref(cfg), ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1),
                                    ctypes.c_void_p(8), 1 << 40, None, ctypes.byref(h)) == 1
    # folded buffer too small
    assert mla.lib.mla_fold_weights(ctypes.byref(cfg), ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1),
                                    ctypes.c_void_p(256), 1024, None, ctypes.byref(h)) == 4
    # calls without a layer
    assert mla.lib.mla_decode(None, *([None] * 4), 1, 1, 1, 1, 1, 0, None, 1, None, None, 0, None) == 1
    assert mla.lib.mla_append_latent(None, *([None] * 4), 1, 1, 1, None, 1, None, 0, None) == 1
    assert mla.lib.mla_decode_workspace_bytes(None, 1, 1, 1, 1, 0) == 0
    assert mla.lib.mla_decode_kv_chunk(None, 1, 1, 1, 0) == -1


def test_status_strings(mla):
    assert [mla.mla_status_string(i) for i in range(5)] == [
        "MLA_OK", "MLA_ERR_INVALID_ARG", "MLA_ERR_UNSUPPORTED", "MLA_ERR_HIP", "MLA_ERR_INSUFFICIENT_WORKSPACE"]


def test_extend_path_choice(mla):
    """AUTO picks the absorbed form for decode-sized query counts and the
    expanded form for long chunks; it never picks a form the layer lacks."""
    ABS, EXP = mla.MLA_EXTEND_ABSORBED, mla.MLA_EXTEND_EXPANDED
    dsv2 = _cfg(mla)
    for q in (1, 2, 8):
        assert mla.mla_extend_choose_path(dsv2, 32, 32 * q, q, 4096) == ABS
    assert mla.mla_extend_choose_path(dsv2, 4, 4 * 1024, 1024, 4096) == EXP
    assert mla.mla_extend_choose_path(dsv2, 2, 2 * 4096, 4096, 4096) == EXP
    # monotone in the chunk length at a fixed context: one crossover
    picks = [mla.mla_extend_choose_path(dsv2, 1, q, q, 8192) for q in range(1, 8193, 97)]
    assert picks[0] == ABS and picks[-1] == EXP
    assert all(a <= b for a, b in zip(picks, picks[1:]))
    # no expanded kernels for fp32 layers or other head widths
    tiny = _cfg(mla, d_model=64, num_attention_heads=4, qk_nope_head_dim=16, qk_rope_head_dim=8,
                v_head_dim=16, kv_lora_rank=32, dtype=0)
    assert mla.mla_extend_choose_path(tiny, 1, 4096, 4096, 4096) == ABS
    assert mla.mla_extend_choose_path(_cfg(mla, qk_nope_head_dim=96), 1, 4096, 4096, 4096) == ABS
    # invalid bounds
    assert mla.mla_extend_choose_path(dsv2, 0, 1, 1, 1) == -1
    assert mla.mla_extend_choose_path(dsv2, 2, 1, 1, 1) == -1          # total_q < batch
    assert mla.mla_extend_choose_path(dsv2, 1, 5, 4, 8) == -1          # total_q > batch * max_q_len
    assert mla.mla_extend_choose_path(dsv2, 1, 8, 8, 4) == -1          # max_seq_len < max_q_len
    assert mla.mla_extend_choose_path(_cfg(mla, page_size=48), 1, 1, 1, 1) == -1


def test_extend_rejects_null_layer(mla):
    assert mla.lib.mla_extend_workspace_bytes(None, 1, 1, 1, 1, 0) == 0
    st = mla.lib.mla_extend(None, None, None, None, None, 1, 1, 1, 1, 1, 0, None, 1, None, None, 0, None)
    assert st == 1 and "null" in mla.mla_last_error()


def test_fp8_cache_format(mla):
    """MLA_CACHE_FP8: 512 code bytes + 64 bf16 rope + a 4-byte scale per token;
    bf16 layers only; unknown formats rejected."""
    assert mla.mla_cache_bytes_per_token(_cfg(mla, cache_format=1)) == 512 + 128 + 4
    assert mla.mla_cache_bytes_per_token(_cfg(mla, cache_format=0)) == 1152
    tiny = _cfg(mla, d_model=64, num_attention_heads=4, qk_nope_head_dim=16, qk_rope_head_dim=8,
                v_head_dim=16, kv_lora_rank=32, dtype=0, cache_format=1)
    assert mla.mla_cache_bytes_per_token(tiny) == 0
    assert mla.mla_folded_bytes(_cfg(mla, cache_format=2)) == 0
    h = ctypes.c_void_p()
    st = mla.lib.mla_fold_weights(ctypes.byref(tiny), ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1),
                                  ctypes.c_void_p(256), 1 << 40, None, ctypes.byref(h))
    assert st == 2 and "bf16" in mla.mla_last_error()
    # the expanded extend form reads bf16 rows: AUTO keeps FP8 layers absorbed
    assert mla.mla_extend_choose_path(_cfg(mla, cache_format=1), 2, 8192, 4096, 4096) == mla.MLA_EXTEND_ABSORBED
    # capacity: the same budget holds 1152 / 644 times more tokens
    GIB = 1 << 30
    n8 = mla.mla_plan_max_sequences(_cfg(mla, cache_format=1), 60, 80 * GIB, 32768)
    assert n8 == (80 * GIB) // (60 * 32768 * 644)
    assert mla.mla_plan_max_sequences(_cfg(mla), 60, 80 * GIB, 32768) == 37


def test_output_form_choice(mla):
    """Folding W_uv into W_o streams H d_c d_model weights instead of
    H d_v (d_c + d_model): a loss unless d_model < d_c d_v / (d_c - d_v)."""
    UNF, FOL = mla.MLA_OUTPUT_UNFOLDED, mla.MLA_OUTPUT_FOLDED
    dsv2 = _cfg(mla)
    for tq in (1, 32, 4096):
        assert mla.mla_output_choose_form(dsv2, tq) == UNF
    # d_v = d_c: the fold removes a product and streams fewer bytes
    wide_v = _cfg(mla, d_model=64, num_attention_heads=4, qk_nope_head_dim=16, qk_rope_head_dim=8,
                  v_head_dim=32, kv_lora_rank=32, dtype=0)
    assert mla.mla_output_choose_form(wide_v, 1) == FOL
    assert mla.mla_output_choose_form(dsv2, 0) == -1
    assert mla.mla_output_folded_bytes(dsv2, UNF) == 128 * 128 * 5120 * 2
    assert mla.mla_output_folded_bytes(dsv2, FOL) == 128 * 512 * 5120 * 2
    assert mla.mla_output_folded_bytes(wide_v, UNF) == 0          # fp32: no projection kernels


def test_query_form_choice(mla):
    """Folding W_uk into the query projection streams H (d_c + d_rope) d_model
    weights instead of H ((d_nope + d_rope) d_model + d_nope d_c): a loss
    unless d_model < d_c d_nope / (d_c - d_nope)."""
    UNF, FOL = mla.MLA_QUERY_UNFOLDED, mla.MLA_QUERY_FOLDED
    dsv2 = _cfg(mla)
    for tq in (1, 32, 4096):
        assert mla.mla_query_choose_form(dsv2, tq) == UNF
    # d_nope 192, d_model 256: 256 < 512 * 192 / 320 = 307.2, the fold wins
    narrow = _cfg(mla, d_model=256, num_attention_heads=16, qk_nope_head_dim=192)
    assert mla.mla_query_choose_form(narrow, 1) == FOL
    # d_nope 128, d_model 256: 256 > 512 * 128 / 384 = 170.7
    assert mla.mla_query_choose_form(_cfg(mla, d_model=256, num_attention_heads=16), 1) == UNF
    assert mla.mla_query_choose_form(dsv2, 0) == -1
    assert mla.mla_query_folded_bytes(dsv2, UNF) == 128 * 192 * 5120 * 2
    assert mla.mla_query_folded_bytes(dsv2, FOL) == 128 * 576 * 5120 * 2
    fp32 = _cfg(mla, d_model=64, num_attention_heads=4, qk_nope_head_dim=16, qk_rope_head_dim=8,
                v_head_dim=16, kv_lora_rank=32, dtype=0)
    assert mla.mla_query_folded_bytes(fp32, FOL) == 0          # fp32: no projection kernels
