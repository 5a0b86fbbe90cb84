"""GPU: mla_decode_step, one layer's whole decode step (append the new tokens'
rows, then attend with the queries) with the query absorb sharing a launch
with the append finish (bf16 pages) or the append GEMM (FP8 pages), against
mla_append_latent followed by mla_decode on the same
inputs: the outputs and every byte of the cache agree bit for bit (the same
device arithmetic runs in a different grouping of launches).  One case is
also checked against the float64 oracle to the decode parity tolerances.
Covered: both split-KV kernels (16 and 128 heads), one and two queries per
sequence, paged and contiguous caches, FP8 pages, every absorb weight
blocking (d_nope 64, 128, 192), an fp32 layer (no fused launch), and a
step with no new tokens (the decode alone, the cache untouched)."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, LLAMA2_7B_MLA, WORKLOADS, Shape, workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mla_compressed_latent_amd as mla  # noqa: E402
from gpu_harness import GpuCase, errors, oracle_outputs  # noqa: E402

SMALL_DSV2 = dataclasses.replace(DSV2, d_model=512)
SMALL_LLAMA = dataclasses.replace(LLAMA2_7B_MLA, d_model=512)
FP8_DSV2 = dataclasses.replace(DSV2, d_model=512, cache_format="fp8")
NOPE64 = Shape(512, 16, 64, 64, 64, 512)
NOPE192 = Shape(512, 16, 192, 64, 128, 512)


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8)


def _step_vs_separate(wl, kv_chunk=0):
    print(f"[step] case {wl.name} B={wl.batch} heads={wl.shape.H} d_nope={wl.shape.qk_nope_head_dim} "
          f"cache={wl.shape.cache_format} kv_chunk={kv_chunk}", flush=True)
    case = GpuCase(wl)   # cache holds the prefixes only
    before = case.cache.clone()
    case.append_new()
    ref = case.decode(kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    cache_ref = case.cache.clone()

    case.cache.copy_(before)
    out = torch.full_like(ref, float("nan"))
    mla.mla_decode_step(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.q_dev, case.cu_q,
                        case.seq_lens, case.page_table, case.cache, out, case.max_q_len, case.max_seq_len,
                        kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref)), "decode step output differs from append + decode"
    assert torch.equal(_bits(case.cache), _bits(cache_ref)), "decode step cache differs from append + decode"
    return case, out


def test_step_dsv2_matches_and_oracle():
    wl = workload("dsv2_b32_ctx4096", name="step_dsv2", shape=SMALL_DSV2, batch=3, fixed_prefix=None,
                  max_prefix=700, paging="random", spare_page_frac=0.2)
    case, out = _step_vs_separate(wl)
    got = out.float().cpu().numpy()
    cu = wl.cu_q()
    for b in range(wl.batch):
        ref = oracle_outputs(wl, b, None, case.w_dkv, case.w_uk, case.w_uv)
        e = errors(got[cu[b]:cu[b + 1]], ref)
        assert e[0] <= 1e-2 and e[1] <= 1e-2, f"seq {b}: errors {e}"


def test_step_llama_two_queries_paged():
    wl = workload("llama2_7b_mla_b64_ctx8192", name="step_llama_q2", shape=SMALL_LLAMA, batch=5,
                  fixed_prefix=None, max_prefix=500, fixed_q_len=None, max_q_len=2, paging="random",
                  spare_page_frac=0.1)
    _step_vs_separate(wl, kv_chunk=256)


def test_step_fp8_pages():
    wl = workload("dsv2_b32_ctx4096", name="step_fp8", shape=FP8_DSV2, batch=3, fixed_prefix=None,
                  max_prefix=300, paging="random", spare_page_frac=0.3, seed=37)
    _step_vs_separate(wl)


@pytest.mark.parametrize("shape", [NOPE64, NOPE192], ids=["nope64", "nope192"])
def test_step_absorb_blockings(shape):
    wl = workload("dsv2_b32_ctx4096", name=f"step_nope{shape.qk_nope_head_dim}", shape=shape, batch=4,
                  fixed_prefix=None, max_prefix=400, fixed_q_len=None, max_q_len=2)
    _step_vs_separate(wl, kv_chunk=128)


def test_step_fp32_layer():
    wl = WORKLOADS["tiny_f32"].with_(name="step_tiny_f32", batch=3, fixed_prefix=None, max_prefix=200,
                                     fixed_q_len=None, max_q_len=2, paging="random", spare_page_frac=0.2)
    _step_vs_separate(wl, kv_chunk=64)


def test_step_workspace_checked():
    wl = workload("dsv2_b32_ctx4096", name="step_ws", shape=SMALL_DSV2, batch=2, fixed_prefix=None,
                  max_prefix=100)
    case = GpuCase(wl)
    total_new, total_q, B = case.x_new_dev.shape[0], case.q_dev.shape[0], wl.batch
    need = mla.mla_decode_step_workspace_bytes(case.layer, B, total_new, total_q, case.max_q_len,
                                               case.max_seq_len)
    dec = mla.mla_decode_workspace_bytes(case.layer, B, total_q, case.max_q_len, case.max_seq_len)
    assert need >= dec + mla.mla_append_workspace_bytes(case.layer, total_new)
    before = case.cache.clone()
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    out = torch.empty((total_q, wl.shape.H, wl.shape.v_head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as ei:
        mla.mla_decode_step(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.q_dev, case.cu_q,
                            case.seq_lens, case.page_table, case.cache, out, case.max_q_len,
                            case.max_seq_len, workspace=ws)
    assert ei.value.status == mla.MLA_ERR_INSUFFICIENT_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(_bits(case.cache), _bits(before)), "a rejected call wrote the cache"


def test_step_without_new_tokens():
    """total_new = 0: no append work, the cache is left as it is and the
    output equals mla_decode's bit for bit."""
    wl = workload("dsv2_b32_ctx4096", name="step_no_new", shape=SMALL_DSV2, batch=3, fixed_prefix=None,
                  max_prefix=500, paging="random", spare_page_frac=0.2)
    case = GpuCase(wl)
    case.append_new()
    ref = case.decode()
    torch.cuda.synchronize()
    before = case.cache.clone()
    out = torch.full_like(ref, float("nan"))
    no_new = torch.zeros(wl.batch + 1, dtype=torch.int32, device="cuda")
    mla.mla_decode_step(case.layer, case.x_new_dev[:0], no_new, case.seq_lens, case.q_dev, case.cu_q,
                        case.seq_lens, case.page_table, case.cache, out, case.max_q_len, case.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref)), "decode step without new tokens differs from mla_decode"
    assert torch.equal(_bits(case.cache), _bits(before)), "decode step without new tokens changed the cache"
