"""GPU: page sizes other than 64 (128 and 256 tokens) under random page
tables, for every attention path: decode with the split-KV kernels (64- and
128-row at 128 heads, 32-row at 32 heads), bf16 and FP8 caches, and both extend forms -- against the oracle,
bf16 tolerances as in the decode parity tests."""
import dataclasses

import pytest
import torch

from mla_synth import DSV2, LLAMA2_7B_MLA, workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mla_compressed_latent_amd as mla  # noqa: E402
from gpu_harness import GpuCase, errors, oracle_outputs  # noqa: E402


def _check(case, out, tag):
    wl = case.wl
    got = out.float().cpu().numpy()
    cu = wl.cu_q()
    for b in range(wl.batch):
        ref = oracle_outputs(wl, b, None, case.w_dkv, case.w_uk, case.w_uv)
        e = errors(got[cu[b]:cu[b + 1]], ref)
        assert e[0] <= 1e-2 and e[1] <= 1e-2, f"{tag} seq {b}: {e}"
    print(f"[pages] {tag} within tolerance", flush=True)


@pytest.mark.parametrize("page_size", [128, 256])
@pytest.mark.parametrize("base,fmt", [(DSV2, "dtype"), (LLAMA2_7B_MLA, "dtype"), (DSV2, "fp8"),
                                      (LLAMA2_7B_MLA, "fp8")],
                         ids=["128heads-bf16", "32heads-bf16", "128heads-fp8", "32heads-fp8"])
def test_decode_page_sizes(page_size, base, fmt):
    shape = dataclasses.replace(base, d_model=512, page_size=page_size, cache_format=fmt)
    wl = workload("dsv2_ragged_paged_256", name=f"pages{page_size}", shape=shape, batch=4, max_prefix=900,
                  prefix_source="hidden", spare_page_frac=0.5, seed=41)
    print(f"[pages] case {page_size} heads={shape.H} {fmt}", flush=True)
    case = GpuCase(wl)
    case.append_new()
    out = case.decode(kv_chunk=128)
    torch.cuda.synchronize()
    _check(case, out, f"decode page {page_size} heads {shape.H} {fmt}")
    if shape.H == 128 and fmt == "dtype":   # the 128-row kernel on the same pages
        mla.mla_layer_set_attention_rows(case.layer, 128)
        out = case.decode(kv_chunk=128)
        torch.cuda.synchronize()
        _check(case, out, f"decode page {page_size} heads {shape.H} {fmt} rows=128")


@pytest.mark.parametrize("page_size", [128, 256])
@pytest.mark.parametrize("path", [mla.MLA_EXTEND_EXPANDED, mla.MLA_EXTEND_ABSORBED])
def test_extend_page_sizes(page_size, path):
    shape = dataclasses.replace(DSV2, d_model=256, num_attention_heads=4, page_size=page_size)
    wl = workload("dsv2_ragged_paged_256", name=f"ext_pages{page_size}", shape=shape, batch=3, max_prefix=400,
                  max_q_len=300, prefix_source="hidden", spare_page_frac=0.5, seed=42)
    print(f"[pages] case extend {page_size} path {path}", flush=True)
    case = GpuCase(wl)
    case.append_new()
    out = case.extend(path)
    torch.cuda.synchronize()
    _check(case, out, f"extend page {page_size} path {path}")
