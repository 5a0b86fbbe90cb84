"""GPU: layer output through the output projection W_o (mla_decode_project),
with the value up-projection kept apart (unfolded) or folded into W_o
(W_uv_h W_o_h, folded once at load) -- both against the oracle's projection
of its own attention output, bf16 tolerances as the decode parity tests."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, WORKLOADS, workload
from oracle import mla_oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mla_compressed_latent_amd as mla  # noqa: E402
from gpu_harness import GpuCase, errors, oracle_outputs, to_dev  # noqa: E402

UNF, FOL = mla.MLA_OUTPUT_UNFOLDED, mla.MLA_OUTPUT_FOLDED


def _run(wl, form, heads_check=True):
    print(f"[project] case {wl.name} B={wl.batch} H={wl.shape.H} form {form}", flush=True)
    case = GpuCase(wl)
    case.append_new()
    w_o = wl.w_o()
    mla.mla_fold_output(case.layer, to_dev(case.w_uv, torch.bfloat16), to_dev(w_o, torch.bfloat16), form)
    y = torch.empty((case.q.shape[0], wl.shape.d_model), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode_project(case.layer, case.q_dev, case.cu_q, case.seq_lens, case.page_table, case.cache, y,
                           case.max_q_len, case.max_seq_len)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    cu = wl.cu_q()
    worst = (0.0, 0.0)
    for b in range(wl.batch):
        ref = mla_oracle.project_output(oracle_outputs(wl, b, None, case.w_dkv, case.w_uk, case.w_uv), w_o)
        e = errors(got[cu[b]:cu[b + 1]], ref)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        assert e[0] <= 1e-2 and e[1] <= 1e-2, (form, b, e)
    print(f"[project] {wl.name} form {form}: max|d|/max|ref| {worst[0]:.3e}, rms ratio {worst[1]:.3e}", flush=True)
    return case


@pytest.mark.parametrize("form", [UNF, FOL])
def test_project_small(form):
    shape = dataclasses.replace(DSV2, d_model=256, num_attention_heads=4, qk_nope_head_dim=64, v_head_dim=64)
    wl = workload("dsv2_ragged_paged_256", name="project_small", shape=shape, batch=3, max_prefix=300,
                  prefix_source="hidden", seed=51)
    _run(wl, form)


@pytest.mark.parametrize("form", [UNF, FOL])
def test_project_dsv2_heads(form):
    """All 128 DeepSeek-V2 heads (d_model 512 to keep the oracle quick)."""
    shape = dataclasses.replace(DSV2, d_model=512)
    wl = workload("dsv2_ragged_paged_256", name="project_dsv2", shape=shape, batch=2, max_prefix=500,
                  prefix_source="hidden", seed=52)
    _run(wl, form)


def test_project_dsv2_wide_output():
    """d_model 4096, unfolded: the projection GEMM carries its accumulator
    through runs of 4 256-wide k chunks per split."""
    shape = dataclasses.replace(DSV2, d_model=4096)
    wl = workload("dsv2_ragged_paged_256", name="project_dsv2_wide", shape=shape, batch=2, max_prefix=300,
                  prefix_source="hidden", seed=54)
    _run(wl, UNF)


def test_project_errors():
    wl = workload("dsv2_ragged_paged_256", name="project_err", shape=dataclasses.replace(
        DSV2, d_model=256, num_attention_heads=4, qk_nope_head_dim=64, v_head_dim=64), batch=2,
        max_prefix=50, prefix_source="hidden", seed=53)
    case = GpuCase(wl)
    case.append_new()
    y = torch.empty((case.q.shape[0], 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as e:      # nothing folded yet
        mla.mla_decode_project(case.layer, case.q_dev, case.cu_q, case.seq_lens, case.page_table, case.cache, y,
                               case.max_q_len, case.max_seq_len)
    assert e.value.status == 1
    tiny = GpuCase(WORKLOADS["tiny_f32"])
    with pytest.raises(mla.MlaError) as e:      # fp32 layers have no projection kernels
        mla.mla_fold_output(tiny.layer, None, torch.zeros((64, 64), device="cuda"), UNF,
                            folded=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 2
