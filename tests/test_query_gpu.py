"""GPU: decode with the queries projected from the layer input
(mla_decode_hidden), the key up-projection kept apart (q = x . W_q, then the
decode's absorb) or folded into the query projection (W_q_h W_uk_h^T, formed
once at load) -- both against the oracle's attention over its own float64
projection of the same x, to the bf16 decode parity tolerances."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, WORKLOADS, Shape, workload
from oracle import mla_oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mla_compressed_latent_amd as mla  # noqa: E402
from gpu_harness import GpuCase, errors, oracle_cache, to_dev  # noqa: E402

UNF, FOL = mla.MLA_QUERY_UNFOLDED, mla.MLA_QUERY_FOLDED
SMALL = dataclasses.replace(DSV2, d_model=256, num_attention_heads=4, qk_nope_head_dim=64, v_head_dim=64)
NOPE192 = Shape(256, 16, 192, 64, 128, 512)


def _run(wl, form):
    print(f"[query] case {wl.name} B={wl.batch} H={wl.shape.H} d_nope={wl.shape.d_nope} form {form}", flush=True)
    s = wl.shape
    case = GpuCase(wl)
    case.append_new()
    w_q = wl.w_q()
    got_form = mla.mla_fold_query(case.layer, to_dev(w_q, torch.bfloat16), to_dev(case.w_uk, torch.bfloat16), form)
    out = torch.full((case.q.shape[0], s.H, s.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_decode_hidden(case.layer, case.x_new_dev, case.cu_q, case.seq_lens, case.page_table, case.cache, out,
                          case.max_q_len, case.max_seq_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    cu = wl.cu_q()
    scale = mla_oracle.default_scale(s.d_nope, s.d_rope)
    worst = (0.0, 0.0)
    for b in range(wl.batch):
        q_b = mla_oracle.project_query(wl.new_hidden(b), w_q, s.H)
        ref = mla_oracle.attend_sequence(q_b, oracle_cache(wl, b, case.w_dkv), case.w_uk, case.w_uv, s.H, s.d_nope,
                                         s.d_v, s.rope_base, scale)
        e = errors(got[cu[b]:cu[b + 1]], ref)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        assert e[0] <= 1e-2 and e[1] <= 1e-2, (form, b, e)
    print(f"[query] {wl.name} form {got_form}: max|d|/max|ref| {worst[0]:.3e}, rms ratio {worst[1]:.3e}", flush=True)
    return got_form, got


@pytest.mark.parametrize("form", [UNF, FOL])
def test_query_small(form):
    wl = workload("dsv2_ragged_paged_256", name="query_small", shape=SMALL, batch=3, max_prefix=300,
                  fixed_q_len=None, max_q_len=3, prefix_source="hidden", seed=61)
    _run(wl, form)


@pytest.mark.parametrize("form", [UNF, FOL])
def test_query_dsv2_heads(form):
    """All 128 DeepSeek-V2 heads, paged (d_model 512 to keep the oracle quick)."""
    wl = workload("dsv2_ragged_paged_256", name="query_dsv2", shape=dataclasses.replace(DSV2, d_model=512),
                  batch=2, max_prefix=500, prefix_source="hidden", paging="random", spare_page_frac=0.2, seed=62)
    _run(wl, form)


@pytest.mark.parametrize("form", [UNF, FOL])
def test_query_dsv2_wide_input(form):
    """d_model 2048: the projection GEMM carries its accumulator through runs
    of 2 (unfolded) and 8 (folded) 256-wide k chunks per split."""
    wl = workload("dsv2_ragged_paged_256", name="query_dsv2_wide", shape=dataclasses.replace(DSV2, d_model=2048),
                  batch=2, max_prefix=300, prefix_source="hidden", seed=65)
    _run(wl, form)


@pytest.mark.parametrize("form", [UNF, FOL])
def test_query_two_heads_d_nope_96(form):
    """Two heads of d_nope 96: the unfolded projection has 320 outputs (not a
    multiple of 128), so it runs the one-wave GEMM blocks instead of the
    four-wave LDS-shared ones."""
    wl = workload("dsv2_ragged_paged_256", name="query_h2", shape=Shape(256, 2, 96, 64, 64, 512), batch=3,
                  max_prefix=300, prefix_source="hidden", seed=68)
    _run(wl, form)


def test_query_forms_agree_and_auto_folds_narrow_model():
    """d_nope 192 at d_model 256: the chooser folds; both forms agree with the
    oracle and with each other."""
    wl = workload("dsv2_ragged_paged_256", name="query_nope192", shape=NOPE192, batch=3, max_prefix=400,
                  prefix_source="hidden", seed=63)
    form_a, a = _run(wl, mla.MLA_QUERY_AUTO)
    assert form_a == FOL
    _, b = _run(wl, UNF)
    d = np.abs(a - b).max() / np.abs(b).max()
    assert d <= 1e-2, d


@pytest.mark.parametrize("form", [UNF, FOL])
def test_query_fp8_cache(form):
    """Queries from the layer input over FP8 pages (the oracle dequantizes
    with its own row quantizer)."""
    wl = workload("dsv2_ragged_paged_256", name="query_fp8",
                  shape=dataclasses.replace(DSV2, d_model=512, cache_format="fp8"), batch=3, max_prefix=400,
                  prefix_source="hidden", paging="random", spare_page_frac=0.2, seed=66)
    _run(wl, form)


@pytest.mark.parametrize("form", [UNF, FOL])
def test_query_graph_replay_matches_eager(form):
    """mla_decode_hidden captured as a graph: three replays, with eager calls
    between them, each bit-identical to the eager call."""
    wl = workload("dsv2_ragged_paged_256", name="query_graph", shape=dataclasses.replace(DSV2, d_model=512),
                  batch=3, max_prefix=300, prefix_source="hidden", seed=67)
    print(f"[query] graph case form {form}", flush=True)
    s = wl.shape
    case = GpuCase(wl)
    case.append_new()
    mla.mla_fold_query(case.layer, to_dev(wl.w_q(), torch.bfloat16), to_dev(case.w_uk, torch.bfloat16), form)
    Tq = case.q.shape[0]
    ws = torch.empty(mla.mla_decode_hidden_workspace_bytes(case.layer, wl.batch, Tq, case.max_q_len,
                                                           case.max_seq_len), dtype=torch.uint8, device="cuda")

    def call(out):
        mla.mla_decode_hidden(case.layer, case.x_new_dev, case.cu_q, case.seq_lens, case.page_table, case.cache,
                              out, case.max_q_len, case.max_seq_len, workspace=ws)

    eager = torch.empty((Tq, s.H, s.d_v), dtype=torch.bfloat16, device="cuda")
    call(eager)
    torch.cuda.synchronize()
    out_g = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            call(out_g)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    other = torch.empty_like(eager)
    for rep in range(3):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"graph replay {rep} differs from the eager result"
        call(other)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


def test_query_errors():
    wl = workload("dsv2_ragged_paged_256", name="query_err", shape=SMALL, batch=2, max_prefix=50,
                  prefix_source="hidden", seed=64)
    case = GpuCase(wl)
    case.append_new()
    s = wl.shape
    out = torch.empty((case.q.shape[0], s.H, s.d_v), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as e:      # nothing folded yet
        mla.mla_decode_hidden(case.layer, case.x_new_dev, case.cu_q, case.seq_lens, case.page_table, case.cache,
                              out, case.max_q_len, case.max_seq_len)
    assert e.value.status == mla.MLA_ERR_INVALID_ARG
    mla.mla_fold_query(case.layer, to_dev(wl.w_q(), torch.bfloat16), None, UNF)
    need = mla.mla_decode_hidden_workspace_bytes(case.layer, wl.batch, case.q.shape[0], case.max_q_len,
                                                 case.max_seq_len)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_hidden(case.layer, case.x_new_dev, case.cu_q, case.seq_lens, case.page_table, case.cache,
                              out, case.max_q_len, case.max_seq_len,
                              workspace=torch.empty(need - 256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == mla.MLA_ERR_INSUFFICIENT_WORKSPACE
    with pytest.raises(mla.MlaError) as e:      # the fold reads W_uk
        mla.mla_fold_query(case.layer, to_dev(wl.w_q(), torch.bfloat16), None, FOL)
    assert e.value.status == mla.MLA_ERR_INVALID_ARG
    tiny = GpuCase(WORKLOADS["tiny_f32"])
    with pytest.raises(mla.MlaError) as e:      # fp32 layers have no projection kernels
        mla.mla_fold_query(tiny.layer, torch.zeros((64, 64), device="cuda"), None, UNF,
                           folded=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED
