"""GPU parity of prefill / chunked extend (mla_extend) through the C ABI:
both forms (absorbed, expanded) against the float64 oracle -- the same
unabsorbed attention the decode tests use -- on chunks that span several
128-query blocks and 64-key tiles with ragged tails, an empty prefix (pure
prefill), single queries, random page tables, every head width the expanded
kernels are built for, and the DeepSeek-V2 chunked-extend size on sampled
(query, head) pairs.  Tolerances as the decode parity tests: bf16
max|d|/max|ref| <= 1e-2 and rms(d)/rms(ref) <= 1e-2."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, WORKLOADS, Shape, workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mla_compressed_latent_amd as mla  # noqa: E402
from gpu_harness import GpuCase, errors, oracle_cache, oracle_outputs, oracle_query  # noqa: E402

BF16_REL_MAX = 1e-2
BF16_REL_RMS = 1e-2
ABS, EXP, AUTO = mla.MLA_EXTEND_ABSORBED, mla.MLA_EXTEND_EXPANDED, mla.MLA_EXTEND_AUTO
PATH_NAME = {ABS: "absorbed", EXP: "expanded", AUTO: "auto"}


def _case(wl):
    print(f"[extend] case {wl.name} B={wl.batch} q_lens={wl.q_lens().tolist()[:8]} "
          f"prefix={wl.prefix_lens().tolist()[:8]}", flush=True)
    case = GpuCase(wl)
    case.append_new()
    return case


def _check_all(case, out, tag):
    wl = case.wl
    got = out.float().cpu().numpy()
    cu = wl.cu_q()
    worst = (0.0, 0.0, 0.0)
    for b in range(wl.batch):
        ref = oracle_outputs(wl, b, None, case.w_dkv, case.w_uk, case.w_uv)
        e = errors(got[cu[b]:cu[b + 1]], ref)
        worst = tuple(max(x, y) for x, y in zip(worst, e))
        assert e[0] <= BF16_REL_MAX and e[1] <= BF16_REL_RMS, f"{tag} seq {b}: errors {e}"
    print(f"[extend] {tag}: max|d|/max|ref| {worst[0]:.3e}, rms(d)/rms(ref) {worst[1]:.3e}", flush=True)


def _shape(dn, dv, H=4):
    return Shape(256, H, dn, 64, dv, 512)


@pytest.mark.parametrize("dn,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("path", [EXP, ABS])
def test_ragged_chunks_paged(dn, dv, path):
    """Three sequences, prefixes ~U[1, 300], chunks ~U[1, 300] (up to three
    query blocks, ragged tails), random page table with spare pages."""
    wl = workload("dsv2_ragged_paged_256", name=f"ext_{dn}_{dv}", shape=_shape(dn, dv), batch=3,
                  max_prefix=300, max_q_len=300, seed=11)
    case = _case(wl)
    out = case.extend(path)
    torch.cuda.synchronize()
    _check_all(case, out, f"ragged dn={dn} dv={dv} {PATH_NAME[path]}")


@pytest.mark.parametrize("path", [EXP, ABS])
def test_prefill_empty_prefix(path):
    """Pure prefill: no cached prefix, 200 and 65 new tokens (a query block
    and a key tile each with a one-token tail)."""
    for q_len in (200, 65):
        wl = workload("dsv2_ragged_paged_256", name=f"prefill_{q_len}", shape=_shape(128, 128, H=3), batch=1,
                      fixed_prefix=0, fixed_q_len=q_len, paging="identity", seed=12)
        case = _case(wl)
        out = case.extend(path)
        torch.cuda.synchronize()
        _check_all(case, out, f"prefill {q_len} {PATH_NAME[path]}")


@pytest.mark.parametrize("H", [2, 6, 8])
def test_expanded_head_groups(H):
    """The expansion runs a workgroup's group of heads (four when they divide
    H, else two, else one) through one copy pipeline: head counts giving
    groups of two (2, 6) and two groups of four (8), ragged and paged."""
    wl = workload("dsv2_ragged_paged_256", name=f"ext_heads{H}", shape=_shape(128, 128, H=H), batch=3,
                  max_prefix=300, max_q_len=300, seed=15)
    case = _case(wl)
    out = case.extend(EXP)
    torch.cuda.synchronize()
    _check_all(case, out, f"expanded H={H}")


def test_expanded_single_queries_and_one_token():
    """Degenerate extends on the expanded path: one query per sequence, and a
    sequence whose whole context is its one query."""
    wl = workload("dsv2_ragged_paged_256", name="ext_q1", shape=_shape(128, 128), batch=5, max_prefix=200,
                  fixed_q_len=1, seed=13)
    case = _case(wl)
    out = case.extend(EXP)
    torch.cuda.synchronize()
    _check_all(case, out, "expanded q_len=1")
    wl = workload("dsv2_ragged_paged_256", name="ext_ctx1", shape=_shape(64, 64), batch=2, fixed_prefix=0,
                  fixed_q_len=1, seed=14)
    case = _case(wl)
    out = case.extend(EXP)
    torch.cuda.synchronize()
    _check_all(case, out, "expanded context 1")


def test_auto_is_the_chosen_path_and_deterministic():
    wl = workload("dsv2_ragged_paged_256", name="ext_auto", shape=_shape(128, 128), batch=2, fixed_prefix=None,
                  max_prefix=100, fixed_q_len=400, seed=15)
    case = _case(wl)
    chosen = mla.mla_extend_choose_path(case.cfg, wl.batch, int(wl.q_lens().sum()), case.max_q_len,
                                        case.max_seq_len)
    assert chosen in (ABS, EXP)
    a = case.extend(AUTO)
    b = case.extend(chosen)
    c = case.extend(chosen)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(b, c)


def test_path_errors():
    tiny = GpuCase(WORKLOADS["tiny_f32"])
    tiny.append_new()
    with pytest.raises(mla.MlaError) as e:
        tiny.extend(EXP)
    assert e.value.status == 2              # no expanded kernels for fp32 layers
    assert mla.mla_extend_workspace_bytes(tiny.layer, 1, 1, 1, tiny.max_seq_len, EXP) == 0
    out = tiny.extend(AUTO)                 # AUTO takes the absorbed form
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    wl = workload("dsv2_ragged_paged_256", name="ext_ws", shape=_shape(64, 64), batch=2, max_prefix=50,
                  fixed_q_len=3, seed=16)
    case = _case(wl)
    need = mla.mla_extend_workspace_bytes(case.layer, 2, 6, 3, case.max_seq_len, EXP)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        case.extend(EXP, workspace=ws)
    assert e.value.status == 4
    with pytest.raises(mla.MlaError) as e:
        case.extend(7)
    assert e.value.status == 1


def test_dsv2_chunked_extend_full_size_sampled():
    """DeepSeek-V2 shape (128 heads, d_model 5120), 4 sequences, prefix 3072,
    chunk 1024 -- the benchmarked chunked-extend configuration -- both forms,
    at sampled (query, head) pairs against the oracle, plus the two forms
    against each other everywhere."""
    wl = WORKLOADS["dsv2_extend_b4_p3072_c1024"]
    case = _case(wl)
    outs = {}
    for path in (EXP, ABS):
        outs[path] = case.extend(path).float().cpu().numpy()
    torch.cuda.synchronize()
    cu = wl.cu_q()
    rng = np.random.default_rng(7)
    for b in (0, wl.batch - 1):
        cache = oracle_cache(wl, b, case.w_dkv)
        q_b = wl.queries(b)
        ql = q_b.shape[0]
        qis = sorted({0, 127, 128, ql - 1, *rng.integers(0, ql, 3).tolist()})
        heads = [0, 77, 127]
        for i in qis:
            ref = oracle_query(wl, b, i, heads, cache, q_b, case.w_uk, case.w_uv)
            for path in (EXP, ABS):
                got = outs[path][cu[b] + i][heads]
                e = errors(got, ref)
                assert e[0] <= BF16_REL_MAX and e[1] <= BF16_REL_RMS, (PATH_NAME[path], b, i, e)
        print(f"[extend] full size seq {b}: queries {qis} heads {heads} within tolerance", flush=True)
    e = errors(outs[ABS], outs[EXP])
    print(f"[extend] full size absorbed vs expanded: {e}", flush=True)
    assert e[0] <= 2 * BF16_REL_MAX and e[1] <= BF16_REL_RMS
