"""GPU parity: the HIP path through the C ABI against the float64 oracle on
the same seeded inputs.

Tolerances: fp32 layers max|gpu - ref| / max|ref| <= 1e-4.  bf16 layers:
with the outputs scaled to unit maximum the largest absolute error is <= 1e-2
(max|gpu - ref| / max|ref| <= 1e-2, inside the 2e-2 maximum relative error),
and the aggregate error rms(gpu - ref) / rms(ref) <= 1e-2.  The bf16 output
is itself a rounding of the exact result (half an ulp is up to 2**-8 of an
element), so no bound on single elements relative to the typical output
magnitude can be tighter than a few times 2**-8."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, LLAMA2_7B_MLA, WORKLOADS, workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import GpuCase, errors, oracle_outputs  # noqa: E402

F32_TOL = 1e-4
BF16_REL_MAX = 1e-2
BF16_REL_RMS = 1e-2


def _check(case: GpuCase, out: torch.Tensor, seqs=None, heads=None, tag=""):
    wl = case.wl
    got = out.float().cpu().numpy()
    cu = wl.cu_q()
    seqs = range(wl.batch) if seqs is None else seqs
    worst = (0.0, 0.0, 0.0)
    bf16 = wl.shape.dtype != "f32"
    for b in seqs:
        ref = oracle_outputs(wl, b, heads, case.w_dkv, case.w_uk, case.w_uv)
        g = got[cu[b]:cu[b + 1]]
        if heads is not None:
            g = g[:, heads]
        e = errors(g, ref)
        worst = tuple(max(x, y) for x, y in zip(worst, e))
        if not bf16:
            assert e[0] <= F32_TOL, f"{tag} seq {b}: rel err {e[0]:.3e}"
        else:
            assert e[0] <= BF16_REL_MAX and e[1] <= BF16_REL_RMS, f"{tag} seq {b}: errors {e}"
    print(f"[parity] {tag}: max|d|/max|ref| {worst[0]:.3e}, rms(d)/rms(ref) {worst[1]:.3e}, "
          f"max|d|/rms(ref) {worst[2]:.3e}", flush=True)
    return worst


def _run(wl, kv_chunk=0, rows=0):
    """rows: split-KV rows per workgroup (0 by shape; 64 or 128 forces that kernel)."""
    import mla_compressed_latent_amd as mla
    print(f"[parity] case {wl.name} B={wl.batch} kv_chunk={kv_chunk} rows={rows}", flush=True)
    case = GpuCase(wl)
    if rows:
        mla.mla_layer_set_attention_rows(case.layer, rows)
    case.append_new()
    out = case.decode(kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    return case, out


def test_tiny_fp32_full():
    wl = WORKLOADS["tiny_f32"]
    case, out = _run(wl)
    _check(case, out, tag="tiny_f32")


def test_tiny_fp32_ragged_paged():
    wl = WORKLOADS["tiny_f32"].with_(name="tiny_f32_ragged", batch=5, fixed_prefix=None, max_prefix=300,
                                     fixed_q_len=None, max_q_len=2, paging="random", spare_page_frac=0.3)
    case, out = _run(wl, kv_chunk=64)
    _check(case, out, tag="tiny_f32_ragged")


SMALL_DSV2 = dataclasses.replace(DSV2, d_model=512)
SMALL_LLAMA = dataclasses.replace(LLAMA2_7B_MLA, d_model=512)


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("kv_chunk", [0, 64, 192])
def test_bf16_dsv2_hidden_prefix(kv_chunk, rows):
    wl = workload("dsv2_b32_ctx4096", name="dsv2_small", shape=SMALL_DSV2, batch=3, fixed_prefix=None,
                  max_prefix=700)
    case, out = _run(wl, kv_chunk=kv_chunk, rows=rows)
    _check(case, out, tag=f"dsv2_small chunk={kv_chunk} rows={rows}")


@pytest.mark.parametrize("rows", [64, 128])
def test_bf16_dsv2_ragged_paged_two_queries(rows):
    wl = workload("dsv2_ragged_paged_256", name="dsv2_ragged_small", batch=7, max_prefix=400)
    case, out = _run(wl, kv_chunk=128, rows=rows)
    _check(case, out, tag=f"dsv2_ragged_small rows={rows}")


@pytest.mark.parametrize("rows", [64, 128])
def test_work_list_ragged(rows):
    """More workgroups than compute units on a ragged batch: the attention
    launches from the device-built list of busy (sequence, split, row group)
    items.  Sampled heads against the oracle."""
    wl = workload("dsv2_ragged_paged_256", name=f"worklist_{rows}", shape=SMALL_DSV2, batch=40, max_prefix=400)
    case, out = _run(wl, kv_chunk=64, rows=rows)
    _check(case, out, heads=[0, 77, 127], tag=f"work list rows={rows}")
    again = case.decode(kv_chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "work-list launch not deterministic"


@pytest.mark.parametrize("rows", [64, 128])
def test_work_list_balanced(rows):
    """The work list ranks the splits by length and deals them over the
    XCDs: splits of many lengths (512-token splits of contexts up to 2500,
    so up to five per sequence and several rounds of sixteen), both row-group
    sizes, heads from every row group of every sequence against the oracle,
    and the same output on a second launch."""
    wl = workload("dsv2_ragged_paged_256", name=f"worklist_balanced_{rows}", shape=SMALL_DSV2, batch=33,
                  max_prefix=2500)
    case, out = _run(wl, kv_chunk=512, rows=rows)
    _check(case, out, heads=[0, 63, 64, 127], tag=f"balanced work list rows={rows}")
    again = case.decode(kv_chunk=512)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "work-list launch not deterministic"


@pytest.mark.parametrize("rows", [64, 128])
def test_partial_row_groups(rows):
    """40 heads: a one-query sequence has 40 rows and a two-query one 80, so
    the last row group of every sequence is partly empty (24 or 48 of 64 rows
    idle in the 64-row kernel, 88 or 48 of 128 in the 128-row one); every
    head against the oracle."""
    from mla_synth import Shape
    wl = workload("dsv2_ragged_paged_256", name=f"heads40_{rows}", shape=Shape(512, 40, 128, 64, 128, 512),
                  batch=5, max_prefix=900)
    case, out = _run(wl, kv_chunk=256, rows=rows)
    _check(case, out, tag=f"40 heads rows={rows}")


def test_attention_rows_override_is_validated():
    import mla_compressed_latent_amd as mla
    case = GpuCase(workload("dsv2_b32_ctx4096", name="rows_arg", shape=SMALL_DSV2, batch=1, fixed_prefix=16))
    for bad in (-1, 32, 96, 256):
        with pytest.raises(mla.MlaError):
            mla.mla_layer_set_attention_rows(case.layer, bad)


def test_bf16_llama_shape():
    wl = workload("llama2_7b_mla_b64_ctx8192", name="llama_small", shape=SMALL_LLAMA, batch=4,
                  fixed_prefix=None, max_prefix=900)
    case, out = _run(wl)
    _check(case, out, tag="llama_small")


def test_bf16_llama_two_queries_paged():
    wl = workload("llama2_7b_mla_b64_ctx8192", name="llama_q2", shape=SMALL_LLAMA, batch=5,
                  fixed_prefix=None, max_prefix=500, fixed_q_len=None, max_q_len=2, paging="random",
                  spare_page_frac=0.1)
    case, out = _run(wl, kv_chunk=256)
    _check(case, out, tag="llama_q2")


@pytest.mark.parametrize("rows", [64, 128])
def test_minimal_contexts(rows):
    """Context 1 (one query on its own row) and context 2 with two queries."""
    for q_len in (1, 2):
        wl = workload("dsv2_ragged_paged_256", name=f"minimal_q{q_len}", batch=2, fixed_prefix=0,
                      fixed_q_len=q_len)
        case, out = _run(wl, rows=rows)
        _check(case, out, tag=f"minimal q_len={q_len} rows={rows}")


def test_deterministic_and_page_permutation_invariant():
    wl = workload("dsv2_ragged_paged_256", name="perm", batch=4, max_prefix=300)
    case, out1 = _run(wl, kv_chunk=128)
    out2 = case.decode(kv_chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "two runs differ"
    # same logical cache, different physical pages (different seed for the permutation)
    wl2 = wl.with_(seed=wl.seed)  # same data
    case2 = GpuCase(wl2)
    perm = np.random.default_rng(99).permutation(case2.num_pages).astype(np.int32)
    new_table = np.where(case2.table_np >= 0, perm[np.maximum(case2.table_np, 0)], -1).astype(np.int32)
    src = torch.from_numpy(case2.table_np[case2.table_np >= 0].astype(np.int64)).cuda()
    dst = torch.from_numpy(new_table[case2.table_np >= 0].astype(np.int64)).cuda()
    moved = case2.cache.clone()
    moved[dst] = case2.cache[src]
    case2.cache = moved
    case2.table_np = new_table
    case2.page_table = torch.from_numpy(new_table).cuda()
    case2.append_new()
    out3 = case2.decode(kv_chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(out1, out3), "page permutation changed the result"


def test_split_invariance():
    import mla_compressed_latent_amd as mla
    wl = workload("dsv2_b32_ctx4096", name="splits", shape=SMALL_DSV2, batch=2, fixed_prefix=1000)
    case, out_a = _run(wl, kv_chunk=64)
    out_b = case.decode(kv_chunk=1024)
    out_c = case.decode(kv_chunk=0)
    mla.mla_layer_set_attention_rows(case.layer, 128)
    out_d = case.decode(kv_chunk=64)
    out_e = case.decode(kv_chunk=1024)
    torch.cuda.synchronize()
    a, *rest = (o.float().cpu().numpy() for o in (out_a, out_b, out_c, out_d, out_e))
    scale = np.abs(a).max()
    for r in rest:
        assert np.abs(a - r).max() / scale < 1e-2


def test_many_splits_separate_combine():
    """More splits than the fused combine stages (64): the separate combine and
    output-projection kernels run instead; sampled heads against the oracle."""
    import mla_compressed_latent_amd as mla
    wl = workload("dsv2_b32_ctx4096", name="many_splits", shape=SMALL_DSV2, batch=2, fixed_prefix=4500)
    case, out = _run(wl, kv_chunk=64)
    heads = [0, 37, 127]
    _check(case, out, heads=heads, tag="many_splits chunk=64 (71 splits)")
    out_fused = case.decode(kv_chunk=128)     # 36 splits: fused combine + projection
    torch.cuda.synchronize()
    _check(case, out_fused, heads=heads, tag="many_splits chunk=128 (36 splits)")
    mla.mla_layer_set_attention_rows(case.layer, 128)   # bf16 partials of the 128-row kernel
    for chunk in (64, 128):
        out128 = case.decode(kv_chunk=chunk)
        torch.cuda.synchronize()
        _check(case, out128, heads=heads, tag=f"many_splits chunk={chunk} rows=128")


def test_split_limit():
    """The planner's largest split count: a 65536-token context in 64-token
    splits is 1024 splits of two 64-row groups (a launch from the balanced
    work list, the separate combine with 1024 split weights staged on
    chip), sampled heads of both row groups against the oracle; one token
    more needs 1025 splits and the planner refuses it, as it refuses a launch
    grid past the int range."""
    import mla_compressed_latent_amd as mla
    wl = workload("dsv2_b32_ctx4096", name="split_limit", shape=SMALL_DSV2, batch=1, fixed_prefix=65535)
    case, out = _run(wl, kv_chunk=64)
    _check(case, out, heads=[0, 63, 64, 127], tag="1024 splits of 64 tokens")
    assert mla.mla_decode_workspace_bytes(case.layer, 1, 1, 1, 64 * 1024, 64) > 0
    assert mla.mla_decode_workspace_bytes(case.layer, 1, 1, 1, 64 * 1024 + 1, 64) == 0
    # a launch grid past 2^31 workgroups is refused too (2^21 sequences x 1024 splits x 2 row groups)
    assert mla.mla_decode_workspace_bytes(case.layer, 1 << 21, 1 << 21, 1, 64 * 1024, 64) == 0


def test_split_plan_of_the_benchmarked_shapes():
    """The planner's split sizes for the benchmarked decode shapes on a
    256-CU MI355X (one wave of workgroups, splits up to 8192 tokens; 128-row
    workgroups where their split reaches 1024 tokens, 64-row ones else)."""
    import mla_compressed_latent_amd as mla
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("split sizes are stated for 256 compute units")
    cases = [  # (shape, batch, max_q_len, max_seq_len, expected tokens per split)
        (SMALL_DSV2, 32, 1, 4096, 1024),
        (SMALL_DSV2, 8, 1, 131072, 4096),
        (SMALL_DSV2, 256, 2, 32770, 8192),
        (SMALL_LLAMA, 64, 1, 8192, 2048),
    ]
    for shape, B, q, L, expect in cases:
        case = GpuCase(workload("dsv2_b32_ctx4096", name="plan", shape=shape, batch=1, fixed_prefix=16))
        got = mla.mla_decode_kv_chunk(case.layer, B, q, L)
        assert got == expect, (shape.H, B, q, L, got)
