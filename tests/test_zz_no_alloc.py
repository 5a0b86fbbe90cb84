"""mla_decode_no_alloc (the decode entry point that works in the library's
static device scratch) against mla_decode on the same inputs: two calls in a
row, the second with a smaller batch, for the bf16 kernels of both row
blockings, for FP8 pages and for an fp32 layer, and the rejection of a call whose workspace
exceeds the scratch.  Both entry points run the same kernels with the same
split plan, so their outputs must be bit-identical."""
import dataclasses

import pytest
import torch

from mla_synth import DSV2, WORKLOADS, workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import GpuCase, errors, oracle_outputs  # noqa: E402

SMALL_DSV2 = dataclasses.replace(DSV2, d_model=512)


def _both(case, kv_chunk=0):
    """(mla_decode output, mla_decode_no_alloc output) for the case's queries."""
    mla = case.mla
    s = case.wl.shape
    ref = case.decode(kv_chunk=kv_chunk)
    got = torch.full((case.q.shape[0], s.H, s.d_v), float("nan"), dtype=case.dt, device="cuda")
    mla.mla_decode_no_alloc(case.layer, case.q_dev, case.cu_q, case.seq_lens, case.page_table, case.cache, got,
                            case.max_q_len, case.max_seq_len, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    return ref, got


def _case(wl, rows):
    case = GpuCase(wl)
    if rows:
        case.mla.mla_layer_set_attention_rows(case.layer, rows)
    case.append_new()
    return case


@pytest.mark.parametrize("rows", [64, 128])
def test_no_alloc_matches_decode_two_calls(rows):
    big = workload("dsv2_ragged_paged_256", name="noalloc_big", shape=SMALL_DSV2, batch=6, max_prefix=1500)
    small = workload("dsv2_ragged_paged_256", name="noalloc_small", shape=SMALL_DSV2, batch=2, max_prefix=300,
                     seed=big.seed + 1)
    for wl in (big, small):
        print(f"[no_alloc] {wl.name} B={wl.batch} rows={rows}", flush=True)
        case = _case(wl, rows)
        need = case.mla.mla_decode_workspace_bytes(case.layer, wl.batch, case.q.shape[0], case.max_q_len,
                                                  case.max_seq_len, 0)
        assert 0 < need <= case.mla.MLA_NO_ALLOC_SCRATCH_BYTES
        ref, got = _both(case)
        assert torch.equal(ref, got), f"{wl.name}: no-alloc output differs from mla_decode"
    # the smaller call also against the oracle, on a few heads
    cu = small.cu_q()
    heads = [0, 77, 127]
    out = got.float().cpu().numpy()
    for b in range(small.batch):
        e = errors(out[cu[b]:cu[b + 1]][:, heads], oracle_outputs(small, b, heads, case.w_dkv, case.w_uk,
                                                                  case.w_uv))
        assert e[0] <= 1e-2 and e[1] <= 1e-2, (b, e)


def test_no_alloc_with_work_list():
    """A ragged batch big enough that the attention launches from its
    device-built work list (kept in the scratch too)."""
    wl = workload("dsv2_ragged_paged_256", name="noalloc_list", shape=SMALL_DSV2, batch=40, max_prefix=400)
    case = _case(wl, 0)
    # 128-token splits: 40 x 4 x 4 = 640 workgroups (more than one wave of
    # them, so the list is used) in 31 MB of scratch
    ref, got = _both(case, kv_chunk=128)
    assert torch.equal(ref, got)


def test_no_alloc_fp8_pages_two_calls():
    """FP8 pages (the eight-wave kernel's converting path), two calls in a
    row, the second with a smaller batch."""
    fp8 = dataclasses.replace(SMALL_DSV2, cache_format="fp8")
    for batch, prefix in ((5, 900), (2, 200)):
        wl = workload("dsv2_ragged_paged_256", name=f"noalloc_fp8_b{batch}", shape=fp8, batch=batch,
                      max_prefix=prefix, prefix_source="hidden", seed=40 + batch)
        print(f"[no_alloc] {wl.name} B={wl.batch}", flush=True)
        case = _case(wl, 0)
        ref, got = _both(case, kv_chunk=64)
        assert torch.equal(ref, got), f"{wl.name}: no-alloc output differs from mla_decode"


def test_no_alloc_fp32_layer_two_calls():
    for batch, prefix in ((4, 250), (2, 90)):
        wl = WORKLOADS["tiny_f32"].with_(name=f"noalloc_f32_b{batch}", batch=batch, fixed_prefix=None,
                                         max_prefix=prefix)
        print(f"[no_alloc] {wl.name}", flush=True)
        case = _case(wl, 0)
        ref, got = _both(case, kv_chunk=64)
        assert torch.equal(ref, got), wl.name


def test_no_alloc_rejects_a_workspace_beyond_the_scratch():
    mla = __import__("mla_compressed_latent_amd")
    wl = workload("dsv2_b32_ctx4096", name="noalloc_over", shape=SMALL_DSV2, batch=8, fixed_prefix=4500)
    case = _case(wl, 64)
    need = mla.mla_decode_workspace_bytes(case.layer, wl.batch, case.q.shape[0], case.max_q_len,
                                          case.max_seq_len, 64)
    assert need > mla.MLA_NO_ALLOC_SCRATCH_BYTES
    out = torch.empty((case.q.shape[0], wl.shape.H, wl.shape.d_v), dtype=case.dt, device="cuda")
    with pytest.raises(mla.MlaError) as ei:
        mla.mla_decode_no_alloc(case.layer, case.q_dev, case.cu_q, case.seq_lens, case.page_table, case.cache,
                                out, case.max_q_len, case.max_seq_len, kv_chunk=64)
    assert ei.value.status == 4 and "scratch" in str(ei.value)     # MLA_ERR_INSUFFICIENT_WORKSPACE
    # the same batch with longer splits fits and matches mla_decode
    ref, got = _both(case, kv_chunk=1024)
    assert torch.equal(ref, got)
