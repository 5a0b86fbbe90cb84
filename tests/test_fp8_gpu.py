"""GPU: the 8-bit float latent cache (MLA_CACHE_FP8).

Append: every cached latent element decodes (code * 2^e, read back from the
page bytes) to within half a code spacing of the oracle's exact latent, plus
the GPU's fp32 accumulation error; the scale is the oracle's power of two;
the rope key matches as in a bf16 cache; bytes of rows that were not
appended stay untouched.  Attention: mla_decode over FP8 pages (both split-KV
kernels: 32 and 128 heads) against the oracle attending over its own
quantized rows, to the bf16 tolerances of the decode parity tests."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, LLAMA2_7B_MLA, WORKLOADS, workload
from oracle import fp8

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mla_compressed_latent_amd as mla  # noqa: E402
from oracle import mla_oracle  # noqa: E402
from gpu_harness import SENTINEL_BYTE, GpuCase, errors, oracle_cache, oracle_outputs, oracle_query  # noqa: E402

FP8_DSV2 = dataclasses.replace(DSV2, d_model=512, cache_format="fp8")
FP8_LLAMA = dataclasses.replace(LLAMA2_7B_MLA, d_model=512, cache_format="fp8")
ROW = 640


def _case(wl):
    print(f"[fp8] case {wl.name} B={wl.batch} heads={wl.shape.H}", flush=True)
    case = GpuCase(wl)
    case.append_new()
    torch.cuda.synchronize()
    return case


def _read_rows(case, b):
    """(codes [L][512], scales [L], rope [L][64] float) of sequence b from the page bytes."""
    wl, ps = case.wl, case.wl.shape.page_size
    L = int(case.seq_lens_np[b])
    pages = case.cache.cpu().numpy()
    codes, scales, rope = [], [], []
    for t in range(L):
        pg = pages[case.table_np[b, t // ps]]
        r = t % ps
        row = pg[r * ROW:(r + 1) * ROW]
        codes.append(row[:512])
        scales.append(pg[ps * ROW + 4 * r: ps * ROW + 4 * r + 4].view(np.float32)[0])
        rope.append((row[512:].view(np.uint16).astype(np.uint32) << 16).view(np.float32))
    return np.array(codes), np.array(scales, dtype=np.float64), np.array(rope, dtype=np.float64)


def test_append_fp8_rows():
    wl = workload("dsv2_b32_ctx4096", name="fp8_append", shape=FP8_DSV2, batch=3, fixed_prefix=None,
                  max_prefix=300, paging="random", spare_page_frac=0.3, seed=31)
    case = _case(wl)
    for b in range(wl.batch):
        codes, scales, rope = _read_rows(case, b)
        ref = oracle_cache(wl, b, case.w_dkv, quantize=False)
        c = ref[:, :512]
        assert not np.isnan(fp8.DECODE_TABLE[codes]).any()
        e = np.log2(scales)
        assert np.array_equal(e, np.round(e)), "scales are powers of two"
        amax = np.abs(c).max(axis=1)
        e_ref = np.array([fp8.row_scale_exponent(a) for a in amax])
        near = np.abs(np.log2(amax / 448.0) - np.round(np.log2(amax / 448.0))) < 1e-5
        assert np.all((e == e_ref) | near), "scale exponent differs away from a binade boundary"
        deq = fp8.DECODE_TABLE[codes] * scales[:, None]
        a = np.abs(c) * (1 + 1e-5) / scales[:, None]
        spacing = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3), 2.0 ** -9)
        bound = 0.5 * spacing * scales[:, None] + 1e-5 * amax[:, None]
        assert np.all(np.abs(deq - c) <= bound), float((np.abs(deq - c) / bound).max())
        rr = ref[:, 512:]
        assert np.all(np.abs(rope - rr) <= 2.0 ** -8 * np.abs(rr) + 1e-5 * np.abs(rr).max())
    # rows past each sequence's end, and pages nobody owns, were never written
    pages = case.cache.cpu().numpy()
    ps = wl.shape.page_size
    owned = set()
    for b in range(wl.batch):
        L = int(case.seq_lens_np[b])
        for p_i in range((L + ps - 1) // ps):
            pg = int(case.table_np[b, p_i])
            owned.add(pg)
            last = min(ps, L - p_i * ps)
            assert (pages[pg][last * ROW: ps * ROW] == SENTINEL_BYTE).all()
            assert (pages[pg][ps * ROW + 4 * last:] == SENTINEL_BYTE).all()
    for pg in range(case.num_pages):
        if pg not in owned:
            assert (pages[pg] == SENTINEL_BYTE).all()


def _unquantized_outputs(case, b, heads):
    """The oracle's attention over sequence b's rows WITHOUT the FP8 rounding
    (information only: how far the quantized cache moves the output)."""
    wl, s = case.wl, case.wl.shape
    rows = oracle_cache(wl, b, case.w_dkv, quantize=False)
    return mla_oracle.attend_sequence(wl.queries(b), rows, case.w_uk, case.w_uv, s.H, s.d_nope, s.d_v, s.rope_base,
                                      mla_oracle.default_scale(s.d_nope, s.d_rope), heads)


def _check(case, out, tag, heads=None):
    """Parity against the oracle over its own quantized rows (asserted), and
    the deviation from the unquantized oracle (printed beside it)."""
    wl = case.wl
    got = out.float().cpu().numpy()
    cu = wl.cu_q()
    worst = (0.0, 0.0)
    dev = (0.0, 0.0)
    for b in range(wl.batch):
        ref = oracle_outputs(wl, b, heads, case.w_dkv, case.w_uk, case.w_uv)
        g = got[cu[b]:cu[b + 1]]
        if heads is not None:
            g = g[:, heads]
        e = errors(g, ref)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        assert e[0] <= 1e-2 and e[1] <= 1e-2, f"{tag} seq {b}: {e}"
        u = errors(g, _unquantized_outputs(case, b, heads))
        dev = (max(dev[0], u[0]), max(dev[1], u[1]))
    print(f"[fp8] {tag}: max|d|/max|ref| {worst[0]:.3e}, rms ratio {worst[1]:.3e}; against the unquantized "
          f"oracle (information): max|d|/max|ref| {dev[0]:.3e}, rms ratio {dev[1]:.3e}", flush=True)


@pytest.mark.parametrize("shape", [FP8_DSV2, FP8_LLAMA], ids=["128heads", "32heads"])
@pytest.mark.parametrize("kv_chunk", [0, 64])
def test_fp8_decode_parity(shape, kv_chunk):
    """Ragged prefixes ~U[1, 700], one or two queries, random pages, several
    splits: the eight-wave kernel (128 heads) and the 32-row kernel (32 heads)."""
    wl = workload("dsv2_ragged_paged_256", name=f"fp8_decode_{shape.H}", shape=shape, batch=4,
                  max_prefix=700, prefix_source="hidden", seed=32)
    case = _case(wl)
    out = case.decode(kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    _check(case, out, f"decode heads={shape.H} chunk={kv_chunk}")


def test_fp8_work_list():
    """FP8 pages on a ragged decode batch larger than one wave of workgroups
    (40 sequences, 64-token splits): the eight-wave kernel launched from the
    balanced work list, heads of every row group against the oracle."""
    wl = workload("dsv2_ragged_paged_256", name="fp8_work_list", shape=FP8_DSV2, batch=40,
                  max_prefix=600, prefix_source="hidden", seed=35)
    case = _case(wl)
    out = case.decode(kv_chunk=64)
    torch.cuda.synchronize()
    _check(case, out, "decode work list chunk=64", heads=[0, 63, 64, 127])


def test_fp8_deterministic():
    wl = workload("dsv2_ragged_paged_256", name="fp8_det", shape=FP8_DSV2, batch=3, max_prefix=400,
                  prefix_source="hidden", seed=33)
    case = _case(wl)
    a = case.decode(kv_chunk=128)
    b = case.decode(kv_chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_fp8_extend():
    """Chunked extend over FP8 pages: the absorbed form (what AUTO takes);
    the expanded form reads bf16 rows and refuses the layer."""
    wl = workload("dsv2_ragged_paged_256", name="fp8_extend", shape=FP8_DSV2, batch=2, max_prefix=200,
                  fixed_q_len=150, prefix_source="hidden", seed=34)
    case = _case(wl)
    out = case.extend(mla.MLA_EXTEND_AUTO)
    torch.cuda.synchronize()
    _check(case, out, "extend auto (absorbed)")
    with pytest.raises(mla.MlaError) as e:
        case.extend(mla.MLA_EXTEND_EXPANDED)
    assert e.value.status == 2


def test_fp8_full_size_sampled():
    """The benchmarked FP8 configuration (DeepSeek-V2, batch 32, context 4096)
    at sampled sequences and heads."""
    wl = WORKLOADS["dsv2_b32_ctx4096_fp8"]
    case = _case(wl)
    out = case.decode().float().cpu().numpy()
    torch.cuda.synchronize()
    heads = [0, 63, 127]
    for b in (0, 17, 31):
        cache = oracle_cache(wl, b, case.w_dkv)
        ref = oracle_query(wl, b, 0, heads, cache, wl.queries(b), case.w_uk, case.w_uv)
        e = errors(out[b][heads], ref)
        assert e[0] <= 1e-2 and e[1] <= 1e-2, (b, e)
    print("[fp8] full size sampled within tolerance", flush=True)
