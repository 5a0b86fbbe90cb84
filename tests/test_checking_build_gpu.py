"""The checking build (libmla_debug.so: device-resident offsets, lengths and
page ids verified by a kernel before each call's own kernels) on valid
inputs: its append, decode, decode-step and expanded-extend results are
bit-identical to the release build's on the same inputs.  Bad ids are
tested on the CPU only (tests/test_host_sanitized.py drives the same check
functions)."""
import dataclasses

import pytest
import torch

from mla_synth import DSV2, workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import GpuCase  # noqa: E402

SMALL_DSV2 = dataclasses.replace(DSV2, d_model=512)


def _outputs(wl):
    case = GpuCase(wl)
    case.append_new()
    dec = case.decode(kv_chunk=128)
    s = wl.shape
    step = torch.empty_like(dec)
    case.mla.mla_decode_step(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.q_dev, case.cu_q,
                             case.seq_lens, case.page_table, case.cache, step, case.max_q_len, case.max_seq_len)
    ext = case.extend(case.mla.MLA_EXTEND_EXPANDED)
    torch.cuda.synchronize()
    return {"cache": case.cache.clone(), "decode": dec, "step": step, "extend": ext,
            "shape": (case.q.shape[0], s.H, s.d_v)}


def test_checking_build_matches_release_on_valid_inputs():
    import mla_compressed_latent_amd as mla
    wl = workload("dsv2_ragged_paged_256", name="checked", shape=SMALL_DSV2, batch=5, max_prefix=300)
    print(f"[checking build] {wl.name} B={wl.batch}: release", flush=True)
    ref = _outputs(wl)
    mla.use_library("debug")
    try:
        print("[checking build] same inputs through libmla_debug.so", flush=True)
        got = _outputs(wl)
    finally:
        mla.use_library("release")
    for k in ("cache", "decode", "step", "extend"):
        assert torch.equal(ref[k], got[k]), f"{k} differs between the release and checking builds"
