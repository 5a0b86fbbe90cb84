"""GPU parity at the full sizes of every decode workload, in the launch
configuration bench.py times (one mla_decode_step per layer, the library's
own split choice): the whole batch is appended and decoded on the GPU, and
sampled (sequence, head) outputs are compared with the float64 oracle
computed one sequence at a time (for FP8 pages, over the oracle's own
quantized rows).  Tolerances as in test_parity_gpu.py."""
import time

import numpy as np
import pytest
import torch

from mla_synth import WORKLOADS

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import GpuCase, errors, oracle_outputs  # noqa: E402

BF16_REL_MAX = 1e-2
BF16_REL_RMS = 1e-2


def _sampled(name):
    wl = WORKLOADS[name]
    if name == "dsv2_ragged_paged_256":
        L, ql = wl.seq_lens(), wl.q_lens()
        seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), int(np.argmax(ql == 2))})
        return wl, seqs, [0, 64, 127]
    H = wl.shape.H
    return wl, [0, wl.batch - 1], [0, H // 2 + 5, H - 1]


@pytest.mark.parametrize("name", ["dsv2_b32_ctx4096", "llama2_7b_mla_b64_ctx8192", "dsv2_b8_ctx131072",
                                  "dsv2_ragged_paged_256", "dsv2_b32_ctx4096_fp8",
                                  "llama2_7b_mla_b64_ctx8192_fp8"])
def test_full_size_sampled(name):
    wl, seqs, heads = _sampled(name)
    t0 = time.time()
    print(f"\n[full] {name}: B={wl.batch}, max context {int(wl.seq_lens().max())}, building the cache",
          flush=True)
    case = GpuCase(wl, fill_sentinel=False)
    print(f"[full] {name}: cache built in {time.time() - t0:.0f}s; decode step", flush=True)
    s = wl.shape
    out = torch.empty((case.q.shape[0], s.H, s.d_v), dtype=case.dt, device="cuda")
    case.mla.mla_decode_step(case.layer, case.x_new_dev, case.cu_q, case.prefix_dev, case.q_dev, case.cu_q,
                             case.seq_lens, case.page_table, case.cache, out, case.max_q_len, case.max_seq_len)
    torch.cuda.synchronize()
    chunk = case.mla.mla_decode_kv_chunk(case.layer, wl.batch, case.max_q_len, case.max_seq_len, 0)
    got = out.float().cpu().numpy()
    cu = wl.cu_q()
    print(f"[full] {name}: decoded (kv_chunk {chunk}); oracle on sequences {seqs}, heads {heads}", flush=True)
    del out, case
    torch.cuda.empty_cache()
    for b in seqs:
        ref = oracle_outputs(wl, b, heads)
        e = errors(got[cu[b]:cu[b + 1]][:, heads], ref)
        print(f"[full] {name} seq {b} (L={int(wl.seq_lens()[b])}, q_len={int(wl.q_lens()[b])}): "
              f"max|d|/max|ref| {e[0]:.3e}, rms(d)/rms(ref) {e[1]:.3e}", flush=True)
        assert e[0] <= BF16_REL_MAX and e[1] <= BF16_REL_RMS, f"{name} seq {b}: errors {e}"
