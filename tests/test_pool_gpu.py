"""GPU: a stack of layers over one pool-managed page table (mla_pool_*).

Three layers with different weights share the pages of three sequences that
the pool placed among pages other sequences took and gave back; each layer
appends its prefixes and new tokens and decodes through the same table.
Every layer's output matches the float64 oracle for that layer's weights
(bf16 tolerances of the decode parity tests), and pages that belong to no
sequence of the batch are untouched in every layer."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, workload

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mla_compressed_latent_amd as mla  # noqa: E402
from gpu_harness import SENTINEL_BYTE, errors, i32, oracle_outputs, to_dev  # noqa: E402

LAYERS = 3


def test_layer_stack_on_pool_pages():
    shape = dataclasses.replace(DSV2, d_model=512)
    wl = workload("dsv2_ragged_paged_256", name="pool_stack", shape=shape, batch=3, max_prefix=400,
                  seed=21, prefix_source="hidden")
    print(f"[pool] case {wl.name} prefix={wl.prefix_lens().tolist()} q={wl.q_lens().tolist()}", flush=True)
    ps = shape.page_size
    pool = mla.PagePool(48, ps, 8, 8)
    # other sequences come and go first, so the batch's pages are scattered
    pool.reserve(5, 200)
    pool.reserve(6, 3 * ps)
    pool.reserve(7, ps)              # stays alive: its page sits among the batch's
    pool.release(5)
    seq_ids = [1, 4, 2]
    seq_lens = wl.seq_lens()
    for b, sid in enumerate(seq_ids):
        pool.reserve(sid, int(wl.prefix_lens()[b]))
        if b == 1:
            pool.release(6)
    for b, sid in enumerate(seq_ids):           # grow by the new tokens
        pool.reserve(sid, int(seq_lens[b]))
    table_np = pool.page_table(seq_ids)
    owned = sorted({int(p) for p in table_np.ravel() if p >= 0})
    rows = [[int(p) for p in r if p >= 0] for r in table_np]
    assert any(r != list(range(r[0], r[0] + len(r))) for r in rows), "some row should be scattered"
    assert owned != list(range(len(owned))), "another sequence's page should sit among them"
    table = i32(table_np)
    caches = torch.empty((LAYERS, 48, ps, shape.row_width), dtype=torch.bfloat16, device="cuda")
    caches.view(torch.uint8).fill_(SENTINEL_BYTE)

    B = wl.batch
    prefix = wl.prefix_lens()
    xs = [wl.prefix_hidden(b) for b in range(B)]
    x_pre = to_dev(np.concatenate(xs, axis=0), torch.bfloat16)
    cu_pre = i32(np.concatenate([[0], np.cumsum([x.shape[0] for x in xs])]))
    x_new = to_dev(wl.new_hidden(), torch.bfloat16)
    q = to_dev(wl.queries(), torch.bfloat16)
    cu_q = i32(wl.cu_q())
    outs, weights = [], []
    for l in range(LAYERS):
        # layer l: the workload's weights with columns rotated by 7 l
        w = [np.ascontiguousarray(np.roll(a, 7 * l, axis=1)) for a in (wl.w_dkv(), wl.w_uk(), wl.w_uv())]
        weights.append(w)
        layer = mla.mla_fold_weights(mla.config_from_shape(shape), *(to_dev(a, torch.bfloat16) for a in w))
        cache = caches[l]
        mla.mla_append_latent(layer, x_pre, cu_pre, i32(np.zeros(B)), table, cache)
        mla.mla_append_latent(layer, x_new, cu_q, i32(prefix), table, cache)
        out = torch.empty((q.shape[0], shape.H, shape.d_v), dtype=torch.bfloat16, device="cuda")
        mla.mla_decode(layer, q, cu_q, i32(seq_lens), table, cache, out, int(wl.q_lens().max()),
                       int(seq_lens.max()))
        outs.append(out)
    torch.cuda.synchronize()
    cu = wl.cu_q()
    for l in range(LAYERS):
        got = outs[l].float().cpu().numpy()
        for b in range(B):
            ref = oracle_outputs(wl, b, None, *weights[l])
            e = errors(got[cu[b]:cu[b + 1]], ref)
            assert e[0] <= 1e-2 and e[1] <= 1e-2, (l, b, e)
        print(f"[pool] layer {l} within tolerance", flush=True)
    # pages no sequence of the batch owns were never written, in any layer
    free_pages = [p for p in range(48) if p not in owned]
    untouched = caches[:, free_pages].view(torch.uint8)
    assert bool((untouched == SENTINEL_BYTE).all())
    # the layers differ (different weights), so the test is not vacuous
    assert not torch.equal(caches[0, owned[0]], caches[1, owned[0]])
