"""The seeded input generator: determinism, bf16 rounding, lengths and page
tables.  (Host-only; no GPU.)"""
import numpy as np
import pytest
import torch

from mla_synth import WORKLOADS, bf16_bits, bf16_bits_to_f32, round_to_bf16, workload
from oracle.rounding import bf16_value_to_bits, rne_bf16_value


def test_bf16_rounding_matches_torch_and_oracle_rounding():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, 65504.0])])
    mine = round_to_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(mine, ref)
    assert np.array_equal(bf16_bits(mine), bf16_value_to_bits(rne_bf16_value(a.astype(np.float64))))
    assert np.array_equal(bf16_bits_to_f32(bf16_bits(mine)), mine)


def test_deterministic_and_per_sequence_keyed():
    wl = workload("dsv2_b32_ctx4096", fixed_prefix=20, batch=3)
    a, b = wl.w_uk(), wl.w_uk()
    assert np.array_equal(a, b) and a.shape == (512, 128 * 128)
    # sequence 1's prefix does not depend on the batch size
    assert np.array_equal(wl.prefix_hidden(1), wl.with_(batch=5).prefix_hidden(1))
    assert not np.array_equal(wl.prefix_hidden(0), wl.prefix_hidden(1))
    assert np.array_equal(round_to_bf16(a), a)        # already bf16-exact
    q = wl.queries()
    assert q.shape == (3, 128, 192)


def test_weight_scale():
    wl = workload("dsv2_b32_ctx4096")
    w = wl.w_dkv()
    assert w.shape == (5120, 576)
    assert abs(w.std() * np.sqrt(5120) - 1.0) < 0.01


def test_ragged_lengths_and_random_pages():
    wl = WORKLOADS["dsv2_ragged_paged_256"]
    p, ql, L = wl.prefix_lens(), wl.q_lens(), wl.seq_lens()
    assert p.min() >= 1 and p.max() <= 32768 and set(np.unique(ql)) == {1, 2}
    assert np.array_equal(L, p + ql)
    table, n = wl.page_table()
    npg = wl.pages_per_seq()
    used = np.concatenate([table[b, :npg[b]] for b in range(wl.batch)])
    assert len(np.unique(used)) == len(used) and used.min() >= 0 and used.max() < n
    assert n >= int(1.05 * npg.sum())
    for b in range(wl.batch):
        assert np.all(table[b, npg[b]:] == -1)


def test_identity_pages():
    wl = WORKLOADS["tiny_f32"]
    table, n = wl.page_table()
    assert table.tolist() == [[0, 1]] and n == 2
    assert wl.seq_lens().tolist() == [128]


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_shapes(name):
    wl = WORKLOADS[name]
    s = wl.shape
    assert s.row_width == s.kv_lora_rank + s.qk_rope_head_dim
    assert wl.cu_q()[-1] == wl.total_q()
