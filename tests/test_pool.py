"""Capacity planner and page pool (host code of the C library, no GPU).

The planner is pinned to the table the page prints ("Multi-head Latent
Attention: the KV cache, compressed", section "Where the saving actually
lands": DeepSeek-V2 shape, 60 layers, 80 GiB of cache -> 303 / 75 / 37 / 9
sequences at 4k / 16k / 32k / 128k context; section "The one formula" with the
decoupled rope key: 69,120 bytes per token) and to the oracle's closed forms
at other budgets.  The pool is checked against a plain Python model of the
same allocator over a seeded random sequence of operations."""
import json
import os

import numpy as np
import pytest

from oracle import closed_forms as cf

GIB = 1 << 30


@pytest.fixture(scope="module")
def mla():
    import mla_compressed_latent_amd as m
    return m


def _dsv2(mla, page_size=64):
    return mla.MlaConfig(d_model=5120, num_attention_heads=128, qk_nope_head_dim=128, qk_rope_head_dim=64,
                         v_head_dim=128, kv_lora_rank=512, page_size=page_size, rope_base=10000.0,
                         softmax_scale=0.0, dtype=1)


def test_capacity_table_of_the_page(mla, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page1_capacity.json")))
    cfg = _dsv2(mla)
    budget = g["budget_gib"] * GIB
    for r in g["rows"]:
        assert mla.mla_plan_max_sequences(cfg, 60, budget, r["context"]) == r["mla_seqs"]
    assert mla.mla_plan_max_sequences(cfg, 60, budget, 32768) == g["seqs_at_32k"]["mla"]
    plan = mla.mla_plan_cache(cfg, 60, budget)
    assert plan.bytes_per_token == 69120                   # 60 x 576 x 2
    assert plan.page_bytes == 64 * 1152
    assert plan.num_pages == budget // (60 * 64 * 1152)
    assert plan.total_bytes <= budget < plan.total_bytes + 60 * plan.page_bytes
    assert plan.layer_bytes == plan.num_pages * plan.page_bytes


@pytest.mark.parametrize("budget_gib", [1, 80, 192, 288])
@pytest.mark.parametrize("context", [1, 64, 1000, 4096, 32768, 131072])
@pytest.mark.parametrize("page_size", [64, 256])
def test_capacity_against_closed_forms(mla, budget_gib, context, page_size):
    """Whole pages per sequence: the closed form at the page-rounded context."""
    cfg = _dsv2(mla, page_size)
    rounded = -(-context // page_size) * page_size
    want = cf.seqs_in_budget(cf.latent_cache_size(60, 512, 64, rounded), budget_gib * GIB)
    assert mla.mla_plan_max_sequences(cfg, 60, budget_gib * GIB, context) == want


def test_plan_rejections(mla):
    cfg = _dsv2(mla)
    assert mla.mla_plan_max_sequences(cfg, 0, GIB, 10) == -1
    assert mla.mla_plan_max_sequences(cfg, 60, GIB, 0) == -1
    assert mla.mla_plan_max_sequences(_dsv2(mla, 48), 60, GIB, 10) == -1
    with pytest.raises(mla.MlaError) as e:
        mla.mla_plan_cache(cfg, 60, 60 * 64 * 1152 - 1)   # not one page of every layer
    assert e.value.status == 4
    assert mla.mla_plan_cache(cfg, 60, 60 * 64 * 1152).num_pages == 1


class _ModelPool:
    """The allocator as the header states it, in plain Python."""

    def __init__(self, n, ps, seqs, mpps):
        self.free = list(range(n - 1, -1, -1))   # top = end
        self.ps, self.mpps = ps, mpps
        self.pages = [[] for _ in range(seqs)]
        self.length = [0] * seqs

    def reserve(self, s, length):
        if length > self.mpps * self.ps:
            return 1
        need = -(-length // self.ps)
        more = need - len(self.pages[s])
        if more > len(self.free):
            return 4
        for _ in range(max(0, more)):
            self.pages[s].append(self.free.pop())
        self.length[s] = max(self.length[s], length)
        return 0

    def release(self, s):
        for p in reversed(self.pages[s]):
            self.free.append(p)
        self.pages[s] = []
        self.length[s] = 0


def test_pool_against_model(mla):
    N, PS, S, MPPS = 97, 64, 9, 20
    pool = mla.PagePool(N, PS, S, MPPS)
    model = _ModelPool(N, PS, S, MPPS)
    rng = np.random.default_rng(3)
    for step in range(3000):
        s = int(rng.integers(S))
        if rng.random() < 0.25:
            pool.release(s)
            model.release(s)
        else:
            length = int(rng.integers(0, MPPS * PS + 40))
            want = model.reserve(s, length)
            if want == 0:
                pool.reserve(s, length)
            else:
                with pytest.raises(mla.MlaError) as e:
                    pool.reserve(s, length)
                assert e.value.status == want
        assert pool.free_pages() == len(model.free)
        assert pool.length(s) == model.length[s]
        if step % 50 == 0:
            table = pool.page_table(list(range(S)))
            owned = [p for row in table for p in row if p >= 0]
            assert len(owned) == len(set(owned)) == N - pool.free_pages()   # no page twice
            for i in range(S):
                assert table[i][:len(model.pages[i])].tolist() == model.pages[i]
                assert (table[i][len(model.pages[i]):] == -1).all()


def test_pool_basics(mla):
    pool = mla.PagePool(10, 64, 3, 4)
    pool.reserve(0, 100)                 # 2 pages
    pool.reserve(1, 1)                   # 1 page
    pool.reserve(0, 129)                 # grows to 3 pages, keeps the first two
    t = pool.page_table([0, 1, 2])
    assert t.tolist() == [[0, 1, 3, -1], [2, -1, -1, -1], [-1, -1, -1, -1]]
    pool.reserve(0, 10)                  # never shrinks
    assert pool.length(0) == 129 and pool.page_table([0])[0].tolist() == [0, 1, 3, -1]
    pool.release(0)
    pool.reserve(2, 256)                 # reuses 0's pages in their old order
    assert pool.page_table([2])[0].tolist() == [0, 1, 3, 4]
    with pytest.raises(mla.MlaError) as e:
        pool.reserve(1, 5 * 64)          # beyond max_pages_per_seq
    assert e.value.status == 1
    with pytest.raises(mla.MlaError):
        pool.reserve(3, 1)               # no such sequence
    assert pool.free_pages() == 10 - 5
