"""Closed-form pins: the oracle's byte/parameter/MAC counts reproduce the
numbers printed on "Multi-head Latent Attention: the KV cache, compressed"
(stored in tests/golden with their sections)."""
import json
import os

import pytest

from oracle import closed_forms as cf

GIB = 1 << 30


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_cache_bytes_per_token_tables(golden_dir):
    g = _load(golden_dir, "page1_cache_bytes.json")
    for s in g["shapes"]:
        L, H, hd, dt = s["layers"], s["heads"], s["head_dim"], s["dtype_bytes"]
        mha = cf.kv_cache_size(L, H, hd, 1, dt)
        gqa = cf.kv_cache_size(L, 8, hd, 1, dt)
        mla = cf.latent_cache_size(L, s["d_c"], s["d_rope"], 1, dt)
        assert (mha, gqa, mla) == (s["mha"], s["gqa8"], s["mla"]), s["name"]
        assert round(mha / gqa, 1) == s["gqa8_smaller_x"]
        assert round(mha / mla, 1) == s["mla_smaller_x"]
        assert round(gqa / mla, 1) == s["mla_vs_gqa8_x"]


def test_decoupled_rope_cost(golden_dir):
    d = _load(golden_dir, "page1_cache_bytes.json")["decoupled_rope_cost"]
    lat = cf.latent_cache_size(d["layers"], d["d_c"], 0, 1, d["dtype_bytes"])
    full = cf.latent_cache_size(d["layers"], d["d_c"], d["d_rope"], 1, d["dtype_bytes"])
    assert (lat, full, full - lat) == (d["latent_only"], d["with_rope"], d["extra"])
    assert round(100.0 * (full - lat) / lat, 1) == d["extra_pct"]
    assert round(cf.kv_cache_size(60, 128, 128, 1) / full, 1) == d["vs_mha_x"]


def test_latent_elements_per_token(golden_dir):
    d = _load(golden_dir, "page1_cache_bytes.json")["latent_elements_per_token"]
    assert d["kv_lora_rank"] + d["qk_rope_head_dim"] == d["elements"]
    # elements of a token's full K and V across heads (bytes / dtype, one layer)
    assert cf.kv_cache_size(1, d["heads"], d["head_dim"], 1, 1) == d["mha_elements"]
    assert cf.latent_cache_size(1, d["kv_lora_rank"], d["qk_rope_head_dim"], 1, 1) == d["elements"]


def test_capacity_table(golden_dir):
    g = _load(golden_dir, "page1_capacity.json")
    budget = g["budget_gib"] * GIB
    for r in g["rows"]:
        n = r["context"]
        mha = cf.kv_cache_size(60, 128, 128, n)
        gqa = cf.kv_cache_size(60, 8, 128, n)
        mla = cf.latent_cache_size(60, 512, 64, n)
        assert round(mha / GIB, 2) == pytest.approx(r["mha_gib"])
        assert round(gqa / GIB, 2) == pytest.approx(r["gqa8_gib"])
        assert round(mla / GIB, 2) == pytest.approx(r["mla_gib"])
        assert cf.seqs_in_budget(mla, budget) == r["mla_seqs"]
    s = g["seqs_at_32k"]
    n = 32768
    assert cf.seqs_in_budget(cf.kv_cache_size(60, 128, 128, n), budget) == s["mha"]
    assert cf.seqs_in_budget(cf.kv_cache_size(60, 8, 128, n), budget) == s["gqa8"]
    assert cf.seqs_in_budget(cf.latent_cache_size(60, 512, 64, n), budget) == s["mla"]
    c = g["cache_at_32768_batch1_gib"]
    assert round(cf.kv_cache_size(60, 128, 128, n) / GIB, 2) == c["mha"]
    assert round(cf.kv_cache_size(60, 8, 128, n) / GIB, 2) == c["gqa8"]
    assert round(cf.latent_cache_size(60, 512, 64, n) / GIB, 2) == c["mla"]


def test_parameter_counts_fix_weight_layout(golden_dir):
    """229,441,536 holds only if W_dkv is d_model x (d_c + d_rope) (it makes
    the rope key) and W_q is d_model x H*(d_nope + d_rope) (one rope query
    per head) -- the two layout readings the decode library relies on."""
    p = _load(golden_dir, "page1_params_and_macs.json")["params"]
    dm, H, hd = p["d_model"], p["heads"], p["head_dim"]
    assert cf.params_mha(dm, H, hd) == p["mha"]
    assert cf.params_gqa(dm, H, hd, p["kv_heads_gqa"]) == p["gqa8"]
    mla = cf.params_mla(dm, H, hd, p["d_rope"], hd, p["d_c"])
    assert mla == p["mla"]
    assert round(mla / p["mha"], 2) == p["mla_over_mha_x"]
    assert round(mla / p["gqa8"], 2) == p["mla_over_gqa8_x"]
    # the alternative readings miss the printed number
    no_rope_in_wdkv = mla - dm * p["d_rope"]
    shared_rope_query = mla - dm * (H - 1) * p["d_rope"]
    assert no_rope_in_wdkv != p["mla"] and shared_rope_query != p["mla"]


def test_mac_counts(golden_dir):
    m = _load(golden_dir, "page1_params_and_macs.json")["macs"]
    for r in m["rows"]:
        e = cf.macs_expanded_per_head(m["d_model"], m["head_dim"], m["d_c"], r["n"])
        a = cf.macs_absorbed_per_head(m["d_model"], m["d_c"], r["n"])
        assert (e, a) == (r["expanded"], r["absorbed"])
        assert round(e / a, 2) == r["saving_x"]


def test_rebuild_tax(golden_dir):
    t = _load(golden_dir, "page1_params_and_macs.json")["rebuild_tax"]
    assert cf.macs_rebuild_fold(t["heads"], t["d_model"], t["head_dim"], t["d_c"], t["steps"]) \
        == t["extra_macs"]


def test_reduction_claims(golden_dir):
    """The quoted 93.3% is not derivable from either shape on the pages; the
    closed forms give 98.24% (DeepSeek-V2 shape vs 128-head MHA) and 92.97%
    (Llama-2-7B shape).  Only its consistency with the ~6.7% remainder in the
    comparison table is checked."""
    r = _load(golden_dir, "page1_params_and_macs.json")["reduction_claim"]
    assert round(100.0 - r["reduction_pct"], 1) == r["remaining_pct"]
    ds = 1.0 - cf.latent_cache_size(60, 512, 64, 1) / cf.kv_cache_size(60, 128, 128, 1)
    ll = 1.0 - cf.latent_cache_size(32, 512, 64, 1) / cf.kv_cache_size(32, 32, 128, 1)
    assert round(100 * ds, 2) == 98.24
    assert round(100 * ll, 2) == 92.97
