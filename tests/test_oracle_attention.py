"""Pins for the oracle's attention: scalar brute force, special cases with
known answers, a hand-computed example, the absorbed-vs-unabsorbed identity
in float64, and checks that plausible mistakes are detected."""
import math

import numpy as np
import pytest

from oracle import brute
from oracle.absorbed_fp64 import attend_sequence_absorbed
from oracle.mla_oracle import attend_sequence, decode, default_scale, latent_rows, rope_rotate


def _rand_case(rng, H=2, d_n=3, d_r=4, d_v=3, d_c=5, L=7, lq=2, d_model=6):
    return dict(
        x=rng.standard_normal((L, d_model)),
        w_dkv=rng.standard_normal((d_model, d_c + d_r)) / math.sqrt(d_model),
        w_uk=rng.standard_normal((d_c, H * d_n)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((d_c, H * d_v)) / math.sqrt(d_c),
        q=rng.standard_normal((lq, H, d_n + d_r)),
        H=H, d_n=d_n, d_r=d_r, d_v=d_v, d_c=d_c, L=L, lq=lq)


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / np.max(np.abs(np.asarray(b)))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_agreement(seed):
    rng = np.random.default_rng(seed)
    k = _rand_case(rng, H=3 if seed else 2, L=5 + 4 * seed, lq=1 + seed % 2)
    base, scale = 10000.0, default_scale(k["d_n"], k["d_r"])
    cache = latent_rows(k["x"], k["w_dkv"], np.arange(k["L"]), k["d_c"], base)
    for t in range(k["L"]):
        row = brute.brute_latent_row(list(k["x"][t]), k["w_dkv"].tolist(), t, k["d_c"], base)
        assert cache[t] == pytest.approx(row, rel=1e-12, abs=1e-13)
    out = attend_sequence(k["q"], cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], base, scale)
    ref = brute.brute_attend(k["q"].tolist(), cache.tolist(), k["w_uk"].tolist(), k["w_uv"].tolist(),
                             k["H"], k["d_n"], k["d_v"], base, scale)
    assert _rel(out, ref) <= 1e-12


def test_single_token_returns_its_value():
    rng = np.random.default_rng(5)
    k = _rand_case(rng, L=1, lq=1)
    cache = rng.standard_normal((1, k["d_c"] + k["d_r"]))
    out = attend_sequence(k["q"], cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, 0.3)
    for h in range(k["H"]):
        assert out[0, h] == pytest.approx(cache[0, :k["d_c"]] @ k["w_uv"][:, h * k["d_v"]:(h + 1) * k["d_v"]],
                                          rel=1e-14)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(6)
    k = _rand_case(rng, L=9, lq=2)
    q = np.zeros_like(k["q"])
    cache = rng.standard_normal((9, k["d_c"] + k["d_r"]))
    out = attend_sequence(q, cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, 0.5)
    for i, visible in enumerate((8, 9)):          # query 0 sees 8 rows, query 1 sees 9
        mean_c = cache[:visible, :k["d_c"]].mean(axis=0)
        for h in range(k["H"]):
            assert out[i, h] == pytest.approx(mean_c @ k["w_uv"][:, h * k["d_v"]:(h + 1) * k["d_v"]], rel=1e-13)


def test_identical_rows_give_that_rows_value():
    rng = np.random.default_rng(7)
    k = _rand_case(rng, L=6, lq=1)
    row = rng.standard_normal(k["d_c"] + k["d_r"])
    row[k["d_c"]:] = 0.0          # no position signal, so every score is equal
    cache = np.tile(row, (6, 1))
    out = attend_sequence(k["q"], cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, 0.4)
    for h in range(k["H"]):
        assert out[0, h] == pytest.approx(row[:k["d_c"]] @ k["w_uv"][:, h * k["d_v"]:(h + 1) * k["d_v"]], rel=1e-13)


def test_large_scale_selects_argmax():
    # d_c = d_nope = 4, W_uk = I: head 0's content score is c_t[0]; rope part zero.
    L, d_c, d_r = 9, 4, 2
    w_uk = np.eye(d_c)
    w_uv = np.arange(d_c * 3, dtype=np.float64).reshape(d_c, 3) / 7.0
    cache = np.zeros((L, d_c + d_r))
    cache[:, 0] = -((np.arange(L) - 3.0) ** 2)          # maximal at token 3
    cache[:, 1:d_c] = np.random.default_rng(8).standard_normal((L, d_c - 1))
    q = np.zeros((1, 1, d_c + d_r))
    q[0, 0, 0] = 1.0
    out = attend_sequence(q, cache, w_uk, w_uv, 1, d_c, 3, 1e4, 1e6)
    assert out[0, 0] == pytest.approx(cache[3, :d_c] @ w_uv, rel=1e-12)


def test_hand_computed_two_tokens():
    """One head, d_c = d_nope = d_rope = d_v = 2, W_uk = W_uv = I, scale 1/2.

    Content only: q_nope = (2 ln 3, 0) scores (ln 3, 0) -> weights (3/4, 1/4).
    Position only: cached rope keys are (1,0) rotated to their positions, the
    query (1,0) is rotated to position 1, so the rope scores are (cos 1, 1).
    """
    w = np.eye(2)
    cache = np.array([[1.0, 0.0, 1.0, 0.0],
                      [0.0, 1.0, math.cos(1.0), math.sin(1.0)]])
    q = np.array([[[2 * math.log(3.0), 0.0, 0.0, 0.0]]])
    out = attend_sequence(q, cache, w, w, 1, 2, 2, 10000.0, 0.5)
    assert out[0, 0] == pytest.approx([0.75, 0.25], abs=1e-15)
    q = np.array([[[0.0, 0.0, 1.0, 0.0]]])
    out = attend_sequence(q, cache, w, w, 1, 2, 2, 10000.0, 0.5)
    e0, e1 = math.exp(0.5 * math.cos(1.0)), math.exp(0.5)
    assert out[0, 0] == pytest.approx([e0 / (e0 + e1), e1 / (e0 + e1)], abs=1e-15)


@pytest.mark.parametrize("shape", ["toy", "dsv2"])
def test_absorbed_identity_fp64(shape):
    """Folding W_uk into the query and W_uv onto the output leaves the result
    unchanged up to float64 rounding (the pages print ~8e-15 on their toy)."""
    rng = np.random.default_rng(9)
    if shape == "toy":
        k = _rand_case(rng, H=4, d_n=8, d_r=8, d_v=8, d_c=16, L=64, lq=2, d_model=32)
        heads, bound = None, 1e-12
    else:
        k = _rand_case(rng, H=128, d_n=128, d_r=64, d_v=128, d_c=512, L=300, lq=2, d_model=64)
        heads, bound = [0, 37, 127], 1e-10
    scale = default_scale(k["d_n"], k["d_r"])
    cache = latent_rows(k["x"], k["w_dkv"], np.arange(k["L"]), k["d_c"], 1e4)
    a = attend_sequence(k["q"], cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, scale, heads)
    b = attend_sequence_absorbed(k["q"], cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, scale, heads)
    assert _rel(a, b) <= bound
    assert np.max(np.abs(a - b)) < 1e-11


def test_plausible_mistakes_are_caught():
    """Absorbing the wrong matrix (W_uv for W_uk: same shape, no error) or
    dropping the decoupled rope part changes the output far beyond any
    tolerance used for the GPU ("Now break it" on the paperfordummies page)."""
    rng = np.random.default_rng(10)
    k = _rand_case(rng, H=4, d_n=8, d_r=8, d_v=8, d_c=16, L=64, lq=1, d_model=32)
    scale = default_scale(k["d_n"], k["d_r"]) * 4.0
    cache = latent_rows(k["x"], k["w_dkv"], np.arange(k["L"]), k["d_c"], 1e4)
    ok = attend_sequence(k["q"], cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, scale)
    wrong_w = attend_sequence(k["q"], cache, k["w_uv"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, scale)
    q0 = k["q"].copy()
    q0[..., k["d_n"]:] = 0.0
    no_rope = attend_sequence(q0, cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, scale)
    unrotated = cache.copy()
    unrotated[:, k["d_c"]:] = (k["x"] @ k["w_dkv"])[:, k["d_c"]:]
    no_key_rot = attend_sequence(k["q"], unrotated, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, scale)
    for bad in (wrong_w, no_rope, no_key_rot):
        assert _rel(bad, ok) > 5e-2


def test_causal_consistency():
    """With two queries, query 0 equals a one-query decode of the sequence
    without its last row."""
    rng = np.random.default_rng(11)
    k = _rand_case(rng, H=3, L=12, lq=2)
    cache = rng.standard_normal((12, k["d_c"] + k["d_r"]))
    two = attend_sequence(k["q"], cache, k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, 0.4)
    one = attend_sequence(k["q"][:1], cache[:11], k["w_uk"], k["w_uv"], k["H"], k["d_n"], k["d_v"], 1e4, 0.4)
    assert two[0] == pytest.approx(one[0], rel=1e-13, abs=1e-15)


def test_query_rotation_uses_its_own_position():
    """Query i of a q_len block sits at position L - q_len + i.  With d_rope
    = 2 (one frequency, 1 rad per position), cached rope keys are the unit
    vector turned to their own positions and the query is (1, 0): the rope
    score of token t is cos(p - t), maximal exactly at t = p.  A huge scale
    then selects V[p] for each query."""
    L, lq, d_c = 7, 2, 2
    cache = np.zeros((L, d_c + 2))
    cache[:, 0] = np.arange(L)                     # V[t] = (t, 0) with W_uv = I
    cache[:, 2] = np.cos(np.arange(L))
    cache[:, 3] = np.sin(np.arange(L))
    q = np.zeros((lq, 1, 1 + 2))
    q[:, 0, 1] = 1.0                               # d_nope = 1 (zero), rope part (1, 0)
    w_uk = np.zeros((d_c, 1))
    out = attend_sequence(q, cache, w_uk, np.eye(d_c), 1, 1, d_c, 10000.0, 1e4)
    assert out[:, 0, 0] == pytest.approx([L - 2, L - 1], abs=1e-9)


def test_batch_decode_and_errors():
    rng = np.random.default_rng(13)
    k = _rand_case(rng, H=2, L=6, lq=1)
    caches = [rng.standard_normal((n, k["d_c"] + k["d_r"])) for n in (3, 6, 1)]
    q = rng.standard_normal((4, 2, k["d_n"] + k["d_r"]))
    out = decode(q, caches, k["w_uk"], k["w_uv"], [1, 2, 1], 2, k["d_n"], k["d_v"], 1e4, 0.5)
    assert out.shape == (4, 2, k["d_v"])
    ref = attend_sequence(q[1:3], caches[1], k["w_uk"], k["w_uv"], 2, k["d_n"], k["d_v"], 1e4, 0.5)
    assert np.array_equal(out[1:3], ref)
    with pytest.raises(ValueError):
        attend_sequence(q[:3], caches[0][:2], k["w_uk"], k["w_uv"], 2, k["d_n"], k["d_v"], 1e4, 0.5)


def test_default_scale_stated_values():
    """The scale the workloads state: 1/sqrt(192) for the DeepSeek-V2-shaped
    layer (d_nope 128 + d_rope 64) and 1/sqrt(24) for the tiny fp32 layer
    (16 + 8); one query-key width per head, content and position parts joined
    ("Multi-head Latent Attention: the KV cache, compressed", section "RoPE,
    and why the explanations stop here": the position key is a separate
    block of the same dot product)."""
    assert default_scale(128, 64) == 1.0 / math.sqrt(192.0)
    assert default_scale(16, 8) == 1.0 / math.sqrt(24.0)
    assert default_scale(128, 64) == pytest.approx(0.07216878364870322, rel=1e-15)


@pytest.mark.parametrize("a,r", [(2 * math.log(3.0), 0.0), (0.0, 2 * math.log(3.0)),
                                 (math.log(3.0), math.log(3.0))])
def test_default_scale_applies_to_the_summed_score(a, r):
    """One head, d_c = d_nope = d_rope = d_v = 2, W_uk = W_uv = I, query at
    position 1 with q = (0, a | r, 0).  Token 0 caches (1, 0 | 0, 0); token 1
    caches (0, 1 | cos 1, sin 1), the key (1, 0) already rotated to position
    1.  Content scores (0, a), position scores (0, r) (the query's (r, 0)
    rotated by 1 rad meets the same rotation), so with one scale
    1/sqrt(2 + 2) = 1/2 on their sum the weights are (1/4, 3/4) whenever
    a + r = 2 ln 3 -- whichever stream carries the score."""
    w = np.eye(2)
    cache = np.array([[1.0, 0.0, 0.0, 0.0],
                      [0.0, 1.0, math.cos(1.0), math.sin(1.0)]])
    q = np.array([[[0.0, a, r, 0.0]]])
    out = attend_sequence(q, cache, w, w, 1, 2, 2, 10000.0, default_scale(2, 2))
    assert out[0, 0] == pytest.approx([0.25, 0.75], abs=1e-14)
