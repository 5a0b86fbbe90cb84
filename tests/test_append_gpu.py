"""Cache append: placement and arithmetic are bit-exact.

With small-integer hidden states and weights in {-1, 0, 1}, every partial sum
of x W_dkv is an integer below 2**24, so the latent block is exactly
round_to_nearest_even(integer sum) in any accumulation order; the oracle's
own rounding gives the expected bits.  The rotated rope block goes through
sin/cos and is compared with a tolerance.  Every byte of the page pool that
no appended token maps to keeps its sentinel."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_synth import DSV2, TINY, workload
from oracle.mla_oracle import latent_rows
from oracle.rounding import bf16_value_to_bits, rne_bf16_value

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import SENTINEL_BYTE, i32, to_dev  # noqa: E402


@pytest.mark.parametrize("shape", ["bf16", "f32"])
def test_append_bit_exact_random_pages(shape):
    import mla_compressed_latent_amd as mla
    s = dataclasses.replace(DSV2, d_model=512) if shape == "bf16" else TINY
    dt = torch.bfloat16 if shape == "bf16" else torch.float32
    rng = np.random.default_rng(2024)
    B, ps = 5, s.page_size
    prefix = rng.integers(0, 200, size=B)
    n_new = rng.integers(1, 70, size=B)            # crosses page boundaries
    L = prefix + n_new
    npg = (L + ps - 1) // ps
    total_pages = int(npg.sum() + 7)
    perm = rng.permutation(total_pages)
    table = np.full((B, int(npg.max())), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    x = rng.integers(-3, 4, size=(int(n_new.sum()), s.d_model)).astype(np.float32)
    w = rng.integers(-1, 2, size=(s.d_model, s.row_width)).astype(np.float32)
    w_uk = np.zeros((s.d_c, s.H * s.d_nope), np.float32)
    w_uv = np.zeros((s.d_c, s.H * s.d_v), np.float32)
    cfg = mla.config_from_shape(s)
    layer = mla.mla_fold_weights(cfg, to_dev(w, dt), to_dev(w_uk, dt), to_dev(w_uv, dt))
    cache = torch.empty((total_pages, ps, s.row_width), dtype=dt, device="cuda")
    cache.view(torch.uint8).fill_(SENTINEL_BYTE)
    cu = np.concatenate([[0], np.cumsum(n_new)])
    print(f"[append] dtype={shape} tokens={int(n_new.sum())} pages={total_pages}", flush=True)
    mla.mla_append_latent(layer, to_dev(x, dt), i32(cu), i32(prefix), i32(table), cache)
    torch.cuda.synchronize()
    got = cache.cpu()
    got_bits = got.view(torch.int16).numpy().view(np.uint16) if shape == "bf16" else got.view(torch.int32).numpy()
    expect_written = np.zeros((total_pages, ps), bool)
    for b in range(B):
        pos = prefix[b] + np.arange(n_new[b])
        xb = x[cu[b]:cu[b + 1]]
        exact = xb.astype(np.int64) @ w.astype(np.int64)              # exact latent sums
        ref_rows = latent_rows(xb, w, pos, s.d_c, s.rope_base)       # float64 incl. rotation
        assert np.array_equal(ref_rows[:, :s.d_c], exact[:, :s.d_c])
        pages, slots = table[b, pos // ps], pos % ps
        expect_written[pages, slots] = True
        row_bits = got_bits[pages, slots]
        if shape == "bf16":
            want = bf16_value_to_bits(rne_bf16_value(exact[:, :s.d_c].astype(np.float64)))
            assert np.array_equal(row_bits[:, :s.d_c], want), f"latent bits differ in sequence {b}"
            rope = got[pages, slots, s.d_c:].float().numpy()
            tol = 2.0 ** -8 * np.abs(ref_rows[:, s.d_c:]).max()
        else:
            want = exact[:, :s.d_c].astype(np.float32).view(np.int32)
            assert np.array_equal(row_bits[:, :s.d_c], want), f"latent bits differ in sequence {b}"
            rope = got[pages, slots, s.d_c:].numpy()
            tol = 1e-5 * np.abs(ref_rows[:, s.d_c:]).max()
        assert np.abs(rope - ref_rows[:, s.d_c:]).max() <= tol
    # every other byte of the pool is untouched
    raw = got.view(torch.uint8).numpy().reshape(total_pages, ps, -1)
    assert np.all(raw[~expect_written] == SENTINEL_BYTE)


def test_append_empty_is_noop():
    import mla_compressed_latent_amd as mla
    s = TINY
    cfg = mla.config_from_shape(s)
    z = torch.zeros
    layer = mla.mla_fold_weights(cfg, z((s.d_model, s.row_width), device="cuda"),
                                 z((s.d_c, s.H * s.d_nope), device="cuda"), z((s.d_c, s.H * s.d_v), device="cuda"))
    cache = torch.full((2, s.page_size, s.row_width), 7.0, device="cuda")
    mla.mla_append_latent(layer, torch.zeros((0, s.d_model), device="cuda"), i32([0, 0]), i32([5]),
                          i32([[0, 1]]), cache)
    torch.cuda.synchronize()
    assert torch.all(cache == 7.0)
