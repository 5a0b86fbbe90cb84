"""Pins of the oracle's output projection: brute force on tiny inputs, and
the fold the page describes (value up-projection folded into the output
projection) reproduced with explicit per-head loops."""
import numpy as np

from oracle import mla_oracle


def test_project_brute_force():
    rng = np.random.default_rng(5)
    tq, H, dv, dm = 3, 4, 5, 7
    out = rng.standard_normal((tq, H, dv))
    w_o = rng.standard_normal((H * dv, dm))
    y = mla_oracle.project_output(out, w_o)
    for t in range(tq):
        for j in range(dm):
            acc = 0.0
            for h in range(H):
                for v in range(dv):
                    acc += out[t, h, v] * w_o[h * dv + v, j]
            assert abs(y[t, j] - acc) < 1e-12


def test_fold_into_output_projection():
    """sum_h o_lat_h (W_uv_h W_o_h) equals projecting o_lat_h W_uv_h: heads are
    the column blocks h*d_v .. of W_uv and the row blocks of W_o."""
    rng = np.random.default_rng(6)
    tq, H, dc, dv, dm = 2, 3, 8, 4, 5
    o_lat = rng.standard_normal((tq, H, dc))
    w_uv = rng.standard_normal((dc, H * dv))
    w_o = rng.standard_normal((H * dv, dm))
    out = np.stack([o_lat[:, h] @ w_uv[:, h * dv:(h + 1) * dv] for h in range(H)], axis=1)
    folded = sum(o_lat[:, h] @ (w_uv[:, h * dv:(h + 1) * dv] @ w_o[h * dv:(h + 1) * dv]) for h in range(H))
    assert np.allclose(mla_oracle.project_output(out, w_o), folded, rtol=1e-12, atol=1e-12)
