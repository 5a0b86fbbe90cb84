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


def test_project_query_brute_force():
    rng = np.random.default_rng(7)
    tq, H, dq, dm = 3, 4, 6, 5
    x = rng.standard_normal((tq, dm))
    w_q = rng.standard_normal((dm, H * dq))
    q = mla_oracle.project_query(x, w_q, H)
    assert q.shape == (tq, H, dq)
    for t in range(tq):
        for h in range(H):
            for i in range(dq):
                acc = sum(x[t, k] * w_q[k, h * dq + i] for k in range(dm))
                assert abs(q[t, h, i] - acc) < 1e-12


def test_query_fold_scores_match_materialised_keys():
    """The page's query-side fold W_abs_h = W_q_h W_uk_h^T (d_model x d_c per
    head), applied to x and dotted with a cached latent c, gives the content
    score q_nope . k_h of the textbook form, k_h = c W_uk_h built explicitly.
    Pins the orientation the query projection and the fold share: heads are
    column blocks h*(d_nope + d_rope) of W_q (content first) and h*d_nope of
    W_uk."""
    rng = np.random.default_rng(8)
    H, dn, dr, dc, dm, n = 3, 4, 2, 6, 5, 7
    x = rng.standard_normal((2, dm))
    w_q = rng.standard_normal((dm, H * (dn + dr)))
    w_uk = rng.standard_normal((dc, H * dn))
    lat = rng.standard_normal((n, dc))
    q = mla_oracle.project_query(x, w_q, H)
    for h in range(H):
        k_h = np.array([[sum(lat[t, j] * w_uk[j, h * dn + i] for j in range(dc)) for i in range(dn)]
                        for t in range(n)])
        textbook = q[:, h, :dn] @ k_h.T
        w_abs = w_q[:, h * (dn + dr):h * (dn + dr) + dn] @ w_uk[:, h * dn:(h + 1) * dn].T
        assert w_abs.shape == (dm, dc)
        assert np.allclose((x @ w_abs) @ lat.T, textbook, rtol=1e-12, atol=1e-12)
