"""Scalar-loop MLA decode for tiny inputs (pure Python floats, no BLAS).

TEST INFRASTRUCTURE ONLY (see ``oracle/mla_oracle.py``).

Written from the same definition as the oracle but with explicit loops over
every index, so that a vectorisation slip in the oracle (a transposed
operand, a wrong column block, an off-by-one in the visible range) shows up
as a disagreement.  Use only for H <= 4, L <= 32.
"""
from __future__ import annotations

import math


def rot_pair(x0, x1, angle):
    c, s = math.cos(angle), math.sin(angle)
    return x0 * c - x1 * s, x0 * s + x1 * c


def rotate(vec, pos, base):
    d = len(vec)
    out = [0.0] * d
    for i in range(d // 2):
        theta = base ** (-(2.0 * i) / d)
        out[2 * i], out[2 * i + 1] = rot_pair(vec[2 * i], vec[2 * i + 1], pos * theta)
    return out


def brute_latent_row(x_row, w_dkv, pos, d_c, base):
    width = len(w_dkv[0])
    u = [sum(x_row[k] * w_dkv[k][j] for k in range(len(x_row))) for j in range(width)]
    return u[:d_c] + rotate(u[d_c:], pos, base)


def brute_attend(q, cache, w_uk, w_uv, n_heads, d_nope, d_v, base, scale):
    """q: nested lists [Lq][H][d_nope + d_rope]; cache: [L][d_c + d_rope];
    w_uk: [d_c][H*d_nope]; w_uv: [d_c][H*d_v].  Returns [Lq][H][d_v]."""
    lq, L = len(q), len(cache)
    d_c = len(w_uk)
    out = []
    for i in range(lq):
        pos = L - lq + i
        row_out = []
        for h in range(n_heads):
            qh = q[i][h]
            q_rot = rotate(qh[d_nope:], pos, base)
            scores = []
            for t in range(pos + 1):
                s = 0.0
                for a in range(d_nope):
                    k_ta = 0.0
                    for j in range(d_c):
                        k_ta += cache[t][j] * w_uk[j][h * d_nope + a]
                    s += qh[a] * k_ta
                for r in range(len(q_rot)):
                    s += q_rot[r] * cache[t][d_c + r]
                scores.append(scale * s)
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = sum(e)
            o = []
            for v in range(d_v):
                acc = 0.0
                for t in range(pos + 1):
                    val = 0.0
                    for j in range(d_c):
                        val += cache[t][j] * w_uv[j][h * d_v + v]
                    acc += (e[t] / z) * val
                o.append(acc)
            row_out.append(o)
        out.append(row_out)
    return out
