"""The absorbed (re-associated) MLA decode, float64, for pinning the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/mla_oracle.py``).

This is the second algebraic route to the same numbers.  Instead of
expanding keys and values per head, the query is folded into the latent
space and the attention weights sum latents, which are then projected out:

    q_lat   = W_uk_h @ q_nope                (d_c wide)
    s_t     = scale * (q_lat . c_t + rot(q_rope, p) . k_rope_t)
    o_lat   = sum_t softmax(s)_t c_t
    out     = o_lat @ W_uv_h

Sources: "Multi-head Latent Attention: the KV cache, compressed", sections
"Store the archive, not the files" and "Absorption: the part that makes it
free" (fold W_uk into the query side once; keys never built); "Multi-head
Latent Attention and KV Cache Compression", section "The absorption trick
and decoupled RoPE" (q^T W_u c = (W_u^T q)^T c; the value-side up-projection
folds into the output side the same way).

Agreement with the unabsorbed oracle to float64 rounding is the identity the
pages demonstrate (differences of order 1e-14 on their toy sizes).
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import rope_rotate, softmax


def attend_sequence_absorbed(q, cache, w_uk, w_uv, n_heads, d_nope, d_v, base, scale, heads=None):
    q = np.asarray(q, dtype=np.float64)
    cache = np.asarray(cache, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    lq, L = q.shape[0], cache.shape[0]
    d_c = w_uk.shape[0]
    heads = list(range(n_heads)) if heads is None else list(heads)
    c, k_rope = cache[:, :d_c], cache[:, d_c:]
    out = np.zeros((lq, len(heads), d_v), dtype=np.float64)
    for j, h in enumerate(heads):
        wuk_h = w_uk[:, h * d_nope:(h + 1) * d_nope]      # [d_c][d_nope]
        wuv_h = w_uv[:, h * d_v:(h + 1) * d_v]            # [d_c][d_v]
        for i in range(lq):
            pos = L - lq + i
            q_lat = wuk_h @ q[i, h, :d_nope]                # folded query, [d_c]
            q_rot = rope_rotate(q[i, h, d_nope:], pos, base)
            content = c[: pos + 1] @ q_lat
            position = k_rope[: pos + 1] @ q_rot
            w = softmax(scale * (content + position))
            o_lat = w @ c[: pos + 1]                        # [d_c]
            out[i, j] = o_lat @ wuv_h
    return out
