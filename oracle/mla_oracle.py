"""CPU oracle for one MLA decode layer: plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
does, and this module never imports the GPU library.

What it computes is the textbook, *unabsorbed* reading of Multi-head Latent
Attention: every head's keys and values are materialised from the cached
latent and ordinary softmax attention is run over them.  The GPU path computes
the same result by re-association (the absorption), so the two agree up to
rounding.

Sources (web pages, cited by title and section):

* "Multi-head Latent Attention: the KV cache, compressed" (paperfordummies.in)
  - section "The one formula": the cached row per token and layer is the
    d_c-wide latent plus the d_rope-wide decoupled position key.
  - section "The code", functions ``latent`` and ``attention_via_latent``:
    the latent is ``x @ W_dkv``; keys and values are ``C @ W_uk`` and
    ``C @ W_uv`` per head; attention is ``softmax(Q K^T / sqrt(d)) V``.
  - section "The code", function ``decoupled_score`` and section "RoPE, and
    why the explanations stop here": the score is the content part plus a
    separately rotated position part whose key is cached already rotated,
    one copy shared by all heads.
* "Multi-head Latent Attention and KV Cache Compression" (jongkwan.dev),
  section "The absorption trick and decoupled RoPE": two streams (NoPE and
  RoPE); a head's score adds the content dot product and the position dot
  product.
* "Multi-Head Latent Attention (MLA)" (superteams.ai glossary), section "The
  Mechanism": cached element count per token is kv_lora_rank + rope dim.

Readings taken where the pages are silent:

* Rotary embedding pairs interleaved elements (2i, 2i+1) and rotates each
  pair counter-clockwise by ``p * base**(-2i/d_rope)``; positions are
  0-based token indices.
* The weight producing the cached row, W_dkv, has d_c + d_rope output
  columns; the last d_rope of them form the position key, which is rotated
  at its own token's position before caching.  Each head's query has d_nope
  content elements followed by d_rope position elements.
* Scale: ``1/sqrt(d_nope + d_rope)`` applied to the summed score.
* Sequence b holds L_b cached rows after the new tokens are appended; its
  q_len_b queries sit at positions L_b - q_len_b + i and each attends to
  every position not after its own.
* Where queries are asked for from the layer's input, they are
  ``x . W_q`` with W_q of shape [d_model][H * (d_nope + d_rope)], head h
  owning the columns h * (d_nope + d_rope) .., content part first
  (``project_query``).
* Output per query and head is ``sum_t w_t V_h[t]`` (no output projection);
  where a layer output is asked for, it is the concatenated heads times an
  output projection W_o of shape [H * d_v][d_model] (``project_output``).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rope_inv_freq",
    "rope_rotate",
    "latent_rows",
    "softmax",
    "attend_sequence",
    "decode",
    "default_scale",
    "project_output",
    "project_query",
]


def default_scale(d_nope: int, d_rope: int) -> float:
    """Softmax scale 1/sqrt(query-key width); the key of one head is its
    d_nope content part joined with the d_rope position part."""
    return 1.0 / np.sqrt(float(d_nope + d_rope))


def rope_inv_freq(d_rope: int, base: float) -> np.ndarray:
    """Angular frequency of rotary pair i: base ** (-2 i / d_rope)."""
    if d_rope % 2:
        raise ValueError("rotary width must be even")
    i = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / float(d_rope))


def rope_rotate(v: np.ndarray, positions, base: float) -> np.ndarray:
    """Rotate the last axis of ``v`` (width d_rope) at the given positions.

    ``positions`` broadcasts against ``v.shape[:-1]``.  Pair (2i, 2i+1) is
    rotated by angle a = p * theta_i:
        out[2i]   = v[2i] cos a - v[2i+1] sin a
        out[2i+1] = v[2i] sin a + v[2i+1] cos a
    """
    v = np.asarray(v, dtype=np.float64)
    d_rope = v.shape[-1]
    theta = rope_inv_freq(d_rope, base)
    p = np.asarray(positions, dtype=np.float64)[..., None]
    ang = p * theta                                   # [..., d_rope/2]
    cos, sin = np.cos(ang), np.sin(ang)
    even, odd = v[..., 0::2], v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape, ang.shape[:-1] + (d_rope,)), dtype=np.float64)
    out[..., 0::2] = even * cos - odd * sin
    out[..., 1::2] = even * sin + odd * cos
    return out


def latent_rows(x: np.ndarray, w_dkv: np.ndarray, positions, d_c: int, base: float) -> np.ndarray:
    """The row cached for each token: [c | k_rope], float64.

    u = x @ W_dkv; c = u[:, :d_c]; k_rope = rotate(u[:, d_c:], position).
    """
    x = np.asarray(x, dtype=np.float64)
    u = x @ np.asarray(w_dkv, dtype=np.float64)
    out = u.copy()
    out[:, d_c:] = rope_rotate(u[:, d_c:], np.asarray(positions), base)
    return out


def softmax(s: np.ndarray) -> np.ndarray:
    """Textbook softmax over the last axis: subtract the max, exp, normalise."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attend_sequence(q: np.ndarray, cache: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                    n_heads: int, d_nope: int, d_v: int, base: float, scale: float,
                    heads=None) -> np.ndarray:
    """Unabsorbed MLA attention for one sequence.

    q      [Lq][H][d_nope + d_rope]  queries before rotation
    cache  [L][d_c + d_rope]         cached rows, position t at row t
    w_uk   [d_c][H * d_nope]         head h uses columns h*d_nope ... +d_nope
    w_uv   [d_c][H * d_v]            head h uses columns h*d_v ... +d_v
    Returns [Lq][len(heads)][d_v] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    cache = np.asarray(cache, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    lq = q.shape[0]
    L = cache.shape[0]
    d_c = w_uk.shape[0]
    if lq < 1 or L < lq:
        raise ValueError("need 1 <= q_len <= cached length")
    heads = list(range(n_heads)) if heads is None else list(heads)
    c, k_rope = cache[:, :d_c], cache[:, d_c:]
    out = np.zeros((lq, len(heads), d_v), dtype=np.float64)
    for j, h in enumerate(heads):
        k_content = c @ w_uk[:, h * d_nope:(h + 1) * d_nope]     # [L][d_nope]  expanded keys
        v = c @ w_uv[:, h * d_v:(h + 1) * d_v]                   # [L][d_v]     expanded values
        keys = np.concatenate([k_content, k_rope], axis=1)       # [L][d_nope + d_rope]
        for i in range(lq):
            pos = L - lq + i
            qh = q[i, h]
            query = np.concatenate([qh[:d_nope], rope_rotate(qh[d_nope:], pos, base)])
            s = scale * (keys[: pos + 1] @ query)
            w = softmax(s)
            out[i, j] = w @ v[: pos + 1]
    return out


def decode(q: np.ndarray, caches, w_uk, w_uv, q_lens, n_heads: int, d_nope: int, d_v: int,
           base: float, scale: float) -> np.ndarray:
    """Whole batch: q [Tq][H][d_nope+d_rope] with sequences in order,
    ``caches[b]`` the rows of sequence b.  Returns [Tq][H][d_v]."""
    outs = []
    off = 0
    for b, cache in enumerate(caches):
        lq = int(q_lens[b])
        outs.append(attend_sequence(q[off:off + lq], cache, w_uk, w_uv, n_heads, d_nope, d_v,
                                    base, scale))
        off += lq
    return np.concatenate(outs, axis=0)


def project_output(out: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """Layer output y[t] = concat_h out[t][h] . W_o for out [Tq][H][d_v] and
    W_o [H * d_v][d_model] ("Multi-head Latent Attention and KV Cache
    Compression", section "The absorption trick and decoupled RoPE": the value
    up-projection can be folded into this output projection)."""
    out = np.asarray(out, dtype=np.float64)
    tq, h, dv = out.shape
    return out.reshape(tq, h * dv) @ np.asarray(w_o, dtype=np.float64)


def project_query(x: np.ndarray, w_q: np.ndarray, n_heads: int) -> np.ndarray:
    """Queries from the layer's input: q[t] = x[t] . W_q, split per head, for
    x [Tq][d_model] and W_q [d_model][H * (d_nope + d_rope)] ("Multi-head
    Latent Attention: the KV cache, compressed", section "Store the archive,
    not the files": the query is a plain linear map of the token's hidden
    state, into which the key up-projection can be folded once at load).
    Returns [Tq][H][d_nope + d_rope]."""
    x = np.asarray(x, dtype=np.float64)
    w_q = np.asarray(w_q, dtype=np.float64)
    tq = x.shape[0]
    return (x @ w_q).reshape(tq, n_heads, w_q.shape[1] // n_heads)
