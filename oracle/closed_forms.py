"""Closed-form byte, parameter and operation counts for MLA.

TEST INFRASTRUCTURE ONLY (see ``oracle/mla_oracle.py``).

Sources: "Multi-head Latent Attention: the KV cache, compressed", sections
"The one formula" (a cache's size is the number of values it keeps per
token and layer times layers, tokens and element size: a key and a value
per kv head for ordinary attention, the latent plus the shared position key
for MLA), "The table that is
the whole argument", "Where the saving actually lands" (sequences that fit a
cache budget), "What it costs, said plainly" (parameters per attention
layer), "Absorption: the part that makes it free" (multiply-accumulates per
head per decode step) and "Now break it" (cost of rebuilding the folded
matrix on every step).
"""
from __future__ import annotations

GIB = 1 << 30


def cache_footprint(per_token_layer_elems, n_layers, n_tokens, elem_size):
    """Bytes of a cache that keeps ``per_token_layer_elems`` numbers of
    ``elem_size`` bytes for every token in every layer."""
    return per_token_layer_elems * n_layers * n_tokens * elem_size


def kv_cache_size(n_layers, n_kv_heads, width, n_tokens, elem_size=2):
    """Classic attention cache: a key vector and a value vector, each
    ``width`` wide, for every kv head."""
    return cache_footprint(2 * n_kv_heads * width, n_layers, n_tokens, elem_size)


def latent_cache_size(n_layers, latent_rank, rope_width, n_tokens, elem_size=2):
    """Latent cache: one latent of ``latent_rank`` numbers plus one rotated
    position key of ``rope_width`` numbers per token, whatever the head
    count."""
    return cache_footprint(latent_rank + rope_width, n_layers, n_tokens, elem_size)


def seqs_in_budget(bytes_per_seq, budget_bytes):
    """Whole sequences that fit in a cache budget."""
    return budget_bytes // bytes_per_seq


def params_mha(d_model, heads, head_dim):
    """W_q, W_k, W_v (d_model x H*hd each) and W_o (H*hd x d_model)."""
    return 4 * d_model * heads * head_dim


def params_gqa(d_model, heads, head_dim, kv_heads):
    """W_q and W_o full width; W_k and W_v only kv_heads wide."""
    return 2 * d_model * heads * head_dim + 2 * d_model * kv_heads * head_dim


def params_mla(d_model, heads, d_nope, d_rope, d_v, d_c):
    """W_q (d_model x H*(d_nope+d_rope)), W_dkv (d_model x (d_c+d_rope)),
    W_uk (d_c x H*d_nope), W_uv (d_c x H*d_v), W_o (H*d_v x d_model)."""
    w_q = d_model * heads * (d_nope + d_rope)
    w_dkv = d_model * (d_c + d_rope)
    w_uk = d_c * heads * d_nope
    w_uv = d_c * heads * d_v
    w_o = heads * d_v * d_model
    return w_q + w_dkv + w_uk + w_uv + w_o


def macs_expanded_per_head(d_model, head_dim, d_c, n_cached):
    """Per head per decode step without the fold: project the query
    (d_model x hd), rebuild every cached key (n x d_c x hd), score (n x hd)."""
    return d_model * head_dim + n_cached * d_c * head_dim + n_cached * head_dim


def macs_absorbed_per_head(d_model, d_c, n_cached):
    """Per head per decode step with the fold: project the query straight
    into latent space (d_model x d_c), score against the latents (n x d_c)."""
    return d_model * d_c + n_cached * d_c


def macs_rebuild_fold(heads, d_model, head_dim, d_c, steps):
    """Extra work of recomputing W_q_h @ W_uk_h^T on every step."""
    return heads * (d_model * head_dim * d_c) * steps
