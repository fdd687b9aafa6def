"""Byte model of one decode step: crossover length and ideal byte bounds.

TEST INFRASTRUCTURE (see the package docstring).

Source: [Cross/list] "Where Activation Sparsity and KV-Cache Sparsity Cross
in LLM Decoding", list view -- Abstract (a decode step rereads the
projection weights, a fixed amount, and the KV cache, which grows with the
context; the crossover is the context at which the two branches save the
same bytes; ideal speedups follow from model dimensions and keep ratios
alone), Table 1 (crossover over the seven projections and over the
feed-forward projections only), Table 2 (crossover per keep pair), Table 9
(shares of the step reads and bytes saved), Tables 11 and 17 (byte bounds),
Table 14 (batched crossover from the union of activated channels).

All quantities are element counts unless a byte width is given; with weights
and cache in one dtype, the width cancels from every ratio.

Notation: d model width, d_ff feed-forward width, q_dim = H_q * d_h,
kv_dim = H_kv * d_h, L layers, r_P projection keep, r_KV KV keep.
"""

from __future__ import annotations


def layer_weights(d: int, d_ff: int, q_dim: int, kv_dim: int) -> int:
    """Elements of the seven projections of one layer: Q and O (d x q_dim
    each), K and V (d x kv_dim each), gate, up and down (d x d_ff each)."""
    return 2 * d * q_dim + 2 * d * kv_dim + 3 * d * d_ff


def ff_weights(d: int, d_ff: int) -> int:
    """Elements of the three feed-forward projections of one layer."""
    return 3 * d * d_ff


def kv_per_token(kv_dim: int) -> int:
    """Cache elements one token adds to one layer: its key and its value."""
    return 2 * kv_dim


def crossover(weights: int, kv_token: int, r_p: float, r_kv: float) -> float:
    """Context length (tokens) at which the projection branch at keep r_P and
    the KV branch at keep r_KV remove the same number of bytes per layer:
    (1 - r_P) * weights = (1 - r_KV) * n * kv_token."""
    return (1.0 - r_p) * weights / ((1.0 - r_kv) * kv_token)


def batched_crossover(weights: int, kv_token: int, union: float, batch: int,
                      r_kv: float) -> float:
    """Table 14: with B sequences a sparse projection reads the union fraction
    u_B of its weights once, while every sequence reads its own cache, so the
    crossover becomes (1 - u_B) * weights / (B * (1 - r_KV) * kv_token)."""
    return (1.0 - union) * weights / (batch * (1.0 - r_kv) * kv_token)


def step_parts(n: int, *, layers: int, d: int, d_ff: int, q_dim: int,
               kv_dim: int, vocab: int, width: int = 2) -> dict:
    """Bytes one dense decode step reads, split as in Table 9: MLP (the three
    feed-forward projections of every layer), Attn (the four attention
    projections), KV (the cache of n tokens in every layer) and Other (the
    vocab x d output head, which no branch sparsifies)."""
    mlp = layers * ff_weights(d, d_ff) * width
    attn = layers * (layer_weights(d, d_ff, q_dim, kv_dim) - ff_weights(d, d_ff)) * width
    kv = n * layers * kv_per_token(kv_dim) * width
    other = vocab * d * width
    return {"mlp": mlp, "attn": attn, "kv": kv, "other": other}


def step_bytes(n: int, *, r_p: float = 1.0, r_kv: float = 1.0, **dims) -> float:
    """Bytes of one decode step when all seven projections keep r_P of their
    weights and the cache keeps r_KV of its tokens (Tables 11 and 17)."""
    p = step_parts(n, **dims)
    return r_p * (p["mlp"] + p["attn"]) + p["other"] + r_kv * p["kv"]


def byte_bound(n: int, *, r_p: float = 1.0, r_kv: float = 1.0, **dims) -> float:
    """Ideal step speedup over dense: dense bytes / sparse bytes."""
    return step_bytes(n, **dims) / step_bytes(n, r_p=r_p, r_kv=r_kv, **dims)
