"""Throughput of one device's share of a causal Ring Attention forward pass.

(placeholder: accounting only; the timed path is added with the HIP library)
"""
from __future__ import annotations


def useful_pairs(layout: str, u: int, P: int, b: int, causal: bool) -> int:
    """Allowed (query, key) pairs of rank u over all P visiting blocks, per head.

    Non-causal: every pair, P*b^2.  Causal, contiguous shards: blocks r < u are
    fully allowed, block u is the lower triangle with its diagonal, blocks r > u
    are fully masked: u*b^2 + b(b+1)/2.  Causal, striped shards (token t on
    device t mod P): local key j of block r may be seen by local query i iff
    j <= i when r <= u and j < i when r > u, so blocks r <= u give b(b+1)/2 and
    blocks r > u give b(b-1)/2: P*b(b-1)/2 + (u+1)*b.
    """
    if not causal:
        return P * b * b
    if layout == "contiguous":
        return u * b * b + b * (b + 1) // 2
    if layout == "striped":
        return P * b * (b - 1) // 2 + (u + 1) * b
    raise ValueError(layout)


def useful_flops(pairs: int, d: int, heads: int) -> float:
    """Two contractions per allowed pair and head, QK^T and PV: 4*d FLOPs
    (the transformer-math page's 4*b^2*d per block pair, counted on allowed
    pairs only)."""
    return 4.0 * d * pairs * heads


def hop_bytes(b: int, d: int, heads_kv: int, elem_bytes: int) -> int:
    """Bytes of one key/value block on the wire: K and V, b tokens each."""
    return 2 * b * d * heads_kv * elem_bytes
