"""Byte, FLOP and arithmetic-intensity counts for decode attention.

[HEA] "Hardware-Efficient Attention for Fast Decoding" ("What carries the
argument", "Core claim", Figure 3 caption): decoding is bound by loading the
KV cache; its arithmetic intensity is about 2 g_q / m_kv FLOPs per byte for
16-bit caches (g_q query heads per KV head, m_kv = 2 for separate K and V,
1 for a tied state); sharding over N tensor-parallel ranks duplicates the
cache ceil(N g_q / h_q) times.

Counting rules (algorithmic work): every cached element of every visible
token is read once; every visible (query row, key) pair costs one QK dot
product and one P.V accumulation, 2 FLOPs per multiply-add.  exp and RoPE
are not counted as FLOPs.
"""
from __future__ import annotations

import math

import numpy as np

from . import attention as _att


def kv_bytes_per_token(kind: str, groups: int, head_dim: int, d_rope: int,
                       elem_bytes: int) -> int:
    if kind == "gqa":
        return 2 * groups * head_dim * elem_bytes
    if kind == "gta":
        return (groups * head_dim + d_rope) * elem_bytes
    if kind == "latent":
        return (groups * head_dim + d_rope) * elem_bytes
    raise ValueError(kind)


def flops_per_token_row(kind: str, head_dim: int, d_rope: int) -> int:
    """FLOPs for one (query row, visible key) pair."""
    if kind in ("gqa", "gta"):
        return 2 * head_dim + 2 * head_dim
    if kind == "latent":
        return 2 * (head_dim + d_rope) + 2 * head_dim
    raise ValueError(kind)


def _visible_keys(seqlens, q_len: int, causal: bool) -> int:
    """Sum over sequences and query positions of the visible key counts."""
    total = 0
    for L in np.asarray(seqlens, dtype=np.int64).tolist():
        if causal and q_len > 1:
            total += sum(L - q_len + 1 + t for t in range(q_len))
        else:
            total += L * q_len
    return total


def kv_bytes(w, seqlens) -> int:
    per_tok = kv_bytes_per_token(w.kind, w.groups, w.head_dim, w.d_rope, w.elem_bytes)
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * per_tok


def flops(w, seqlens) -> int:
    return _visible_keys(seqlens, w.q_len, w.causal) * w.h_q * flops_per_token_row(
        w.kind, w.head_dim, w.d_rope)


def intensity(w, seqlens) -> float:
    return flops(w, seqlens) / kv_bytes(w, seqlens)


def intensity_model(g_q: float, m_kv: int) -> float:
    """[HEA]: about 2 g_q / m_kv FLOPs per byte (16-bit cache, q_len 1)."""
    return 2.0 * g_q / m_kv


def tp_duplication(n_shards: int, g_q: int, h_q: int) -> int:
    """[HEA] "Core claim": cache duplication factor ceil(N g_q / h_q)."""
    return int(math.ceil(n_shards * g_q / h_q))


def count_touched_rows(w, inp) -> int:
    """Run the oracle with gather tracing on; return the distinct bytes read.

    Counts every distinct (pool, page, slot, head) row the oracle gathered,
    times the row width, in the cache's storage element size.
    """
    _att._GATHER_TRACE = []
    try:
        _att.decode(w, inp)
        trace = _att._GATHER_TRACE
    finally:
        _att._GATHER_TRACE = None
    by_pool = {}
    for pid, flat, width in trace:
        by_pool.setdefault((pid, width), []).append(flat)
    total = 0
    for (_, width), parts in by_pool.items():
        total += np.unique(np.concatenate(parts)).size * width * w.elem_bytes
    return int(total)
