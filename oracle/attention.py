"""Decode attention over a paged KV cache, written out in float64.

Sources (web pages; cited by title and section):
  [HEA]  "Hardware-Efficient Attention for Fast Decoding" (Zadouri, Strauss,
         Dao; Pith review page of arXiv 2505.21487): GTA (tied KV state, partial
         RoPE key from a separate single-head projection broadcast to the group,
         Figure 2 caption and "Assumptions & free parameters"), GLA / MLA
         (latent heads, "What carries the argument", "Core claim"), speculative
         verification with query length > 1 ("If this is right"), paged KV
         ("If this is right": page size 1 vs 64).
  [GIST] "The Gist Talk" podcast page: GQA divides the query heads into groups
         that each share one key head and one value head; MQA is the one-group
         case; the Transformer summary names scaled dot-product attention.
  [EI]   "Efficient Inference" tag page, Hydragen entry: attention over a
         split key set is recombined through the softmax denominators.

Readings where the pages are silent (each also listed in the design notes):
  * query head h belongs to group floor(h / g), g = h_q / groups;
  * key i of a sequence sits at position i; query t of a q_len-T call sits at
    position L - T + t, and with causal masking it sees keys i <= L - T + t;
  * RoPE pairs element k with element k + d_r/2 ("rotate half") and uses the
    frequency theta ** (-2k / d_r);
  * GTA: the key is [tied[0 : d - d_r] || RoPE(rope_key, i)], the value is the
    full tied state; the query's last d_r entries are rotated at its position;
  * latent (MLA: one latent head; GLA: h_c heads): scores use
    [latent_j || rope_key] against the (already absorbed and rotated) query,
    and the output is the probability-weighted latent_j (d_c wide);
  * the softmax scale is an explicit argument and LSE is natural-log and
    includes the scale;  an empty sequence gives O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf

# When not None, every gather appends (pool id, int64 flat row ids, row width
# in elements) here, so the rows the oracle actually reads can be counted.
_GATHER_TRACE = None


# ---------------------------------------------------------------- paging
def logical_positions(L: int) -> np.ndarray:
    return np.arange(int(L), dtype=np.int64)


def gather_rows(pool: np.ndarray, table_row: np.ndarray, L: int, page_size: int,
                head: int) -> np.ndarray:
    """Rows [L, width] of one head of one sequence, in float64.

    Logical token i lives in physical page table_row[i // page_size], slot
    i % page_size (the paged-KV indirection of [HEA] "If this is right").
    All index arithmetic is int64.
    """
    i = logical_positions(L)
    pages = np.asarray(table_row, dtype=np.int64)[i // page_size]
    if L and (pages < 0).any():
        raise IndexError("page table entry -1 inside the sequence")
    if L and (pages >= pool.shape[0]).any():
        raise IndexError("page id beyond the pool")
    slots = i % page_size
    if _GATHER_TRACE is not None:
        flat = (pages * pool.shape[1] + slots) * pool.shape[2] + head
        _GATHER_TRACE.append((id(pool), flat, pool.shape[3]))
    return pool[pages, slots, head, :].astype(np.float64)


# ---------------------------------------------------------------- RoPE
def rope_rotate_half(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding of the last axis (width d_r, even), rotate-half pairing.

    For k < d_r/2, the pair (x_k, x_{k+d_r/2}) is rotated by the angle
    pos * theta**(-2k/d_r).  ``pos`` broadcasts against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    d_r = x.shape[-1]
    if d_r % 2:
        raise ValueError("RoPE width must be even")
    half = d_r // 2
    k = np.arange(half, dtype=np.float64)
    freq = float(theta) ** (-2.0 * k / d_r)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# ---------------------------------------------------------------- core
def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
           q_pos=None, return_probs: bool = False):
    """Scaled dot-product softmax attention of R query rows over L keys.

    q [R, D], k [L, D], v [L, Dv] (float64).  With ``q_pos`` given, row r only
    sees keys i <= q_pos[r].  Returns (o [R, Dv], lse [R]) (and p [R, L]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, L = q.shape[0], k.shape[0]
    if L == 0:
        o = np.zeros((R, v.shape[1]))
        lse = np.full(R, NEG_INF)
        return (o, lse, np.zeros((R, 0))) if return_probs else (o, lse)
    s = scale * (q @ k.T)
    if q_pos is not None:
        hidden = logical_positions(L)[None, :] > np.asarray(q_pos, dtype=np.int64)[:, None]
        s = np.where(hidden, NEG_INF, s)
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=l[:, None] > 0)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m_safe + np.log(l), NEG_INF)
    return (o, lse, p) if return_probs else (o, lse)


def attend_partial(q, k, v, scale, key_idx, q_pos=None):
    """Attention restricted to the key subset ``key_idx``.

    Returns (o_s, lse_s): the normalised output over that subset and its
    log-sum-exp, the per-chunk state a split-KV pass produces.
    """
    key_idx = np.asarray(key_idx, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    s = scale * (q @ np.asarray(k, dtype=np.float64)[key_idx].T)
    if q_pos is not None:
        s = np.where(key_idx[None, :] > np.asarray(q_pos)[:, None], NEG_INF, s)
    if key_idx.size == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], NEG_INF)
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    o = np.divide(e @ np.asarray(v, dtype=np.float64)[key_idx], l[:, None],
                  out=np.zeros((q.shape[0], v.shape[1])), where=l[:, None] > 0)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m_safe + np.log(l), NEG_INF)
    return o, lse


def merge_partials(os_, lses):
    """Recombine per-chunk (o_s, lse_s) through the softmax denominators ([EI]).

    With M = max_s lse_s and w_s = exp(lse_s - M):
        o = sum_s w_s o_s / sum_s w_s,   lse = M + ln sum_s w_s.
    os_ [S, R, Dv], lses [S, R].
    """
    os_ = np.asarray(os_, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lses - M_safe[None, :])
    W = w.sum(axis=0)
    o = np.divide((w[:, :, None] * os_).sum(axis=0), W[:, None],
                  out=np.zeros(os_.shape[1:]), where=W[:, None] > 0)
    with np.errstate(divide="ignore"):
        lse = np.where(W > 0, M_safe + np.log(W), NEG_INF)
    return o, lse


# ---------------------------------------------------------------- kinds
def _rows_of_group(q_b: np.ndarray, j: int, g: int) -> np.ndarray:
    """Query rows of group j for one sequence, ordered (t, head-in-group)."""
    T = q_b.shape[0]
    return q_b[:, j * g:(j + 1) * g, :].reshape(T * g, q_b.shape[-1]).astype(np.float64)


def _row_positions(L: int, T: int, g: int) -> np.ndarray:
    t = np.repeat(np.arange(T, dtype=np.int64), g)
    return L - T + t


def _check_common(q, page_table, seqlens, groups, causal):
    B, T, H, _ = q.shape
    if H % groups:
        raise ValueError("h_q must be a multiple of the number of groups")
    if page_table.shape[0] != B or len(seqlens) != B:
        raise ValueError("batch mismatch")
    if causal and T > 1 and (np.asarray(seqlens) < T).any():
        raise ValueError("causal decode needs seqlen >= q_len")
    return B, T, H, H // groups


def decode_gqa(q, k_pool, v_pool, page_table, seqlens, page_size, scale, causal=False):
    """GQA decode ([GIST] GQA summary; MQA when there is one KV head).

    q [B, T, H, d]; k_pool, v_pool [pages, P, h_kv, d].
    Returns out [B, T, H, d] and lse [B, T, H] in float64.
    """
    q = np.asarray(q)
    G = k_pool.shape[2]
    B, T, H, g = _check_common(q, page_table, seqlens, G, causal)
    out = np.zeros((B, T, H, v_pool.shape[-1]))
    lse = np.zeros((B, T, H))
    for b in range(B):
        L = int(seqlens[b])
        pos = _row_positions(L, T, g) if (causal and T > 1) else None
        for j in range(G):
            k = gather_rows(k_pool, page_table[b], L, page_size, j)
            v = gather_rows(v_pool, page_table[b], L, page_size, j)
            o, s = attend(_rows_of_group(q[b], j, g), k, v, scale, pos)
            out[b, :, j * g:(j + 1) * g] = o.reshape(T, g, -1)
            lse[b, :, j * g:(j + 1) * g] = s.reshape(T, g)
    return out, lse


def gta_key_value(tied_rows: np.ndarray, rope_rows: np.ndarray, d_rope: int, theta: float):
    """Assemble GTA key and value rows of one KV head ([HEA] Figure 2 caption).

    The full tied state is the value; the key is the un-rotated leading
    d - d_r entries of the tied state followed by the shared single-head
    RoPE key rotated at each token's position.
    """
    L, d = tied_rows.shape
    v = tied_rows
    if d_rope == 0:
        return tied_rows, v
    k_rope = rope_rotate_half(rope_rows, logical_positions(L), theta) if theta > 0 else rope_rows
    k = np.concatenate([tied_rows[:, :d - d_rope], k_rope], axis=1)
    return k, v


def decode_gta(q, tied_pool, rope_pool, page_table, seqlens, page_size, d_rope, theta,
               scale, causal=False):
    """GTA decode ([HEA] Figure 2 caption, "Assumptions & free parameters").

    q [B, T, H, d] with its last d_rope entries un-rotated (rotated here at
    the query position when theta > 0); tied_pool [pages, P, h_kv, d];
    rope_pool [pages, P, 1, d_rope] (one RoPE head broadcast to all groups).
    """
    q = np.asarray(q)
    G, d = tied_pool.shape[2], tied_pool.shape[3]
    B, T, H, g = _check_common(q, page_table, seqlens, G, causal)
    out = np.zeros((B, T, H, d))
    lse = np.zeros((B, T, H))
    for b in range(B):
        L = int(seqlens[b])
        qpos_all = _row_positions(L, T, g)
        pos = qpos_all if (causal and T > 1) else None
        r = gather_rows(rope_pool, page_table[b], L, page_size, 0) if d_rope else None
        for j in range(G):
            s_rows = gather_rows(tied_pool, page_table[b], L, page_size, j)
            k, v = gta_key_value(s_rows, r, d_rope, theta)
            qr = _rows_of_group(q[b], j, g)
            if d_rope and theta > 0:
                qr = np.concatenate([qr[:, :d - d_rope],
                                     rope_rotate_half(qr[:, d - d_rope:], qpos_all, theta)], axis=1)
            o, s = attend(qr, k, v, scale, pos)
            out[b, :, j * g:(j + 1) * g] = o.reshape(T, g, -1)
            lse[b, :, j * g:(j + 1) * g] = s.reshape(T, g)
    return out, lse


def decode_latent(q, latent_pool, rope_pool, page_table, seqlens, page_size, scale,
                  causal=False):
    """MLA / GLA decode in the weight-absorbed latent space ([HEA] "Core claim").

    q [B, T, H, d_c + d_r] (absorbed, RoPE part already rotated);
    latent_pool [pages, P, h_c, d_c]; rope_pool [pages, P, 1, d_r].
    Query head h uses latent head floor(h / (H / h_c)); the key is
    [latent_j || rope], the value is latent_j.  MLA is h_c = 1.
    """
    q = np.asarray(q)
    G, d_c = latent_pool.shape[2], latent_pool.shape[3]
    B, T, H, g = _check_common(q, page_table, seqlens, G, causal)
    out = np.zeros((B, T, H, d_c))
    lse = np.zeros((B, T, H))
    for b in range(B):
        L = int(seqlens[b])
        pos = _row_positions(L, T, g) if (causal and T > 1) else None
        r = gather_rows(rope_pool, page_table[b], L, page_size, 0)
        for j in range(G):
            c = gather_rows(latent_pool, page_table[b], L, page_size, j)
            k = np.concatenate([c, r], axis=1)
            o, s = attend(_rows_of_group(q[b], j, g), k, c, scale, pos)
            out[b, :, j * g:(j + 1) * g] = o.reshape(T, g, -1)
            lse[b, :, j * g:(j + 1) * g] = s.reshape(T, g)
    return out, lse


def decode(w, inp, batch_index=None):
    """Dispatch on a workload description (attributes as in the input module).

    ``batch_index`` restricts the computation to a subset of sequences (for
    sampled checks at full size); the result then has that many rows.
    """
    q, table, seqlens = inp["q"], inp["page_table"], inp["seqlens"]
    if batch_index is not None:
        idx = np.asarray(batch_index, dtype=np.int64)
        q, table, seqlens = q[idx], table[idx], seqlens[idx]
    if w.kind == "gqa":
        return decode_gqa(q, inp["pool0"], inp["pool1"], table, seqlens, w.page_size,
                          w.softmax_scale, w.causal)
    if w.kind == "gta":
        return decode_gta(q, inp["pool0"], inp["rope"], table, seqlens, w.page_size,
                          w.d_rope, w.rope_theta, w.softmax_scale, w.causal)
    if w.kind == "latent":
        return decode_latent(q, inp["pool0"], inp["rope"], table, seqlens, w.page_size,
                             w.softmax_scale, w.causal)
    raise ValueError(w.kind)
