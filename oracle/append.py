"""Paged KV append, written out in float64 (TEST INFRASTRUCTURE ONLY).

The step before each decode call writes the new tokens' cache rows into
their pages: for sequence b holding L_b tokens after the write, query token t
of a q_len-T step sits at position L_b - T + t (the same positions the decode
oracle gives the query rows), in physical page page_table[b][pos // P],
slot pos % P.  GQA writes the key and value rows, GTA the tied state and the
raw RoPE key (the decode rotates it), MLA / GLA the latent rows and the RoPE
key rotated at its position (the decode reads it as stored: "Hardware-
Efficient Attention for Fast Decoding", review page, Core claim and the
Circularity Check's free parameters, partial RoPE on a separate key head).

Only tests may import this module; it shares no code with the HIP path.
"""
import numpy as np

from .attention import rope_rotate_half


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (round to nearest, ties to even) of x taken to
    float32 first, returned as float32."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), f, out)


def kv_append(pool0, pool1, rope, page_table, seqlens, page_size, new0, new1, new_rope,
              theta: float, dtype: str):
    """Copies of the pools with the new tokens' rows written.

    pool0/pool1 [pages, P, heads, width], rope [pages, P, 1, d_r] (None when
    absent); new0/new1 [B, T, heads, width], new_rope [B, T, d_r].  With
    theta > 0 the RoPE key of position pos is rotated (rotate-half, frequency
    theta ** (-2k / d_r)) before it is stored.  bf16 pools store the value
    rounded to the nearest bfloat16.
    """
    out = [None if a is None else np.array(a, copy=True) for a in (pool0, pool1, rope)]
    B, T = new0.shape[0], new0.shape[1]
    for b in range(B):
        L = int(seqlens[b])
        for t in range(T):
            pos = L - T + t
            if pos < 0:
                continue
            page = int(page_table[b, pos // page_size])
            slot = pos % page_size
            out[0][page, slot] = new0[b, t]
            if out[1] is not None and new1 is not None:
                out[1][page, slot] = new1[b, t]
            if out[2] is not None and new_rope is not None:
                r = np.asarray(new_rope[b, t], dtype=np.float64)
                if theta > 0:
                    r = rope_rotate_half(r, np.float64(pos), theta)
                out[2][page, slot, 0] = round_bf16(r) if dtype == "bf16" else r
    return tuple(out)
