"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws numbers and lays them out: query tensors, KV/latent
pools, per-sequence lengths and a page table.  It holds none of the attention
arithmetic, so both the fp64 oracle and the HIP path can consume exactly the
same host arrays.  Nothing here imports the rest of the package.

Layout of every pool (row-major, "token-major" paging):
    pool[num_pages, page_size, heads, width]
GQA: pool0 = K, pool1 = V.  GTA: pool0 = tied state, rope = shared RoPE key.
Latent (MLA/GLA): pool0 = latent heads, rope = shared (pre-rotated) RoPE key.

Workload shapes follow the decode-attention configurations studied in
"Hardware-Efficient Attention for Fast Decoding" (GQA, GTA with a
single-head partial-RoPE key, MLA with one 512-wide latent plus a 64-wide
RoPE key, GLA with two 256-wide latent heads).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16, so a
    later float32 -> bfloat16 conversion is lossless.  Inputs are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "gqa" | "gta" | "latent"
    dtype: str                # "fp32" | "bf16"
    batch: int
    q_len: int
    h_q: int
    groups: int               # KV heads (gqa/gta) or latent heads h_c (latent)
    head_dim: int             # d (gqa/gta) or d_c (latent)
    d_rope: int               # 0 (gqa) / RoPE width (gta, latent)
    seqlen_lo: int
    seqlen_hi: int            # inclusive; lo == hi means fixed length
    page_size: int
    max_seqlen: int           # sizes the page table: ceil(max_seqlen / page_size)
    permute_pages: bool
    q_std: float
    kv_std: float
    softmax_scale: float
    causal: bool
    seed: int
    rope_theta: float = 0.0   # > 0: RoPE applied inside the kernel (gta)

    @property
    def group_size(self) -> int:
        return self.h_q // self.groups

    @property
    def q_width(self) -> int:
        return self.head_dim + (self.d_rope if self.kind == "latent" else 0)

    @property
    def v_dim(self) -> int:
        return self.head_dim

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.max_seqlen // self.page_size)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _wl(**kw) -> Workload:
    return Workload(**kw)


# The five workloads (plus the companions the comparisons need).
WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 GQA, contiguous KV (one page per sequence)
    "gqa_fp32_tiny": _wl(name="gqa_fp32_tiny", kind="gqa", dtype="fp32", batch=2, q_len=1,
                          h_q=8, groups=2, head_dim=64, d_rope=0, seqlen_lo=256,
                          seqlen_hi=256, page_size=256, max_seqlen=256, permute_pages=False,
                          q_std=1.0, kv_std=1.0, softmax_scale=1.0 / 8.0, causal=False, seed=1),
    # Llama-3-8B-shaped GQA layer, ragged lengths
    "gqa_llama8b": _wl(name="gqa_llama8b", kind="gqa", dtype="bf16", batch=32, q_len=1,
                        h_q=32, groups=8, head_dim=128, d_rope=0, seqlen_lo=1024,
                        seqlen_hi=8192, page_size=64, max_seqlen=8192, permute_pages=True,
                        q_std=0.5, kv_std=0.5, softmax_scale=1.0 / math.sqrt(128.0),
                        causal=False, seed=2),
    # same shape at a fixed 8K context
    "gqa_llama8b_8k": _wl(name="gqa_llama8b_8k", kind="gqa", dtype="bf16", batch=32, q_len=1,
                           h_q=32, groups=8, head_dim=128, d_rope=0, seqlen_lo=8192,
                           seqlen_hi=8192, page_size=64, max_seqlen=8192, permute_pages=True,
                           q_std=0.5, kv_std=0.5, softmax_scale=1.0 / math.sqrt(128.0),
                           causal=False, seed=22),
    # GTA: 4 tied heads of 128, one shared 64-wide RoPE key, RoPE applied in-kernel
    "gta_8k": _wl(name="gta_8k", kind="gta", dtype="bf16", batch=64, q_len=1, h_q=32,
                   groups=4, head_dim=128, d_rope=64, seqlen_lo=8192, seqlen_hi=8192,
                   page_size=64, max_seqlen=8192, permute_pages=True, q_std=1.0, kv_std=1.0,
                   softmax_scale=1.0 / math.sqrt(128.0), causal=False, seed=3,
                   rope_theta=10000.0),
    # GQA-4 companion at the GTA shape (separate K and V)
    "gqa4_8k": _wl(name="gqa4_8k", kind="gqa", dtype="bf16", batch=64, q_len=1, h_q=32,
                    groups=4, head_dim=128, d_rope=0, seqlen_lo=8192, seqlen_hi=8192,
                    page_size=64, max_seqlen=8192, permute_pages=True, q_std=1.0, kv_std=1.0,
                    softmax_scale=1.0 / math.sqrt(128.0), causal=False, seed=33),
    # MLA: one 512-wide latent head + shared 64-wide RoPE key, 128 query heads
    "mla": _wl(name="mla", kind="latent", dtype="bf16", batch=128, q_len=1, h_q=128,
                groups=1, head_dim=512, d_rope=64, seqlen_lo=2048, seqlen_hi=32768,
                page_size=64, max_seqlen=32768, permute_pages=True, q_std=0.5, kv_std=0.5,
                softmax_scale=1.0 / math.sqrt(576.0), causal=False, seed=4),
    # GLA-2: two 256-wide latent heads (64 query heads each) + shared RoPE key
    "gla2": _wl(name="gla2", kind="latent", dtype="bf16", batch=128, q_len=1, h_q=128,
                 groups=2, head_dim=256, d_rope=64, seqlen_lo=2048, seqlen_hi=32768,
                 page_size=64, max_seqlen=32768, permute_pages=True, q_std=0.5, kv_std=0.5,
                 softmax_scale=1.0 / math.sqrt(320.0), causal=False, seed=4),
    # long-context speculative verify: 4 causal draft tokens, GLA-2 layout
    "gla2_spec4_128k": _wl(name="gla2_spec4_128k", kind="latent", dtype="bf16", batch=16,
                            q_len=4, h_q=128, groups=2, head_dim=256, d_rope=64,
                            seqlen_lo=131072, seqlen_hi=131072, page_size=64,
                            max_seqlen=131072, permute_pages=True, q_std=0.5, kv_std=0.5,
                            softmax_scale=1.0 / math.sqrt(320.0), causal=True, seed=5),
    # MLA companion of the speculative-verify workload
    "mla_spec4_128k": _wl(name="mla_spec4_128k", kind="latent", dtype="bf16", batch=16,
                           q_len=4, h_q=128, groups=1, head_dim=512, d_rope=64,
                           seqlen_lo=131072, seqlen_hi=131072, page_size=64,
                           max_seqlen=131072, permute_pages=True, q_std=0.5, kv_std=0.5,
                           softmax_scale=1.0 / math.sqrt(576.0), causal=True, seed=55),
}


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        x = round_bf16(x)
    return x


def make_projection_inputs(n_tok: int, h_q: int, d_nope: int, d_c: int, d_rope: int, d_v: int,
                           seed: int, q_std: float = 0.5) -> Dict[str, np.ndarray]:
    """Seeded inputs of the projections around the latent decode.

    Draw order from ``PCG64(seed)``: q_nope [n_tok, h_q, d_nope], q_rope
    [n_tok, h_q, d_rope] (None when d_rope is 0), w_uk [h_q, d_c, d_nope],
    w_uv [h_q, d_v, d_c], o_lat [n_tok, h_q, d_c].  Queries and o_lat are
    N(0,1)*q_std; weights are random-init N(0, 1/fan_in) (fan_in d_nope for
    w_uk, d_c for w_uv).  All bfloat16-exact float32.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out: Dict[str, np.ndarray] = {}
    out["q_nope"] = _normal(rng, (n_tok, h_q, d_nope), q_std, "bf16")
    out["q_rope"] = _normal(rng, (n_tok, h_q, d_rope), q_std, "bf16") if d_rope else None
    out["w_uk"] = _normal(rng, (h_q, d_c, d_nope), 1.0 / math.sqrt(d_nope), "bf16")
    out["w_uv"] = _normal(rng, (h_q, d_v, d_c), 1.0 / math.sqrt(d_c), "bf16")
    out["o_lat"] = _normal(rng, (n_tok, h_q, d_c), q_std, "bf16")
    return out


def draw_seqlens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.seqlen_lo == w.seqlen_hi:
        return np.full(w.batch, w.seqlen_lo, dtype=np.int32)
    return rng.integers(w.seqlen_lo, w.seqlen_hi + 1, size=w.batch).astype(np.int32)


def build_page_table(seqlens: np.ndarray, page_size: int, max_pages: int, permute: bool,
                     rng: Optional[np.random.Generator], extra_pages: int = 0):
    """Assign physical pages to every (sequence, logical page).

    Returns (page_table int32 [B, max_pages] padded with -1, num_pages).
    With ``permute`` the physical ids are a random permutation over all pages
    (including ``extra_pages`` that no sequence references).
    """
    seqlens = np.asarray(seqlens, dtype=np.int64)
    pages_per_seq = (seqlens + page_size - 1) // page_size
    if (pages_per_seq > max_pages).any():
        raise ValueError("sequence longer than the page table allows")
    n_used = int(pages_per_seq.sum())
    n_total = n_used + int(extra_pages)
    if permute:
        phys = rng.permutation(n_total).astype(np.int32)
    else:
        phys = np.arange(n_total, dtype=np.int32)
    table = np.full((len(seqlens), max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq.tolist()):
        table[b, :n] = phys[off:off + n]
        off += n
    return table, n_total


def _fill_unused(pool: np.ndarray, table: np.ndarray, seqlens: np.ndarray, page_size: int,
                 value: float) -> None:
    """Write ``value`` into every slot no sequence position maps to."""
    used = np.zeros(pool.shape[0], dtype=bool)
    for b, L in enumerate(seqlens.tolist()):
        n = -(-L // page_size)
        if n == 0:
            continue
        pages = table[b, :n]
        used[pages] = True
        tail = L - (n - 1) * page_size
        if tail < page_size:
            pool[pages[-1], tail:] = value
    pool[~used] = value


def make_inputs(w: Workload, *, seqlens=None, tail_fill: float = 0.0, extra_pages: int = 0,
                seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one batch of inputs for workload ``w``.

    Draw order from ``PCG64(seed)``: sequence lengths, page permutation,
    queries, pool0 (K / tied / latent), then pool1 (V) or the RoPE-key pool.
    Values are N(0,1)*std in float32, rounded to bfloat16 for bf16 workloads
    (returned as float32 arrays holding bf16-exact values).
    Unused page slots and unreferenced pages hold ``tail_fill``.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    if seqlens is None:
        seqlens = draw_seqlens(w, rng)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    if seqlens.shape != (w.batch,):
        raise ValueError("seqlens must have one entry per sequence")
    table, n_pages = build_page_table(seqlens, w.page_size, w.max_pages_per_seq,
                                      w.permute_pages, rng, extra_pages)
    P, G = w.page_size, w.groups
    out: Dict[str, np.ndarray] = {"seqlens": seqlens, "page_table": table}
    out["q"] = _normal(rng, (w.batch, w.q_len, w.h_q, w.q_width), w.q_std, w.dtype)
    out["pool0"] = _normal(rng, (n_pages, P, G, w.head_dim), w.kv_std, w.dtype)
    if w.kind == "gqa":
        out["pool1"] = _normal(rng, (n_pages, P, G, w.head_dim), w.kv_std, w.dtype)
        out["rope"] = None
    else:
        out["pool1"] = None
        out["rope"] = _normal(rng, (n_pages, P, 1, w.d_rope), w.kv_std, w.dtype)
    for key in ("pool0", "pool1", "rope"):
        if out[key] is not None:
            _fill_unused(out[key], table, seqlens, P, tail_fill)
    return out
