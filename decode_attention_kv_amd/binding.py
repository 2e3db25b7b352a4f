"""ctypes binding of libattn_decode.so (declared in include/attn_decode.h).

Argument marshalling only: every step of the decode (planning, paged
gather, scores, softmax, P.V, split merge) runs inside the native library.
The functions named like the C entry points take raw pointers and sizes;
``decode`` below accepts torch tensors, builds the descriptor and plan,
allocates the workspace with torch (plumbing) and calls them.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_decode.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_HIP = -4
ATTN_FP32 = 0
ATTN_BF16 = 1
ATTN_CAUSAL = 1
ATTN_DEFER_MERGE = 2
ATTN_KIND = {"gqa": 0, "gta": 1, "latent": 2}
TILE = 64


class PagedKV(Structure):
    _fields_ = [("pool0", c_void_p), ("pool1", c_void_p), ("rope_pool", c_void_p),
                ("page_table", c_void_p), ("seqlens", c_void_p), ("batch", c_int32),
                ("max_pages_per_seq", c_int32), ("page_size", c_int32), ("num_pages", c_int32),
                ("page_stride", c_int64), ("token_stride", c_int64), ("head_stride", c_int64),
                ("rope_page_stride", c_int64), ("rope_token_stride", c_int64),
                ("rope_head_stride", c_int64), ("dtype", c_int)]


class Shape(Structure):
    _fields_ = [("kind", c_int), ("dtype", c_int), ("batch", c_int32), ("q_len", c_int32),
                ("h_q", c_int32), ("groups", c_int32), ("head_dim", c_int32), ("d_rope", c_int32),
                ("page_size", c_int32), ("flags", c_int32)]


def shape(kind: str, dtype: int, batch: int, q_len: int, h_q: int, groups: int, head_dim: int,
          d_rope: int, page_size: int, causal: bool) -> Shape:
    return Shape(ATTN_KIND[kind], dtype, batch, q_len, h_q, groups, head_dim, d_rope, page_size,
                 ATTN_CAUSAL if causal else 0)


class Plan(Structure):
    _fields_ = [("n_items", c_int32), ("batch", c_int32), ("n_groups", c_int32),
                ("q_len", c_int32), ("max_splits", c_int32), ("n_partial_slots", c_int32),
                ("items", c_void_p), ("seqinfo", c_void_p), ("counters", c_void_p),
                ("items_host", c_void_p), ("seqinfo_host", c_void_p), ("inline_ok", c_int32),
                ("queue", c_void_p)]


ATTN_PLAN_INLINE_MAX = 800


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {attn_status_string(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """Load the native library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    L.attn_status_string.argtypes = [c_int]
    L.attn_status_string.restype = c_char_p
    L.attn_decode_plan_max_items.argtypes = [c_int, c_int, c_int]
    L.attn_decode_plan_max_items.restype = c_int
    L.attn_decode_plan.argtypes = [POINTER(Shape), c_void_p, c_int, c_int, c_void_p, c_void_p,
                                   c_int, POINTER(Plan)]
    L.attn_decode_plan.restype = c_int
    L.attn_decode_workspace_size.argtypes = [POINTER(Plan), c_int, c_int]
    L.attn_decode_workspace_size.restype = c_size_t
    L.attn_decode_counter_count.argtypes = [POINTER(Plan), c_int]
    L.attn_decode_counter_count.restype = c_size_t
    common_tail = [c_float, c_int, POINTER(Plan), c_void_p, c_size_t, c_void_p]
    L.attn_decode_gqa.argtypes = ([POINTER(PagedKV), c_void_p, c_void_p, c_void_p, c_int, c_int,
                                   c_int, c_int] + common_tail)
    L.attn_decode_gqa.restype = c_int
    L.attn_decode_gqa_static.argtypes = [POINTER(PagedKV), c_void_p, c_void_p, c_void_p, c_int,
                                         c_int, c_int, c_int, c_float, c_int, POINTER(Plan),
                                         c_void_p]
    L.attn_decode_gqa_static.restype = c_int
    L.attn_decode_gta.argtypes = ([POINTER(PagedKV), c_void_p, c_void_p, c_void_p, c_int, c_int,
                                   c_int, c_int, c_int, c_int, c_float] + common_tail)
    L.attn_decode_gta.restype = c_int
    L.attn_decode_latent.argtypes = ([POINTER(PagedKV), c_void_p, c_void_p, c_void_p, c_int, c_int,
                                      c_int, c_int, c_int] + common_tail)
    L.attn_decode_latent.restype = c_int
    L.attn_decode_merge.argtypes = [POINTER(Plan), c_int, c_int, c_int, c_void_p, c_size_t,
                                    c_void_p, c_void_p, c_void_p]
    L.attn_decode_merge.restype = c_int
    L.attn_kv_append.argtypes = [POINTER(PagedKV), c_int, c_int, c_int, c_void_p, c_void_p, c_int,
                                 c_void_p, c_float, c_void_p]
    L.attn_kv_append.restype = c_int
    L.attn_paged_kv_check.argtypes = [POINTER(PagedKV)]
    L.attn_paged_kv_check.restype = c_int
    L.attn_latent_absorb_query.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                           c_int, c_int, c_int, c_void_p]
    L.attn_latent_absorb_query.restype = c_int
    L.attn_latent_project_output.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                             c_int, c_void_p]
    L.attn_latent_project_output.restype = c_int
    L.attn_probe_stream_read.argtypes = [c_void_p, c_size_t, c_int, c_void_p, c_void_p]
    L.attn_probe_stream_read.restype = c_int
    L.attn_probe_mfma.argtypes = [c_int, c_void_p, POINTER(ctypes.c_double), c_void_p]
    L.attn_probe_mfma.restype = c_int
    _lib = L
    return L


# ------------------------------------------------------------ C entry points
def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def attn_decode_plan_max_items(batch: int, n_groups: int, max_seqlen: int) -> int:
    return lib().attn_decode_plan_max_items(batch, n_groups, max_seqlen)


def attn_decode_plan(shape_: Shape, seqlens_host: np.ndarray, cu_count: int, chunk_tokens: int,
                     items_host: np.ndarray, seqinfo_host: np.ndarray, max_items: int):
    """Returns (status, Plan).  Host numpy arrays, int32, C-contiguous."""
    for a in (seqlens_host, items_host, seqinfo_host):
        if a.dtype != np.int32 or not a.flags.c_contiguous:
            raise ValueError("planner arrays must be C-contiguous int32")
    plan = Plan()
    st = lib().attn_decode_plan(ctypes.byref(shape_), seqlens_host.ctypes.data, cu_count,
                                chunk_tokens, items_host.ctypes.data, seqinfo_host.ctypes.data,
                                max_items, ctypes.byref(plan))
    return st, plan


def attn_decode_workspace_size(plan: Plan, h_q: int, d_v: int) -> int:
    return lib().attn_decode_workspace_size(ctypes.byref(plan), h_q, d_v)


def attn_decode_counter_count(plan: Plan, h_q: int) -> int:
    return lib().attn_decode_counter_count(ctypes.byref(plan), h_q)


def attn_decode_gqa(kv, q, out, lse, q_len, h_q, h_kv, d, scale, flags, plan, ws, ws_bytes,
                    stream) -> int:
    return lib().attn_decode_gqa(ctypes.byref(kv), q, out, lse, q_len, h_q, h_kv, d, scale,
                                 flags, ctypes.byref(plan), ws, ws_bytes, stream)


def attn_decode_gqa_static(kv, q, out, lse, q_len, h_q, h_kv, d, scale, flags, plan,
                           stream) -> int:
    return lib().attn_decode_gqa_static(ctypes.byref(kv), q, out, lse, q_len, h_q, h_kv, d, scale,
                                        flags, ctypes.byref(plan), stream)


ATTN_STATIC_SCRATCH_BYTES = 16 << 20


def attn_decode_gta(kv, q, out, lse, q_len, h_q, h_kv, d, d_rope, n_rope_heads, rope_theta,
                    scale, flags, plan, ws, ws_bytes, stream) -> int:
    return lib().attn_decode_gta(ctypes.byref(kv), q, out, lse, q_len, h_q, h_kv, d, d_rope,
                                 n_rope_heads, rope_theta, scale, flags, ctypes.byref(plan), ws,
                                 ws_bytes, stream)


def attn_decode_latent(kv, q, out, lse, q_len, h_q, h_c, d_c, d_rope, scale, flags, plan, ws,
                       ws_bytes, stream) -> int:
    return lib().attn_decode_latent(ctypes.byref(kv), q, out, lse, q_len, h_q, h_c, d_c, d_rope,
                                    scale, flags, ctypes.byref(plan), ws, ws_bytes, stream)


def attn_decode_merge(plan, h_q, d_v, dtype, ws, ws_bytes, out, lse, stream) -> int:
    return lib().attn_decode_merge(ctypes.byref(plan), h_q, d_v, dtype, ws, ws_bytes, out, lse,
                                   stream)


def attn_kv_append(kv, q_len, heads, width, new0, new1, d_rope, new_rope, rope_theta,
                   stream) -> int:
    return lib().attn_kv_append(ctypes.byref(kv), q_len, heads, width, new0, new1, d_rope,
                                new_rope, rope_theta, stream)


def attn_paged_kv_check(kv: PagedKV) -> int:
    return lib().attn_paged_kv_check(ctypes.byref(kv))


def attn_latent_absorb_query(q_nope, q_rope, w_uk, q_out, n_tok, h_q, d_nope, d_c, d_rope,
                             stream) -> int:
    return lib().attn_latent_absorb_query(q_nope, q_rope, w_uk, q_out, n_tok, h_q, d_nope, d_c,
                                          d_rope, stream)


def attn_latent_project_output(o_lat, w_uv, out, n_tok, h_q, d_c, d_v, stream) -> int:
    return lib().attn_latent_project_output(o_lat, w_uv, out, n_tok, h_q, d_c, d_v, stream)


def attn_probe_stream_read(buf, nbytes, mode, sink, stream) -> int:
    return lib().attn_probe_stream_read(buf, nbytes, mode, sink, stream)


def attn_probe_mfma(iters, sink, stream):
    """Returns (status, FLOPs of the launch)."""
    fl = ctypes.c_double(0.0)
    st = lib().attn_probe_mfma(iters, sink, ctypes.byref(fl), stream)
    return st, fl.value


# ------------------------------------------------------------ torch plumbing
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def paged_kv(pool0, pool1, rope, page_table, seqlens) -> PagedKV:
    """Descriptor over torch tensors pool [pages, P, heads, width] (any strides
    whose innermost stride is 1), page_table int32 [B, max_pages], seqlens
    int32 [B].  Works for host tensors too (for attn_paged_kv_check)."""
    import torch

    if pool0.dim() != 4 or pool0.stride(-1) != 1 or (pool1 is not None and pool1.stride(-1) != 1):
        raise ValueError("pools must be [pages, P, heads, width] with contiguous rows")
    # the kernels read the page table as int32 rows of max_pages entries and
    # one int32 length per sequence
    if (page_table.dtype != torch.int32 or page_table.dim() != 2 or
            not page_table.is_contiguous()):
        raise ValueError("page_table must be a contiguous int32 [B, max_pages] tensor")
    if (seqlens.dtype != torch.int32 or seqlens.dim() != 1 or not seqlens.is_contiguous() or
            seqlens.shape[0] != page_table.shape[0]):
        raise ValueError("seqlens must be a contiguous int32 [B] tensor")
    for t in (pool1, rope, page_table, seqlens):
        if t is not None and t.device != pool0.device:
            raise ValueError("the pools, page table and lengths must be on one device")
    # the descriptor holds one set of strides for pool0 and pool1
    if pool1 is not None and (pool1.shape != pool0.shape or pool1.stride() != pool0.stride()):
        raise ValueError("pool1 must have pool0's shape and strides")
    kv = PagedKV()
    kv.pool0, kv.pool1, kv.rope_pool = _ptr(pool0), _ptr(pool1), _ptr(rope)
    kv.page_table, kv.seqlens = page_table.data_ptr(), seqlens.data_ptr()
    kv.batch = page_table.shape[0]
    kv.max_pages_per_seq = page_table.shape[1]
    kv.page_size = pool0.shape[1]
    kv.num_pages = pool0.shape[0]
    kv.page_stride, kv.token_stride, kv.head_stride = pool0.stride(0), pool0.stride(1), pool0.stride(2)
    if rope is not None:
        kv.rope_page_stride, kv.rope_token_stride, kv.rope_head_stride = (
            rope.stride(0), rope.stride(1), rope.stride(2))
    if pool0.dtype == torch.bfloat16:
        kv.dtype = ATTN_BF16
    elif pool0.dtype == torch.float32:
        kv.dtype = ATTN_FP32
    else:
        raise ValueError(f"unsupported dtype {pool0.dtype}")
    return kv


class DevicePlan:
    """A host plan plus its device copy (keeps the device arrays alive)."""

    def __init__(self, shape_: Shape, seqlens_host, device, cu_count=256, chunk_tokens=0,
                 fused_merge=False, inline=False, queue=None):
        import torch

        seqlens_host = np.ascontiguousarray(seqlens_host, dtype=np.int32)
        batch = len(seqlens_host)
        max_items = attn_decode_plan_max_items(batch, shape_.groups,
                                               int(max(1, seqlens_host.max(initial=0))))
        if max_items < 0:
            raise AttnError(max_items, "attn_decode_plan_max_items")
        self.items_host = np.zeros((max_items, 4), dtype=np.int32)
        self.seqinfo_host = np.zeros((batch, 4), dtype=np.int32)
        st, plan = attn_decode_plan(shape_, seqlens_host, cu_count, chunk_tokens,
                                    self.items_host, self.seqinfo_host, max_items)
        if st != ATTN_OK:
            raise AttnError(st, "attn_decode_plan")
        if inline:
            # the plan travels in the kernels' launch arguments (read from the
            # host arrays this object keeps alive)
            if not plan.inline_ok:
                raise AttnError(ATTN_ERR_INVALID_ARG, "plan does not fit the launch arguments")
            self.items_dev = self.seqinfo_dev = None
            plan.items = plan.seqinfo = None
        else:
            self.items_dev = torch.from_numpy(self.items_host[:plan.n_items].copy()).to(device)
            self.seqinfo_dev = torch.from_numpy(self.seqinfo_host).to(device)
            plan.items = self.items_dev.data_ptr()
            plan.seqinfo = self.seqinfo_dev.data_ptr()
        # optional merge counters, zero-filled once; with them the streaming
        # kernels merge split rows themselves (one launch instead of two)
        self.counters = None
        if fused_merge:
            n = attn_decode_counter_count(plan, shape_.h_q)
            self.counters = torch.zeros(max(n, 1), dtype=torch.int32, device=device)
            plan.counters = self.counters.data_ptr()
        # optional work-queue counter (zero before first use; calls leave it zero)
        self.queue = queue
        if queue is not None:
            plan.queue = queue.data_ptr()
        self.plan = plan


def decode(kind: str, q, pool0, pool1, rope, page_table, seqlens, seqlens_host, *, groups: int,
           scale: float, causal: bool = False, rope_theta: float = 0.0, d_rope: int = 0,
           out=None, lse=None, chunk_tokens: int = 0, cu_count: int = 256, plan=None,
           workspace=None, stream=None, defer_merge: bool = False, fused_merge: bool = False,
           inline_plan: bool = False, queue=None):
    """Run one decode through the native library on torch tensors.

    kind: "gqa" | "gta" | "latent".  q [B, T, H, Dq]; pools as in the header.
    Returns (out, lse, plan, workspace) so callers can reuse plan/workspace.
    With ``defer_merge`` the split partials stay in the workspace and the
    caller finishes with ``merge``.  With ``fused_merge`` a new plan carries
    merge counters and the decode kernel merges split rows itself; otherwise
    the merge is a second launch on the stream.  With ``inline_plan`` a new
    plan is passed in the kernels' launch arguments instead of device arrays.
    ``queue`` (a zeroed int32 device tensor of one element) lets the GQA
    streaming kernel hand items out dynamically.
    """
    import torch

    B, T, H, _ = q.shape
    width = pool0.shape[-1]
    d_v = width
    if plan is None:
        dtype = ATTN_BF16 if pool0.dtype == torch.bfloat16 else ATTN_FP32
        sh = shape(kind, dtype, B, T, H, groups, width, d_rope, pool0.shape[1], causal)
        plan = DevicePlan(sh, seqlens_host, q.device, cu_count=cu_count, chunk_tokens=chunk_tokens,
                          fused_merge=fused_merge, inline=inline_plan, queue=queue)
    need = attn_decode_workspace_size(plan.plan, H, d_v)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    kv = paged_kv(pool0, pool1, rope, page_table, seqlens)
    s = (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream
    flags = (ATTN_CAUSAL if causal else 0) | (ATTN_DEFER_MERGE if defer_merge else 0)
    if kind == "gqa":
        st = attn_decode_gqa(kv, q.data_ptr(), out.data_ptr(), lse.data_ptr(), T, H, groups, width,
                             scale, flags, plan.plan, workspace.data_ptr(), need, s)
    elif kind == "gta":
        st = attn_decode_gta(kv, q.data_ptr(), out.data_ptr(), lse.data_ptr(), T, H, groups, width,
                             d_rope, 1, rope_theta, scale, flags, plan.plan,
                             workspace.data_ptr(), need, s)
    elif kind == "latent":
        st = attn_decode_latent(kv, q.data_ptr(), out.data_ptr(), lse.data_ptr(), T, H, groups,
                                width, d_rope, scale, flags, plan.plan,
                                workspace.data_ptr(), need, s)
    else:
        raise ValueError(kind)
    if st != ATTN_OK:
        raise AttnError(st, f"attn_decode_{kind}")
    return out, lse, plan, workspace


def kv_append(pool0, pool1, rope, page_table, seqlens, new0, new1=None, new_rope=None,
              rope_theta: float = 0.0, stream=None):
    """Write a step's new rows (new0/new1 [B, q_len, heads, width], new_rope
    [B, q_len, d_rope]) into the paged pools (attn_kv_append)."""
    import torch

    kv = paged_kv(pool0, pool1, rope, page_table, seqlens)
    B, T, Hh, Wd = new0.shape
    for t in (new0, new1, new_rope):
        if t is not None and not t.is_contiguous():
            raise ValueError("new rows must be contiguous")
    d_rope = 0 if new_rope is None else new_rope.shape[-1]
    s = (stream if stream is not None else torch.cuda.current_stream(new0.device)).cuda_stream
    st = attn_kv_append(kv, T, Hh, Wd, new0.data_ptr(), _ptr(new1), d_rope, _ptr(new_rope),
                        float(rope_theta), s)
    if st != ATTN_OK:
        raise AttnError(st, "attn_kv_append")


def absorb_query(q_nope, q_rope, w_uk, out=None, stream=None):
    """Latent decode query [.., h_q, d_c + d_r] from q_nope [.., h_q, d_nope],
    q_rope [.., h_q, d_r] (or None) and w_uk [h_q, d_c, d_nope], all bf16
    (attn_latent_absorb_query); leading dims are the step's tokens."""
    import torch

    h_q, d_nope = q_nope.shape[-2], q_nope.shape[-1]
    d_c = w_uk.shape[1]
    d_rope = 0 if q_rope is None else q_rope.shape[-1]
    lead = q_nope.shape[:-2]
    n_tok = int(np.prod(lead)) if len(lead) else 1
    for t in (q_nope, q_rope, w_uk):
        if t is not None and (not t.is_contiguous() or t.dtype != torch.bfloat16):
            raise ValueError("inputs must be contiguous bfloat16")
    if tuple(w_uk.shape) != (h_q, d_c, d_nope):
        raise ValueError("w_uk must be [h_q, d_c, d_nope]")
    if out is None:
        out = torch.empty(*lead, h_q, d_c + d_rope, dtype=torch.bfloat16, device=q_nope.device)
    s = (stream if stream is not None else torch.cuda.current_stream(q_nope.device)).cuda_stream
    st = attn_latent_absorb_query(q_nope.data_ptr(), _ptr(q_rope), w_uk.data_ptr(),
                                  out.data_ptr(), n_tok, h_q, d_nope, d_c, d_rope, s)
    if st != ATTN_OK:
        raise AttnError(st, "attn_latent_absorb_query")
    return out


def project_output(o_lat, w_uv, out=None, stream=None):
    """Per-head output [.., h_q, d_v] from the latent output o_lat
    [.., h_q, d_c] and w_uv [h_q, d_v, d_c], bf16 (attn_latent_project_output)."""
    import torch

    h_q, d_c = o_lat.shape[-2], o_lat.shape[-1]
    d_v = w_uv.shape[1]
    lead = o_lat.shape[:-2]
    n_tok = int(np.prod(lead)) if len(lead) else 1
    for t in (o_lat, w_uv):
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("inputs must be contiguous bfloat16")
    if tuple(w_uv.shape) != (h_q, d_v, d_c):
        raise ValueError("w_uv must be [h_q, d_v, d_c]")
    if out is None:
        out = torch.empty(*lead, h_q, d_v, dtype=torch.bfloat16, device=o_lat.device)
    s = (stream if stream is not None else torch.cuda.current_stream(o_lat.device)).cuda_stream
    st = attn_latent_project_output(o_lat.data_ptr(), w_uv.data_ptr(), out.data_ptr(), n_tok, h_q,
                                    d_c, d_v, s)
    if st != ATTN_OK:
        raise AttnError(st, "attn_latent_project_output")
    return out


def merge(plan: DevicePlan, out, lse, workspace, stream=None):
    """Finish a decode made with ``defer_merge`` (attn_decode_merge)."""
    import torch

    B, T, H, d_v = out.shape
    dtype = ATTN_BF16 if out.dtype == torch.bfloat16 else ATTN_FP32
    need = attn_decode_workspace_size(plan.plan, H, d_v)
    s = (stream if stream is not None else torch.cuda.current_stream(out.device)).cuda_stream
    st = attn_decode_merge(plan.plan, H, d_v, dtype, workspace.data_ptr(), need, out.data_ptr(),
                           None if lse is None else lse.data_ptr(), s)
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_merge")
