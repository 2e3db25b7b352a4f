"""Randomised checks of the library's host-only entry points (split planner,
workspace and counter sizing, descriptor check, status strings), meant to
run against a build of the host code with AddressSanitizer and UBSan:
tests/test_host_sanitized.py builds it and runs

    python3 -m tests.host_fuzz <library> <cases> <seed>

in a child process with the sanitizer runtime preloaded.  Every plan is
checked against the invariants the kernels rely on; invalid arguments must
come back as error codes.  Exit status 0 means every case passed and no
sanitizer reported anything.
"""
import ctypes
import sys
from ctypes import POINTER, c_int, c_size_t, c_void_p

import numpy as np

from decode_attention_kv_amd.binding import (ATTN_BF16, ATTN_ERR_INVALID_ARG, ATTN_ERR_WORKSPACE,
                                             ATTN_FP32, ATTN_KIND, ATTN_OK, PagedKV, Plan, Shape)

TILE = 64


def load(path):
    L = ctypes.CDLL(path)
    L.attn_status_string.argtypes = [c_int]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_decode_plan_max_items.argtypes = [c_int, c_int, c_int]
    L.attn_decode_plan_max_items.restype = c_int
    L.attn_decode_plan.argtypes = [POINTER(Shape), c_void_p, c_int, c_int, c_void_p, c_void_p,
                                   c_int, POINTER(Plan)]
    L.attn_decode_plan.restype = c_int
    L.attn_decode_workspace_size.argtypes = [POINTER(Plan), c_int, c_int]
    L.attn_decode_workspace_size.restype = c_size_t
    L.attn_decode_counter_count.argtypes = [POINTER(Plan), c_int]
    L.attn_decode_counter_count.restype = c_size_t
    L.attn_paged_kv_check.argtypes = [POINTER(PagedKV)]
    L.attn_paged_kv_check.restype = c_int
    return L


def random_shape(rng):
    kind = ["gqa", "gta", "latent"][rng.integers(3)]
    if kind == "gqa":
        d, d_rope = [64, 128][rng.integers(2)], 0
    elif kind == "gta":
        d, d_rope = 128, 64
    else:
        d, d_rope = [256, 512][rng.integers(2)], 64
    groups = int([1, 2, 4, 8][rng.integers(4)])
    g = int([1, 2, 3, 4, 8, 16, 64][rng.integers(7)])
    q_len = int(rng.integers(1, 17))
    causal = q_len > 1 and rng.random() < 0.7
    page = int(2 ** rng.integers(0, 9))
    dtype = ATTN_BF16 if rng.random() < 0.85 else ATTN_FP32
    return dict(kind=kind, d=d, d_rope=d_rope, groups=groups, h_q=groups * g, q_len=q_len,
                causal=causal, page=page, dtype=dtype)


def random_seqlens(rng, batch, q_len, causal):
    mode = rng.integers(4)
    if mode == 0:
        s = rng.integers(0, 300, size=batch)
    elif mode == 1:
        s = rng.integers(0, 20000, size=batch)
    elif mode == 2:
        s = np.full(batch, int(rng.integers(1, 140000)))
    else:
        s = rng.integers(0, 140000, size=batch)
        s[rng.random(batch) < 0.3] = 0
    if causal:
        s = np.maximum(s, q_len)
    return s.astype(np.int32)


def plan(L, sh, seqlens, cu, chunk, max_items=None):
    batch = len(seqlens)
    mi = L.attn_decode_plan_max_items(batch, sh["groups"], int(max(1, seqlens.max())))
    assert mi > 0, "max_items"
    cap = mi if max_items is None else max_items
    items = np.zeros((max(cap, 1), 4), np.int32)
    info = np.zeros((batch, 4), np.int32)
    shape = Shape(ATTN_KIND[sh["kind"]], sh["dtype"], batch, sh["q_len"], sh["h_q"], sh["groups"],
                  sh["d"], sh["d_rope"], sh["page"], 1 if sh["causal"] else 0)
    p = Plan()
    st = L.attn_decode_plan(ctypes.byref(shape), seqlens.ctypes.data, cu, chunk, items.ctypes.data,
                            info.ctypes.data, cap, ctypes.byref(p))
    return st, p, items, info, mi


def check_plan(L, sh, seqlens, p, items, info, mi, chunk):
    batch, G = len(seqlens), sh["groups"]
    assert 0 < p.n_items <= mi
    assert (p.batch, p.n_groups, p.q_len) == (batch, G, sh["q_len"])
    items = items[:p.n_items]
    # every (sequence, group) covered by its chunks exactly once, in order
    n, base, Ls, ch = info.T
    assert (Ls == seqlens).all() and (n >= 1).all() and (ch > 0).all() and (ch % TILE == 0).all()
    if chunk:
        assert (ch == chunk).all()
    assert ((n - 1) * ch < np.maximum(Ls, 1)).all() and (n * ch >= Ls).all()
    seen = np.zeros((batch, G, int(n.max())), np.int32)
    for b, j, s, t0 in items.tolist():
        assert 0 <= b < batch and 0 <= j < G and 0 <= s < n[b] and t0 == s * ch[b]
        seen[b, j, s] += 1
    for b in range(batch):
        assert (seen[b, :, :n[b]] == 1).all() and (seen[b, :, n[b]:] == 0).all()
    # partial slots: contiguous, one per split of every split sequence
    nxt = 0
    for b in range(batch):
        if n[b] > 1:
            assert base[b] == nxt
            nxt += n[b]
        else:
            assert base[b] == -1
    assert nxt == p.n_partial_slots and p.max_splits == n.max()
    d_v = sh["d"]
    ws = L.attn_decode_workspace_size(ctypes.byref(p), sh["h_q"], d_v)
    rows = p.n_partial_slots * sh["q_len"] * sh["h_q"]
    assert ws >= rows * (d_v + 1) * 4 and ws % 256 == 0
    per = -(-(sh["h_q"] // G) * sh["q_len"] // 32)
    assert L.attn_decode_counter_count(ctypes.byref(p), sh["h_q"]) == batch * G * per


def check_paged_kv(L, rng):
    batch, maxp = int(rng.integers(1, 20)), int(rng.integers(1, 40))
    P = int(2 ** rng.integers(0, 8))
    num_pages = int(rng.integers(1, 200))
    table = rng.integers(-1, num_pages + 2, size=(batch, maxp)).astype(np.int32)
    seqlens = rng.integers(0, maxp * P + 3 * P, size=batch).astype(np.int32)
    kv = PagedKV()
    kv.pool0 = 4096
    kv.page_table, kv.seqlens = table.ctypes.data, seqlens.ctypes.data
    kv.batch, kv.max_pages_per_seq, kv.page_size, kv.num_pages = batch, maxp, P, num_pages
    ok = True
    for b in range(batch):
        need = -(-int(seqlens[b]) // P)
        if need > maxp or ((table[b, :need] < 0) | (table[b, :need] >= num_pages)).any():
            ok = False
    got = L.attn_paged_kv_check(ctypes.byref(kv))
    assert got == (ATTN_OK if ok else ATTN_ERR_INVALID_ARG), (got, ok)


def main(path, n_cases, seed):
    L = load(path)
    for s in (0, -1, -2, -3, -4, -99):
        assert L.attn_status_string(s)
    rng = np.random.default_rng(seed)
    n_plans = 0
    for case in range(n_cases):
        sh = random_shape(rng)
        batch = int(rng.integers(1, 64)) if rng.random() < 0.9 else int(rng.integers(64, 1500))
        seqlens = random_seqlens(rng, batch, sh["q_len"], sh["causal"])
        cu = int([1, 8, 80, 256, 304][rng.integers(5)])
        chunk = 0 if rng.random() < 0.6 else TILE * int(rng.integers(1, 40))
        st, p, items, info, mi = plan(L, sh, seqlens, cu, chunk)
        assert st == ATTN_OK, (case, st, sh)
        check_plan(L, sh, seqlens, p, items, info, mi, chunk)
        n_plans += 1
        # less room for items: a forced chunk length must fail; the automatic
        # split settles for fewer splits while the unsplit plan fits
        if p.n_items > 1:
            cap = p.n_items - 1
            st2, p2, items2, info2, mi2 = plan(L, sh, seqlens, cu, chunk, max_items=cap)
            if chunk or cap < batch * sh["groups"]:
                assert st2 == ATTN_ERR_WORKSPACE, (case, st2)
            else:
                assert st2 == ATTN_OK and p2.n_items <= cap, (case, st2, p2.n_items, cap)
                check_plan(L, sh, seqlens, p2, items2, info2, mi2, chunk)
        # invalid arguments come back as errors
        bad = seqlens.copy()
        bad[int(rng.integers(batch))] = -int(rng.integers(1, 1000))
        assert plan(L, sh, bad, cu, chunk)[0] == ATTN_ERR_INVALID_ARG
        assert plan(L, sh, seqlens, cu, TILE * 2 + 1)[0] == ATTN_ERR_INVALID_ARG
        if sh["causal"]:
            short = seqlens.copy()
            short[0] = sh["q_len"] - 1
            assert plan(L, sh, short, cu, chunk)[0] == ATTN_ERR_INVALID_ARG
        check_paged_kv(L, rng)
    print(f"host fuzz: {n_plans} plans checked", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1], int(sys.argv[2]), int(sys.argv[3])))
