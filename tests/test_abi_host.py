"""The C ABI on the host: the library loads, exports every declared entry
point, and its host-only logic (planning, workspace sizing, descriptor
checks, argument validation) behaves as the header states.  No GPU needed:
every call here returns before anything is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

from decode_attention_kv_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "attn_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 8, names
    lib = binding.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert binding.attn_status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert binding.attn_status_string(s) not in ("ok", "unknown status")
    assert binding.attn_status_string(12345) == "unknown status"


def _plan(seqlens, q_len=1, h_q=32, groups=8, kind="gqa", d=128, d_rope=0, page=64, cu=256,
          chunk=0, causal=0, dtype=binding.ATTN_BF16):
    seqlens = np.asarray(seqlens, dtype=np.int32)
    mi = binding.attn_decode_plan_max_items(len(seqlens), groups, int(max(1, seqlens.max())))
    items = np.zeros((mi, 4), np.int32)
    info = np.zeros((len(seqlens), 4), np.int32)
    sh = binding.shape(kind, dtype, len(seqlens), q_len, h_q, groups, d, d_rope, page, causal)
    st, plan = binding.attn_decode_plan(sh, seqlens, cu, chunk, items, info, mi)
    return st, plan, items[:max(plan.n_items, 0)], info


@pytest.mark.parametrize("chunk", [0, 64, 320])
def test_plan_covers_every_token_once(chunk):
    rng = np.random.default_rng(3)
    seqlens = rng.integers(0, 5000, size=37).astype(np.int32)
    seqlens[5] = 0
    st, plan, items, info = _plan(seqlens, chunk=chunk)
    assert st == 0
    G = 8
    cover = {}
    for b, j, s, t0 in items.tolist():
        n, base, L, ch = info[b]
        assert L == seqlens[b] and 0 <= s < n and t0 == s * ch and ch % 64 == 0
        cover.setdefault((b, j), []).append((t0, min(t0 + ch, L)))
    for b, L in enumerate(seqlens.tolist()):
        for j in range(G):
            spans = sorted(cover[(b, j)])
            assert spans[0][0] == 0 and spans[-1][1] == L
            for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
                assert a1 == b0 and a0 < a1
    # partial slots: contiguous, one per split of every split sequence
    slots = [(info[b, 1], info[b, 0]) for b in range(len(seqlens)) if info[b, 0] > 1]
    assert sum(n for _, n in slots) == plan.n_partial_slots
    nxt = 0
    for base, n in slots:
        assert base == nxt
        nxt += n
    assert all(info[b, 1] == -1 for b in range(len(seqlens)) if info[b, 0] == 1)
    assert plan.max_splits == info[:, 0].max()
    if chunk:
        assert (info[:, 3] == chunk).all()


def test_plan_is_deterministic_and_longest_first():
    seqlens = np.array([100, 8000, 3000, 64], np.int32)
    a = _plan(seqlens)
    b = _plan(seqlens)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])
    items, info = a[2], a[3]
    lens = [min(t0 + info[b_, 3], info[b_, 2]) - t0 for b_, _, _, t0 in items.tolist()]
    # chunks in launch order, longest first
    assert lens == sorted(lens, reverse=True)
    # a forced chunk length: full chunks first, then the tails longest first
    items, info = _plan(seqlens, chunk=1024)[2:]
    lens = [min(t0 + 1024, info[b_, 2]) - t0 for b_, _, _, t0 in items.tolist()]
    full = [l == 1024 for l in lens]
    assert (info[:, 3] == 1024).all() and full == sorted(full, reverse=True)
    tails = [l for l, f in zip(lens, full) if not f]
    assert tails == sorted(tails, reverse=True)


@pytest.mark.parametrize("batch,groups,kind", [(512, 8, "gqa"), (4096, 8, "gqa"),
                                               (256, 1, "latent")])
def test_plan_large_batches(batch, groups, kind):
    # many more work items than the GPU has slots, with ragged lengths
    rng = np.random.default_rng(batch)
    seqlens = rng.integers(1, 20000, size=batch).astype(np.int32)
    d, d_rope, h_q = (128, 0, 32) if kind == "gqa" else (512, 64, 128)
    st, plan, items, info = _plan(seqlens, h_q=h_q, groups=groups, kind=kind, d=d,
                                  d_rope=d_rope)
    assert st == 0 and plan.n_items == len(items) >= batch * groups
    _assert_balanced(info)


def _assert_balanced(info):
    """Automatic plans: a sequence split n ways has n chunks of equal length
    (whole 64-token tiles) of which only the last is shorter."""
    for n, _, L, ch in info.tolist():
        assert ch % 64 == 0 and ch > 0
        tiles = -(-L // 64)
        if n > 1:
            assert ch == -(-tiles // n) * 64 and (n - 1) * ch < L <= n * ch


def test_plan_auto_split_balances_load():
    # one long sequence must be split so its chunks do not dominate
    seqlens = np.array([131072] * 16, np.int32)
    st, plan, items, info = _plan(seqlens, q_len=4, h_q=128, groups=2, kind="latent", d=256,
                                  d_rope=64, causal=1)
    assert st == 0 and plan.max_splits > 1
    _assert_balanced(info)
    # partial traffic stays a small fraction of the cache bytes
    part = plan.n_partial_slots * 4 * 128 * (256 + 1) * 4 * 2
    kv = int(seqlens.sum()) * 1152
    assert part < 0.1 * kv
    # a short uniform batch that already fills the GPU is not split
    st, plan, _, _ = _plan(np.full(512, 256, np.int32), groups=8)
    assert plan.max_splits == 1


def test_plan_errors():
    assert _plan([10, 20], chunk=100)[0] == binding.ATTN_ERR_INVALID_ARG
    assert _plan([10, -1])[0] == binding.ATTN_ERR_INVALID_ARG
    assert _plan([2, 20], q_len=4, causal=1)[0] == binding.ATTN_ERR_INVALID_ARG
    assert _plan([10, 20], h_q=30, groups=8)[0] == binding.ATTN_ERR_INVALID_ARG
    assert _plan([10, 20], kind="gqa", d=0)[0] == binding.ATTN_ERR_INVALID_ARG
    seq = np.array([5000], np.int32)
    items = np.zeros((2, 4), np.int32)
    info = np.zeros((1, 4), np.int32)
    sh = binding.shape("gqa", binding.ATTN_BF16, 1, 1, 32, 8, 128, 0, 64, False)
    st, _ = binding.attn_decode_plan(sh, seq, 256, 64, items, info, 2)
    assert st == binding.ATTN_ERR_WORKSPACE
    bad = binding.shape("gqa", binding.ATTN_BF16, 1, 1, 32, 8, 128, 0, 64, False)
    bad.kind = 7
    st, _ = binding.attn_decode_plan(bad, seq, 256, 0, np.zeros((200, 4), np.int32), info, 200)
    assert st == binding.ATTN_ERR_INVALID_ARG


def _ws_expect(plan, slots, h_q, d_v):
    rows = slots * plan.q_len * h_q
    pad = lambda x: (x + 255) // 256 * 256
    group_rows = h_q // plan.n_groups * plan.q_len
    row_blocks = max(1, -(-group_rows // 32))
    units = -(-plan.n_items // plan.n_groups)
    flags = -(-units // 8) * 8 * plan.n_groups * row_blocks * 4
    return pad(rows * d_v * 4) + pad(rows * 4) + pad(flags)


def test_workspace_size():
    st, plan, _, info = _plan([5000, 100], chunk=64)
    slots = int(info[info[:, 0] > 1, 0].sum())
    assert slots == plan.n_partial_slots
    assert binding.attn_decode_workspace_size(plan, 32, 128) == _ws_expect(plan, slots, 32, 128)
    # nothing split: only the per-workgroup flags remain
    st, plan, _, _ = _plan([100, 100], chunk=0)
    assert plan.n_partial_slots == 0
    assert binding.attn_decode_workspace_size(plan, 32, 128) == _ws_expect(plan, 0, 32, 128)
    st, plan, _, _ = _plan([4096] * 4, q_len=4, h_q=128, groups=2, kind="latent", d=256,
                           d_rope=64, causal=1)
    assert binding.attn_decode_workspace_size(plan, 128, 256) == _ws_expect(
        plan, plan.n_partial_slots, 128, 256)


def test_counter_count():
    # one merge counter per (sequence, group, block of 32 query rows)
    st, plan, _, _ = _plan([5000, 100, 7], groups=8, h_q=32)
    assert binding.attn_decode_counter_count(plan, 32) == 3 * 8 * 1
    st, plan, _, _ = _plan([4096] * 4, q_len=4, h_q=128, groups=2, kind="latent", d=256,
                           d_rope=64, causal=1)
    assert binding.attn_decode_counter_count(plan, 128) == 4 * 2 * 8
    st, plan, _, _ = _plan([300] * 5, h_q=128, groups=1, kind="latent", d=512, d_rope=64)
    assert binding.attn_decode_counter_count(plan, 128) == 5 * 1 * 4
    assert binding.attn_decode_counter_count(plan, 0) == 0
    assert plan.counters is None  # the planner leaves it to the caller


def _host_kv(seqlens, table, num_pages, P=64):
    import torch

    kv = binding.PagedKV()
    seqlens = np.ascontiguousarray(seqlens, np.int32)
    table = np.ascontiguousarray(table, np.int32)
    kv.page_table, kv.seqlens = table.ctypes.data, seqlens.ctypes.data
    kv.batch, kv.max_pages_per_seq = table.shape
    kv.page_size, kv.num_pages = P, num_pages
    kv.pool0 = 4096
    return kv, (seqlens, table)


def test_paged_kv_check():
    table = np.array([[0, 3, -1], [2, 1, -1]], np.int32)
    kv, keep = _host_kv([100, 65], table, 4)
    assert binding.attn_paged_kv_check(kv) == 0
    kv, keep = _host_kv([100, 129], table, 4)      # needs a third page: -1
    assert binding.attn_paged_kv_check(kv) == binding.ATTN_ERR_INVALID_ARG
    kv, keep = _host_kv([100, 65], table, 3)       # page id 3 out of range
    assert binding.attn_paged_kv_check(kv) == binding.ATTN_ERR_INVALID_ARG
    kv, keep = _host_kv([200, 65], table, 4)       # longer than the table allows
    assert binding.attn_paged_kv_check(kv) == binding.ATTN_ERR_INVALID_ARG


def test_paged_kv_needs_one_layout_for_both_pools():
    """The descriptor has one set of strides: a V pool laid out differently
    from the K pool is refused rather than read with the K pool's strides."""
    import torch

    table = torch.zeros((2, 3), dtype=torch.int32)
    seqlens = torch.tensor([5, 9], dtype=torch.int32)
    k = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16)
    kv = binding.paged_kv(k, torch.zeros_like(k), None, table, seqlens)
    assert (kv.page_stride, kv.token_stride, kv.head_stride) == (16 * 2 * 64, 2 * 64, 64)
    head_major = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16).permute(0, 2, 1, 3)
    with pytest.raises(ValueError):
        binding.paged_kv(k, head_major, None, table, seqlens)
    with pytest.raises(ValueError):
        binding.paged_kv(k, torch.zeros((4, 16, 2, 32), dtype=torch.bfloat16), None, table, seqlens)
    # the same non-default layout for both pools is fine
    kv = binding.paged_kv(head_major, head_major.clone(memory_format=torch.preserve_format),
                          None, table, seqlens)
    assert kv.token_stride == 64 and kv.head_stride == 16 * 64


def test_paged_kv_refuses_index_arrays_the_kernels_cannot_read():
    """The kernels read the page table as contiguous int32 rows and one int32
    length per sequence: other dtypes, shapes or layouts are refused when
    the descriptor is built, as are tensors on different devices."""
    import torch

    k = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16)
    table = torch.zeros((2, 3), dtype=torch.int32)
    seqlens = torch.tensor([5, 9], dtype=torch.int32)
    binding.paged_kv(k, k, None, table, seqlens)
    bad = [(table.long(), seqlens), (table.t().contiguous().t(), seqlens), (table[0], seqlens),
           (table, seqlens.long()), (table, seqlens[:1]), (table, torch.zeros((2, 1), dtype=torch.int32))]
    for t, l in bad:
        with pytest.raises(ValueError):
            binding.paged_kv(k, k, None, t, l)
    with pytest.raises(ValueError):
        binding.paged_kv(k[0], k[0], None, table, seqlens)      # not [pages, P, heads, width]
    with pytest.raises(ValueError):
        binding.paged_kv(k, k, None, table.to("meta"), seqlens)  # another device
    with pytest.raises(ValueError):
        binding.attn_decode_plan(binding.shape("gqa", binding.ATTN_BF16, 2, 1, 8, 2, 64, 0, 16,
                                               False),
                                 np.array([5, 9], dtype=np.int64), 256, 0,
                                 np.zeros((8, 4), np.int32), np.zeros((2, 4), np.int32), 8)


def _fake_call(kind="gqa", **over):
    """A decode call with fake (never dereferenced) aligned device pointers:
    validation must reject it before any launch."""
    st, plan, items, info = _plan(over.pop("plan_seqlens", [100, 200]),
                                  groups=over.pop("plan_groups", 8), chunk=64,
                                  q_len=over.pop("plan_q_len", 1),
                                  causal=over.pop("plan_causal", 0))
    edit = over.pop("edit_host", None)
    if edit is not None:  # tamper with the host arrays the call checks
        edit(items, info)
    plan.items, plan.seqinfo = 0x10000, 0x20000
    for k, v in over.pop("plan_fields", {}).items():
        setattr(plan, k, v)
    kv = binding.PagedKV()
    kv.pool0, kv.pool1, kv.rope_pool = 0x100000, 0x200000, 0x300000
    kv.page_table, kv.seqlens = 0x400000, 0x500000
    kv.batch, kv.max_pages_per_seq, kv.page_size, kv.num_pages = 2, 4, 64, 8
    kv.page_stride, kv.token_stride, kv.head_stride = 64 * 8 * 128, 8 * 128, 128
    kv.rope_page_stride, kv.rope_token_stride = 64 * 64, 64
    kv.dtype = binding.ATTN_BF16
    args = dict(q=0x600000, out=0x700000, lse=0, q_len=1, h_q=32, groups=8, d=128,
                ws=0x800000, ws_bytes=0, flags=0)
    for k, v in over.items():
        if hasattr(kv, k):
            setattr(kv, k, v)
        else:
            args[k] = v
    _fake_call.keep = (items, info)  # the plan's host arrays outlive the call
    if kind == "gqa":
        return binding.attn_decode_gqa(kv, args["q"], args["out"], args["lse"], args["q_len"],
                                       args["h_q"], args["groups"], args["d"], 0.1, args["flags"], plan,
                                       args["ws"], args["ws_bytes"], None)
    if kind == "gta":
        return binding.attn_decode_gta(kv, args["q"], args["out"], args["lse"], args["q_len"],
                                       args["h_q"], args["groups"], args["d"],
                                       args.get("d_rope", 64), args.get("n_rope", 1), 10000.0,
                                       0.1, args["flags"], plan, args["ws"], args["ws_bytes"], None)
    return binding.attn_decode_latent(kv, args["q"], args["out"], args["lse"], args["q_len"],
                                      args["h_q"], args["groups"], args["d"],
                                      args.get("d_rope", 64), 0.1, args["flags"], plan, args["ws"],
                                      args["ws_bytes"], None)


def test_validation_rejects_before_launch():
    E, U, WS = binding.ATTN_ERR_INVALID_ARG, binding.ATTN_ERR_UNSUPPORTED, binding.ATTN_ERR_WORKSPACE
    assert _fake_call(q=0) == E
    assert _fake_call(pool1=None) == E
    assert _fake_call(page_size=48) == E                 # not a power of two
    assert _fake_call(pool0=0x100008) == E               # misaligned pool
    assert _fake_call(token_stride=8 * 128 + 4) == E     # misaligned rows
    assert _fake_call(h_q=30) == E                       # h_q % groups
    assert _fake_call(batch=3) == E                      # plan / descriptor mismatch
    assert _fake_call(q_len=2) == E                      # plan made for q_len 1
    assert _fake_call(q_len=17) == E
    assert _fake_call(flags=4, ws_bytes=1 << 30) == E    # unknown flag bit
    assert _fake_call() == WS                            # splits need workspace
    assert _fake_call(ws=0x800010, ws_bytes=1 << 30) == WS   # misaligned workspace
    assert _fake_call(d=96, ws_bytes=1 << 30) == U
    assert _fake_call("gta", ws_bytes=1 << 30, d_rope=32) == U
    assert _fake_call("gta", ws_bytes=1 << 30, n_rope=2) == E
    assert _fake_call("gta", ws_bytes=1 << 30, rope_pool=None) == E
    assert _fake_call("latent", ws_bytes=1 << 30, d=384, groups=2, plan_groups=2) == U
    assert _fake_call("latent", ws_bytes=1 << 30, dtype=binding.ATTN_FP32, d=256, groups=2,
                      plan_groups=2) == U


def test_merge_validation():
    st, plan, items, info = _plan([5000, 100], chunk=64)
    plan.items, plan.seqinfo = 0x10000, 0x20000
    need = binding.attn_decode_workspace_size(plan, 32, 128)
    M = binding.attn_decode_merge
    assert M(plan, 32, 96, binding.ATTN_BF16, 0x800000, need, 0x700000, None, None) == binding.ATTN_ERR_UNSUPPORTED
    assert M(plan, 32, 128, binding.ATTN_BF16, 0x800000, need - 1, 0x700000, None, None) == binding.ATTN_ERR_WORKSPACE
    assert M(plan, 32, 128, 7, 0x800000, need, 0x700000, None, None) == binding.ATTN_ERR_INVALID_ARG
    assert M(plan, 32, 128, binding.ATTN_BF16, 0x800000, need, 0, None, None) == binding.ATTN_ERR_INVALID_ARG
    # a plan whose host arrays were altered after planning is refused
    info[1, 1] = 10_000                  # partial slots past the plan's count
    assert M(plan, 32, 128, binding.ATTN_BF16, 0x800000, need, 0x700000, None, None) == binding.ATTN_ERR_INVALID_ARG
    st, plan, items, info = _plan([100, 100])
    plan.items, plan.seqinfo = 0x10000, 0x20000
    # nothing split: a no-op that succeeds without touching the GPU
    assert M(plan, 32, 128, binding.ATTN_BF16, 0, 0, 0x700000, None, None) == binding.ATTN_OK
    assert M(plan, 30, 128, binding.ATTN_BF16, 0, 0, 0x700000, None, None) == binding.ATTN_ERR_INVALID_ARG


def _set(arr, idx, val):
    def f(items, info):
        (items if arr == "items" else info)[idx] = val
    return f


@pytest.mark.parametrize("kind", ["gqa", "gta", "latent"])
def test_decode_checks_the_plan_against_the_descriptor(kind):
    """The decode kernels take lengths, splits and chunks from the plan, not
    from kv->seqlens: a plan whose lengths overrun the page table's row
    (max_pages_per_seq * page_size = 256 here), a causal plan shorter than
    q_len, or host arrays altered after planning are refused before any
    launch (fake, never dereferenced device pointers)."""
    E, WS = binding.ATTN_ERR_INVALID_ARG, binding.ATTN_ERR_WORKSPACE
    d = dict(gqa=128, gta=128, latent=256)[kind]
    ex = dict(d=d, ws_bytes=0)  # the plan is checked before the (missing) workspace
    if kind == "latent":
        ex.update(plan_groups=2, groups=2)
    assert _fake_call(kind, **ex) == WS
    assert _fake_call(kind, plan_seqlens=[256, 1], **ex) == WS            # exactly 4 pages of 64
    assert _fake_call(kind, plan_seqlens=[100, 257], **ex) == E           # one token more
    for edit in (_set("info", (1, 2), 300),        # length past the page-table row
                 _set("info", (0, 0), 0),          # zero splits
                 _set("info", (0, 3), 32),         # chunks no longer cover the length
                 _set("info", (1, 1), 999),        # partial slots past the count
                 _set("items", (0, 0), 2),         # a sequence that does not exist
                 _set("items", (0, 1), 1),         # groups out of plan order
                 _set("items", (1, 2), 7),         # a split past the sequence's count
                 _set("items", (1, 3), 5)):        # first token off its chunk
        assert _fake_call(kind, edit_host=edit, **ex) == E
    # causal q_len 4: every length must hold at least the 4 query tokens
    causal = dict(plan_q_len=4, plan_causal=1, q_len=4, flags=1, **ex)
    assert _fake_call(kind, **causal) == WS
    assert _fake_call(kind, edit_host=_set("info", (0, 2), 3), **causal) == E


def _append_kv():
    kv = binding.PagedKV()
    kv.pool0, kv.pool1, kv.rope_pool = 0x100000, 0x200000, 0x300000
    kv.page_table, kv.seqlens = 0x400000, 0x500000
    kv.batch, kv.max_pages_per_seq, kv.page_size, kv.num_pages = 2, 4, 64, 8
    kv.page_stride, kv.token_stride, kv.head_stride = 64 * 8 * 128, 8 * 128, 128
    kv.rope_page_stride, kv.rope_token_stride, kv.rope_head_stride = 64 * 64, 64, 0
    kv.dtype = binding.ATTN_BF16
    return kv


@pytest.mark.parametrize("case", ["null_kv", "null_new0", "q_len0", "width_not_16B", "odd_rope",
                                  "rope_too_wide", "rope_without_pool", "values_without_pool",
                                  "page_not_pow2", "unaligned_new0", "neg_stride"])
def test_append_rejects_bad_arguments(case):
    """attn_kv_append validates on the host and enqueues nothing on error
    (fake, never dereferenced device pointers)."""
    kv = _append_kv()
    args = dict(q_len=1, heads=8, width=128, new0=0x600000, new1=0x700000, d_rope=64,
                new_rope=0x800000, theta=0.0)
    if case == "null_kv":
        assert binding.lib().attn_kv_append(None, 1, 8, 128, 0x600000, None, 0, None, 0.0,
                                            None) == binding.ATTN_ERR_INVALID_ARG
        return
    if case == "null_new0":
        args["new0"] = None
    elif case == "q_len0":
        args["q_len"] = 0
    elif case == "width_not_16B":
        args["width"] = 100
    elif case == "odd_rope":
        args["d_rope"] = 63
    elif case == "rope_too_wide":
        args["d_rope"] = 128
    elif case == "rope_without_pool":
        kv.rope_pool = None
    elif case == "values_without_pool":
        kv.pool1 = None
    elif case == "page_not_pow2":
        kv.page_size = 48
    elif case == "unaligned_new0":
        args["new0"] = 0x600008
    elif case == "neg_stride":
        kv.token_stride = -1024
    st = binding.attn_kv_append(kv, args["q_len"], args["heads"], args["width"], args["new0"],
                                args["new1"], args["d_rope"], args["new_rope"], args["theta"],
                                None)
    assert st == binding.ATTN_ERR_INVALID_ARG, case


def test_launch_argument_plan_capacity():
    # 3 * batch + chunks int32 must fit ATTN_PLAN_INLINE_MAX
    st, plan, items, info = _plan([5000, 100, 7], groups=8, h_q=32)
    chunks = plan.n_items // plan.n_groups
    assert plan.inline_ok == 1 and 3 * 3 + chunks <= binding.ATTN_PLAN_INLINE_MAX
    assert plan.items_host and plan.seqinfo_host
    st, plan, _, _ = _plan([8192] * 200, groups=8, h_q=32)      # 600 + 200 chunks fit
    assert plan.inline_ok == 1 and plan.n_items // plan.n_groups <= 200
    st, plan, _, _ = _plan([8192] * 267, groups=8, h_q=32)      # 801 + chunks > 800
    assert plan.inline_ok == 0


def test_launch_argument_plan_half_word_chunks():
    # batches of at most 2048 sequences split at most 32 ways take half an
    # int32 per chunk: 3 * 128 + 400 chunks = 784 words in the full form,
    # 3 * 128 + 200 in the half form; 3 * 200 + 400 does not fit either
    lens = [4096] * 128
    st, plan, items, info = _plan(lens, groups=1, h_q=16, chunk=1024)
    chunks = plan.n_items // plan.n_groups
    assert st == binding.ATTN_OK and chunks == 512 and plan.max_splits == 4
    assert 3 * 128 + chunks > binding.ATTN_PLAN_INLINE_MAX   # full form would not fit
    assert plan.inline_ok == 1                                  # half form: 640 words
    st, plan, _, _ = _plan([4096] * 200, groups=1, h_q=16, chunk=512)
    assert plan.max_splits == 8 and 3 * 200 + plan.n_items // 2 > binding.ATTN_PLAN_INLINE_MAX
    assert plan.inline_ok == 0
    # more than 32 splits: full-width chunk entries only
    st, plan, _, _ = _plan([64 * 40] * 4, groups=1, h_q=16, chunk=64)
    assert plan.max_splits == 40 and plan.inline_ok == 1        # 12 + 160 words


@pytest.mark.parametrize("kind", ["gqa", "gta", "latent"])
def test_plan_without_device_arrays_needs_inline_ok(kind):
    """Decode calls reject a plan with neither device arrays nor a fitting
    launch-argument form, or with one device array only (fake, never
    dereferenced device pointers)."""
    d = dict(gqa=128, gta=128, latent=256)[kind]
    extra = dict(d=d) if kind != "latent" else dict(d=d, plan_groups=2, groups=2)
    for fields in (dict(items=None, seqinfo=None, inline_ok=0), dict(seqinfo=None),
                   dict(items=None, seqinfo=None, items_host=None)):
        assert _fake_call(kind, plan_fields=fields, **extra) == binding.ATTN_ERR_INVALID_ARG, fields


@pytest.mark.parametrize("case", ["ok_empty", "neg_tok", "no_heads", "nope_not_32", "dc_not_64",
                                  "rope_not_8", "rope_ptr_without_width", "rope_width_without_ptr",
                                  "null_w", "unaligned_out"])
def test_absorb_query_validates_arguments(case):
    """attn_latent_absorb_query checks its arguments on the host and enqueues
    nothing on error; an empty step is accepted without a launch (fake,
    never dereferenced device pointers)."""
    a = dict(q_nope=0x600000, q_rope=0x610000, w_uk=0x620000, q_out=0x630000, n_tok=1, h_q=16,
             d_nope=128, d_c=512, d_rope=64)
    want = binding.ATTN_ERR_INVALID_ARG
    if case == "ok_empty":
        a.update(n_tok=0, q_nope=None, q_out=None)
        want = binding.ATTN_OK
    elif case == "neg_tok":
        a["n_tok"] = -1
    elif case == "no_heads":
        a["h_q"] = 0
    elif case == "nope_not_32":
        a["d_nope"] = 48
    elif case == "dc_not_64":
        a["d_c"] = 96
    elif case == "rope_not_8":
        a["d_rope"] = 4
    elif case == "rope_ptr_without_width":
        a["d_rope"] = 0
    elif case == "rope_width_without_ptr":
        a["q_rope"] = None
    elif case == "null_w":
        a["w_uk"] = None
    elif case == "unaligned_out":
        a["q_out"] = 0x630008
    st = binding.attn_latent_absorb_query(a["q_nope"], a["q_rope"], a["w_uk"], a["q_out"],
                                          a["n_tok"], a["h_q"], a["d_nope"], a["d_c"], a["d_rope"],
                                          None)
    assert st == want, case


@pytest.mark.parametrize("case", ["ok_empty", "dc_not_32", "dv_not_64", "null_out", "unaligned_in"])
def test_project_output_validates_arguments(case):
    a = dict(o_lat=0x600000, w_uv=0x620000, out=0x630000, n_tok=1, h_q=16, d_c=512, d_v=128)
    want = binding.ATTN_ERR_INVALID_ARG
    if case == "ok_empty":
        a.update(n_tok=0, out=None)
        want = binding.ATTN_OK
    elif case == "dc_not_32":
        a["d_c"] = 40
    elif case == "dv_not_64":
        a["d_v"] = 100
    elif case == "null_out":
        a["out"] = None
    elif case == "unaligned_in":
        a["o_lat"] = 0x600004
    st = binding.attn_latent_project_output(a["o_lat"], a["w_uv"], a["out"], a["n_tok"], a["h_q"],
                                            a["d_c"], a["d_v"], None)
    assert st == want, case
