"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases run the oracle on every output; they span several 64-key tiles
with ragged tails, forced and automatic splits, every variant and the edge
cases.  Full-size workloads (the launch configuration the benchmark times)
are checked on sampled sequences plus properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_amd import binding, synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def small(base, **kw):
    return W[base].with_(**kw)


SMALL = {
    "gqa_fp32_tiny": W["gqa_fp32_tiny"],
    "gqa_fp32_d128": small("gqa_fp32_tiny", head_dim=128, seqlen_lo=1, seqlen_hi=500,
                           page_size=16, max_seqlen=512, permute_pages=True, batch=3),
    "gqa_llama8b": small("gqa_llama8b", batch=4, seqlen_lo=1, seqlen_hi=700, max_seqlen=704),
    "gqa_d64_mqa": small("gqa_llama8b", batch=3, groups=1, head_dim=64, seqlen_lo=30,
                         seqlen_hi=300, max_seqlen=320, softmax_scale=0.125),
    "gqa_mha": small("gqa_llama8b", batch=2, h_q=8, groups=8, seqlen_lo=60, seqlen_hi=260,
                     max_seqlen=320),
    "gqa_causal3": small("gqa_llama8b", batch=3, q_len=3, causal=True, seqlen_lo=3,
                         seqlen_hi=400, max_seqlen=448),
    "gta_8k": small("gta_8k", batch=3, seqlen_lo=100, seqlen_hi=1000, max_seqlen=1024),
    "gqa4_8k": small("gqa4_8k", batch=3, seqlen_lo=100, seqlen_hi=1000, max_seqlen=1024),
    "gta_causal2": small("gta_8k", batch=2, q_len=2, causal=True, seqlen_lo=2,
                         seqlen_hi=300, max_seqlen=320),
    "mla": small("mla", batch=2, seqlen_lo=64, seqlen_hi=600, max_seqlen=640),
    "gla2": small("gla2", batch=2, seqlen_lo=64, seqlen_hi=600, max_seqlen=640),
    "gla2_spec4": small("gla2_spec4_128k", batch=2, seqlen_lo=4, seqlen_hi=700, max_seqlen=704),
    "mla_spec4": small("mla_spec4_128k", batch=2, seqlen_lo=4, seqlen_hi=500, max_seqlen=512),
    "gla2_h32": small("gla2", batch=2, h_q=32, seqlen_lo=1, seqlen_hi=300, max_seqlen=320),
    # sweep points: q_len up to 8, per-device shares of fewer heads
    "gqa_q8": small("gqa_llama8b", batch=2, q_len=8, causal=True, seqlen_lo=8, seqlen_hi=400,
                    max_seqlen=448),
    "mla_q8": small("mla", batch=2, q_len=8, causal=True, seqlen_lo=8, seqlen_hi=300,
                    max_seqlen=320),
    "gla2_q2": small("gla2", batch=2, q_len=2, causal=True, seqlen_lo=2, seqlen_hi=500,
                     max_seqlen=512),
    "gla8_share": small("gla2", batch=3, h_q=16, groups=1, seqlen_lo=1, seqlen_hi=600,
                        max_seqlen=640),
    "mla_h16": small("mla", batch=2, h_q=16, seqlen_lo=1, seqlen_hi=400, max_seqlen=448),
    # 33-64 rows per group (four row tiles per wave): full, ragged (48, 40
    # rows), head dim 64, single-token-row pages; past 64 rows: the general kernel
    "gqa4_q8": small("gqa4_8k", batch=2, q_len=8, causal=True, seqlen_lo=8, seqlen_hi=400,
                     max_seqlen=448),
    "gta_q6": small("gta_8k", batch=2, q_len=6, causal=True, seqlen_lo=6, seqlen_hi=400,
                    max_seqlen=448),
    "gqa_q10_p4": small("gqa_llama8b", batch=2, q_len=10, causal=True, page_size=4,
                        seqlen_lo=10, seqlen_hi=300, max_seqlen=320),
    "gqa_d64_q16": small("gqa_llama8b", batch=2, head_dim=64, q_len=16, causal=True,
                         seqlen_lo=16, seqlen_hi=300, max_seqlen=320, softmax_scale=0.125),
    "gta_q8_p1": small("gta_8k", batch=2, q_len=8, causal=True, page_size=1, seqlen_lo=8,
                       seqlen_hi=200, max_seqlen=200),
    "gqa4_q12": small("gqa4_8k", batch=2, q_len=12, causal=True, seqlen_lo=12,
                      seqlen_hi=300, max_seqlen=320),
    # 64-row groups on whole slices: one workgroup of two row halves
    "gta_q8": small("gta_8k", batch=2, q_len=8, causal=True, seqlen_lo=8, seqlen_hi=400,
                    max_seqlen=448),
    "gqa4_q8_p16": small("gqa4_8k", batch=2, q_len=8, causal=True, page_size=16, seqlen_lo=8,
                         seqlen_hi=400, max_seqlen=448),
    # latent groups whose rows are no multiple of 16: 24 rows (one partial
    # row tile), 60 (two row tiles, the last partial), 144 (row blocks of
    # 64, 64 and 16), and 3 rows in each of four GLA groups
    "mla_h24": small("mla", batch=3, h_q=24, seqlen_lo=1, seqlen_hi=500, max_seqlen=512),
    "gla2_h40_q3": small("gla2", batch=2, h_q=40, q_len=3, causal=True, seqlen_lo=3,
                         seqlen_hi=400, max_seqlen=448),
    "mla_h72_q2": small("mla", batch=2, h_q=72, q_len=2, causal=True, seqlen_lo=2,
                        seqlen_hi=300, max_seqlen=320),
    "gla4_h12": small("gla2", batch=3, h_q=12, groups=4, seqlen_lo=1, seqlen_hi=400,
                      max_seqlen=448),
    # 256-wide latent groups of more than 64 rows (128-row workgroups, the
    # pipelined schedule): 68 rows (the second row half holds 4), 96 rows,
    # 192 rows (a full and a half-empty workgroup), 512 rows
    "gla2_h68_q2": small("gla2", batch=2, h_q=68, q_len=2, causal=True, seqlen_lo=2,
                         seqlen_hi=500, max_seqlen=512),
    "gla2_h96_q2": small("gla2", batch=3, h_q=96, q_len=2, causal=True, seqlen_lo=2,
                         seqlen_hi=400, max_seqlen=448),
    "gla2_q3": small("gla2", batch=2, q_len=3, causal=True, seqlen_lo=3, seqlen_hi=600,
                     max_seqlen=640),
    "gla2_q8": small("gla2", batch=2, q_len=8, causal=True, seqlen_lo=8, seqlen_hi=300,
                     max_seqlen=320),
    # paired GTA groups: three pairs, and groups of 4 rows (half a row tile)
    "gta_h6": small("gta_8k", batch=2, h_q=48, groups=6, seqlen_lo=1, seqlen_hi=700,
                    max_seqlen=704),
    "gta_g4": small("gta_8k", batch=3, h_q=8, groups=2, seqlen_lo=1, seqlen_hi=500,
                    max_seqlen=512),
}


def _check(w, inp, tag, **kw):
    d = H.to_device(w, inp)
    out, lse, plan = H.run(w, d, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(w, inp)
    H.compare(H.to_np(out), H.to_np(lse), ref, ref_lse, H.value_max(w, inp), tag)
    return out, lse, plan


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("chunk", [0, 64, 192])
def test_small_parity(name, chunk):
    w = SMALL[name]
    print(f"[parity] {name} chunk={chunk}", flush=True)
    inp = synth.make_inputs(w)
    _check(w, inp, f"{name}/chunk{chunk}", chunk_tokens=chunk)


@pytest.mark.parametrize("name", ["gqa_llama8b", "gta_8k", "gla2_spec4", "mla"])
def test_nan_sentinels_in_unused_slots(name):
    w = SMALL[name]
    print(f"[nan] {name}", flush=True)
    inp = synth.make_inputs(w, tail_fill=np.nan, extra_pages=7)
    _check(w, inp, f"{name}/nan", chunk_tokens=128)


def _head_major(d):
    """The same logical pools over head-major storage [pages][heads][page][width]."""
    for k in ("pool0", "pool1", "rope"):
        if d[k] is not None:
            d[k] = d[k].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    return d


# every power-of-two page size: single-token and other pages smaller than a
# 16-key slice (per-row page ids), pages of 16..32 tokens (one id per slice
# in the GQA/GTA kernel, per-row ids in the latent one), and whole tiles
PAGE_NAMES = ["gqa_llama8b", "gqa_d64_mqa", "gta_8k", "gta_causal2", "mla", "gla2", "gla2_spec4",
              "gla2_h32"]


@pytest.mark.parametrize("name", PAGE_NAMES)
@pytest.mark.parametrize("page_size", [1, 2, 4, 8, 16, 32, 128, 256])
def test_page_sizes(name, page_size):
    w = SMALL[name].with_(page_size=page_size)
    chunk = 192 if page_size in (2, 32) else 0
    print(f"[page] {name} P={page_size} chunk={chunk}", flush=True)
    _check(w, synth.make_inputs(w), f"{name}/P{page_size}", chunk_tokens=chunk)


@pytest.mark.parametrize("name", ["gqa_llama8b", "gta_8k", "mla", "gla2_spec4"])
@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_small_pages_head_major_and_nan_tails(name, page_size):
    """Head-major pools (other strides) and NaN in every unused page slot
    and unreferenced page."""
    w = SMALL[name].with_(page_size=page_size)
    print(f"[page-hnd] {name} P={page_size}", flush=True)
    inp = synth.make_inputs(w, tail_fill=np.nan, extra_pages=5)
    d = _head_major(H.to_device(w, inp))
    out, lse, _ = H.run(w, d, chunk_tokens=128)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(w, inp)
    H.compare(H.to_np(out), H.to_np(lse), ref, ref_lse, H.value_max(w, inp), f"{name}/hnd/P{page_size}")


def _slot_major(t, n_pages):
    """t's pages as the first pages of a slot-major pool [slot][n_pages][heads]
    [width] (token stride n_pages * heads * width elements)."""
    P, Hh, Wd = t.shape[1:]
    big = torch.empty((P, n_pages, Hh, Wd), dtype=t.dtype, device=t.device)
    view = big.permute(1, 0, 2, 3)
    view[: t.shape[0]] = t
    return view


# (workload, page size, token stride in bytes to reach): a 16-row slice's
# per-lane offsets of the GQA/GTA streaming kernel pass 2^32 bytes, a 64-row
# tile's offsets of the latent one 2^31; both then take the general kernel
@pytest.mark.parametrize("name,page_size,stride_bytes", [("gqa_llama8b", 16, 2 ** 32 // 15),
                                                          ("gta_8k", 16, 2 ** 32 // 15),
                                                          ("mla", 64, 2 ** 31 // 63)])
def test_token_strides_past_32_bit_offsets(name, page_size, stride_bytes):
    w = SMALL[name].with_(page_size=page_size)
    print(f"[stride] {name} P={page_size}", flush=True)
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    row = d["pool0"].shape[2] * d["pool0"].shape[3] * 2
    n_pages = -(-stride_bytes // row) + 1
    assert n_pages * row > stride_bytes and n_pages >= d["pool0"].shape[0]
    d["pool0"] = _slot_major(d["pool0"], n_pages)
    if d["pool1"] is not None:
        d["pool1"] = _slot_major(d["pool1"], n_pages)
    out, lse, _ = H.run(w, d, chunk_tokens=128)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(w, inp)
    H.compare(H.to_np(out), H.to_np(lse), ref, ref_lse, H.value_max(w, inp), f"{name}/stride")
    del d
    torch.cuda.empty_cache()


def _random_cases(n=60, seed=2026):
    """Seeded random shapes inside the supported envelope (the same list on
    every run): kind, head and latent widths, group counts and sizes, q_len,
    page size, lengths, chunk length and pool layout."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ("gqa", "gta", "latent")[i % 3]
        q_len = int(rng.choice([1, 1, 2, 3, 5, 8]))
        if kind == "gqa":
            d = int(rng.choice([64, 128]))
            groups, g = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
            base = W["gqa_llama8b"].with_(head_dim=d, softmax_scale=d ** -0.5,
                                          dtype="fp32" if rng.random() < 0.2 else "bf16")
        elif kind == "gta":
            groups, g = int(rng.choice([1, 2, 4, 6])), int(rng.choice([1, 2, 4, 5, 8]))
            base = W["gta_8k"]
        else:
            d = int(rng.choice([256, 512]))
            groups, g = int(rng.choice([1, 2, 4])), int(rng.choice([1, 3, 8, 16, 32, 48]))
            base = W["gla2"].with_(head_dim=d, softmax_scale=(d + 64) ** -0.5)
        page = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
        hi = int(rng.integers(q_len + 1, 700))
        w = base.with_(name=f"rand{i}", batch=int(rng.integers(1, 5)), q_len=q_len,
                       causal=q_len > 1, h_q=groups * g, groups=groups, page_size=page,
                       seqlen_lo=q_len, seqlen_hi=hi, max_seqlen=hi + int(rng.integers(0, 64)),
                       permute_pages=True, seed=1000 + i)
        out.append((w, int(rng.choice([0, 64, 128, 192])), bool(rng.random() < 0.3)))
    return out


RANDOM_CASES = _random_cases()


@pytest.mark.parametrize("case", range(len(RANDOM_CASES)))
def test_random_shapes(case):
    w, chunk, head_major = RANDOM_CASES[case]
    print(f"[random] {w.name} {w.kind} {w.dtype} d={w.head_dim} G={w.groups} h_q={w.h_q} "
          f"T={w.q_len} P={w.page_size} chunk={chunk} head_major={head_major}", flush=True)
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    if head_major:
        d = _head_major(d)
    out, lse, _ = H.run(w, d, chunk_tokens=chunk)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(w, inp)
    H.compare(H.to_np(out), H.to_np(lse), ref, ref_lse, H.value_max(w, inp), w.name)


def test_empty_and_single_token_sequences():
    w = SMALL["gqa_llama8b"]
    inp = synth.make_inputs(w, seqlens=np.array([0, 1, 65, 0], dtype=np.int32))
    out, lse, _ = _check(w, inp, "empty", chunk_tokens=64)
    o = H.to_np(out)
    assert (o[0] == 0).all() and (o[3] == 0).all()
    assert np.isneginf(H.to_np(lse)[[0, 3]]).all()


def test_minimum_causal_length():
    w = SMALL["gla2_spec4"]
    inp = synth.make_inputs(w, seqlens=np.array([4, 5], dtype=np.int32))
    _check(w, inp, "causal-min")


def test_physical_permutation_is_bit_exact():
    w = SMALL["gta_8k"]
    inp = synth.make_inputs(w)
    out1, lse1, _ = _check(w, inp, "perm-a", chunk_tokens=128)
    # same logical cache under a different physical page permutation
    rng = np.random.default_rng(2024)
    n = inp["pool0"].shape[0]
    perm = rng.permutation(n)
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["pool0"] = inp["pool0"][perm]
    inp2["rope"] = inp["rope"][perm]
    t = inp["page_table"].copy()
    t[t >= 0] = inv[t[t >= 0]]
    inp2["page_table"] = t
    out2, lse2, _ = H.run(w, H.to_device(w, inp2), chunk_tokens=128)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_run_to_run_determinism():
    w = SMALL["mla"]
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    o1, l1, plan = H.run(w, d, chunk_tokens=128)
    o2, l2, _ = H.run(w, d, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["gqa_llama8b", "gla2_spec4"])
def test_deferred_merge_matches_fused_call(name):
    w = SMALL[name]
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    o1, l1, plan = H.run(w, d, chunk_tokens=64)
    o2, l2, plan2, ws = binding.decode(
        w.kind, d["q"], d["pool0"], d["pool1"], d["rope"], d["page_table"], d["seqlens"],
        d["seqlens_host"], groups=w.groups, scale=w.softmax_scale, causal=w.causal,
        rope_theta=w.rope_theta, d_rope=w.d_rope, plan=plan, defer_merge=True)
    binding.merge(plan, o2, l2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gather_probe_recovers_physical_rows():
    """V rows encode their own (page, slot) as exact integers; a query that
    dominates one chosen key must return exactly that key's code."""
    w = W["gqa_fp32_tiny"].with_(batch=2, groups=1, h_q=1, head_dim=64, seqlen_lo=200,
                                 seqlen_hi=200, page_size=16, max_seqlen=256,
                                 permute_pages=True, softmax_scale=1.0)
    inp = synth.make_inputs(w)
    kp = np.zeros_like(inp["pool0"])
    vp = np.zeros_like(inp["pool1"])
    npages = kp.shape[0]
    for pg in range(npages):
        for sl in range(w.page_size):
            vp[pg, sl, 0, :] = pg * 1000 + sl
    targets = [137, 41]
    q = np.zeros_like(inp["q"])
    for b, tgt in enumerate(targets):
        pg = inp["page_table"][b, tgt // w.page_size]
        kp[pg, tgt % w.page_size, 0, 0] = 1.0
        q[b, 0, 0, 0] = 200.0
    inp.update(pool0=kp, pool1=vp, q=q)
    out, _, _ = H.run(w, H.to_device(w, inp), chunk_tokens=64)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for b, tgt in enumerate(targets):
        pg = inp["page_table"][b, tgt // w.page_size]
        assert np.all(np.rint(o[b, 0, 0]) == pg * 1000 + tgt % w.page_size)


def _probe_codes(pg, sl):
    """Exact bf16 integers (< 256) that name a physical row."""
    return np.array([pg % 256, pg // 256, sl % 256, 7.0])


@pytest.mark.parametrize("kind", ["gqa", "gta", "mla", "gla2"])
@pytest.mark.parametrize("page_size", [1, 4, 16, 64])
def test_gather_probe_streaming_kernels(kind, page_size):
    """bf16 streaming kernels: values encode their own physical (page, slot)
    as exact integers and one key per sequence dominates its query by 128
    (natural log units: every other weight underflows to exactly zero), so
    the output must name exactly that row."""
    base = {"gqa": "gqa_llama8b", "gta": "gta_8k", "mla": "mla", "gla2": "gla2"}[kind]
    w = SMALL[base].with_(batch=3, seqlen_lo=300, seqlen_hi=700, max_seqlen=768,
                          page_size=page_size, q_std=0.0)
    inp = synth.make_inputs(w)
    p0 = np.zeros_like(inp["pool0"])
    p1 = None if inp["pool1"] is None else np.zeros_like(inp["pool1"])
    rp = None if inp["rope"] is None else np.zeros_like(inp["rope"])
    vals = p1 if kind == "gqa" else p0   # the values the call attends over
    for pg in range(p0.shape[0]):
        for sl in range(w.page_size):
            vals[pg, sl, :, :4] = _probe_codes(pg, sl)
    L = inp["seqlens"]
    targets = [int(L[0]) - 1, 3, int(L[2]) // 2]
    q = np.zeros_like(inp["q"])
    for b, tgt in enumerate(targets):
        pg = inp["page_table"][b, tgt // w.page_size]
        sl = tgt % w.page_size
        if kind == "gqa":
            p0[pg, sl, :, 5] = 1.0
            q[b, :, :, 5] = 128.0
        elif kind == "gta":
            # the key's non-RoPE half is the tied row's first half
            p0[pg, sl, :, 5] = 1.0
            q[b, :, :, 5] = 128.0
        else:
            rp[pg, sl, 0, 0] = 1.0        # pre-rotated RoPE key
            q[b, :, :, w.head_dim] = 128.0
    inp.update(pool0=p0, pool1=p1, rope=rp, q=q)
    w = w.with_(softmax_scale=1.0)
    out, _, _ = H.run(w, H.to_device(w, inp), chunk_tokens=128)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    for b, tgt in enumerate(targets):
        pg = int(inp["page_table"][b, tgt // w.page_size])
        want = _probe_codes(pg, tgt % w.page_size)
        got = o[b, :, :, :4].reshape(-1, 4)
        assert np.all(got == want), f"{kind} P={page_size} seq {b}: {got[0]} != {want}"


# ------------------------------------------------------------ full size
FULL = ["gqa_fp32_tiny", "gqa_llama8b", "gta_8k", "mla", "gla2", "gla2_spec4_128k",
        "gqa_llama8b_8k", "gqa4_8k", "mla_spec4_128k", "gqa_llama8b@P1", "gla2@P1",
        "gta_8k@P1", "gqa4_8k@P1"]

# (pool layout, plan delivery): token-major or head-major pools; the plan as
# device arrays with the merge launched by the decode call, or the way the
# benchmark runs it (in the launch arguments when it fits, the decode
# deferring the merge to a separate attn_decode_merge launch)
FULL_MODES = [("nhd", "device"), ("hnd", "device"), ("nhd", "bench"), ("hnd", "bench")]


def _run_mode(w, d, layout, mode):
    dd = _head_major(dict(d)) if layout == "hnd" else d
    if mode == "device":
        out, lse, plan = H.run(w, dd)
        return out, lse, plan
    sh = binding.shape(w.kind, binding.ATTN_BF16 if w.dtype == "bf16" else binding.ATTN_FP32,
                       w.batch, w.q_len, w.h_q, w.groups, w.head_dim, w.d_rope, w.page_size,
                       w.causal)
    probe = binding.DevicePlan(sh, d["seqlens_host"], d["q"].device)
    plan = binding.DevicePlan(sh, d["seqlens_host"], d["q"].device,
                              inline=bool(probe.plan.inline_ok))
    out, lse, plan, ws = binding.decode(
        w.kind, dd["q"], dd["pool0"], dd["pool1"], dd["rope"], dd["page_table"], dd["seqlens"],
        dd["seqlens_host"], groups=w.groups, scale=w.softmax_scale, causal=w.causal,
        rope_theta=w.rope_theta, d_rope=w.d_rope, plan=plan, defer_merge=True)
    binding.merge(plan, out, lse, ws)
    return out, lse, plan


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    """Every benchmark workload at full size, in every pool layout and plan
    delivery, including exactly the launch configuration the benchmark
    times: properties on every row, and sampled sequences against the
    oracle (computed once)."""
    base, _, pg = name.partition("@P")
    w = W[base] if not pg else W[base].with_(page_size=int(pg))
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    L = inp["seqlens"]
    pick = sorted({int(np.argmax(L)), int(np.argmin(L)), int(np.random.default_rng(0).integers(len(L)))})
    ref, ref_lse = oracle.decode(w, inp, batch_index=pick)
    vmax_all, vmax = H.value_max(w, inp), H.value_max(w, inp, pick)
    first = None
    for layout, mode in FULL_MODES:
        print(f"[full] {name} {layout} {mode}", flush=True)
        out, lse, plan = _run_mode(w, d, layout, mode)
        torch.cuda.synchronize()
        o, l = H.to_np(out), H.to_np(lse)
        # properties on every row: finite, and each output is a convex
        # combination of its values, so bounded by the largest |value|
        assert np.isfinite(o).all() and np.isfinite(l).all()
        assert np.abs(o).max() <= vmax_all * (1 + 2 ** -7)
        H.compare(o[pick], l[pick], ref, ref_lse, vmax, f"{name}/{layout}/{mode}")
        # the same plan and layout-independent arithmetic: one result
        if first is None:
            first = (out, lse)
        else:
            assert torch.equal(first[0], out) and torch.equal(first[1], lse), (layout, mode)
        del out, lse, plan
    del d
    torch.cuda.empty_cache()


# head-major pools with whole pages of 64 tokens and more, in both plan
# deliveries: the paired-GTA kernel (even groups of at most 8 rows) and the
# latent kernel's whole-tile path, as the benchmark runs them
HEAD_MAJOR = ["gta_8k", "gta_h6", "gta_g4", "gqa_llama8b", "gqa4_8k", "gla2", "gla2_spec4", "mla",
              "mla_spec4", "gla2_h40_q3", "mla_h72_q2", "gla8_share"]


@pytest.mark.parametrize("name", HEAD_MAJOR)
@pytest.mark.parametrize("page_size", [64, 128])
@pytest.mark.parametrize("inline", [False, True])
def test_head_major_whole_pages(name, page_size, inline):
    w = SMALL[name].with_(page_size=page_size)
    print(f"[hnd] {name} P={page_size} inline={inline}", flush=True)
    inp = synth.make_inputs(w, tail_fill=np.nan, extra_pages=3)
    d = _head_major(H.to_device(w, inp))
    ref, ref_lse = oracle.decode(w, inp)
    for chunk in (0, 128):
        out, lse, _ = H.run(w, d, chunk_tokens=chunk, inline_plan=inline)
        torch.cuda.synchronize()
        H.compare(H.to_np(out), H.to_np(lse), ref, ref_lse, H.value_max(w, inp),
                  f"{name}/hnd/P{page_size}/inline{inline}/chunk{chunk}")


@pytest.mark.parametrize("name", ["mla", "gla2", "gla2_spec4"])
def test_scores_far_above_first_tile(name):
    """Scores that grow by far more than 2^64 (log2 units) after the first
    64-key tile: the streaming latent kernel must take its second pass with
    the true maxima and still match the oracle."""
    w = SMALL[name].with_(batch=2, seqlen_lo=300, seqlen_hi=300, max_seqlen=320,
                          softmax_scale=1.0)
    inp = synth.make_inputs(w)
    # keys of later tokens get a large component along the queries' first axis
    q = inp["q"].copy()
    q[..., 0] = 4.0
    lat = inp["pool0"].copy()
    for b in range(w.batch):
        for i in range(300):
            pg = inp["page_table"][b, i // w.page_size]
            lat[pg, i % w.page_size, :, 0] = 0.0 if i < 64 else synth.round_bf16(
                np.array([min(40.0, i / 4.0)], np.float32))[0]
    inp.update(q=synth.round_bf16(q), pool0=lat)
    _check(w, inp, f"{name}/far", chunk_tokens=0)


@pytest.mark.parametrize("name", ["gqa_llama8b", "gta_8k", "gta_h6", "gla2", "mla_spec4", "gqa4_q8",
                                  "gla2_h40_q3", "mla_h72_q2"])
def test_fused_merge_counters_return_to_zero(name):
    """Split rows are merged inside the streaming kernels by the last split
    workgroup of each row block, counted with wrapping counters: after every
    call the counters are back to zero, one counter array serves consecutive
    plans, and the result equals the separate merge launch bit for bit."""
    w = SMALL[name]
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    ref, ref_lse = oracle.decode(w, inp)
    vmax = H.value_max(w, inp)
    kw = dict(groups=w.groups, scale=w.softmax_scale, causal=w.causal,
              rope_theta=w.rope_theta, d_rope=w.d_rope)
    args = (w.kind, d["q"], d["pool0"], d["pool1"], d["rope"], d["page_table"], d["seqlens"],
            d["seqlens_host"])
    counters = None
    for chunk in (64, 192, 128):
        plan = binding.DevicePlan(
            binding.shape(w.kind, binding.ATTN_BF16, w.batch, w.q_len, w.h_q, w.groups,
                          w.head_dim, w.d_rope, w.page_size, w.causal),
            d["seqlens_host"], d["q"].device, chunk_tokens=chunk, fused_merge=True)
        if counters is None:
            counters = plan.counters
        plan.plan.counters = counters.data_ptr()  # one array for every plan
        out, lse, _, _ = binding.decode(*args, plan=plan, **kw)
        sep, sep_lse, _, _ = binding.decode(*args, chunk_tokens=chunk, fused_merge=False, **kw)
        torch.cuda.synchronize()
        print(f"[fused] {name} chunk={chunk} splits={plan.plan.max_splits}", flush=True)
        assert plan.plan.max_splits > 1
        H.compare(H.to_np(out), H.to_np(lse), ref, ref_lse, vmax, f"{name}/fused{chunk}")
        assert torch.equal(out, sep) and torch.equal(lse, sep_lse)
        assert int(counters.count_nonzero()) == 0


@pytest.mark.parametrize("name", ["gqa_llama8b", "gta_causal2", "mla", "gla2_spec4",
                                  "gqa_fp32_d128", "gqa_mha", "gla8_share"])
@pytest.mark.parametrize("page_size", [1, 64])
def test_launch_argument_plan_matches_device_plan(name, page_size):
    """A plan passed in the kernels' launch arguments (no device copy) gives
    bit-identical results, for the decode call and for a deferred merge."""
    w = SMALL[name].with_(page_size=page_size) if w_pages_ok(name) else SMALL[name]
    print(f"[inline] {name} P={w.page_size}", flush=True)
    d = H.to_device(w, synth.make_inputs(w))
    o1, l1, _ = H.run(w, d, chunk_tokens=128)
    o2, l2, plan2 = H.run(w, d, chunk_tokens=128, inline_plan=True)
    assert plan2.plan.items is None and plan2.plan.seqinfo is None
    o3, l3, plan3, ws = binding.decode(
        w.kind, d["q"], d["pool0"], d["pool1"], d["rope"], d["page_table"], d["seqlens"],
        d["seqlens_host"], groups=w.groups, scale=w.softmax_scale, causal=w.causal,
        rope_theta=w.rope_theta, d_rope=w.d_rope, chunk_tokens=128, defer_merge=True,
        inline_plan=True)
    binding.merge(plan3, o3, l3, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


# launch-argument forms: full-width chunk entries (a sequence split more
# than 32 ways) and half-word ones (an odd chunk count included)
@pytest.mark.parametrize("name,lo,hi,form", [("gqa_llama8b", 4000, 4160, 1), ("mla", 2200, 2500, 1),
                                             ("gla2_spec4", 2100, 2200, 1),
                                             ("gqa_llama8b", 100, 700, 2), ("gla2", 300, 900, 2)])
def test_launch_argument_plan_forms(name, lo, hi, form):
    """Plans packed into the launch arguments with full-width or half-word
    chunk entries give the device plan's results bit for bit, for the
    decode and for a deferred merge."""
    w = SMALL[name].with_(batch=3, seqlen_lo=lo, seqlen_hi=hi, max_seqlen=hi + 64)
    d = H.to_device(w, synth.make_inputs(w))
    o1, l1, plan1 = H.run(w, d, chunk_tokens=64)
    chunks = plan1.plan.n_items // plan1.plan.n_groups
    print(f"[inline form] {name} splits={plan1.plan.max_splits} chunks={chunks}", flush=True)
    assert (plan1.plan.max_splits > 32) == (form == 1)
    if form == 2:
        assert chunks % 2 == 1 or name != "gla2"   # the last half word half used
    o2, l2, plan2 = H.run(w, d, chunk_tokens=64, inline_plan=True)
    assert plan2.plan.items is None and plan2.plan.seqinfo is None
    o3, l3, plan3, ws = binding.decode(
        w.kind, d["q"], d["pool0"], d["pool1"], d["rope"], d["page_table"], d["seqlens"],
        d["seqlens_host"], groups=w.groups, scale=w.softmax_scale, causal=w.causal,
        rope_theta=w.rope_theta, d_rope=w.d_rope, chunk_tokens=64, defer_merge=True,
        inline_plan=True)
    binding.merge(plan3, o3, l3, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def w_pages_ok(name):
    # fp32 shapes run on the general kernel at their own page size
    return SMALL[name].dtype == "bf16"


@pytest.mark.parametrize("page_size,chunk", [(64, 64), (1, 128), (16, 128)])
def test_work_queue_matches_fixed_assignment(page_size, chunk):
    """More items than resident workgroups: with a work-queue counter the GQA
    kernel hands out items dynamically; the result is bit-identical to the
    fixed assignment, matches the oracle, and the counter returns to zero
    after each call (two calls in a row share it)."""
    w = SMALL["gqa_llama8b"].with_(batch=9, seqlen_lo=500, seqlen_hi=2000, max_seqlen=2048,
                                   page_size=page_size)
    print(f"[queue] P={page_size} chunk={chunk}", flush=True)
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    o1, l1, plan1 = H.run(w, d, chunk_tokens=chunk)
    assert plan1.plan.n_items > 512
    queue = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rep in range(2):
        o2, l2, _ = H.run(w, d, chunk_tokens=chunk, queue=queue)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), rep
        assert int(queue.item()) == 0, rep
    ref, ref_lse = oracle.decode(w, inp)
    H.compare(H.to_np(o2), H.to_np(l2), ref, ref_lse, H.value_max(w, inp), "queue")


def test_work_queue_full_size():
    w = W["gqa_llama8b"]
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    queue = torch.zeros(1, dtype=torch.int32, device="cuda")
    o1, l1, _ = H.run(w, d)
    o2, l2, plan = H.run(w, d, queue=queue)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and int(queue.item()) == 0
    del d
    torch.cuda.empty_cache()
