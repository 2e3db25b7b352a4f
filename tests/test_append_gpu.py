"""GPU parity of the paged KV append (attn_kv_append) against the oracle.

Copied rows must be bit-exact and every other cache row untouched; RoPE
keys rotated on the way in (latent caches) are float32 rotations rounded to
the cache dtype, so they may differ from the fp64 oracle by one bfloat16
unit in the last place (or by the float32 rotation error where a rotated
pair nearly cancels).  A decode over a cache whose newest tokens were
written by the append must match the oracle on the original cache.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_amd import binding, synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = {
    "gqa": W["gqa_llama8b"].with_(batch=3, seqlen_lo=1, seqlen_hi=300, max_seqlen=320),
    "gta": W["gta_8k"].with_(batch=3, seqlen_lo=1, seqlen_hi=300, max_seqlen=320),
    "mla": W["mla"].with_(batch=3, seqlen_lo=1, seqlen_hi=300, max_seqlen=320),
    "gla2": W["gla2"].with_(batch=3, seqlen_lo=1, seqlen_hi=300, max_seqlen=320),
    "fp32": W["gqa_fp32_tiny"].with_(batch=3, seqlen_lo=1, seqlen_hi=250, max_seqlen=256,
                                     page_size=16, permute_pages=True),
}


def _new_rows(w, T, seed):
    rng = np.random.default_rng(seed)
    shape = (w.batch, T, w.groups, w.head_dim)
    r = lambda s: synth.round_bf16(rng.standard_normal(s).astype(np.float32)) \
        if w.dtype == "bf16" else rng.standard_normal(s).astype(np.float32)
    new0 = r(shape)
    new1 = r(shape) if w.kind == "gqa" else None
    newr = r((w.batch, T, w.d_rope)) if w.kind != "gqa" else None
    return new0, new1, newr


def _dev(a, dt):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("page_size", [1, 16, 64])
@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("layout", ["nhd", "hnd"])
def test_append_matches_oracle(name, page_size, T, layout):
    w = CASES[name].with_(page_size=page_size, q_len=T)
    print(f"[append] {name} P={page_size} T={T} {layout}", flush=True)
    inp = synth.make_inputs(w)
    new0, new1, newr = _new_rows(w, T, seed=page_size * 10 + T)
    theta = 10000.0 if w.kind == "latent" else 0.0   # latent caches hold rotated keys
    d = H.to_device(w, inp)
    pools = [d["pool0"], d["pool1"], d["rope"]]
    if layout == "hnd":
        pools = [None if p is None else p.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
                 for p in pools]
    dt = pools[0].dtype
    binding.kv_append(pools[0], pools[1], pools[2], d["page_table"], d["seqlens"],
                      _dev(new0, dt), _dev(new1, dt), _dev(newr, dt), rope_theta=theta)
    torch.cuda.synchronize()
    want = oracle.kv_append(inp["pool0"], inp["pool1"], inp["rope"], inp["page_table"],
                            inp["seqlens"], w.page_size, new0, new1, newr, theta, w.dtype)
    for k, (got_t, exp) in enumerate(zip(pools, want)):
        if exp is None:
            continue
        got = got_t.float().cpu().numpy()
        if k < 2 or theta <= 0:
            assert np.array_equal(got, exp.astype(np.float32)), f"{name} pool{k}"
        else:
            # rotated rows: within one bfloat16 unit of the value, plus the
            # float32 rotation's absolute error (sin/cos and the products, a
            # few 2^-20 of inputs of order 1) where the pair cancels; all
            # other rows exact
            diff = np.abs(got - exp)
            assert (diff <= 2 ** -7 * np.abs(exp) + 2 ** -14).all(), f"{name} rope max {diff.max()}"
            changed = (got != inp["rope"]).any(axis=(1, 2, 3))
            rows_written = np.zeros_like(changed)
            for b in range(w.batch):
                L = int(inp["seqlens"][b])
                for t in range(T):
                    if L - T + t >= 0:
                        rows_written[inp["page_table"][b, (L - T + t) // w.page_size]] = True
            assert not (changed & ~rows_written).any(), "rows outside the append changed"


@pytest.mark.parametrize("name", ["gqa", "gta", "mla", "gla2"])
@pytest.mark.parametrize("page_size", [1, 64])
def test_decode_after_append(name, page_size):
    """Erase the newest T rows of every sequence, write them back with the
    append, and decode: the result must match the oracle on the original
    cache."""
    T = 2
    w = CASES[name].with_(page_size=page_size, q_len=T, causal=True, seqlen_lo=T)
    print(f"[append+decode] {name} P={page_size}", flush=True)
    inp = synth.make_inputs(w)
    new = {"pool0": [], "pool1": [], "rope": []}
    erased = {k: (None if inp[k] is None else inp[k].copy()) for k in new}
    for k in new:
        if inp[k] is None:
            continue
        rows = np.zeros((w.batch, T) + inp[k].shape[2:], np.float32)
        for b in range(w.batch):
            L = int(inp["seqlens"][b])
            for t in range(T):
                pos = L - T + t
                pg, sl = inp["page_table"][b, pos // w.page_size], pos % w.page_size
                rows[b, t] = inp[k][pg, sl]
                erased[k][pg, sl] = np.nan
        new[k] = rows
    d = H.to_device(w, dict(inp, pool0=erased["pool0"], pool1=erased["pool1"], rope=erased["rope"]))
    dt = d["pool0"].dtype
    newr = None if inp["rope"] is None else new["rope"][:, :, 0, :]
    binding.kv_append(d["pool0"], d["pool1"], d["rope"], d["page_table"], d["seqlens"],
                      _dev(new["pool0"], dt), _dev(new["pool1"] if inp["pool1"] is not None
                                                   else None, dt), _dev(newr, dt))
    out, lse, _ = H.run(w, d)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(w, inp)
    H.compare(H.to_np(out), H.to_np(lse), ref, ref_lse, H.value_max(w, inp), f"{name}/append")


@pytest.mark.parametrize("name", ["gqa", "mla"])
def test_append_skips_rows_outside_the_table(name):
    """Rows the append cannot place are skipped, leaving the pools
    untouched: a position past the sequence's page-table row, a page-table
    entry of -1, and a page id past the pools.  The one well-formed
    sequence is written as the oracle writes it."""
    T = 2
    w = CASES[name].with_(batch=4, q_len=T, seqlen_lo=100, seqlen_hi=200, max_seqlen=256,
                          page_size=16)
    print(f"[append-bounds] {name}", flush=True)
    inp = synth.make_inputs(w)
    new0, new1, newr = _new_rows(w, T, seed=7)
    theta = 10000.0 if w.kind == "latent" else 0.0
    n_pages = inp["pool0"].shape[0]
    max_pages = inp["page_table"].shape[1]
    table = inp["page_table"].copy()
    seqlens = inp["seqlens"].copy()
    seqlens[1] = max_pages * w.page_size + T + 1       # past the table row
    for b, bad in ((2, -1), (3, n_pages + 5)):          # unassigned / past the pools
        L = int(seqlens[b])
        for t in range(T):
            table[b, (L - T + t) // w.page_size] = bad
    d = H.to_device(w, inp)
    d["page_table"] = torch.from_numpy(table).cuda()
    d["seqlens"] = torch.from_numpy(seqlens).cuda()
    dt = d["pool0"].dtype
    binding.kv_append(d["pool0"], d["pool1"], d["rope"], d["page_table"], d["seqlens"],
                      _dev(new0, dt), _dev(new1, dt), _dev(newr, dt), rope_theta=theta)
    torch.cuda.synchronize()
    # expected: only sequence 0's rows written
    want = oracle.kv_append(inp["pool0"], inp["pool1"], inp["rope"], table[:1], seqlens[:1],
                            w.page_size, new0[:1], None if new1 is None else new1[:1],
                            None if newr is None else newr[:1], theta, w.dtype)
    for k, (got_t, exp) in enumerate(zip((d["pool0"], d["pool1"], d["rope"]), want)):
        if exp is None:
            continue
        got = got_t.float().cpu().numpy()
        if k < 2 or theta <= 0:
            assert np.array_equal(got, exp.astype(np.float32)), f"{name} pool{k}"
        else:
            diff = np.abs(got - exp)
            assert (diff <= 2 ** -7 * np.abs(exp) + 2 ** -14).all(), f"{name} rope"
