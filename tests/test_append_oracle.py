"""Pins for the oracle's paged KV append (CPU only).

* Building a cache one decode step at a time with the append oracle gives
  back exactly the cache the seeded generator laid out directly (its page
  table and physical rows), for every kind and page size: the positions
  L_b - T + t, the page / slot mapping and the per-pool copies.
* Rotated latent RoPE keys equal the complex-multiplication form of the
  rotation at their position, rounded to bfloat16.
* The bfloat16 rounding equals torch's float32 -> bfloat16 conversion.
* Plausible mistakes planted in copies of the append fail these pins.
"""
import numpy as np
import pytest
import torch

from oracle import append as app
from decode_attention_kv_amd import synth


def tiny(kind, **kw):
    base = dict(name="tiny", kind=kind, dtype="bf16", batch=3, q_len=1, h_q=8, groups=2,
                head_dim=16, d_rope=0, seqlen_lo=1, seqlen_hi=40, page_size=8,
                max_seqlen=48, permute_pages=True, q_std=1.0, kv_std=1.0,
                softmax_scale=0.3, causal=False, seed=11)
    if kind == "gta":
        base.update(d_rope=8, rope_theta=10000.0)
    if kind == "latent":
        base.update(groups=2, head_dim=32, d_rope=8)
    base.update(kw)
    return synth.Workload(**base)


def _rows(pool, table, b, i, P):
    """Row of logical token i of sequence b, looked up in the page table."""
    return pool[table[b, i // P], i % P]


def build_by_steps(w, inp, T, append_fn=app.kv_append):
    """Empty (NaN) pools filled by successive append steps of T tokens."""
    L = inp["seqlens"].astype(np.int64)
    table = inp["page_table"]
    P = w.page_size
    pools = [None if inp[k] is None else np.full_like(inp[k], np.nan)
             for k in ("pool0", "pool1", "rope")]
    n_steps = -(-int(L.max()) // T) if L.max() > 0 else 0
    for s in range(1, n_steps + 1):
        cur = np.minimum(L, s * T)                  # lengths after this step
        new0 = np.zeros((w.batch, T) + inp["pool0"].shape[2:], np.float32)
        new1 = None if inp["pool1"] is None else np.zeros_like(new0)
        newr = None if inp["rope"] is None else np.zeros((w.batch, T, w.d_rope), np.float32)
        # the step's T positions L_b - T .. L_b - 1 (a sequence already
        # complete, or with fewer than T new tokens, rewrites its last
        # tokens with the same rows)
        for b in range(w.batch):
            for t in range(T):
                pos = int(cur[b]) - T + t
                if pos < 0:
                    continue
                new0[b, t] = _rows(inp["pool0"], table, b, pos, P)
                if new1 is not None:
                    new1[b, t] = _rows(inp["pool1"], table, b, pos, P)
                if newr is not None:
                    newr[b, t] = _rows(inp["rope"], table, b, pos, P)[0]
        pools = list(append_fn(pools[0], pools[1], pools[2], table, cur.astype(np.int32), P,
                               new0, new1, newr, 0.0, w.dtype))
    return pools


def _same_used_rows(w, inp, pools):
    """Every row a sequence uses equals the generator's, bit for bit."""
    L, table, P = inp["seqlens"], inp["page_table"], w.page_size
    for k, got in zip(("pool0", "pool1", "rope"), pools):
        if inp[k] is None:
            continue
        for b in range(w.batch):
            for i in range(int(L[b])):
                a, e = _rows(got, table, b, i, P), _rows(inp[k], table, b, i, P)
                if not np.array_equal(a, e):
                    return False
    return True


@pytest.mark.parametrize("kind", ["gqa", "gta", "latent"])
@pytest.mark.parametrize("P", [1, 4, 8, 64])
@pytest.mark.parametrize("T", [1, 3])
def test_stepwise_append_rebuilds_the_cache(kind, P, T):
    w = tiny(kind, page_size=P, q_len=T)
    inp = synth.make_inputs(w)
    pools = build_by_steps(w, inp, T)
    assert _same_used_rows(w, inp, pools)


def test_rotated_latent_key_is_complex_rotation():
    rng = np.random.default_rng(3)
    w = tiny("latent", page_size=4)
    inp = synth.make_inputs(w)
    T, d_r, theta = 2, w.d_rope, 10000.0
    new0 = rng.standard_normal((w.batch, T) + inp["pool0"].shape[2:]).astype(np.float32)
    newr = synth.round_bf16(rng.standard_normal((w.batch, T, d_r)).astype(np.float32))
    _, _, rope = app.kv_append(inp["pool0"], None, inp["rope"], inp["page_table"],
                               inp["seqlens"], w.page_size, new0, None, newr, theta, "bf16")
    half = d_r // 2
    for b in range(w.batch):
        L = int(inp["seqlens"][b])
        for t in range(T):
            pos = L - T + t
            if pos < 0:
                continue
            z = newr[b, t, :half].astype(np.float64) + 1j * newr[b, t, half:].astype(np.float64)
            z = z * np.exp(1j * pos * theta ** (-2.0 * np.arange(half) / d_r))
            want = torch.tensor(np.concatenate([z.real, z.imag]), dtype=torch.float32)
            want = want.to(torch.bfloat16).to(torch.float32).numpy()
            got = _rows(rope, inp["page_table"], b, pos, w.page_size)[0]
            # float32 -> bfloat16 of the same fp64 value, up to a tie decided
            # differently by the fp64 rotation's last bits
            assert np.allclose(got, want, rtol=2 ** -8, atol=1e-30)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4096) * 10 ** rng.uniform(-30, 30, 4096),
                        [0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), np.inf,
                         -np.inf, 3.0e38]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = app.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.isnan(app.round_bf16(np.array([np.nan], np.float32))).all()


def _buggy_append(pos_shift=0, slot_zero=False, swap=False):
    """A copy of the append with one plausible mistake."""
    def fn(pool0, pool1, rope, table, seqlens, P, new0, new1, newr, theta, dtype):
        out = [None if a is None else np.array(a, copy=True) for a in (pool0, pool1, rope)]
        src0, src1 = (new1, new0) if swap else (new0, new1)
        B, T = new0.shape[:2]
        for b in range(B):
            for t in range(T):
                pos = int(seqlens[b]) - T + t + pos_shift
                if pos < 0:
                    continue
                page, slot = table[b, pos // P], (0 if slot_zero else pos % P)
                out[0][page, slot] = src0[b, t]
                if out[1] is not None:
                    out[1][page, slot] = src1[b, t]
        return tuple(out)
    return fn


@pytest.mark.parametrize("bad", [dict(pos_shift=1), dict(pos_shift=-1), dict(slot_zero=True),
                                 dict(swap=True)])
def test_append_pins_catch_planted_mistakes(bad):
    w = tiny("gqa", page_size=4, q_len=2)
    inp = synth.make_inputs(w)
    try:
        ok = _same_used_rows(w, inp, build_by_steps(w, inp, 2, _buggy_append(**bad)))
    except (IndexError, ValueError):
        ok = False
    assert not ok, bad
