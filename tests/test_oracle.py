"""Pins for the fp64 oracle: it is checked against things other than itself.

Closed forms, library routines (torch scaled_dot_product_attention in
float64, scipy softmax / logsumexp, complex multiplication for RoPE), brute
force on tiny inputs, structural identities between the attention variants,
invariants of paging / splitting, and the numbers the pages print for the
byte and FLOP model (tests/golden/pages_counts.json).  The last block plants
plausible mistakes in copies of oracle functions and shows the pins catch
them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as att
from oracle import counts
from decode_attention_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_counts.json")
RNG = np.random.default_rng(12345)


def rnd(*shape, rng=None):
    return (rng or RNG).standard_normal(shape)


def tiny(kind="gqa", **kw):
    base = dict(name="tiny", kind=kind, dtype="bf16", batch=3, q_len=1, h_q=8, groups=2,
                head_dim=16, d_rope=0, seqlen_lo=1, seqlen_hi=70, page_size=8,
                max_seqlen=80, permute_pages=True, q_std=1.0, kv_std=1.0,
                softmax_scale=0.3, causal=False, seed=7)
    if kind == "gta":
        base.update(d_rope=8, rope_theta=10000.0)
    if kind == "latent":
        base.update(groups=2, head_dim=32, d_rope=8)
    base.update(kw)
    return synth.Workload(**base)


# ------------------------------------------------------------ core closed forms
def test_single_key_returns_its_value():
    q, k, v = rnd(3, 5), rnd(1, 5), rnd(1, 4)
    o, lse = att.attend(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.repeat(v, 3, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * (q @ k[0]), rtol=1e-15, atol=1e-15)


def test_two_keys_logistic():
    q, k, v = rnd(4, 6), rnd(2, 6), rnd(2, 3)
    s0, s1 = 0.5 * (q @ k[0]), 0.5 * (q @ k[1])
    p0 = 1.0 / (1.0 + np.exp(s1 - s0))
    o, lse = att.attend(q, k, v, 0.5)
    np.testing.assert_allclose(o, p0[:, None] * v[0] + (1 - p0)[:, None] * v[1], atol=1e-14)
    np.testing.assert_allclose(lse, np.logaddexp(s0, s1), atol=1e-14)


def test_zero_query_averages_values():
    L = 37
    k, v = rnd(L, 8), rnd(L, 5)
    o, lse = att.attend(np.zeros((2, 8)), k, v, 1.0)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (2, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, np.log(L), atol=1e-14)


def test_constant_value_is_returned():
    L = 50
    c = rnd(7)
    o, _ = att.attend(rnd(3, 4), rnd(L, 4), np.tile(c, (L, 1)), 1.3)
    np.testing.assert_allclose(o, np.tile(c, (3, 1)), atol=1e-14)


def test_dominant_key_selects_its_value():
    L, D = 20, 6
    k = rnd(L, D)
    q = 200.0 * k[13][None, :] / np.linalg.norm(k[13])
    k_other = k.copy()
    k_other[np.arange(L) != 13] *= 1e-3
    v = rnd(L, 3)
    o, _ = att.attend(q, k_other, v, 1.0)
    np.testing.assert_allclose(o[0], v[13], atol=1e-12)


def test_probs_sum_to_one_and_match_scipy():
    q, k, v = rnd(5, 9), rnd(33, 9), rnd(33, 4)
    o, lse, p = att.attend(q, k, v, 0.4, return_probs=True)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    s = 0.4 * np.einsum("rd,ld->rl", q, k)
    np.testing.assert_allclose(p, scipy.special.softmax(s, axis=1), atol=1e-15)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=1), atol=1e-13)
    np.testing.assert_allclose(o, scipy.special.softmax(s, axis=1) @ v, atol=1e-14)


def test_score_shift_invariance():
    q, k, v = rnd(2, 4), rnd(9, 4), rnd(9, 3)
    # a key direction orthogonal to nothing: add a constant to every score by
    # appending a coordinate that is 1 for all keys and c for the query
    c = 3.25
    q2 = np.concatenate([q, np.full((2, 1), c)], 1)
    k2 = np.concatenate([k, np.ones((9, 1))], 1)
    o1, l1 = att.attend(q, k, v, 1.0)
    o2, l2 = att.attend(q2, k2, v, 1.0)
    np.testing.assert_allclose(o2, o1, atol=1e-14)
    np.testing.assert_allclose(l2, l1 + c, atol=1e-13)


def test_empty_sequence():
    o, lse = att.attend(rnd(3, 4), np.zeros((0, 4)), np.zeros((0, 6)), 1.0)
    assert (o == 0).all() and o.shape == (3, 6)
    assert np.isneginf(lse).all()


def _brute(q, k, v, scale, qpos):
    R, L = len(q), len(k)
    o = [[0.0] * len(v[0]) for _ in range(R)]
    lse = []
    for r in range(R):
        vis = [i for i in range(L) if qpos is None or i <= qpos[r]]
        sc = [scale * sum(q[r][d] * k[i][d] for d in range(len(q[r]))) for i in vis]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        tot = sum(e)
        for n, i in enumerate(vis):
            for c in range(len(v[0])):
                o[r][c] += e[n] / tot * v[i][c]
        lse.append(m + math.log(tot))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("L,D,causal", [(1, 1, False), (3, 2, False), (6, 4, False),
                                         (6, 3, True), (5, 4, True)])
def test_brute_force_tiny(L, D, causal):
    rng = np.random.default_rng(L * 10 + D)
    q, k, v = rnd(3, D, rng=rng), rnd(L, D, rng=rng), rnd(L, 2, rng=rng)
    qpos = np.array([L - 3 + t for t in range(3)]) if causal else None
    if causal:
        qpos = np.maximum(qpos, 0)
    o, lse = att.attend(q, k, v, 0.9, qpos)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), 0.9, None if qpos is None else qpos.tolist())
    np.testing.assert_allclose(o, ob, atol=1e-13)
    np.testing.assert_allclose(lse, lb, atol=1e-13)


# ------------------------------------------------------------ library routine
def _sdpa_dense(qd, kd, vd, scale, causal):
    """torch SDPA (float64, CPU).  qd [H, T, D], kd/vd [G, L, D].

    Causal: SDPA's is_causal aligns query i with key i, so the T real queries
    are placed at positions L-T..L-1 of an L-long query block.
    """
    H, T, D = qd.shape
    G, L, _ = kd.shape
    qt = torch.from_numpy(np.ascontiguousarray(qd))
    if causal and T > 1:
        full = torch.zeros((H, L, D), dtype=torch.float64)
        full[:, L - T:] = qt
        qt = full
    out = F.scaled_dot_product_attention(
        qt[None], torch.from_numpy(np.ascontiguousarray(kd))[None],
        torch.from_numpy(np.ascontiguousarray(vd))[None], scale=scale,
        is_causal=bool(causal and T > 1), enable_gqa=True)[0]
    if causal and T > 1:
        out = out[:, L - T:]
    return out.numpy()


def _dense_rows(pool, table_row, L, P, head):
    i = np.arange(L)
    return pool[table_row[i // P], i % P, head].astype(np.float64)


def check_gqa_vs_sdpa(decode_fn, w, inp):
    out, _ = decode_fn(inp["q"], inp["pool0"], inp["pool1"], inp["page_table"], inp["seqlens"],
                       w.page_size, w.softmax_scale, w.causal)
    for b, L in enumerate(inp["seqlens"].tolist()):
        kd = np.stack([_dense_rows(inp["pool0"], inp["page_table"][b], L, w.page_size, j)
                       for j in range(w.groups)])
        vd = np.stack([_dense_rows(inp["pool1"], inp["page_table"][b], L, w.page_size, j)
                       for j in range(w.groups)])
        ref = _sdpa_dense(inp["q"][b].transpose(1, 0, 2).astype(np.float64), kd, vd,
                          w.softmax_scale, w.causal)
        np.testing.assert_allclose(out[b], ref.transpose(1, 0, 2), atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("T,causal", [(1, False), (3, True), (2, False)])
def test_gqa_matches_torch_sdpa(T, causal):
    w = tiny("gqa", q_len=T, causal=causal, seqlen_lo=4)
    check_gqa_vs_sdpa(att.decode_gqa, w, synth.make_inputs(w))


def test_gqa_lse_matches_scipy():
    w = tiny("gqa")
    inp = synth.make_inputs(w)
    _, lse = oracle.decode(w, inp)
    g = w.group_size
    for b, L in enumerate(inp["seqlens"].tolist()):
        for h in range(w.h_q):
            k = _dense_rows(inp["pool0"], inp["page_table"][b], L, w.page_size, h // g)
            s = w.softmax_scale * (k @ inp["q"][b, 0, h].astype(np.float64))
            assert abs(lse[b, 0, h] - scipy.special.logsumexp(s)) < 1e-12


def test_mqa_and_mha_cases():
    # h_kv = 1 (MQA) and g = 1 (MHA) both against SDPA
    for groups in (1, 8):
        w = tiny("gqa", groups=groups)
        check_gqa_vs_sdpa(att.decode_gqa, w, synth.make_inputs(w))


def test_head_permutation_within_group_permutes_outputs():
    w = tiny("gqa")
    inp = synth.make_inputs(w)
    out, _ = oracle.decode(w, inp)
    perm = np.arange(w.h_q)
    perm[0:4] = [2, 0, 3, 1]          # inside group 0 (g = 4)
    inp2 = dict(inp, q=inp["q"][:, :, perm])
    out2, _ = oracle.decode(w, inp2)
    np.testing.assert_array_equal(out2, out[:, :, perm])


# ------------------------------------------------------------ RoPE
def _rope_complex(x, pos, theta):
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    f = theta ** (-np.arange(half) * 2.0 / d)
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * f)
    return np.concatenate([z.real, z.imag], axis=-1)


def check_rope(rope_fn):
    x = rnd(11, 16)
    pos = np.arange(11) * 37 + 5
    np.testing.assert_allclose(rope_fn(x, pos, 10000.0), _rope_complex(x, pos, 10000.0),
                               atol=1e-12)
    np.testing.assert_array_equal(rope_fn(x, np.zeros(11), 500.0), x)
    np.testing.assert_allclose(np.linalg.norm(rope_fn(x, pos, 77.0), axis=1),
                               np.linalg.norm(x, axis=1), rtol=1e-13)
    # relative-position property: <R(a)q, R(b)k> depends on b - a only
    q, k = rnd(16), rnd(16)
    d1 = rope_fn(q[None], np.array([100]), 10000.0) @ rope_fn(k[None], np.array([130]), 10000.0).T
    d2 = rope_fn(q[None], np.array([7]), 10000.0) @ rope_fn(k[None], np.array([37]), 10000.0).T
    np.testing.assert_allclose(d1, d2, atol=1e-12)
    # explicit 2x2 rotation of pair (0, 8) at position 3, frequency 1
    ang = 3.0
    rot = np.array([[math.cos(ang), -math.sin(ang)], [math.sin(ang), math.cos(ang)]])
    y = rope_fn(x[:1], np.array([3]), 10000.0)[0]
    np.testing.assert_allclose([y[0], y[8]], rot @ [x[0, 0], x[0, 8]], atol=1e-14)


def test_rope_pins():
    check_rope(att.rope_rotate_half)


# ------------------------------------------------------------ GTA
def check_gta(decode_gta_fn, w, inp):
    out, _ = decode_gta_fn(inp["q"], inp["pool0"], inp["rope"], inp["page_table"],
                           inp["seqlens"], w.page_size, w.d_rope, w.rope_theta,
                           w.softmax_scale, w.causal)
    d, dr = w.head_dim, w.d_rope
    for b, L in enumerate(inp["seqlens"].tolist()):
        r = _dense_rows(inp["rope"], inp["page_table"][b], L, w.page_size, 0)
        kr = _rope_complex(r, np.arange(L), w.rope_theta)
        S = np.stack([_dense_rows(inp["pool0"], inp["page_table"][b], L, w.page_size, j)
                      for j in range(w.groups)])
        kd = np.concatenate([S[:, :, :d - dr], np.broadcast_to(kr, (w.groups, L, dr))], 2)
        qb = inp["q"][b].astype(np.float64)            # [T, H, d]
        qpos = (L - w.q_len + np.arange(w.q_len))[:, None]
        qb = np.concatenate([qb[..., :d - dr], _rope_complex(qb[..., d - dr:], qpos, w.rope_theta)], -1)
        ref = _sdpa_dense(qb.transpose(1, 0, 2), kd, S, w.softmax_scale, w.causal)
        np.testing.assert_allclose(out[b], ref.transpose(1, 0, 2), atol=1e-12)


@pytest.mark.parametrize("T,causal", [(1, False), (2, True)])
def test_gta_matches_sdpa_on_materialised_kv(T, causal):
    w = tiny("gta", q_len=T, causal=causal, seqlen_lo=3)
    check_gta(att.decode_gta, w, synth.make_inputs(w))


def test_gta_without_rope_equals_gqa_with_k_equal_v():
    w = tiny("gta", d_rope=0, rope_theta=0.0)
    inp = synth.make_inputs(w, seed=99)
    o_gta, l_gta = att.decode_gta(inp["q"], inp["pool0"], None, inp["page_table"], inp["seqlens"],
                                  w.page_size, 0, 0.0, w.softmax_scale)
    o_gqa, l_gqa = att.decode_gqa(inp["q"], inp["pool0"], inp["pool0"], inp["page_table"],
                                  inp["seqlens"], w.page_size, w.softmax_scale)
    np.testing.assert_array_equal(o_gta, o_gqa)
    np.testing.assert_array_equal(l_gta, l_gqa)


# ------------------------------------------------------------ latent (MLA / GLA)
def check_latent(decode_latent_fn, w, inp):
    out, _ = decode_latent_fn(inp["q"], inp["pool0"], inp["rope"], inp["page_table"],
                              inp["seqlens"], w.page_size, w.softmax_scale, w.causal)
    for b, L in enumerate(inp["seqlens"].tolist()):
        r = _dense_rows(inp["rope"], inp["page_table"][b], L, w.page_size, 0)
        C = np.stack([_dense_rows(inp["pool0"], inp["page_table"][b], L, w.page_size, j)
                      for j in range(w.groups)])
        kd = np.concatenate([C, np.broadcast_to(r, (w.groups,) + r.shape)], 2)
        ref = _sdpa_dense(inp["q"][b].astype(np.float64).transpose(1, 0, 2), kd, C,
                          w.softmax_scale, w.causal)
        np.testing.assert_allclose(out[b], ref.transpose(1, 0, 2), atol=1e-12)


@pytest.mark.parametrize("groups,T,causal", [(1, 1, False), (2, 1, False), (2, 4, True),
                                              (1, 3, True)])
def test_latent_matches_sdpa(groups, T, causal):
    w = tiny("latent", groups=groups, head_dim=64 // groups, q_len=T, causal=causal,
             seqlen_lo=4)
    check_latent(att.decode_latent, w, synth.make_inputs(w))


def test_gla2_equals_two_mla_calls():
    w = tiny("latent", groups=2, head_dim=16, h_q=8)
    inp = synth.make_inputs(w)
    out, lse = oracle.decode(w, inp)
    g = w.group_size
    for j in range(2):
        o_j, l_j = att.decode_latent(inp["q"][:, :, j * g:(j + 1) * g],
                                     inp["pool0"][:, :, j:j + 1], inp["rope"], inp["page_table"],
                                     inp["seqlens"], w.page_size, w.softmax_scale)
        np.testing.assert_array_equal(out[:, :, j * g:(j + 1) * g], o_j)
        np.testing.assert_array_equal(lse[:, :, j * g:(j + 1) * g], l_j)


def test_mla_equals_gqa_on_materialised_kv():
    w = tiny("latent", groups=1, head_dim=24)
    inp = synth.make_inputs(w)
    o_mla, l_mla = oracle.decode(w, inp)
    kpool = np.concatenate([inp["pool0"], inp["rope"]], axis=3)
    o_gqa, l_gqa = att.decode_gqa(inp["q"], kpool, inp["pool0"], inp["page_table"],
                                  inp["seqlens"], w.page_size, w.softmax_scale)
    np.testing.assert_array_equal(o_mla, o_gqa)
    np.testing.assert_array_equal(l_mla, l_gqa)


# ------------------------------------------------------------ causal
@pytest.mark.parametrize("kind", ["gqa", "gta", "latent"])
def test_causal_row_equals_truncated_decode(kind):
    T = 4
    w = tiny(kind, q_len=T, causal=True, seqlen_lo=5)
    inp = synth.make_inputs(w)
    out, lse = oracle.decode(w, inp)
    w1 = w.with_(q_len=1, causal=False)
    for t in range(T):
        inp1 = dict(inp, q=inp["q"][:, t:t + 1], seqlens=inp["seqlens"] - (T - 1 - t))
        o1, l1 = oracle.decode(w1, inp1)
        np.testing.assert_allclose(out[:, t], o1[:, 0], atol=1e-13)
        np.testing.assert_allclose(lse[:, t], l1[:, 0], atol=1e-13)


def test_causal_is_noop_at_q_len_1():
    w = tiny("gqa")
    inp = synth.make_inputs(w)
    a, _ = oracle.decode(w, inp)
    b, _ = oracle.decode(w.with_(causal=True), inp)
    np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------ paging
def _repage(w, inp, page_size, seed):
    """Same logical cache in a different paging (page size, permutation)."""
    rng = np.random.default_rng(seed)
    max_pages = -(-w.max_seqlen // page_size)
    table, n = synth.build_page_table(inp["seqlens"], page_size, max_pages, True, rng)
    out = dict(inp, page_table=table)
    for key in ("pool0", "pool1", "rope"):
        src = inp[key]
        if src is None:
            continue
        dst = np.full((n, page_size) + src.shape[2:], np.nan, dtype=src.dtype)
        for b, L in enumerate(inp["seqlens"].tolist()):
            i = np.arange(L)
            rows = src[inp["page_table"][b][i // w.page_size], i % w.page_size]
            dst[table[b][i // page_size], i % page_size] = rows
        out[key] = dst
    return w.with_(page_size=page_size), out


@pytest.mark.parametrize("kind", ["gqa", "gta", "latent"])
def test_paging_is_bit_exact(kind):
    w = tiny(kind)
    inp = synth.make_inputs(w)
    ref, ref_lse = oracle.decode(w, inp)
    for P, seed in ((1, 1), (16, 2), (128, 3), (8, 4)):
        w2, inp2 = _repage(w, inp, P, seed)
        o, l = oracle.decode(w2, inp2)
        np.testing.assert_array_equal(o, ref)
        np.testing.assert_array_equal(l, ref_lse)


def test_nan_in_unused_slots_never_read():
    w = tiny("latent")
    inp = synth.make_inputs(w, tail_fill=np.nan, extra_pages=5)
    assert np.isnan(inp["pool0"]).any()
    out, lse = oracle.decode(w, inp)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_page_table_minus_one_inside_sequence_raises():
    w = tiny("gqa")
    inp = synth.make_inputs(w)
    bad = inp["page_table"].copy()
    bad[0, 0] = -1
    with pytest.raises(IndexError):
        oracle.decode(w, dict(inp, page_table=bad))


# ------------------------------------------------------------ split / combine
def check_split_merge(merge_fn):
    rng = np.random.default_rng(5)
    L = 301
    q, k, v = rnd(6, 12, rng=rng), rnd(L, 12, rng=rng), rnd(L, 7, rng=rng)
    qpos = np.array([L - 6 + t for t in range(6)])
    ref_o, ref_l = att.attend(q, k, v, 0.35, qpos)
    for n_chunks in (1, 2, 5, 17):
        cuts = np.sort(rng.choice(np.arange(1, L), n_chunks - 1, replace=False))
        parts = np.split(np.arange(L), cuts)
        os_, ls_ = zip(*[att.attend_partial(q, k, v, 0.35, idx, qpos) for idx in parts])
        o, l = merge_fn(np.stack(os_), np.stack(ls_))
        np.testing.assert_allclose(o, ref_o, atol=1e-13)
        np.testing.assert_allclose(l, ref_l, atol=1e-13)
    # a chunk that every row masks (its keys lie beyond all query positions)
    last = np.arange(L - 3, L)
    o_m, l_m = att.attend_partial(q[:2], k, v, 0.35, last, qpos[:2])
    assert np.isneginf(l_m).all() and (o_m == 0).all()


def test_split_merge_equals_unsplit():
    check_split_merge(att.merge_partials)


# ------------------------------------------------------------ counts vs pages
def _count_wl(kind, h_q, groups, head_dim, d_rope):
    return synth.Workload(name="x", kind=kind, dtype="bf16", batch=1, q_len=1, h_q=h_q,
                          groups=groups, head_dim=head_dim, d_rope=d_rope, seqlen_lo=64,
                          seqlen_hi=64, page_size=64, max_seqlen=64, permute_pages=False,
                          q_std=1, kv_std=1, softmax_scale=1.0, causal=False, seed=0)


def test_counts_against_page_values():
    with open(GOLDEN) as f:
        entries = json.load(f)["entries"]
    for e in entries:
        tol = e["rel_tol"]
        if e["check"] in ("intensity", "intensity_vs_model"):
            w = _count_wl(e["kind"], e["h_q"], e["groups"], e["head_dim"], e["d_rope"])
            got = counts.intensity(w, [4096])
            if e["check"] == "intensity_vs_model":
                assert counts.intensity_model(e["g_q"], e["m_kv"]) == e["value"], e["id"]
        elif e["check"] == "bytes_ratio":
            a, b = e["a"], e["b"]
            got = (counts.kv_bytes_per_token(a["kind"], a["groups"], a["head_dim"], a["d_rope"], 2)
                   / counts.kv_bytes_per_token(b["kind"], b["groups"], b["head_dim"], b["d_rope"], 2))
        elif e["check"] == "tp_dup":
            got = counts.tp_duplication(e["n"], e["g_q"], e["h_q"])
        else:
            raise AssertionError(e["check"])
        assert abs(got - e["value"]) <= tol * abs(e["value"]), (e["id"], got)


@pytest.mark.parametrize("kind,T,causal", [("gqa", 1, False), ("gta", 1, False),
                                            ("latent", 1, False), ("latent", 3, True)])
def test_bytes_read_equal_analytical_cache_size(kind, T, causal):
    w = tiny(kind, q_len=T, causal=causal, seqlen_lo=3)
    inp = synth.make_inputs(w)
    assert counts.count_touched_rows(w, inp) == counts.kv_bytes(w, inp["seqlens"])


def test_flops_equal_visible_pairs():
    w = tiny("latent", q_len=3, causal=True, seqlen_lo=3)
    inp = synth.make_inputs(w)
    pairs = 0
    for L in inp["seqlens"].tolist():
        for t in range(3):
            pairs += sum(1 for i in range(L) if i <= L - 3 + t)
    per = 2 * (w.head_dim + w.d_rope) + 2 * w.head_dim
    assert counts.flops(w, inp["seqlens"]) == pairs * w.h_q * per


def test_workload_intensities():
    W = synth.WORKLOADS
    assert counts.intensity(W["gqa_llama8b"], [8192]) == 4.0
    assert counts.intensity(W["gla2"], [8192]) == 128.0
    assert abs(counts.intensity(W["mla"], [8192]) - 278528 / 1152) < 1e-9
    assert abs(counts.intensity(W["gta_8k"], [8192]) - 16384 / 1152) < 1e-9
    # speculative verify: causal pairs make it slightly below 4x the q_len-1 value
    L = 131072
    assert counts.flops(W["gla2_spec4_128k"], [L]) == (4 * L - 6) * 128 * (2 * 320 + 2 * 256)


# ------------------------------------------------------------ planted mistakes
def _fails(fn, *a):
    try:
        fn(*a)
    except AssertionError:
        return True
    return False


def test_pins_catch_planted_mistakes(monkeypatch):
    # RoPE: wrong rotation sign; interleaved pairing; frequency off by one
    def rope_sign(x, pos, theta):
        return att.rope_rotate_half(x, -np.asarray(pos), theta)

    def rope_interleaved(x, pos, theta):
        x = np.asarray(x, dtype=np.float64)
        y = np.empty_like(x)
        y[..., 0::2], y[..., 1::2] = x[..., : x.shape[-1] // 2], x[..., x.shape[-1] // 2:]
        return att.rope_rotate_half(y, pos, theta)

    def rope_freq(x, pos, theta):
        d = x.shape[-1]
        half = d // 2
        f = theta ** (-2.0 * (np.arange(half) + 1) / d)
        ang = np.asarray(pos, dtype=np.float64)[..., None] * f
        a, b = x[..., :half], x[..., half:]
        return np.concatenate([a * np.cos(ang) - b * np.sin(ang), a * np.sin(ang) + b * np.cos(ang)], -1)

    for bad in (rope_sign, rope_interleaved, rope_freq):
        assert _fails(check_rope, bad), bad.__name__

    # GQA: head h mapped to group h % G instead of h // g; scale dropped;
    # causal window aligned to the start instead of the end of the sequence
    w = tiny("gqa", q_len=2, causal=True, seqlen_lo=4)
    inp = synth.make_inputs(w)

    def gqa_modmap(q, kp, vp, table, seqlens, P, scale, causal=False):
        B, T, H, _ = q.shape
        G = kp.shape[2]
        perm = np.argsort([h % G for h in range(H)], kind="stable")
        o, l = att.decode_gqa(q[:, :, perm], kp, vp, table, seqlens, P, scale, causal)
        inv = np.argsort(perm)
        return o[:, :, inv], l[:, :, inv]

    def gqa_noscale(q, kp, vp, table, seqlens, P, scale, causal=False):
        return att.decode_gqa(q, kp, vp, table, seqlens, P, 1.0, causal)

    def gqa_topleft(q, kp, vp, table, seqlens, P, scale, causal=False):
        orig = att._row_positions
        monkeypatch.setattr(att, "_row_positions", lambda L, T, g: orig(T, T, g))
        try:
            return att.decode_gqa(q, kp, vp, table, seqlens, P, scale, causal)
        finally:
            monkeypatch.setattr(att, "_row_positions", orig)

    for bad in (gqa_modmap, gqa_noscale, gqa_topleft):
        assert _fails(check_gqa_vs_sdpa, bad, w, inp), bad.__name__

    # GTA: RoPE applied to the tied half instead of the separate key; query
    # rotated at position 0
    wg = tiny("gta", seqlen_lo=3)
    inpg = synth.make_inputs(wg)

    def gta_wrong_half(q, tp, rp, table, seqlens, P, dr, theta, scale, causal=False):
        tp2 = tp.copy()
        tp2[..., -dr:], tp2[..., :dr] = tp[..., :dr], tp[..., -dr:]
        q2 = q.copy()
        q2[..., -dr:], q2[..., :dr] = q[..., :dr], q[..., -dr:]
        return att.decode_gta(q2, tp2, rp, table, seqlens, P, dr, theta, scale, causal)

    def gta_qpos0(q, tp, rp, table, seqlens, P, dr, theta, scale, causal=False):
        orig = att.rope_rotate_half
        calls = {"n": 0}

        def rope_q0(x, pos, th):
            # the query rotation is the call made on a 2-D row block
            if np.asarray(pos).ndim == 1 and x.shape[0] == len(pos) and calls["n"] % 2:
                pos = np.zeros_like(pos)
            calls["n"] += 1
            return orig(x, pos, th)

        monkeypatch.setattr(att, "rope_rotate_half", rope_q0)
        try:
            return att.decode_gta(q, tp, rp, table, seqlens, P, dr, theta, scale, causal)
        finally:
            monkeypatch.setattr(att, "rope_rotate_half", orig)

    for bad in (gta_wrong_half, gta_qpos0):
        assert _fails(check_gta, bad, wg, inpg), bad.__name__

    # latent: RoPE key dropped from the score
    wl = tiny("latent")
    inpl = synth.make_inputs(wl)

    def latent_norope(q, lp, rp, table, seqlens, P, scale, causal=False):
        return att.decode_latent(q, lp, np.zeros_like(rp), table, seqlens, P, scale, causal)

    assert _fails(check_latent, latent_norope, wl, inpl)

    # split merge: weights taken as exp(M - lse) instead of exp(lse - M)
    def merge_bad(os_, ls_):
        M = ls_.max(0)
        wgt = np.exp(M[None] - ls_)
        return (wgt[:, :, None] * os_).sum(0) / wgt.sum(0)[:, None], M + np.log(wgt.sum(0))

    assert _fails(check_split_merge, merge_bad)
