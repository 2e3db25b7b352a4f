"""Pins for the oracle's projections around the latent decode (CPU only).

* Attention through the absorbed latent path (absorb_query, the latent
  decode oracle, project_output) equals ordinary multi-head attention over
  explicitly decompressed per-head keys [U_h c_i || r_i] and values V_h c_i,
  computed here with plain per-row loops: this pins the weight orientation,
  the head indexing, the RoPE pass-through and the output projection
  against the associativity identity q . (U c) = (U^T q) . c.
* Identity key weights return the query unchanged (zero-padded).
* Plausible mistakes planted in copies of the projections fail the pin.
"""
import numpy as np
import pytest

import oracle
from oracle import absorb as ab
from decode_attention_kv_amd import synth


def tiny_latent(groups, q_len, page_size, causal):
    return synth.Workload(name="tiny", kind="latent", dtype="bf16", batch=3, q_len=q_len, h_q=8,
                          groups=groups, head_dim=24, d_rope=8, seqlen_lo=q_len, seqlen_hi=37,
                          page_size=page_size, max_seqlen=40, permute_pages=True, q_std=1.0,
                          kv_std=1.0, softmax_scale=0.2, causal=causal, seed=5)


def explicit_mha(w, inp, proj):
    """Multi-head attention with decompressed keys and values, row by row."""
    B, T, H = w.batch, w.q_len, w.h_q
    g = H // w.groups
    P, table = w.page_size, inp["page_table"]
    w_uk, w_uv = proj["w_uk"].astype(np.float64), proj["w_uv"].astype(np.float64)
    q_nope = proj["q_nope"].astype(np.float64).reshape(B, T, H, -1)
    q_rope = proj["q_rope"].astype(np.float64).reshape(B, T, H, -1)
    out = np.zeros((B, T, H, w_uv.shape[1]))
    for b in range(B):
        L = int(inp["seqlens"][b])
        for t in range(T):
            last = L - T + t if w.causal else L - 1
            for h in range(H):
                j = h // g
                q = np.concatenate([q_nope[b, t, h], q_rope[b, t, h]])
                scores, values = [], []
                for i in range(0, last + 1):
                    page, slot = table[b, i // P], i % P
                    c = inp["pool0"][page, slot, j].astype(np.float64)
                    r = inp["rope"][page, slot, 0].astype(np.float64)
                    k = np.concatenate([w_uk[h].T @ c, r])
                    scores.append(w.softmax_scale * float(q @ k))
                    values.append(w_uv[h] @ c)
                s = np.array(scores)
                p = np.exp(s - s.max())
                out[b, t, h] = (p[:, None] * np.array(values)).sum(0) / p.sum()
    return out


def absorbed_path(w, inp, proj, absorb=ab.absorb_query, project=ab.project_output):
    B, T, H = w.batch, w.q_len, w.h_q
    q = absorb(proj["q_nope"], proj["q_rope"], proj["w_uk"]).reshape(B, T, H, -1)
    o_lat, _ = oracle.decode_latent(q, inp["pool0"], inp["rope"], inp["page_table"],
                                    inp["seqlens"], w.page_size, w.softmax_scale, w.causal)
    return project(o_lat.reshape(B * T, H, -1), proj["w_uv"]).reshape(B, T, H, -1)


def inputs(groups, q_len, page_size, causal, d_nope=16, d_v=12):
    w = tiny_latent(groups, q_len, page_size, causal)
    inp = synth.make_inputs(w)
    proj = synth.make_projection_inputs(w.batch * q_len, w.h_q, d_nope, w.head_dim, w.d_rope, d_v,
                                        seed=groups * 10 + q_len)
    return w, inp, proj


@pytest.mark.parametrize("groups", [1, 2])
@pytest.mark.parametrize("q_len,causal", [(1, False), (3, True)])
@pytest.mark.parametrize("page_size", [4, 16])
def test_absorbed_path_equals_decompressed_attention(groups, q_len, causal, page_size):
    w, inp, proj = inputs(groups, q_len, page_size, causal)
    got = absorbed_path(w, inp, proj)
    want = explicit_mha(w, inp, proj)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_identity_key_weights_return_the_query():
    rng = np.random.default_rng(2)
    n, H, dn, dc, dr = 5, 3, 16, 24, 8
    q_nope, q_rope = rng.standard_normal((n, H, dn)), rng.standard_normal((n, H, dr))
    w_uk = np.zeros((H, dc, dn))
    w_uk[:, :dn, :] = np.eye(dn)
    got = ab.absorb_query(q_nope, q_rope, w_uk)
    want = np.concatenate([q_nope, np.zeros((n, H, dc - dn)), q_rope], axis=2)
    assert np.array_equal(got, want)
    w_uv = np.zeros((H, dn, dc))
    w_uv[:, :, :dn] = np.eye(dn)
    assert np.array_equal(ab.project_output(got[:, :, :dc], w_uv), q_nope)


def _shifted_heads(q_nope, q_rope, w_uk):
    return ab.absorb_query(q_nope, q_rope, np.roll(w_uk, 1, axis=0))


def _dropped_rope(q_nope, q_rope, w_uk):
    lat = ab.absorb_query(q_nope, None, w_uk)
    return np.concatenate([lat, np.zeros_like(q_rope, dtype=np.float64)], axis=2)


def _reversed_latent_dims(q_nope, q_rope, w_uk):
    return ab.absorb_query(q_nope, q_rope, w_uk[:, ::-1, :])


def _value_weights_of_next_head(o_lat, w_uv):
    return ab.project_output(o_lat, np.roll(w_uv, -1, axis=0))


@pytest.mark.parametrize("bad", ["shift", "rope", "reverse", "value"])
def test_pin_catches_planted_mistakes(bad):
    w, inp, proj = inputs(2, 1, 4, False)
    kw = {"shift": dict(absorb=_shifted_heads), "rope": dict(absorb=_dropped_rope),
          "reverse": dict(absorb=_reversed_latent_dims),
          "value": dict(project=_value_weights_of_next_head)}[bad]
    got = absorbed_path(w, inp, proj, **kw)
    want = explicit_mha(w, inp, proj)
    assert not np.allclose(got, want, rtol=1e-6, atol=1e-9)
