"""The projections around the latent decode, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Hardware-Efficient Attention for Fast Decoding" (Pith review page of
arXiv 2505.21487), "Core claim" and "What carries the argument": MLA and GLA
cache latent rows (h_c latent heads) plus a shared RoPE key and attend in the
latent space.  The page gives no formula for how a query head reaches that
space; the reading used here (also in the design notes) is the usual weight
absorption: head h's key up-projection U_h (d_nope x d_c) and value
up-projection V_h (d_v x d_c) act on the query and on the latent output,

    q_lat = U_h^T q_nope        so that  q_lat . c = q_nope . (U_h c)
    o     = V_h o_lat

Weights are stored as the kernels read them: w_uk[h] is U_h^T, shape
[d_c][d_nope] (row n holds latent dimension n's weights), and w_uv[h] is
V_h, shape [d_v][d_c].

Parity pins (tests/test_absorb_oracle.py): attention through the absorbed
latent path equals ordinary multi-head attention over explicitly
decompressed keys [U_h c || RoPE] and values V_h c; identity weights give
the query back.
"""
from __future__ import annotations

import numpy as np


def absorb_query(q_nope, q_rope, w_uk):
    """[U_h^T q_nope || q_rope] for every token and head, float64.

    q_nope [n, H, d_nope], q_rope [n, H, d_r] or None, w_uk [H, d_c, d_nope];
    returns [n, H, d_c + d_r]: the latent decode's query.
    """
    q = np.asarray(q_nope, dtype=np.float64)
    w = np.asarray(w_uk, dtype=np.float64)
    if w.shape[0] != q.shape[1] or w.shape[2] != q.shape[2]:
        raise ValueError("w_uk must be [H, d_c, d_nope]")
    lat = np.einsum("mhk,hnk->mhn", q, w)
    if q_rope is None:
        return lat
    return np.concatenate([lat, np.asarray(q_rope, dtype=np.float64)], axis=2)


def project_output(o_lat, w_uv):
    """V_h o_lat for every token and head, float64.

    o_lat [n, H, d_c], w_uv [H, d_v, d_c]; returns [n, H, d_v].
    """
    o = np.asarray(o_lat, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    if w.shape[0] != o.shape[1] or w.shape[2] != o.shape[2]:
        raise ValueError("w_uv must be [H, d_v, d_c]")
    return np.einsum("mhc,hnc->mhn", o, w)
