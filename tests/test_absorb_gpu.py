"""GPU parity of the projections around the latent decode
(attn_latent_absorb_query, attn_latent_project_output) against the oracle.

Each output element is an fp32 sum of exact bf16 x bf16 products, rounded
once to bf16, so it may differ from the fp64 value ref by at most
2^-8 |ref| (the rounding) plus K * 2^-24 * S (fp32 summation of K terms in
any order, S = sum_k |a_k w_k|; doubled here in case the matrix cores'
internal additions truncate rather than round); the test asserts that bound
per element and
the rel-L2 <= 5e-3 of the decode's parity bar.  The RoPE part of the
absorbed query is a copy and must be bit-exact.  The chain absorb -> latent
decode -> output projection must match the oracle's chain to the decode's
tolerances.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_amd import binding, synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

# (n_tok, h_q, d_nope, d_c, d_rope, d_v)
SHAPES = {
    "mla_c4": (128, 128, 128, 512, 64, 128),
    "gla2_c4": (128, 128, 128, 256, 64, 128),
    "spec4": (64, 128, 128, 256, 64, 128),
    "one_token": (1, 16, 128, 512, 64, 128),
    "ragged_no_rope": (100, 16, 64, 256, 0, 64),
    "ragged_tail": (130, 8, 32, 64, 8, 64),
}


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()


def _check(got, ref, bound_sum, K, tag):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), tag
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2 * K * 2.0 ** -24 * bound_sum + 1e-30
    bad = err > bound
    assert not bad.any(), f"{tag}: {bad.sum()} elements outside the rounding bound, max err " \
                          f"{err.max():.3e}"
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= H.REL_L2, f"{tag}: rel-L2 {rel:.3e}"


@pytest.mark.parametrize("name", list(SHAPES))
def test_absorb_query_matches_oracle(name):
    n, hq, dn, dc, dr, dv = SHAPES[name]
    print(f"[absorb] {name}", flush=True)
    p = synth.make_projection_inputs(n, hq, dn, dc, dr, dv, seed=n + hq + dc)
    got = binding.absorb_query(_dev(p["q_nope"]), _dev(p["q_rope"]), _dev(p["w_uk"]))
    torch.cuda.synchronize()
    got = got.float().cpu().numpy()
    ref = oracle.absorb_query(p["q_nope"], p["q_rope"], p["w_uk"])
    S = oracle.absorb_query(np.abs(p["q_nope"]), None, np.abs(p["w_uk"]))
    _check(got[:, :, :dc], ref[:, :, :dc], S, dn, f"{name} latent")
    if dr:
        assert np.array_equal(got[:, :, dc:], p["q_rope"]), f"{name}: RoPE part not copied exactly"


@pytest.mark.parametrize("name", list(SHAPES))
def test_project_output_matches_oracle(name):
    n, hq, dn, dc, dr, dv = SHAPES[name]
    print(f"[project] {name}", flush=True)
    p = synth.make_projection_inputs(n, hq, dn, dc, dr, dv, seed=2 * n + hq + dc)
    got = binding.project_output(_dev(p["o_lat"]), _dev(p["w_uv"]))
    torch.cuda.synchronize()
    ref = oracle.project_output(p["o_lat"], p["w_uv"])
    S = oracle.project_output(np.abs(p["o_lat"]), np.abs(p["w_uv"]))
    _check(got.float().cpu().numpy(), ref, S, dc, f"{name} output")


def test_empty_step_is_a_no_op():
    p = synth.make_projection_inputs(4, 2, 32, 64, 8, 64, seed=1)
    q_out = torch.full((0, 2, 72), 7.0, dtype=torch.bfloat16, device="cuda")
    binding.absorb_query(_dev(p["q_nope"])[:0], _dev(p["q_rope"])[:0], _dev(p["w_uk"]), out=q_out)
    torch.cuda.synchronize()
    assert q_out.numel() == 0


@pytest.mark.parametrize("wl", ["mla", "gla2"])
def test_absorb_decode_project_chain(wl):
    """absorb -> latent decode -> output projection against the oracle's chain."""
    w = synth.WORKLOADS[wl].with_(batch=4, seqlen_lo=2, seqlen_hi=700, max_seqlen=704, q_len=2,
                                  causal=True)
    print(f"[chain] {wl}", flush=True)
    inp = synth.make_inputs(w)
    n = w.batch * w.q_len
    p = synth.make_projection_inputs(n, w.h_q, 128, w.head_dim, w.d_rope, 128, seed=9)
    q_abs = binding.absorb_query(_dev(p["q_nope"]), _dev(p["q_rope"]), _dev(p["w_uk"]))
    d = H.to_device(w, inp)
    d["q"] = q_abs.view(w.batch, w.q_len, w.h_q, -1)
    o_lat, _, _ = H.run(w, d)
    out = binding.project_output(o_lat.contiguous().view(n, w.h_q, -1), _dev(p["w_uv"]))
    torch.cuda.synchronize()
    # the oracle's own chain from the same inputs; its absorbed query is
    # rounded to bf16 as the interface stores it (the decode reads bf16)
    q_ref = oracle.round_bf16(oracle.absorb_query(p["q_nope"], p["q_rope"], p["w_uk"])
                              .astype(np.float32)).reshape(w.batch, w.q_len, w.h_q, -1)
    o_ref, _ = oracle.decode_latent(q_ref, inp["pool0"], inp["rope"], inp["page_table"],
                                    inp["seqlens"], w.page_size, w.softmax_scale, w.causal)
    ref = oracle.project_output(o_ref.reshape(n, w.h_q, -1), p["w_uv"])
    got = out.float().cpu().numpy()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= H.REL_L2, f"{wl}: chain rel-L2 {rel:.3e}"


def _random_shapes(n=20, seed=77):
    """Seeded shapes inside the documented limits: both projections, the
    streamed-weight form (K of 128, 256, 512) and the register-only one."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append((int(rng.integers(1, 300)), int(rng.choice([1, 2, 3, 5, 8, 16, 24, 128])),
                    int(rng.choice([32, 64, 96, 128, 192, 256])),
                    int(rng.choice([64, 128, 192, 256, 512])), int(rng.choice([0, 8, 16, 64])),
                    int(rng.choice([64, 128, 192, 256]))))
    return out


RANDOM_SHAPES = _random_shapes()


@pytest.mark.parametrize("case", range(len(RANDOM_SHAPES)))
def test_random_shapes(case):
    n, hq, dn, dc, dr, dv = RANDOM_SHAPES[case]
    print(f"[proj-random] n={n} h={hq} d_nope={dn} d_c={dc} d_rope={dr} d_v={dv}", flush=True)
    p = synth.make_projection_inputs(n, hq, dn, dc, dr, dv, seed=300 + case)
    got = binding.absorb_query(_dev(p["q_nope"]), _dev(p["q_rope"]), _dev(p["w_uk"]))
    out = binding.project_output(_dev(p["o_lat"]), _dev(p["w_uv"]))
    torch.cuda.synchronize()
    got = got.float().cpu().numpy()
    ref = oracle.absorb_query(p["q_nope"], p["q_rope"], p["w_uk"])
    S = oracle.absorb_query(np.abs(p["q_nope"]), None, np.abs(p["w_uk"]))
    _check(got[:, :, :dc], ref[:, :, :dc], S, dn, f"random {case} latent")
    if dr:
        assert np.array_equal(got[:, :, dc:], p["q_rope"]), f"random {case}: RoPE part"
    ref = oracle.project_output(p["o_lat"], p["w_uv"])
    S = oracle.project_output(np.abs(p["o_lat"]), np.abs(p["w_uv"]))
    _check(out.float().cpu().numpy(), ref, S, dc, f"random {case} output")
