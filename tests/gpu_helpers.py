"""Shared helpers for the GPU tests: move seeded inputs to the device, run
the native library through the binding, and compare with the oracle."""
import numpy as np
import torch

from decode_attention_kv_amd import binding

# Tolerances for bf16 inputs with fp32 accumulation: relative L2 error of the
# whole output <= 5e-3 and max abs error <= 1e-2 * max|V| (V = the values the
# call attends over).  LSE (natural log, scale included) is compared in
# absolute terms: its error is the relative error of the softmax denominator
# plus the score error from rounding the rotated GTA query/key to bf16,
# bounded here by 5e-3.
REL_L2 = 5e-3
MAX_ABS_FRAC = 1e-2
LSE_ABS = 5e-3


def device():
    return torch.device("cuda:0")


def to_device(w, inp, dev=None):
    dev = dev or device()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def t(a):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    return dict(q=t(inp["q"]), pool0=t(inp["pool0"]), pool1=t(inp["pool1"]), rope=t(inp["rope"]),
                page_table=torch.from_numpy(inp["page_table"]).to(dev),
                seqlens=torch.from_numpy(inp["seqlens"]).to(dev),
                seqlens_host=inp["seqlens"])


def run(w, dinp, **kw):
    out, lse, plan, ws = binding.decode(
        w.kind, dinp["q"], dinp["pool0"], dinp["pool1"], dinp["rope"], dinp["page_table"],
        dinp["seqlens"], dinp["seqlens_host"], groups=w.groups, scale=w.softmax_scale,
        causal=w.causal, rope_theta=w.rope_theta, d_rope=w.d_rope, **kw)
    return out, lse, plan


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def value_max(w, inp, batch_index=None):
    """max |V| over the values the call reads (V pool, tied state or latent)."""
    src = inp["pool1"] if w.kind == "gqa" else inp["pool0"]
    vals = []
    seqlens = inp["seqlens"]
    idx = range(len(seqlens)) if batch_index is None else batch_index
    for b in idx:
        L = int(seqlens[b])
        n = -(-L // w.page_size)
        if n == 0:
            continue
        pages = inp["page_table"][b, :n]
        v = src[pages].reshape(-1, src.shape[2], src.shape[3])[:L]
        vals.append(float(np.abs(v).max()))
    return max(vals) if vals else 1.0


def compare(out, lse, ref_out, ref_lse, vmax, tag=""):
    out = np.asarray(out, dtype=np.float64)
    ref_out = np.asarray(ref_out, dtype=np.float64)
    assert np.isfinite(out).all(), f"{tag}: non-finite output"
    err = out - ref_out
    denom = np.linalg.norm(ref_out)
    rel = np.linalg.norm(err) / denom if denom > 0 else np.linalg.norm(err)
    mx = np.abs(err).max() if err.size else 0.0
    assert rel <= REL_L2, f"{tag}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_FRAC * vmax, f"{tag}: max-abs {mx:.3e} > {MAX_ABS_FRAC} * {vmax}"
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        fin = np.isfinite(ref_lse)
        assert (np.isneginf(lse) == ~fin).all(), f"{tag}: LSE -inf pattern differs"
        if fin.any():
            le = np.abs(lse[fin] - ref_lse[fin]).max()
            assert le <= LSE_ABS, f"{tag}: LSE abs err {le:.3e}"
    return rel, mx
