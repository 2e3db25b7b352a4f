"""The allocation-free GQA decode (attn_decode_gqa_static) through the C ABI:
the same results as attn_decode_gqa with a caller workspace, bit for bit,
and within the parity bar of the oracle, on two calls in a row (the second
with a smaller input, so the library's array holds the first call's
partials when the second starts)."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kv_amd import binding, synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _static_call(w, d, plan):
    B, T, Hq = w.batch, w.q_len, w.h_q
    out = torch.empty((B, T, Hq, w.head_dim), dtype=d["q"].dtype, device=d["q"].device)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=d["q"].device)
    kv = binding.paged_kv(d["pool0"], d["pool1"], None, d["page_table"], d["seqlens"])
    flags = binding.ATTN_CAUSAL if w.causal else 0
    s = torch.cuda.current_stream(d["q"].device).cuda_stream
    st = binding.attn_decode_gqa_static(kv, d["q"].data_ptr(), out.data_ptr(), lse.data_ptr(), T,
                                        Hq, w.groups, w.head_dim, w.softmax_scale, flags,
                                        plan.plan, s)
    assert st == binding.ATTN_OK, binding.attn_status_string(st)
    return out, lse


@pytest.mark.parametrize("inline", [False, True])
def test_static_workspace_matches_caller_workspace(inline):
    cases = [W["gqa_llama8b"].with_(batch=6, seqlen_lo=300, seqlen_hi=2000, max_seqlen=2048),
             W["gqa_llama8b"].with_(batch=2, q_len=3, causal=True, seqlen_lo=3, seqlen_hi=500,
                                    max_seqlen=512, seed=77)]
    for k, w in enumerate(cases):
        print(f"[static] call {k} B={w.batch} T={w.q_len} inline={inline}", flush=True)
        inp = synth.make_inputs(w)
        d = H.to_device(w, inp)
        # chunks of 64 tokens: every sequence splits, so the partials and
        # the merge go through the library's array
        ref_out, ref_lse, plan = H.run(w, d, chunk_tokens=64, inline_plan=inline)
        assert plan.plan.max_splits > 1
        assert binding.attn_decode_workspace_size(plan.plan, w.h_q, w.head_dim) <= \
            binding.ATTN_STATIC_SCRATCH_BYTES
        out, lse = _static_call(w, d, plan)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), k
        ref, ref_l = oracle.decode(w, inp)
        H.compare(H.to_np(out), H.to_np(lse), ref, ref_l, H.value_max(w, inp), f"static{k}")


def test_static_workspace_limits():
    """Plans needing more than the library's array, and deferred merges
    (whose partials the caller could not reach), are refused before any
    launch."""
    w = W["gqa_llama8b"].with_(batch=64, seqlen_lo=8192, seqlen_hi=8192, max_seqlen=8192)
    inp = synth.make_inputs(w)
    d = H.to_device(w, inp)
    sh = binding.shape("gqa", binding.ATTN_BF16, w.batch, 1, w.h_q, w.groups, w.head_dim, 0,
                       w.page_size, False)
    big = binding.DevicePlan(sh, inp["seqlens"], d["q"].device, chunk_tokens=64)
    assert binding.attn_decode_workspace_size(big.plan, w.h_q, w.head_dim) > \
        binding.ATTN_STATIC_SCRATCH_BYTES
    kv = binding.paged_kv(d["pool0"], d["pool1"], None, d["page_table"], d["seqlens"])
    out = torch.empty((w.batch, 1, w.h_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    st = binding.attn_decode_gqa_static(kv, d["q"].data_ptr(), out.data_ptr(), None, 1, w.h_q,
                                        w.groups, w.head_dim, w.softmax_scale, 0, big.plan, s)
    assert st == binding.ATTN_ERR_WORKSPACE
    small = binding.DevicePlan(sh, inp["seqlens"], d["q"].device)
    st = binding.attn_decode_gqa_static(kv, d["q"].data_ptr(), out.data_ptr(), None, 1, w.h_q,
                                        w.groups, w.head_dim, w.softmax_scale,
                                        binding.ATTN_DEFER_MERGE, small.plan, s)
    assert st == binding.ATTN_ERR_INVALID_ARG
