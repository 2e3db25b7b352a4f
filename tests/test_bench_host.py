"""Host-side checks of bench.py (no GPU): the byte and FLOP counts its
roofline divides by agree with the oracle's pinned counters for every
workload, the roof it picks for each configuration is the one the
intensity model gives, committed counter runs are only used for the
source they were taken on, and it refuses more than one GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from decode_attention_kv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cases():
    for name, w in synth.WORKLOADS.items():
        yield name, w
    # the sweep points of the benchmark's --set overrides
    yield "gqa_q8", bench.apply_overrides(synth.WORKLOADS["gqa_llama8b"], ["q_len=8"])
    yield "gla2_q2", bench.apply_overrides(synth.WORKLOADS["gla2"], ["q_len=2"])
    yield "gta_p1", bench.apply_overrides(synth.WORKLOADS["gta_8k"], ["page_size=1"])
    yield "mla_h16", bench.apply_overrides(synth.WORKLOADS["mla"], ["h_q=16"])


@pytest.mark.parametrize("name,w", list(_cases()), ids=[n for n, _ in _cases()])
def test_roofline_counts_match_the_oracle(name, w):
    L = synth.draw_seqlens(w, np.random.Generator(np.random.PCG64(w.seed)))
    assert bench.kv_bytes(w, L) == oracle.kv_bytes(w, L)
    assert bench.flops(w, L) == oracle.flops(w, L)


def _bound(w):
    L = synth.draw_seqlens(w, np.random.Generator(np.random.PCG64(w.seed)))
    t_mfma = bench.flops(w, L) / (bench.MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = bench.kv_bytes(w, L) / (bench.HBM_PEAK_GBPS * 1e9)
    return "mfma" if t_mfma > t_hbm else "hbm"


def test_roof_per_configuration():
    """At the spec peaks (ridge 312 FLOP/B) the q_len 4 latent workloads
    (512 and 967 FLOP/B) sit on the matrix-core roof, everything at q_len 1
    on the HBM roof, MLA at 242 FLOP/B included."""
    W = synth.WORKLOADS
    for name in ("gqa_llama8b", "gqa_llama8b_8k", "gta_8k", "gqa4_8k", "mla", "gla2"):
        assert _bound(W[name]) == "hbm", name
    for name in ("gla2_spec4_128k", "mla_spec4_128k"):
        assert _bound(W[name]) == "mfma", name


def test_counter_runs_are_used_only_for_their_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "decode_kernel_gta_8k_page_size_1_counters.txt").write_text(
        "# header: not a field\nkernel_source_sha256_16: 0123456789abcdef\n"
        "hbm_bytes_per_launch: 618779977\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    tag = bench.profile_tag("gta_8k[page_size=1]")
    assert tag == "gta_8k_page_size_1"
    assert bench.load_traffic("gta_8k[page_size=1]", "0123456789abcdef") == 618779977.0
    assert bench.load_traffic("gta_8k[page_size=1]", "fedcba9876543210") is None
    assert bench.load_traffic("gta_8k", "0123456789abcdef") is None


def test_overrides_rename_the_workload():
    w = bench.apply_overrides(synth.WORKLOADS["gqa_llama8b"], ["q_len=4"])
    assert w.name == "gqa_llama8b[q_len=4,causal=True]" and w.q_len == 4 and w.causal
    with pytest.raises(SystemExit):
        bench.apply_overrides(synth.WORKLOADS["gqa_llama8b"], ["name=x"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--gpus 1" in r.stderr
