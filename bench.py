#!/usr/bin/env python3
"""Benchmark of paged-KV decode attention on one MI355X.

One step is the whole hot path over one batch: the host split plan (packed
into the kernels' launch arguments when it fits, else uploaded), the
split-KV decode kernel and the log-sum-exp merge kernel.  Inputs
are seeded and synthetic and sit in HBM before timing starts.  Before every
timed step a 1 GiB read evicts the caches (L2 and the 256 MB Infinity
Cache) outside the timed interval, so every step reads its cache from HBM
(a read leaves no dirty lines whose write-back would compete with the step).

Prints one JSON line: KV GB/s (algorithmic cache bytes / step time) as the
value, tokens/s, the decode kernel's roofline (achieved GB/s from HIP events
on the launch stream vs the 8 TB/s HBM peak) and the fp64 oracle timed on a
bounded sample on the host cores.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "decode_attention_kv_amd", "csrc")
# sources that define the decode kernel a workload runs (shared headers + its
# kernel family); the hash ties committed counter runs to that code
KERNEL_SRCS = {
    "narrow": ("attn_device.h", "attn_kernels.h", "attn_narrow.hip"),
    "wide": ("attn_device.h", "attn_kernels.h", "attn_wide.hip"),
    "general": ("attn_device.h", "attn_kernels.h", "attn_general.hip"),
}
DESCRIPTIONS = {
    "gqa_llama8b": "GQA decode, Llama-3-8B layer: bf16, B=32, q_len=1, h_q=32, h_kv=8, d=128, "
                   "seqlen ~ U[1024,8192], page 64, permuted page table",
    "gqa_llama8b_8k": "GQA decode, Llama-3-8B layer at 8K: bf16, B=32, h_q=32, h_kv=8, d=128, "
                      "seqlen 8192, page 64, permuted",
    "gta_8k": "GTA decode: bf16, B=64, h_q=32, 4 tied heads x 128 + one 64-wide RoPE key "
              "(theta 1e4, in-kernel), seqlen 8192, page 64, permuted",
    "gqa4_8k": "GQA-4 at the GTA shape: bf16, B=64, h_q=32, h_kv=4, d=128, seqlen 8192",
    "mla": "MLA latent decode: bf16, B=128, h_q=128, d_c=512 + RoPE 64, seqlen ~ U[2048,32768]",
    "gla2": "GLA-2 latent decode: bf16, B=128, h_q=128, 2 x d_c=256 + RoPE 64, "
            "seqlen ~ U[2048,32768]",
    "gla2_spec4_128k": "GLA-2 speculative verify: bf16, B=16, q_len=4 causal, h_q=128, "
                       "2 x 256 + 64, seqlen 131072",
    "mla_spec4_128k": "MLA speculative verify: bf16, B=16, q_len=4 causal, h_q=128, 512 + 64, "
                      "seqlen 131072",
    "gqa_fp32_tiny": "GQA decode fp32 tiny: B=2, h_q=8, h_kv=2, d=64, seqlen 256",
}


def kv_bytes(w, seqlens):
    """Algorithmic cache bytes of one step: every cached element of every
    token read once (K and V, or tied state + RoPE key, or latent + RoPE)."""
    if w.kind == "gqa":
        per_tok = 2 * w.groups * w.head_dim * w.elem_bytes
    else:
        per_tok = (w.groups * w.head_dim + w.d_rope) * w.elem_bytes
    return int(sum(int(L) for L in seqlens)) * per_tok


def flops(w, seqlens):
    """2 FLOPs per multiply-add of QK^T and P.V over every visible
    (query row, key) pair."""
    per = 4 * w.head_dim if w.kind != "latent" else 2 * (w.head_dim + w.d_rope) + 2 * w.head_dim
    pairs = 0
    for L in seqlens:
        L = int(L)
        pairs += sum(L - w.q_len + 1 + t for t in range(w.q_len)) if (w.causal and w.q_len > 1) \
            else L * w.q_len
    return pairs * w.h_q * per


def kernel_family(w):
    """Decode kernel family of a workload (the streaming kernels take bf16 at
    any page size; the general kernel fp32 and the shapes they do not)."""
    if w.dtype != "bf16":
        return "general"
    if w.kind == "latent":
        return "wide" if w.d_rope == 64 and w.head_dim in (256, 512) else "general"
    ok = (w.head_dim in (64, 128) if w.kind == "gqa" else (w.head_dim == 128 and w.d_rope == 64))
    return "narrow" if ok and w.group_size * w.q_len <= 64 else "general"


def kernel_sha(w):
    """Hash of the sources of the workload's decode kernel and of the build
    script (its compiler flags): counter-based traffic is reported only while
    it was taken on exactly this code."""
    h = hashlib.sha256()
    for name in KERNEL_SRCS[kernel_family(w)]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "decode_attention_kv_amd", "_build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def profile_tag(workload):
    """File-name form of a workload name (overrides such as
    gqa_llama8b_8k[page_size=1] become gqa_llama8b_8k_page_size_1)."""
    import re
    return re.sub(r"[^A-Za-z0-9_.-]+", "_", workload).strip("_")


def load_traffic(workload, sha):
    """HBM bytes per decode launch from committed rocprofv3 counter runs,
    only if they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{profile_tag(workload)}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def apply_overrides(w, items):
    """Workload `w` with FIELD=VALUE overrides (typed like the field); the
    name records them, so no committed counter run is attributed to it."""
    import dataclasses
    if not items:
        return w
    types = {f.name: f.type for f in dataclasses.fields(w)}
    kw = {}
    for it in items:
        k, _, v = it.partition("=")
        if k not in types or k == "name":
            raise SystemExit(f"--set: unknown workload field {k!r}")
        t = types[k] if isinstance(types[k], type) else \
            {"int": int, "float": float, "bool": bool, "str": str}[types[k]]
        kw[k] = (v.lower() in ("1", "true", "yes")) if t is bool else t(v)
    if "seqlen_hi" in kw and "max_seqlen" not in kw:
        kw["max_seqlen"] = max(w.max_seqlen, kw["seqlen_hi"])
    if kw.get("q_len", w.q_len) > 1 and "causal" not in kw:
        kw["causal"] = True
    tag = ",".join(f"{k}={v}" for k, v in kw.items())
    return w.with_(name=f"{w.name}[{tag}]", **kw)


def value_max(w, inp, batch_index):
    """max |V| over the values the sampled sequences attend (V pool, tied
    state or latent), read through the page table."""
    import numpy as np

    src = inp["pool1"] if w.kind == "gqa" else inp["pool0"]
    m = 0.0
    for b in batch_index:
        L = int(inp["seqlens"][b])
        n = -(-L // w.page_size)
        if n:
            v = src[inp["page_table"][b, :n]].reshape(-1, src.shape[2], src.shape[3])[:L]
            m = max(m, float(np.abs(v).max()))
    return m or 1.0


# parity bar for bf16 inputs with fp32 accumulation: relative L2 error of the
# compared output <= 5e-3 and max abs error <= 1e-2 * max|V|
REL_L2_MAX = 5e-3
MAX_ABS_FRAC = 1e-2


def cpu_baseline(w, inp, seconds, gpu_out=None):
    """The fp64 oracle on a bounded sample of the same batch: whole sequences
    in batch order, repeating the batch, until about `seconds` of work.

    With `gpu_out` (the benched step's output, [B, T, H, d_v] on the host),
    the oracle's output for every sequence of the first pass is also compared
    with the GPU's rows of that sequence (outside the timed oracle work)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    cores = len(os.sched_getaffinity(0))
    done, t_used = [], 0.0
    err2 = ref2 = 0.0
    max_abs, compared = 0.0, []
    while t_used < seconds and w.batch > 0:
        for b in range(w.batch):
            t0 = time.perf_counter()
            ref, _ = oracle.decode(w, inp, batch_index=[b])
            t_used += time.perf_counter() - t0
            if gpu_out is not None and b not in compared:
                e = gpu_out[b].astype(np.float64) - ref[0]
                err2 += float((e * e).sum())
                ref2 += float((ref[0] * ref[0]).sum())
                max_abs = max(max_abs, float(np.abs(e).max()) if e.size else 0.0)
                compared.append(b)
            done.append(b)
            if t_used >= seconds:
                break
    L = inp["seqlens"][done]
    kvb = oracle.kv_bytes(w, L)
    passes = len(done) / w.batch
    res = {"value": kvb / t_used / 1e9, "unit": "GB/s", "cores": cores, "blas_threads": blas,
           "kind": "oracle",
           "sample": f"{len(done)} sequence decodes ({passes:.2f} passes over the {w.batch}-sequence "
                     f"batch, lengths {int(L.min())}..{int(L.max())}) in {t_used:.1f} s; "
                     f"{len(done) * w.q_len / t_used:.1f} decode tokens/s"}
    parity = None
    if gpu_out is not None and compared:
        rel = (err2 ** 0.5) / (ref2 ** 0.5) if ref2 > 0 else err2 ** 0.5
        bound = MAX_ABS_FRAC * value_max(w, inp, compared)
        parity = {"sequences": compared, "rel_l2": rel, "max_abs": max_abs,
                  "rel_l2_max": REL_L2_MAX, "max_abs_max": bound,
                  "pass": bool(rel <= REL_L2_MAX and max_abs <= bound)}
    return res, parity


def measure_ceilings(dev, binding, reps=5):
    """Streaming-read and bf16 MFMA ceilings of this GPU from the library's
    probe kernels (event-timed on the launch stream): reads of a 4 GiB
    buffer (far past the 256 MB Infinity Cache) into registers and straight
    into LDS, and register-only MFMA products."""
    import torch

    n = 4 << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    out = {}
    for mode, name in ((0, "read_vgpr_nt_gbps"), (1, "read_lds_nt_gbps")):
        best = 0.0
        for k in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = binding.attn_probe_stream_read(buf.data_ptr(), n, mode, sink.data_ptr(), s)
            e1.record(stream)
            if st != binding.ATTN_OK:
                raise binding.AttnError(st, "attn_probe_stream_read")
            e1.synchronize()
            if k >= 2:
                best = max(best, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        out[name] = round(best, 1)
    del buf
    best = 0.0
    for k in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st, fl = binding.attn_probe_mfma(20000, sink.data_ptr(), s)
        e1.record(stream)
        if st != binding.ATTN_OK:
            raise binding.AttnError(st, "attn_probe_mfma")
        e1.synchronize()
        if k >= 2:
            best = max(best, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    out["mfma_bf16_tflops"] = round(best, 1)
    out["hbm_read_gbps"] = max(out["read_vgpr_nt_gbps"], out["read_lds_nt_gbps"])
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_llama8b_8k",
                    help="default: the Llama-3-8B-shaped GQA layer at 8K context")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="evict L2 / Infinity Cache before each timed step by reading (default) "
                         "or writing a 1 GiB buffer, outside the timed interval")
    ap.add_argument("--layout", choices=["nhd", "hnd"], default="hnd",
                    help="pool layout: [pages][page][heads][width] (nhd) or "
                         "[pages][heads][page][width] (hnd), passed to the kernel as strides")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--chunk-tokens", type=int, default=0, help="force the split chunk size")
    ap.add_argument("--merge", choices=["fused", "launch"], default="launch",
                    help="launch: a merge launch after the decode (faster here); fused: "
                         "the decode kernel merges split rows itself (plan counters)")
    ap.add_argument("--plan-mem", choices=["auto", "inline", "device", "host"], default="auto",
                    help="inline: the plan travels in the kernels' launch arguments (no "
                         "upload); device: copy each step's plan to HBM; host: kernels read "
                         "it from pinned host memory; auto: inline when it fits, else device")
    ap.add_argument("--with-append", action="store_true",
                    help="each step first writes the q_len newest cache rows of every sequence "
                         "(attn_kv_append, the same rows again) before planning and decoding")
    ap.add_argument("--with-absorb", action="store_true",
                    help="latent workloads: each step also forms the decode's query from "
                         "q_nope / q_rope with per-head key up-projections (128 -> d_c) before "
                         "the decode and projects the latent output to 128 per head after it "
                         "(attn_latent_absorb_query / attn_latent_project_output, random "
                         "weights)")
    ap.add_argument("--queue", choices=["auto", "on", "off"], default="auto",
                    help="on: the GQA kernel hands items out through a work-queue counter; "
                         "auto (default): on for GQA pages under 16 tokens, where it measured "
                         "faster on ragged lengths (slower on larger pages)")
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=VALUE",
                    help="override a workload field (e.g. q_len=2, h_q=16, groups=1, "
                         "page_size=1, batch=64); the result is then not the named workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure this GPU's streaming-read and bf16 MFMA ceilings with "
                         "the library's probe kernels and print them")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the ceiling probes after the timed steps")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU decode path only; run it with --gpus 1 "
              "(sharding across GPUs is described, not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decode_attention_kv_amd import binding, synth

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return
    if args.ceilings:
        print(json.dumps(measure_ceilings(dev, binding)))
        return

    w = apply_overrides(synth.WORKLOADS[args.workload], args.set)
    print(f"[bench] drawing inputs for {w.name}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev_t(a):
        return None if a is None else torch.from_numpy(a).to(dt).to(dev)

    def dev_pool(a):
        t = dev_t(a)
        if t is None or args.layout == "nhd":
            return t
        # same logical [pages][page][heads][width] view over head-major storage
        return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)

    q = dev_t(inp["q"])
    pool0, pool1, rope = dev_pool(inp["pool0"]), dev_pool(inp["pool1"]), dev_pool(inp["rope"])
    page_table = torch.from_numpy(inp["page_table"]).to(dev)
    seqlens = torch.from_numpy(inp["seqlens"]).to(dev)
    seqlens_host = np.ascontiguousarray(inp["seqlens"], dtype=np.int32)
    B, T, H = w.batch, w.q_len, w.h_q
    d_v = w.head_dim
    kv = binding.paged_kv(pool0, pool1, rope, page_table, seqlens)
    shp = binding.shape(w.kind, kv.dtype, B, T, H, w.groups, w.head_dim, w.d_rope, w.page_size,
                        w.causal)
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    fused = args.merge == "fused"
    flags = (binding.ATTN_CAUSAL if w.causal else 0) | (0 if fused else binding.ATTN_DEFER_MERGE)

    max_items = binding.attn_decode_plan_max_items(B, w.groups, int(max(1, seqlens_host.max())))
    # two pinned host plan buffers (a step rewrites one while the other may
    # still be in flight to the device), each [seqinfo rows | item rows], so a
    # step uploads its plan with one copy
    host_buf = [torch.zeros((B + max_items, 4), dtype=torch.int32).pin_memory() for _ in range(2)]
    # end event of the last step that read each host buffer
    released = [None, None]
    dev_buf = torch.zeros((B + max_items, 4), dtype=torch.int32, device=dev)
    counters = None  # merge counters (zero-filled once), sized from the first plan
    placement = [None]  # where the last plan went: inline / device / host
    use_queue = args.queue == "on" or (args.queue == "auto" and w.kind == "gqa" and
                                       w.page_size < 16)
    queue = torch.zeros(1, dtype=torch.int32, device=dev) if use_queue else None

    def make_plan(k):
        i = k % 2
        if released[i] is not None:
            released[i].synchronize()
        hb = host_buf[i].numpy()
        st, plan = binding.attn_decode_plan(shp, seqlens_host, cu, args.chunk_tokens, hb[B:],
                                            hb[:B], max_items)
        if st != binding.ATTN_OK:
            raise binding.AttnError(st, "attn_decode_plan")
        n = B + plan.n_items
        if args.plan_mem == "inline" or (args.plan_mem == "auto" and plan.inline_ok):
            if not plan.inline_ok:
                raise SystemExit("the plan does not fit the launch arguments")
            # packed from the host arrays into the kernels' launch arguments
            plan.seqinfo = plan.items = None
            placement[0] = "inline"
        elif args.plan_mem == "host":
            # pinned host memory is mapped into the device address space
            base = host_buf[i].data_ptr()
            plan.seqinfo, plan.items = base, base + B * 16
            placement[0] = "host"
        else:
            dev_buf[:n].copy_(host_buf[i][:n], non_blocking=True)
            base = dev_buf.data_ptr()
            plan.seqinfo, plan.items = base, base + B * 16
            placement[0] = "device"
        if queue is not None:
            plan.queue = queue.data_ptr()
        if fused:
            nonlocal counters
            if counters is None:
                counters = torch.zeros(max(1, binding.attn_decode_counter_count(plan, H)),
                                       dtype=torch.int32, device=dev)
            plan.counters = counters.data_ptr()
        return plan, i

    plan0, _ = make_plan(0)
    torch.cuda.synchronize()
    ws_bytes = binding.attn_decode_workspace_size(plan0, H, d_v)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, H, d_v), dtype=dt, device=dev)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    flush = None if args.flush == "none" else torch.ones(1 << 28, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream

    if args.with_append:
        # the newest q_len rows of every sequence, written back in place each step
        T_new = w.q_len
        rows = {}
        for key, pool in (("new0", pool0), ("new1", pool1), ("rope", rope)):
            if pool is None:
                rows[key] = None
                continue
            t = torch.empty((B, T_new) + tuple(pool.shape[2:]), dtype=pool.dtype, device=dev)
            for b in range(B):
                for tt in range(T_new):
                    pos = int(seqlens_host[b]) - T_new + tt
                    if pos >= 0:
                        t[b, tt] = pool[int(inp["page_table"][b, pos // w.page_size]),
                                        pos % w.page_size]
            rows[key] = t if key != "rope" else t[:, :, 0, :].contiguous()
        app_args = (T_new, pool0.shape[2], pool0.shape[3], rows["new0"].data_ptr(),
                    None if rows["new1"] is None else rows["new1"].data_ptr(),
                    0 if rows["rope"] is None else w.d_rope,
                    None if rows["rope"] is None else rows["rope"].data_ptr(), 0.0)

    if args.with_absorb:
        if w.kind != "latent":
            print("--with-absorb applies to latent workloads", file=sys.stderr)
            sys.exit(2)
        D_NOPE = D_V = 128
        pin = synth.make_projection_inputs(B * T, H, D_NOPE, d_v, w.d_rope, D_V, seed=w.seed + 1)

        def _bf(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)

        q_nope, q_rope, w_uk, w_uv = (_bf(pin["q_nope"]), _bf(pin["q_rope"]), _bf(pin["w_uk"]),
                                      _bf(pin["w_uv"]))
        out_v = torch.empty((B * T, H, D_V), dtype=torch.bfloat16, device=dev)

    def step(k, evs, inner):
        """One step: plan (host) + upload, decode (which merges split rows
        itself, or a merge launch after it).  evs = [start, before decode,
        after decode, end]; the inner two are recorded only when `inner`
        (each recorded event costs the stream a few microseconds, so steps
        without them give the step time)."""
        evs[0].record(stream)
        if args.with_append:
            st = binding.attn_kv_append(kv, *app_args, s)
            if st != binding.ATTN_OK:
                raise binding.AttnError(st, "attn_kv_append")
        plan, slot = make_plan(k)
        if args.with_absorb:  # the decode's query, written in place
            st = binding.attn_latent_absorb_query(q_nope.data_ptr(), q_rope.data_ptr(),
                                                  w_uk.data_ptr(), q.data_ptr(), B * T, H,
                                                  D_NOPE, d_v, w.d_rope, s)
            if st != binding.ATTN_OK:
                raise binding.AttnError(st, "attn_latent_absorb_query")
        if inner:
            evs[1].record(stream)
        if w.kind == "gqa":
            st = binding.attn_decode_gqa(kv, q.data_ptr(), out.data_ptr(), lse.data_ptr(), T, H,
                                         w.groups, d_v, w.softmax_scale, flags, plan,
                                         ws.data_ptr(), ws_bytes, s)
        elif w.kind == "gta":
            st = binding.attn_decode_gta(kv, q.data_ptr(), out.data_ptr(), lse.data_ptr(), T, H,
                                         w.groups, d_v, w.d_rope, 1, w.rope_theta,
                                         w.softmax_scale, flags, plan, ws.data_ptr(), ws_bytes, s)
        else:
            st = binding.attn_decode_latent(kv, q.data_ptr(), out.data_ptr(), lse.data_ptr(), T,
                                            H, w.groups, d_v, w.d_rope, w.softmax_scale, flags,
                                            plan, ws.data_ptr(), ws_bytes, s)
        if st != binding.ATTN_OK:
            raise binding.AttnError(st, "decode")
        if inner:
            evs[2].record(stream)
        if not fused:
            st = binding.attn_decode_merge(plan, H, d_v, kv.dtype, ws.data_ptr(), ws_bytes,
                                           out.data_ptr(), lse.data_ptr(), s)
            if st != binding.ATTN_OK:
                raise binding.AttnError(st, "merge")
        if args.with_absorb:
            st = binding.attn_latent_project_output(out.data_ptr(), w_uv.data_ptr(),
                                                    out_v.data_ptr(), B * T, H, d_v, D_V, s)
            if st != binding.ATTN_OK:
                raise binding.AttnError(st, "attn_latent_project_output")
        if inner and fused and not args.with_absorb:
            evs[3] = evs[2]  # the step ends with the decode kernel
        else:
            evs[3].record(stream)
        released[slot] = evs[3]

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for k in range(args.warmup):
        step(k, [torch.cuda.Event() for _ in range(4)], False)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    # odd steps bracket the decode kernel for its launch duration; even
    # steps (all steps when only one is timed) give the step time
    inner = [args.steps > 1 and k % 2 == 1 for k in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        if args.flush == "write":
            flush.fill_(k)
        elif args.flush == "read":
            flush.max()
        step(k, evs[k], inner[k])
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall

    step_ms = np.array([e[0].elapsed_time(e[3]) for e, f in zip(evs, inner) if not f])
    inst = [e for e, f in zip(evs, inner) if f] or evs[:0]
    if inst:
        dec_ms = np.array([e[1].elapsed_time(e[2]) for e in inst])
        merge_ms = np.array([e[2].elapsed_time(e[3]) if e[3] is not e[2] else 0.0 for e in inst])
        inst_step_ms = np.array([e[0].elapsed_time(e[3]) for e in inst])
    else:  # a single timed step: its whole time stands for the kernel
        dec_ms = merge_ms = inst_step_ms = step_ms
    kvb = kv_bytes(w, seqlens_host)
    fl = flops(w, seqlens_host)
    ms = float(step_ms.mean())
    gbps = kvb / (ms * 1e-3) / 1e9
    dec_gbps = kvb / (float(dec_ms.mean()) * 1e-3) / 1e9
    dec_tflops = fl / (float(dec_ms.mean()) * 1e-3) / 1e12
    tokens = B * T
    sha = kernel_sha(w)

    # the last timed step's output, kept for the comparison with the oracle
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    out_host = out.float().cpu().numpy()

    ceil = None
    if not args.no_ceilings:
        print("[bench] ceiling probes", file=sys.stderr, flush=True)
        ceil = measure_ceilings(dev, binding)

    # the dominant kernel's roof: HBM unless the bf16 matrix work takes longer
    # at peak than the cache read (latent heads at high intensity)
    mfma_bound = fl / (MFMA_BF16_PEAK_TFLOPS * 1e12) > kvb / (HBM_PEAK_GBPS * 1e9)
    if mfma_bound:
        roofline = {"bound": "mfma", "achieved": round(dec_tflops, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(dec_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4)}
    roofline.update({"traffic": load_traffic(w.name, sha),
                     "algorithmic_bytes_per_launch": int(kvb),
                     "algorithmic_flops_per_launch": int(fl),
                     "hbm_gbps": round(dec_gbps, 1),
                     "hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "mfma_tflops": round(dec_tflops, 1),
                     "mfma_frac": round(dec_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "kernel_ms_mean": round(float(dec_ms.mean()), 5),
                     "kernel_source_sha256_16": sha})
    if ceil is not None:
        roofline["measured_ceilings"] = ceil
        roofline["frac_of_measured"] = round(
            dec_tflops / ceil["mfma_bf16_tflops"] if mfma_bound
            else dec_gbps / ceil["hbm_read_gbps"], 4)

    line = {"metric": "decode-attn KV GB/s (% of MI355X HBM peak) and tokens/s at 8K ctx",
            "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": f"{w.name}: {DESCRIPTIONS.get(w.name.split('[')[0], w.name)}",
                       "batch": B, "q_len": T, "h_q": H, "groups": w.groups,
                       "head_dim": w.head_dim, "d_rope": w.d_rope,
                       "mean_seqlen": float(seqlens_host.mean()), "page_size": w.page_size,
                       "kv_bytes_per_step": int(kvb), "gpus": 1, "layout": args.layout,
                       "cache_flush": args.flush, "plan_mem": placement[0],
                       "with_append": bool(args.with_append),
                       "with_absorb": bool(args.with_absorb), "queue": "on" if use_queue else "off",
                       "merge": args.merge},
            "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
            "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "step_ms_median": round(float(np.median(step_ms)), 5),
            "decode_ms_mean": round(float(dec_ms.mean()), 5),
            "merge_ms_mean": round(float(merge_ms.mean()), 5),
            "instrumented_step_ms_mean": round(float(inst_step_ms.mean()), 5),
            "timing": "value and ms_per_step from the steps without inner events; decode and "
                      "merge times from the steps that bracket them",
            "wall_ms_per_step_incl_flush": round(1e3 * t_wall / args.steps, 5),
            "plan": {"items": int(plan0.n_items), "max_splits": int(plan0.max_splits),
                     "partial_slots": int(plan0.n_partial_slots)},
            "roofline": roofline}
    parity = None
    if not args.no_cpu_baseline:
        print("[bench] oracle cpu baseline (and the benched output against it)", file=sys.stderr,
              flush=True)
        line["cpu_baseline"], parity = cpu_baseline(w, inp, args.cpu_seconds, out_host)
        line["parity"] = parity
    print(json.dumps(line), flush=True)
    if parity is not None and not parity["pass"]:
        print(f"[bench] the benched output does not match the oracle: {parity}", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
