"""Compile libattn_decode.so (gfx950) in-tree with hipcc.

Sources: csrc/attn_host.cpp (host-only planning and checks),
csrc/attn_decode.hip (entry points, merge kernel), one translation unit
per decode kernel family (attn_general.hip, attn_narrow.hip,
attn_wide.hip), the cache append (attn_append.hip), the projections
around the latent kernel (attn_absorb.hip) and the measurement probes
(attn_probe.hip), compiled in parallel.  Packed-fp32 VALU ops are disabled
for device code.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libattn_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ("attn_host.cpp", "attn_decode.hip", "attn_general.hip", "attn_narrow.hip",
           "attn_wide.hip", "attn_append.hip", "attn_absorb.hip", "attn_probe.hip")

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source flags.  The GQA/GTA streaming kernel accumulates its MFMAs in
# ordinary VGPRs: in the accumulation registers (the compiler's default) it
# copied every accumulator out and back around each 16-key slice, for the
# rarely taken rescale branch and the loop exits, which cost about as many
# cycles as the slice's MFMAs; measured no occupancy loss for any of its
# instantiations, and fewer spills.
EXTRA_FLAGS = {"attn_narrow.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"),
          "--offload-arch=" + ARCH]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + out)
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = True) -> str:
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC] + COMMON + DEVICE_FLAGS + EXTRA_FLAGS.get(src, []) + lang +
                    ["-c", os.path.join(PKG, "csrc", src), "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
