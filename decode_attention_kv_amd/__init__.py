"""MI355X-native paged-KV decode attention (GQA, GTA, MLA, GLA).

The compute path is the HIP library ``libattn_decode.so`` (gfx950 kernels
behind a C ABI, declared in include/attn_decode.h); ``binding`` is its thin
ctypes wrapper.  ``synth`` draws seeded inputs.  Submodules load lazily so
that drawing inputs never touches the GPU library.
"""
__all__ = ["binding", "synth"]
