"""fp64 CPU oracle for paged-KV decode attention (GQA, GTA, MLA, GLA).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package never imports the product: the two share no
code.  Inputs come from the seeded generator module, which holds no attention
arithmetic.

Every function computes the plain definition in float64 on the exact input
values (bfloat16 inputs are upcast exactly), without blocking, fusion or
reordering beyond what the definition states.
"""
from .attention import (  # noqa: F401
    attend,
    attend_partial,
    decode_gqa,
    decode_gta,
    decode_latent,
    decode,
    gather_rows,
    logical_positions,
    merge_partials,
    rope_rotate_half,
)
from .append import kv_append, round_bf16  # noqa: F401
from .absorb import absorb_query, project_output  # noqa: F401
from .counts import (  # noqa: F401
    kv_bytes,
    kv_bytes_per_token,
    flops,
    flops_per_token_row,
    intensity,
    intensity_model,
    tp_duplication,
    count_touched_rows,
)
