"""CPU oracle for the VSA-H3 attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in
this package.  The product path (``video_dit_block_amd``) never imports it and
shares no code, header, table or helper with it.

See ``oracle/vsa_h3.py`` for the definition, the readings taken where the pages
leave a step open, and which functions are pinned by which tests.
"""
from .vsa_h3 import (  # noqa: F401
    TEXT, COND, AUDIO, VIDEO,
    Geometry, GeometryError, geometry, topk_count, to_f32, pool_canonical,
    scores_canonical, select_topk, key_tiles, fine_item, fine, coarse, combine,
    round_bf16_from_f64, forward, forward_head, qk_norm_rope, prep_qk, e4m3_encode,
    ref_keep_count, select_ref,
    e4m3_decode, quantize_rows, dequantize_rows, E4M3_MAX,
)
