"""Seeded synthetic video-DiT Q/K/V generator shared by the tests and the bench.

Holds no attention, pooling or selection arithmetic: it only draws inputs.
"""

from .video_qkv import (  # noqa: F401
    CONFIGS,
    VideoSpec,
    config_spec,
    gen_qkv,
    merge_sides,
    micro_heads,
    mod_pattern_mask,
    rotation_offset,
)
