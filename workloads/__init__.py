"""Seeded synthetic inputs for paged-attention workloads.

This module is shared by the tests, the benchmark and the smoke check: it feeds
the same inputs to the HIP library and to the CPU oracle. It holds none of the
method's arithmetic (no attention, no softmax, no scatter of values into
slots); it only draws shapes, context lengths, block-table structure, random
values and the NaN poison of slots that no sequence owns.
"""

from .generators import (  # noqa: F401
    CONFIGS,
    DecodeCase,
    PagedLayout,
    PrefillPart,
    draw_layout,
    make_case,
    make_config_case,
    to_numpy_bits,
)
