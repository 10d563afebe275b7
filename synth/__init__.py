"""Seeded synthetic inputs shared by the tests, the benchmark and smoke().

This package holds no arithmetic of the method: it only draws random
numbers and packs them.  Both the oracle side and the HIP side consume the
same bytes produced here.
"""
from .packs import (  # noqa: F401
    CONFIGS,
    PackConfig,
    Pack,
    pack_lengths,
    make_pack,
    make_custom_pack,
    random_block_lists,
)
