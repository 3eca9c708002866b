"""MI355X (gfx950) ChunkAttention decode step: prefix-tree KV cache and
two-phase partition attention behind the C ABI of ``libchunkattn.so``."""

from .chunkattn import ChunkAttention, load_workload, slot_bytes, slots_needed  # noqa: F401
from ._capi import CaError  # noqa: F401
