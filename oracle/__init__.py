"""CPU oracle for Reference Sliding Window Attention (R-SWA).

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
float64 definition that the HIP path is checked against. Only the test suite,
the smoke check of the package entry file and the CPU-baseline leg of the
benchmark may import it. The HIP library and its Python binding never import
it, and it imports nothing from them: the two share no code, tables or
constants. Inputs come from the separate `workloads` generator module.

Every function here is pinned by a CPU test against something other than
itself (hand-derived visible sets and queue states, closed forms, a library
attention routine, brute force with a dense mask) except where its docstring
says "parity unpinned".
"""
from .rswa import (  # noqa: F401
    reference_segment, decode_window, visible_positions, attend, decode_output,
    cache_size_mha, cache_size_rswa, cache_ratio, FifoCache, ring_slot, ring_image,
    simulate_decode, masked_visible_columns, masked_attention_rows,
    masked_logsumexp_rows, masked_attention_backward,
    PREFIX_CAUSAL, PREFIX_FULL,
)
