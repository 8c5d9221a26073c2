"""CPU oracle for exact blockwise attention and the blockwise feed-forward (fp64, numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the bench's CPU-baseline leg, never
by the library or its binding.  It shares no code with the HIP path.  See ``oracle.fp64`` (attention, the
merge, the chunked fold) and ``oracle.ffn64`` (the blockwise feed-forward) for the passages each function
follows and the readings taken where the pages are silent.
"""
from .fp64 import (NEG_INF, attention, blockwise_head, chunk_bounds, chunked_head, merge,  # noqa: F401
                        naive_head, visible)
