"""CPU fp64 oracle for batched speculative-sampling verification.

TEST INFRASTRUCTURE. Only the tests, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import, call or execute anything in
this package. The product path (the HIP library and its Python binding) never
touches it, and it shares no code, tables or helpers with that path.

Everything is plain NumPy in float64, written from the pages' description of
the method (cited per function) and from the published definition of the
Philox4x32-10 generator.
"""

from . import philox  # noqa: F401
from .specverify import (  # noqa: F401
    ACCEPT, SAMPLE, FLAG_EPS, decode_logits, normalize_rows, accept_from_logprobs, verify,
)
from .acceptance import acceptance_probability, outcome_law, expected_accept_length  # noqa: F401
from .speculation_cache import geometric_fanout, residual_topf, cache_lookup  # noqa: F401
from . import bandit  # noqa: F401
from . import branch_pruning  # noqa: F401
