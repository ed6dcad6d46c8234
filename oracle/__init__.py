"""Float64 CPU oracle of the batched speculative-sampling verifier.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports, links or calls it, and
the oracle shares no code with that path.
"""

from .verifier import (  # noqa: F401
    SAMPLE_FALLBACK_MASS,
    accept_draft,
    adjusted_target_probs,
    inverse_cdf,
    inverse_cdf_many,
    residual_weights,
    row_statistics,
    target_probs,
    verify_greedy,
    verify_probs,
    verify_ragged,
    verify_request,
)
