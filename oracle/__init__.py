"""CPU oracle of the ISD verify/propose step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP path.
"""

from .isd_oracle import (  # noqa: F401
    TIE_WINDOW,
    accept_ratio,
    alpha_sample,
    argmax_first,
    decode_logits,
    inverse_cdf,
    lm_head,
    propose_greedy,
    propose_sample,
    softmax,
    verify_greedy,
    verify_sample,
)
