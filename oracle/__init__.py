"""CPU oracle for the exact attention forward (float64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does, and it shares no
code with the GPU library.

* ``attention``: the plain materialised definition (the oracle itself).
* ``online``: a float64 model of the tiled online-softmax method, checked
  against the oracle to show the method is exact before any kernel exists.

Every function here is pinned by tests that do not reuse its own formulas
(arbitrary-precision brute force, a second library's attention routine,
closed forms and invariants); none is "parity unpinned".
"""
from .attention import (attention_forward, attention_rows, attention_decode,  # noqa: F401
                        attention_varlen, attention_varlen_rows, packed_segments,
                        probabilities,
                        masked_scores, softmax_stats, allowed_mask, clamp_key_len)
from .online import online_forward  # noqa: F401
from .backward import attention_backward  # noqa: F401
