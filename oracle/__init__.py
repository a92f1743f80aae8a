"""Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
anything from this package.  The HIP library never calls it, and it imports
nothing from the HIP side (``gated_delta_rule_76_amd``), not even the input
generators: callers hand it numpy arrays.

What it follows: dimsnsums.com, page "GLM-5.3-FLASH" (the attention page),
section "How can a layer remember without rereading?" -- the printed update
rule S_t = (I - beta k k^T) Diag(alpha_t) S_{t-1} + beta k v^T, the sentence
under it that names S_t, I, beta and Diag(alpha_t), and the statement in the
same section that each head keeps a 128x128 state updated once per token.

Modules
-------
recurrence   token-by-token recurrence, fp64 numpy (the oracle proper)
bruteforce   the printed matrix product formed literally, fp64, tiny sizes
exact        the printed matrix product in exact rational arithmetic
scalar_gate  the scalar-gate (Gated DeltaNet) form: one decay rate per token
             and head instead of one per key channel
prologue     rates, strengths and unit q, k from pre-activations, then the
             recurrence
speculative  several tokens per sequence from a live state, every
             intermediate state kept, and the rollback to the accepted one
backward     gradients of the recurrence with respect to q, k, v, alpha, beta
             and the initial state, for given dL/do and dL/dS_T

Pins (every function is pinned by tests/test_oracle_pins.py,
tests/test_oracle_scalar_gate.py, tests/test_oracle_prologue.py,
tests/test_oracle_speculative.py and tests/test_oracle_backward.py against closed forms, invariants, a library
routine and a hand-worked golden example; see the module docstrings).  No function here is "parity unpinned".
"""

from .recurrence import (  # noqa: F401
    kda_recurrent,
    kda_decode_step,
    kda_step,
    rel_l2,
)
from .bruteforce import kda_bruteforce  # noqa: F401
from .exact import kda_exact  # noqa: F401
from .scalar_gate import gdn_decode_step, gdn_recurrent, gdn_step  # noqa: F401
from . import backward, prologue, speculative  # noqa: F401
