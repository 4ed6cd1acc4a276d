"""CPU oracle for the selected-token logprob — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or call anything in this package. The library (``invariant_lm_head_deterministic_amd``) never does,
and this package imports nothing from it: the two share no code, no constants and no helpers.
Both are fed the same bytes by ``datagen``.

What it computes is the plain mathematical definition, in float64, of the path the pages centre
on: the LM-head projection, log-softmax over the vocabulary, and the gather of the target token's
log-probability (nxbn.cn blog, §3.1: logprob is log_softmax of the logits taken at the token; the
RL-Kernel v0.1.0 summary page, strict-path boundary table, row "Linear logprob"). The vocab split,
target ownership and cross-rank merge that the pages prescribe only change rounding, so the oracle
computes the unsplit reduction. Parity status of each function is stated in its docstring and in
``oracle.logprob.PINS``.
"""

from .backward import dlogits, grads, rmsnorm_backward  # noqa: F401
from .backward import PINS as BACKWARD_PINS  # noqa: F401
from .logprob import (  # noqa: F401
    PINS,
    bf16_bits_to_f64,
    entropy_rows,
    log_softmax_rows,
    logits,
    logprob,
    logprob_bruteforce,
    logsumexp_rows,
    rmsnorm_bf16,
    round_to_bf16,
    sample_targets,
    select_logprob,
)
