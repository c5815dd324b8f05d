"""fp64 CPU oracle for speculative-decoding verification — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The library never does, and the two share no code;
inputs reach both from the ``workloads`` generators.

Parity pins (each checked by ``tests/test_oracle_*.py`` without a GPU):
  * Philox4x64-10: bit-exact against numpy's independent Philox generator.
  * softmax: scipy's softmax, closed forms (uniform, two-token logistic).
  * bf16 widening: torch's bfloat16 -> float32 conversion.
  * inverse CDF and acceptance: exact law computed with Fractions, interval
    probes, numpy's searchsorted on cumulative sums.
  * the whole sampling rule: exact enumeration showing the output law equals
    the target's (the pages' exactness guarantee), chi-square at 10^6 trials.
  * greedy: argmax-prefix properties, and the sampling rule's T -> 0 limit.
  * tree: a chain tree equals greedy; brute-force path enumeration.
  * ragged batches: every request equals the dense rule on its own rows with
    the same uniforms, whatever the mix of draft counts; bad offsets refuse
    only their own request.
  * grammar bitmasks: the bit layout against numpy's own bit unpacking; an
    all-ones mask changes nothing; emitted tokens are always allowed and
    disallowed drafts are always rejected.
  * top-k / top-p filters: brute force over every upper set of a row
    (top-k: the largest cut holding at least k tokens; top-p: the largest
    cut holding at least top_p of the mass), hand-computed small rows, the
    switched-off and single-token limits, and the exact law of the filtered
    rule (it emits the filtered target distribution).
Parity unpinned: individual draws whose uniform lies within 1e-5 of an
acceptance threshold or CDF boundary (the GPU works in fp32); they are
counted by the parity tests, not matched.
"""
from .philox import philox4x64_10, request_uniforms, uniform24  # noqa: F401
from .verify import *  # noqa: F401,F403
