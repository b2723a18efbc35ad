"""CPU oracle for the DSpark verify sampler — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

* :mod:`oracle.philox`    Philox4x32-10 from its published definition, and the
                          uniforms / exponential clocks drawn from it.
* :mod:`oracle.dspark`    fp64 numpy reference of every step: Markov bias,
                          softmaxes, token-wise and block verification, the
                          exponential-race sampler (one clock per vocabulary id),
                          confidence head and adaptive choice.
* :mod:`oracle.schedule`  batch-level draft scheduler (greedy over prefix
                          survival against a token-count cost table, plain fp64)
                          and the online cost table rebuilt from live medians.
* :mod:`oracle.enumerate` exact enumeration of emitted-sequence distributions
                          on tiny vocabularies (no randomness).

Pins (tests marked ``not gpu``): Random123 known-answer vectors for Philox;
exact enumeration showing both verifiers reproduce target-only sampling;
closed forms (two-point softmax, one-hot Markov rows, 1 - TV acceptance,
k = 1 equivalence, q = p); the pages' worked numbers; Monte Carlo of the full
sampler against the enumeration; Monte Carlo of the Markov path (drafts from
the Markov drafter, verified, continued by the target) against target-only
sampling, with planted slips caught; brute force over every draft-count vector
for the batch scheduler and hand-computed medians for the online table.  Parity unpinned: which token the sampler
emits at a given seed is fixed only by this package's sampling convention
(any exact sampler is equally correct in distribution).
"""
from . import philox, dspark, enumerate, schedule  # noqa: F401

__all__ = ["philox", "dspark", "enumerate", "schedule"]
