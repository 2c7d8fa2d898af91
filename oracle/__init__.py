"""Plain, slow, fp64 CPU oracle of the spatially-adaptive DiT attention step.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU-baseline leg are the
only code allowed to import it; the product path (the HIP library and its Python binding) never does,
and this package imports nothing from that path.  It shares no code with it either: the only module
both sides use is `synthetic`, which draws seeded inputs and holds none of the method's arithmetic.

Parts (each module header names the passage of the pages it follows):
- attention: joint image+text softmax attention, dense (anchor refresh) and sensitive-row forms,
  with optional kept additive mask and the warmup cross-attention emission;
- elision: the row-constant mask-removal criterion;
- pcsp: sensitivity scores and the exact top-|S| partition;
- swcfg: per-token guidance combine;
- schedule: the warmup / anchor / sensitive-row trajectory.

Parity-unpinned readings (consistent, not checked against any printed value): the synthetic
image-block log-sum-exp, the blob law of the synthetic cross-attention logits and the min-max
normalisation of the scores.
"""
from . import attention, elision, pcsp, swcfg, schedule  # noqa: F401
