"""CPU oracle for the MTP draft round.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the GPU library
computes: the draft-head step and the pending-pair flush (``head``), the draft
KV append and rollback (``kvcache``), speculative verification (``verify``) and
the round driver with its synthetic targets (``rounds``).  Arithmetic is fp64
except where a floating-point comparison decides an integer result (the
sampler's penalty, temperature, top-k and min-p steps), which both sides take
in fp32.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP path and imports nothing
from it; inputs arrive as numpy arrays produced by the seeded generators.

Sources (pages): "Ollama qwen3_5 MTP loader and SelfDraft path" (Facts),
"feat(inference): support the qwen3_5_mtp drafter for Qwen3.5/3.6/3.8 MTP
speculative decoding" (sections "Where the MTP weights actually live",
"Upstream contract to port", "Acceptance criteria" and the #1174 comment), and
the Ollama x/mlxrunner commit log.

Parity status: every function is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` (closed forms, special cases, invariants and brute
force); none is "parity unpinned".
"""
