"""CPU oracle for the batch-invariant speculative-verify path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct reference that the GPU library is checked against.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import
it.  The library itself never imports, calls or links anything here, and
nothing here imports the library: the two share no kernels, helpers,
tables or layout code.  Floating point is evaluated in fp64 from the exact
values of the fp16 / bf16 / fp32 inputs.

Sources (cited by page title and section in each module):

* tokenstrom.com, "'Lossless,' but not quite: why speculative decoding
  changes your LLM's answers".
* ramgpt.org, "When Lossless Speculation Stops Being Lossless on Blackwell".
* proofoftech.org, "'Lossless' speculative decoding is a property of the
  math, not your deployment."

Modules:

* ``formats``   exact decoding of fp16 / bf16 bits and of the 4-bit codes.
* ``qgemm``     4-bit block-quantised matrix times a few activation rows.
* ``attention`` causal decode attention over a paged cache (plain softmax,
                plus the chunked log-sum-exp form used only as a pin).
* ``philox``    Philox4x32-10 counter-based generator.
* ``verify``    argmax with lowest-index ties, greedy accept-prefix, and the
                rejection-sampling accept rule.
* ``kvcache``   paged append, commit / rollback by truncation, position ids.

Every function is pinned by tests that do not re-type its formula: brute
force on tiny inputs, closed forms, invariants, hand-worked examples and an
independent implementation (Philox) -- see the ``tests`` directory.
"""
