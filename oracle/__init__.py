"""CPU oracle for the split-backward pipeline stage.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call,
link or run anything here; only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  The oracle shares no code with the HIP path: it is plain
numpy in float64 with no intermediate rounding, plus the C loop nests of
``loopnest.c`` (fp64, sums in index order).

Sources ("the pages"):

* [Guide]    "Zero-Bubble Pipeline Parallelism Guide for LLMs" (aifetchly blog)
* [Abstract] "Zero Bubble Pipeline Parallelism" (mlsanity paper page, arXiv
             2401.10241 abstract)
* [Ghost]    "The Ghost in the Machine: Scaling Zero-Bubble Pipeline
             Parallelism" (architects-blueprint blog)

Modules:

* ``dense``    -- F / B / W of a linear layer, the GPT MLP block and the
                  Llama decoder layer; a fused backward for the B+W
                  invariant; the stash-and-pop stage object.
* ``schedule`` -- integer-time pipeline simulator for GPipe, 1F1B, the
                  memory-limited zero-bubble greedy schedule (one iteration
                  and several) and interleaved 1F1B.
* ``loopnest`` -- F, B and W of a linear layer as plain fp64 C loop nests
                  (``loopnest.c``, OpenMP over output rows): the products'
                  defining sums, timed as the benchmark's CPU baseline.
* ``fp8``      -- E4M3 decoding, rounding and per-tensor power-of-two
                  scaling, the fp8 product, and the Llama stage with every
                  linear product on fp8 operands.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``: finite differences, textbook/library special
cases (torch fp64 autograd, SDPA, rms_norm, gelu), brute-force loops on tiny
inputs, and the closed forms and table values printed on the pages.  Every
function in this package is pinned; none is "parity unpinned".
"""
