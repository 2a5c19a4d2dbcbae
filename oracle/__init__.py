"""CPU oracle for the per-rank blockwise ring-attention step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 numpy
statement of what the hot path computes.  Only the test-suite, the smoke check of
the graft entry point and the CPU-baseline leg of the benchmark may import it.
It shares no code with the HIP library under ``ring_attention_blockwise_amd``
(no kernels, headers, helpers or tables) and neither side imports the other; the
only common module is ``seeded_inputs``, which draws input numbers and holds none
of the method's arithmetic.

Modules
-------
``index_maps``  chunk-to-rank maps (contiguous, zigzag), the ring schedule and
                the FULL/DIAG/SKIP classification of (query, key) blocks.
``attention``   full-softmax attention over the concatenated sequence (the
                definition), per-block partials, the log-sum-exp merge and the
                oracle's own ring decomposition (used as an invariant only).
``relayout``    the Ulysses sequence<->head regrouping.
``attention_backward``  dQ, dK, dV of the definition (the backward pass),
                pinned by ``tests/test_oracle_backward.py`` against finite
                differences of the forward definition.

Every function cites the passage of the source pages it follows: the ringmaster
package description (sections "Why", "Status", "Layout"), the blog posts
"Sequence Parallelism II/III/IV", the dictionary entry "context parallelism",
the TASP paper page, and the DeDLOC guide (sections "The Geo-Distributed
Long-Context Crisis", "3. Online Softmax Rescaling Across Decentralized Ranks",
"Step 3", "Step 4" and the "Best Practices" table).

Parity status: every function here is pinned by ``tests/test_oracle.py`` against
brute force, closed forms, a library routine or an exact invariant.  The pages
print no worked numeric example, so no pin is a printed value from the pages;
the hand-derived fixtures in ``tests/golden/`` state their derivations.
"""
