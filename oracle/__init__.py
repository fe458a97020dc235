"""Plain fp64 CPU oracle for speculative-verify attention over a paged,
rollback-able KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product (``speculative_verify_attention_amd``) never imports, links or runs
it, and the two share no code: no kernels, helpers, constants or generators.
Every function here is written for a reader who checks it against the pages by
eye, so it is deliberately slow: no blocking, no fusion, no reordering beyond
what the definition it follows states.

Modules
-------
``splitmix``     SplitMix64 and the seeded draws built on it (free-list
                 permutation, rotation signs, QJL Gaussian matrix).
``bookkeeping``  the block allocator / block table / seq_len model with
                 O(1) rollback.
``attention``    masked, soft-capped, grouped-query softmax attention for the
                 1+k verify rows of one sequence, written as its definition.
``tq3``          the compressed-cache codec: Lloyd-Max codebook solver,
                 Sylvester-Hadamard rotation, encode and decode.
``accept``       acceptance of the drafts after the verify forward: greedy
                 argmax and rejection sampling against the draft
                 distribution, with the caller's uniforms.
``ngram``        the n-gram self-drafter that proposes the drafts (bigram /
                 trigram continuation tables, EMA acceptance gate).

Every function cites the passage of the pages it follows; where the pages are
silent the plainest reading is taken and named in the docstring.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, library routines or published tables.
"""

from . import splitmix, bookkeeping, attention, tq3, accept, ngram  # noqa: F401
