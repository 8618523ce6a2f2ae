"""CPU oracle for the exact attention forward: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(the HIP library and its Python binding) never calls it, and this package
imports nothing from the product path.

Everything here runs on the host in float64 with NumPy.  The functions follow
the two source pages:

* "NTU Hung-yi Lee ML 2026 Guide: Faster Generation, Part 1: Flash Attention"
  (quidproquo.cc), sections "Intuition: the naive way makes many warehouse
  trips" and "Mechanism: run with the wrong answer, then correct it" with its
  two "Expand" formula boxes (slides 11-27);
* "6.3 FlashAttention" (comfyai.app), sections 6.3.2 "Standard Attention and
  Safe Softmax" and 6.3.3 "FlashAttention Forward Process" (its "Decoupled
  Softmax", "A Simple Example" and "Full Forward Process" parts).

``attention_bwd`` is the gradient of ``attention`` with respect to q, k and
v for an upstream gradient of O (the chapter's note that the training
backward recomputes instead of storing), written as the plain chain rule.

``attention_ex`` / ``attention_ex_bwd`` add a general mask (boolean or
additive) and dropout on the weights, with the keep pattern drawn from the
counter-based generator in ``philox.py`` (Philox4x32-10 from its published
definition).

Pins (in ``tests/test_oracle.py``; the masked / dropout ones in
``tests/test_oracle_ex.py``; the backward's in
``tests/test_oracle_bwd.py``: finite differences, float64 autograd, closed
forms, invariants and planted mistakes): the two-block worked example [1,2,3,4],
closed forms (identical keys, constant values, zero scale, one key, causal
row 0), invariants (row permutation, key shift), SciPy's ``softmax`` /
``logsumexp`` on explicit score matrices, and brute force over every chunk
partition for L <= 8 across the independent recurrences below.
"""

from .attention import (  # noqa: F401
    attention,
    attention_bwd,
    attention_ex,
    attention_ex_bwd,
    decode_varlen,
    one_pass_chunked,
    tiled_outer_kv,
    two_pass_chunked,
    decoupled_softmax,
)
