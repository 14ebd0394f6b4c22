"""CPU oracle for single-step MLA / GQLA decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``head_latent_attention_02_amd``) never imports it, and this package
never imports the product path: the two share no code.  Inputs come from the seeded
generators in ``workloads`` (random draws only, none of the method's arithmetic).

Everything here is plain numpy in float64, written from the pages' definitions:

* ``mla``   - the plain definition (naive, non-absorbed MLA that materialises per-head
              keys and values) plus the plain definitions of each step of the absorbed
              path (query absorption, per-split softmax partials, split combine, value
              up-projection) and of the GQLA per-group path and cache expansion.
* ``brute`` - the same naive attention as pure-Python scalar loops, for tiny shapes,
              used to pin ``mla`` against an independent implementation.
* ``append`` - the cache-append step on the write side: latent down-projection, RoPE
              key projection and rotation, paged write of the new tokens' rows.
* ``projections`` - the query projection from the hidden state and the output projection
              back to it, unfolded and with W_UK / W_UV folded into them offline.

Parity status: every function in ``mla`` is pinned by tests/test_oracle.py against
something other than itself (pure-Python brute force, torch's scaled-dot-product
attention as a library routine, closed forms for special cases, the absorbed/expanded
and MQA-absorb/GQA-path equivalences the pages state, and the cache sizes the pages
print); every function in ``append`` by tests/test_oracle_append.py (the rotation's
group properties, a complex-number formulation, pure-Python loops, closed forms and the
positions the decode path's visibility rule fixes); every function in ``projections`` by
tests/test_oracle_projections.py (associativity of the fold, pure-Python loops, identity
weights, and the whole step through the naive decode).  No function here is "parity
unpinned".
"""
from . import mla, brute, append, projections  # noqa: F401
