"""Plain fp64 CPU oracle for single-token GQA decode attention with query-aware
top-k selection of KV tokens or pages.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The GPU library never imports, links or calls it, and it shares no code,
header, table or helper with the GPU library. Inputs reach both sides from
``kvsynth`` (seeded synthetic data only; no attention arithmetic there).

Sources, cited by page title and the section/table on that page:

* [Cross/cards] "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
  Decoding" (cards view): three abstracts -- pre-hoc sparsity with dropped
  mass delta, EntmaxKV (query-aware page scoring, candidate selection, sparse
  attention; output error controlled by delta), SparDA.
* [Cross/list] the same title, list view: the byte-crossover paper -- its
  Abstract (dense and sparse modes share one split-K kernel; attention-scored
  KV selection) and Tables 1-17.
* [Mass] "Attention-Mass Condensation for Sparse Decoding": the attention-mass
  top-k oracle abstract (dense attention, then a top-k support, then attention
  recomputed on that support only).
* [SparDA] "SparDA: Sparse Decoupled Attention for Efficient Long-Context LLM
  Inference" summary page: Section 3.1 (attention over the attended blocks
  only), Appendix A (selected block set), Appendix C (64-token blocks).

Modules:

* :mod:`oracle.sdref` -- logits, dense and sparse attention, page bounds,
  page and token scores, keep count, top-k selection, dropped mass, and a
  whole decode step.
* :mod:`oracle.bytemodel` -- the byte-crossover and byte-bound model of
  [Cross/list] Abstract and Tables 1, 2, 9, 11, 14 and 17.

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, invariants or brute force.
"""

from . import sdref, bytemodel, entmaxref  # noqa: F401
