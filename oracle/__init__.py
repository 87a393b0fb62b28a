"""CPU oracle for the copy-on-write paged KV cache -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package. The library in
``paged_kv_cache_amd`` never calls it and shares no code with it.

What it computes, in plain numpy (attention in float64):

* ``OraclePool`` -- a pool of fixed-size KV blocks with reference counts,
  per-sequence block tables, fork as a copy of the parent's table that bumps
  each block's count, copy-on-write of a shared, partly filled tail block
  when a sequence appends, and release. Each sequence also carries its
  *materialised* K/V: the values it logically holds, independent of pages.
  Source: the Dendrite author's description of a paged cache in fixed blocks
  with O(1) CoW forking by shallow pointer copy, and of the rule that a block
  being written may not be aliased (HN page, "How is this different from
  vLLM's paged attention?" and "Why Rust?").
* A prompt cache inside ``OraclePool``: full blocks keyed by their token ids
  and the entry before them, longest-prefix match into a new sequence,
  parked blocks that outlive their sequence, least-recently-used eviction of
  entries only the cache holds when the pool runs dry. Source: Ferrite
  project page, section 07 and the "Agents" measurement.
* ``decode`` -- softmax(q K^T * scale) V over each sequence's materialised
  tokens, one query per sequence and head (grouped-query heads: head h reads
  KV head h // (Hq / Hkv)).
* ``verify`` -- draft-tree verification: each node attends to the request's
  context plus the tree nodes on its own root path (itself included). Source:
  Ferrite project page, section 04 ("DFlash2 verify trees"), drafts checked
  as best-first trees in one pass of the big model.

Pins (tests/test_oracle.py): dense unpaged attention through torch's
scaled_dot_product_attention on independently assembled sequences, hand
derivations stored under tests/golden/, closed forms (a single token returns
its V, a zero query returns the mean of V, equal keys return the mean of V),
refcount invariants and closed-form refcount histograms, and brute-force
equivalences (verify on a chain tree equals causal attention; each tree node
equals a decode over its ancestor path; a cache match equals the longest
cached prefix found by spelling out every entry; a resumed sequence equals
one computed in full), and a hand-derived eviction order. Every function here is pinned; none
is "parity unpinned".
"""

from .pool import InvalidError, OOMError, OraclePool  # noqa: F401
from .attention import ancestors, decode, decode_one, verify  # noqa: F401
