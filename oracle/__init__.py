"""CPU oracle for EAGLE draft-tree verification — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 reference of what the verification step computes:

* ``oracle.attention``  tree-masked attention, computed per node as ordinary
  attention over the keys it may see (prefix + its root path), gathered
  explicitly, with no mask at all;
* ``oracle.accept``     multi-round speculative sampling over the vocabulary,
  run as a scalar left-to-right walk that visits only the nodes the walk
  reaches;
* ``oracle.philox``     Philox4x32-10 counter-based uniforms, written from the
  published definition.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``eagle_draft_tree_attention_amd``) and never imports it.
"""
from . import philox, attention, accept  # noqa: F401
