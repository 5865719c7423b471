"""CPU oracle for the shared-prefix decode-attention path (TEST INFRASTRUCTURE).

This package is the slow, obviously-correct statement of what the decode step
computes, written from the GraniKV pages:

* "GraniKV: Asymmetric Granularity KV-Cache Paging for Multi-Agent Systems with
  Long Shared Prefix" (paperlayer.ai summary), §2 Related Work bullet
  "Prefix–suffix attention", §3 "Asymmetric KV-cache paging", §3 "Per-step
  dispatch", Appendix B.10 "Cross-pool admission and promotion policy";
* the observer.broadside.tech reading card, "Key ideas" (HOT bump-pointer slab,
  COLD token-level free list, M_eff = B x n_q/n_kv).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The HIP library never imports, links or calls it,
and it shares no code with the HIP library: it works on the *logical* token
sequences (prefix tokens followed by suffix tokens) in float64 and never looks
at the HOT/COLD pools.

Modules
-------
attention  softmax attention over prefix || suffix, and the log-sum-exp merge
alloc      HOT first-fit extent allocator model and COLD LIFO free-list model
append     scatter model of appending new K/V rows into COLD slots
dispatch   the per-step backend rule M_eff >= M_sat
registry   the shared-prefix registry: HOT-first admission, COLD fallback, no
           demotion, cached prefixes evicted least recently released first,
           and the f_p partition of a KV budget

Pins (tests/test_oracle_pins.py, tests/test_oracle_alloc_pins.py,
tests/test_oracle_registry_pins.py): closed forms, a pure-Python brute force,
torch CPU float64 scaled_dot_product_attention, the merge invariant,
hand-derived allocator and registry traces, and invariants restated by brute
force.  Every public function here is pinned.
"""

from .attention import attend, decode_step, merge, softmax_scale  # noqa: F401
from .alloc import ColdAllocModel, HotAllocModel, NoSpace, NotFound  # noqa: F401
from .append import append_model  # noqa: F401
from .dispatch import BACKEND_CASCADE, BACKEND_DENSE, choose_backend, m_eff  # noqa: F401
from .registry import COLD, HOT, InvalidArg, RegistryModel, partition  # noqa: F401
