"""CPU oracle for the MoE verify layer and for cost-aware draft selection.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never calls it, shares no code with it, and must fail loudly rather
than fall back to it.

Plain, slow, obviously correct NumPy in float64 (float32 exactly where the
pages or the chosen reading fix float32 arithmetic: the biased logits and the
selection score).  Each function cites the passage it follows; the readings
taken where the pages are silent or garbled are listed in the function
docstrings:

* ``moe``     router logits, top-k, gate weights, reuse-aware soft bias,
              expert union, token-by-expert CSR, per-token dense MoE layer,
              per-layer union statistics;
* ``select``  EcoSpec cost-aware greedy draft selection;
* ``expand``  S^2-MoE utility-driven adaptive expansion of a draft tree;
* ``ragged``  confidence-gated per-sequence depths and per-sequence union
              statistics of a ragged verify call;
* ``fp``      bf16 and OCP FP8 E4M3FN decoding from their definitions.

Parity status: every function is pinned by CPU tests against closed forms,
invariants, brute force or the pages' worked example, except the numeric form
of the reuse-bias steps (importance g, TopCap, bias size), whose formulas are
missing from the page; that part is pinned to the stated reading and to the
page's qualitative example only ("parity pinned to the reading").
"""
from . import expand, fp, moe, ragged, select  # noqa: F401
