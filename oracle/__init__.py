"""fp64 CPU oracle for packed block-diagonal causal attention and its planner.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP path and never imports it; the library never imports this package.

* ``oracle.attention``: the attention forward (O, LSE) and backward (dQ, dK, dV)
  in float64, evaluated per sample and head from the definition.
* ``oracle.plan``: SH-Tiles with eq. 8 pair counts, the work items and their
  executed-work costs, and Algorithm 2 placement (with the L2 residency
  term), in plain Python.
* ``oracle.vrsp``: variance-reduced sequence placement (Algorithm 1).
* ``oracle.bf16_reference``: the plain bf16 PyTorch evaluation whose error
  scales the pages' tolerance criterion (Libra paper, section 6.7).

Pins (tests marked ``not gpu``): brute-force dense masked attention on tiny
packs, packed == per-sample, tiled == untiled, the sum-of-squares closed form
and hand-derived eq. 8 tables, first-token and identical-V pass-through, the
zero-key prefix-mean closed form, finite differences of the backward, GQA ==
repeated MHA, hand-worked placement and cost cases, and the bf16 reference's
float64 graph against the oracle plus its stored errors.  No function here is
left unpinned.
"""
from . import attention, plan, vrsp  # noqa: F401
