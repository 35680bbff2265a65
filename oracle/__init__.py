"""Plain fp64 CPU oracle for sparse fixed-offset attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls, links or
executes anything in this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code,
tables or helpers with the HIP library: it is written from the three source
pages directly and is deliberately slow and obvious.

Sources (cited by page title and the part of the page):

* "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static Schedules
  Beat Learned Dilation and Extrapolate Where Dense Attention Fails" (page 1):
  the key set (dense window plus scaled Fibonacci rungs), the fib equation, the
  interpolated gather after RoPE, the alpha parameterisation and the four
  per-layer schedules, the reach-matched power-of-2 control.
* "Critical power-law sparse attention" (page 2), items 1-2: power-law edge
  lists and masked softmax over them.
* "Christoffel-Balanced Sparse Attention" (page 3): the carry word, its
  offset set and the gather/softmax/value-sum pseudocode.

Every module states which of its functions are pinned by tests against facts
the pages or mathematics fix.  No function here is "parity unpinned".
"""

from . import offsets, christoffel, powerlaw, rope, attention  # noqa: F401
