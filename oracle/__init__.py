"""fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package. The HIP library never depends on it, and it shares no code, table or
constant generator with the HIP library: both sides receive the same seeded
inputs (from ``fa_inputs``) and nothing else.

Sources (the three web pages this library is built from):

* [LIB] "FlashAttention v1/v2/v3/v4: the librarian who never clears the desk —
  IO-awareness, async and Blackwell's asymmetry" (blog.lo0.es).
* [HUB] "FlashAttention" concept page (research hub, gunjandhanuka.github.io).
* [LIN] "The FlashAttention lineage — FA1 / FA2 / FA3 / FA4".

Modules:

* ``attention`` – forward and backward by definition (S and P materialised),
  plus the online (m, l) recurrence used only as a diagnostic.
* ``fp8`` – fp32 emulation of the e4m3 block quantiser and the random-sign
  Hadamard rotation, bit-for-bit in the order the kernels use.

Parity status of each function is stated in its docstring; every function is
pinned by ``tests/test_oracle_pins.py`` except where it says "parity unpinned".
"""

from . import attention, fp8  # noqa: F401
