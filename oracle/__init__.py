"""CPU oracle for the exact attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

* ``oracle.ref``   -- numpy float64 implementation that materialises every
  score row and applies the plain softmax (no online softmax, no tiling).
* ``oracle.brute`` -- scalar pure-Python loops (``math.fsum``) for tiny shapes;
  it is written separately from ``ref`` and used to pin it.

The oracle shares no code with the HIP kernels or their host layer.
"""

from . import ref, brute  # noqa: F401
