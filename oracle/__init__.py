"""fp64 CPU oracle for the Domino head drafting loop.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import this package.  The HIP
library never calls it, and this package never loads the HIP library.

Two independent implementations live here:

* ``draft`` / ``accept_len`` / ``verify`` / ``param_count``: the plain C oracle
  (domino_oracle.c), loops in double, called through ctypes;
* ``oracle.numpy_ref``: a vectorised NumPy float64 rewrite used only to
  cross-check the C oracle on small shapes.
"""
from .core import draft, accept_len, verify, param_count, build, lib_path, max_threads  # noqa: F401
