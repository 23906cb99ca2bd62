"""Plain float64 CPU oracle for ReadKV decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it, to check and to time the HIP implementation.  It
shares no code with the HIP path; it knows the store layout only from the
written format description.

``oracle.lloyd`` holds the pages' own codec (Gaussian Lloyd tree,
Hadamard-sign transforms, calibration) and the decode step over it.
"""
from .readkv import *  # noqa: F401,F403
from .store_format import pack_unit, unpack_unit  # noqa: F401
