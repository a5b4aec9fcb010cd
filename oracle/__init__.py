"""CPU fp64 oracle of the Muon optimizer step -- test infrastructure only.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the product package.
"""

from . import brute, muon_oracle, spectral, svd_entropy  # noqa: F401
