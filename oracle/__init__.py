"""CPU fp64 oracle for exact attention — TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The GPU library under ``io_aware_exact_flash_amd/`` never imports,
links or calls anything here, and nothing here imports that library.

Modules
-------
``attention``      the plain definition of attention and its gradient,
                   materialising S and P in float64 (the parity oracle).
``online``         the pages' blocked online-softmax recurrences, written out
                   step by step; used only to pin ``attention`` (Theorem 1).
``philox``         the Philox4x32-10 counter-based generator (from its
                   published definition) and the dropout keep decisions.

Every function in ``attention`` is pinned by ``tests/test_oracle.py`` against
facts the pages or mathematics fix (worked example, closed forms, finite
differences, invariants); none is "parity unpinned".
"""
