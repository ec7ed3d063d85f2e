"""TEST INFRASTRUCTURE ONLY: the reference (oracle) for the verification step.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``hierarchical_sparse_kv_verify_amd``) and never imports it.
"""
from .model import (  # noqa: F401
    CLS_HOT, CLS_MISS, CLS_RESIDENT, CLS_TAIL, HOT, RESIDENT, RING, STAGED,
    HierOracle, OracleConfig, StepResult, completed_rows, loc_code, ring_addr, ring_rows, staging_bytes,
)
from .residency import OptResidency  # noqa: F401
from . import native  # noqa: F401
