"""CPU float64 oracle of the frame-wise GDN scan (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library.
"""

from .gdn_oracle import (  # noqa: F401
    chunk_bounds,
    combine,
    compose,
    default_key_scale,
    frame_terms,
    prepare_keys,
    readout,
    scan_bidir_chunked,
    scan_fwd,
    scan_reverse_chunked,
    transition,
)
