"""CPU oracle (test infrastructure only; see ``oracle.reference``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .reference import (  # noqa: F401
    to_f64,
    round_to_storage,
    head_blocks,
    exact_total_ok,
    split,
    unsplit,
    rope_angles,
    rmsnorm,
    rope_rotate_half,
    rope_rotate_half_inverse,
    forward_gqa,
    backward_gqa,
    latent_forward,
    paged_slots,
    staged_then_scatter,
)
from .mla_drafter import absorb, drafter_layer  # noqa: F401,E402
from .projection import project, projected_forward_gqa  # noqa: F401,E402
