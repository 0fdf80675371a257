"""Plain CPU oracle for the Muon step (momentum, Frobenius normalisation,
Newton–Schulz orthogonalisation, weight update).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library under ``muon_newton_schulz_06_amd/``.

Every function works in float64 (or exact rationals) on the CPU, written in
the order the method defines it, with no blocking, fusion or reordering.
"""

from .ns_oracle import (  # noqa: F401
    QUINTIC,
    CUBIC,
    bf16_round,
    frobenius_normalize,
    orient,
    newton_schulz,
    muon_orthogonalize,
    polar_svd,
    scalar_map,
    gram_newton_schulz,
    momentum_update,
    lr_shape_scale,
    muon_step,
    gram_flops,
)
from .selected import muon_step_selected, selected_count, select_rows, row_scores  # noqa: F401
from . import rational  # noqa: F401
