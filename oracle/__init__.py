"""Plain fp64 CPU oracle for the Muon step and the AdamW step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package. The product path (``muon_newton_schulz_amd`` and its HIP library)
never touches it, and this package imports nothing from the product.
"""

from .muon_oracle import (  # noqa: F401
    AdamWHP,
    MuonHP,
    adamw_math,
    adamw_step_stored,
    bf16_round,
    ema_momentum,
    fp32_round,
    frobenius_normalise,
    muon_matrix_math,
    muon_step_flat,
    nesterov_lookahead,
    newton_schulz,
    ns_flops,
    ns_iteration,
    update_scale,
)
