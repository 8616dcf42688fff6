"""Sliding-window scaled-dot-product attention (forward + window-bounded
backward) for MI355X / gfx950, as hand-written HIP kernels behind a C ABI
(``include/swa_sdpa.h``).  This package is the thin Python binding."""
from .api import (Backward, backward, forward, sdpa_bwd_plan, sdpa_bwd_relay_expiries, sdpa_bwd_run,
                  sdpa_bwd_run_events,
                  sdpa_bwd_schedule, sdpa_fwd_plan, sdpa_fwd_run)

__all__ = ["forward", "backward", "Backward", "sdpa_bwd_plan", "sdpa_bwd_relay_expiries", "sdpa_bwd_run",
           "sdpa_bwd_run_events", "sdpa_bwd_schedule", "sdpa_fwd_plan", "sdpa_fwd_run"]
