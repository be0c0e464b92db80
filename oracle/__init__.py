"""CPU oracle (test infrastructure only; see ``tsel_oracle``)."""
from .tsel_oracle import (attention_forward, attention_segments, attention_stats, budget_k, compact, compact_loop,
                          default_scale, default_workers, forward_rows, fp8_e4m3_to_f64, lse_rows, mass_budget, mass_budget_k,
                          mass_units, pool_bounds,
                          request_of_candidate, rope_positions, run, scores, to_f64, topk)

__all__ = ["attention_forward", "attention_segments", "attention_stats", "budget_k", "compact", "compact_loop",
           "default_scale", "default_workers", "forward_rows", "fp8_e4m3_to_f64", "lse_rows", "mass_budget", "mass_budget_k",
           "mass_units", "pool_bounds",
           "request_of_candidate", "rope_positions", "run", "scores", "to_f64", "topk"]
