"""Attention-score visual-token selection on AMD MI355X (gfx950).

The compute runs in ``libtsel.so`` (hand-written HIP kernels behind the
C-ABI in ``include/tsel.h``); ``binding`` is a thin ctypes layer with the same
call names.
"""
from .binding import (EXPORTS, LIB_PATH, Layout, TselError, lib, select, tsel_attention_fwd,
                      tsel_budget_mass, tsel_budget_topk,
                      tsel_colscore, tsel_colscore_noalloc, tsel_compact, tsel_lse,
                      tsel_mrope_positions, tsel_workspace_size)

__all__ = ["EXPORTS", "LIB_PATH", "Layout", "TselError", "lib", "select", "tsel_attention_fwd",
           "tsel_budget_mass", "tsel_budget_topk",
           "tsel_colscore", "tsel_colscore_noalloc", "tsel_compact", "tsel_lse",
           "tsel_mrope_positions", "tsel_workspace_size"]
