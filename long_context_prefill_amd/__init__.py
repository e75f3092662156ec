"""S2O causal-prefill attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libs2o.so`` (C ABI in include/s2o.h);
this package only binds it.  ``synth`` draws seeded synthetic inputs.
"""

from ._lib import (S2OError, Problem, problem, problem_for, check_problem, list_entries,
                   list_offset, score_workspace_bytes, build_index_workspace_bytes, s2o_score,
                   s2o_score_noalloc, SCORE_NOALLOC_MAX_WORKSPACE, s2o_build_index, s2o_attn_fwd, dense_attn_fwd, s2o_attention, lib, EXPORTS,
                   LIB_PATH)

__all__ = ["S2OError", "Problem", "problem", "problem_for", "check_problem", "list_entries",
           "list_offset", "score_workspace_bytes", "build_index_workspace_bytes", "s2o_score",
           "s2o_score_noalloc", "SCORE_NOALLOC_MAX_WORKSPACE", "s2o_build_index", "s2o_attn_fwd", "dense_attn_fwd", "s2o_attention", "lib",
           "EXPORTS", "LIB_PATH"]
