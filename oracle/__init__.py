"""CPU oracle for rank-major MoE expert-parallel dispatch and combine.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never does.
"""

from .moe_ep import (ALL_RANKS, MAX_RANKS, UNSPECIFIED_BYTE, DispatchRecord, OracleError,
                     OracleMoEEp, Params, RankResult, active_rank_mask, destination_mask,
                     expert_owner, expert_standin, step_tokens_per_rank)
from .numerics import bf16_bits_to_f32, f32_to_bf16_bits_rne

__all__ = [
    "ALL_RANKS", "MAX_RANKS", "UNSPECIFIED_BYTE", "DispatchRecord", "OracleError", "OracleMoEEp",
    "Params", "RankResult", "active_rank_mask", "destination_mask", "expert_owner",
    "expert_standin", "step_tokens_per_rank", "bf16_bits_to_f32", "f32_to_bf16_bits_rne",
]
