"""CPU oracle (test infrastructure only: imported by tests/, the smoke check
and the CPU-baseline leg of bench.py, never by the product path)."""
from .qwen3 import (OracleConfig, OracleState, Qwen3Oracle, apply_rope, attention,  # noqa: F401
                    greedy_trajectory, pick_token, rms_norm, rope_angles, silu, softmax_rows)
from .metrics import step_metrics  # noqa: F401
